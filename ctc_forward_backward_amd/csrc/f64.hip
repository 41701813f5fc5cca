// The float64 path: CTC loss and gradient of float64 log probabilities computed in float64.
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities".  Its loss module sends float64 log probabilities to the padded path, which keeps
// float64 precision (test file, `test_float64_takes_padded_path`); here they keep float64 on the
// packed layout instead.  The recursions are the Triton file's: `_alpha_kernel` (alpha[0] holds the
// first blank and the first label; alpha[t][s] is the log-sum-exp of alpha[t-1] at s, s-1 and, into
// a label whose id differs from the label two states back, s-2, plus the frame's log probability at
// the state's class; the loss is minus the log-sum-exp of the last two states) and
// `_beta_grad_kernel` (beta mirrors it from the last frame, and each frame's posteriors and gradient
// row are formed as beta passes it: gradient = w * (exp(lp) - posterior summed per class)).
//
// Design (precision first; the float32 / 16-bit inputs take the pipelined kernels):
//   - one workgroup per utterance; the S = 2U+1 states are split into contiguous ranges of at least
//     two states over up to 1024 threads, each range in registers; per frame every thread publishes
//     its two edge states in a double-buffered LDS array and reads its neighbour's, one barrier per
//     frame;
//   - natural-log space, log-sum-exp as max + log1p(exp(-|a - b|)) with HIP's float64 exp / log1p;
//   - alpha is stored in float64 in the workspace's state region (T_total rows of Gmax * 128
//     doubles); beta is not stored: the second kernel forms each frame's posteriors from the stored
//     alpha and its own beta, normalised by the frame's own total (the posteriors of a frame sum to
//     1), and writes the gradient row in float64 right away.
#include <math.h>

#include "pctc_internal.h"

namespace pctc {

namespace {

constexpr int kT64 = 1024;   // threads per workgroup
// PER, a kernel's template argument: states a thread holds at most (each thread holds ceil or floor
// of S / n states, n = min(1024, S / 2)): 4 for S <= 4096, 8 for S <= 8192, 16 up to 16383 =
// 2 * 8191 + 1.  The register arrays take PER entries, so the smallest that fits the call's target
// bound is launched (16 for every call kept the arrays' registers and spilled them).
constexpr double kNegInf = -INFINITY;

__device__ __forceinline__ double lse2d(double a, double b) {
  const double hi = fmax(a, b), lo = fmin(a, b);
  if (!(lo > kNegInf)) return hi;  // lo = -inf (or both): nothing to add
  return hi + log1p(exp(lo - hi));
}

// state split of an utterance with S states over n threads: thread i holds [lo, hi), at least two
// states each (except a single state when S = 1)
struct Split {
  int n, lo, hi;
};

__device__ __forceinline__ int threads_for(int S) { return S < 2 ? 1 : min(kT64, S / 2); }

__device__ __forceinline__ Split split_of(int S, int tid) {
  Split sp;
  sp.n = threads_for(S);
  sp.lo = (int)((int64_t)S * tid / sp.n);
  sp.hi = (int)((int64_t)S * (tid + 1) / sp.n);
  return sp;
}

// class of state s: the blank for even s, label (s + 1) / 2 for odd s (lab[0] is the blank)
__device__ __forceinline__ int class_of(const int* lab, int s) { return lab[(s & 1) ? (s + 1) >> 1 : 0]; }

__device__ __forceinline__ double ld_lp(const void* lp, int64_t i) { return static_cast<const double*>(lp)[i]; }

// workgroup reductions over the active threads (blockDim.x threads take part; LDS red: 32 doubles)
__device__ __forceinline__ double block_max(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = kNegInf;
  for (int i = 0; i < nw; ++i) r = fmax(r, red[i]);
  return r;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < nw; ++i) r += red[i];  // fixed order: reproducible
  return r;
}

__device__ __forceinline__ bool block_any(bool v, double* red) { return block_sum(v ? 1.0 : 0.0, red) > 0.0; }

// Alpha of utterance blockIdx.x (launched with 1024 threads; threads beyond the split idle at the
// barriers), the loss, and the NaN flag of the emissions it read.  Workgroup 0 also clears the
// health word (this path has no waits on other workgroups).
template <int PER>
__global__ void __launch_bounds__(kT64) f64_alpha_kernel(Inputs in, Layout L, Pointers P) {
  __shared__ double bnd[2][kT64][2];
  __shared__ double red[32];
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b == 0 && tid == 0) P.ctl->err = 0;
  if (b >= L.B) return;
  const Meta m = P.meta[b];
  const int T = m.T, U = m.U, S = 2 * U + 1;
  if (T == 0) {
    if (tid == 0) P.nll[b] = U == 0 ? 0.0 : (double)INFINITY;
    return;
  }
  const int* lab = P.lab + (int64_t)b * (L.Umax + 1);
  const Split sp = split_of(S, tid);
  const bool active = tid < sp.n;
  const int cnt = active ? sp.hi - sp.lo : 0;
  const int64_t Ss = L.Gmax * 128, D = L.D;
  double* A = reinterpret_cast<double*>(P.ABa);
  int cls[PER];
  bool skip[PER];
  double a[PER];
  bool nan = false;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int s = sp.lo + k;
    cls[k] = k < cnt ? class_of(lab, s) : 0;
    skip[k] = k < cnt && (s & 1) && s >= 3 && lab[(s + 1) >> 1] != lab[(s - 1) >> 1];
    a[k] = kNegInf;
    if (k < cnt && s <= 1) {
      const double e = ld_lp(in.log_probs, m.start * D + cls[k]);
      nan |= e != e;
      a[k] = e;
    }
    if (k < cnt) A[m.start * Ss + s] = a[k];
  }
  for (int t = 1; t < T; ++t) {
    const int buf = t & 1;
    const int64_t r = m.start + t;
    if (active) {  // the two highest states of this range at t-1
      bnd[buf][tid][0] = cnt >= 1 ? a[cnt - 1] : kNegInf;
      bnd[buf][tid][1] = cnt >= 2 ? a[cnt - 2] : kNegInf;
    }
    __syncthreads();
    if (active) {
      // alpha[t-1] at lo-1 and lo-2 (the previous range holds at least two states)
      double p1 = tid > 0 ? bnd[buf][tid - 1][0] : kNegInf;
      double p2 = tid > 0 ? bnd[buf][tid - 1][1] : kNegInf;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        if (k < cnt) {
          const double cur = a[k];
          double v = lse2d(cur, p1);
          if (skip[k]) v = lse2d(v, p2);
          const double e = ld_lp(in.log_probs, r * D + cls[k]);
          nan |= e != e;
          a[k] = v + e;
          A[r * Ss + sp.lo + k] = a[k];
          p2 = p1;
          p1 = cur;
        }
      }
    }
  }
  // loss: the last blank and the last label at the last frame
  double fin = kNegInf;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if (k < cnt && sp.lo + k >= S - 2) fin = lse2d(fin, a[k]);
  // the final states sit in at most two threads: combine them as a sum in linear space relative
  // to the larger
  const double top = block_max(fin, red);
  const double part = top > kNegInf && fin > kNegInf ? exp(fin - top) : 0.0;
  const double tot = block_sum(part, red);
  const bool any_nan = block_any(nan, red);
  if (tid == 0) {
    const double ll = top > kNegInf ? top + log(tot) : kNegInf;
    P.nll[b] = any_nan ? (double)NAN : (ll > kNegInf ? -ll : (double)INFINITY);
  }
}

// Beta of utterance blockIdx.x and, as it passes each frame, the frame's posteriors (from the stored
// alpha) and its gradient row.  acc: (Umax + 1) doubles of LDS (dynamic), the class sums by rank.
template <int PER>
__global__ void __launch_bounds__(kT64) f64_beta_rows_kernel(Inputs in, Layout L, Pointers P, double* grad) {
  if (skipped(P)) return;
  extern __shared__ double acc[];
  __shared__ double bnd[2][kT64][2];
  __shared__ double red[32];
  const int b = blockIdx.x, tid = threadIdx.x;
  const Meta m = P.meta[b];
  const int T = m.T, U = m.U, S = 2 * U + 1;
  if (T == 0) return;
  const int64_t Ss = L.Gmax * 128, D = L.D;
  const double nll = P.nll[b];
  const double w = utterance_weight64(in, L.B, b, nll == (double)INFINITY);
  if (w == 0.0 || !(nll < (double)INFINITY)) {
    // zero weight: zero rows; no alignment or a NaN input with a weight: NaN rows
    const double fill = w == 0.0 ? 0.0 : (double)NAN;
    for (int64_t i = tid; i < (int64_t)T * D; i += blockDim.x) grad[m.start * D + i] = fill;
    return;
  }
  const int* lab = P.lab + (int64_t)b * (L.Umax + 1);
  const int* dmap = P.dmap + (int64_t)b * (L.Umax + 1);
  const uint32_t* cbits = P.cbits + (int64_t)b * L.Dw;
  const int* cpref = P.cpref + (int64_t)b * L.Dw;
  const Split sp = split_of(S, tid);
  const bool active = tid < sp.n;
  const int cnt = active ? sp.hi - sp.lo : 0;
  const double* A = reinterpret_cast<const double*>(P.ABa);
  int cls[PER], rank[PER];
  bool skip[PER];
  double bt[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int s = sp.lo + k;
    cls[k] = k < cnt ? class_of(lab, s) : 0;
    rank[k] = k < cnt ? dmap[(s & 1) ? (s + 1) >> 1 : 0] : 0;
    // the skip from s + 2 back into the label s (beta's direction): ids of s and s + 2 differ
    skip[k] = k < cnt && (s & 1) && s + 2 < S && lab[(s + 1) >> 1] != lab[(s + 3) >> 1];
    bt[k] = kNegInf;
  }
  for (int i = tid; i <= U; i += blockDim.x) acc[i] = 0.0;
  for (int t = T - 1; t >= 0; --t) {
    const int64_t r = m.start + t;
    const double* lp = static_cast<const double*>(in.log_probs) + r * D;
    // beta at t (emission of frame t included)
    if (t == T - 1) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (k < cnt && sp.lo + k >= S - 2) bt[k] = lp[cls[k]];
    } else {
      const int buf = t & 1;
      if (active) {  // the two lowest states of this range at t+1
        bnd[buf][tid][0] = cnt >= 1 ? bt[0] : kNegInf;
        bnd[buf][tid][1] = cnt >= 2 ? bt[1] : kNegInf;
      }
      __syncthreads();
      if (active) {
        // beta[t+1] at hi and hi+1 (the next range holds at least two states)
        const bool last = tid + 1 >= sp.n;
        double n1 = last ? kNegInf : bnd[buf][tid + 1][0];
        double n2 = last ? kNegInf : bnd[buf][tid + 1][1];
#pragma unroll
        for (int k = PER - 1; k >= 0; --k) {
          if (k < cnt) {
            const double cur = bt[k];
            double v = lse2d(cur, n1);
            if (skip[k]) v = lse2d(v, n2);
            bt[k] = v + lp[cls[k]];
            n2 = n1;
            n1 = cur;
          }
        }
      }
    }
    // posteriors of frame t: alpha + beta - lp per state, normalised by the frame's own total
    double e[PER];
    double mx = kNegInf;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      e[k] = kNegInf;
      if (k < cnt) {
        const double ak = A[r * Ss + sp.lo + k];
        if (ak > kNegInf && bt[k] > kNegInf) e[k] = ak + bt[k] - lp[cls[k]];
        mx = fmax(mx, e[k]);
      }
    }
    mx = block_max(mx, red);
    double z = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (k < cnt && e[k] > kNegInf) {
        e[k] = exp(e[k] - mx);
        z += e[k];
      } else {
        e[k] = 0.0;
      }
    }
    z = block_sum(z, red);  // (its barriers also order the zeroed class sums before the adds)
    const double scale = z > 0.0 ? w / z : 0.0;
    // label states add into their class's sum; the blank states (all one class) are summed per
    // thread first
    double bsum = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (k < cnt && e[k] != 0.0) {
        if ((sp.lo + k) & 1) atomicAdd(&acc[rank[k]], e[k] * scale);
        else bsum += e[k] * scale;
      }
    }
    if (bsum != 0.0) atomicAdd(&acc[dmap[0]], bsum);
    __syncthreads();
    // the gradient row: w exp(lp) minus the class sum at the columns that carry a class
    double* g = grad + r * D;
    for (int64_t c = tid; c < D; c += blockDim.x) {
      const int wi = (int)(c >> 5);
      const uint32_t bits = cbits[wi];
      double v = w * exp(lp[c]);
      if ((bits >> (c & 31)) & 1u) v -= acc[cpref[wi] + __builtin_popcount(bits & ((1u << (c & 31)) - 1u))];
      g[c] = v;
    }
    __syncthreads();
    for (int i = tid; i <= U; i += blockDim.x) acc[i] = 0.0;
  }
}

}  // namespace

// states per thread of the longest target the call allows
int per_thread(const Layout& L) {
  const int64_t S = 2 * L.Umax + 1;
  return S <= 4096 ? 4 : (S <= 8192 ? 8 : 16);
}

hipError_t launch_f64_alpha(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(L.B > 0 ? L.B : 1);
  const int per = per_thread(L);
  if (per == 4) f64_alpha_kernel<4><<<grid, kT64, 0, s>>>(in, L, P);
  else if (per == 8) f64_alpha_kernel<8><<<grid, kT64, 0, s>>>(in, L, P);
  else f64_alpha_kernel<16><<<grid, kT64, 0, s>>>(in, L, P);
  return hipGetLastError();
}

hipError_t launch_f64_beta_rows(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s) {
  if (L.B == 0 || L.T_total == 0 || L.D == 0) return hipGetLastError();
  const size_t lds = sizeof(double) * (size_t)(L.Umax + 1);
  auto launch = [&](auto kernel) {
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    kernel<<<static_cast<unsigned>(L.B), kT64, lds, s>>>(in, L, P, static_cast<double*>(grad_out));
    return hipGetLastError();
  };
  const int per = per_thread(L);
  if (per == 4) return launch(&f64_beta_rows_kernel<4>);
  if (per == 8) return launch(&f64_beta_rows_kernel<8>);
  return launch(&f64_beta_rows_kernel<16>);
}

}  // namespace pctc
