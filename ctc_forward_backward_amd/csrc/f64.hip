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
//   - one workgroup per utterance, of 512 or 1024 threads by the call's longest target; the
//     S = 2U+1 states are split into contiguous ranges of at least two states, each range in
//     registers; per frame every thread publishes its two edge states in a double-buffered LDS array
//     and reads its neighbour's;
//   - what a frame reads (emissions, the stored alpha, the first columns of the gradient row) does
//     not depend on the recursion and is fetched a frame ahead where the registers allow it (four
//     states per thread in alpha, under 1024 threads in beta); the frames' barriers order LDS only, so those loads and the alpha and
//     gradient stores stay in flight across them; the beta side takes two barriers per frame (one
//     after the posteriors are added into the class sums, one after the gradient row), with the
//     class sums in two copies by frame parity, and takes each state's posterior relative to the
//     likelihood (at most 1) before normalising by the frame's own total;
//   - natural-log space, with HIP's float64 exp / log1p: a state's update is one three-term
//     log-sum-exp, the largest term plus log1p of the sum of the other two's exponentials relative
//     to it (the third term -inf where the skip is not allowed); alpha computes every slot of a
//     thread's range with no branch, so that the slots' chains interleave;
//   - alpha is stored in float64 in the workspace's state region (T_total rows of Gmax * 128
//     doubles); beta is not stored: the second kernel forms each frame's posteriors from the stored
//     alpha and its own beta, normalised by the frame's own total (the posteriors of a frame sum to
//     1), and writes the gradient row in float64 right away.
#include <math.h>

#include "pctc_internal.h"

namespace pctc {

namespace {

constexpr int kT64 = 1024;   // threads per workgroup, at most
// PER and NT, a kernel's template arguments: states a thread holds at most (each thread holds ceil
// or floor of S / n states, n = min(NT, S / 2)) and the workgroup's threads: PER 4 for S <= 4096
// (NT 512 up to S = 1024, else 1024), 8 for S <= 8192, 16 up to 16383 = 2 * 8191 + 1.
// The register arrays take PER entries, so the smallest that fits the call's target bound is
// launched (16 for every call kept the arrays' registers and spilled them).
constexpr double kNegInf = -INFINITY;

__device__ __forceinline__ double lse2d(double a, double b) {
  const double hi = fmax(a, b), lo = fmin(a, b);
  if (!(lo > kNegInf)) return hi;  // lo = -inf (or both): nothing to add
  return hi + log1p(exp(lo - hi));
}

// log(e^a + e^b + e^c) with no branch: the largest plus log1p of the other two relative to it (both
// exponentials at once, then one log1p: the depth of a two-term log-sum-exp); a term at -inf adds
// nothing, and all three at -inf give -inf
__device__ __forceinline__ double lse3d(double a, double b, double c) {
  const double hi = fmax(a, b), lo = fmin(a, b);
  const double m = fmax(hi, c), mid = fmin(hi, c);
  const double ref = m > kNegInf ? m : 0.0;
  return m + log1p(exp(lo - ref) + exp(mid - ref));
}

// state split of an utterance with S states over n threads: thread i holds [lo, hi), at least two
// states each (except a single state when S = 1)
struct Split {
  int n, lo, hi;
};

__device__ __forceinline__ int threads_for(int S, int nt) { return S < 2 ? 1 : min(nt, S / 2); }

// (nt: the workgroup's threads)
__device__ __forceinline__ Split split_of(int S, int tid, int nt) {
  Split sp;
  sp.n = threads_for(S, nt);
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

// Alpha of utterance blockIdx.x (launched with NT threads; threads beyond the split idle at the
// barriers), the loss, and the NaN flag of the emissions it read.  Workgroup 0 also clears the
// health word (this path has no waits on other workgroups).
template <int PER, int NT>
__global__ void __launch_bounds__(NT) f64_alpha_kernel(Inputs in, Layout L, Pointers P) {
  __shared__ double bnd[2][NT][2];
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
  const Split sp = split_of(S, tid, NT);
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
  // a frame's emissions do not depend on the recursion: fetched one frame ahead (every thread loads,
  // at a valid column), and the frame's barrier orders LDS only, so neither these loads nor the
  // alpha stores are waited for at it
  double en[PER];
  auto fetch = [&](int t) {
    const int64_t r = m.start + t;
#pragma unroll
    for (int k = 0; k < PER; ++k) en[k] = ld_lp(in.log_probs, r * D + cls[k]);
  };
  // (ahead only with four states per thread: with more, the second set of registers spills)
  constexpr bool kAhead = PER == 4;
  if (kAhead && T > 1) fetch(1);
  for (int t = 1; t < T; ++t) {
    const int buf = t & 1;
    const int64_t r = m.start + t;
    if (!kAhead) fetch(t);
    double ec[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) ec[k] = en[k];
    if (kAhead && t + 1 < T) fetch(t + 1);
    if (active) {  // the two highest states of this range at t-1
      bnd[buf][tid][0] = cnt >= 1 ? a[cnt - 1] : kNegInf;
      bnd[buf][tid][1] = cnt >= 2 ? a[cnt - 2] : kNegInf;
    }
    lds_barrier();
    if (active) {
      // alpha[t-1] at lo-1 and lo-2 (the previous range holds at least two states); every slot of
      // the range is computed, with no branch, so that the slots' chains interleave (a slot past the
      // range computes from -inf and is not kept)
      const double p1 = tid > 0 ? bnd[buf][tid - 1][0] : kNegInf;
      const double p2 = tid > 0 ? bnd[buf][tid - 1][1] : kNegInf;
      double na[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const double s1 = k == 0 ? p1 : a[k - 1], s2 = k == 0 ? p2 : (k == 1 ? p1 : a[k - 2]);
        na[k] = lse3d(a[k], s1, skip[k] ? s2 : kNegInf) + ec[k];
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        if (k < cnt) {
          nan |= ec[k] != ec[k];
          a[k] = na[k];
          A[r * Ss + sp.lo + k] = a[k];
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
// alpha) and its gradient row.  acc: (Umax + 1) doubles of LDS (dynamic), the class sums by rank, or
// twice that when two is set.
template <int PER, int NT>
__global__ void __launch_bounds__(NT) f64_beta_rows_kernel(Inputs in, Layout L, Pointers P, double* grad, int two) {
  if (skipped(P)) return;
  extern __shared__ double acc[];
  __shared__ double bnd[2][NT][2];
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
  const Split sp = split_of(S, tid, NT);
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
  // the class sums by rank, in two copies taken by frame parity when the LDS holds both (then one
  // barrier fewer per frame: a frame fills one copy while the other is cleared)
  const int64_t Cs = L.Umax + 1;
  const bool dual = two;
  for (int i = tid; i < (dual ? 2 * Cs : Cs); i += blockDim.x) acc[i] = 0.0;
  const int dblank = dmap[0];
  const double ll = -nll;  // the log likelihood: every state's posterior is at most 1 relative to it
  const int lane = tid & 63, wv = tid >> 6, nw = (blockDim.x + 63) >> 6;
  // What a frame reads (its emissions at the states' classes, the stored alpha, the thread's first
  // GC columns of the gradient row) does not depend on beta: below 1024 threads it is fetched for
  // frame t-1 as soon as frame t has used it (every thread loads, at valid addresses), and the
  // frame's barriers order LDS only, so these loads run under frame t's barriers and gradient row,
  // and the gradient stores are not waited for at them.  The class rank of each of those GC columns
  // (-1: no class) is found once: the class bitmap does not change between frames.
  constexpr int GC = NT < kT64 ? 8 : 1;
  double lq[PER], aq[PER], gq[GC];
  int rk[GC];
#pragma unroll
  for (int j = 0; j < GC; ++j) {
    const int64_t c = min((int64_t)tid + (int64_t)j * NT, D - 1);
    const int wi = (int)(c >> 5);
    const uint32_t bits = cbits[wi];
    rk[j] = (bits >> (c & 31)) & 1u ? cpref[wi] + __builtin_popcount(bits & ((1u << (c & 31)) - 1u)) : -1;
  }
  auto fetch_states = [&](int t) {
    const int64_t r = m.start + t;
    const double* lp = static_cast<const double*>(in.log_probs) + r * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      lq[k] = lp[cls[k]];
      aq[k] = A[r * Ss + min(sp.lo + k, S - 1)];
    }
  };
  auto fetch_col = [&](int t) {
    const double* lp = static_cast<const double*>(in.log_probs) + (m.start + t) * D;
#pragma unroll
    for (int j = 0; j < GC; ++j) gq[j] = lp[min((int64_t)tid + (int64_t)j * NT, D - 1)];
  };
  // (ahead only below 1024 threads: at that register budget the loads ahead spill)
  constexpr bool kAhead = NT < kT64;
  if (kAhead) {
    fetch_states(T - 1);
    fetch_col(T - 1);
  }
  __syncthreads();
  for (int t = T - 1; t >= 0; --t) {
    const int64_t r = m.start + t;
    const double* lp = static_cast<const double*>(in.log_probs) + r * D;
    const int par = t & 1;
    double* cs = acc + (dual ? par * Cs : 0);
    // a state's emission and alpha at frame t: fetched ahead, or read here
    auto emis = [&](int k) { if constexpr (kAhead) return lq[k]; else return lp[cls[k]]; };
    auto alph = [&](int k) { if constexpr (kAhead) return aq[k]; else return A[r * Ss + sp.lo + k]; };
    // beta at t (emission of frame t included)
    if (t == T - 1) {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (k < cnt && sp.lo + k >= S - 2) bt[k] = emis(k);
    } else if (active) {
      // beta[t+1] at hi and hi+1, as the next range left them (it holds at least two states)
      const bool last = tid + 1 >= sp.n;
      const double n1 = last ? kNegInf : bnd[par ^ 1][tid + 1][0];
      const double n2 = last ? kNegInf : bnd[par ^ 1][tid + 1][1];
      // (the range's own states one after another: here the frame's posteriors and gradient row,
      // not this chain, set the pace, and computing every slot costs more than it saves)
      double s1 = n1, s2 = n2;
#pragma unroll
      for (int k = PER - 1; k >= 0; --k) {
        if (k < cnt) {
          const double cur = bt[k];
          bt[k] = lse3d(cur, s1, skip[k] ? s2 : kNegInf) + emis(k);
          s2 = s1;
          s1 = cur;
        }
      }
    }
    if (active) {  // the two lowest states of this range at t, for frame t-1
      bnd[par][tid][0] = cnt >= 1 ? bt[0] : kNegInf;
      bnd[par][tid][1] = cnt >= 2 ? bt[1] : kNegInf;
    }
    // posteriors of frame t: alpha + beta - lp per state relative to the likelihood; label states
    // add into their class's sum, the blank states (all one class) are summed per wave first; the
    // frame's own total normalises them when the row is written
    double x[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const double ak = k < cnt ? alph(k) : kNegInf;
      x[k] = k < cnt && ak > kNegInf && bt[k] > kNegInf ? ak + bt[k] - emis(k) - ll : kNegInf;
    }
    double z = 0.0, bsum = 0.0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (x[k] > kNegInf) {
        const double e = exp(x[k]);
        z += e;
        if ((sp.lo + k) & 1) atomicAdd(&cs[rank[k]], e);
        else bsum += e;
      }
    }
    if (kAhead && t > 0) fetch_states(t - 1);
    for (int o = 32; o > 0; o >>= 1) {
      z += __shfl_xor(z, o);
      bsum += __shfl_xor(bsum, o);
    }
    if (lane == 0) {
      red[wv] = z;
      if (bsum != 0.0) atomicAdd(&cs[dblank], bsum);
    }
    lds_barrier();
    double ztot = 0.0;
    for (int i = 0; i < nw; ++i) ztot += red[i];  // fixed order: reproducible
    const double scale = ztot > 0.0 ? w / ztot : 0.0;
    // the gradient row: w exp(lp) minus the class sum at the columns that carry a class
    double* g = grad + r * D;
    int64_t c0 = tid;
    if constexpr (kAhead) {
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        const int64_t c = (int64_t)tid + (int64_t)j * NT;
        if (c < D) g[c] = w * exp(gq[j]) - (rk[j] >= 0 ? cs[rk[j]] * scale : 0.0);
      }
      c0 += (int64_t)GC * NT;
    }
    for (int64_t c = c0; c < D; c += NT) {
      const int wi = (int)(c >> 5);
      const uint32_t bits = cbits[wi];
      double v = w * exp(lp[c]);
      if ((bits >> (c & 31)) & 1u) v -= cs[cpref[wi] + __builtin_popcount(bits & ((1u << (c & 31)) - 1u))] * scale;
      g[c] = v;
    }
    if (kAhead && t > 0) fetch_col(t - 1);
    lds_barrier();  // (the sums and the totals are read; this frame's copy is cleared for frame t-2)
    for (int i = tid; i <= U; i += blockDim.x) cs[i] = 0.0;
    if (!dual) lds_barrier();  // one copy: cleared before frame t-1 adds into it
  }
}

}  // namespace

// states per thread (PER) and threads per workgroup (NT) of the longest target the call allows:
// every thread holds at least two states, at most PER; a target of up to 511 labels takes 512
// threads (a larger register budget per thread, for the loads fetched ahead; 256 threads measured
// 3% slower: fewer waves share the gradient row)
struct F64Shape {
  int per, nt;
};

F64Shape f64_shape(const Layout& L) {
  const int64_t S = 2 * L.Umax + 1;
  if (S <= 1024) return {4, 512};
  if (S <= 4096) return {4, kT64};
  return {S <= 8192 ? 8 : 16, kT64};
}

hipError_t launch_f64_alpha(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(L.B > 0 ? L.B : 1);
  const F64Shape sh = f64_shape(L);
  if (sh.nt == 512) f64_alpha_kernel<4, 512><<<grid, 512, 0, s>>>(in, L, P);
  else if (sh.per == 4) f64_alpha_kernel<4, kT64><<<grid, kT64, 0, s>>>(in, L, P);
  else if (sh.per == 8) f64_alpha_kernel<8, kT64><<<grid, kT64, 0, s>>>(in, L, P);
  else f64_alpha_kernel<16, kT64><<<grid, kT64, 0, s>>>(in, L, P);
  return hipGetLastError();
}

hipError_t launch_f64_beta_rows(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s) {
  if (L.B == 0 || L.T_total == 0 || L.D == 0) return hipGetLastError();
  const F64Shape sh = f64_shape(L);
  // two copies of the class sums when they fit beside the kernel's static LDS (the boundary
  // exchange, 32 B per thread, and the wave totals)
  const size_t stat = 32 * (size_t)sh.nt + 256;
  const bool two = 2 * sizeof(double) * (size_t)(L.Umax + 1) + stat <= 160 * 1024;
  const size_t lds = (two ? 2 : 1) * sizeof(double) * (size_t)(L.Umax + 1);
  auto launch = [&](auto kernel, int nt) {
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    kernel<<<static_cast<unsigned>(L.B), nt, lds, s>>>(in, L, P, static_cast<double*>(grad_out), two ? 1 : 0);
    return hipGetLastError();
  };
  if (sh.nt == 512) return launch(&f64_beta_rows_kernel<4, 512>, 512);
  if (sh.per == 4) return launch(&f64_beta_rows_kernel<4, kT64>, kT64);
  if (sh.per == 8) return launch(&f64_beta_rows_kernel<8, kT64>, kT64);
  return launch(&f64_beta_rows_kernel<16, kT64>, kT64);
}

}  // namespace pctc
