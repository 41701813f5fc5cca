// Posteriors and the dense gradient rows of packed CTC.
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities", Triton file, `_beta_grad_kernel` and `_PackedCTCLoss.backward`: the posterior of
// state s at frame t is exp(alpha + beta - lp + nll) scaled by the utterance's gradient weight and
// formed only when that weight is non-zero; each gradient row is weight * exp(lp) minus the
// posteriors summed per class (blank states at the blank column, label states at their label's
// column); rows owned by no utterance are zero; the row is stored in the dtype of the log probs.
//
// Design for gfx950:
//   - one workgroup per row at a time (grid-stride), 256 threads;
//   - posteriors are formed as the per-frame softmax over states of alpha + beta - lp (equal to the
//     page's exp(alpha + beta - lp + nll) for a feasible utterance, since the sum over states of
//     alpha*beta/p is the likelihood at every frame); this removes nll and every per-frame shift
//     of the recursions from the exponent, so the float32 exponent stays small;
//   - per-class sums go into a D-float LDS accumulator with LDS float atomics, then the row is
//     streamed once, coalesced, reading log_probs and writing the gradient in its dtype.
#include "pctc_internal.h"

namespace pctc {

namespace {

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  lds_barrier();
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  float r = 0.0f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += red[i];
  lds_barrier();
  return r;
}

__global__ void __launch_bounds__(256) dense_kernel(Inputs in, Layout L, Pointers P, void* grad) {
  extern __shared__ float acc[];  // D floats
  __shared__ float red[16];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int64_t D = L.D;
  for (int64_t r = blockIdx.x; r < L.T_total; r += gridDim.x) {
    const int b = P.rowmap[r];
    const float w = b >= 0 ? P.w[b] : 0.0f;
    const int64_t base = r * D;
    if (w == 0.0f) {
      for (int64_t c = tid; c < D; c += nthr) store_grad(grad, in.dtype, base + c, 0.0f);
      continue;
    }
    const double nll = P.nll[b];
    if (!(nll < (double)INFINITY)) {  // no alignment (or NaN input) with a non-zero weight
      for (int64_t c = tid; c < D; c += nthr) store_grad(grad, in.dtype, base + c, __builtin_nanf(""));
      continue;
    }
    const int U = P.meta[b].U, S = 2 * U + 1;
    const int64_t Gm = L.Gmax, TT = L.T_total;
    const float* Er = P.E + r * L.E_stride;
    const int* lab = P.lab + (int64_t)b * (L.Umax + 1);
    // alpha of state s: block ja = (s/2)/64, position s - 128 ja; beta of state s: block
    // jb = ((s+1)/2)/64, position s + 1 - 128 jb.  Each block's integer offset is brought to a common
    // reference exactly before it meets the float values.
    // each block stores its offset once per chunk, at the row of the chunk's first frame; frame 0
    // of either recursion has offset 0
    const int64_t start = P.meta[b].start, Tb = P.meta[b].T;
    const int sa = static_cast<int>(r - start), sb = static_cast<int>(start + Tb - 1 - r);
    const int64_t rowa = sa == 0 ? -1 : start + 1 + ((sa - 1) / kChunk) * kChunk;
    const int64_t rowb = sb == 0 ? -1 : start + Tb - 1 - (1 + ((sb - 1) / kChunk) * kChunk);
    auto ioff = [&](int s) {
      const int ja = (s >> 1) >> 6, jb = ((s + 1) >> 1) >> 6;
      return (rowa < 0 ? 0 : P.sig[ja * TT + rowa]) + (rowb < 0 ? 0 : P.sig[(Gm + jb) * TT + rowb]);
    };
    auto xval = [&](int s, int iref) {
      const int ja = (s >> 1) >> 6, jb = ((s + 1) >> 1) >> 6;
      const float a = P.AB[(ja * TT + r) * 128 + (s - 128 * ja)];
      const float bt = P.AB[((Gm + jb) * TT + r) * 128 + (s + 1 - 128 * jb)];
      return (a + bt - Er[(s & 1) ? ((s + 1) >> 1) : 0]) + static_cast<float>(ioff(s) - iref);
    };

    for (int64_t c = tid; c < D; c += nthr) acc[c] = 0.0f;
    float im = kNeg;
    for (int s = tid; s < S; s += nthr) im = fmaxf(im, static_cast<float>(ioff(s)));
    const int iref = static_cast<int>(block_max(im, red));  // also orders the accumulator zeroing
    float mx = kNeg;
    for (int s = tid; s < S; s += nthr) mx = fmaxf(mx, xval(s, iref));
    mx = block_max(mx, red);
    float z = 0.0f;
    for (int s = tid; s < S; s += nthr) z += exp2_fast(xval(s, iref) - mx);
    z = block_sum(z, red);
    const float scale = (mx > kNegHalf && z > 0.0f) ? w / z : 0.0f;
    float bsum = 0.0f;
    for (int s = tid; s < S; s += nthr) {
      const float g = exp2_fast(xval(s, iref) - mx) * scale;
      if (s & 1) {
        atomicAdd(&acc[lab[(s + 1) >> 1]], g);
      } else {
        bsum += g;
      }
    }
    bsum = block_sum(bsum, red);
    if (tid == 0) acc[in.blank] += bsum;
    lds_barrier();
    for (int64_t c = tid; c < D; c += nthr) {
      const float p = exp2_fast(load_lp(in.log_probs, in.dtype, base + c) * kLog2e);
      store_grad(grad, in.dtype, base + c, w * p - acc[c]);
    }
    lds_barrier();
  }
}

}  // namespace

hipError_t launch_dense(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s) {
  if (L.T_total == 0 || L.D == 0) return hipSuccess;
  const size_t lds = (size_t)L.D * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  int64_t grid = L.T_total < 2048 ? L.T_total : 2048;
  dense_kernel<<<static_cast<unsigned>(grid), 256, lds, s>>>(in, L, P, grad_out);
  return hipGetLastError();
}

}  // namespace pctc
