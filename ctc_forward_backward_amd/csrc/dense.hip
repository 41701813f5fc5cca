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
//   - one wave per row (no workgroup barriers): the wave's lanes cover the utterance's state pairs
//     block by block, then stream the row;
//   - one pass over the stored alpha and beta: 2^(alpha + beta - lp) is taken relative to the
//     likelihood the alpha recursion reached (the block offsets of alpha and beta meet in that
//     constant, so every term is at most about 1); the class sums are accumulated unnormalised
//     and the frame's own total z of the terms scales them at the end, so the posteriors of every
//     frame sum to exactly the weight (the page's exp(alpha + beta - lp + nll) for a feasible
//     utterance, with the rounding drift of the recursions divided out);
//   - per-class sums go into an LDS array indexed by the class's rank among the utterance's
//     classes (at most U+1 entries); the row is then streamed once in aligned 16-byte chunks, eight
//     loads in flight per lane, and a per-utterance class bitmap (with per-word prefix counts) tells
//     which columns of a chunk carry a class and its rank, so the correction is applied in
//     registers before the single store.
#include "pctc_internal.h"

namespace pctc {

namespace {

constexpr int kBlocks = 4;  // state-pair blocks whose loads are issued together

template <int DT>
__global__ void __launch_bounds__(256) dense_kernel(Inputs in, Layout L, Pointers P, void* grad, int per_wave) {
  extern __shared__ uint32_t dsm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Dw = static_cast<int>(L.Dw);
  const int Ua = per_wave - 2 * Dw;
  float* acc = reinterpret_cast<float*>(dsm + wave * per_wave);
  uint32_t* bits = dsm + wave * per_wave + Ua;
  const int* pref = reinterpret_cast<const int*>(bits + Dw);
  const int64_t D = L.D, TT = L.T_total, Gm = L.Gmax;
  int cur_b = -1;

  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < TT; r += (int64_t)gridDim.x * 4) {
    const int b = P.rowmap[r];
    const float w = b >= 0 ? P.w[b] : 0.0f;
    const int64_t f0 = r * D, f1 = f0 + D;
    const bool feasible = b >= 0 && P.nll[b] < (double)INFINITY;  // false for no alignment and NaN input
    if (w == 0.0f || !feasible) {
      const float fill = w == 0.0f ? 0.0f : __builtin_nanf("");
      wave_segment<DT>(
          nullptr, f0, f1, lane,
          [&](int64_t q, int64_t, const float*) {
            const float v[8] = {fill, fill, fill, fill, fill, fill, fill, fill};
            store8<DT>(grad, q, v);
          },
          [&](int64_t f) { store_grad(grad, DT, f, fill); });
      continue;
    }
    if (b != cur_b) {  // this utterance's class bitmap and prefix counts into the wave's LDS
      const uint32_t* gb = P.cbits + (int64_t)b * Dw;
      const int* gp = P.cpref + (int64_t)b * Dw;
      for (int i = lane; i < Dw; i += 64) {
        bits[i] = gb[i];
        bits[Dw + i] = static_cast<uint32_t>(gp[i]);
      }
      cur_b = b;
    }
    const Meta m = P.meta[b];
    const int U = m.U, G = (U + 64) >> 6;
    const int64_t start = m.start, T = m.T;
    // each recursion block stores its offset once per chunk, at the row of the chunk's first frame
    const int64_t sa = r - start, sb = start + T - 1 - r;
    const int64_t rowa = sa == 0 ? -1 : start + 1 + ((sa - 1) / kChunk) * kChunk;
    const int64_t rowb = sb == 0 ? -1 : start + T - 1 - (1 + ((sb - 1) / kChunk) * kChunk);
    auto offA = [&](int j) { return rowa < 0 ? 0 : P.sig[j * TT + rowa]; };
    auto offB = [&](int j) { return rowb < 0 ? 0 : P.sig[(Gm + j) * TT + rowb]; };
    const double lsh = P.lsh[b];
    const float* Er = P.E + r * L.E_stride;
    const float eb = Er[0];
    const int* dmap = P.dmap + (int64_t)b * (L.Umax + 1);
    // LDS operations of one wave complete in order: zeroing, atomics and reads need no barrier
    for (int i = lane; i <= U; i += 64) acc[i] = 0.0f;

    float z = 0.0f, bsum = 0.0f;
    for (int j0 = 0; j0 < G; j0 += kBlocks) {
      // pair k = 64 j + lane: state 2k (blank) takes alpha at 2k and beta at 2k + 1; state 2k + 1
      // (label k + 1) alpha at 2k + 1 and beta at 2k + 2, which for lane 63 is the next block's first
      float2 a[kBlocks];
      float b0[kBlocks], b1[kBlocks], el[kBlocks], c0[kBlocks], c1[kBlocks];
      int d1[kBlocks];
#pragma unroll
      for (int u = 0; u < kBlocks; ++u) {
        const int j = j0 + u, k = 64 * j + lane;
        a[u] = make_float2(kNeg, kNeg);
        b0[u] = b1[u] = el[u] = 0.0f;
        c0[u] = c1[u] = 0.0f;
        d1[u] = 0;
        if (j < G) {
          const int oa = offA(j), ob0 = offB(j);
          const int ob1 = lane < 63 ? ob0 : (j + 1 < G ? offB(j + 1) : ob0);
          c0[u] = static_cast<float>((double)(oa + ob0) - lsh);
          c1[u] = static_cast<float>((double)(oa + ob1) - lsh);
          const int64_t rb = ((Gm + j) * TT + r) * 128;
          if (k <= U) {
            a[u] = *reinterpret_cast<const float2*>(P.AB + ((int64_t)j * TT + r) * 128 + 2 * lane);
            b0[u] = P.AB[rb + 2 * lane + 1];
          }
          if (k < U) {  // then for lane 63 the next block exists
            b1[u] = P.AB[lane < 63 ? rb + 2 * lane + 2 : rb + TT * 128];
            el[u] = Er[k + 1];
            d1[u] = dmap[k + 1];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kBlocks; ++u) {
        const int k = 64 * (j0 + u) + lane;
        // each term is at most about 1; the clamp only guards the exponent against garbage
        const float p0 = k <= U ? exp2_fast(fminf(a[u].x + b0[u] - eb + c0[u], 64.0f)) : 0.0f;
        const float p1 = k < U ? exp2_fast(fminf(a[u].y + b1[u] - el[u] + c1[u], 64.0f)) : 0.0f;
        z += p0 + p1;
        bsum += p0;
        if (k < U) atomicAdd(&acc[d1[u]], p1);
      }
    }
    z = wave_sum(z);
    bsum = wave_sum(bsum);
    if (lane == 0) atomicAdd(&acc[dmap[0]], bsum);
    const float scale = z > 0.0f ? w / z : 0.0f;

    // stream the row once: w * exp(lp) minus the class posterior at the columns that carry one
    auto rank = [&](int64_t c) {
      const int wi = static_cast<int>(c >> 5);
      return pref[wi] + __builtin_popcount(bits[wi] & ((1u << (c & 31)) - 1u));
    };
    auto has = [&](int64_t c) { return (bits[c >> 5] >> (c & 31)) & 1u; };
    wave_segment<DT>(
        in.log_probs, f0, f1, lane,
        [&](int64_t q, int64_t f, const float* x) {
          float v[8];
          const int64_t c0 = f - f0;
          const int wi = static_cast<int>(c0 >> 5), sh = static_cast<int>(c0 & 31);
          uint32_t m8 = bits[wi] >> sh;
          if (sh > 24 && wi + 1 < Dw) m8 |= bits[wi + 1] << (32 - sh);
          m8 &= 0xffu;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = w * exp2_fast(x[e] * kLog2e);
          while (m8) {
            const int e = __builtin_ctz(m8);
            m8 &= m8 - 1;
            v[e] -= acc[rank(c0 + e)] * scale;
          }
          store8<DT>(grad, q, v);
        },
        [&](int64_t f) {
          const int64_t c = f - f0;
          float g = w * exp2_fast(load_lp(in.log_probs, DT, f) * kLog2e);
          if (has(c)) g -= acc[rank(c)] * scale;
          store_grad(grad, DT, f, g);
        });
  }
}

}  // namespace

hipError_t launch_dense(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s) {
  if (L.T_total == 0 || L.D == 0) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // per wave: the class accumulators (U+1, rounded to 4), the class bitmap and its prefix counts
  const int per_wave = static_cast<int>(((L.Umax + 1 + 3) / 4) * 4 + 2 * L.Dw);
  const size_t lds = 4 * sizeof(uint32_t) * (size_t)per_wave;
  const int64_t want = (L.T_total + 3) / 4;
  const int grid = static_cast<int>(want < 4 * (int64_t)cus ? want : 4 * (int64_t)cus);
  auto launch = [&](auto kernel) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
    kernel<<<grid, 256, lds, s>>>(in, L, P, grad_out, per_wave);
    return hipGetLastError();
  };
  if (in.dtype == kF32) return launch(&dense_kernel<kF32>);
  if (in.dtype == kF16) return launch(&dense_kernel<kF16>);
  return launch(&dense_kernel<kBF16>);
}

}  // namespace pctc
