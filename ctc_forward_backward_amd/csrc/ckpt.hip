// Posteriors of the rows when alpha is kept only every K-th step (alpha checkpointing).
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities", Triton file: `_alpha_kernel` stores every alpha row in a (T_total, S_max) buffer
// that `_beta_grad_kernel` reads back while it forms the posteriors exp(alpha + beta - lp + nll).
// Here the alpha recursion keeps only the steps 0, K, 2K, ... of each utterance, and the rows of the
// K steps that follow a kept one are formed by recomputing alpha from it: alpha[t][s] is the
// log-sum-exp of alpha[t-1] at s, s-1 and, into a label whose id differs from the one two states
// back, s-2, plus the frame's log probability at the state's class (the same recursion, the same
// emission table).  Beta is kept for every step as in the full-storage mode.
//
// Design for gfx950: one workgroup per (utterance, K-step interval), one wave per 64-pair state
// block (up to 16 blocks: targets of up to 1023 labels); each step, block j-1 hands its highest
// label to block j through LDS, and every lane renormalises its pair by its own integer offset.
// Each row's posteriors are then formed as in the full-storage pass: 2^(alpha + beta) relative to
// the likelihood, blank states summed per wave, label states added into LDS class sums by rank,
// normalised by the frame's own total and written as the row's compact class sums.
#include <algorithm>

#include "rows.h"

namespace pctc {

namespace {

constexpr int kCkWaves = kMaxCheckpointBlocks;

__global__ void __launch_bounds__(64 * kCkWaves) ckpt_posterior_kernel(Layout L, Pointers P) {
  if (skipped(P)) return;
  extern __shared__ float cacc[];  // C_stride floats: the current row's class sums by rank
  __shared__ float edge_v[2][kCkWaves];
  __shared__ int edge_o[2][kCkWaves];
  __shared__ float zred[kCkWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = static_cast<int>(L.K);
  const int64_t TT = L.T_total, NC = L.NCH, Es = L.E_stride;
  const int B = static_cast<int>(L.B);
  const int total = P.qbase[B];
  for (int i = tid; i < L.C_stride; i += blockDim.x) cacc[i] = 0.0f;
  __syncthreads();
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // the utterance of this slot: the last b with qbase[b] <= item
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (P.qbase[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int b = __builtin_amdgcn_readfirstlane(lo);
    float wgt;
    if (!rows::row_live(P, b, wgt)) continue;  // (uniform) the gradient kernel fills these rows
    const Meta m = P.meta[b];
    const int U = m.U, G = (U + 64) >> 6, T = m.T;
    const int q = item - P.qbase[b];
    const int s0 = q * K, s1 = min(s0 + K, T) - 1;
    const int j = w, k = 64 * j + lane;
    const bool act = j < G;
    const int* lab = P.lab + (int64_t)b * (L.Umax + 1);
    const int* dmap = P.dmap + (int64_t)b * (L.Umax + 1);
    const int cb0 = P.cbase[b];
    const double lsh = P.lsh[b];
    // this lane's state pair (2k, 2k+1): whether the label exists, its skip, its emission column
    const bool vl = act && k < U;
    const bool sk = vl && k >= 1 && lab[k + 1] != lab[k];
    const int eidx = vl ? k + 1 : U + 1;
    const int d1 = vl ? dmap[k + 1] : 0;
    // alpha at the kept step s0, in its lane's offset for that step's chunk
    float xb = kNeg, xl = kNeg, off = 0.0f;
    if (act) {
      const float2 v = *reinterpret_cast<const float2*>(P.ABa + ((int64_t)j * L.NQ + P.qbase[b] + q) * 128 + 2 * lane);
      xb = v.x;
      xl = v.y;
      if (s0 > 0) off = static_cast<float>(P.sig[((int64_t)j * NC + cb0 + (s0 - 1) / kChunk) * 64 + lane]);
    }
    for (int st = s0; st <= s1; ++st) {
      const int64_t r = m.start + st;
      if (st > s0) {
        // one alpha step: the neighbour label of lane 0 comes from block j-1 through LDS
        const int par = st & 1;
        if (act && lane == 63) {
          edge_v[par][j] = xl;
          edge_o[par][j] = static_cast<int>(off);
        }
        __syncthreads();
        float hin = kNeg;
        if (act && j > 0) hin = edge_v[par][j - 1] + (static_cast<float>(edge_o[par][j - 1]) - off);
        const float shift = dpp_f32<0x138>(off, off) - off;  // lane 0: 0
        const float n = dpp_f32<0x138>(hin, xl) + shift;
        const float el = act ? P.E[r * Es + eidx] : kNeg;
        const float eb = P.Eb[r];
        const float t = lse2(xb, n);
        const float nb = t + eb;
        const float a2 = sk ? t : xb;
        const float nl = lse2(xl, a2) + el;
        xb = act ? nb : kNeg;
        xl = act ? nl : kNeg;
        const float mx = fmaxf(xb, xl);
        const float d = mx > kNegHalf ? floorf(mx) : 0.0f;
        xb -= d;
        xl -= d;
        off += d;
      }
      // the row's posteriors: beta (and its offsets) as stored, this alpha, relative to the likelihood
      float z = 0.0f, bsum = 0.0f;
      if (act) {
        const int sb = T - 1 - st;
        const int64_t slotB = sb == 0 ? -1 : cb0 + (sb - 1) / kChunk;
        const int jn = lane < 63 ? j : min(j + 1, G - 1), ln = lane < 63 ? lane + 1 : 0;
        const int ob0 = slotB < 0 ? 0 : P.sig[((L.Gmax + j) * NC + slotB) * 64 + lane];
        const int ob1 = slotB < 0 ? 0 : P.sig[((L.Gmax + jn) * NC + slotB) * 64 + ln];
        const int64_t rb = ((int64_t)j * TT + r) * 128;
        const float c0 = static_cast<float>((double)off + (double)ob0 - lsh);
        const float c1 = static_cast<float>((double)off + (double)ob1 - lsh);
        if (k <= U) {
          const float p0 = exp2_fast(fminf(xb + P.ABb[rb + 2 * lane + 1] + c0, 64.0f));
          z += p0;
          bsum += p0;
        }
        if (k < U) {
          const float p1 = exp2_fast(fminf(xl + P.ABb[lane < 63 ? rb + 2 * lane + 2 : rb + TT * 128] + c1, 64.0f));
          z += p1;
          atomicAdd(&cacc[d1], p1);
        }
      }
      z = wave_sum(z);
      bsum = wave_sum(bsum);
      if (lane == 0) {
        zred[w] = z;
        if (act) atomicAdd(&cacc[dmap[0]], bsum);
      }
      __syncthreads();
      float ztot = 0.0f;
      for (int i = 0; i < kCkWaves; ++i) ztot += zred[i];  // fixed order
      const float scale = ztot > 0.0f ? 1.0f / ztot : 0.0f;  // (the gradient rows apply the weight)
      float* out = P.post + r * L.C_stride;
      for (int i = tid; i <= U; i += blockDim.x) {
        out[i] = cacc[i] * scale;
        cacc[i] = 0.0f;
      }
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_ckpt_posteriors(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s) {
  (void)in;
  if (L.T_total == 0 || L.B == 0) return hipGetLastError();
  const size_t lds = sizeof(float) * (size_t)L.C_stride;
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ckpt_posterior_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const int64_t grid = std::min<int64_t>(L.NQ, 4096);
  ckpt_posterior_kernel<<<static_cast<unsigned>(grid > 0 ? grid : 1), 64 * kCkWaves, lds, s>>>(L, P);
  return hipGetLastError();
}

}  // namespace pctc
