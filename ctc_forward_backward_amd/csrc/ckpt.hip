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
// Design for gfx950: one 4-wave workgroup per (utterance, K-step interval); the target's 64-pair
// state blocks (up to 16: targets of up to 1023 labels) are dealt to the waves in turn, so a short
// target puts one block on each wave and a long one gives each wave up to four to interleave, rather
// than one wave per block with most of them idle in the barriers.  Each step, block j-1 hands its
// highest label to block j through LDS, and every lane renormalises its pair by its own integer
// offset.  What a step reads (the frame's emissions and beta) does not depend on the recursion, so
// it is loaded two steps ahead, beta's offsets once per interval, and the step's one barrier orders
// LDS only: a step waits for no memory round trip.  Each row's posteriors are then formed as in the
// full-storage pass: 2^(alpha + beta) relative to the likelihood, blank states summed per wave,
// label states added into LDS class sums by rank, normalised by the frame's own total and written as
// the row's compact class sums.  Measured, the pass issues about half the vector instructions the
// chip can and moves about a quarter of the bytes it can: what limits it is each step's chain of
// dependent operations (the log-sum-exps, the wave sums, the barrier).
#include <algorithm>

#include "rows.h"

namespace pctc {

namespace {

// NW waves per workgroup, NB state blocks per wave: wave w holds the blocks w, w + NW, w + 2 NW, ...
// (a short target spreads over the waves, a long one gives each wave several blocks to interleave)
template <int NW, int NB>
__global__ void __launch_bounds__(64 * NW) ckpt_posterior_kernel(Layout L, Pointers P, int group) {
  if (skipped(P)) return;
  constexpr int NJ = NW * NB;
  extern __shared__ float cacc[];  // 2 x C_stride floats: a row's class sums by rank, by step parity
  __shared__ float edge_v[2][NJ];
  __shared__ int edge_o[2][NJ];
  __shared__ float zred[2][NW];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = static_cast<int>(L.K);
  const int64_t TT = L.T_total, NC = L.NCH, Es = L.E_stride, Gm = L.Gmax;
  const int B = static_cast<int>(L.B);
  const int total = P.qbase[B];
  const int64_t Cs = L.C_stride;
  for (int i = tid; i < 2 * Cs; i += blockDim.x) cacc[i] = 0.0f;
  __syncthreads();
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // the utterance of this slot: the last b with qbase[b] <= item (qbase[0] = 0, qbase[B] = total),
    // for up to 255 utterances by counting the entries <= item over the wave in one round trip
    int b;
    if (B < 256) {
      int qv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) qv[c] = P.qbase[min(64 * c + lane, B)];  // (all issued at once)
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) cnt += __popcll(__ballot(64 * c + lane <= B && qv[c] <= item));
      b = cnt - 1;
    } else {
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (P.qbase[mid] <= item) lo = mid;
        else hi = mid - 1;
      }
      b = lo;
    }
    b = __builtin_amdgcn_readfirstlane(b);
    // everything the slot needs from b, loaded together (b >= 0: qbase[0] = 0 <= item)
    const Meta m = P.meta[b];
    const int qb = P.qbase[b], cb0 = P.cbase[b];
    const double lsh = P.lsh[b], nll = P.nll[b];
    const float wgt = P.w[b];
    const int gb = P.gid[b];
    // (uniform) a zero weight or an infinite loss: the gradient kernel fills these rows; another
    // group's utterance: its own launch takes it
    if (wgt == 0.0f || !(nll < (double)INFINITY) || (group >= 0 && gb != group)) continue;
    const int U = m.U, G = (U + 64) >> 6, T = m.T;
    // the likelihood as an integer and a fraction in [0, 1): the offsets are integers, so a state's
    // shift off + ob - lsh is formed exactly in integers and rounded once
    const double lfl = floor(lsh);
    const int lsh_i = static_cast<int>(lfl);
    const float lsh_f = static_cast<float>(lsh - lfl);
    const int q = item - qb;
    const int s0 = q * K, s1 = min(s0 + K, T) - 1;
    const int* lab = P.lab + (int64_t)b * (L.Umax + 1);
    const int* dmap = P.dmap + (int64_t)b * (L.Umax + 1);
    const int dblank = dmap[0];
    // per block i of this wave (j = w + NW i): whether it exists (uniform), and this lane's state pair
    // (2k, 2k+1): the label's skip, its emission column, its class rank; the neighbour pair's block
    // and lane (lane 63: lane 0 of the next block, if any)
    bool act[NB], sk[NB];
    int eidx[NB], d1[NB], jn[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = w + NW * i, k = 64 * j + lane;
      act[i] = j < G;
      const bool vl = act[i] && k < U;
      // (loaded for every lane, at an index inside the utterance's U + 1 entries, then selected)
      const int l1 = lab[min(k + 1, U)], l0 = lab[min(k, U)], dm = dmap[min(k + 1, U)];
      sk[i] = vl && k >= 1 && l1 != l0;
      eidx[i] = vl ? k + 1 : U + 1;
      d1[i] = vl ? dm : 0;
      jn[i] = lane < 63 ? j : min(j + 1, G - 1);
    }
    const int ln = lane < 63 ? lane + 1 : 0;
    // beta's offsets (per 32-frame chunk of steps counted from the end): the interval's K <= 32 steps
    // meet at most two chunks, the first step's and the last's, both loaded here (the slot index
    // stays in range: the table has a spare slot past the last utterance's); the last frame has none
    const int chA = T - 1 - s0 > 0 ? (T - 2 - s0) / kChunk : 0;
    const int chB = T - 1 - s1 > 0 ? (T - 2 - s1) / kChunk : 0;
    int oA0[NB], oA1[NB], oB0[NB], oB1[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = act[i] ? w + NW * i : 0, jj = act[i] ? jn[i] : 0;
      oA0[i] = P.sig[((Gm + j) * NC + cb0 + chA) * 64 + lane];
      oA1[i] = P.sig[((Gm + jj) * NC + cb0 + chA) * 64 + ln];
      oB0[i] = P.sig[((Gm + j) * NC + cb0 + chB) * 64 + lane];
      oB1[i] = P.sig[((Gm + jj) * NC + cb0 + chB) * 64 + ln];
    }
    // what a step reads, none of it from the recursion: fetched two steps ahead into one of four
    // register sets taken in turn (no set is copied into another, so no copy waits for a load), so
    // that a step waits for no memory round trip of its own
    struct StepIn {
      float eb;
      float el[NB], b0[NB], b1[NB];
    };
    auto fetch = [&](int st, StepIn& v) {
      const int64_t r = m.start + st;
      v.eb = P.Eb[r];
      // every step issues the same loads (a block past the target reads block 0's, unused), so that
      // the wait for a set counts the loads issued after it exactly
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int j = act[i] ? w + NW * i : 0, jj = act[i] ? jn[i] : 0;
        v.el[i] = P.E[r * Es + eidx[i]];
        const int64_t rb = ((int64_t)j * TT + r) * 128;
        v.b0[i] = P.ABb[rb + 2 * lane + 1];
        v.b1[i] = P.ABb[lane < 63 ? rb + 2 * lane + 2 : (jj > j ? rb + TT * 128 : rb)];
      }
    };
    // alpha at the kept step s0, in its lane's offset for that step's chunk
    float xb[NB], xl[NB], off[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      // (a block past the target reads block 0's; the slot is in range for s0 = 0 too: the table
      // has a spare slot past the last utterance's)
      const int j = act[i] ? w + NW * i : 0;
      const float2 v = *reinterpret_cast<const float2*>(P.ABa + ((int64_t)j * L.NQ + item) * 128 + 2 * lane);
      const int o = P.sig[((int64_t)j * NC + cb0 + (s0 > 0 ? (s0 - 1) / kChunk : 0)) * 64 + lane];
      xb[i] = act[i] ? v.x : kNeg;
      xl[i] = act[i] ? v.y : kNeg;
      off[i] = act[i] && s0 > 0 ? static_cast<float>(o) : 0.0f;
    }
    StepIn R[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      R[a].eb = kNeg;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        R[a].el[i] = R[a].b0[i] = R[a].b1[i] = kNeg;
      }
    }
    fetch(s0, R[0]);
    fetch(min(s0 + 1, s1), R[1]);
    // one barrier per step: a step's LDS (class sums, wave totals, handed-on labels) alternates
    // between two copies by the step's parity, so step st+1 fills the other copy while step st's
    // sums are still being written out
    auto step = [&](int st, const StepIn& cur, StepIn& ahead) {
      fetch(min(st + 2, s1), ahead);
      const int64_t r = m.start + st;
      const int par = st & 1;
      float* acc = cacc + par * Cs;
      if (st > s0) {
        // one alpha step: the neighbour label of each block's lane 0 comes from block j-1, as the
        // previous step left it in LDS
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (!act[i]) continue;  // (uniform)
          const int j = w + NW * i;
          float hin = kNeg;
          if (j > 0) hin = edge_v[par ^ 1][j - 1] + (static_cast<float>(edge_o[par ^ 1][j - 1]) - off[i]);
          const float shift = dpp_f32<0x138>(off[i], off[i]) - off[i];  // lane 0: 0
          const float n = dpp_f32<0x138>(hin, xl[i]) + shift;
          const float t = lse2(xb[i], n);
          const float a2 = sk[i] ? t : xb[i];
          xb[i] = t + cur.eb;
          xl[i] = lse2(xl[i], a2) + cur.el[i];
          const float mx = fmaxf(xb[i], xl[i]);
          const float d = mx > kNegHalf ? floorf(mx) : 0.0f;
          xb[i] -= d;
          xl[i] -= d;
          off[i] += d;
        }
      }
      // this step's highest label of each block, for the next step of the block above
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (act[i] && lane == 63) {
          edge_v[par][w + NW * i] = xl[i];
          edge_o[par][w + NW * i] = static_cast<int>(off[i]);
        }
      }
      // the row's posteriors: beta (and its offsets) as stored, this alpha, relative to the likelihood
      const bool lastf = st == T - 1;  // beta of the last frame is stored without an offset
      const bool inA = lastf || (T - 2 - st) / kChunk == chA;
      float z = 0.0f, bsum = 0.0f;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (!act[i]) continue;  // (uniform)
        const int k = 64 * (w + NW * i) + lane;
        const int oi = static_cast<int>(off[i]) - lsh_i;
        const int ob0 = lastf ? 0 : inA ? oA0[i] : oB0[i], ob1 = lastf ? 0 : inA ? oA1[i] : oB1[i];
        const float c0 = static_cast<float>(oi + ob0) - lsh_f;
        const float c1 = static_cast<float>(oi + ob1) - lsh_f;
        if (k <= U) {
          const float p0 = exp2_fast(fminf(xb[i] + cur.b0[i] + c0, 64.0f));
          z += p0;
          bsum += p0;
        }
        if (k < U) {
          const float p1 = exp2_fast(fminf(xl[i] + cur.b1[i] + c1, 64.0f));
          z += p1;
          atomicAdd(&acc[d1[i]], p1);
        }
      }
      z = wave_sum(z);
      bsum = wave_sum(bsum);
      if (lane == 0) {
        zred[par][w] = z;
        if (act[0]) atomicAdd(&acc[dblank], bsum);
      }
      lds_barrier();
      float ztot = 0.0f;
      for (int i = 0; i < NW; ++i) ztot += zred[par][i];  // fixed order
      const float scale = ztot > 0.0f ? 1.0f / ztot : 0.0f;  // (the gradient rows apply the weight)
      float* out = P.post + r * Cs;
      for (int i = tid; i <= U; i += 64 * NW) {
        out[i] = acc[i] * scale;
        acc[i] = 0.0f;
      }
    };
    for (int st = s0; st <= s1; st += 4) {
      step(st, R[0], R[2]);
      if (st + 1 <= s1) step(st + 1, R[1], R[3]);
      if (st + 2 <= s1) step(st + 2, R[2], R[0]);
      if (st + 3 <= s1) step(st + 3, R[3], R[1]);
    }
    lds_barrier();  // the last step's sums are written out before the next item fills either copy
  }
}

}  // namespace

hipError_t launch_ckpt_posteriors(const Inputs& in, const Layout& L, const Pointers& P, int group, hipStream_t s) {
  (void)in;
  if (L.T_total == 0 || L.B == 0) return hipGetLastError();
  const size_t lds = 2 * sizeof(float) * (size_t)L.C_stride;
  const int64_t grid = std::min<int64_t>(L.NQ, 4096);
  const unsigned g = static_cast<unsigned>(grid > 0 ? grid : 1);
  auto go = [&](auto kern, int nw) {
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    kern<<<g, 64 * nw, lds, s>>>(L, P, group);
    return hipGetLastError();
  };
  // four waves; each holds up to four of the (at most 16) blocks
  static_assert(4 * 4 >= kMaxCheckpointBlocks, "four waves of four blocks cover a checkpointed target");
  if (L.Gmax <= 4) return go(&ckpt_posterior_kernel<4, 1>, 4);
  if (L.Gmax <= 8) return go(&ckpt_posterior_kernel<4, 2>, 4);
  if (L.Gmax <= 12) return go(&ckpt_posterior_kernel<4, 3>, 4);
  return go(&ckpt_posterior_kernel<4, 4>, 4);
}

}  // namespace pctc
