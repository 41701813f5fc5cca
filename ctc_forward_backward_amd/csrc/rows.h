// Per-row work of the packed CTC gradient: the posteriors of one row (class sums) and the gradient
// row itself.  Device functions only: the standalone row kernels and the persistent worker that
// overlaps them with the recursions both call these.
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities", Triton file, `_beta_grad_kernel` and `_PackedCTCLoss.backward`: the posterior of
// state s at frame t is exp(alpha + beta - lp + nll), formed only when the utterance's gradient weight
// is non-zero; each gradient row is the weight times exp(lp) minus the posteriors summed per class
// (blank states at the blank column, label states at their label's column); rows owned by no
// utterance are zero; the row is stored in the dtype of the log probs.  Here the class sums in P.post
// are kept without the weight (a split forward forms them before the weight is known); the gradient
// row scales them by it as it loads them.
//
// Design for gfx950:
//   - posterior_row: one pass over the stored alpha and beta (beta is stored without the frame's
//     own emission, so alpha + beta is already alpha + beta - lp), 2^(alpha + beta) taken relative
//     to the likelihood the alpha recursion reached (the per-lane offsets of alpha and beta meet in
//     that constant, so every term is at most about 1).  Blank states are summed in registers,
//     label states added into an LDS array indexed by the rank of their class among the
//     utterance's classes (at most U+1 entries).  The frame's own total z of the terms normalises
//     them, so the posteriors of every frame sum to exactly the weight (the page's
//     exp(alpha + beta - lp + nll) for a feasible utterance, with the rounding drift of the
//     recursions divided out).  The row's class sums, times w / z, are written compactly: U+1
//     floats per row.
//   - dense_row: the row in batches of aligned 16-byte chunks (the first batch loaded together with
//     the row's compact class sums); the row is streamed once, and a per-utterance class bitmap with
//     per-word prefix counts (in LDS) tells which columns of a chunk carry a class and its rank,
//     so the correction is applied in registers before the single store.
#pragma once

#include "pctc_internal.h"

namespace pctc {
namespace rows {

constexpr int kBlocks = 4;  // state-pair blocks whose loads are issued together
constexpr int kLook = 4;    // row chunks whose class lookups are issued together
constexpr int kPost = 8;    // compact class sums per lane held in registers (U+1 <= 512)

// aligned 8-element row chunks per lane loaded at once (the default).  Four, not a whole row: fewer
// registers let more waves stream rows side by side, which measured faster than more bytes in flight
// per wave (a large-vocabulary group: 139 us at 4 chunks, 136 at 8, 153 at 16).  The streamed
// kernel takes 8 for 16-bit rows of 4096 classes or more, where its registers allow it.
template <int DT>
constexpr int row_batch() { return 4; }

// a row gets a gradient from its utterance only if the utterance has a non-zero weight and an
// alignment (a NaN input makes the loss NaN, which also fails the test)
__device__ __forceinline__ bool row_live(const Pointers& P, int b, float& w) {
  w = b >= 0 ? P.w[b] : 0.0f;
  return w != 0.0f && b >= 0 && P.nll[b] < (double)INFINITY;
}

// class sums of row r of live utterance b (weight w) into P.post; acc: this wave's LDS (C_stride)
__device__ __forceinline__ void posterior_row(const Layout& L, const Pointers& P, float* acc, int64_t r, int b,
                                              int lane) {
  const int64_t TT = L.T_total, Gm = L.Gmax;
  const Meta m = P.meta[b];
  const int U = m.U, G = (U + 64) >> 6;
  const int64_t start = m.start, T = m.T;
  // every lane of a recursion block stores its offset once per chunk; the first frame (step 0) has
  // offset 0
  const int64_t sa = r - start, sb = start + T - 1 - r;
  const int64_t NC = L.NCH, cb0 = P.cbase[b];
  const int64_t slotA = sa == 0 ? -1 : cb0 + (sa - 1) / kChunk;
  const int64_t slotB = sb == 0 ? -1 : cb0 + (sb - 1) / kChunk;
  auto offA = [&](int j, int ln) { return slotA < 0 ? 0 : P.sig[((int64_t)j * NC + slotA) * 64 + ln]; };
  auto offB = [&](int j, int ln) { return slotB < 0 ? 0 : P.sig[((Gm + j) * NC + slotB) * 64 + ln]; };
  const double lsh = P.lsh[b];
  const int* dmap = P.dmap + (int64_t)b * (L.Umax + 1);
  // LDS operations of one wave complete in order: zeroing, atomics and reads need no barrier
  for (int i = lane; i <= U; i += 64) acc[i] = 0.0f;

  float z = 0.0f, bsum = 0.0f;
  for (int j0 = 0; j0 < G; j0 += kBlocks) {
    // pair k = 64 j + lane: state 2k (blank) takes alpha at 2k and beta at 2k + 1; state 2k + 1
    // (label k + 1) alpha at 2k + 1 and beta at 2k + 2, which for lane 63 is the next block's first
    float2 a[kBlocks];
    float b0[kBlocks], b1[kBlocks], c0[kBlocks], c1[kBlocks];
    int d1[kBlocks];
#pragma unroll
    for (int u = 0; u < kBlocks; ++u) {
      const int j = j0 + u, k = 64 * j + lane;
      a[u] = make_float2(kNeg, kNeg);
      b0[u] = b1[u] = 0.0f;
      c0[u] = c1[u] = 0.0f;
      d1[u] = 0;
      if (j < G) {
        // state 2k: alpha and beta of this lane; state 2k+1: alpha of this lane, beta of the next
        const int oa = offA(j, lane), ob0 = offB(j, lane);
        const int ob1 = lane < 63 ? offB(j, lane + 1) : (j + 1 < G ? offB(j + 1, 0) : ob0);
        c0[u] = static_cast<float>((double)(oa + ob0) - lsh);
        c1[u] = static_cast<float>((double)(oa + ob1) - lsh);
        const int64_t rb = ((int64_t)j * TT + r) * 128;
        if (k <= U) {
          a[u] = *reinterpret_cast<const float2*>(P.ABa + rb + 2 * lane);
          b0[u] = P.ABb[rb + 2 * lane + 1];
        }
        if (k < U) {  // then for lane 63 the next block exists
          b1[u] = P.ABb[lane < 63 ? rb + 2 * lane + 2 : rb + TT * 128];
          d1[u] = dmap[k + 1];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kBlocks; ++u) {
      const int k = 64 * (j0 + u) + lane;
      // each term is at most about 1; the clamp only guards the exponent against garbage
      const float p0 = k <= U ? exp2_fast(fminf(a[u].x + b0[u] + c0[u], 64.0f)) : 0.0f;
      const float p1 = k < U ? exp2_fast(fminf(a[u].y + b1[u] + c1[u], 64.0f)) : 0.0f;
      z += p0 + p1;
      bsum += p0;
      if (k < U) atomicAdd(&acc[d1[u]], p1);
    }
  }
  z = wave_sum(z);
  bsum = wave_sum(bsum);
  if (lane == 0) atomicAdd(&acc[dmap[0]], bsum);
  const float scale = z > 0.0f ? 1.0f / z : 0.0f;
  float* out = P.post + r * L.C_stride;
  for (int i = lane; i <= U; i += 64) out[i] = acc[i] * scale;
}

// device-scope loads (sc1): they read the device-coherent copy, never a line an earlier access left
// in a cache, so data that recursions on other compute units stored and then published is seen
// without a cache invalidation on the reading side
__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__builtin_bit_cast(float, static_cast<uint32_t>(v)), __builtin_bit_cast(float, static_cast<uint32_t>(v >> 32)));
}

// Streamed pipeline: the posteriors of row r of utterance b while the recursions may still be running
// (the band scheduler has seen both pass this frame).  The likelihood is not known yet, so the
// exponent reference is an integer found on the way: the first batch of blocks with mass sets it at
// its largest term, a later batch with a larger term raises it and scales the sums so far down.  The
// states and the per-lane offsets are read with device-scope loads (ld_dev).  Leaves the row's class
// sums times w / z in acc (U+1 floats, by class rank; w = 1: the sums alone); false when the frame
// carries no mass (the utterance has no alignment).
__device__ __forceinline__ bool posterior_stream(const Layout& L, const Pointers& P, float* acc, int64_t r, int b,
                                                 float w, int lane) {
  const int64_t TT = L.T_total, Gm = L.Gmax;
  const Meta m = P.meta[b];
  const int U = m.U, G = (U + 64) >> 6;
  const int64_t start = m.start, T = m.T;
  const int64_t sa = r - start, sb = start + T - 1 - r;
  const int64_t NC = L.NCH, cb0 = P.cbase[b];
  const int64_t slotA = sa == 0 ? -1 : cb0 + (sa - 1) / kChunk;
  const int64_t slotB = sb == 0 ? -1 : cb0 + (sb - 1) / kChunk;
  auto offA = [&](int j, int ln) { return slotA < 0 ? 0 : ld_dev(P.sig + ((int64_t)j * NC + slotA) * 64 + ln); };
  auto offB = [&](int j, int ln) { return slotB < 0 ? 0 : ld_dev(P.sig + ((Gm + j) * NC + slotB) * 64 + ln); };
  const int* dmap = P.dmap + (int64_t)b * (L.Umax + 1);
  for (int i = lane; i <= U; i += 64) acc[i] = 0.0f;

  // the reference starts at 0 and moves to the first batch with mass (no round trip of its own)
  int ref = 0;
  bool have = false;
  float z = 0.0f, bsum = 0.0f;
  for (int j0 = 0; j0 < G; j0 += kBlocks) {
    // a term's exponent is (alpha + beta) + (its blocks' offsets - ref): the sum of the stored values
    // and the integer part are kept apart, so that the exponent is formed only after the reference
    // has moved near the largest term (a long utterance's offsets reach 1e5, where float has no
    // digits left for the fraction)
    float s0[kBlocks], s1[kBlocks];
    int c0[kBlocks], c1[kBlocks], d1[kBlocks];
#pragma unroll
    for (int u = 0; u < kBlocks; ++u) {
      const int j = j0 + u, k = 64 * j + lane;
      s0[u] = s1[u] = kNeg;
      c0[u] = c1[u] = 0;
      d1[u] = 0;
      if (j < G) {
        // state 2k+1 takes beta (and its offset) from the next lane: lane 63 from the next block's lane 0
        const int jn = lane < 63 ? j : min(j + 1, G - 1), ln = lane < 63 ? lane + 1 : 0;
        const int oa = offA(j, lane), ob0 = offB(j, lane), ob1 = offB(jn, ln);
        const int64_t rb = ((int64_t)j * TT + r) * 128;
        c0[u] = oa + ob0 - ref;
        c1[u] = oa + ob1 - ref;
        if (k <= U) {
          const float2 a = ld_dev2(P.ABa + rb + 2 * lane);
          s0[u] = a.x + ld_dev(P.ABb + rb + 2 * lane + 1);
          if (k < U) {
            s1[u] = a.y + ld_dev(P.ABb + (lane < 63 ? rb + 2 * lane + 2 : rb + TT * 128));
            d1[u] = dmap[k + 1];
          }
        }
      }
    }
    float mx = kNeg;  // (approximate: only its integer part is used)
#pragma unroll
    for (int u = 0; u < kBlocks; ++u)
      mx = fmaxf(mx, fmaxf(s0[u] + static_cast<float>(c0[u]), s1[u] + static_cast<float>(c1[u])));
    mx = wave_max(mx);
    if (mx > kNegHalf && (!have || mx > 0.0f)) {  // wave-uniform
      const int sh = static_cast<int>(floorf(mx));
      if (have) {
        const float sc = exp2_fast(-static_cast<float>(sh));
        z *= sc;
        bsum *= sc;
        for (int i = lane; i <= U; i += 64) acc[i] *= sc;
      }
      ref += sh;
      have = true;
#pragma unroll
      for (int u = 0; u < kBlocks; ++u) {
        c0[u] -= sh;
        c1[u] -= sh;
      }
    }
#pragma unroll
    for (int u = 0; u < kBlocks; ++u) {
      const int k = 64 * (j0 + u) + lane;
      const float p0 = k <= U ? exp2_fast(fminf(s0[u] + static_cast<float>(c0[u]), 64.0f)) : 0.0f;
      const float p1 = k < U ? exp2_fast(fminf(s1[u] + static_cast<float>(c1[u]), 64.0f)) : 0.0f;
      z += p0 + p1;
      bsum += p0;
      if (k < U) atomicAdd(&acc[d1[u]], p1);
    }
  }
  z = wave_sum(z);
  bsum = wave_sum(bsum);
  if (lane == 0) atomicAdd(&acc[dmap[0]], bsum);
  if (!(z > 0.0f)) return false;
  const float scale = w / z;
  for (int i = lane; i <= U; i += 64) acc[i] *= scale;
  return true;
}

// row r of a dead utterance (zero weight: 0, no alignment or NaN: NaN) or of no utterance (0)
template <int DT>
__device__ __forceinline__ void fill_row(const Layout& L, void* grad, int64_t r, float fill, int lane) {
  const int64_t f0 = r * L.D, f1 = f0 + L.D;
  wave_segment<DT>(
      nullptr, f0, f1, lane,
      [&](int64_t q, int64_t, const float*) {
        const float v[8] = {fill, fill, fill, fill, fill, fill, fill, fill};
        store8<DT>(grad, q, v);
      },
      [&](int64_t f) { store_grad(grad, DT, f, fill); });
}

// gradient row r of live utterance b (weight w), its class sums taken from P.post.  lds: this
// wave's words, the class sums (C_stride) then the class bitmap (Dw) and its prefix counts (Dw);
// cur_b: the utterance whose bitmap the LDS holds (updated here).
// SUMS_IN_LDS: the class sums are already in the wave's LDS (streamed pipeline), not in P.post.
// RB: aligned row chunks per lane in flight (row_batch by default)
template <int DT, bool SUMS_IN_LDS = false, int RB = row_batch<DT>()>
__device__ __forceinline__ void dense_row(const Inputs& in, const Layout& L, const Pointers& P, void* grad,
                                          uint32_t* lds, int64_t r, int b, float w, int lane, int& cur_b) {
  const int Dw = static_cast<int>(L.Dw);
  float* acc = reinterpret_cast<float*>(lds);
  uint32_t* bits = lds + L.C_stride;
  const int* pref = reinterpret_cast<const int*>(bits + Dw);
  const int64_t D = L.D;
  const int64_t f0 = r * D, f1 = f0 + D;
  // aligned chunks [qb, qe) of the row: the first batch and the row's class sums load together
  int64_t a0 = (f0 + 7) & ~int64_t(7), a1 = f1 & ~int64_t(7);
  if (a0 > a1) a0 = a1 = f1;  // shorter than one aligned chunk: all single elements
  const int64_t qb = a0 >> 3, qe = a1 >> 3;
  Raw8<DT> raw[RB];
  if (qe > qb) {
#pragma unroll
    for (int u = 0; u < RB; ++u) raw[u] = ld8<DT>(in.log_probs, min(qb + lane + 64 * u, qe - 1));  // clamped
  }
  const int U = P.meta[b].U;
  const float* pr = P.post + r * L.C_stride;
  float pv[kPost];
  if (!SUMS_IN_LDS) {
#pragma unroll
    for (int k = 0; k < kPost; ++k) pv[k] = pr[min(lane + 64 * k, U)];
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
  // LDS operations of one wave complete in order: these writes precede every read below
  if (!SUMS_IN_LDS) {
#pragma unroll
    for (int k = 0; k < kPost; ++k)
      if (lane + 64 * k <= U) acc[lane + 64 * k] = pv[k] * w;  // (P.post holds the sums without the weight)
    for (int i = lane + 64 * kPost; i <= U; i += 64) acc[i] = pr[i] * w;  // long targets
  }

  // stream the row once: w * exp(lp) minus the class posterior (times w) at the columns that carry one.
  // The classes of an aligned chunk of 8 columns are consecutive in rank order, so one rank per
  // chunk (classes before its first column) locates them all.  Per group of kLook chunks: all
  // bitmap and prefix reads, then the class-sum reads, then the arithmetic, so each kind of
  // latency is paid once per group.
  auto rank = [&](int64_t c) {
    const int wi = static_cast<int>(c >> 5);
    return pref[wi] + __builtin_popcount(bits[wi] & ((1u << (c & 31)) - 1u));
  };
  auto has = [&](int64_t c) { return (bits[c >> 5] >> (c & 31)) & 1u; };
  auto single = [&](int64_t f) {
    const int64_t c = f - f0;
    float g = w * exp2_fast(load_lp(in.log_probs, DT, f) * kLog2e);
    if (has(c)) g -= acc[rank(c)];
    store_grad(grad, DT, f, g);
  };
  if (f0 + lane < a0) single(f0 + lane);
  auto batch = [&](int64_t q0) {
#pragma unroll
    for (int h = 0; h < RB; h += kLook) {
      uint32_t m8[kLook];
      int rk[kLook];
#pragma unroll
      for (int u = 0; u < kLook; ++u) {
        const int64_t c0 = min((q0 + 64 * (h + u)) * 8 - f0, D - 1);
        const int wi = static_cast<int>(c0 >> 5), sh = static_cast<int>(c0 & 31);
        const uint32_t b0 = bits[wi], b1 = wi + 1 < Dw ? bits[wi + 1] : 0u;
        m8[u] = static_cast<uint32_t>((((uint64_t)b1 << 32) | b0) >> sh) & 0xffu;
        rk[u] = pref[wi] + __builtin_popcount(b0 & ((1u << sh) - 1u));
      }
      float c0v[kLook], c1v[kLook];
#pragma unroll
      for (int u = 0; u < kLook; ++u) {
        c0v[u] = acc[rk[u]];  // rank <= U+1: inside this wave's class sums and bitmap
        c1v[u] = acc[rk[u] + 1];
      }
#pragma unroll
      for (int u = 0; u < kLook; ++u) {
        const int64_t q = q0 + 64 * (h + u);
        if (q >= qe) continue;
        float v[8];
        unpack8<DT>(raw[h + u], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = w * exp2_fast(v[e] * kLog2e);
        uint32_t mm = m8[u];
        int j = 0;
        while (mm) {
          const int e = __builtin_ctz(mm);
          mm &= mm - 1;
          v[e] -= j == 0 ? c0v[u] : (j == 1 ? c1v[u] : acc[rk[u] + j]);
          ++j;
        }
        store8<DT>(grad, q, v);
      }
    }
  };
  if (qe > qb) {
    batch(qb + lane);
    for (int64_t q0 = qb + lane + 64 * RB; q0 < qe + lane; q0 += 64 * RB) {  // rows longer than one batch
#pragma unroll
      for (int u = 0; u < RB; ++u) raw[u] = ld8<DT>(in.log_probs, min(q0 + 64 * u, qe - 1));
      batch(q0);
    }
  }
  if (a1 + lane < f1 && a1 + lane >= a0) single(a1 + lane);
}

}  // namespace rows
}  // namespace pctc
