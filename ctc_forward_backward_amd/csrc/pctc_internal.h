// Internal declarations of the packed CTC HIP library (gfx950 only).
//
// Data flow of one packed_ctc_loss call, all on the caller's stream:
//   prep      per utterance: clamp metadata, extended-label ids, row -> utterance map
//   gather    per owned row: the U+1 distinct emissions log2 p(blank), log2 p(l_1..l_U) of that row,
//             shifted by an integer per-row offset so that they sit near 0
//   chains    one workgroup per (utterance, direction): the alpha and the beta recursions run
//             concurrently in one launch, each frame renormalised by the previous frame's maximum
//   weights   per utterance: loss, zero_infinity, gradient weight; the sum / mean reduction
//   dense     per owned row: posteriors as a per-frame softmax over states of alpha + beta - lp,
//             summed per class in LDS, then one coalesced pass writing w*exp(lp) - posterior
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pctc {

// log-space "minus infinity": finite so that max-based log-sum-exp never forms inf - inf
constexpr float kNeg = -1.0e30f;
constexpr float kNegHalf = -5.0e29f;  // values below this carry no probability mass
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453;

constexpr int kMaxTargetLength = 8191;  // S = 2U+1 <= 16383 states per utterance
constexpr int kMaxClasses = 32768;      // per-class posterior accumulator in LDS (128 KB)

enum Dtype { kF32 = 0, kBF16 = 1, kF16 = 2, kF64 = 3 };

struct Meta {
  int start;  // first row
  int T;      // frames (clamped so that rows stay inside the buffer)
  int U;      // labels (clamped to the workspace bound)
  int flags;  // kNanInput: a NaN log probability was gathered; kNoAlignment: T < U + repeats
};
constexpr int kNanInput = 1;
constexpr int kNoAlignment = 2;

// Workspace carve-up.  Every region is 256-byte aligned.
// Frames per chunk of the recursions: their prefetch depth and the period of their integer shift.
// Each lane (state pair) keeps an integer offset of its own, stored once per chunk.
constexpr int kChunk = 32;

// 64-pair state blocks per segment of a recursion: the waves of one workgroup, one per SIMD, linked
// through LDS; segments link through a global ring.  (Two recursion waves on one SIMD slow both more
// than a global link costs.)
constexpr int kSegWaves = 4;

// Least LDS a row kernel takes per workgroup: with the recursion workgroups' reservation it keeps
// the two kinds of workgroup off each other's compute units.
constexpr size_t kRowKernelLds = 8 * 1024;

// Rows of padding before and after the emission table: the recursions prefetch up to two chunks
// of frames past either end of an utterance without clamping.
constexpr int kEPad = 72;

struct Layout {
  int64_t T_total, D, B, Umax;
  int64_t E_stride;  // floats per row of the emission table (>= Umax + 2)
  int64_t Gmax;      // state-pair blocks of the longest target: ceil((Umax + 1) / 64)
  int64_t Dw;        // 32-bit words of a class bitmap: ceil(D / 32)
  int64_t C_stride;  // floats per row of the compact class sums (>= Umax + 1)
  int64_t NCH;       // chunk slots of the per-lane offsets: >= sum over utterances of ceil((T - 1) / kChunk)
  int64_t K;         // checkpoint interval of alpha: every K-th step kept (1: every step)
  int64_t band;      // streamed pipeline: frames a side per row band of a long utterance (by the row's bytes)
  int64_t NQ;        // alpha rows kept per block: T_total (K = 1), else >= sum over utterances of ceil(T / K)
  size_t off_qbase, off_cbase, off_cbits, off_cpref, off_dmap, off_meta, off_lab, off_rowmap, off_rowoff, off_E, off_Eb, off_AB, off_nll, off_llb, off_lsh, off_w, off_post, off_order, off_cum, off_gid, off_ring,
      off_sig, off_items, off_ctl, off_prog, off_bands, total;
};

// Utterances are sorted by frame count (longest first) and cut into up to kMaxGroups groups of
// consecutive sorted positions; each group runs its gather, recursions and rows on a stream of its
// own, so the rows of short utterances overlap the recursions of long ones.  Three streams (the
// caller's and two more) fit the hardware queues a process gets by default; group g ends where the
// groups so far hold a set share of the rows (schedule kernel), so that the group of the longest
// recursion has few rows left to do after it.
constexpr int kMaxGroups = 3;

// the work of one group
struct GroupQ {
  int qlen;     // recursion segments of the group
  int qcount;   // next segment to claim
  int itemoff;  // first segment of the group in the segment list
  int first;    // first sorted position of the group
  int count;    // utterances in the group
  int nrows;    // rows owned by the group's utterances
  int pad[2];
};

// control words of the recursion work queues
struct ChainCtl {
  int err;      // non-zero: a wave gave up a bounded wait; the losses of the call are NaN
  int ngroups;
  int nbands;   // streamed pipeline: row bands queued after group 0's recursion segments
  int post_ready;  // a streamed forward formed every row's class sums (the backward only forms the rows)
  int rows_for;    // 1 + zero_infinity + 2 reduction: the gradient rows for unit upstream weights were
                   // written by the forward with these (packed_ctc_forward_grad); 0 otherwise
  int unit;        // a gradient update found unit upstream weights for rows_for: its row kernels skip
  int pad[2];
  GroupQ g[kMaxGroups];
};

// Streamed pipeline: the rows of an utterance are handed out in bands of up to 2 n rows (n = L.band
// frames a side, kBand or kWideBand), band k holding the frames t whose later-finished recursion step
// max(t, T-1-t) lies in [T/2 + k n, T/2 + (k+1) n): a band can be formed as soon as both recursions
// have passed its last such step, so the bands of an utterance become ready from the middle frames
// outwards.  kBand is also the smallest band, which sizes the band queue.
constexpr int kBand = 16;
// bands of kWideBand frames a side where a row (log probs in and gradient out) holds fewer than
// kBandRowBytes: fewer, larger bands spread each band's fixed cost (its claim, wait and first
// loads) over more rows, while expensive rows keep the last band of a long utterance short
constexpr int kWideBand = 24;
constexpr int64_t kBandRowBytes = 16384;
// frames a side per band of an utterance with T frames: L.band, or kBand below 4 wide bands (a wide
// first band of a short utterance would cover most of it and be ready only at its end)
__host__ __device__ inline int band_frames(const Layout& L, int T) {
  return T >= 4 * kWideBand ? static_cast<int>(L.band) : kBand;
}
// a queue item holding both chains of one utterance of at most two 64-pair blocks (the recursions'
// work queue; other items are (chain << 12) | segment)
constexpr int kBothChains = 1 << 30;
// Each progress word sits on a cache line of its own (128 bytes): the bands of many utterances poll
// them from every compute unit while the chains' last blocks write them, and words sharing lines
// measured up to 55 us slower per call (asr_bpe).
constexpr int kProgStride = 32;
// workgroup of the streamed pipeline: four recursion waves (one per SIMD), or sixteen row waves
constexpr int kStreamWaves = 16;

Layout make_layout(int64_t T_total, int64_t D, int64_t B, int64_t Umax, int64_t K = 1);
constexpr int kMaxCheckpoint = 32;        // checkpoint intervals: powers of two up to the chunk
constexpr int kMaxCheckpointBlocks = 16;  // checkpointed utterances: up to 16 state blocks (U <= 1023)

struct Pointers {
  Meta* meta;
  int* lab;      // (B, Umax + 1): j = 0 the blank, j >= 1 targets[b][j-1]
  int* rowmap;   // (T_total,): owning utterance, written for owned rows only (see row_owner)
  int* rowoff;   // (T_total,): integer offset subtracted from the row's gathered log2 emissions
  float* E;      // (T_total, E_stride): columns 0..U the labels, U+1 holds -1e30; kEPad rows of padding on either side
  float* Eb;     // (T_total,): column 0 of E (the blank) again, contiguous for the recursions; kEPad padding each side
  // Normalised log2 alpha and beta per block of 64 state pairs and per row, 128 floats each.  Alpha
  // pair k sits at 2k, 2k+1 (states 2k, 2k+1); beta pair k at 2k, 2k+1 (states 2k-1, 2k), i.e. beta
  // of state s at position s+1, each relative to its lane's offset for that chunk (sig).
  //   ABa: alpha, (Gmax, NQ, 128): K = 1 row-indexed (NQ = T_total); K > 1 the kept steps 0, K, 2K,
  //        ... of utterance b at slots qbase[b] + step / K
  //   ABb: beta, (Gmax, T_total, 128), row-indexed
  // (K = 1: ABb follows ABa, and the float64 path uses the two as one float64 array)
  float* ABa;
  float* ABb;
  int* qbase;    // (B + 1) first alpha slot of each utterance (K > 1: exclusive prefix of ceil(T / K))
  double* nll;   // (B,) raw negative log-likelihood in nats (+inf: no alignment)
  double* llb;   // (B,) log2 likelihood from the beta side (consistency check)
  double* lsh;   // (B,) log2 likelihood from the alpha side without the row offsets
  float* w;      // (B,) gradient weight
  unsigned long long* ring;  // (2, Gmax, T_total) block-boundary values (value, offset) per frame
  // (2, Gmax, NCH, 64) integer offset of each lane's stored values (its state pair), per chunk: chunk c
  // of utterance b at slot cbase[b] + c
  int* sig;
  int* cbase;    // (B + 1) first chunk slot of each utterance (exclusive prefix of ceil((T - 1) / kChunk))
  int* items;    // (2 B Gmax) queued recursion segments, by group: (utterance * 2 + direction) << 12 | segment
  int* order;    // (B) utterances by frame count, longest first (ties by index)
  int* cum;      // (B) per sorted position: rows of the group's earlier utterances
  int* gid;      // (B) per utterance: its group
  ChainCtl* ctl;
  // classes of each utterance's extended labels (blank and labels), for the gradient rows:
  uint32_t* cbits;  // (B, Dw) bitmap of the classes present
  int* cpref;       // (B, Dw) number of classes present in the words before each word
  int* dmap;        // (B, Umax + 1) rank among the present classes of lab[j]
  float* post;      // (T_total, C_stride) per row: the class sums over z (without the weight), by class rank
  // streamed pipeline: per (utterance, direction) the recursion steps whose states every block has
  // stored where any compute unit sees them, and the queue of row bands (utterance, band), readiest
  // first
  int* prog;        // (2 B) words, kProgStride ints apart
  int2* bands;      // (T_total / kBand + 2 B + 1): at most ceil(ceil(T/2) / kBand) <= T/64 + 2 per utterance
  // the gradient update (packed_ctc_backward_update): &ctl->unit, which its row kernels read first
  // and return at once when set; null in every other call
  const int* skip;
};
// a row kernel of a gradient update whose rows the forward already wrote
__device__ __forceinline__ bool skipped(const Pointers& P) {
  return P.skip && __builtin_amdgcn_readfirstlane(*P.skip) != 0;
}

Pointers carve(void* workspace, const Layout& L);

// ---- device helpers ----------------------------------------------------------------------------

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// log2(2^a + 2^b) with the finite sentinel: the result stays at the sentinel when both are.
__device__ __forceinline__ float lse2(float a, float b) {
  const float hi = fmaxf(a, b), lo = fminf(a, b);
  return hi + log2_fast(1.0f + exp2_fast(lo - hi));
}

__device__ __forceinline__ float load_lp(const void* p, int dtype, int64_t i) {
  if (dtype == kF32) return static_cast<const float*>(p)[i];
  if (dtype == kF64) return static_cast<float>(static_cast<const double*>(p)[i]);
  if (dtype == kF16) return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  const uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16;
  return __builtin_bit_cast(float, bits);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);  // quiet NaN
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void store_grad(void* p, int dtype, int64_t i, float v) {
  if (dtype == kF32) {
    static_cast<float*>(p)[i] = v;
  } else if (dtype == kF64) {
    static_cast<double*>(p)[i] = static_cast<double>(v);
  } else if (dtype == kF16) {
    static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
  } else {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(v);
  }
}

__device__ __forceinline__ int64_t load_index(const void* p, bool i64, int64_t i) {
  return i64 ? static_cast<const int64_t*>(p)[i] : static_cast<int64_t>(static_cast<const int32_t*>(p)[i]);
}

// The rows of group g as one list (its utterances in sorted order, each utterance's rows in order):
// fn(r, b) for list entries [j0, j1).  Everything here is uniform over the wave.
template <typename F>
__device__ __forceinline__ void group_rows(const Pointers& P, int g, int64_t j0, int64_t j1, F fn) {
  const GroupQ& q = P.ctl->g[g];
  if (j0 >= j1 || q.count <= 0) return;
  // the last sorted position whose first list entry is at or before j0
  int lo = q.first, hi = q.first + q.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (P.cum[mid] <= j0) lo = mid;
    else hi = mid - 1;
  }
  int64_t j = j0;
  for (int i = lo; j < j1 && i < q.first + q.count; ++i) {
    const int b = __builtin_amdgcn_readfirstlane(P.order[i]);
    const Meta m = P.meta[b];
    const int64_t off = j - P.cum[i];  // row of the utterance
    const int64_t take = min(j1 - j, (int64_t)m.T - off);
    for (int64_t k = 0; k < take; ++k) fn(m.start + off + k, b);
    if (take > 0) j += take;
  }
}

// The utterance that owns row r, or -1.  The row map is written for owned rows only; the entry of a
// row that no utterance owns is left from earlier use of the workspace and names (if any) an
// utterance whose rows do not hold r, so an entry counts only where that utterance's rows hold r.
__device__ __forceinline__ int row_owner(const Layout& L, const Pointers& P, int64_t r) {
  const int b = P.rowmap[r];
  if (b < 0 || b >= L.B) return -1;
  const Meta m = P.meta[b];
  return r >= m.start && r < (int64_t)m.start + m.T ? b : -1;
}

// list entries [j0, j1) of wave `wid` out of `waves` over group g's rows
__device__ __forceinline__ void wave_share(const Pointers& P, int g, int64_t wid, int64_t waves, int64_t& j0,
                                           int64_t& j1) {
  const int64_t n = P.ctl->g[g].nrows;
  const int64_t per = (n + waves - 1) / waves;
  j0 = min(wid * per, n);
  j1 = min(j0 + per, n);
}

// ---- 8-element chunks of a (T_total, D) log-prob / gradient buffer ----------------------------
// Chunk q holds flat elements [8q, 8q+8): 16 aligned bytes for 16-bit dtypes, 32 for float32, 64 for
// float64 (read into float32 arithmetic; the gradient goes back as float64).

// Row chunks are read once and written once: non-temporal loads and stores keep them from
// displacing reused data (the recursions' states, class sums) in the caches.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  const u32x4_nt w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<u32x4_nt*>(p));
}

// Raw bytes of one chunk, held while its load is in flight.
template <int DT>
struct Raw8 {
  uint4 u[DT == kF64 ? 4 : (DT == kF32 ? 2 : 1)];
};

template <int DT>
__device__ __forceinline__ Raw8<DT> ld8(const void* base, int64_t q) {
  Raw8<DT> r;
  constexpr int n = DT == kF64 ? 4 : (DT == kF32 ? 2 : 1);
  const uint4* p = static_cast<const uint4*>(base) + n * q;
#pragma unroll
  for (int i = 0; i < n; ++i) r.u[i] = ld_stream(p + i);
  return r;
}

template <int DT>
__device__ __forceinline__ void unpack8(const Raw8<DT>& r, float v[8]) {
  if constexpr (DT == kF64) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = static_cast<float>(__builtin_bit_cast(double, (uint64_t)r.u[i].x | ((uint64_t)r.u[i].y << 32)));
      v[2 * i + 1] = static_cast<float>(__builtin_bit_cast(double, (uint64_t)r.u[i].z | ((uint64_t)r.u[i].w << 32)));
    }
  } else if constexpr (DT == kF32) {
    const uint32_t w[8] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w, r.u[1].x, r.u[1].y, r.u[1].z, r.u[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, w[i]);
  } else {
    const uint32_t w[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == kF16) {
        v[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xffffu)));
        v[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
      } else {
        v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t q, const float v[8]) {
  if constexpr (DT == kF64) {
    uint4* p = static_cast<uint4*>(base) + 4 * q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t a = __builtin_bit_cast(uint64_t, static_cast<double>(v[2 * i]));
      const uint64_t b = __builtin_bit_cast(uint64_t, static_cast<double>(v[2 * i + 1]));
      st_stream(p + i, make_uint4(static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32), static_cast<uint32_t>(b),
                                  static_cast<uint32_t>(b >> 32)));
    }
  } else if constexpr (DT == kF32) {
    uint4* p = static_cast<uint4*>(base) + 2 * q;
    st_stream(p, make_uint4(__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                            __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])));
    st_stream(p + 1, make_uint4(__builtin_bit_cast(uint32_t, v[4]), __builtin_bit_cast(uint32_t, v[5]),
                                __builtin_bit_cast(uint32_t, v[6]), __builtin_bit_cast(uint32_t, v[7])));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo, hi;
      if constexpr (DT == kF16) {
        lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[2 * i]));
        hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[2 * i + 1]));
      } else {
        lo = f32_to_bf16_rne(v[2 * i]);
        hi = f32_to_bf16_rne(v[2 * i + 1]);
      }
      w[i] = lo | (hi << 16);
    }
    st_stream(static_cast<uint4*>(base) + q, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// Visit the flat elements [f0, f1) of a (T_total, D) buffer with one wave: aligned 8-element
// chunks in the middle and single elements (fn1(element)) at the ragged ends; nothing outside
// [f0, f1) is touched.  With a source buffer, up to kBatch chunks per lane are loaded before any is
// used (fn8(chunk index, first element, values)), so a wave keeps that many loads in flight;
// without one (src == nullptr) fn8 gets no values.
constexpr int kBatch = 8;

template <int DT, typename F8, typename F1>
__device__ __forceinline__ void wave_segment(const void* src, int64_t f0, int64_t f1, int lane, F8 fn8, F1 fn1) {
  int64_t a0 = (f0 + 7) & ~int64_t(7), a1 = f1 & ~int64_t(7);
  if (a0 > a1) a0 = a1 = f1;  // shorter than one aligned chunk: all single elements
  if (f0 + lane < a0) fn1(f0 + lane);
  const int64_t qe = a1 >> 3;
  for (int64_t q0 = (a0 >> 3) + lane; q0 < qe; q0 += 64 * kBatch) {
    if (src) {
      Raw8<DT> raw[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (q0 + 64 * u < qe) raw[u] = ld8<DT>(src, q0 + 64 * u);
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (q0 + 64 * u < qe) {
          float v[8];
          unpack8<DT>(raw[u], v);
          fn8(q0 + 64 * u, (q0 + 64 * u) << 3, v);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (q0 + 64 * u < qe) {
          float v[8];
          fn8(q0 + 64 * u, (q0 + 64 * u) << 3, v);
        }
      }
    }
  }
  if (a1 + lane < f1 && a1 + lane >= a0) fn1(a1 + lane);
}

// DPP lane moves (gfx9 encodings): row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143,
// wave_shr:1 = 0x138, wave_shl:1 = 0x130.  Lanes without a source, and rows outside ROWS, keep `old`.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, src),
                                                               CTRL, ROWS, 0xf, false));
}

// maximum over the 64 lanes of a wave, returned to every lane
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0x111>(kNeg, x));
  x = fmaxf(x, dpp_f32<0x112>(kNeg, x));
  x = fmaxf(x, dpp_f32<0x114>(kNeg, x));
  x = fmaxf(x, dpp_f32<0x118>(kNeg, x));
  x = fmaxf(x, dpp_f32<0x142, 0xa>(kNeg, x));  // row r (r = 1, 3) takes lane 15 of row r-1
  x = fmaxf(x, dpp_f32<0x143, 0xc>(kNeg, x));  // rows 2, 3 take lane 31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// sum over the 64 lanes of a wave, returned to every lane
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0x111>(0.0f, x);
  x += dpp_f32<0x112>(0.0f, x);
  x += dpp_f32<0x114>(0.0f, x);
  x += dpp_f32<0x118>(0.0f, x);
  x += dpp_f32<0x142, 0xa>(0.0f, x);
  x += dpp_f32<0x143, 0xc>(0.0f, x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Workgroup barrier that orders LDS accesses only: global loads and stores stay in flight across it
// (a full __syncthreads() is a workgroup fence over every address space and drains them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- launchers (each in its own translation unit) ----------------------------------------------

struct Inputs {
  const void* log_probs;
  int dtype;
  int64_t T_total, D;
  const void* cu_seqlens;
  const void* lengths;
  int64_t B;
  const void* targets;
  int64_t target_width;
  const void* target_lengths;
  int index_flags;
  int blank;
  int zero_infinity;
  int reduction;
  const void* grad_scale;
  int64_t wait_ticks;  // bound of every wait on another wave, in wall_clock64() ticks
};

// grad_scale[b] in the loss type of the input dtype (float64 for float64 inputs, else float32), or 1
__device__ __forceinline__ double grad_scale_of(const Inputs& in, int64_t b) {
  if (!in.grad_scale) return 1.0;
  return in.dtype == kF64 ? static_cast<const double*>(in.grad_scale)[b] : (double)static_cast<const float*>(in.grad_scale)[b];
}

// The gradient weight of utterance b in float64 (the float64 path): as utterance_weight below.
__device__ __forceinline__ double utterance_weight64(const Inputs& in, int64_t B, int64_t b, bool infinite) {
  const int64_t U = load_index(in.target_lengths, in.index_flags & 8, b);
  double w = grad_scale_of(in, b);
  if (in.reduction == 2) w /= (double)B * (U > 1 ? (double)U : 1.0);
  if (in.zero_infinity && infinite) w = 0.0;
  return w;
}

// The gradient weight of utterance b: grad_scale[b] (or 1), over B * max(U, 1) for the mean (U as
// the caller gave it), and 0 under zero_infinity for an utterance without alignment.
__device__ __forceinline__ float utterance_weight(const Inputs& in, int64_t B, int64_t b, bool infinite) {
  const int64_t U = load_index(in.target_lengths, in.index_flags & 8, b);
  const double Uc = U > 1 ? (double)U : 1.0;
  double w = grad_scale_of(in, b);
  if (in.reduction == 2) w /= (double)B * Uc;
  if (in.zero_infinity && infinite) w = 0.0;
  return static_cast<float>(w);
}

// setup (streamed pipeline): also clears the recursion rings and forms the class maps
hipError_t launch_prep(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s, bool setup = false);
// gaps: when given (the gradient), rows owned by no utterance are zeroed in the same launch
hipError_t launch_gather(const Inputs& in, const Layout& L, const Pointers& P, int group, hipStream_t s,
                         void* gaps = nullptr);
// streamed pipeline: whether the gather launch also builds the schedule (its first workgroup, beside
// the gathering ones: the batch has at most 512 utterances and the schedule's LDS fits beside the
// gather's residency); otherwise the schedule launch runs before the gather
bool schedule_in_gather(const Layout& L);
// streamed pipeline: the gather over all rows in their natural order, with the gap rows zeroed when
// `gaps` is given, and the schedule in its first workgroup when schedule_in_gather(L)
hipError_t launch_gather_stream(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s, void* gaps);
// sorts the utterances and cuts them into `groups` groups (see GroupQ)
// setup (streamed pipeline, one group): the rings are already clear; also builds the row-band queue
hipError_t launch_schedule(const Inputs& in, const Layout& L, const Pointers& P, int groups, hipStream_t s,
                           bool setup = false);
// dense log-space HMM forward (hmm.hip): one log-likelihood per observation sequence
hipError_t launch_hmm_forward(const float* log_init, const float* log_trans, const float* log_emit, const void* obs,
                              int obs_i64, int64_t B, int64_t T, int S, int O, float* out, hipStream_t s);
constexpr int kHmmMaxStates = 64;
constexpr int64_t kHmmMaxTable = 16384;  // S * O floats of the emission table in LDS

// store: keep alpha, beta and the block offsets for the posteriors (false: the loss only)
hipError_t launch_chains(const Inputs& in, const Layout& L, const Pointers& P, int group, bool store, hipStream_t s);
// rows: 0, or kRowsMark (the call wrote the gradient for unit upstream weights: recorded in
// ctl->rows_for), or kRowsUpdate (a gradient update: sets ctl->unit, see ChainCtl)
constexpr int kRowsMark = 1, kRowsUpdate = 2;
hipError_t launch_weights(const Inputs& in, const Layout& L, const Pointers& P, void* losses_out, void* reduced_out,
                          hipStream_t s, int rows = 0);
hipError_t launch_classes(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s);
hipError_t launch_posteriors(const Inputs& in, const Layout& L, const Pointers& P, int group, hipStream_t s);
hipError_t launch_dense(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, int group, hipStream_t s);
// streamed pipeline (one group): the queue of row bands, then one persistent launch running the
// recursions and, as their frames become ready, the posteriors and gradient rows
bool stream_fits(const Inputs& in, const Layout& L);
// sums (with grad_out): each row's class sums are kept in P.post too, for a later gradient update
hipError_t launch_stream(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s,
                         bool sums = false);
// float64 inputs in float64 arithmetic (f64.hip): alpha of every utterance (stored in the state region
// as float64) and its loss; then beta with each frame's posteriors and gradient row (needs the
// weights and the class maps)
hipError_t launch_f64_alpha(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s);
hipError_t launch_f64_beta_rows(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s);
// alpha checkpointing (ckpt.hip): the class sums of the rows of group `group` (-1: every row) from alpha
// recomputed out of the kept steps
hipError_t launch_ckpt_posteriors(const Inputs& in, const Layout& L, const Pointers& P, int group, hipStream_t s);
// zero gradient rows owned by no utterance
hipError_t launch_gaps(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s);
hipError_t launch_reduce(const float* losses, const void* target_lengths, bool i64, int64_t B, int reduction, float* out,
                         hipStream_t s);

}  // namespace pctc
