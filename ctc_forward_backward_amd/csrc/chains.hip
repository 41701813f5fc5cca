// The alpha and beta recursions of packed CTC as a pipeline of one-wave state blocks.
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities", Triton file, `_alpha_kernel` and `_beta_grad_kernel`:
//   alpha[0] holds the first blank and the first label; alpha[t][s] is the log-sum-exp of
//   alpha[t-1][s], alpha[t-1][s-1] and, into a label whose id differs from the label two states
//   back, alpha[t-1][s-2], plus the frame's log probability at the state's class; the loss is
//   -log(alpha[T-1][S-1] + alpha[T-1][S-2]).  beta mirrors it from the last frame, emission
//   included, starting in the last blank and the last label; its start-state sum is the same
//   likelihood.
//
// Design for gfx950 (not the page's one-program-per-utterance Triton design):
//   - A recursion is latency-bound: one frame is one dependent log-sum-exp step.  The states of an
//     utterance are cut into blocks of 64 state pairs, one wave per block, one pair per lane.
//     Lane i of block j owns pair k = 64 j + i: (2k, 2k+1) = (blank, label k+1) for alpha and
//     (2k-1, 2k) = (label k, blank) for beta.  Either way a lane needs one value per frame from
//     outside its pair, the label of the neighbouring pair, moved one lane by DPP (wave_shr:1 for
//     alpha, wave_shl:1 for beta).
//   - Per pair and frame the step is two two-way log-sum-exps: t = lse(blank, neighbour) gives the
//     new blank, and lse(label, skip allowed ? t : blank) the new label (the three-way sum of the
//     label state is the two-way sum of the label with t).  A label state that does not exist reads
//     an emission column that holds -1e30, so it stays far below every real state and needs no
//     mask; the lanes past the last pair only feed lanes that do not exist either.
//   - Between blocks the neighbour value flows one way (alpha: block j-1 -> j; beta: j+1 -> j).
//     Four consecutive blocks form a segment run by the four waves of one workgroup (one per SIMD):
//     inside a segment the edge value goes through a 128-slot LDS ring, between segments through a
//     global ring slot per frame (one 64-bit system-scope store into a slot that starts at zero).
//     A slot holds the value and, in its high word, the producer's integer offset and a validity
//     mark (the LDS ring also tags the chunk, since its slots are reused).  Nobody waits on a later
//     block, so the pipeline has no round trip per frame, only a fill latency per block.
//   - A consumer takes the neighbour values of a whole 32-frame chunk at the chunk's start, one per
//     lane, checks them with one ballot and converts them to its own offset; a frame then costs one
//     v_readlane.  Global slots are loaded one chunk ahead.
//   - Segments are items of one work queue, producers first (see the schedule kernel), claimed by
//     a persistent grid: a claimed segment's producer is always already running.  Every wait is
//     bounded; a wave that gives up raises ctl->err and continues, so the kernel always ends.
//   - base-2 log space (emissions pre-scaled by log2 e) so v_exp_f32 / v_log_f32 apply directly;
//     emissions carry an integer per-row offset, and each block shifts its values by an integer
//     (its maximum) every chunk, so stored values stay near 0; the offsets are stored per
//     (block, chunk) and summed in float64 for the loss.
//   - Per frame a wave issues one 512-byte store of its 128 states (a block-major time series) and
//     one load of next chunk's label emission, both through buffer resources rebased per chunk so
//     that every offset is a scalar register; the blank emissions of a chunk are one contiguous load,
//     one frame per lane.
#include <algorithm>
#include <type_traits>

#include "rows.h"

namespace pctc {

namespace {

constexpr int kK = kChunk;             // frames per chunk (prefetch depth and renormalisation period)
constexpr int kR = 128;                // LDS ring slots per wave boundary (4 chunks)
constexpr int kWaves = kSegWaves;      // blocks per segment = waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer resource, gfx9 family
constexpr int kStoreSc1 = 16;                 // cache policy of a buffer store: sc1, written through to device scope
static_assert(2 * kK + 1 <= kEPad, "emission padding must cover two chunks of prefetch");
static_assert(kR % kK == 0, "a chunk's ring slots must not wrap");

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned long long gload(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void gstore(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ unsigned long long lload(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void lstore(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// high word of a ring slot: integer offset << 8 | 0x80 (written) | producer chunk & 127
// (chunk -1 is the first frame)
__device__ __forceinline__ uint32_t slot_hi(float off, int chunk) {
  return (static_cast<uint32_t>(static_cast<int>(off)) << 8) | 0x80u | (static_cast<uint32_t>(chunk) & 127u);
}

__device__ __forceinline__ unsigned long long pack(float v, uint32_t hi) {
  return (unsigned long long)__builtin_bit_cast(uint32_t, v) | ((unsigned long long)hi << 32);
}

__device__ __forceinline__ uint32_t slot_hi_of(unsigned long long v) { return static_cast<uint32_t>(v >> 32); }

// the slot's value in the frame of a reader whose offset is `off`
__device__ __forceinline__ float slot_value(unsigned long long v, float off) {
  const int o = static_cast<int>(slot_hi_of(v)) >> 8;
  return __builtin_bit_cast(float, static_cast<uint32_t>(v)) + (static_cast<float>(o) - off);
}

__device__ __forceinline__ float lanef(float v, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
}

__device__ __forceinline__ void give_up(int* err) {
  __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ bool gave_up(int* err) {
  return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0;
}

// chunk of the frame at `step` (chunk c holds steps 1 + c*kK .. (c+1)*kK; step 0 is chunk -1)
__device__ __forceinline__ int chunk_of(int step) { return step == 0 ? -1 : (step - 1) / kK; }

__device__ __forceinline__ bool global_ok(unsigned long long v) { return (slot_hi_of(v) & 0x80u) != 0; }

__device__ __forceinline__ bool lds_ok(unsigned long long v, int chunk) {
  return (slot_hi_of(v) & 0xffu) == (0x80u | (static_cast<uint32_t>(chunk) & 127u));
}

// Every wait on another wave is bounded in wall-clock time (wall_clock64(), a constant-rate counter;
// the bound is a launch argument): a wave that runs out of time, or finds that another one already
// has, raises the health word and carries on with whatever it holds, so every kernel ends.  Then
// the losses of the call are NaN (weights kernel) and the gradient rows formed afterwards too.
__device__ __forceinline__ bool out_of_time(uint64_t t0, int64_t ticks, int* err) {
  return (int64_t)(wall_clock64() - t0) > ticks || gave_up(err);
}

// Bounded wait until every lane that `needs` it holds a written global slot (each lane re-reads
// its own slot); on give-up the missing values are -inf at offset 0.  The waits are inline: a call
// in the frame loop would make the compiler drain every load and store in flight at each chunk.
__device__ __forceinline__ unsigned long long wait_global(const unsigned long long* p, unsigned long long v, bool need,
                                                       int64_t ticks, int* err) {
  const uint64_t t0 = wall_clock64();
  while (__ballot(need && !global_ok(v))) {
    if (out_of_time(t0, ticks, err)) {
      give_up(err);
      if (need && !global_ok(v)) v = pack(kNeg, 0x80u);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
    if (need && !global_ok(v)) v = gload(p);
  }
  return v;
}

// the same for LDS slots tagged with the chunk each lane expects
__device__ __forceinline__ unsigned long long wait_lds(const unsigned long long* p, unsigned long long v, bool need,
                                                    int chunk, int64_t ticks, int* err) {
  const uint64_t t0 = wall_clock64();
  while (__ballot(need && !lds_ok(v, chunk))) {
    if (out_of_time(t0, ticks, err)) {
      give_up(err);
      if (need && !lds_ok(v, chunk)) v = pack(kNeg, 0x80u | (static_cast<uint32_t>(chunk) & 127u));
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    if (need && !lds_ok(v, chunk)) v = lload(p);
  }
  return v;
}

// bounded wait until the consumer wave has taken the neighbour values of chunk `c`
__device__ __forceinline__ void wait_progress(int* prog, int c, int64_t ticks, int* err) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < c) {
    if (out_of_time(t0, ticks, err)) {
      give_up(err);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

struct Shared {
  unsigned long long ring[kWaves][kR];  // ring[w]: between waves w and w+1; ring[kWaves-1]: sink
  // per wave, where the lanes other than the edge lane put their (unused) ring stores: every lane
  // stores each frame, at a distinct address, so the loop needs no change of the execution mask
  unsigned long long junk[kWaves][64 + kK];
  int prog[kWaves];
  int item;
};

// Per-wave constants of one block.
struct Ctx {
  int b, T, U, j, k, lane;
  int64_t start;
  bool vl, sk;
  bool no_in;               // no producer: every neighbour slot is (-inf, offset 0), nothing to load
  int eidx;                 // this lane's label column in the emission table (U+1: the -1e30 column)
  int64_t Es;               // floats per emission row
  const unsigned long long* gin;  // global ring read by this block (row-indexed)
  unsigned long long* gout;       // global ring written by this block
  unsigned long long* lin;        // LDS ring read by this block
  unsigned long long* lout;       // LDS ring written by this block (a sink if there is no consumer)
  unsigned long long* junk;       // this wave's junk slots (the ring stores of the other lanes)
  bool lout_live;
  int* prog_cons;
  int* prog_self;
  int* sig;                 // this block's per-lane offsets of the utterance's chunk 0 (64 ints per chunk)
  float* ab;                // this block's 128 states per row (row 0), or (ck) per kept step (slot 0)
  bool ck;                  // alpha kept only every K-th step (the grouped pipeline's checkpointing)
  int lk;                   // log2 K
  bool store;               // keep the states and offsets (false: loss only, nothing is written)
  int* prog;                // streamed pipeline, the chain's last block: where it publishes its stored steps
  int* err;
  int64_t ticks;            // wall-clock bound of every wait
  const Inputs* in;
  int64_t B;
};

// a 64-bit value the caller knows to be the same in every lane, moved to scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// vmcnt(62) with the other counters left alone (gfx9 s_waitcnt encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm62 = (3 << 14) | (15 << 8) | (7 << 4) | 14;

// The recursion of one block, specialised on the direction and on the kinds of its links, so that
// the frame loop carries no branch on any of them.
//
// Offsets.  Every lane keeps an integer offset of its own, renormalised once per chunk to the floor of
// its larger state, so a lane's values stay near 0 wherever its mass sits relative to the rest of the
// block (with one offset per block, states carrying posterior mass can sit hundreds of units below
// the block's largest, where float32 keeps few fraction bits, and the rounding of each step then
// accumulates with the number of frames).  The neighbour value a lane takes each frame is moved into
// its own offset by the integer difference of the two lanes' offsets, fixed over a chunk.
//
// STREAM (the streamed pipeline, where the posteriors of a frame are formed on other compute units,
// possibly other XCDs, while the recursions still run): the states are stored write-through to the
// device-coherent level (sc1) and the offsets with device-scope stores, and the chain's last block
// (every other block of the chain is at least one chunk ahead of it) publishes how many steps are
// stored.  At the start of chunk c it waits until at most 62 of its vector memory operations are
// outstanding (s_waitcnt vmcnt(62); the counter is decremented in issue order, loads and stores
// alike, per the CDNA3 instruction set guide's data-dependency rules, which the compiler's own waits
// in this loop rely on too) and, having issued at least 64 in chunk c-1 (a label-emission load and a
// state store per frame), knows that every store of chunk c-2 and before has completed; then it
// publishes the steps through chunk c-2.  A block ahead of it in the chain has issued its own chunk
// c-1 and c operations since its chunk c-2 stores, so those have completed as well (at most 63
// operations can be outstanding).  The last publication, after the last frame, is a device-scope
// release.  The row side reads the progress word, then the states and offsets with device-scope
// loads.
template <bool BETA, bool IN_GLOBAL, bool OUT_GLOBAL, bool STREAM>
__device__ __forceinline__ void run_block(const Ctx& cx, const Pointers& P) {
  const int lane = cx.lane, k = cx.k, T = cx.T, U = cx.U;
  const int edge = BETA ? 0 : 63;      // the lane whose label this block passes on
  const int edge_in = BETA ? 63 : 0;   // the lane that takes the producer's label
  const int64_t drow = BETA ? -1 : 1;
  const int64_t r0 = cx.start + (BETA ? T - 1 : 0);  // row of step 0
  const bool sk = cx.sk;
  const int64_t Es = cx.Es;
  int* err = cx.err;
  const int64_t ticks = cx.ticks;

  auto dpp = [&](float old, float x) { return BETA ? dpp_f32<0x130>(old, x) : dpp_f32<0x138>(old, x); };
  // the neighbour's label moved one lane and shifted into this lane's offset (the edge lane, which
  // has no source lane, takes `old`, the producer's value, and a shift of 0)
  auto dpp_shifted = [&](float old, float x, float sh) { return dpp(old, x) + sh; };
  auto row = [&](int64_t step) { return r0 + drow * step; };
  // lowest row of chunk c (its first frame for alpha, its last for beta) and a frame's place in it
  auto chunk_lo = [&](int c) { return BETA ? row((int64_t)(c + 1) * kK) : row(1 + (int64_t)c * kK); };
  auto in_chunk = [&](int i) { return BETA ? kK - 1 - i : i; };
  // what the neighbour lane's value must gain to be in this lane's offset (0 on the edge lane, whose
  // neighbour value comes through the ring, already converted)
  auto lane_shift = [&](float off) { return dpp(off, off) - off; };

  // ---- first frame ----
  float xb, xl, off = 0.0f;
  {
    const int64_t r = row(0);
    const float eb = P.Eb[r];
    const float el = P.E[r * Es + cx.eidx];
    const bool first = BETA ? (k == U) : (k == 0);
    xb = first ? eb : kNeg;
    xl = (first && cx.vl) ? el : kNeg;
    // beta is stored without the frame's own emission (the empty sum 0 at its start states), so that
    // alpha + stored beta is the posterior's exponent with no emission to take out
    if (cx.store) {
      const float2 v0 = BETA ? make_float2((first && cx.vl) ? 0.0f : kNeg, first ? 0.0f : kNeg) : make_float2(xb, xl);
      if (STREAM) {
        const __amdgpu_buffer_rsrc_t ab0 = __builtin_amdgcn_make_buffer_rsrc(cx.ab + r * 128, 0, 512, kRsrcWord3);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{__builtin_bit_cast(uint32_t, v0.x), __builtin_bit_cast(uint32_t, v0.y)},
                                              ab0, lane * 8, 0, kStoreSc1);
      } else {
        *reinterpret_cast<float2*>(cx.ab + (cx.ck ? 0 : r * 128) + 2 * lane) = v0;  // step 0 is always kept
      }
    }
    if (lane == edge) {
      const unsigned long long v = pack(xl, slot_hi(0.0f, -1));
      if (OUT_GLOBAL) gstore(cx.gout + r, v);
      else lstore(cx.lout + (kR - 1), v);
    }
  }

  const int nsteps = T - 1;
  if (nsteps > 0) {
    // build a lead over a producer in another segment: its slots are loaded a chunk ahead
    if (IN_GLOBAL && !cx.no_in) {
      const unsigned long long* p = cx.gin + row(min(2 * kK, T - 1));
      wait_global(p, gload(p), true, ticks, err);
    }
    // label emissions of chunk 0 (register i: the frame of step 1 + i); blank emissions and, across
    // a segment boundary, the neighbour slots of chunk 0, one per lane
    float el[kK];
    {
      const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(P.E + chunk_lo(0) * Es), 0, static_cast<int>(kK * Es * 4), kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kK; ++i)
        el[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(er, cx.eidx * 4, in_chunk(i) * Es * 4, 0));
    }
    const int lk = lane & (kK - 1);
    float ebv = P.Eb[row(1 + lk)];
    const unsigned long long none = pack(kNeg, 0x80u);
    unsigned long long hraw = 0;
    if (IN_GLOBAL) hraw = cx.no_in ? none : gload(cx.gin + row(min(lk, nsteps)));

    auto run_chunk = [&](auto full, int c, int nvalid) {
      constexpr bool FULL = decltype(full)::value;
      // neighbour values of this chunk: lane i < kK holds the producer's frame at step c*kK + i
      const bool need = lane < (FULL ? kK : nvalid);
      const int want = lane == 0 ? c - 1 : c;
      const unsigned long long* lp = cx.lin + ((c * kK + lk - 1) & (kR - 1));
      unsigned long long raw = IN_GLOBAL ? hraw : lload(lp);
      const bool check_cons = !OUT_GLOBAL && cx.lout_live && c >= kR / kK - 1;
      const int cons = check_cons ? __hip_atomic_load(cx.prog_cons, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0;
      const float ebn = P.Eb[row(1 + (int64_t)(c + 1) * kK + lk)];
      if (cx.store) {
        if (STREAM)
          __hip_atomic_store(cx.sig + c * 64 + lane, static_cast<int>(off), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          cx.sig[c * 64 + lane] = static_cast<int>(off);
      }
      if (STREAM && cx.prog && c >= 2) {
        __builtin_amdgcn_s_waitcnt(kWaitVm62);
        if (lane == 0) __hip_atomic_store(cx.prog, (c - 1) * kK + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (IN_GLOBAL) {
        if (__ballot(need && !global_ok(raw)))
          raw = wait_global(cx.gin + row(min(c * kK + lk, nsteps)), raw, need, ticks, err);
        hraw = cx.no_in ? none : gload(cx.gin + row(min((c + 1) * kK + lk, nsteps)));
      } else {
        if (__ballot(need && !lds_ok(raw, want))) raw = wait_lds(lp, raw, need, want, ticks, err);
        if (lane == 0) __hip_atomic_store(cx.prog_self, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      // the consumer of this block's LDS ring must have taken the chunk whose slots this one reuses
      if (check_cons && cons < c - (kR / kK - 1)) wait_progress(cx.prog_cons, c - (kR / kK - 1), ticks, err);
      // the producer's values in the offset of the lane that takes them
      const float hv = slot_value(raw, lanef(off, edge_in));
      const float shift = lane_shift(off);
      // loss only: a resource of no bytes, so the hardware discards the per-frame stores (range check).
      // Checkpointing (alpha, grouped pipeline): the chunk's kept steps 32c + K, 32c + 2K, ... go to
      // consecutive slots; the other frames' stores fall outside the resource and are discarded.
      const bool ck = !BETA && !STREAM && cx.ck;
      const int64_t abase = ck ? (((int64_t)c * kK >> cx.lk) + 1) * 128 : chunk_lo(c) * 128;
      const int arec = cx.store ? (ck ? (kK >> cx.lk) * 512 : kK * 512) : 0;
      const __amdgpu_buffer_rsrc_t ab = __builtin_amdgcn_make_buffer_rsrc(cx.ab + abase, 0, arec, kRsrcWord3);
      const int kmask = (1 << cx.lk) - 1;
      const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(P.E + chunk_lo(c + 1) * Es), 0, static_cast<int>(kK * Es * 4), kRsrcWord3);
      const uint32_t hi = slot_hi(off, c);
      // the same for the edge lane alone (the global ring's store is made by every lane at once)
      const uint32_t hi_edge = OUT_GLOBAL ? slot_hi(lanef(off, edge), c) : 0u;
      unsigned long long* gslot = cx.gout + row(1 + (int64_t)c * kK);
      // LDS ring: the edge lane's slots of this chunk, the other lanes' junk slots
      unsigned long long* lslot = lane == edge ? cx.lout + ((c * kK) & (kR - 1)) : cx.junk + lane;
      // the neighbour of frame 0; each later frame's neighbour is formed as soon as the label value
      // it shifts exists, ahead of that frame's stores
      float n = dpp_shifted(lanef(hv, 0), xl, shift);
      // this lane's byte offset in the chunk's state rows.  In the streamed kernel it is formed anew
      // each chunk (an empty asm hides its value), so the per-frame offsets beyond the 12-bit
      // immediate are added in vector registers; kept from chunk to chunk they were held in scalar
      // registers for the whole loop and reloaded from spill lanes every frame
      int vo = lane * 8;
      if (STREAM) __asm__ volatile("" : "+v"(vo));
#pragma unroll
      for (int i = 0; i < kK; ++i) {
        if (!FULL && i >= nvalid) continue;  // uniform: the last chunk's missing frames
        // blank: lse(blank, neighbour) + emission; label: lse(label, skip ? that sum : blank) + emission
        const float d1 = xb - n;
        const float l1 = log2_fast(1.0f + exp2_fast(-fabsf(d1)));
        const float h1 = __builtin_amdgcn_fmed3f(xb, n, 3.0e38f);
        const float t = h1 + l1;
        const float nb = t + lanef(ebv, i);
        const float a2 = sk ? t : xb;
        const float d2 = xl - a2;
        const float l2 = log2_fast(1.0f + exp2_fast(-fabsf(d2)));
        const float h2 = __builtin_amdgcn_fmed3f(xl, a2, 3.0e38f);
        // beta stores the sums before the emission: t for the blank, h2 + l2 for the label
        const float pl = BETA ? h2 + l2 : 0.0f;
        const float nl = BETA ? pl + el[i] : (h2 + el[i]) + l2;
        if (i + 1 < kK) n = dpp_shifted(lanef(hv, i + 1), nl, shift);
        el[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(er, cx.eidx * 4, in_chunk(i) * Es * 4, 0));
        xb = nb;
        xl = nl;
        const u32x2 st = BETA ? u32x2{__builtin_bit_cast(uint32_t, pl), __builtin_bit_cast(uint32_t, t)}
                              : u32x2{__builtin_bit_cast(uint32_t, xb), __builtin_bit_cast(uint32_t, xl)};
        const int so = !ck ? 0 : (((i + 1) & kmask) == 0 ? (((i + 1) >> cx.lk) - 1) * 512 : 0x40000000);
        __builtin_amdgcn_raw_buffer_store_b64(st, ab, vo + (!ck ? in_chunk(i) * 512 : 0), so, STREAM ? kStoreSc1 : 0);
        // the edge lane's label for the next block: to the global ring every lane stores the edge
        // lane's value (one write to one address), to the LDS ring each lane its own (the other
        // lanes' go to their junk slots); either way the loop keeps one execution mask
        if (OUT_GLOBAL) gstore(gslot + drow * i, pack(lanef(xl, edge), hi_edge));
        else lstore(lslot + i, pack(xl, hi));
      }
      // each lane shifts by its own integer maximum so that its values stay near 0 (a lane without
      // mass keeps its offset)
      const float mx = fmaxf(xb, xl);
      const float d = mx > kNegHalf ? floorf(mx) : 0.0f;
      xb -= d;
      xl -= d;
      off += d;
      ebv = ebn;
    };

    // the first chunk is peeled so that the loop starts from the same memory-counter state it
    // leaves with, and the compiler's waits do not drain the stores and loads in flight
    const int nfull = nsteps / kK, nrem = nsteps % kK;
    if (nfull > 0) run_chunk(std::true_type{}, 0, kK);
    for (int c = 1; c < nfull; ++c) run_chunk(std::true_type{}, c, kK);
    if (nrem > 0) run_chunk(std::false_type{}, nfull, nrem);
  }
  if (STREAM && cx.prog && lane == 0) __hip_atomic_store(cx.prog, T, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

  // ---- likelihood: the block holding the last states (alpha) or the first states (beta) ----
  const bool owner = BETA ? (cx.j == 0) : (cx.j == (U >> 6));
  if (!owner) return;
  float h = kNeg;
  if (!BETA) {  // the producer's label at the last frame, in the offset of lane 0 (the lane it feeds)
    const int step = T - 1;
    const float off0 = lanef(off, 0);
    if (IN_GLOBAL) {
      const unsigned long long* p = cx.gin + row(step);
      h = cx.no_in ? kNeg : slot_value(wait_global(p, gload(p), true, ticks, err), off0);
    } else {
      const unsigned long long* p = cx.lin + ((step - 1) & (kR - 1));
      h = slot_value(wait_lds(p, lload(p), true, chunk_of(step), ticks, err), off0);
    }
  }
  // alpha: blank of pair U with the label of pair U-1; beta: blank of pair 0 with the label of pair 1
  const float n = dpp(h, xl) + lane_shift(off);
  const float fin = lse2(xb, n);
  int rs = 0;
  for (int t = lane; t < T; t += 64) rs += P.rowoff[cx.start + t];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) rs += __shfl_xor(rs, o);
  const int ol = BETA ? 0 : (U & 63);
  if (lane == ol) {
    const bool feasible = fin > kNegHalf;
    const double log2p = (double)rs + (double)off + (double)fin;
    if (!BETA) {
      const bool nan = P.meta[cx.b].flags & kNanInput;
      P.nll[cx.b] = nan ? (double)NAN : (feasible ? -log2p * kLn2 : (double)INFINITY);
      P.lsh[cx.b] = (double)off + (double)fin;
      P.w[cx.b] = utterance_weight(*cx.in, cx.B, cx.b, !nan && !feasible);  // for this group's rows
    } else {
      P.llb[cx.b] = feasible ? log2p : -(double)INFINITY;
    }
  }
}

// The block wave w runs for queue item `item`: one segment of a chain ((chain << 12) | seg: block
// kWaves seg + w), or both chains of an utterance of at most two blocks (kBothChains | (b << 12):
// alpha's blocks on waves 0 .. G-1, beta's on waves G .. 2G-1, so each chain's blocks sit on
// consecutive waves and link through the LDS rings as in a segment).  False: no block for this wave.
__device__ __forceinline__ bool wave_block(const Pointers& P, int item, int w, int& chain, int& j) {
  if (item & kBothChains) {
    const int b = (item & ~kBothChains) >> 12;
    const int G = (P.meta[b].U + 1 + 63) >> 6;
    chain = 2 * b + (w >= G ? 1 : 0);
    j = w >= G ? w - G : w;
    return w < 2 * G;
  }
  chain = item >> 12;
  j = (item & 4095) * kWaves + w;
  return true;
}

// Block j_block of chain (utterance, direction), on wave w of the workgroup.
template <bool STREAM>
__device__ __forceinline__ void run_wave(const Inputs& in, const Layout& L, const Pointers& P, Shared& sh, int chain,
                                         int j_block, int w, int lane, bool store) {
  Ctx cx;
  cx.b = chain >> 1;
  const bool beta = chain & 1;
  const Meta m = P.meta[cx.b];
  cx.T = m.T;
  cx.U = m.U;
  cx.start = m.start;
  const int G = (cx.U + 1 + 63) >> 6;
  cx.j = j_block;
  if (cx.j >= G) return;
  const int j = cx.j, U = cx.U;
  cx.lane = lane;
  cx.k = j * 64 + lane;
  const int k = cx.k;
  const int* lab = P.lab + (int64_t)cx.b * (L.Umax + 1);
  cx.vl = beta ? (k >= 1 && k <= U) : (k < U);
  if (!beta) cx.sk = cx.vl && k >= 1 && lab[k + 1] != lab[k];     // skip 2k-1 -> 2k+1
  else cx.sk = cx.vl && k + 1 <= U && lab[k] != lab[k + 1];       // skip 2k-1 -> 2k+1 (backwards)
  cx.eidx = cx.vl ? (beta ? k : k + 1) : U + 1;
  cx.Es = L.E_stride;
  // neighbours: alpha takes from block j-1 and gives to j+1; beta the other way round
  const bool has_in = beta ? (j + 1 < G) : (j > 0);
  const bool has_out = beta ? (j > 0) : (j + 1 < G);
  const bool in_global = !has_in || (beta ? (w == kWaves - 1) : (w == 0));
  const bool out_global = has_out && (beta ? (w == 0) : (w == kWaves - 1));
  const int dir = beta ? 1 : 0;
  const int64_t Gm = L.Gmax, TT = L.T_total;
  cx.no_in = !has_in;
  const int64_t jin = has_in ? (beta ? j + 1 : j - 1) : j;  // without a producer the slab is never read
  cx.gin = P.ring + (dir * Gm + jin) * TT;
  cx.gout = P.ring + (dir * Gm + j) * TT;
  // LDS ring[w] links waves w and w+1 (alpha) or w+1 and w (beta); ring[kWaves-1] is a sink
  cx.lin = sh.ring[beta ? min(w, kWaves - 2) : max(w - 1, 0)];
  cx.lout_live = has_out && !out_global;
  cx.lout = cx.lout_live ? sh.ring[beta ? w - 1 : w] : sh.ring[kWaves - 1];
  cx.junk = sh.junk[w];
  cx.prog_cons = &sh.prog[beta ? max(w - 1, 0) : min(w + 1, kWaves - 1)];
  cx.prog_self = &sh.prog[w];
  cx.sig = P.sig + ((dir * Gm + j) * L.NCH + P.cbase[cx.b]) * 64;
  // beta: row-indexed; alpha: row-indexed, or (checkpointing) the utterance's kept steps.  The base is
  // one offset from the alpha table, made explicitly uniform: the per-frame stores take it as a
  // buffer resource, which must sit in scalar registers
  cx.ck = !STREAM && !beta && L.K > 1;
  cx.lk = __builtin_ctz(static_cast<unsigned>(L.K));
  const int64_t abo = beta ? (Gm * L.NQ + j * TT) * 128 : (cx.ck ? (j * L.NQ + P.qbase[cx.b]) * 128 : j * TT * 128);
  cx.ab = P.ABa + uniform64(abo);
  cx.store = store;
  cx.prog = (STREAM && (beta ? j == 0 : j == G - 1)) ? P.prog + chain * kProgStride : nullptr;
  cx.err = &P.ctl->err;
  cx.ticks = in.wait_ticks;
  cx.in = &in;
  cx.B = L.B;
  // the recursions are the critical path: their waves win the SIMD over row kernels sharing it
  __builtin_amdgcn_s_setprio(3);
  if (!beta) {
    if (in_global) {
      if (out_global) run_block<false, true, true, STREAM>(cx, P);
      else run_block<false, true, false, STREAM>(cx, P);
    } else {
      if (out_global) run_block<false, false, true, STREAM>(cx, P);
      else run_block<false, false, false, STREAM>(cx, P);
    }
  } else {
    if (in_global) {
      if (out_global) run_block<true, true, true, STREAM>(cx, P);
      else run_block<true, true, false, STREAM>(cx, P);
    } else {
      if (out_global) run_block<true, false, true, STREAM>(cx, P);
      else run_block<true, false, false, STREAM>(cx, P);
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

__global__ void __launch_bounds__(kThreads, 1) chain_workers(Inputs in, Layout L, Pointers P, int group, int store) {
  __shared__ Shared sh;
  // the wave index and the claimed item are wave-uniform: say so, so that every address derived
  // from them stays in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  GroupQ* q = &P.ctl->g[group];
  const int qlen = q->qlen;
  const int* items = P.items + q->itemoff;
  for (;;) {
    // a fresh segment: clear the rings (tag 0 matches no frame) and the progress words
    for (int i = tid; i < kWaves * kR; i += kThreads) (&sh.ring[0][0])[i] = 0ull;
    if (tid < kWaves) sh.prog[tid] = -1;
    if (tid == 0) sh.item = atomicAdd(&q->qcount, 1);
    __syncthreads();
    const int idx = __builtin_amdgcn_readfirstlane(sh.item);
    if (idx >= qlen) break;
    const int item = __builtin_amdgcn_readfirstlane(items[idx]);
    int chain, j;
    if (wave_block(P, item, w, chain, j)) run_wave<false>(in, L, P, sh, chain, j, w, lane, store != 0);
    __syncthreads();
  }
}

// ---- streamed pipeline ----------------------------------------------------------------------------

// bounded wait until a chain has published at least `steps` stored steps
__device__ __forceinline__ void wait_steps(const int* prog, int steps, int64_t ticks, int* err) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < steps) {
    if (out_of_time(t0, ticks, err)) {
      give_up(err);
      return;
    }
    __builtin_amdgcn_s_sleep(32);
  }
}

// Band k of utterance b (L.band frames a side, see kBand): one wave waits until both recursions have
// passed the band (the others wait at the barrier, so polling stays one load per workgroup and
// microsecond), then the band's rows are shared out over the waves, one row per wave at a time.
// The states and offsets the recursions stored on other compute units are read with device-scope
// loads (rows.h: ld_dev), which take the device-coherent copy; a device-scope acquire here instead
// (a cache invalidation per band) measured 25-40 us slower per call.  Each row: the posteriors into
// the wave's LDS, then the gradient row; a row of an utterance with a NaN input, no alignment or a
// zero weight is filled (NaN, or 0 where the weight is 0 -- under zero_infinity an utterance without
// alignment has weight 0), and after any give-up the rows are NaN.
// POST (a split forward): the band's rows get their class sums over z in P.post instead (the weights
// come with the backward, whose gradient rows apply them).  RB: row chunks per lane in flight.
// sums (not POST): the rows' class sums go to P.post as well (a forward whose gradient a later
// update may form again with other weights: packed_ctc_forward_grad).
template <int DT, bool POST, int RB>
__device__ __forceinline__ void row_band(const Inputs& in, const Layout& L, const Pointers& P, void* grad,
                                         uint32_t* lds, int b, int k, int w, int lane, int& cur_b, int sums) {
  const Meta m = P.meta[b];
  const int T = m.T;
  const int band = band_frames(L, T);
  const int ra = T / 2 + k * band, re = min(ra + band, T) - 1;  // its later steps max(t, T-1-t)
  const int n1 = re - ra + 1;                                       // frames ra .. re
  const int lo2 = T - 1 - re, hi2 = min(T - 1 - ra, ra - 1);        // and their mirrors
  const int n = n1 + max(hi2 - lo2 + 1, 0);
  if (w == 0) {
    wait_steps(P.prog + (2 * b) * kProgStride, re + 1, in.wait_ticks, &P.ctl->err);
    wait_steps(P.prog + (2 * b + 1) * kProgStride, re + 1, in.wait_ticks, &P.ctl->err);
  }
  __syncthreads();  // (also keeps the compiler from moving the row's loads above the wait)
  if (w >= n) return;
  const bool broken = __builtin_amdgcn_readfirstlane(gave_up(&P.ctl->err));
  if (POST) {
    // every row of an utterance with an alignment and no NaN input (the backward fills the others,
    // from the loss); a frame without mass gets zero sums
    if (broken || m.flags != 0) return;
    float* acc = reinterpret_cast<float*>(lds);
    for (int i = w; i < n; i += kStreamWaves) {
      const int64_t r = (int64_t)m.start + (i < n1 ? ra + i : lo2 + (i - n1));
      const bool ok = rows::posterior_stream(L, P, acc, r, b, 1.0f, lane);
      float* out = P.post + r * L.C_stride;
      for (int c = lane; c <= m.U; c += 64) out[c] = ok ? acc[c] : 0.0f;
    }
    return;
  }
  // rows are formed unless the call gave up, the weight is 0, or the utterance has a NaN input or no
  // alignment (its recursions are not run; the schedule published them as done); a row whose frame
  // has no mass is filled too
  const int flags = m.flags;
  const float w0 = utterance_weight(in, L.B, b, false);
  const bool live = !broken && flags == 0 && w0 != 0.0f;
  const float fill = !broken && (w0 == 0.0f || (!(flags & kNanInput) && in.zero_infinity)) ? 0.0f : __builtin_nanf("");
  float* acc = reinterpret_cast<float*>(lds);
  for (int i = w; i < n; i += kStreamWaves) {
    const int t = i < n1 ? ra + i : lo2 + (i - n1);
    const int64_t r = (int64_t)m.start + t;
    bool ok = false;
    if (live && sums) {
      // the sums over z alone to P.post (0 where the frame has no mass), then weighted in LDS
      ok = rows::posterior_stream(L, P, acc, r, b, 1.0f, lane);
      float* out = P.post + r * L.C_stride;
      for (int c = lane; c <= m.U; c += 64) {
        const float v = ok ? acc[c] : 0.0f;
        out[c] = v;
        acc[c] = v * w0;
      }
    } else if (live) {
      ok = rows::posterior_stream(L, P, acc, r, b, w0, lane);
    }
    if (ok) rows::dense_row<DT, true, RB>(in, L, P, grad, lds, r, b, w0, lane, cur_b);
    else rows::fill_row<DT>(L, grad, r, fill, lane);
  }
}

// One persistent workgroup per compute unit.  The queue holds the recursion segments (producers
// first, longest utterances first), then the row bands, readiest first.  A segment runs on waves
// 0-3 while the other twelve wait at the barrier; a band runs on all sixteen.  A band is claimed
// only after every segment has been claimed by a running workgroup, so the recursions it waits for
// always progress.
// POST: a split forward (see row_band); the backward then skips its posterior pass.
template <int DT, bool POST, int RB>
__global__ void __launch_bounds__(64 * kStreamWaves, 1) stream_workers(Inputs in, Layout L, Pointers P, void* grad,
                                                                       int per_wave, int sums) {
  if ((POST || sums) && blockIdx.x == 0 && threadIdx.x == 0) P.ctl->post_ready = 1;
  extern __shared__ __attribute__((aligned(16))) unsigned char ssm[];
  Shared& sh = *reinterpret_cast<Shared*>(ssm);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t* lds = reinterpret_cast<uint32_t*>(ssm + ((sizeof(Shared) + 15) & ~size_t(15))) + (int64_t)w * per_wave;
  GroupQ* q = &P.ctl->g[0];
  const int qlen = q->qlen;
  // Two phases, each its own loop, so that the band phase's values are not live (and do not take
  // registers) while the recursion loop runs: first the recursion segments, then the bands; the
  // first claim past the segments is the workgroup's first band.
  int idx;
  for (;;) {
    for (int i = tid; i < kWaves * kR; i += 64 * kStreamWaves) (&sh.ring[0][0])[i] = 0ull;
    if (tid < kWaves) sh.prog[tid] = -1;
    if (tid == 0) sh.item = atomicAdd(&q->qcount, 1);
    __syncthreads();
    idx = __builtin_amdgcn_readfirstlane(sh.item);
    if (idx >= qlen) break;
    if (w < kWaves) {
      const int item = __builtin_amdgcn_readfirstlane(P.items[q->itemoff + idx]);
      int chain, j;
      if (wave_block(P, item, w, chain, j)) run_wave<true>(in, L, P, sh, chain, j, w, lane, true);
    }
    __syncthreads();
  }
  const int nbands = P.ctl->nbands;
  int cur_b = -1;
  while (idx < qlen + nbands) {
    const int2 bd = P.bands[idx - qlen];
    row_band<DT, POST, RB>(in, L, P, grad, lds, __builtin_amdgcn_readfirstlane(bd.x), __builtin_amdgcn_readfirstlane(bd.y),
                       w, lane, cur_b, sums);
    __syncthreads();
    if (tid == 0) sh.item = atomicAdd(&q->qcount, 1);
    __syncthreads();
    idx = __builtin_amdgcn_readfirstlane(sh.item);
  }
}

// LDS words per row wave: class sums, class bitmap and its prefix counts
int64_t stream_words(const Layout& L) { return L.C_stride + 2 * L.Dw; }

size_t stream_lds(const Layout& L) {
  return ((sizeof(Shared) + 15) & ~size_t(15)) + sizeof(uint32_t) * kStreamWaves * (size_t)stream_words(L);
}

}  // namespace

// LDS a workgroup reserves beyond its rings: nearly all of a compute unit's 160 KB, so that no compute
// unit holds two recursion workgroups and no row kernel (each takes some LDS) shares a SIMD with a
// recursion wave -- a streaming wave beside it more than doubles its time per frame
constexpr size_t kChainReserve = 152 * 1024;
static_assert(kChainReserve + sizeof(Shared) <= 160 * 1024 && kChainReserve + sizeof(Shared) + kRowKernelLds > 160 * 1024,
              "one recursion workgroup per compute unit, alone");

hipError_t launch_chains(const Inputs& in, const Layout& L, const Pointers& P, int group, bool store, hipStream_t s) {
  if (L.B == 0 || L.T_total == 0) return hipGetLastError();
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chain_workers), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kChainReserve));
  if (e != hipSuccess) return e;
  // at most one workgroup (a segment of four waves, one per SIMD) per compute unit
  chain_workers<<<cus > 0 ? cus : 256, kThreads, kChainReserve, s>>>(in, L, P, group, store ? 1 : 0);
  return hipGetLastError();
}

// The streamed pipeline takes the 16-bit and float32 inputs of batches whose row waves' LDS fits a
// compute unit beside the recursion rings and whose band queue one workgroup builds quickly.
bool stream_fits(const Inputs& in, const Layout& L) {
  return in.dtype != kF64 && L.B > 0 && L.B <= 2048 && L.T_total > 0 && L.D > 0 && stream_lds(L) <= 150 * 1024;
}

hipError_t launch_stream(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s,
                         bool sums) {
  if (!stream_fits(in, L)) return hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // at least 96 KB: one workgroup per compute unit, so a recursion workgroup is alone on its unit
  const size_t lds = std::max(stream_lds(L), (size_t)96 * 1024);
  const int per_wave = static_cast<int>(stream_words(L));
  auto launch = [&](auto kernel) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
    kernel<<<cus > 0 ? cus : 256, 64 * kStreamWaves, lds, s>>>(in, L, P, grad_out, per_wave, sums && grad_out ? 1 : 0);
    return hipGetLastError();
  };
  // without a gradient (a split forward) the rows' class sums only: no log-prob row is read, so one
  // kernel serves every dtype
  if (!grad_out) return launch(&stream_workers<kF32, true, 4>);
  if (in.dtype == kF32) return launch(&stream_workers<kF32, false, 4>);
  // 16-bit rows of 4096 classes or more: 8 chunks of 16 bytes per lane in flight (half the round trips
  // of a row; the registers fit beside the recursion's), shorter rows 4 (more would only take registers)
  const bool wide = L.D >= 4096;
  if (in.dtype == kF16) return wide ? launch(&stream_workers<kF16, false, 8>) : launch(&stream_workers<kF16, false, 4>);
  return wide ? launch(&stream_workers<kBF16, false, 8>) : launch(&stream_workers<kBF16, false, 4>);
}

}  // namespace pctc
