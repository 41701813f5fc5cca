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
//   - Between blocks that value flows one way (alpha: block j-1 -> j; beta: j+1 -> j).  Four
//     consecutive blocks form a segment run by the four waves of one workgroup (one per SIMD):
//     inside a segment the edge value goes through a 64-slot LDS ring, tagged with its frame;
//     between segments through a global ring slot per frame (one 64-bit system-scope store into a
//     slot that starts empty).  Nobody waits on a later block, so the pipeline has no round trip
//     per frame, only a fill latency per block.  An edge block reads a ring that holds -inf.
//   - Segments are items of one work queue, producers first (see the schedule kernel), claimed by
//     a persistent grid: a claimed segment's producer is always already running.  Every wait is
//     bounded; a wave that gives up raises ctl->err and continues, so the kernel always ends.
//   - base-2 log space (emissions pre-scaled by log2 e) so v_exp_f32 / v_log_f32 apply directly;
//     emissions carry an integer per-row offset, and each block shifts its values by an integer
//     (its maximum) every chunk, so stored values stay near 0; the offsets are stored per
//     (block, chunk) and summed in float64 for the loss.
//   - Per frame a wave issues one 512-byte store of its 128 states (a block-major time series, so
//     the address moves by a constant) and one edge value, both unconditional.
//   - Emissions and global neighbour values are prefetched a 16-frame chunk ahead: the blank
//     emission and the global slot one frame per lane (read back with v_readlane), the lane's own
//     label emission in a ring of 16 registers, each reloaded right after its use.  Loads and
//     stores share one in-order counter on this GPU, so the loop keeps fewer than 64 of them in
//     flight and starts (first chunk peeled) from the state it ends with.
#include "pctc_internal.h"

namespace pctc {

namespace {

constexpr int kK = kChunk;             // frames per chunk (prefetch depth and renormalisation period)
constexpr int kR = 64;                 // LDS ring slots per wave boundary
constexpr int kWaves = 4;              // blocks per segment = waves per workgroup
constexpr unsigned long long kEmpty = ~0ull;
constexpr int kSpinLimit = 1 << 20;    // polls before a wave gives up waiting (about a second)
static_assert(2 * kK + 1 <= kEPad, "emission padding must cover two chunks of prefetch");

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

__device__ __forceinline__ unsigned long long pack_global(float v, float off) {
  return (unsigned long long)__builtin_bit_cast(uint32_t, v) |
         ((unsigned long long)__builtin_bit_cast(uint32_t, off) << 32);
}

// LDS slot: value | (integer offset << 8 | 0x80 | frame & 127) -- the tag tells this frame's entry
// from the one 64 frames earlier and from a cleared slot (tag 0)
__device__ __forceinline__ uint32_t lds_tag(int step) { return 0x80u | (static_cast<uint32_t>(step) & 127u); }

__device__ __forceinline__ unsigned long long pack_lds(float v, float off, int step) {
  const uint32_t hi = (static_cast<uint32_t>(static_cast<int>(off)) << 8) | lds_tag(step);
  return (unsigned long long)__builtin_bit_cast(uint32_t, v) | ((unsigned long long)hi << 32);
}

__device__ __forceinline__ unsigned long long uniform64(unsigned long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (unsigned long long)lo | ((unsigned long long)hi << 32);
}

__device__ __forceinline__ unsigned long long lane64(unsigned long long v, int i) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), i);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), i);
  return (unsigned long long)lo | ((unsigned long long)hi << 32);
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

// bounded wait for a global ring slot; on give-up the neighbour value is -inf
__device__ __noinline__ unsigned long long wait_global(const unsigned long long* p, int* err) {
  unsigned long long v = uniform64(gload(p));
  int spins = 0;
  while (v == kEmpty) {
    if (++spins > kSpinLimit || gave_up(err)) {
      give_up(err);
      return pack_global(kNeg, 0.0f);
    }
    __builtin_amdgcn_s_sleep(2);
    v = uniform64(gload(p));
  }
  return v;
}

// bounded wait for the LDS ring slot of frame `step`
__device__ __noinline__ unsigned long long wait_lds(unsigned long long* p, int step, int* err) {
  unsigned long long v = uniform64(lload(p));
  int spins = 0;
  while (((v >> 32) & 0xffu) != lds_tag(step)) {
    if (++spins > kSpinLimit || gave_up(err)) {
      give_up(err);
      return pack_lds(kNeg, 0.0f, step);
    }
    __builtin_amdgcn_s_sleep(1);
    v = uniform64(lload(p));
  }
  return v;
}

// bounded wait until the consumer wave has finished chunk `c`
__device__ __noinline__ void wait_progress(int* prog, int c, int* err) {
  int spins = 0;
  while (__hip_atomic_load(prog, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < c) {
    if (++spins > kSpinLimit || gave_up(err)) {
      give_up(err);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ float gvalue(unsigned long long v, float off) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(v)) +
         (__builtin_bit_cast(float, static_cast<uint32_t>(v >> 32)) - off);
}

__device__ __forceinline__ float lvalue(unsigned long long v, float off) {
  const int o = static_cast<int>(static_cast<uint32_t>(v >> 32)) >> 8;
  return __builtin_bit_cast(float, static_cast<uint32_t>(v)) + (static_cast<float>(o) - off);
}

struct Shared {
  unsigned long long ring[kWaves][kR];  // ring[w]: between waves w and w+1; ring[kWaves-1]: sink
  int prog[kWaves];
  int item;
};

// Per-wave constants of one block.
struct Ctx {
  int b, T, U, j, k, lane;
  int64_t start;
  bool vl, sk;
  const float* E;           // emission of this lane's label at row 0 (row stride Es)
  const float* Eb;          // blank emission at row 0
  int64_t Es;
  const unsigned long long* gin;  // global ring read by this block (row-indexed)
  unsigned long long* gout;       // global ring written by this block
  unsigned long long* lin;        // LDS ring read by this block
  unsigned long long* lout;       // LDS ring written by this block (a sink if there is no consumer)
  bool lout_live;
  int* prog_cons;
  int* prog_self;
  int* sig;                 // this block's offset per chunk, at the row of the chunk's first frame
  float* ab;                // this block's 128 states per row, at this lane's pair
  int* err;
};

// The recursion of one block, specialised on the direction and on the kinds of its links, so that
// the frame loop carries no branch on any of them.
template <bool BETA, bool IN_GLOBAL, bool OUT_GLOBAL>
__device__ __forceinline__ void run_block(const Ctx& cx, const Pointers& P) {
  const int lane = cx.lane, k = cx.k, T = cx.T, U = cx.U;
  const int edge = BETA ? 0 : 63;
  const int64_t drow = BETA ? -1 : 1;
  const int64_t r0 = cx.start + (BETA ? T - 1 : 0);  // row of step 0
  const bool vl = cx.vl, sk = cx.sk;
  const bool vb = k <= U;
  int* err = cx.err;

  auto dpp = [&](float old, float x) { return BETA ? dpp_f32<0x130>(old, x) : dpp_f32<0x138>(old, x); };
  auto row = [&](int step) { return r0 + drow * step; };
  // lane-distributed loads of chunk c (steps 1 + c*kK ...): lane i holds the blank emission of its
  // frame and, across a segment boundary, the neighbour slot of the frame before; clamped to the
  // utterance
  auto lane_loads = [&](int c, float& eb, unsigned long long& hg) {
    eb = cx.Eb[row(min(1 + c * kK + lane, T - 1)) * cx.Es];
    if (IN_GLOBAL) hg = gload(cx.gin + row(min(c * kK + lane, T - 1)));
  };

  // ---- first frame ----
  float xb, xl, off = 0.0f;
  {
    const int64_t r = row(0);
    const float eb = cx.Eb[r * cx.Es];
    const float el = cx.E[r * cx.Es];
    const bool first = BETA ? (k == U) : (k == 0);
    xb = first ? eb : kNeg;
    xl = (first && vl) ? el : kNeg;
    *reinterpret_cast<float2*>(cx.ab + r * 128) = BETA ? make_float2(xl, xb) : make_float2(xb, xl);
    const float e = lanef(xl, edge);
    if (OUT_GLOBAL) gstore(cx.gout + r, pack_global(e, 0.0f));
    else lstore(cx.lout + 0, pack_lds(e, 0.0f, 0));
  }

  // build a lead over the producer: two chunks across a segment boundary (its slots are prefetched
  // a chunk ahead), a few frames inside a segment (the LDS slot is read one frame ahead)
  if (IN_GLOBAL && T > 1) wait_global(cx.gin + row(min(2 * kK, T - 1)), err);
  if (!IN_GLOBAL && T > 1) {
    const int s0 = min(4, T - 1);
    wait_lds(cx.lin + (s0 & (kR - 1)), s0, err);
  }

  // label emissions: register i holds the frame of step 1 + c*kK + i of the current chunk c and is
  // reloaded with the frame one chunk later right after its use (may read into the row padding)
  float el[kK];
  {
    const float* e = cx.E + row(1) * cx.Es;
#pragma unroll
    for (int i = 0; i < kK; ++i) el[i] = e[drow * i * cx.Es];
  }
  float eb = 0.0f, ebn = 0.0f;
  unsigned long long hg = 0, hgn = 0;
  lane_loads(0, eb, hg);
  bool more = T > 1;
  unsigned long long lnext = 0;  // LDS input: the slot of the previous frame, read one frame ahead
  if (!IN_GLOBAL) lnext = lload(cx.lin);
  float* abp = cx.ab + row(1) * 128;

  auto run_chunk = [&](int c) {
    lane_loads(c + 1, ebn, hgn);
    if (!OUT_GLOBAL && cx.lout_live && c >= 1) wait_progress(cx.prog_cons, c - 1, err);
    cx.sig[row(min(1 + c * kK, T - 1))] = static_cast<int>(off);  // this chunk's offset
    const float* enext = cx.E + row(1 + (c + 1) * kK) * cx.Es;
#pragma unroll
    for (int i = 0; i < kK; ++i) {
      const int step = 1 + c * kK + i;
      if (step >= T) {
        more = false;
        break;
      }
      float h;
      if (IN_GLOBAL) {
        unsigned long long v = lane64(hg, i);
        if (v == kEmpty) v = wait_global(cx.gin + row(step - 1), err);
        h = gvalue(v, off);
      } else {
        unsigned long long v = uniform64(lnext);
        if (((v >> 32) & 0xffu) != lds_tag(step - 1)) v = wait_lds(cx.lin + ((step - 1) & (kR - 1)), step - 1, err);
        h = lvalue(v, off);
        lnext = lload(cx.lin + (step & (kR - 1)));
      }
      const float n = dpp(h, xl);
      const float nb = lse2(xb, n) + lanef(eb, i);
      const float nl = lse3(xl, xb, sk ? n : kNeg) + el[i];
      el[i] = enext[drow * i * cx.Es];
      xb = vb ? nb : kNeg;
      xl = vl ? nl : kNeg;
      *reinterpret_cast<float2*>(abp) = BETA ? make_float2(xl, xb) : make_float2(xb, xl);
      abp += drow * 128;
      const float e = lanef(xl, edge);
      if (OUT_GLOBAL) gstore(cx.gout + row(step), pack_global(e, off));
      else lstore(cx.lout + (step & (kR - 1)), pack_lds(e, off, step));
    }
    if (!IN_GLOBAL && lane == 0) __hip_atomic_store(cx.prog_self, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // shift by the block's integer maximum so the values stay near 0
    const float mx = wave_max(fmaxf(xb, xl));
    const float d = mx > kNegHalf ? floorf(mx) : 0.0f;
    xb -= d;
    xl -= d;
    off += d;
    eb = ebn;
    hg = hgn;
  };

  // the first chunk is peeled so that the loop starts from the same memory-counter state it
  // leaves with, and the compiler's waits do not drain the stores and loads in flight
  int c = 0;
  if (more) run_chunk(c++);
  while (more) run_chunk(c++);

  // ---- likelihood: the block holding the last states (alpha) or the first states (beta) ----
  const bool owner = BETA ? (cx.j == 0) : (cx.j == (U >> 6));
  if (!owner) return;
  float h = kNeg;
  if (!BETA) {
    if (IN_GLOBAL) h = gvalue(wait_global(cx.gin + row(T - 1), err), off);
    else h = lvalue(wait_lds(cx.lin + ((T - 1) & (kR - 1)), T - 1, err), off);
  }
  // alpha: blank of pair U with the label of pair U-1; beta: blank of pair 0 with the label of pair 1
  const float n = dpp(h, xl);
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
      const bool nan = P.meta[cx.b].flags & 1;
      P.nll[cx.b] = nan ? (double)NAN : (feasible ? -log2p * kLn2 : (double)INFINITY);
      P.lsh[cx.b] = (double)off + (double)fin;
    } else {
      P.llb[cx.b] = feasible ? log2p : -(double)INFINITY;
    }
  }
}

// One block (this wave) of segment `seg` of chain (utterance, direction).
__device__ __forceinline__ void run_wave(const Layout& L, const Pointers& P, Shared& sh, int chain, int seg, int w,
                                         int lane) {
  Ctx cx;
  cx.b = chain >> 1;
  const bool beta = chain & 1;
  const Meta m = P.meta[cx.b];
  cx.T = m.T;
  cx.U = m.U;
  cx.start = m.start;
  const int G = (cx.U + 1 + 63) >> 6;
  cx.j = seg * kWaves + w;
  if (cx.j >= G) return;
  const int j = cx.j, U = cx.U;
  cx.lane = lane;
  cx.k = j * 64 + lane;
  const int k = cx.k;
  const int* lab = P.lab + (int64_t)cx.b * (L.Umax + 1);
  cx.vl = beta ? (k >= 1 && k <= U) : (k < U);
  if (!beta) cx.sk = cx.vl && k >= 1 && lab[k + 1] != lab[k];     // skip 2k-1 -> 2k+1
  else cx.sk = cx.vl && k + 1 <= U && lab[k] != lab[k + 1];       // skip 2k-1 -> 2k+1 (backwards)
  const int eidx = cx.vl ? (beta ? k : k + 1) : 0;
  cx.Es = L.E_stride;
  cx.E = P.E + eidx;
  cx.Eb = P.E;
  // neighbours: alpha takes from block j-1 and gives to j+1; beta the other way round
  const bool has_in = beta ? (j + 1 < G) : (j > 0);
  const bool has_out = beta ? (j > 0) : (j + 1 < G);
  const bool in_global = !has_in || (beta ? (w == kWaves - 1) : (w == 0));
  const bool out_global = has_out && (beta ? (w == 0) : (w == kWaves - 1));
  const int dir = beta ? 1 : 0;
  const int64_t Gm = L.Gmax, TT = L.T_total;
  cx.gin = has_in ? P.ring + (dir * Gm + (beta ? j + 1 : j - 1)) * TT : P.nring;
  cx.gout = P.ring + (dir * Gm + j) * TT;
  // LDS ring[w] links waves w and w+1 (alpha) or w+1 and w (beta); ring[kWaves-1] is a sink
  cx.lin = sh.ring[beta ? min(w, kWaves - 2) : max(w - 1, 0)];
  cx.lout_live = has_out && !out_global;
  cx.lout = cx.lout_live ? sh.ring[beta ? w - 1 : w] : sh.ring[kWaves - 1];
  cx.prog_cons = &sh.prog[beta ? max(w - 1, 0) : min(w + 1, kWaves - 1)];
  cx.prog_self = &sh.prog[w];
  cx.sig = P.sig + (dir * Gm + j) * TT;
  cx.ab = P.AB + (dir * Gm + j) * TT * 128 + 2 * lane;
  cx.err = &P.ctl->err;
  if (!beta) {
    if (in_global) {
      if (out_global) run_block<false, true, true>(cx, P);
      else run_block<false, true, false>(cx, P);
    } else {
      if (out_global) run_block<false, false, true>(cx, P);
      else run_block<false, false, false>(cx, P);
    }
  } else {
    if (in_global) {
      if (out_global) run_block<true, true, true>(cx, P);
      else run_block<true, true, false>(cx, P);
    } else {
      if (out_global) run_block<true, false, true>(cx, P);
      else run_block<true, false, false>(cx, P);
    }
  }
}

__global__ void __launch_bounds__(256, 1) chain_workers(Layout L, Pointers P) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int qlen = P.ctl->qlen;
  for (;;) {
    // a fresh segment: clear the rings (tag 0 matches no frame) and the progress words
    for (int i = tid; i < kWaves * kR; i += 256) (&sh.ring[0][0])[i] = 0ull;
    if (tid < kWaves) sh.prog[tid] = -1;
    if (tid == 0) sh.item = atomicAdd(&P.ctl->qcount, 1);
    __syncthreads();
    const int idx = sh.item;
    if (idx >= qlen) break;
    const int item = P.items[idx];
    run_wave(L, P, sh, item >> 12, item & 4095, w, lane);
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_chains(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s) {
  (void)in;
  if (L.B == 0 || L.T_total == 0) return hipGetLastError();
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // one workgroup (a segment of four waves, one per SIMD) per compute unit
  chain_workers<<<cus > 0 ? cus : 256, 256, 0, s>>>(L, P);
  return hipGetLastError();
}

}  // namespace pctc
