// Per-utterance preparation, the emission gather, loss finalisation and reductions.
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities", Triton file: `_extended_labels` (state s is the blank for even s and
// targets[b][(s-1)/2] for odd s), `_frame_log_probs` (the per-frame log probabilities at the states'
// classes, computed in float32), `_PackedCTCLoss.forward` (zero_infinity on the loss) and
// `_beta_grad_kernel` (the gradient scale, zero under zero_infinity for an infinite loss); `ctc.py`
// `forward_packed` (sum, and the mean of each loss over its clamped target length, then the batch mean).
#include "rows.h"

namespace pctc {

namespace {

__global__ void fill_i32_kernel(int* p, int64_t n, int v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void zero_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// One workgroup per utterance: clamp the metadata so that every later access stays in bounds,
// write the U+1 distinct class ids of the extended label sequence, claim the utterance's rows.
__device__ __forceinline__ void class_maps(const Layout& L, const Pointers& P, int b, uint32_t* cw, int* wsum,
                                           const int* lab);
__device__ void schedule_body(const Layout& L, const Pointers& P, int sort, int groups, int bands, int* sh, int nhist,
                              int ocap);

// classes: the class maps too (the streamed pipeline).  Workgroups past the B utterances' (streamed
// pipeline) clear the recursion rings' ring_words words instead: every slot starts unwritten (its
// written mark clear), and nothing else in this launch touches them.
__global__ void __launch_bounds__(256) prep_kernel(Inputs in, Layout L, Pointers P, int classes, int64_t ring_words) {
  if (blockIdx.x >= L.B) {
    const int64_t fills = gridDim.x - L.B;
    int* q = reinterpret_cast<int*>(P.ring);
    for (int64_t i = (blockIdx.x - L.B) * 256 + threadIdx.x; i < ring_words; i += fills * 256) q[i] = 0;
    return;
  }
  const int b = blockIdx.x;
  __shared__ Meta m;
  if (threadIdx.x == 0) {
    int64_t start = load_index(in.cu_seqlens, in.index_flags & 1, b);
    int64_t T = load_index(in.lengths, in.index_flags & 2, b);
    int64_t U = load_index(in.target_lengths, in.index_flags & 8, b);
    if (T < 0) T = 0;
    if (start < 0 || start > L.T_total) {
      start = 0;
      T = 0;
    }
    if (T > L.T_total - start) T = L.T_total - start;
    if (U < 0) U = 0;
    if (U > L.Umax) U = L.Umax;
    if (U > in.target_width) U = in.target_width;
    m.start = static_cast<int>(start);
    m.T = static_cast<int>(T);
    m.U = static_cast<int>(U);
    m.flags = 0;
    P.meta[b] = m;
  }
  __syncthreads();
  const Meta mm = m;
  int* lab = P.lab + (int64_t)b * (L.Umax + 1);
  // classes (the streamed pipeline's setup): the labels are kept in LDS too, after the class maps'
  // 2 Dw words, and read back from there
  extern __shared__ __attribute__((aligned(16))) uint32_t pcw[];
  int* sl = reinterpret_cast<int*>(pcw + 2 * L.Dw);
  const bool t64 = in.index_flags & 4;
  for (int j = threadIdx.x; j <= mm.U; j += blockDim.x) {
    int64_t c = in.blank;
    if (j > 0) {
      c = load_index(in.targets, t64, (int64_t)b * in.target_width + (j - 1));
      if (c < 0) c = 0;
      if (c >= L.D) c = L.D - 1;
    }
    lab[j] = static_cast<int>(c);
    if (classes) sl[j] = static_cast<int>(c);
  }
  const int* lr = classes ? sl : lab;
  for (int t = threadIdx.x; t < mm.T; t += blockDim.x) P.rowmap[mm.start + t] = b;
  // No alignment fits when the utterance has fewer frames than its labels need: one frame per label
  // and a blank frame between two equal neighbours (the skip is barred between equal ids).  Such an
  // utterance is marked here; its recursions are not run, since no state path reaches the end.
  // (U + repeats <= 2U - 1, so only an utterance with fewer frames than that needs the count)
  __shared__ int repeats;
  if (threadIdx.x == 0) repeats = 0;
  if (mm.U > 0 && mm.T < 2 * mm.U - 1) {  // uniform
    __syncthreads();  // (also: this workgroup's label writes above are visible to its loads below)
    int rep = 0;
    for (int j = threadIdx.x + 1; j < mm.U; j += blockDim.x) rep += lr[j + 1] == lr[j];
    if (rep) atomicAdd(&repeats, rep);
    __syncthreads();
  }
  if (threadIdx.x == 0 && mm.U > 0 && mm.T < mm.U + repeats) {
    // what the recursions' owner blocks would record: an infinite loss and its weight (the gather
    // turns both to those of a NaN loss if it meets a NaN at one of the utterance's columns)
    P.meta[b].flags = kNoAlignment;
    P.nll[b] = (double)INFINITY;
    P.lsh[b] = 0.0;
    P.llb[b] = -(double)INFINITY;
    P.w[b] = utterance_weight(in, L.B, b, true);
  }
  if (classes) {  // the class maps of this utterance (its labels are in LDS)
    __shared__ int wsum[4];
    class_maps(L, P, b, pcw, wsum, sl);
  }
}

// One wave per owned row: the log2 emissions of the row at the utterance's U+1 label columns,
// minus the row's integer offset floor(max over those columns), so that the recursions work on
// values near 0.  Lanes read their labels' values straight from the row, so only the memory
// sectors that hold a label are fetched (the offset needs nothing else of the row).  A wave takes
// a contiguous range of rows: the label ids of its utterance stay in registers from row to row,
// and for U+1 <= 512 the values too, so the table row is written once.
constexpr int kGLab = 8;  // label columns per lane held in registers
// LDS per wave of the streamed gather's class-ordered rows: two rows of 64 kGLab floats
constexpr size_t kGatherRowsLds = 2 * 64 * kGLab * sizeof(float);

template <int DT>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  if constexpr (DT == kF32) return static_cast<const float*>(p)[i];
  else if constexpr (DT == kF64) return static_cast<float>(static_cast<const double*>(p)[i]);
  else if constexpr (DT == kF16) return static_cast<float>(static_cast<const _Float16*>(p)[i]);
  else return __builtin_bit_cast(float, static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
}

// element c of a row that starts at `row` (uniform): a 32-bit offset from a uniform base, one register
// per address; NT: non-temporal (the line is not kept in the caches)
template <int DT, bool NT>
__device__ __forceinline__ float ld_row(const void* row, int c) {
  constexpr uint32_t esz = DT == kF64 ? 8 : (DT == kF32 ? 4 : 2);
  const char* p = static_cast<const char*>(row) + static_cast<uint32_t>(c) * esz;  // (c >= 0: a zero-extended offset)
  if constexpr (DT == kF32) {
    const float* q = reinterpret_cast<const float*>(p);
    return NT ? __builtin_nontemporal_load(q) : *q;
  } else if constexpr (DT == kF64) {
    const double* q = reinterpret_cast<const double*>(p);
    return static_cast<float>(NT ? __builtin_nontemporal_load(q) : *q);
  } else if constexpr (DT == kF16) {
    const _Float16* q = reinterpret_cast<const _Float16*>(p);
    return static_cast<float>(NT ? __builtin_nontemporal_load(q) : *q);
  } else {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
    return __builtin_bit_cast(float, static_cast<uint32_t>(NT ? __builtin_nontemporal_load(q) : *q) << 16);
  }
}


// The label ids of the utterance a wave is on (kept while its rows follow one another); in the
// class-ordered form (gather_rows, SORTED), the utterance's classes in increasing order and the rank
// of each label's class instead
struct GatherCur {
  int b = -1, U = 0, ncls = 0;
  const int* lab = nullptr;
  int col[kGLab];
  int dm[kGLab];
};

template <int DT>
__device__ __forceinline__ void gather_row(const Inputs& in, const Layout& L, const Pointers& P, int64_t r, int b,
                                           GatherCur& g, int lane) {
  if (b != g.b) {
    g.U = P.meta[b].U;
    g.lab = P.lab + (int64_t)b * (L.Umax + 1);
#pragma unroll
    for (int k = 0; k < kGLab; ++k) g.col[k] = g.lab[min(lane + 64 * k, g.U)];
    g.b = b;
  }
  const int U = g.U;
  float* E = P.E + r * L.E_stride;
  const int64_t row = r * L.D;
  float mx = kNeg;
  int nan = 0;
  if (U < 64 * kGLab) {
    float v[kGLab];
#pragma unroll
    for (int k = 0; k < kGLab; ++k) v[k] = ld1<DT>(in.log_probs, row + g.col[k]);  // all loads in flight
#pragma unroll
    for (int k = 0; k < kGLab; ++k) {
      const bool ok = lane + 64 * k <= U;
      float x = v[k] * kLog2e;
      nan |= ok && (x != x);
      x = fmaxf(x, kNeg);  // -inf (and NaN, flagged above) become the finite sentinel
      v[k] = x;
      if (ok) mx = fmaxf(mx, x);
    }
    mx = wave_max(mx);
    const float off = mx > kNegHalf ? floorf(mx) : 0.0f;
#pragma unroll
    for (int k = 0; k < kGLab; ++k)
      if (lane + 64 * k <= U) E[lane + 64 * k] = v[k] - off;
    if (lane == 0) P.rowoff[r] = static_cast<int>(off);
  } else {  // long targets: two passes over the table row
    for (int j = lane; j <= U; j += 64) {
      float x = ld1<DT>(in.log_probs, row + g.lab[j]) * kLog2e;
      nan |= (x != x);
      x = fmaxf(x, kNeg);
      mx = fmaxf(mx, x);
      E[j] = x;
    }
    mx = wave_max(mx);
    const float off = mx > kNegHalf ? floorf(mx) : 0.0f;
    for (int j = lane; j <= U; j += 64) E[j] -= off;
    if (lane == 0) P.rowoff[r] = static_cast<int>(off);
  }
  if (lane == 0) {
    E[U + 1] = kNeg;  // the column of label states that do not exist
    P.Eb[r] = E[0];   // (this lane wrote E[0] above)
  }
  if (nan) {
    atomicOr(&P.meta[b].flags, kNanInput);
    if (P.meta[b].flags & kNoAlignment) {  // its loss is NaN, not +inf (no recursion will say so)
      P.nll[b] = (double)NAN;
      P.w[b] = utterance_weight(in, L.B, b, false);
    }
  }
}

template <int DT>
__global__ void __launch_bounds__(256) gather_kernel(Inputs in, Layout L, Pointers P, int group, void* gaps) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t j0, j1;
  wave_share(P, group, wid, (int64_t)gridDim.x * 4, j0, j1);
  GatherCur g;
  group_rows(P, group, j0, j1, [&](int64_t r, int b) { gather_row<DT>(in, L, P, r, b, g, lane); });
  if (gaps) {  // rows owned by no utterance get a zero gradient here
    const int64_t waves = (int64_t)gridDim.x * 4;
    for (int64_t r = wid; r < L.T_total; r += waves)
      if (__builtin_amdgcn_readfirstlane(row_owner(L, P, r)) < 0) rows::fill_row<DT>(L, gaps, r, 0.0f, lane);
  }
}

// ---- the streamed gather, two rows at a time where they share an utterance ----

// a row of a long target (U + 1 > 64 kGLab): two passes over its label columns in label order
template <int DT>
__device__ __forceinline__ void gather_row_long(const Inputs& in, const Layout& L, const Pointers& P, int64_t r, int b,
                                             int U, int lane) {
  constexpr int64_t esz = DT == kF64 ? 8 : (DT == kF32 ? 4 : 2);
  const int* lab = P.lab + (int64_t)b * (L.Umax + 1);
  const void* row = static_cast<const char*>(in.log_probs) + r * L.D * esz;
  float* E = P.E + r * L.E_stride;
  float mx = kNeg;
  int nan = 0;
  for (int j = lane; j <= U; j += 64) {
    float x = ld_row<DT, false>(row, lab[j]) * kLog2e;
    nan |= (x != x);
    x = fmaxf(x, kNeg);
    mx = fmaxf(mx, x);
    E[j] = x;
  }
  mx = wave_max(mx);
  const float off = mx > kNegHalf ? floorf(mx) : 0.0f;
  for (int j = lane; j <= U; j += 64) E[j] -= off;  // (each lane its own entries)
  if (lane == 0) {
    P.rowoff[r] = static_cast<int>(off);
    E[U + 1] = kNeg;  // the column of label states that do not exist
    P.Eb[r] = E[0];   // (this lane wrote E[0] above)
  }
  if (nan) {
    atomicOr(&P.meta[b].flags, kNanInput);
    if (P.meta[b].flags & kNoAlignment) {  // its loss is NaN, not +inf (no recursion will say so)
      P.nll[b] = (double)NAN;
      P.w[b] = utterance_weight(in, L.B, b, false);
    }
  }
}

// The utterance's columns for a wave (one round trip: its label count, label ids or class bitmap,
// label ranks): label order, lane i of load k takes label 64 k + i (the blank where there is none);
// class order (SORTED), it takes the class of rank 64 k + i and dm holds each label's class rank.
template <bool SORTED>
__device__ __forceinline__ void gather_prepare(const Inputs& in, const Layout& L, const Pointers& P, int b,
                                               GatherCur& g, int lane, float* wl) {
  const int Umax = static_cast<int>(L.Umax);
  int pre[kGLab];
  if (SORTED) {
    const int Dw = static_cast<int>(L.Dw);
    const uint32_t* gb = P.cbits + (int64_t)b * Dw;
    const int* gp = P.cpref + (int64_t)b * Dw;
    const int* dmap = P.dmap + (int64_t)b * (Umax + 1);
#pragma unroll
    for (int k = 0; k < kGLab; ++k) pre[k] = dmap[min(lane + 64 * k, Umax)];
    g.U = P.meta[b].U;
    g.ncls = gp[Dw - 1] + __builtin_popcount(gb[Dw - 1]);
    // the classes by rank: the bitmap's set bits in order, written at their ranks (the first
    // 64 kGLab: a longer target is gathered by gather_row_long, and the wave's LDS holds no more)
    for (int i = lane; i < Dw; i += 64) {
      uint32_t bits = gb[i];
      int k = gp[i];
      while (bits && k < 64 * kGLab) {
        const int e = __builtin_ctz(bits);
        bits &= bits - 1u;
        wl[k++] = static_cast<float>(32 * i + e);  // (exact: class ids are below 2^24)
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < kGLab; ++k) {
      g.col[k] = static_cast<int>(wl[min(lane + 64 * k, g.ncls - 1)]);
      g.dm[k] = lane + 64 * k <= g.U ? pre[k] : 0;  // (ranks past U: stale; every LDS read stays in bounds)
    }
  } else {
    const int* lab = P.lab + (int64_t)b * (Umax + 1);
#pragma unroll
    for (int k = 0; k < kGLab; ++k) pre[k] = lab[min(lane + 64 * k, Umax)];
    g.U = P.meta[b].U;
    g.ncls = g.U + 1;
    g.lab = lab;
#pragma unroll
    for (int k = 0; k < kGLab; ++k) g.col[k] = lane + 64 * k <= g.U ? pre[k] : in.blank;  // (ids past U: stale)
  }
  g.b = b;
}

// NR (1 or 2) consecutive rows r .. r + NR - 1 of utterance g.b, U + 1 <= 64 kGLab: every load of
// both rows in flight at once, then each row's offset and table row.
// SORTED: the values at the utterance's distinct classes, read in increasing column order (lane i of
// load k takes the class of rank 64 k + i), so that each 128-byte line is requested by one load,
// and with non-temporal loads: the log probs are read again only by the gradient rows, much later,
// and their lines kept in the caches would displace the emission table written here, which the
// recursions read next (large_vocab: the stream launch 16 us faster; with the values read in label
// order, where one line serves several loads, the non-temporal form fetched lines again and the
// gather took 30 us longer).  The values go to the label order through the wave's LDS (wl: NR x
// 64 kGLab floats) and the rank of each label's class (the class maps, class_maps).
template <int DT, bool SORTED, int NR>
__device__ __forceinline__ void gather_rows(const Inputs& in, const Layout& L, const Pointers& P, int64_t r,
                                            GatherCur& g, int lane, float* wl) {
  const int U = g.U, n = g.ncls, b = g.b;
  constexpr int64_t esz = DT == kF64 ? 8 : (DT == kF32 ? 4 : 2);
  float v[NR][kGLab];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const void* row = static_cast<const char*>(in.log_probs) + (r + j) * L.D * esz;
#pragma unroll
    for (int k = 0; k < kGLab; ++k) v[j][k] = ld_row<DT, SORTED>(row, g.col[k]);
  }
  int nan = 0;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float mx = kNeg;
#pragma unroll
    for (int k = 0; k < kGLab; ++k) {
      const bool ok = lane + 64 * k < n;
      float x = v[j][k] * kLog2e;
      nan |= ok && (x != x);
      x = fmaxf(x, kNeg);  // -inf (and NaN, flagged above) become the finite sentinel
      v[j][k] = x;
      if (ok) mx = fmaxf(mx, x);
    }
    mx = wave_max(mx);
    const float off = mx > kNegHalf ? floorf(mx) : 0.0f;
    float* E = P.E + (r + j) * L.E_stride;
    float eb;
    if (SORTED) {
      // LDS operations of one wave complete in order: these writes follow the reads of this area's
      // previous row (or of the class list) and precede the reads below
      float* w = wl + j * (64 * kGLab);
#pragma unroll
      for (int k = 0; k < kGLab; ++k)
        if (lane + 64 * k < n) w[lane + 64 * k] = v[j][k] - off;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < kGLab; ++k)
        if (lane + 64 * k <= U) E[lane + 64 * k] = w[g.dm[k]];
      eb = w[g.dm[0]];
    } else {
#pragma unroll
      for (int k = 0; k < kGLab; ++k)
        if (lane + 64 * k <= U) E[lane + 64 * k] = v[j][k] - off;
      eb = v[j][0] - off;
    }
    if (lane == 0) {
      P.rowoff[r + j] = static_cast<int>(off);
      E[U + 1] = kNeg;  // the column of label states that do not exist
      P.Eb[r + j] = eb;
    }
  }
  if (nan) {
    atomicOr(&P.meta[b].flags, kNanInput);
    if (P.meta[b].flags & kNoAlignment) {  // its loss is NaN, not +inf (no recursion will say so)
      P.nll[b] = (double)NAN;
      P.w[b] = utterance_weight(in, L.B, b, false);
    }
  }
}

// Streamed pipeline (one group): the rows in their natural order, each wave a contiguous share, its
// rows' owners found 64 at a time (as row_owner does); rows owned by no utterance get a zero gradient
// when `gaps` is given.
// With sched (nhist, ocap: see schedule_body), workgroup 0 builds the schedule instead, beside the
// gathering workgroups: it reads only what prep wrote, and nothing here reads what it writes.
// SORTED: rows of up to 64 kGLab labels are read in class order (gather_rows); taken for rows
// of at least kSortedRowBytes, where it pays (on short rows the lines serve every load anyway, and
// its registers cost occupancy: small and char_level 8 us slower)
// TWO: two rows of an utterance in flight at once, for rows of at least kTwoRowBytes (on shorter
// rows the loads of one row are few and the second row's registers cost more occupancy than its
// latency saves: small 1.7 us slower, asr_bpe 4.7 us faster)
constexpr int64_t kSortedRowBytes = 4096, kTwoRowBytes = 1024;
template <int DT, bool SORTED, bool TWO>
__global__ void __launch_bounds__(256) gather_stream_kernel(Inputs in, Layout L, Pointers P, void* gaps, int sched,
                                                            int nhist, int ocap) {
  extern __shared__ __attribute__((aligned(16))) int gsh[];  // (at least 4 waves x 64 kGLab words)
  if (sched && blockIdx.x == 0) {
    schedule_body(L, P, 1, 1, 1, gsh, nhist, ocap);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t first = sched ? 1 : 0;
  const int64_t waves = ((int64_t)gridDim.x - first) * 4;
  const int64_t wid = ((int64_t)blockIdx.x - first) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t per = (L.T_total + waves - 1) / waves;
  const int64_t r0 = min(wid * per, L.T_total), r1 = min(r0 + per, L.T_total);
  GatherCur g;  // the utterance whose columns this wave holds
  float* wl = reinterpret_cast<float*>(gsh) + (threadIdx.x >> 6) * (kGatherRowsLds / 4);
  for (int64_t q = r0; q < r1; q += 64) {
    const int n = static_cast<int>(min((int64_t)64, r1 - q));
    int own = lane < n ? P.rowmap[q + lane] : -1;
    if (own < 0 || own >= L.B) {
      own = -1;
    } else {
      const Meta m = P.meta[own];
      if (q + lane < m.start || q + lane >= (int64_t)m.start + m.T) own = -1;
    }
    for (int i = 0; i < n;) {  // (everything wave-uniform)
      const int b = __builtin_amdgcn_readlane(own, i);
      if (b < 0) {
        if (gaps) rows::fill_row<DT>(L, gaps, q + i, 0.0f, lane);
        ++i;
        continue;
      }
      // a new utterance: its columns, taken as if its target were short (the loads stay in bounds either
      // way); a long target (U + 1 > 64 kGLab) goes row by row in label order (gather_row, cursor gl)
      if (b != g.b) gather_prepare<SORTED>(in, L, P, b, g, lane, wl);
      if (g.U >= 64 * kGLab) {
        gather_row_long<DT>(in, L, P, q + i, b, g.U, lane);
        ++i;
        continue;
      }
      const bool two = TWO && i + 1 < n && __builtin_amdgcn_readlane(own, i + 1) == b;
      if (two) gather_rows<DT, SORTED, 2>(in, L, P, q + i, g, lane, wl);
      else gather_rows<DT, SORTED, 1>(in, L, P, q + i, g, lane, wl);
      i += two ? 2 : 1;
    }
  }
}

// Per utterance (one workgroup): the bitmap of the classes its extended labels use (the blank and
// its labels), the number of classes before each bitmap word, and for each label index j the rank
// of lab[j] among the present classes.  The gradient rows add each class's posterior at its
// column through these ranks.  cw: 2 Dw words of LDS.
// lab: the utterance's U + 1 labels (LDS in the prep launch, the workspace copy otherwise)
__device__ __forceinline__ void class_maps(const Layout& L, const Pointers& P, int b, uint32_t* cw, int* wsum,
                                           const int* lab) {
  const int tid = threadIdx.x;
  const int Dw = static_cast<int>(L.Dw);
  const int U = P.meta[b].U;
  for (int i = tid; i < Dw; i += 256) cw[i] = 0u;
  __syncthreads();
  for (int j = tid; j <= U; j += 256) atomicOr(&cw[lab[j] >> 5], 1u << (lab[j] & 31));
  __syncthreads();
  uint32_t* gbits = P.cbits + (int64_t)b * Dw;
  int* gpref = P.cpref + (int64_t)b * Dw;
  // exclusive prefix count of set bits over the words, 256 words at a time
  int carry = 0;
  for (int w0 = 0; w0 < Dw; w0 += 256) {
    const int i = w0 + tid;
    const uint32_t bits = i < Dw ? cw[i] : 0u;
    int v = __builtin_popcount(bits);
    // inclusive scan within the wave
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o);
      if (lane >= o) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int before = carry;
    for (int k = 0; k < wave; ++k) before += wsum[k];
    if (i < Dw) {
      const int pref = before + v - __builtin_popcount(bits);
      gbits[i] = bits;
      gpref[i] = pref;
      cw[Dw + i] = static_cast<uint32_t>(pref);
    }
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  __syncthreads();
  // rank of each label's class
  int* dmap = P.dmap + (int64_t)b * (L.Umax + 1);
  for (int j = tid; j <= U; j += 256) {
    const int c = lab[j], wi = c >> 5;
    dmap[j] = static_cast<int>(cw[Dw + wi]) + __builtin_popcount(cw[wi] & ((1u << (c & 31)) - 1u));
  }
}

__global__ void __launch_bounds__(256) classes_kernel(Layout L, Pointers P) {
  if (skipped(P)) return;
  extern __shared__ uint32_t cw[];  // Dw bitmap words, then Dw prefix counts
  __shared__ int wsum[4];
  class_maps(L, P, blockIdx.x, cw, wsum, P.lab + (int64_t)blockIdx.x * (L.Umax + 1));
}

// Losses after zero_infinity, gradient weights and the sum / mean reduction (one workgroup,
// a fixed summation tree so that the reduced value is reproducible).
__global__ void __launch_bounds__(256) weights_kernel(Inputs in, Layout L, Pointers P, void* losses_out,
                                                      void* reduced_out, int rows) {
  __shared__ double part[256];
  __shared__ int nonunit;
  if (threadIdx.x == 0) nonunit = 0;
  __syncthreads();
  double acc = 0.0;
  const int64_t B = L.B;
  // a wave of the recursions gave up a bounded wait: the results of the call are unspecified, and
  // every loss and the reduced value say so with NaN
  const bool broken = P.ctl->err != 0;
  for (int64_t b = threadIdx.x; b < B; b += blockDim.x) {
    const double nll = broken ? (double)NAN : P.nll[b];
    const bool inf = nll == (double)INFINITY;
    const double loss = (in.zero_infinity && inf) ? 0.0 : nll;
    if (losses_out) {  // in the loss type of the input dtype: float64 for float64 inputs, else float32
      if (in.dtype == kF64) static_cast<double*>(losses_out)[b] = loss;
      else static_cast<float*>(losses_out)[b] = static_cast<float>(loss);
    }
    // the target length of the reductions is the caller's value, as the page's reductions divide by it
    int64_t U = load_index(in.target_lengths, in.index_flags & 8, b);
    const double Uc = U > 1 ? (double)U : 1.0;
    double w = grad_scale_of(in, b);
    if (rows == kRowsUpdate && w != 1.0) nonunit = 1;
    if (in.reduction == 2) w /= (double)B * Uc;
    if (in.zero_infinity && inf) w = 0.0;
    P.w[b] = static_cast<float>(w);
    acc += in.reduction == 2 ? loss / Uc : loss;
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  // the record of what grad_out holds: rows for unit upstream weights (a forward that wrote them), or
  // not (any other call; an update with other weights rewrites the rows); an update with unit
  // weights and the forward's zero_infinity and reduction leaves them as they are
  if (threadIdx.x == 0) {
    const int mark = 1 + in.zero_infinity + 2 * in.reduction;
    if (rows == kRowsUpdate) {
      const bool unit = !nonunit && P.ctl->rows_for == mark;
      P.ctl->unit = unit ? 1 : 0;
      if (!unit) P.ctl->rows_for = 0;
    } else {
      P.ctl->rows_for = rows == kRowsMark ? mark : 0;
    }
  }
  if (threadIdx.x == 0 && reduced_out && in.reduction != 0) {
    double v = part[0];
    if (in.reduction == 2) v = B > 0 ? v / (double)B : (double)NAN;
    if (broken) v = (double)NAN;
    if (in.dtype == kF64) *static_cast<double*>(reduced_out) = v;
    else *static_cast<float*>(reduced_out) = static_cast<float>(v);
  }
}

__global__ void __launch_bounds__(256) reduce_kernel(const float* losses, const void* tl, bool i64, int64_t B,
                                                     int reduction, float* out) {
  __shared__ double part[256];
  double acc = 0.0;
  for (int64_t b = threadIdx.x; b < B; b += blockDim.x) {
    const int64_t U = load_index(tl, i64, b);
    acc += reduction == 2 ? (double)losses[b] / (U > 1 ? (double)U : 1.0) : (double)losses[b];
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    double v = part[0];
    if (reduction == 2) v = B > 0 ? v / (double)B : (double)NAN;
    *out = static_cast<float>(v);
  }
}

// Work queue of the recursions (one workgroup).  Utterances are ordered by frame count, longest
// first, so that the longest chains start first; each utterance contributes its alpha segments
// (kSegWaves 64-pair state blocks each) in producer order (segment 0 first) interleaved with its beta
// segments in producer order (last segment first).  A segment only ever waits on its producer,
// which sits earlier in the queue, so segments claimed in queue order can always finish.
// Frameless utterances get their loss here.
constexpr int kBandBuckets = 4096;  // LDS buckets of 16 ready steps (a counting sort up to 65535 frames)
__device__ void build_bands(const Layout& L, const Pointers& P, const int* sT, const int* sU, int* first, int* hist,
                            int nhist, int* owner, int ocap);
// LDS words for the band queue's owner map: a bound on the number of bands, at most 8192 (beyond
// it, each band finds its utterance by a binary search instead)
__host__ __device__ inline int owner_cap(const Layout& L) {
  const int64_t n = (L.T_total + L.B) / 32 + 2 * L.B + 1;
  return static_cast<int>(n < 8192 ? n : 8192);
}

// exclusive prefix sum of a[0..n) in place, with a[n] = the total (one workgroup; every thread calls
// it); wsum: blockDim / 64 words of LDS
__device__ void block_exclusive_scan(int* a, int n, int* wsum) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
  int s = 0;
  for (int i = i0; i < i1; ++i) s += a[i];
  const int lane = tid & 63, wave = tid >> 6;
  int v = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int run = v - s;
  for (int k = 0; k < wave; ++k) run += wsum[k];
  for (int i = i0; i < i1; ++i) {
    const int x = a[i];
    a[i] = run;
    run += x;
  }
  if (tid == 0) {
    int t = 0;
    for (int k = 0; k < nt / 64; ++k) t += wsum[k];
    a[n] = t;
  }
  __syncthreads();
}

// the same for two arrays of n at once (one pair of barriers); wsum: 2 blockDim / 64 words
__device__ void block_exclusive_scan2(int* a, int* c, int n, int* wsum) {
  const int tid = threadIdx.x, nt = blockDim.x, nw = nt / 64;
  const int per = (n + nt - 1) / nt;
  const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
  int s = 0, u = 0;
  for (int i = i0; i < i1; ++i) {
    s += a[i];
    u += c[i];
  }
  const int lane = tid & 63, wave = tid >> 6;
  int v = s, x = u;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o), y = __shfl_up(x, o);
    if (lane >= o) {
      v += t;
      x += y;
    }
  }
  if (lane == 63) {
    wsum[wave] = v;
    wsum[nw + wave] = x;
  }
  __syncthreads();
  int run = v - s, run2 = x - u;
  for (int k = 0; k < wave; ++k) {
    run += wsum[k];
    run2 += wsum[nw + k];
  }
  for (int i = i0; i < i1; ++i) {
    const int p = a[i], q = c[i];
    a[i] = run;
    c[i] = run2;
    run += p;
    run2 += q;
  }
  if (tid == 0) {
    int t = 0, t2 = 0;
    for (int k = 0; k < nw; ++k) {
      t += wsum[k];
      t2 += wsum[nw + k];
    }
    a[n] = t;
    c[n] = t2;
  }
  __syncthreads();
}

// sh (dynamic LDS): sort ? [T (B) | order (B) | U (B) | rows before each sorted position (B + 1) |
// queue entries before each sorted position (B + 1) | bands: first band of each utterance (B + 1) |
// band buckets] : unused
// bands: nhist band buckets and an owner map of up to ocap bands in sh (see schedule_lds)
__device__ void schedule_body(const Layout& L, const Pointers& P, int sort, int groups, int bands, int* sh, int nhist,
                              int ocap) {
  __shared__ int wsum[32];
  __shared__ int gfirst[kMaxGroups + 1];
  const int B = static_cast<int>(L.B);
  const int tid = threadIdx.x, nt = blockDim.x;
  // segments per direction; an utterance without alignment gets none (prep recorded its loss)
  auto nseg_of = [](int U, int flags) {
    return (flags & kNoAlignment) ? 0 : (((U + 1 + 63) >> 6) + kSegWaves - 1) / kSegWaves;
  };
  // queue items of an utterance with frames: one for both chains when each has at most two blocks
  // (they fill at most the four waves of one workgroup), else one per segment and direction
  auto items_of = [&](int U, int flags) {
    if (flags & kNoAlignment) return 0;
    return ((U + 1 + 63) >> 6) <= 2 ? 1 : 2 * nseg_of(U, flags);
  };
  // group g ends where the groups so far hold the share of the rows below (each group at least one
  // utterance); its segments in sorted order, each utterance's producers first.  With three
  // groups (cut points measured on uniformly spread lengths): the longest recursions with about
  // half the rows on the caller's stream, then the middle, then the short ones, whose gathers,
  // recursions and rows all finish under the long recursions
  const float share[kMaxGroups][kMaxGroups] = {{1.0f, 1.0f, 1.0f}, {0.15f, 1.0f, 1.0f}, {0.45f, 0.75f, 1.0f}};
  // first slot of each utterance's chunks in the per-lane offset table: chunk c holds steps
  // 1 + c kChunk .. (c + 1) kChunk, so an utterance of T frames has ceil((T - 1) / kChunk) chunks
  // and, with alpha checkpointing (interval K), the first slot of each utterance's kept steps
  // 0, K, 2K, ... <= T - 1
  const int K = static_cast<int>(L.K);
  auto chunks_of = [](int T) { return T > 1 ? (T - 1 + kChunk - 1) / kChunk : 0; };
  auto kept_of = [K](int T) { return T > 0 ? (T - 1) / K + 1 : 0; };
  // a frameless utterance gets its loss here
  auto frameless = [&](int b, const Meta& m) {
    if (m.T == 0) {
      P.nll[b] = m.U == 0 ? 0.0 : (double)INFINITY;
      P.llb[b] = m.U == 0 ? 0.0 : -(double)INFINITY;
    }
  };
  if (sort) {
    int* sT = sh;
    int* order = sh + B;
    int* sU = sh + 2 * B;
    int* cT = sh + 3 * B;
    int* cS = sh + 4 * B + 1;
    // the metadata, read once; the chunk and kept-step counts are scanned in the space the sorted
    // sums take afterwards
    for (int b = tid; b < B; b += nt) {
      const Meta m = P.meta[b];
      sT[b] = m.T;
      sU[b] = (m.flags & kNoAlignment) ? -1 : m.U;  // -1: no alignment
      cT[b] = chunks_of(m.T);
      cS[b] = kept_of(m.T);
      frameless(b, m);
    }
    __syncthreads();
    block_exclusive_scan2(cT, cS, B, wsum);
    for (int b = tid; b <= B; b += nt) {
      P.cbase[b] = cT[b];
      P.qbase[b] = cS[b];
    }
    // rank by frame count, longest first (ties by index), four counts per LDS read
    for (int b = tid; b < B; b += nt) {
      const int Tb = sT[b];
      int rank = 0, c = 0;
      const bool vec = (reinterpret_cast<uintptr_t>(sT) & 15) == 0;  // (the dynamic LDS is 16-aligned)
      auto before4 = [&](const int4 q, int c0) {
        return (q.x > Tb || (q.x == Tb && c0 < b)) + (q.y > Tb || (q.y == Tb && c0 + 1 < b)) +
               (q.z > Tb || (q.z == Tb && c0 + 2 < b)) + (q.w > Tb || (q.w == Tb && c0 + 3 < b));
      };
      for (; vec && c + 16 <= B; c += 16) {  // four reads in flight
        const int4 q0 = *reinterpret_cast<const int4*>(sT + c), q1 = *reinterpret_cast<const int4*>(sT + c + 4);
        const int4 q2 = *reinterpret_cast<const int4*>(sT + c + 8), q3 = *reinterpret_cast<const int4*>(sT + c + 12);
        rank += before4(q0, c) + before4(q1, c + 4) + before4(q2, c + 8) + before4(q3, c + 12);
      }
      for (; vec && c + 4 <= B; c += 4) rank += before4(*reinterpret_cast<const int4*>(sT + c), c);
      for (; c < B; ++c) rank += sT[c] > Tb || (sT[c] == Tb && c < b);
      order[rank] = b;
    }
    __syncthreads();
    // frames and queue entries per sorted position, then their prefix sums
    for (int i = tid; i < B; i += nt) {
      const int b = order[i];
      cT[i] = sT[b];
      cS[i] = sT[b] > 0 ? items_of(sU[b], sU[b] < 0 ? kNoAlignment : 0) : 0;
    }
    __syncthreads();
    block_exclusive_scan2(cT, cS, B, wsum);
    if (tid == 0) {
      // the cuts: group g takes positions [p0, p1), p1 the first position past p0 where the rows so far
      // reach the group's share, at most B - (groups after it)
      const int64_t total = cT[B];
      int pos = 0;
      for (int g = 0; g < kMaxGroups; ++g) {
        GroupQ q{};
        if (g < groups) {
          const int p0 = pos, keep = groups - 1 - g;
          int p1 = B;
          if (g < groups - 1) {
            const int64_t goal = static_cast<int64_t>(share[groups - 1][g] * (double)total);
            int lo = p0 + 1, hi = B - keep;  // smallest p1 in [p0 + 1, B - keep] with cT[p1] >= goal
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if ((int64_t)cT[mid] >= goal) hi = mid;
              else lo = mid + 1;
            }
            p1 = lo;
          }
          q.itemoff = cS[p0];
          q.qlen = cS[p1] - cS[p0];
          q.first = p0;
          q.count = p1 - p0;
          q.nrows = cT[p1] - cT[p0];
          gfirst[g] = p0;
          pos = p1;
        }
        P.ctl->g[g] = q;
      }
      gfirst[groups] = B;
      P.ctl->err = 0;
      P.ctl->ngroups = groups;
      P.ctl->post_ready = 0;
    }
    __syncthreads();
    for (int i = tid; i < B; i += nt) {
      const int b = order[i];
      P.order[i] = b;
      int g = 0;
      while (g + 1 < groups && gfirst[g + 1] <= i) ++g;
      P.cum[i] = cT[i] - cT[gfirst[g]];
      P.gid[b] = g;
      if (sT[b] == 0 || sU[b] < 0) continue;
      int n = cS[i];
      if (((sU[b] + 1 + 63) >> 6) <= 2) {
        P.items[n] = kBothChains | (b << 12);
        continue;
      }
      const int nseg = nseg_of(sU[b], 0);
      for (int j = 0; j < nseg; ++j) {
        P.items[n++] = ((2 * b) << 12) | j;
        P.items[n++] = ((2 * b + 1) << 12) | (nseg - 1 - j);
      }
    }
  } else {  // too many utterances to sort: identity order, serial (groups is 1 here)
    for (int b = tid; b < B; b += nt) {
      const Meta m = P.meta[b];
      P.cbase[b] = chunks_of(m.T);
      P.qbase[b] = kept_of(m.T);
      frameless(b, m);
    }
    __syncthreads();
    block_exclusive_scan2(P.cbase, P.qbase, B, wsum);
    for (int i = tid; i < B; i += nt) P.order[i] = i;
    if (tid == 0) {
      int64_t total = 0;
      for (int i = 0; i < B; ++i) total += P.meta[i].T;
      int n = 0, pos = 0;
      int64_t done = 0;
      for (int g = 0; g < kMaxGroups; ++g) {
        GroupQ q{};
        if (g < groups) {
          const int p0 = pos;
          const int64_t goal = g == groups - 1 ? total : static_cast<int64_t>(share[groups - 1][g] * (double)total);
          int p1 = p0;
          const int keep = groups - 1 - g;  // utterances to leave for the groups after this one
          do {
            done += P.meta[p1].T;
            ++p1;
          } while (p1 < B - keep && (done < goal || g == groups - 1));
          q.itemoff = n;
          q.first = p0;
          q.count = p1 - p0;
          int rows = 0;
          for (int i = p0; i < p1; ++i) {
            const Meta m = P.meta[i];
            P.cum[i] = rows;
            P.gid[i] = g;
            rows += m.T;
            if (m.T == 0) continue;
            const int nseg = nseg_of(m.U, m.flags);
            for (int j = 0; j < nseg; ++j) {
              P.items[n++] = ((2 * i) << 12) | j;
              P.items[n++] = ((2 * i + 1) << 12) | (nseg - 1 - j);
            }
          }
          q.qlen = n - q.itemoff;
          q.nrows = rows;
          pos = p1;
        }
        P.ctl->g[g] = q;
      }
      P.ctl->err = 0;
      P.ctl->ngroups = groups;
      P.ctl->post_ready = 0;
    }
  }
  if (bands) {  // streamed pipeline (sorted, one group): the queue of row bands
    __syncthreads();
    build_bands(L, P, sh, sh + 2 * B, sh + 5 * B + 2, sh + 6 * B + 3, nhist, sh + 6 * B + 4 + nhist, ocap);
  }
}

__global__ void __launch_bounds__(1024) schedule_kernel(Layout L, Pointers P, int sort, int groups, int bands,
                                                        int nhist, int ocap) {
  extern __shared__ __attribute__((aligned(16))) int ssh[];
  schedule_body(L, P, sort, groups, bands, ssh, nhist, ocap);
}

// Streamed pipeline: the queue of row bands (built by the schedule workgroup).  Band k of utterance b
// (T frames; `band` = band_frames(L, T) frames a side) holds the frames whose later recursion step
// max(t, T-1-t) lies in [T/2 + k band, T/2 + (k+1) band), and is ready once both recursions have
// stored min(T/2 + (k+1) band, T) steps.  The bands are queued by that step.  Also clears the
// progress words.
__device__ __forceinline__ int bands_of(int T, int band) { return T > 0 ? ((T + 1) / 2 + band - 1) / band : 0; }

// bands of an utterance with T frames that become ready before step `key`
__device__ __forceinline__ int bands_before(int T, int key, int band) {
  if (T <= 0) return 0;
  const int n = bands_of(T, band);
  if (key > T) return n;
  const int x = key - T / 2;
  if (x <= 0) return 0;
  return min(max((x + band - 1) / band - 1, 0), n);
}

// (one workgroup) sT: the frame counts (LDS, B); sU: the label counts, -1 for an utterance without
// alignment, whose bands are ready at once and go first; first: B + 1 words of LDS
__device__ void build_bands(const Layout& L, const Pointers& P, const int* sT, const int* sU, int* first, int* hist,
                            int nhist, int* owner, int ocap) {
  const int B = static_cast<int>(L.B);
  const int tid = threadIdx.x, nt = blockDim.x;
  __shared__ int bsum[16];
  __shared__ int tmax;
  if (tid == 0) tmax = 0;
  // progress words start at 0; an utterance without alignment has no recursions to wait for
  for (int i = tid; i < 2 * B; i += nt) P.prog[i * kProgStride] = sU[i >> 1] < 0 ? sT[i >> 1] : 0;
  for (int b = tid; b < B; b += nt) first[b] = bands_of(sT[b], band_frames(L, sT[b]));
  __syncthreads();
  for (int b = tid; b < B; b += nt) atomicMax(&tmax, sT[b]);
  block_exclusive_scan(first, B, bsum);
  const int N = first[B];
  if (tid == 0) P.ctl->nbands = N;
  // each band's utterance: from an owner map written utterance by utterance (one thread each) when
  // it fits and the utterances are short (32 bands on average: the serial fill costs less than the
  // binary searches it replaces), else by a binary search over the first bands
  const bool map = N <= ocap && N <= 32 * B;
  if (map) {
    for (int b = tid; b < B; b += nt)
      for (int i = first[b]; i < first[b + 1]; ++i) owner[i] = b;
    __syncthreads();
  }
  auto band_of = [&](int i, int& b, int& k, int& key) {  // entry i: utterance, band, ready step
    if (map) {
      b = owner[i];
    } else {
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      b = lo;
    }
    k = i - first[b];
    key = sU[b] < 0 ? 0 : min(sT[b] / 2 + (k + 1) * band_frames(L, sT[b]), sT[b]);
  };
  const int nb = (tmax >> 4) + 1;  // buckets of 16 steps
  if (nb <= nhist) {
    // counting sort by 16-step bucket of the ready step; within a bucket, in order of arrival (bands
    // ready within 16 steps of each other: the order only schedules, it changes no result)
    for (int q = tid; q <= nb; q += nt) hist[q] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += nt) {
      int b, k, key;
      band_of(i, b, k, key);
      atomicAdd(&hist[key >> 4], 1);
    }
    __syncthreads();
    block_exclusive_scan(hist, nb, bsum);
    for (int i = tid; i < N; i += nt) {
      int b, k, key;
      band_of(i, b, k, key);
      P.bands[atomicAdd(&hist[key >> 4], 1)] = make_int2(b, k);
    }
    return;
  }
  // longer utterances: the exact order by ready step, ties by utterance (and by band within an
  // utterance without alignment, all of whose bands are ready at step 0), each band's place counted
  auto before = [&](int c, int key) {
    const int bc = band_frames(L, sT[c]);
    return sU[c] < 0 ? (key > 0 ? bands_of(sT[c], bc) : 0) : bands_before(sT[c], key, bc);
  };
  for (int i = tid; i < N; i += nt) {
    int b, k, key;
    band_of(i, b, k, key);
    int rank = sU[b] < 0 ? k : 0;
    for (int c = 0; c < B; ++c) {
      const int bf = before(c, key);
      rank += bf;
      if (c < b) rank += before(c, key + 1) - bf;  // a band of c ready at the same step
    }
    P.bands[rank] = make_int2(b, k);
  }
}

// dynamic LDS of the schedule: the sorted path's arrays (setup: also the first band per utterance,
// nhist + 1 band buckets and an owner map of ocap words)
size_t schedule_lds(const Layout& L, bool sort, bool setup, int nhist, int ocap) {
  return sort ? sizeof(int) * (5 * (size_t)L.B + 2 + (setup ? (size_t)L.B + 1 + nhist + 1 + ocap : 0)) : 0;
}

// The schedule in the gather launch: at most 512 utterances, and LDS that leaves the gather's
// residency (7 workgroups of 4 waves per compute unit, set by its registers) as it is: buckets for
// ready steps up to the batch's frame count (at most kBandBuckets), and an owner map as far as the
// rest allows (beyond it, the bands find their utterance by binary search)
constexpr size_t kGatherSchedLds = 22 * 1024;
struct GatherSched {
  bool on = false;
  int nhist = 0, ocap = 0;
  size_t lds = 0;
};
GatherSched gather_sched(const Layout& L) {
  GatherSched g;
  if (L.B < 1 || L.B > 512) return g;
  g.nhist = static_cast<int>(std::min<int64_t>(kBandBuckets, L.T_total / 16 + 2));
  const size_t base = schedule_lds(L, true, true, g.nhist, 0);
  if (base > kGatherSchedLds) return g;
  g.ocap = static_cast<int>(std::min<int64_t>(owner_cap(L), (int64_t)((kGatherSchedLds - base) / sizeof(int))));
  g.lds = std::max(kRowKernelLds, schedule_lds(L, true, true, g.nhist, g.ocap));
  g.on = true;
  return g;
}

int grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g > 4096) g = 4096;
  return g < 1 ? 1 : static_cast<int>(g);
}

}  // namespace

hipError_t launch_prep(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s, bool setup) {
  // setup (streamed pipeline): the recursion rings are cleared by workgroups of the same launch and
  // the class maps are formed by the prep workgroups.  The row map is written for owned rows only
  // (row_owner tells the others).
  const int64_t ring_words = setup ? 2 * 2 * L.Gmax * L.T_total : 0;
  if (L.B > 0) {
    const size_t lds = setup ? sizeof(uint32_t) * (2 * (size_t)L.Dw + (size_t)L.Umax + 1) : 0;
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    const int fills = ring_words > 0 ? std::min(grid_for(ring_words, 256), 1024) : 0;
    prep_kernel<<<static_cast<unsigned>(L.B + fills), 256, lds, s>>>(in, L, P, setup ? 1 : 0, ring_words);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const Inputs& in, const Layout& L, const Pointers& P, int group, hipStream_t s, void* gaps) {
  if (L.T_total == 0 || L.B == 0) return hipGetLastError();
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // 64 waves per compute unit (more than fit at once: the shares are finer, so the last waves end
  // sooner; measured against 32 and 128 per unit on every workload), each on a contiguous share of
  // the group's rows.  The kernel uses no LDS, but takes some so that it is never placed beside a
  // recursion workgroup (which reserves the rest of a compute unit's LDS)
  const int grid = 16 * (cus > 0 ? cus : 256);
  const size_t lds = kRowKernelLds;
  if (in.dtype == kF32) gather_kernel<kF32><<<grid, 256, lds, s>>>(in, L, P, group, gaps);
  else if (in.dtype == kF64) gather_kernel<kF64><<<grid, 256, lds, s>>>(in, L, P, group, gaps);
  else if (in.dtype == kF16) gather_kernel<kF16><<<grid, 256, lds, s>>>(in, L, P, group, gaps);
  else gather_kernel<kBF16><<<grid, 256, lds, s>>>(in, L, P, group, gaps);
  return hipGetLastError();
}

bool schedule_in_gather(const Layout& L) { return gather_sched(L).on; }

hipError_t launch_gather_stream(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s, void* gaps) {
  const GatherSched gs = gather_sched(L);
  if (L.T_total == 0 && !gs.on) return hipGetLastError();
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // as in the grouped gather: 16 workgroups per compute unit, each wave a contiguous share of the
  // rows (plus the schedule's workgroup)
  const int grid = 16 * (cus > 0 ? cus : 256) + (gs.on ? 1 : 0);
  const bool sorted = L.D * (in.dtype == kF32 ? 4 : 2) >= kSortedRowBytes;
  // (class-ordered rows: two rows' values per wave in LDS)
  const size_t lds = std::max(gs.on ? gs.lds : kRowKernelLds, sorted ? 4 * kGatherRowsLds : 0);
  auto go = [&](auto kern) {
    if (lds > 48 * 1024) {
      hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e2 != hipSuccess) return e2;
    }
    kern<<<grid, 256, lds, s>>>(in, L, P, gaps, gs.on ? 1 : 0, gs.nhist, gs.ocap);
    return hipGetLastError();
  };
  const bool two = L.D * (in.dtype == kF32 ? 4 : 2) >= kTwoRowBytes;
  if (in.dtype == kF32)
    return sorted ? go(&gather_stream_kernel<kF32, true, true>)
                  : (two ? go(&gather_stream_kernel<kF32, false, true>) : go(&gather_stream_kernel<kF32, false, false>));
  if (in.dtype == kF64) return go(&gather_stream_kernel<kF64, false, false>);
  if (in.dtype == kF16)
    return sorted ? go(&gather_stream_kernel<kF16, true, true>)
                  : (two ? go(&gather_stream_kernel<kF16, false, true>) : go(&gather_stream_kernel<kF16, false, false>));
  return sorted ? go(&gather_stream_kernel<kBF16, true, true>)
                : (two ? go(&gather_stream_kernel<kBF16, false, true>) : go(&gather_stream_kernel<kBF16, false, false>));
}

hipError_t launch_classes(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s) {
  (void)in;
  if (L.B == 0) return hipGetLastError();
  const size_t lds = 2 * sizeof(uint32_t) * (size_t)L.Dw;
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&classes_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  classes_kernel<<<static_cast<unsigned>(L.B), 256, lds, s>>>(L, P);
  return hipGetLastError();
}

hipError_t launch_schedule(const Inputs& in, const Layout& L, const Pointers& P, int groups, hipStream_t s, bool setup) {
  (void)in;
  if (L.B == 0) {  // nothing to queue: the control words still start clean for the status read
    zero_u32_kernel<<<1, 256, 0, s>>>(reinterpret_cast<uint32_t*>(P.ctl), sizeof(ChainCtl) / 4);
    return hipGetLastError();
  }
  // every ring slot starts unwritten (zero: the written mark 0x80 of its high word is clear); a
  // block publishes (value, offset << 8 | 0x80 | tag) into it once
  // (setup: cleared with the row map, in the prep launch)
  const int64_t words = 2 * 2 * L.Gmax * L.T_total;
  if (words > 0 && !setup) fill_i32_kernel<<<grid_for(words, 256), 256, 0, s>>>(reinterpret_cast<int*>(P.ring), words, 0);
  const int sort = L.B <= 7168 ? 1 : 0;  // (the sorted path's LDS: 5 B words, at most 140 KB)
  if (setup && !sort) return hipErrorInvalidValue;  // the band queue needs the sorted frame counts
  const int nhist = kBandBuckets, ocap = owner_cap(L);
  const size_t lds = schedule_lds(L, sort, setup, nhist, ocap);
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&schedule_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  schedule_kernel<<<1, 1024, lds, s>>>(L, P, sort, groups, setup ? 1 : 0, nhist, ocap);
  return hipGetLastError();
}

hipError_t launch_weights(const Inputs& in, const Layout& L, const Pointers& P, void* losses_out, void* reduced_out,
                          hipStream_t s, int rows) {
  weights_kernel<<<1, 256, 0, s>>>(in, L, P, losses_out, reduced_out, rows);
  return hipGetLastError();
}

hipError_t launch_reduce(const float* losses, const void* target_lengths, bool i64, int64_t B, int reduction, float* out,
                         hipStream_t s) {
  reduce_kernel<<<1, 256, 0, s>>>(losses, target_lengths, i64, B, reduction, out);
  return hipGetLastError();
}

}  // namespace pctc
