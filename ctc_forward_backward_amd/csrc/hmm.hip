// Dense log-space HMM forward: the HMM module of the POPCORNBENCH page "HMM forward, Kimi-K2.6
// l2_p50".  The initial, transition and emission log weights are each normalised by their
// log-sum-exp (over states, over next states per row, over symbols per row); per observation
// sequence alpha_0 = log pi + log B[:, o_0], alpha_t[j] = logsumexp_i(alpha_{t-1}[i] + log A[i, j]) +
// log B[j, o_t], and the log-likelihood is the log-sum-exp of the last alpha over all states.
// It is the dense-topology form of the recursion the CTC path runs banded.
//
// Design for gfx950 (not the page's one-thread-per-state CUDA block):
//   - One wave per sequence.  For S <= 16, four lanes per state (below); otherwise lane j holds
//     state j (S <= 64).  A step is a matrix-vector product
//     in the log semiring: lane j needs every alpha_{t-1}[i].  v_readlane broadcasts alpha_{t-1}[i]
//     as a scalar operand, so lane j forms alpha[i] + log A[i][j] against its own column of A held
//     in registers, takes the maximum and sums 2^(x - max): no LDS traffic and no barrier in the
//     step.
//   - The normalised emission table (S x O) sits in LDS, written once per workgroup; each lane reads
//     its entry for the step's symbol at the start of the step (the read completes while the
//     log-sum-exp is formed).  Symbols are loaded 64 frames at a time, one per lane, the next 64
//     prefetched a block ahead, and broadcast by v_readlane.
//   - Base-2 log space (inputs times log2 e); unreachable values are held at -1e30 so that no
//     difference of infinities arises; a log-likelihood below -1e29 is reported as -inf.
#include <cstdint>

#include "pctc_internal.h"

namespace pctc {

namespace {

constexpr float kFloorH = -1e30f;

__device__ __forceinline__ float bcast(float v, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
}

__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// base-2 log-sum-exp over the wave's lanes (lanes without a state hold kFloorH)
__device__ __forceinline__ float wave_lse2(float v) {
  const float m = wave_max64(v);
  return m + log2_fast(wave_sum64(exp2_fast(v - m)));
}

__device__ __forceinline__ int symbol(const void* obs, int i64, int64_t i, int O) {
  int64_t o = i64 ? static_cast<const int64_t*>(obs)[i] : static_cast<int64_t>(static_cast<const int32_t*>(obs)[i]);
  return static_cast<int>(o < 0 ? 0 : (o >= O ? O - 1 : o));  // out-of-range symbols are a precondition violation
}

template <int SMAX>
__global__ void __launch_bounds__(256) hmm_forward_kernel(const float* __restrict__ log_init,
                                                          const float* __restrict__ log_trans,
                                                          const float* __restrict__ log_emit, const void* obs,
                                                          int obs_i64, int64_t B, int64_t T, int S, int O,
                                                          float* __restrict__ out) {
  extern __shared__ float le2[];  // (S, O) normalised base-2 emission log weights
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // emission rows, one wave per row at a time
  for (int s = w; s < S; s += 4) {
    const float* row = log_emit + (int64_t)s * O;
    float m = kFloorH;
    for (int o = lane; o < O; o += 64) m = fmaxf(m, row[o] * kLog2e);
    m = wave_max64(m);
    float sum = 0.0f;
    for (int o = lane; o < O; o += 64) sum += exp2_fast(row[o] * kLog2e - m);
    const float lse = m + log2_fast(wave_sum64(sum));
    for (int o = lane; o < O; o += 64) le2[s * O + o] = fmaxf(row[o] * kLog2e - lse, kFloorH);
  }
  // lane j: log2 pi[j] and column j of log2 A (row i normalised by its own log-sum-exp)
  const bool on = lane < S;
  float pi = kFloorH;
  if (on) pi = fmaxf(log_init[lane] * kLog2e, kFloorH);
  const float pil = wave_lse2(pi);
  pi = on ? fmaxf(pi - pil, kFloorH) : kFloorH;
  float rowlse = 0.0f;
  if (on) {
    const float* row = log_trans + (int64_t)lane * S;
    float m = kFloorH;
    for (int k = 0; k < S; ++k) m = fmaxf(m, row[k] * kLog2e);
    float sum = 0.0f;
    for (int k = 0; k < S; ++k) sum += exp2_fast(row[k] * kLog2e - m);
    rowlse = m + log2_fast(sum);
  }
  float a2[SMAX];
#pragma unroll
  for (int i = 0; i < SMAX; ++i) {
    const float ri = bcast(rowlse, i);
    a2[i] = kFloorH;
    if (i < S && on) a2[i] = fmaxf(log_trans[(int64_t)i * S + lane] * kLog2e - ri, kFloorH);
  }
  __syncthreads();  // the emission table is complete

  const int64_t b = (int64_t)blockIdx.x * 4 + w;
  if (b >= B) return;
  const int64_t base = b * T;
  int sym = symbol(obs, obs_i64, base + min((int64_t)lane, T - 1), O);  // frames [0, 64)
  int nxt = sym;
  // every lane reads an entry inside the table; lanes without a state discard theirs
  const int erow = on ? lane * O : 0;
  float alpha = fmaxf(pi + le2[erow + __builtin_amdgcn_readlane(sym, 0)], kFloorH);
  if (!on) alpha = kFloorH;
  for (int64_t t = 1; t < T; ++t) {
    const int k = static_cast<int>(t & 63);
    if (k == 0) sym = nxt;
    if (k == 1) nxt = symbol(obs, obs_i64, base + min(t - 1 + 64 + lane, T - 1), O);  // frames [t-1+64, t-1+128)
    const float e = le2[erow + __builtin_amdgcn_readlane(sym, k)];
    float x[SMAX];
#pragma unroll
    for (int i = 0; i < SMAX; ++i) x[i] = bcast(alpha, i) + a2[i];
    float m = x[0];
#pragma unroll
    for (int i = 1; i < SMAX; ++i) m = fmaxf(m, x[i]);
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < SMAX; ++i) sum += exp2_fast(x[i] - m);
    alpha = on ? fmaxf(m + log2_fast(sum) + e, kFloorH) : kFloorH;
  }
  const float ll = wave_lse2(alpha);
  if (lane == 0) out[b] = ll < -1e29f ? -INFINITY : ll * kLn2;
}

// S <= 16: four lanes per state.  Lane 4j + q holds state j and takes the terms i = q, q+4, q+8,
// q+12 of its log-sum-exp (alpha_{t-1}[i] fetched by ds_bpermute from lane 4i); the maximum and
// then the sum of a state's terms are reduced over its quad with quad-permute DPP moves, so every
// lane of the quad ends with the state's new alpha.  A step is then a quarter of the
// one-lane-per-state work.
template <int CTRL>
__device__ __forceinline__ float quad_swap(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                                               CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float from_lane(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src * 4, __builtin_bit_cast(int, x)));
}

__global__ void __launch_bounds__(256) hmm_forward16_kernel(const float* __restrict__ log_init,
                                                            const float* __restrict__ log_trans,
                                                            const float* __restrict__ log_emit, const void* obs,
                                                            int obs_i64, int64_t B, int64_t T, int S, int O,
                                                            float* __restrict__ out) {
  extern __shared__ float le2[];  // (S, O) normalised base-2 emission log weights
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int s = w; s < S; s += 4) {
    const float* row = log_emit + (int64_t)s * O;
    float m = kFloorH;
    for (int o = lane; o < O; o += 64) m = fmaxf(m, row[o] * kLog2e);
    m = wave_max64(m);
    float sum = 0.0f;
    for (int o = lane; o < O; o += 64) sum += exp2_fast(row[o] * kLog2e - m);
    const float lse = m + log2_fast(wave_sum64(sum));
    for (int o = lane; o < O; o += 64) le2[s * O + o] = fmaxf(row[o] * kLog2e - lse, kFloorH);
  }
  const int j = lane >> 2, q = lane & 3;
  const bool on = j < S;
  const bool lead = on && q == 0;  // the lane that stands for state j in sums over states
  float pi = kFloorH;
  if (on) pi = fmaxf(log_init[j] * kLog2e, kFloorH);
  const float pil = wave_lse2(lead ? pi : kFloorH);
  pi = on ? fmaxf(pi - pil, kFloorH) : kFloorH;
  float rowlse = 0.0f;  // lane 4i: the log-sum-exp of transition row i
  if (lead) {
    const float* row = log_trans + (int64_t)j * S;
    float m = kFloorH;
    for (int k = 0; k < S; ++k) m = fmaxf(m, row[k] * kLog2e);
    float sum = 0.0f;
    for (int k = 0; k < S; ++k) sum += exp2_fast(row[k] * kLog2e - m);
    rowlse = m + log2_fast(sum);
  }
  float a2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = q + 4 * k;
    const float ri = from_lane(rowlse, 4 * i);
    a2[k] = kFloorH;
    if (on && i < S) a2[k] = fmaxf(log_trans[(int64_t)i * S + j] * kLog2e - ri, kFloorH);
  }
  __syncthreads();  // the emission table is complete

  const int64_t b = (int64_t)blockIdx.x * 4 + w;
  if (b >= B) return;
  const int64_t base = b * T;
  int sym = symbol(obs, obs_i64, base + min((int64_t)lane, T - 1), O);  // frames [0, 64)
  int nxt = sym;
  const int erow = on ? j * O : 0;  // every lane reads inside the table
  float alpha = fmaxf(pi + le2[erow + __builtin_amdgcn_readlane(sym, 0)], kFloorH);
  if (!on) alpha = kFloorH;
  for (int64_t t = 1; t < T; ++t) {
    const int k64 = static_cast<int>(t & 63);
    if (k64 == 0) sym = nxt;
    if (k64 == 1) nxt = symbol(obs, obs_i64, base + min(t - 1 + 64 + lane, T - 1), O);
    const float e = le2[erow + __builtin_amdgcn_readlane(sym, k64)];
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = from_lane(alpha, 4 * (q + 4 * k)) + a2[k];
    // the state's maximum over its 16 terms first (quad_perm [1,0,3,2] then [2,3,0,1]), so the
    // partial sums share it and merge by plain addition
    float m = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    m = fmaxf(m, quad_swap<0xB1>(m));
    m = fmaxf(m, quad_swap<0x4E>(m));
    float sum = (exp2_fast(x[0] - m) + exp2_fast(x[1] - m)) + (exp2_fast(x[2] - m) + exp2_fast(x[3] - m));
    sum += quad_swap<0xB1>(sum);
    sum += quad_swap<0x4E>(sum);
    alpha = on ? fmaxf(m + log2_fast(sum) + e, kFloorH) : kFloorH;
  }
  const float ll = wave_lse2(lead ? alpha : kFloorH);
  if (lane == 0) out[b] = ll < -1e29f ? -INFINITY : ll * kLn2;
}

}  // namespace

hipError_t launch_hmm_forward(const float* log_init, const float* log_trans, const float* log_emit, const void* obs,
                              int obs_i64, int64_t B, int64_t T, int S, int O, float* out, hipStream_t s) {
  if (B == 0) return hipGetLastError();
  const size_t lds = sizeof(float) * (size_t)S * (size_t)O;
  const unsigned grid = static_cast<unsigned>((B + 3) / 4);
  auto launch = [&](auto kernel) {
    if (lds > 48 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    kernel<<<grid, 256, lds, s>>>(log_init, log_trans, log_emit, obs, obs_i64, B, T, S, O, out);
    return hipGetLastError();
  };
  if (S <= 16) return launch(&hmm_forward16_kernel);
  if (S <= 32) return launch(&hmm_forward_kernel<32>);
  return launch(&hmm_forward_kernel<64>);
}

}  // namespace pctc
