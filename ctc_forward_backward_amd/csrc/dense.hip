// Row kernels of the packed CTC gradient: the posteriors (class sums) of a group's rows, then its
// gradient rows, on the group's stream after its recursions; and the zero rows owned by no
// utterance.  The per-row work is in rows.h.
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities", Triton file, `_beta_grad_kernel` and `_PackedCTCLoss.backward` (see rows.h).
//
// Design for gfx950: one wave per row, each wave on a contiguous share of the group's rows (its
// utterance, and the class bitmap in LDS, rarely change); the latency-bound posterior kernel runs at
// high occupancy, the gradient kernel streams whole rows.
#include <algorithm>

#include "rows.h"

namespace pctc {

namespace {

__device__ __forceinline__ int64_t wave_id() {
  return (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__global__ void __launch_bounds__(256) posterior_kernel(Layout L, Pointers P, int per_wave, int group) {
  // a streamed forward has already formed every row's class sums
  if (__builtin_amdgcn_readfirstlane(P.ctl->post_ready) != 0 || skipped(P)) return;
  extern __shared__ float psm[];
  const int lane = threadIdx.x & 63;
  float* acc = psm + (threadIdx.x >> 6) * per_wave;
  int64_t j0, j1;
  wave_share(P, group, wave_id(), (int64_t)gridDim.x * 4, j0, j1);
  group_rows(P, group, j0, j1, [&](int64_t r, int b) {
    float w;
    if (rows::row_live(P, b, w)) rows::posterior_row(L, P, acc, r, b, lane);
  });
}

template <int DT>
__global__ void __launch_bounds__(256) dense_kernel(Inputs in, Layout L, Pointers P, void* grad, int per_wave,
                                                    int group) {
  if (skipped(P)) return;
  extern __shared__ uint32_t dsm[];
  const int lane = threadIdx.x & 63;
  uint32_t* lds = dsm + (threadIdx.x >> 6) * per_wave;
  int cur_b = -1;
  int64_t j0, j1;
  wave_share(P, group, wave_id(), (int64_t)gridDim.x * 4, j0, j1);
  // a wave of the recursions gave up waiting: the rows are NaN (the losses too, weights kernel)
  const bool broken = __builtin_amdgcn_readfirstlane(P.ctl->err) != 0;
  group_rows(P, group, j0, j1, [&](int64_t r, int b) {
    float w;
    if (!broken && rows::row_live(P, b, w)) rows::dense_row<DT>(in, L, P, grad, lds, r, b, w, lane, cur_b);
    else rows::fill_row<DT>(L, grad, r, !broken && w == 0.0f ? 0.0f : __builtin_nanf(""), lane);
  });
}

// rows owned by no utterance (gaps between utterances, over-allocation) get a zero gradient
template <int DT>
__global__ void __launch_bounds__(256) gap_kernel(Layout L, Pointers P, void* grad, int rows_per_wave) {
  if (skipped(P)) return;
  const int lane = threadIdx.x & 63;
  const int64_t r0 = wave_id() * rows_per_wave, r1 = min(r0 + rows_per_wave, L.T_total);
  for (int64_t r = r0; r < r1; ++r)
    if (__builtin_amdgcn_readfirstlane(row_owner(L, P, r)) < 0) rows::fill_row<DT>(L, grad, r, 0.0f, lane);
}

int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// workgroups of a 256-thread kernel that are resident over the whole device (at least one per
// compute unit)
int resident_groups(const void* kernel, size_t lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess || per_cu < 1) per_cu = 1;
  return per_cu * compute_units();
}

}  // namespace

hipError_t launch_posteriors(const Inputs& in, const Layout& L, const Pointers& P, int group, hipStream_t s) {
  (void)in;
  if (L.T_total == 0 || L.B == 0) return hipGetLastError();
  // per wave: the class sums (U+1, rounded to 4); as many waves as fit, each on a contiguous share
  const int per_wave = static_cast<int>(L.C_stride);
  const size_t lds = std::max(4 * sizeof(float) * (size_t)per_wave, kRowKernelLds);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&posterior_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  const int grid = resident_groups(reinterpret_cast<const void*>(&posterior_kernel), lds);
  posterior_kernel<<<grid, 256, lds, s>>>(L, P, per_wave, group);
  return hipGetLastError();
}

hipError_t launch_dense(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, int group,
                        hipStream_t s) {
  if (L.T_total == 0 || L.D == 0 || L.B == 0) return hipGetLastError();
  // per wave: the class sums (U+1, rounded to 4), the class bitmap and its prefix counts
  const int per_wave = static_cast<int>(L.C_stride + 2 * L.Dw);
  const size_t lds = std::max(4 * sizeof(uint32_t) * (size_t)per_wave, kRowKernelLds);
  auto launch = [&](auto kernel) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
    const int grid = resident_groups(reinterpret_cast<const void*>(kernel), lds);
    kernel<<<grid, 256, lds, s>>>(in, L, P, grad_out, per_wave, group);
    return hipGetLastError();
  };
  if (in.dtype == kF32) return launch(&dense_kernel<kF32>);
  if (in.dtype == kF64) return launch(&dense_kernel<kF64>);
  if (in.dtype == kF16) return launch(&dense_kernel<kF16>);
  return launch(&dense_kernel<kBF16>);
}

hipError_t launch_gaps(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s) {
  if (L.T_total == 0 || L.D == 0) return hipGetLastError();
  const int64_t waves = 32 * (int64_t)compute_units();
  const int64_t rpw = (L.T_total + waves - 1) / waves;
  const int grid = static_cast<int>(((L.T_total + rpw - 1) / rpw + 3) / 4);
  const int rows = static_cast<int>(rpw);
  if (in.dtype == kF32) gap_kernel<kF32><<<grid, 256, 0, s>>>(L, P, grad_out, rows);
  else if (in.dtype == kF64) gap_kernel<kF64><<<grid, 256, 0, s>>>(L, P, grad_out, rows);
  else if (in.dtype == kF16) gap_kernel<kF16><<<grid, 256, 0, s>>>(L, P, grad_out, rows);
  else gap_kernel<kBF16><<<grid, 256, 0, s>>>(L, P, grad_out, rows);
  return hipGetLastError();
}

}  // namespace pctc
