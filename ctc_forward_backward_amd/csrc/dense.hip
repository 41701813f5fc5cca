// Standalone row kernels of the packed CTC gradient: the posteriors (class sums) of every row, then
// the gradient rows, each as its own launch after the recursions.  The per-row work is in rows.h;
// the persistent worker in chains.hip runs the same row work overlapped with the recursions, and
// these kernels serve when that overlap is switched off.
//
// Method: NVIDIA-NeMo/Speech pull request "feat(asr): native CTC loss kernel over sequence-packed log
// probabilities", Triton file, `_beta_grad_kernel` and `_PackedCTCLoss.backward` (see rows.h).
//
// Design for gfx950: one wave per row, each wave on a contiguous range of rows (its utterance, and
// the class bitmap in LDS, rarely change); the latency-bound posterior kernel runs at high
// occupancy, the gradient kernel streams whole rows.
#include "rows.h"

namespace pctc {

namespace {

// rows [beg, end) of this wave
__device__ __forceinline__ void wave_rows(int rows_per_wave, int64_t TT, int64_t& beg, int64_t& end) {
  const int64_t wid = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  beg = wid * rows_per_wave;
  end = min(beg + rows_per_wave, TT);
}

__global__ void __launch_bounds__(256) posterior_kernel(Layout L, Pointers P, int per_wave, int rows_per_wave) {
  extern __shared__ float psm[];
  const int lane = threadIdx.x & 63;
  float* acc = psm + (threadIdx.x >> 6) * per_wave;
  int64_t rbeg, rend;
  wave_rows(rows_per_wave, L.T_total, rbeg, rend);
  for (int64_t r = rbeg; r < rend; ++r) {
    const int b = __builtin_amdgcn_readfirstlane(P.rowmap[r]);
    float w;
    if (rows::row_live(P, b, w)) rows::posterior_row(L, P, acc, r, b, w, lane);
  }
}

template <int DT>
__global__ void __launch_bounds__(256) dense_kernel(Inputs in, Layout L, Pointers P, void* grad, int per_wave,
                                                    int rows_per_wave) {
  extern __shared__ uint32_t dsm[];
  const int lane = threadIdx.x & 63;
  uint32_t* lds = dsm + (threadIdx.x >> 6) * per_wave;
  int cur_b = -1;
  int64_t rbeg, rend;
  wave_rows(rows_per_wave, L.T_total, rbeg, rend);
  for (int64_t r = rbeg; r < rend; ++r) {
    const int b = __builtin_amdgcn_readfirstlane(P.rowmap[r]);
    float w;
    if (rows::row_live(P, b, w)) rows::dense_row<DT>(in, L, P, grad, lds, r, b, w, lane, cur_b);
    else rows::fill_row<DT>(L, grad, r, w == 0.0f ? 0.0f : __builtin_nanf(""), lane);
  }
}

int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

// resident waves of a 256-thread kernel over the whole device (at least one per compute unit)
int64_t resident_waves(const void* kernel, size_t lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds) != hipSuccess || per_cu < 1) per_cu = 1;
  return 4 * (int64_t)per_cu * compute_units();
}

}  // namespace

hipError_t launch_posteriors(const Inputs& in, const Layout& L, const Pointers& P, hipStream_t s) {
  (void)in;
  if (L.T_total == 0 || L.B == 0) return hipGetLastError();
  // per wave: the class sums (U+1, rounded to 4); as many waves as fit, each on a contiguous range
  const int per_wave = static_cast<int>(L.C_stride);
  const size_t lds = 4 * sizeof(float) * (size_t)per_wave;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&posterior_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  const int64_t waves = resident_waves(reinterpret_cast<const void*>(&posterior_kernel), lds);
  const int64_t rpw = (L.T_total + waves - 1) / waves;
  const int grid = static_cast<int>(((L.T_total + rpw - 1) / rpw + 3) / 4);
  posterior_kernel<<<grid, 256, lds, s>>>(L, P, per_wave, static_cast<int>(rpw));
  return hipGetLastError();
}

hipError_t launch_dense(const Inputs& in, const Layout& L, const Pointers& P, void* grad_out, hipStream_t s) {
  if (L.T_total == 0 || L.D == 0) return hipSuccess;
  // per wave: the class sums (U+1, rounded to 4), the class bitmap and its prefix counts
  const int per_wave = static_cast<int>(L.C_stride + 2 * L.Dw);
  const size_t lds = 4 * sizeof(uint32_t) * (size_t)per_wave;
  // as many resident waves as fit, each on a contiguous range of rows
  auto launch = [&](auto kernel) {
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
    const int64_t waves = resident_waves(reinterpret_cast<const void*>(kernel), lds);
    const int64_t rpw = (L.T_total + waves - 1) / waves;
    const int grid = static_cast<int>(((L.T_total + rpw - 1) / rpw + 3) / 4);
    kernel<<<grid, 256, lds, s>>>(in, L, P, grad_out, per_wave, static_cast<int>(rpw));
    return hipGetLastError();
  };
  if (in.dtype == kF32) return launch(&dense_kernel<kF32>);
  if (in.dtype == kF16) return launch(&dense_kernel<kF16>);
  return launch(&dense_kernel<kBF16>);
}

}  // namespace pctc
