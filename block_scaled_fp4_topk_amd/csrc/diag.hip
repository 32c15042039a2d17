// Measurement helpers used by the benchmark to put the kernels' rooflines
// beside what this GPU actually delivers: a register-only loop of the
// block-scaled matrix instruction the prefill GEMM issues
// (v_mfma_scale_f32_16x16x128_f8f6f4, FP4 weights x FP8 or FP4 activations).
#include "common.h"
#include "kernels.h"

namespace moefp4 {

namespace {

// 8 independent accumulator chains per wave (enough to keep the matrix pipe
// busy); operands derived from the lane so the compiler cannot fold them.
template <bool A4>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink) {
  const int l = threadIdx.x;
  const v8i a = {l, l * 3, l * 5, l * 7, 0, 0, 0, 0};
  const v8i b = A4 ? v8i{l * 11, l * 13, l * 17, l * 19, 0, 0, 0, 0}
                   : v8i{l * 11, l * 13, l * 17, l * 19, l * 23, l * 29, l * 31, l * 37};
  v4f acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 4, A4 ? 4 : 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == 1234.5f) sink[blockIdx.x * 256 + l] = s;  // never true for these operands; keeps the loop live
}

}  // namespace

hipError_t launch_mfma_peak(bool a4, int iters, int blocks, float* sink, hipStream_t s) {
  if (a4)
    hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3(blocks), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(blocks), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace moefp4
