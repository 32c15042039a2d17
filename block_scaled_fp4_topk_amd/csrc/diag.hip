// Measurement helpers used by the benchmark to put the kernels' rooflines
// beside what this GPU actually delivers: a register-only loop of the
// block-scaled matrix instruction the prefill GEMM issues
// (v_mfma_scale_f32_16x16x128_f8f6f4, FP4 weights x FP8 or FP4 activations).
#include "common.h"
#include "kernels.h"

namespace moefp4 {

namespace {

// 64 independent accumulator chains per wave (8 weight x 8 activation
// operands: the shape of one stage of the prefill GEMM, 256 accumulators per
// lane), one workgroup of 4 waves per CU; operands derived from the lane so
// the compiler cannot fold them.  (For FP4 x FP4 the compiler adds about one
// accumulator move per MFMA to this loop, so that rate is a lower bound.)
template <bool A4>
__global__ __launch_bounds__(256, 1) void mfma_peak_kernel(int iters, float* sink) {
  const int l = threadIdx.x;
  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i w[8], x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = v8i{l + i, l * 3 + i, l ^ i, l + 7 * i, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = v8i{l, i, l * 5, 3, l + i, 9, l, i + 1};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int tg = 0; tg < 8; ++tg)
#pragma unroll
      for (int rg = 0; rg < 8; ++rg)
        acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[rg], x[tg], acc[rg][tg], 4, A4 ? 4 : 0, 0,
                                                                      120 + rg, 0, 120 - tg);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
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
