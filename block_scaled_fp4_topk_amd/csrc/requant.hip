// Group16 (E4M3 + FP32 global scale) -> group32 (UE8M0) FP4 requantisation
// kernel: GLM-5.2 NVFP4 group16 MegaMoE notes, Requantization path; the
// DeepGEMM commit that makes requant_fp4_to_gran_k always recompute UE8M0
// scales from the restored values.  Purely bandwidth-bound: each thread
// streams whole 32-element blocks (16 code bytes + 2 scale bytes in, 16 + 1
// out); the arithmetic is in requant_core.h.
#pragma clang fp contract(off)
#include "common.h"
#include "kernels.h"
#include "requant_core.h"

namespace moefp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerThread = 4;  // 32-element blocks handled per thread per step

__global__ __launch_bounds__(kThreads) void requant_kernel(const uint8_t* src, const uint8_t* src_sf,
                                                           const float* __restrict__ gs,
                                                           uint8_t* dst, uint8_t* __restrict__ dst_sf,
                                                           int64_t nblk, int64_t blk_per_expert) {
  const int64_t step = (int64_t)gridDim.x * kThreads * kBlocksPerThread;
  for (int64_t b0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kBlocksPerThread; b0 < nblk;
       b0 += step) {
    uint4 c[kBlocksPerThread];
    uint32_t sf[kBlocksPerThread];
    float g[kBlocksPerThread];
    const int nb = nblk - b0 < kBlocksPerThread ? (int)(nblk - b0) : kBlocksPerThread;
    if (nb == kBlocksPerThread) {
#pragma unroll
      for (int i = 0; i < kBlocksPerThread; ++i) c[i] = ld_nt(src + (b0 + i) * 16);
      const uint2 s = *reinterpret_cast<const uint2*>(src_sf + b0 * 2);
      sf[0] = s.x & 0xFFFF; sf[1] = s.x >> 16; sf[2] = s.y & 0xFFFF; sf[3] = s.y >> 16;
    } else {
      for (int i = 0; i < kBlocksPerThread; ++i) {
        if (i < nb) {
          c[i] = *reinterpret_cast<const uint4*>(src + (b0 + i) * 16);
          sf[i] = *reinterpret_cast<const uint16_t*>(src_sf + (b0 + i) * 2);
        } else {
          c[i] = uint4{0, 0, 0, 0};
          sf[i] = 0;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBlocksPerThread; ++i) {
      const int64_t blk = b0 + i < nblk ? b0 + i : nblk - 1;
      g[i] = gs ? gs[blk / blk_per_expert] : 1.0f;
    }
    uint4 o[kBlocksPerThread];
    uint32_t ob[kBlocksPerThread];
#pragma unroll
    for (int i = 0; i < kBlocksPerThread; ++i) {
      const uint32_t in[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      uint32_t out[4];
      ob[i] = rq::requant_block(in, sf[i], g[i], out);
      o[i] = uint4{out[0], out[1], out[2], out[3]};
    }
    if (nb == kBlocksPerThread) {
#pragma unroll
      for (int i = 0; i < kBlocksPerThread; ++i) st_nt(dst + (b0 + i) * 16, o[i]);
      *reinterpret_cast<uint32_t*>(dst_sf + b0) = ob[0] | (ob[1] << 8) | (ob[2] << 16) | (ob[3] << 24);
    } else {
      for (int i = 0; i < nb; ++i) {
        *reinterpret_cast<uint4*>(dst + (b0 + i) * 16) = o[i];
        dst_sf[b0 + i] = (uint8_t)ob[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_requant_g16_g32(const uint8_t* src, const uint8_t* src_sf, const float* gs,
                                  uint8_t* dst, uint8_t* dst_sf, int64_t E, int64_t N, int64_t K,
                                  hipStream_t s) {
  const int64_t nblk = E * N * (K / 32);
  if (nblk <= 0) return hipSuccess;
  const int64_t per_wg = (int64_t)kThreads * kBlocksPerThread;
  int64_t grid = (nblk + per_wg - 1) / per_wg;
  if (grid > 256 * 32) grid = 256 * 32;
  hipLaunchKernelGGL(requant_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, src, src_sf, gs,
                     dst, dst_sf, nblk, N * (K / 32));
  return hipGetLastError();
}

}  // namespace moefp4
