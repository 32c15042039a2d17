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
constexpr int kBlocksPerThread = 4;  // 32-element blocks handled per lane per step

// grid: x = workgroups per expert (a grid stride over the expert's blocks),
// y = expert.  Each workgroup first tabulates the odd-rounded products of
// all 256 E4M3 scale bytes with |gs| of its expert.
__global__ __launch_bounds__(kThreads) void requant_kernel(const uint8_t* src, const uint8_t* src_sf,
                                                           const float* __restrict__ gs,
                                                           uint8_t* dst, uint8_t* __restrict__ dst_sf,
                                                           int nb) {
  __shared__ float2 s_tab[256];
  __shared__ __attribute__((aligned(16))) uint8_t s_ob[4][64 * kBlocksPerThread];
  const int e = blockIdx.y;
  const float g = gs ? gs[e] : 1.0f;
  const float ag = fabsf(g);
  const uint32_t gneg = rq::bits(g) >> 31;
  {
    float p1, p3;
    rq::ro_pair(threadIdx.x, ag, p1, p3);
    s_tab[threadIdx.x] = float2{p1, p3};
  }
  __syncthreads();
  const size_t eb = (size_t)e * (size_t)nb;
  const uint8_t* sp = src + eb * 16;
  const uint8_t* ssf = src_sf + eb * 2;
  uint8_t* dp = dst + eb * 16;
  uint8_t* dsf = dst_sf + eb;
  // a wavefront handles 256 consecutive blocks per step; load i of lane l is
  // block base + 64 i + l, so every load instruction reads 1 KB contiguous
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int step = gridDim.x * kThreads * kBlocksPerThread;
  for (int base = (blockIdx.x * 4 + wave) * 64 * kBlocksPerThread; base < nb; base += step) {
    uint4 c[kBlocksPerThread];
    uint32_t sf[kBlocksPerThread];
#pragma unroll
    for (int i = 0; i < kBlocksPerThread; ++i) {
      const int b = base + 64 * i + lane;
      const bool ok = b < nb;
      c[i] = ok ? ld_nt(sp + (size_t)b * 16) : uint4{0u, 0u, 0u, 0u};
      sf[i] = ok ? *reinterpret_cast<const uint16_t*>(ssf + (size_t)b * 2) : 0u;
    }
#pragma unroll
    for (int i = 0; i < kBlocksPerThread; ++i) {
      const int b = base + 64 * i + lane;
      const float2 ta = s_tab[sf[i] & 0xFF], tb = s_tab[(sf[i] >> 8) & 0xFF];
      const uint32_t in[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
      uint32_t out[4];
      const uint32_t ob = rq::requant_block_tab(in, sf[i], ta.x, ta.y, tb.x, tb.y, gneg, out);
      if (b < nb) st_nt(dp + (size_t)b * 16, uint4{out[0], out[1], out[2], out[3]});
      s_ob[wave][64 * i + lane] = (uint8_t)ob;
    }
    // the wave's 256 scale bytes leave as one dword per lane (wave-private LDS)
    __builtin_amdgcn_wave_barrier();
    const uint32_t w4 = *reinterpret_cast<const uint32_t*>(&s_ob[wave][4 * lane]);
    if (base + 4 * lane + 3 < nb) {
      *reinterpret_cast<uint32_t*>(dsf + base + 4 * lane) = w4;
    } else {
      for (int j = 0; j < 4; ++j)
        if (base + 4 * lane + j < nb) dsf[base + 4 * lane + j] = (uint8_t)(w4 >> (8 * j));
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Group16 weights straight into the GEMM layout of the prefill kernels, with
// group32 UE8M0 scales (the weight preparation of the DeepGEMM commit that
// lets prepare_fp4_weights_for_mega_moe take raw grouped FP4 weights and
// requantise them on the way into the fused kernel's layout).  Thread = one
// row of a 512-row block over one 512-element scale group: 16 blocks of 32
// (256 code bytes + 32 E4M3 bytes in), requantised as requant_kernel does;
// each block's 16 code bytes are one 16-byte piece of the layout and the 16
// new scale bytes one 16-byte scale piece.  Layout (moe_fp4_prepare_gemm_-
// weights): code piece p of K stage s (128 elements) of block row i goes to
// slot j = 4 i + (p ^ ((i >> 2) & 3)) of image (nb * K/128 + s); the scale
// piece of (nb, g, i) is piece (nb * K/512 + g) * 512 + i.
__global__ __launch_bounds__(kThreads) void requant_prepare_kernel(const uint8_t* __restrict__ src,
                                                                   const uint8_t* __restrict__ src_sf,
                                                                   const float* __restrict__ gs,
                                                                   uint8_t* __restrict__ dst,
                                                                   uint8_t* __restrict__ dst_sf, int N, int K,
                                                                   int w13, int w13_order, int npieces) {
  __shared__ float2 s_tab[256];
  const int e = blockIdx.y;
  const float g = gs ? gs[e] : 1.0f;
  const uint32_t gneg = rq::bits(g) >> 31;
  {
    float p1, p3;
    rq::ro_pair(threadIdx.x, fabsf(g), p1, p3);
    s_tab[threadIdx.x] = float2{p1, p3};
  }
  __syncthreads();
  const int cs = blockIdx.x * kThreads + threadIdx.x;
  if (cs >= npieces) return;
  const int ng = K >> 9;
  const int i = cs & 511, bg = cs >> 9;  // block row, (row block, group)
  const int nb = bg / ng, grp = bg - nb * ng;
  int r = nb * 512 + i;  // source row
  if (w13) {
    const int i0 = nb * 256 + (i & 255);
    r = ((i >= 256) != (w13_order != 0)) ? N / 2 + i0 : i0;
  }
  const size_t ecode = (size_t)e * N * (size_t)(K >> 1);
  const uint8_t* sc = src + ecode + (size_t)r * (K >> 1) + 256 * grp;
  const uint8_t* ss = src_sf + (size_t)e * N * (size_t)(K >> 4) + (size_t)r * (K >> 4) + 32 * grp;
  const uint4 sa = *reinterpret_cast<const uint4*>(ss), sb = *reinterpret_cast<const uint4*>(ss + 16);
  const uint32_t sw[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
  const int sw_i = (i >> 2) & 3;
  uint32_t ob[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int blk = 0; blk < 16; ++blk) {
    const uint4 c = *reinterpret_cast<const uint4*>(sc + 16 * blk);
    const uint32_t sf16 = (sw[blk >> 1] >> (16 * (blk & 1))) & 0xFFFFu;
    const float2 ta = s_tab[sf16 & 0xFF], tb = s_tab[sf16 >> 8];
    const uint32_t in[4] = {c.x, c.y, c.z, c.w};
    uint32_t out[4];
    const uint32_t b = rq::requant_block_tab(in, sf16, ta.x, ta.y, tb.x, tb.y, gneg, out);
    ob[blk >> 2] |= b << (8 * (blk & 3));
    const int st = 4 * grp + (blk >> 2), piece = blk & 3;
    const int j = 4 * i + (piece ^ sw_i);
    *reinterpret_cast<uint4*>(dst + ecode + ((size_t)(nb * (K >> 7) + st) * 2048 + j) * 16) =
        uint4{out[0], out[1], out[2], out[3]};
  }
  *reinterpret_cast<uint4*>(dst_sf + (size_t)e * N * (size_t)(K >> 5) + (size_t)cs * 16) =
      uint4{ob[0], ob[1], ob[2], ob[3]};
}

}  // namespace

hipError_t launch_requant_prepare_gemm(const uint8_t* src, const uint8_t* src_sf, const float* gs, uint8_t* dst,
                                       uint8_t* dst_sf, int64_t E, int64_t N, int64_t K, bool w13, int w13_order,
                                       hipStream_t s) {
  const int64_t npieces = N * K / 512;  // scale pieces per expert
  if (E <= 0 || npieces <= 0) return hipSuccess;
  const int64_t gx = (npieces + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(requant_prepare_kernel, dim3((unsigned)gx, (unsigned)E), dim3(kThreads), 0, s, src, src_sf, gs,
                     dst, dst_sf, (int)N, (int)K, w13 ? 1 : 0, w13_order, (int)npieces);
  return hipGetLastError();
}

hipError_t launch_requant_g16_g32(const uint8_t* src, const uint8_t* src_sf, const float* gs,
                                  uint8_t* dst, uint8_t* dst_sf, int64_t E, int64_t N, int64_t K,
                                  hipStream_t s) {
  const int64_t nb = N * (K / 32);
  if (nb <= 0 || E <= 0) return hipSuccess;
  // One step per workgroup (1024 blocks: 16 KB of codes in and out; at most
  // 2^20 workgroups per expert, N * K / 32 <= 2^30 being checked by the
  // caller).  On the full layer this ran at 6.0 TB/s, against 5.2 TB/s with
  // ~32 grid-striding workgroups per CU and 5.8 TB/s with ~256.
  const int64_t per_wg = (int64_t)kThreads * kBlocksPerThread;
  const int64_t gx = (nb + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(requant_kernel, dim3((unsigned)gx, (unsigned)E), dim3(kThreads), 0, s, src,
                     src_sf, gs, dst, dst_sf, (int)nb);
  return hipGetLastError();
}

}  // namespace moefp4
