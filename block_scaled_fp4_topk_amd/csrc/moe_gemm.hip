// Prefill-shaped grouped GEMMs for FP8 activations (E4M3 + UE8M0 per 32)
// over FP4 weights (E2M1 + UE8M0 per 32): FC1 + SwiGLU + FP8 requantisation
// of h, and FC2.  This is the FP8xFP4 recipe (1, 1, 32) of the GLM-5.2 NVFP4
// group16 MegaMoE notes (Context) in the regime where an expert receives
// many tokens and the MFMA, not HBM, sets the pace.
//
// Tile: 128 activation rows (one expert's 128-row tile) x 256 weight rows
// (FC1: 128 gate rows and the matching 128 up rows, so SwiGLU and the
// per-32 quantisation of h stay inside the workgroup; FC2: 256 output
// rows).  One workgroup of 4 wavefronts per CU; wave (wm, wn) owns 64
// activation rows x 128 weight rows = 4 x 8 tiles of the block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 (A = FP4 weights, B = FP8 activations),
// FP32 accumulators in registers.
//
// Pipeline: K advances in stages of 256 (two 128-wide MFMA steps).  Both
// operands of a stage go HBM/L2 -> LDS with direct-to-LDS 16-byte loads
// (global_load_lds_dwordx4), double-buffered in two LDS stage buffers: the
// loads of stage s + 1 are in flight while stage s is multiplied out of
// LDS.  The block scales (8 bytes per row per stage) go through registers.
//
// LDS layouts (16-byte slots, XOR-swizzled so the MFMA operand reads hit
// every bank once per 16 lanes):
//   activations, per MFMA step: token t, 16-byte piece p (K 16p..16p+15)
//     at slot 8 t + (p ^ ((t >> 1) & 7));
//   weights, per MFMA step: row r, piece p (K 32p..32p+31) at slot
//     4 r + (p ^ ((r >> 2) & 3)).
// Every load instruction of a wave fills 64 consecutive slots: 8 tokens x
// 128 bytes (full lines) or 16 weight rows x 64 contiguous bytes.
//
// Workgroup -> tile mapping: workgroups are dealt to the 8 XCDs round-robin,
// so XCD x gets a contiguous range of (expert tile, row block) work items:
// an expert's tiles and row blocks stay on one XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace moefp4 {

namespace {

constexpr int GM = 128;  // activation rows per tile
constexpr int GN = 256;  // weight rows per tile
constexpr int GK = 256;  // K per pipeline stage

struct alignas(16) StageBuf {
  uint8_t act[2][1024 * 16];  // per MFMA step: 128 tokens x 8 pieces
  uint8_t w[2][1024 * 16];    // per MFMA step: 256 rows x 4 pieces
  uint2 asf[GM];              // the stage's 8 UE8M0 activation scale bytes per token
  uint2 wsf[GN];              // the stage's 8 UE8M0 weight scale bytes per row
};

__device__ __forceinline__ int byte_of(const uint2& v, int idx) {
  const uint32_t w = idx < 4 ? v.x : v.y;
  return (int)((w >> (8 * (idx & 3))) & 0xFFu);
}

template <bool FC1>
__global__ __launch_bounds__(256, 1) void fc_gemm_a8_kernel(FcArgs a, int nblk) {
  __shared__ StageBuf sb0;
  __shared__ StageBuf sb1;
  __shared__ int s_src[GM];

  // work item of this workgroup (XCD-contiguous ranges of the real items)
  const int items = a.ntiles[0] * nblk;
  const int per_xcd = (items + 7) >> 3;
  const int idx = blockIdx.x >> 3;
  if (idx >= per_xcd) return;
  const int v = (blockIdx.x & 7) * per_xcd + idx;
  if (v >= items) return;
  const int tile = v / nblk, nb = v - tile * nblk;
  const int e = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const int ne = a.counts[e], oe = a.offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, N = a.N;

  if (tid < GM) {
    const int m = m0 + tid;
    int src = -1;
    if (m < ne) src = FC1 ? a.sorted_assign[oe + m] / a.top_k : oe + m;
    s_src[tid] = src;
  }
  __syncthreads();

  // global row of WG-local weight row r
  auto wrow = [&](int r) {
    if (FC1) {
      const int i0 = nb * 128 + (r & 127);
      return ((r >= 128) != (a.w13_order != 0)) ? a.I + i0 : i0;
    }
    return nb * 256 + r;
  };

  // ---- load roles -------------------------------------------------------
  // Instruction i (0..7) of wave w fills stage slots S = 512 w + 64 i + lane:
  // MFMA step st = S >> 10, slot s = S & 1023.
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const uint8_t* wbase = a.w + (size_t)e * N * (size_t)(K >> 1);
  int aoff[8], woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int S = 512 * wave + 64 * i + lane;
    const int st = S >> 10, s = S & 1023;
    {  // activations: token t, piece p
      const int t = s >> 3, p = (s & 7) ^ ((t >> 1) & 7);
      const int src = s_src[t];
      aoff[i] = src >= 0 ? src * K + 128 * st + 16 * p : -1;
    }
    {  // weights: row r, piece p
      const int r = s >> 2, p = (s & 3) ^ ((r >> 2) & 3);
      woff[i] = wrow(r) * (K >> 1) + 64 * st + 16 * p;
    }
  }
  // scale roles: weight row tid; activation token tid (tid < 128)
  const uint8_t* wsf_p = a.wsf + ((size_t)e * N + wrow(tid)) * (size_t)(K >> 5);
  const int asrc = tid < GM ? s_src[tid] : -1;
  const uint8_t* asf_p = asrc >= 0 ? a.act_sf + (size_t)asrc * (K >> 5) : nullptr;

  auto issue = [&](StageBuf& b, int k0, uint2& ws, uint2& as) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int S0 = 512 * wave + 64 * i;  // wave-uniform first slot
      uint8_t* abase = &b.act[S0 >> 10][(S0 & 1023) * 16];
      uint8_t* wdst = &b.w[S0 >> 10][(S0 & 1023) * 16];
      if (aoff[i] >= 0)
        __builtin_amdgcn_global_load_lds(act + aoff[i] + k0, abase, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(wbase + woff[i] + (k0 >> 1), wdst, 16, 0, 0);
    }
    ws = *reinterpret_cast<const uint2*>(wsf_p + (k0 >> 5));
    as = uint2{0u, 0u};
    if (asf_p) as = *reinterpret_cast<const uint2*>(asf_p + (k0 >> 5));
  };
  auto put_scales = [&](StageBuf& b, const uint2& ws, const uint2& as) {
    b.wsf[tid] = ws;
    if (tid < GM) b.asf[tid] = as;
  };

  // ---- MFMA over one stage ------------------------------------------------
  v4f acc[8][4];
#pragma unroll
  for (int rg = 0; rg < 8; ++rg)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = v4f{0.f, 0.f, 0.f, 0.f};
  // token groups of this wave that hold at least one token
  int ntg = (ne - m0 - 64 * wm + 15) >> 4;
  ntg = ntg < 0 ? 0 : (ntg > 4 ? 4 : ntg);

  auto compute = [&](const StageBuf& b) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      v8i A[8];
      int sa[8];
#pragma unroll
      for (int rg = 0; rg < 8; ++rg) {
        const int r = FC1 ? (rg < 4 ? 64 * wn + 16 * rg : 128 + 64 * wn + 16 * (rg - 4)) + r16
                          : 128 * wn + 16 * rg + r16;
        const uint4 c = *reinterpret_cast<const uint4*>(
            &b.w[st][(4 * r + (q ^ ((r >> 2) & 3))) * 16]);
        A[rg] = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        sa[rg] = byte_of(b.wsf[r], 4 * st + q);
      }
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        if (tg < ntg) {
          const int t = 64 * wm + 16 * tg + r16;
          const int x = (t >> 1) & 7;
          const uint4 b0 = *reinterpret_cast<const uint4*>(&b.act[st][(8 * t + (q ^ x)) * 16]);
          const uint4 b1 = *reinterpret_cast<const uint4*>(&b.act[st][(8 * t + ((q + 4) ^ x)) * 16]);
          const v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                         (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          const int sb = byte_of(b.asf[t], 4 * st + q);
#pragma unroll
          for (int rg = 0; rg < 8; ++rg)
            acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[rg], B, acc[rg][tg], 4, 0,
                                                                          0, sa[rg], 0, sb);
        }
      }
    }
  };

  // ---- pipeline ---------------------------------------------------------
  // vmcnt(0) (expcnt and lgkmcnt left at their maxima): the direct-to-LDS
  // loads of the next stage have landed
  constexpr int kWaitVm0 = 0x0F70;
  const int ns = K / GK;
  uint2 ws, as;
  issue(sb0, 0, ws, as);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  put_scales(sb0, ws, as);
  __syncthreads();
  for (int c = 0; c < ns; c += 2) {
    if (c + 1 < ns) issue(sb1, (c + 1) * GK, ws, as);
    compute(sb0);
    if (c + 1 < ns) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      put_scales(sb1, ws, as);
    }
    __syncthreads();
    if (c + 1 >= ns) break;
    if (c + 2 < ns) issue(sb0, (c + 2) * GK, ws, as);
    compute(sb1);
    if (c + 2 < ns) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      put_scales(sb0, ws, as);
    }
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------
  // lane holds, for row group rg and token group tg, weight rows 4q..4q+3 of
  // the 16-row group and token r16 of the 16-token group
  const float gsc = a.gs ? a.gs[e] : 1.0f;
#pragma unroll
  for (int tg = 0; tg < 4; ++tg) {
    const int t = 64 * wm + 16 * tg + r16;
    const int m = m0 + t;
    const bool valid = m < ne;
    const int slot = oe + m;
    if (FC1) {
      // 32-wide h blocks j = 0, 1 of this wave: gate groups 2j, 2j+1 with up
      // groups 4+2j, 5+2j; outputs nb*128 + 64 wn + 32 j + [0, 32)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float h[2][4];
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h[u][i] = swiglu(acc[2 * j + u][tg][i] * gsc, acc[4 + 2 * j + u][tg][i] * gsc);
            amax = fmaxf(amax, fabsf(h[u][i]));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        int ex = amax > 0.0f ? ceil_log2_over_448(amax) : -127;
        ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
        const float inv = __builtin_ldexpf(1.0f, -ex);
        if (valid) {
          const int ob = nb * 128 + 64 * wn + 32 * j;
          uint8_t* hrow = static_cast<uint8_t*>(a.h_out) + (size_t)slot * a.I;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            uint32_t wv = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) wv |= f32_to_e4m3_rne(h[u][i] * inv) << (8 * i);
            *reinterpret_cast<uint32_t*>(hrow + ob + 16 * u + 4 * q) = wv;
          }
          if (q == 0) a.h_sf_out[(size_t)slot * (a.I >> 5) + (ob >> 5)] = (uint8_t)(ex + 127);
        }
      }
    } else if (valid) {
      float* y = a.y_out + (size_t)slot * a.H + nb * 256 + 128 * wn + 4 * q;
#pragma unroll
      for (int rg = 0; rg < 8; ++rg)
        *reinterpret_cast<float4*>(y + 16 * rg) =
            float4{acc[rg][tg][0] * gsc, acc[rg][tg][1] * gsc, acc[rg][tg][2] * gsc,
                   acc[rg][tg][3] * gsc};
    }
  }
}

template <bool FC1>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int nblk = FC1 ? a.I / 128 : a.H / 256;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  // enough workgroups for every work item; the ones past the real count
  // (known on the device only) return at once
  const long long items = (long long)max_tiles * nblk;
  const long long grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((fc_gemm_a8_kernel<FC1>), dim3((unsigned)grid), dim3(256), 0, s, a, nblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc_gemm_a8(const FcArgs& a, bool fc1, int max_tiles, hipStream_t s) {
  return fc1 ? launch_one<true>(a, max_tiles, s) : launch_one<false>(a, max_tiles, s);
}

}  // namespace moefp4
