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
// Pipeline: K advances in stages of 256 (two 128-wide MFMA steps).  Every
// operand byte goes HBM/L2 -> LDS with direct-to-LDS loads
// (global_load_lds), each instruction reading whole 128-byte lines: 8
// activation rows x 128 bytes, or 8 weight rows x 128 bytes (a weight row's
// 256 FP4 codes of the stage).  Two stage buffers: stage s + 1 is in flight
// while stage s is multiplied.  The UE8M0 scales go to LDS once per group
// of 4 stages (32 bytes per row), two lanes per row with 16-byte loads, also
// double-buffered.
//
// LDS layouts (16-byte slots, XOR-swizzled so that the 16 lanes of an MFMA
// operand read hit distinct banks):
//   activations, per MFMA step: token t, piece p (K 16p..16p+15) at slot
//     8 t + (p ^ ((t >> 1) & 7));
//   weights, per stage: row r, piece p (K 32p..32p+31, p < 4 first MFMA
//     step) at slot 8 r + (p ^ ((r >> 1) & 7));
//   scales, per group: row r, 16-byte half h at slot 2 r + h.
//
// Workgroup -> tile mapping: workgroups are dealt to the 8 XCDs round-robin,
// so XCD x gets a contiguous range of (expert tile, row block) work items:
// an expert's tiles and row blocks stay on one XCD and share its L2.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace moefp4 {

namespace {

constexpr int GM = 128;  // activation rows per tile
constexpr int GN = 256;  // weight rows per tile
constexpr int GK = 256;  // K per pipeline stage (two MFMA steps)
constexpr int GS = 4;    // stages per scale group (1024 K = 32 scale bytes per row)

struct alignas(16) Stage {
  uint8_t act[2][1024 * 16];  // per MFMA step: 128 tokens x 8 pieces
  uint8_t w[2048 * 16];       // 256 rows x 8 pieces
};
struct alignas(16) Scales {
  uint8_t w[GN * 32];  // per row: the group's 32 UE8M0 bytes
  uint8_t a[GM * 32];  // per token
};

template <bool FC1>
__global__ __launch_bounds__(256, 1) void fc_gemm_a8_kernel(FcArgs a, int nblk) {
  __shared__ Stage st0, st1;
  __shared__ Scales sc0, sc1;
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
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int r16 = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, N = a.N;

  // source row of each tile row; rows past the expert's token count load
  // the tile's first row instead (their MFMA columns are never stored)
  if (tid < GM) {
    const int m = m0 + (m0 + tid < ne ? tid : 0);
    s_src[tid] = FC1 ? a.sorted_assign[oe + m] / a.top_k : oe + m;
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
  // Operand instruction i (0..7) of wave w fills slots S = 512 w + 64 i +
  // lane of the stage's activation array (MFMA step S >> 10) and of its
  // weight array.  Scale instructions: weight slots 64 J + lane (rows
  // 32 J + lane / 2, J = 2 w, 2 w + 1), activation slots 64 w + lane
  // (tokens 32 w + lane / 2).
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const uint8_t* wbase = a.w + (size_t)e * N * (size_t)(K >> 1);
  const uint8_t* wsbase = a.wsf + (size_t)e * N * (size_t)(K >> 5);
  uint32_t aoff[8], woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int S = 512 * wave + 64 * i + lane;
    const int st = S >> 10, s = S & 1023;
    const int t = s >> 3, p = (s & 7) ^ ((t >> 1) & 7);
    aoff[i] = s_src[t] * K + 128 * st + 16 * p;
    const int r = S >> 3, pw = (S & 7) ^ ((r >> 1) & 7);
    woff[i] = wrow(r) * (K >> 1) + 16 * pw;
  }
  uint32_t wsoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wsoff[j] = wrow(32 * (2 * wave + j) + (lane >> 1)) * (K >> 5) + 16 * (lane & 1);
  const uint32_t asoff = s_src[32 * wave + (lane >> 1)] * (K >> 5) + 16 * (lane & 1);
  const int nkb = K >> 5;  // scale bytes per row

  auto issue = [&](Stage& b, uint32_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int S0 = 512 * wave + 64 * i;  // wave-uniform first slot
      __builtin_amdgcn_global_load_lds(act + (aoff[i] + k0), &b.act[S0 >> 10][(S0 & 1023) * 16], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(wbase + (woff[i] + (k0 >> 1)), &b.w[S0 * 16], 16, 0, 0);
    }
  };
  // scale group starting at K block kb0 (32 blocks); 16-byte pieces past the
  // row's last scale byte are not loaded (K % 512 == 0 keeps pieces whole)
  auto issue_scales = [&](Scales& g, int kb0) __attribute__((always_inline)) {
    const bool ok = kb0 + 16 * (lane & 1) < nkb;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (ok) __builtin_amdgcn_global_load_lds(wsbase + (wsoff[j] + kb0), &g.w[(64 * (2 * wave + j)) * 16], 16, 0, 0);
    if (ok) __builtin_amdgcn_global_load_lds(a.act_sf + (asoff + kb0), &g.a[(64 * wave) * 16], 16, 0, 0);
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

  // stage b with scale group g, stage index gs within the group; FULL: all 4
  // token groups (straight-line code), else the first ntg
  auto compute_t = [&](const Stage& b, const Scales& g, int gs, auto full) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full)::value;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const int kb = 8 * gs + 4 * ms + q;  // this lane's K block within the group
      v8i B[4];
      int sb[4];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) {
        if (FULL || tg < ntg) {
          const int t = 64 * wm + 16 * tg + r16;
          const int x = (t >> 1) & 7;
          const uint4 b0 = *reinterpret_cast<const uint4*>(&b.act[ms][(8 * t + (q ^ x)) * 16]);
          const uint4 b1 = *reinterpret_cast<const uint4*>(&b.act[ms][(8 * t + ((q + 4) ^ x)) * 16]);
          B[tg] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                      (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          sb[tg] = g.a[t * 32 + kb];
        }
      }
#pragma unroll
      for (int rg = 0; rg < 8; ++rg) {
        const int r = FC1 ? (rg < 4 ? 64 * wn + 16 * rg : 128 + 64 * wn + 16 * (rg - 4)) + r16
                          : 128 * wn + 16 * rg + r16;
        const uint4 c = *reinterpret_cast<const uint4*>(
            &b.w[(8 * r + ((4 * ms + q) ^ ((r >> 1) & 7))) * 16]);
        const v8i A = {(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
        const int sa = g.w[r * 32 + kb];
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
          if (FULL || tg < ntg)
            acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B[tg], acc[rg][tg], 4, 0,
                                                                          0, sa, 0, sb[tg]);
      }
    }
  };
  auto compute = [&](const Stage& b, const Scales& g, int gs) __attribute__((always_inline)) {
    if (ntg == 4) compute_t(b, g, gs, std::true_type{});
    else compute_t(b, g, gs, std::false_type{});
  };

  // ---- pipeline -----------------------------------------------------------
  // Step c: wait until this wave's loads (stage c, and the scale group of
  // stage c when it starts one) have landed, barrier (every wave's loads
  // visible, every wave done with stage c - 1), start loading stage c + 1
  // into the other stage buffer (and, at a group start, the next scale
  // group into the other scale buffer), multiply stage c.  Buffers are
  // compile-time choices (unrolled by 2 groups = 8 stages) so the compiler
  // sees that loads in flight never alias the buffers being read.
  auto barrier = [&]() __attribute__((always_inline)) {
    // plain s_barrier (__syncthreads() would also wait for the loads just
    // issued); the asm statements keep LDS accesses on their side
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int ns = K / GK;
  auto step = [&](Stage& cur, Stage& nxt, Scales& g, Scales& gnext, int c) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    barrier();
    if (c + 1 < ns) issue(nxt, (c + 1) * GK);
    if ((c & (GS - 1)) == 0 && c + GS < ns) issue_scales(gnext, (c + GS) * (GK / 32));
    compute(cur, g, c & (GS - 1));
  };
  issue_scales(sc0, 0);
  issue(st0, 0);
  for (int c = 0; c < ns; c += 2 * GS) {
    step(st0, st1, sc0, sc1, c);
    if (c + 1 >= ns) break;
    step(st1, st0, sc0, sc1, c + 1);
    if (c + 2 >= ns) break;
    step(st0, st1, sc0, sc1, c + 2);
    if (c + 3 >= ns) break;
    step(st1, st0, sc0, sc1, c + 3);
    if (c + 4 >= ns) break;
    step(st0, st1, sc1, sc0, c + 4);
    if (c + 5 >= ns) break;
    step(st1, st0, sc1, sc0, c + 5);
    if (c + 6 >= ns) break;
    step(st0, st1, sc1, sc0, c + 6);
    if (c + 7 >= ns) break;
    step(st1, st0, sc1, sc0, c + 7);
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
