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
// Pipeline: K advances in stages of 128 (one MFMA step).  Both operands of
// a stage go HBM/L2 -> LDS with direct-to-LDS 16-byte loads
// (global_load_lds_dwordx4): 8 activation rows x 128 bytes or 16 weight rows
// x 64 bytes per instruction.  A ring of 4 stage buffers keeps the loads of
// three stages in flight while one is multiplied; the UE8M0 block scales of
// a group of 4 stages (16 bytes per row or token) go straight to registers,
// one group ahead.  A wave whose 64 activation rows hold no token skips its
// MFMAs.
//
// LDS layouts (16-byte slots, XOR-swizzled so that the 16 lanes of an MFMA
// operand read hit distinct banks):
//   activations: token t, piece p (K 16p..16p+15) at slot
//     8 t + (p ^ ((t >> 1) & 7));
//   weights: row r, piece p (K 32p..32p+31) at slot 4 r + (p ^ ((r >> 2) & 3)).
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
constexpr int GK = 128;  // K per pipeline stage (one MFMA step)
constexpr int GS = 4;    // stages per scale group (512 K = 16 scale bytes per row)

struct alignas(16) Stage {
  uint8_t act[1024 * 16];  // 128 tokens x 8 pieces
  uint8_t w[1024 * 16];    // 256 rows x 4 pieces
};
// s_waitcnt with vmcnt(n), expcnt and lgkmcnt at their maxima (gfx9 encoding)
#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
// operand load instructions per wave per stage: 4 weight + 4 activation
// (FP8: 128 tokens x 128 bytes), or + 2 (A4: 128 tokens x 64 bytes)
template <bool A4> constexpr int kOpsOf = A4 ? 6 : 8;
constexpr int kScaleOps = 12;  // scale load instructions per wave per group (8 weight, 4 activation)

// A4: MXFP4 activations (E2M1 + UE8M0 per 32, K/2 bytes per row) and h
// quantised to MXFP4 by FC1; both MFMA operands FP4.
template <bool FC1, bool A4>
__global__ __launch_bounds__(256, 1) void fc_gemm_a8_kernel(FcArgs a, int nblk) {
  constexpr int kOps = kOpsOf<A4>;
  __shared__ Stage st0, st1, st2, st3;
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
  // Operand instruction i (0..3) of wave w fills slots S = 256 w + 64 i +
  // lane of the stage's activation and weight arrays.
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const uint8_t* wbase = a.w + (size_t)e * N * (size_t)(K >> 1);
  const uint8_t* wsbase = a.wsf + (size_t)e * N * (size_t)(K >> 5);
  uint32_t aoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int S = 256 * wave + 64 * i + lane;
    if (!A4) {
      const int t = S >> 3, p = (S & 7) ^ ((t >> 1) & 7);
      aoff[i] = s_src[t] * K + 16 * p;
    } else {
      // A4 activations: token t, piece p (K 32p..32p+31) at slot 4 t + (p ^
      // ((t >> 2) & 3)), the weights' layout; 2 instructions per wave
      const int S4 = 128 * wave + 64 * (i & 1) + lane;
      const int t = S4 >> 2, p = (S4 & 3) ^ ((t >> 2) & 3);
      aoff[i] = s_src[t] * (K >> 1) + 16 * p;
    }
    const int r = S >> 2, pw = (S & 3) ^ ((r >> 2) & 3);
    woff[i] = wrow(r) * (K >> 1) + 16 * pw;
  }
  // (uniform 64-bit base + 32-bit lane offset: the scalar-base address form)
  auto issue = [&](Stage& b, uint32_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int S0 = 256 * wave + 64 * i;  // wave-uniform first slot
      if (!A4)
        __builtin_amdgcn_global_load_lds(act + (aoff[i] + k0), &b.act[S0 * 16], 16, 0, 0);
      else if (i < 2)
        __builtin_amdgcn_global_load_lds(act + (aoff[i] + (k0 >> 1)), &b.act[(128 * wave + 64 * i) * 16], 16,
                                         0, 0);
      __builtin_amdgcn_global_load_lds(wbase + (woff[i] + (k0 >> 1)), &b.w[S0 * 16], 16, 0, 0);
    }
  };

  // ---- MFMA over one stage ------------------------------------------------
  v4f acc[8][4];
#pragma unroll
  for (int rg = 0; rg < 8; ++rg)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = v4f{0.f, 0.f, 0.f, 0.f};
  // a wave whose 64 tile rows hold no token skips its MFMAs; otherwise all
  // four 16-row groups are multiplied (rows past the token count are
  // never stored)
  const bool wave_has_tokens = ne - m0 - 64 * wm > 0;

  // Per-lane LDS offsets (bytes): the swizzle terms depend only on the lane
  // (row and token group bases are multiples of 16), so every operand read
  // of a stage is one of these plus a compile-time or wave-uniform offset.
  const int lw = 16 * (4 * r16 + (q ^ ((r16 >> 2) & 3)));     // weight row r16, piece q
  const int xr = (r16 >> 1) & 7;
  const int la0 = 16 * (8 * r16 + (q ^ xr));                  // token r16, piece q
  const int la1 = 16 * (8 * r16 + ((q + 4) ^ xr));            // token r16, piece q + 4
  // first WG-local weight row of row group rg
  auto rbase = [&](int rg) { return FC1 ? (rg < 4 ? 64 * wn + 16 * rg : 128 + 64 * wn + 16 * (rg - 4))
                                        : 128 * wn + 16 * rg; };

  // UE8M0 scales, in registers: per group of 4 stages (16 K blocks) the lane
  // holds the 16 scale bytes of its row in each row group and of its token
  // in each token group; stage gs of the group uses byte 4 gs + q.
  struct GroupScales { uint4 w[8], a[4]; };
  const uint8_t* wsrow[8];
#pragma unroll
  for (int rg = 0; rg < 8; ++rg) wsrow[rg] = wsbase + (size_t)wrow(rbase(rg) + r16) * (K >> 5);
  const uint8_t* asrow[4];
#pragma unroll
  for (int tg = 0; tg < 4; ++tg) asrow[tg] = a.act_sf + (size_t)s_src[64 * wm + 16 * tg + r16] * (K >> 5);
  auto load_scales = [&](GroupScales& g, int kb0) __attribute__((always_inline)) {
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) g.w[rg] = *reinterpret_cast<const uint4*>(wsrow[rg] + kb0);
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) g.a[tg] = *reinterpret_cast<const uint4*>(asrow[tg] + kb0);
  };
  auto sbyte = [&](const uint4& v, int gs) {
    const uint32_t w = gs == 0 ? v.x : gs == 1 ? v.y : gs == 2 ? v.z : v.w;
    return (int)((w >> (8 * q)) & 0xFFu);
  };

  // stage b with scale group g, stage index gs within the group
  auto compute = [&](const Stage& b, const GroupScales& g, int gs) __attribute__((always_inline)) {
    if (!wave_has_tokens) return;
    v8i A[8];
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) {
      const uint4 c = *reinterpret_cast<const uint4*>(&b.w[64 * rbase(rg) + lw]);
      A[rg] = v8i{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int tb = 64 * wm + 16 * tg;
      v8i B;
      if (A4) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(&b.act[64 * tb + lw]);
        B = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
      } else {
        const uint4 b0 = *reinterpret_cast<const uint4*>(&b.act[128 * tb + la0]);
        const uint4 b1 = *reinterpret_cast<const uint4*>(&b.act[128 * tb + la1]);
        B = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
      const int sb = sbyte(g.a[tg], gs);
#pragma unroll
      for (int rg = 0; rg < 8; ++rg)
        acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[rg], B, acc[rg][tg], 4, A4 ? 4 : 0, 0,
                                                                      sbyte(g.w[rg], gs), 0, sb);
    }
  };

  // ---- pipeline: 4-stage ring, loads 3 stages ahead ------------------------
  // Stage c lives in ring buffer c % 4; the scales of group c / 4 in
  // registers, loaded one group ahead.  Step c: wait until this wave's loads of stage c (and of
  // its scale group) have landed -- the loads of the next two stages stay
  // in flight --, barrier (every wave's loads visible, every wave done with
  // stage c - 1), at a group start load the next scale group into the other
  // scale buffer, load stage c + 3 into the buffer stage c - 1 used,
  // multiply stage c.  Buffers are compile-time choices (the loop is
  // unrolled by the ring size) so the compiler sees that the loads in flight
  // never alias the buffers being read, and the vmcnt thresholds are static.
  auto barrier = [&]() __attribute__((always_inline)) {
    // plain s_barrier (__syncthreads() would also wait for the loads in
    // flight); the asm statements keep LDS accesses on their side
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto stage_buf = [&](auto bi) -> Stage& {
    constexpr int B = decltype(bi)::value & 3;
    if constexpr (B == 0) return st0;
    else if constexpr (B == 1) return st1;
    else if constexpr (B == 2) return st2;
    else return st3;
  };
  GroupScales gcur, gnext;  // scales of the current and of the next group
  const int ns = K / GK;
  // Step at position P (0..3) of the unrolled loop = stage c % 4.  The loads
  // issued after stage c's: those of steps c - 2 and c - 1 (8 operand loads
  // each, plus 12 scale loads at a group start, i.e. a step at position 0).
  auto step = [&](auto pi, int c, auto steady) __attribute__((always_inline)) {
    constexpr int P = decltype(pi)::value;
    constexpr bool STEADY = decltype(steady)::value;  // every load of the step in range
    constexpr int after = 2 * kOps + (P == 2 || P == 1 ? kScaleOps : 0);
    if (STEADY) {
      WAIT_VM(after);
    } else {
      if (c + 3 >= ns) __builtin_amdgcn_s_waitcnt(0x0F70);  // fewer loads in flight: wait for all
      else WAIT_VM(after);
    }
    barrier();
    if (P == 0 && (STEADY || c + GS < ns)) load_scales(gnext, (c + GS) * (GK / 32));
    if (STEADY || c + 3 < ns) issue(stage_buf(std::integral_constant<int, P + 3>{}), (c + 3) * GK);
    compute(stage_buf(pi), gcur, P);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  load_scales(gcur, 0);
  issue(st0, 0);
  if (ns > 1) issue(st1, GK);
  if (ns > 2) issue(st2, 2 * GK);
  int c = 0;
  // branch-free steady state: all loads of steps c .. c + 3 are in range
  // (operand stages up to c + 6, scale group (c + 4) / 4)
  for (; c + 7 <= ns; c += 4) {
    const std::true_type S{};
    step(I0{}, c, S);
    step(I1{}, c + 1, S);
    step(I2{}, c + 2, S);
    step(I3{}, c + 3, S);
    gcur = gnext;
  }
  for (; c < ns; c += 4) {
    const std::false_type S{};
    step(I0{}, c, S);
    if (c + 1 >= ns) break;
    step(I1{}, c + 1, S);
    if (c + 2 >= ns) break;
    step(I2{}, c + 2, S);
    if (c + 3 >= ns) break;
    step(I3{}, c + 3, S);
    gcur = gnext;
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
        int ex = amax > 0.0f ? (A4 ? ceil_log2_over_6(amax) : ceil_log2_over_448(amax)) : -127;
        ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
        const float inv = __builtin_ldexpf(1.0f, -ex);
        if (valid) {
          const int ob = nb * 128 + 64 * wn + 32 * j;
          if (A4) {
            // E2M1 RNE (hardware conversion, unit scale), two per byte
            uint8_t* hrow = static_cast<uint8_t*>(a.h_out) + (size_t)slot * (a.I >> 1);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, h[u][0] * inv, h[u][1] * inv, 1.0f, 0);
              d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, h[u][2] * inv, h[u][3] * inv, 1.0f, 1);
              *reinterpret_cast<uint16_t*>(hrow + ((ob + 16 * u + 4 * q) >> 1)) = (uint16_t)d;
            }
          } else {
            uint8_t* hrow = static_cast<uint8_t*>(a.h_out) + (size_t)slot * a.I;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              uint32_t wv = 0;
#pragma unroll
              for (int i = 0; i < 4; ++i) wv |= f32_to_e4m3_rne(h[u][i] * inv) << (8 * i);
              *reinterpret_cast<uint32_t*>(hrow + ob + 16 * u + 4 * q) = wv;
            }
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

template <bool FC1, bool A4>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int nblk = FC1 ? a.I / 128 : a.H / 256;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  // enough workgroups for every work item; the ones past the real count
  // (known on the device only) return at once
  const long long items = (long long)max_tiles * nblk;
  const long long grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((fc_gemm_a8_kernel<FC1, A4>), dim3((unsigned)grid), dim3(256), 0, s, a, nblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc_gemm_a8(const FcArgs& a, bool fc1, bool a4, int max_tiles, hipStream_t s) {
  if (a4) return fc1 ? launch_one<true, true>(a, max_tiles, s) : launch_one<false, true>(a, max_tiles, s);
  return fc1 ? launch_one<true, false>(a, max_tiles, s) : launch_one<false, false>(a, max_tiles, s);
}

}  // namespace moefp4
