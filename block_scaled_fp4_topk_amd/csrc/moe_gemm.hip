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
// three stages in flight while one is multiplied.  The UE8M0 block scales of
// a group of 4 stages (16 bytes per row or token) go to LDS the same way,
// one group ahead, and each lane keeps the 4 bytes it uses per stage in one
// register.  A wave whose 64 activation rows hold no token skips its MFMAs.
//
// Persistent: one workgroup per CU walks its share of the work items and
// streams their stages back to back, so the next item's first stages load
// during the current item's last stages and its epilogue (SwiGLU and the
// quantisation of h, or the FP32 store of the expert outputs).  Measured on
// uniform expert tiles (32 experts x 2048 tokens): FC1 1.92 -> 1.77 ms, FC2
// 1.24 -> 1.09 ms against one workgroup per work item, which paid the
// pipeline fill and the epilogue serially each time.
//
// LDS layouts (16-byte slots, XOR-swizzled so that the 16 lanes of an MFMA
// operand read hit distinct banks):
//   activations: token t, piece p (K 16p..16p+15) at slot
//     8 t + (p ^ ((t >> 1) & 7));
//   weights: row r, piece p (K 32p..32p+31) at slot 4 r + (p ^ ((r >> 2) & 3)).
//
// Workgroup -> work items: workgroups are dealt to the 8 XCDs round-robin,
// XCD x owns a contiguous range of the (expert tile, row block) items and
// its workgroups take every nw-th item of it, so the items in flight on an
// XCD are consecutive: an expert's tiles and row blocks share its L2.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace moefp4 {

namespace {

constexpr int GM = 128;  // activation rows per tile
constexpr int GN = 256;  // weight rows per tile
constexpr int GK = 128;  // K per pipeline stage (one MFMA step)
constexpr int GS = 4;    // stages per scale group (512 K = 16 scale bytes per row)

// one pipeline stage: activations (128 tokens x 8 pieces) then weights
// (256 rows x 4 pieces), one array so that the compiler tracks one LDS
// object per stage
struct alignas(16) Stage {
  uint8_t d[2 * 1024 * 16];
};
constexpr int kW = 1024 * 16;  // byte offset of the weights in a stage
// s_waitcnt with vmcnt(n), expcnt and lgkmcnt at their maxima (gfx9 encoding)
#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)
// operand load instructions per wave per stage: 4 weight + 4 activation
// (FP8: 128 tokens x 128 bytes), or + 2 (A4: 128 tokens x 64 bytes)
template <bool A4> constexpr int kOpsOf = A4 ? 6 : 8;

// LDS reads issued as explicit instructions: the compiler does not see them
// as reads of the buffers that direct-to-LDS loads fill (so it adds no waits
// for those loads, whose completion the pipeline's own waits and barriers
// guarantee), and their results are only used after an explicit lgkmcnt
// wait that takes them as operands.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
  v4i v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ int lds_read4(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
// wait for every LDS read in flight; the values pass through the wait
__device__ __forceinline__ void lds_wait(int& a) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a)); }
__device__ __forceinline__ void lds_wait(v4i& a, v4i& b) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b)); }
__device__ __forceinline__ void lds_wait(v4i& a0, v4i& a1, v4i& a2, v4i& a3, v4i& a4, v4i& a5,
                                         v4i& a6, v4i& a7, v4i& a8, v4i& a9, v4i& a10,
                                         v4i& a11) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(a8),
                 "+v"(a9), "+v"(a10), "+v"(a11));
}
__device__ __forceinline__ void lds_wait(v4i& a0, v4i& a1, v4i& a2, v4i& a3, v4i& a4, v4i& a5,
                                         v4i& a6, v4i& a7, v4i& a8, v4i& a9, v4i& a10, v4i& a11,
                                         v4i& a12, v4i& a13, v4i& a14, v4i& a15) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(a8),
                 "+v"(a9), "+v"(a10), "+v"(a11), "+v"(a12), "+v"(a13), "+v"(a14), "+v"(a15));
}
constexpr int kScaleOps = 2;  // scale load instructions per wave per group (weight rows, tile rows)

struct alignas(16) Side {
  uint8_t wsc[256 * 16];
  uint8_t asc[4][64 * 16];
  int idx[4][64];
};

// A4: MXFP4 activations (E2M1 + UE8M0 per 32, K/2 bytes per row) and h
// quantised to MXFP4 by FC1; both MFMA operands FP4.
template <bool FC1, bool A4>
__global__ __launch_bounds__(256, 1) void fc_gemm_a8_kernel(FcArgs a, int nblk) {
  constexpr int kOps = kOpsOf<A4>;
  constexpr int kIdx = FC1 ? 1 : 0;  // token-index loads per wave per group (FC1)
  __shared__ Stage st0, st1, st2, st3;
  // UE8M0 scales of one group of 4 stages (16 K blocks, 16 bytes per row):
  // the 256 weight rows, and the 128 tile rows twice (wave w loads rows
  // 64 (w / 2) .. + 64 into copy w)
  __shared__ Side side;
  __shared__ __attribute__((aligned(16))) int s_desc[64][8];
  auto& s_wsc = side.wsc;
  auto& s_asc = side.asc;
  // (FC1) wave w's copy of the next item's sorted assignments of tile rows
  // 64 (w / 2) .. + 64
  auto& s_idx = side.idx;

  // this workgroup's work items: XCD x owns the contiguous range
  // [x * per_xcd, (x + 1) * per_xcd) of the (expert tile, row block) items,
  // and its nw workgroups take every nw-th item of it
  const int items = a.ntiles[0] * nblk;
  const int per_xcd = (items + 7) >> 3;
  const int nw = gridDim.x >> 3;
  const int lo = (blockIdx.x & 7) * per_xcd;
  const int hi = min(items, lo + per_xcd);
  const int v0 = lo + (blockIdx.x >> 3);
  if (v0 >= hi) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int r16 = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = a.K, N = a.N;
  const int ns = K / GK;  // stages per item (a multiple of GS)

  // Item k of this workgroup is v0 + k nw.  Their descriptors (row block,
  // expert, first tile row, the expert's token count and offset, its global
  // scale) are read 64 at a time into LDS while no load is in flight, so
  // that switching items issues no memory operation.
  struct Item { int nb, e, m0, ne, oe; float gs; };
  const int n_items = (hi - v0 + nw - 1) / nw;
  auto fill_desc = [&](int k0) __attribute__((always_inline)) {
    if (tid < 64) {
      const int vv = v0 + (k0 + tid) * nw;
      int d[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (vv < hi) {
        const int tile = vv / nblk;
        d[0] = vv - tile * nblk;
        d[1] = a.tiles[2 * tile];
        d[2] = a.tiles[2 * tile + 1];
        d[3] = a.counts[d[1]];
        d[4] = a.offsets[d[1]];
        d[5] = __float_as_int(a.gs ? a.gs[d[1]] : 1.0f);
      }
      *reinterpret_cast<int4*>(&s_desc[tid][0]) = int4{d[0], d[1], d[2], d[3]};
      *reinterpret_cast<int4*>(&s_desc[tid][4]) = int4{d[4], d[5], d[6], d[7]};
    }
    __syncthreads();
  };
  auto describe = [&](int k) __attribute__((always_inline)) {
    const uint32_t at = lds_addr(&s_desc[k & 63][0]);
    v4i d0 = lds_read16(at), d1 = lds_read16(at + 16);
    lds_wait(d0, d1);
    Item it;
    it.nb = __builtin_amdgcn_readfirstlane(d0.x);
    it.e = __builtin_amdgcn_readfirstlane(d0.y);
    it.m0 = __builtin_amdgcn_readfirstlane(d0.z);
    it.ne = __builtin_amdgcn_readfirstlane(d0.w);
    it.oe = __builtin_amdgcn_readfirstlane(d1.x);
    it.gs = __int_as_float(__builtin_amdgcn_readfirstlane(d1.y));
    return it;
  };
  // global row of WG-local weight row r of row block nb
  auto wrow = [&](int nb, int r) __attribute__((always_inline)) {
    if (FC1) {
      const int i0 = nb * 128 + (r & 127);
      return ((r >= 128) != (a.w13_order != 0)) ? a.I + i0 : i0;
    }
    return nb * 256 + r;
  };
  // first WG-local weight row of row group rg
  auto rbase = [&](int rg) { return FC1 ? (rg < 4 ? 64 * wn + 16 * rg : 128 + 64 * wn + 16 * (rg - 4))
                                        : 128 * wn + 16 * rg; };

  // ---- token rows ---------------------------------------------------------
  // Every tile row a wave touches lies in its half 64 wm .. 64 wm + 63 of the
  // tile: lane l holds the source row of tile row 64 wm + l (FC1: the token
  // of the sorted assignment; FC2: the assignment itself; rows past the
  // expert's token count repeat the tile's first row, their MFMA columns
  // are never stored), and the other lanes fetch theirs with a cross-lane
  // read.  FC1 copies the next item's assignments to LDS once per scale
  // group (a fixed number of memory operations per group keeps the waits
  // static) and reads them back at the item switch.
  auto row_of = [&](const Item& it) __attribute__((always_inline)) {
    const int t = 64 * wm + lane;
    return it.oe + it.m0 + (it.m0 + t < it.ne ? t : 0);
  };
  auto token_of = [&](const Item& it, int assignment) __attribute__((always_inline)) {
    return FC1 ? assignment / a.top_k : row_of(it);
  };

  // ---- load roles -------------------------------------------------------
  // Operand instruction i (0..3) of wave w fills slots S = 256 w + 64 i +
  // lane of the stage's activation and weight arrays; the weight rows of
  // instruction i are those of instruction 0 plus 16 i.  Scale lines: lane l
  // of wave w loads weight row 64 w + l and tile row 64 (w / 2) + l.
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const uint8_t* wbase;   // weight codes of the loading item's expert
  const uint8_t* wsbase;  // its weight scales
  uint32_t aoff[4], woff0, wsl, asl;
  auto set_loads = [&](const Item& it, int mine) __attribute__((always_inline)) {
    wbase = a.w + (size_t)it.e * N * (size_t)(K >> 1);
    wsbase = a.wsf + (size_t)it.e * N * (size_t)(K >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int S = 256 * wave + 64 * i + lane;
      if (!A4) {
        const int t = S >> 3, p = (S & 7) ^ ((t >> 1) & 7);
        aoff[i] = __shfl(mine, t - 64 * wm, 64) * K + 16 * p;
      } else {
        // A4 activations: token t, piece p (K 32p..32p+31) at slot 4 t + (p ^
        // ((t >> 2) & 3)), the weights' layout; 2 instructions per wave
        const int S4 = 128 * wave + 64 * (i & 1) + lane;
        const int t = S4 >> 2, p = (S4 & 3) ^ ((t >> 2) & 3);
        aoff[i] = __shfl(mine, t - 64 * wm, 64) * (K >> 1) + 16 * p;
      }
    }
    const int r = 64 * wave + (lane >> 2), pw = (lane & 3) ^ ((lane >> 4) & 3);
    woff0 = wrow(it.nb, r) * (K >> 1) + 16 * pw;
    wsl = wrow(it.nb, 64 * wave + lane) * (K >> 5);
    asl = mine * (K >> 5);
  };
  // (uniform 64-bit base + 32-bit lane offset: the scalar-base address form)
  auto issue = [&](Stage& b, uint32_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int S0 = 256 * wave + 64 * i;  // wave-uniform first slot
      if (!A4)
        __builtin_amdgcn_global_load_lds(act + (aoff[i] + k0), &b.d[S0 * 16], 16, 0, 0);
      else if (i < 2)
        __builtin_amdgcn_global_load_lds(act + (aoff[i] + (k0 >> 1)), &b.d[(128 * wave + 64 * i) * 16], 16,
                                         0, 0);
      __builtin_amdgcn_global_load_lds(wbase + (woff0 + 8 * K * i + (k0 >> 1)), &b.d[kW + S0 * 16], 16, 0, 0);
    }
  };
  auto issue_scales = [&](uint32_t kb0) __attribute__((always_inline)) {
    __builtin_amdgcn_global_load_lds(wsbase + (wsl + kb0), &s_wsc[64 * wave * 16], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(a.act_sf + (asl + kb0), &s_asc[wave][0], 16, 0, 0);
  };

  // The lane's scale bytes for a group: stage gs uses byte 4 gs + q of its
  // row's (token's) 16, so it keeps bytes q, 4 + q, 8 + q, 12 + q in one
  // word and the MFMA picks byte gs of it.
  struct LaneScales { uint32_t w[8], a[4]; };
  const uint32_t sel_lo = (uint32_t)q | ((uint32_t)(4 + q) << 8) | 0x0C0C0000u;
  auto lane_bytes = [&](const v4i& v) __attribute__((always_inline)) {
    const uint32_t l = __builtin_amdgcn_perm((uint32_t)v.y, (uint32_t)v.x, sel_lo);
    const uint32_t h = __builtin_amdgcn_perm((uint32_t)v.w, (uint32_t)v.z, sel_lo);
    return __builtin_amdgcn_perm(h, l, 0x05040100u);
  };
  const uint32_t wsc_addr = lds_addr(&s_wsc[((FC1 ? 64 : 128) * wn + r16) * 16]);
  const uint32_t asc_addr = lds_addr(&s_asc[2 * wm][r16 * 16]);
  auto read_scales = [&](LaneScales& d) __attribute__((always_inline)) {
    v4i w[8], t[4];
#pragma unroll
    for (int rg = 0; rg < 8; ++rg)
      w[rg] = lds_read16(wsc_addr + (FC1 ? (rg < 4 ? 16 * rg : 128 + 16 * (rg - 4)) : 16 * rg) * 16);
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) t[tg] = lds_read16(asc_addr + tg * 256);
    lds_wait(w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7], t[0], t[1], t[2], t[3]);
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) d.w[rg] = lane_bytes(w[rg]);
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) d.a[tg] = lane_bytes(t[tg]);
  };

  // ---- MFMA over one stage ------------------------------------------------
  v4f acc[8][4];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rg = 0; rg < 8; ++rg)
#pragma unroll
      for (int tg = 0; tg < 4; ++tg) acc[rg][tg] = v4f{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();

  // Per-lane LDS offsets (bytes): the swizzle terms depend only on the lane
  // (row and token group bases are multiples of 16), so every operand read
  // of a stage is one of these plus a compile-time or wave-uniform offset.
  const int lw = 16 * (4 * r16 + (q ^ ((r16 >> 2) & 3)));     // weight row r16, piece q
  const int xr = (r16 >> 1) & 7;
  const int la0 = 16 * (8 * r16 + (q ^ xr));                  // token r16, piece q
  const int la1 = 16 * (8 * r16 + ((q + 4) ^ xr));            // token r16, piece q + 4

  // stage b, stage gs of its scale group; a wave whose 64 tile rows hold no
  // token skips its MFMAs (otherwise all four 16-row groups are multiplied)
  auto compute = [&](const Stage& b, const LaneScales& g, auto gsi, bool has_tokens)
      __attribute__((always_inline)) {
    constexpr int gs = decltype(gsi)::value;
    if (!has_tokens) return;
    // every operand of the stage: the weight fragments, then the token
    // groups' (FP8: two halves each)
    const uint32_t base = lds_addr(&b.d[0]);
    v4i c[8], x0[4], x1[4];
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) c[rg] = lds_read16(base + kW + 64 * rbase(rg) + lw);
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int tb = 64 * wm + 16 * tg;
      if (A4) {
        x0[tg] = lds_read16(base + 64 * tb + lw);
      } else {
        x0[tg] = lds_read16(base + 128 * tb + la0);
        x1[tg] = lds_read16(base + 128 * tb + la1);
      }
    }
    if (A4)
      lds_wait(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], x0[0], x0[1], x0[2], x0[3]);
    else
      lds_wait(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], x0[0], x0[1], x0[2], x0[3], x1[0], x1[1],
               x1[2], x1[3]);
    v8i A[8];
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) A[rg] = v8i{(int)c[rg].x, (int)c[rg].y, (int)c[rg].z, (int)c[rg].w, 0, 0, 0, 0};
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const v8i B = A4 ? v8i{(int)x0[tg].x, (int)x0[tg].y, (int)x0[tg].z, (int)x0[tg].w, 0, 0, 0, 0}
                       : v8i{(int)x0[tg].x, (int)x0[tg].y, (int)x0[tg].z, (int)x0[tg].w, (int)x1[tg].x,
                             (int)x1[tg].y, (int)x1[tg].z, (int)x1[tg].w};
#pragma unroll
      for (int rg = 0; rg < 8; ++rg)
        acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[rg], B, acc[rg][tg], 4, A4 ? 4 : 0, gs,
                                                                      (int)g.w[rg], gs, (int)g.a[tg]);
    }
  };

  // ---- epilogue of one item ------------------------------------------------
  // lane holds, for row group rg and token group tg, weight rows 4q..4q+3 of
  // the 16-row group and token r16 of the 16-token group
  auto epilogue = [&](const Item& it) __attribute__((always_inline)) {
    const int e = it.e, m0 = it.m0, ne = it.ne, oe = it.oe, nb = it.nb;
    const float gsc = it.gs;
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
              h[u][i] = swiglu_fast(acc[2 * j + u][tg][i] * gsc, acc[4 + 2 * j + u][tg][i] * gsc);
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
                // E4M3 RNE (hardware conversion; bit-identical to f32_to_e4m3_rne
                // over the whole range |y| <= 448, checked exhaustively per
                // exponent and rounding tie), four per word
                int wv = __builtin_amdgcn_cvt_pk_fp8_f32(h[u][0] * inv, h[u][1] * inv, 0, false);
                wv = __builtin_amdgcn_cvt_pk_fp8_f32(h[u][2] * inv, h[u][3] * inv, wv, true);
                *reinterpret_cast<uint32_t*>(hrow + ob + 16 * u + 4 * q) = (uint32_t)wv;
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
  };

  // ---- pipeline ------------------------------------------------------------
  // The workgroup streams the stages of its items back to back through a
  // ring of 4 stage buffers: stage c of the stream lives in buffer c % 4 and
  // its loads are issued three stages ahead, so the first stages of the next
  // item load during the last stages and the epilogue of the current one.
  // The scales of group g + 1 go to LDS during group g (after every wave
  // has taken group g's into registers).  Step c: wait until this wave's
  // loads of stage c (and of its scale group) have landed -- the loads of
  // the next two stages stay in flight --, barrier (every wave's loads
  // visible, every wave done with stage c - 1), load stage c + 3 into the
  // buffer stage c - 1 used, multiply stage c.  Buffers are compile-time
  // choices (the loop is unrolled by the ring size, and an item is a whole
  // number of groups) so the compiler sees that the loads in flight never
  // alias the buffers being read, and the vmcnt thresholds are static: a
  // step waits until no more memory operations are outstanding than those
  // issued at later steps (kOps operand loads per step, plus kIdx index
  // loads at a group's first step and kScaleOps scale loads at its second).
  // The stores of an epilogue only make the next group's first waits count
  // more operations than they need to.
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

  // the current item k and the next one (its loads start in the current
  // item's last group)
  fill_desc(0);
  int k = 0;
  Item cur = describe(0);
  bool has_next = n_items > 1;
  Item nxt = has_next ? describe(1) : cur;
  int next_assign = 0;  // (FC1) the next item's sorted assignment of tile row 64 wm + lane
  set_loads(cur, token_of(cur, FC1 ? a.sorted_assign[row_of(cur)] : 0));
  issue_scales(0);
  issue(st0, 0);
  issue(st1, GK);
  issue(st2, 2 * GK);

  LaneScales gcur;
  int c = 0;  // stage of the current item at the group start
  bool has_tokens = cur.ne - cur.m0 - 64 * wm > 0;
  auto step = [&](auto pi) __attribute__((always_inline)) {
    constexpr int P = decltype(pi)::value;
    constexpr int after = 2 * kOps + (P == 1 || P == 2 ? kIdx : 0) + (P == 2 || P == 3 ? kScaleOps : 0);
    const int cs = c + P;
    const bool last_group = c + GS == ns;
    if (P != 0 && last_group && !has_next) __builtin_amdgcn_s_waitcnt(0x0F70);  // draining: wait for all
    else WAIT_VM(after);
    barrier();
    if (P == 0) {
      read_scales(gcur);
      // (copied at an earlier group start; this group's copy is issued below)
      if (FC1 && last_group && has_next) {
        next_assign = lds_read4(lds_addr(&s_idx[wave][lane]));
        lds_wait(next_assign);
      }
    }
    if (P == 1) {
      if (!last_group) {
        issue_scales((c / GS + 1) * 16);
      } else if (has_next) {
        // every load of the current item is issued: switch to the next one
        set_loads(nxt, token_of(nxt, next_assign));
        issue_scales(0);
      }
    }
    if (cs + 3 < ns) issue(stage_buf(std::integral_constant<int, P + 3>{}), (cs + 3) * GK);
    else if (has_next) issue(stage_buf(std::integral_constant<int, P + 3>{}), (cs + 3 - ns) * GK);
    if (P == 0 && FC1) __builtin_amdgcn_global_load_lds(a.sorted_assign + row_of(nxt), &s_idx[wave][0], 4, 0, 0);
    compute(stage_buf(pi), gcur, pi, has_tokens);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  for (;;) {
    step(I0{});
    step(I1{});
    step(I2{});
    step(I3{});
    if (c + GS < ns) {
      c += GS;
      continue;
    }
    epilogue(cur);
    if (!has_next) break;
    zero_acc();
    cur = nxt;
    ++k;
    has_next = k + 1 < n_items;
    if (has_next) {
      // (a new batch of descriptors: every load in flight is waited for)
      if (((k + 1) & 63) == 0) fill_desc(k + 1);
      nxt = describe(k + 1);
    }
    has_tokens = cur.ne - cur.m0 - 64 * wm > 0;
    c = 0;
  }
}

template <bool FC1, bool A4>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int nblk = FC1 ? a.I / 128 : a.H / 256;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  // one workgroup per CU (the ring takes 128 KB of LDS), a multiple of the 8
  // XCDs; each walks its items
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  const long long items = (long long)max_tiles * nblk;
  const long long grid = std::min<long long>(cus / 8 * 8, (items + 7) / 8 * 8);
  hipLaunchKernelGGL((fc_gemm_a8_kernel<FC1, A4>), dim3((unsigned)grid), dim3(256), 0, s, a, nblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc_gemm_a8(const FcArgs& a, bool fc1, bool a4, int max_tiles, hipStream_t s) {
  if (a4) return fc1 ? launch_one<true, true>(a, max_tiles, s) : launch_one<false, true>(a, max_tiles, s);
  return fc1 ? launch_one<true, false>(a, max_tiles, s) : launch_one<false, false>(a, max_tiles, s);
}

}  // namespace moefp4
