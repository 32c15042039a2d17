// Prefill-shaped grouped GEMMs for FP8 activations (E4M3 + UE8M0 per 32)
// over FP4 weights (E2M1 + UE8M0 per 32): FC1 + SwiGLU + FP8 requantisation
// of h, and FC2.  This is the FP8xFP4 recipe (1, 1, 32) of the GLM-5.2 NVFP4
// group16 MegaMoE notes (Context) in the regime where an expert receives
// many tokens; with MXFP4 activations (A4) both MFMA operands are FP4.
//
// Work item: one expert tile of 128 activation rows x 512 weight rows (FC1:
// 256 gate rows and the matching 256 up rows, so SwiGLU and the per-32
// quantisation of h stay inside the workgroup; FC2: 512 output rows).  One
// workgroup of 4 wavefronts per CU; wave w owns 128 weight rows (FC1: gate
// rows 64w..64w+63 of the block and the matching up rows) x all 128 tile
// rows = 8 x 8 tiles of the block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 (A = FP4 weights, B = FP8 or FP4
// activations), 256 FP32 accumulators per lane.
//
// Why this shape: a stage of K = 128 loads 16 KB of activations and 32 KB of
// weights for 64 MFMAs per wave; with 256 weight rows per workgroup the same
// MFMAs needed 64 KB, and the direct-to-LDS fill rate (about 8 TB/s
// chip-wide for these gathered rows once they miss L2), not the matrix
// pipe, set the pace.
//
// Pipeline: K advances in stages of 128 (one MFMA step).  Both operands of a
// stage go HBM/L2 -> LDS with direct-to-LDS 16-byte loads
// (global_load_lds_dwordx4): 8 activation rows x 128 bytes (A4: 16 x 64) or
// 16 weight rows x 64 bytes per instruction.  A ring of 3 stage buffers
// (144 KB) keeps the loads of two stages in flight while one is multiplied;
// the loads of stage c + 2 are issued one at a time between the MFMAs of
// stage c (an issued load holds the wave for tens of cycles while its 64
// addresses go out, which in front of the MFMAs left the matrix pipe idle).
// The UE8M0 block scales of a group of 4 stages (16 bytes per row or tile
// row) go to LDS the same way, one group ahead; each lane keeps the 4 bytes
// it uses in one register per row group and token group, shifted down one
// byte per stage.  Within a stage the first two token groups' activation
// fragments and the weight fragments are read, the first MFMAs wait only
// for the fragment they use, and each later pair of token groups' MFMAs
// runs while the next pair's fragments are read.
//
// Persistent: one workgroup per CU walks its share of the work items and
// streams their stages back to back, so the next item's first stages load
// during the current item's last stages and its epilogue (SwiGLU and the
// quantisation of h, or the FP32 store of the expert outputs).
//
// LDS layouts (16-byte slots, XOR-swizzled so that the 16 lanes of an MFMA
// operand read hit distinct banks):
//   FP8 activations: token t, piece p (K 16p..16p+15) at slot 8 t + (p ^ ((t >> 1) & 7));
//   FP4 activations and weights: row r, piece p (K 32p..32p+31) at slot
//     4 r + (p ^ ((r >> 2) & 3)).
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

constexpr int GK = 128;  // K per pipeline stage (one MFMA step)
constexpr int GS = 4;    // stages per scale group (512 K = 16 scale bytes per row)
constexpr int kRing = 3;
constexpr int kW = 128 * 128;              // byte offset of the weights in a stage
constexpr int kStage = kW + 512 * 64;      // 48 KB: 128 x 128 activation bytes, 512 x 64 weight bytes

struct alignas(16) Ring {
  uint8_t d[kRing * kStage];
};
struct alignas(16) Side {
  uint8_t wsc[512 * 16];     // weight scales of a group: weight row r at 16 r
  uint8_t asc[4][64 * 16];   // tile-row scales: wave w's lanes l at [w][l], tile row 32 w + (l & 31)
  int idx[4][64];            // (FC1) next item's sorted assignments, same lane layout
  int desc[64][8];           // work item descriptors
};

// s_waitcnt with vmcnt(n), expcnt and lgkmcnt at their maxima (gfx9 encoding)
#define WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

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
// the same with a compile-time byte offset in the instruction's offset field
template <int OFF>
__device__ __forceinline__ v4i lds_read16o(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  v4i v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
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
__device__ __forceinline__ void lds_wait(v4i& a, v4i& b, v4i& c, v4i& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void lds_wait(v4i& a0, v4i& a1, v4i& a2, v4i& a3, v4i& a4, v4i& a5, v4i& a6,
                                         v4i& a7) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7));
}
__device__ __forceinline__ void lds_wait(v4i& a0, v4i& a1, v4i& a2, v4i& a3, v4i& a4, v4i& a5, v4i& a6,
                                         v4i& a7, v4i& a8, v4i& a9, v4i& a10, v4i& a11) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7), "+v"(a8),
                 "+v"(a9), "+v"(a10), "+v"(a11));
}

// An accumulator element read through an explicit instruction: the
// compiler would otherwise read every accumulator into VGPRs at the start of
// the epilogue (hoisting the reads out of its per-row conditions), which
// needs more VGPRs than a lane has next to 256 accumulators.  The epilogue
// first waits for the last MFMA's results (these reads are not seen by the
// compiler's hazard checks).
__device__ __forceinline__ float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

// f(integral_constant<int, i>) for i = 0 .. n - 1
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}
// row offset of a wave's row group rg from its first row: FC1 row groups
// 0..3 are gate rows, 4..7 the matching up rows 256 further on
template <bool FC1>
constexpr int roff(int rg) { return FC1 ? (rg < 4 ? 16 * rg : 256 + 16 * (rg - 4)) : 16 * rg; }

// wait until at most N LDS operations of this wave are in flight (vmcnt and
// expcnt at their maxima); LDS operations complete in order
template <int N>
__device__ __forceinline__ void lgkm_wait_n() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// the value passes through an empty asm statement: uses of it come after the
// wait that precedes this
__device__ __forceinline__ void touch(v4i& a) { asm volatile("" : "+v"(a)); }

// A4: MXFP4 activations (E2M1 + UE8M0 per 32, K/2 bytes per row) and h
// quantised to MXFP4 by FC1; both MFMA operands FP4.  PREP: weights in the
// GEMM layout of moe_fp4_prepare_gemm_weights (each stage of a 512-row block
// a contiguous 32 KB image of the LDS weight area, each scale group a
// contiguous 8 KB image of the weight-scale area).
template <bool FC1, bool A4, bool PREP>
__global__ __launch_bounds__(256, 1) void fc_gemm_a8_kernel(FcArgs a, int nblk) {
  // load instructions per wave: activations (128 rows x 128 or 64 bytes of
  // a stage over 4 waves) + 8 for weights (512 rows x 64 bytes); per scale
  // group 2 weight-scale and 1 tile-row-scale loads; (FC1) 1 index load
  constexpr int kActOps = A4 ? 2 : 4;
  constexpr int kOps = kActOps + 8;
  constexpr int kScaleOps = 3;
  constexpr int kIdx = FC1 ? 1 : 0;
  __shared__ Ring ring;
  __shared__ Side side;

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
      *reinterpret_cast<int4*>(&side.desc[tid][0]) = int4{d[0], d[1], d[2], d[3]};
      *reinterpret_cast<int4*>(&side.desc[tid][4]) = int4{d[4], d[5], d[6], d[7]};
    }
    __syncthreads();
  };
  auto describe = [&](int k) __attribute__((always_inline)) {
    const uint32_t at = lds_addr(&side.desc[k & 63][0]);
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
  // global row of work-item-local weight row r (0..511) of row block nb
  auto wrow = [&](int nb, int r) __attribute__((always_inline)) {
    if (FC1) {
      const int i0 = nb * 256 + (r & 255);
      return ((r >= 256) != (a.w13_order != 0)) ? a.I + i0 : i0;
    }
    return nb * 512 + r;
  };
  // first work-item-local weight row of wave row group rg: wrow0 + roff(rg)
  const int wrow0 = FC1 ? 64 * wave : 128 * wave;

  // ---- token rows ---------------------------------------------------------
  // Lane l of wave w holds the source row of tile row 32 w + (l & 31) (FC1:
  // the token of the sorted assignment; FC2: the assignment itself; rows
  // past the expert's token count repeat the tile's first row, their MFMA
  // columns are never stored); the loads fetch the other lanes' with a
  // cross-lane read.  FC1 copies the next item's assignments to LDS once per
  // scale group (a fixed number of memory operations per group keeps the
  // waits static) and reads them back when it switches items.
  auto row_of = [&](const Item& it) __attribute__((always_inline)) {
    const int t = 32 * wave + (lane & 31);
    return it.oe + it.m0 + (it.m0 + t < it.ne ? t : 0);
  };
  auto token_of = [&](const Item& it, int assignment) __attribute__((always_inline)) {
    return FC1 ? assignment / a.top_k : row_of(it);
  };

  // ---- load roles -------------------------------------------------------
  // Activation instruction i of wave w fills stage slots 256 w + 64 i + lane
  // (A4: 128 w + 64 i + lane); weight instruction i fills slots 512 w + 64 i
  // + lane of the weight part: rows 128 w + 16 i + (lane >> 2).  Scale
  // lines: weight rows 128 w + 64 j + lane (j = 0, 1); tile row 32 w + (lane
  // & 31) into the wave's own region.
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const uint8_t* wbase = a.w;   // weight codes of the loading item's expert
  const uint8_t* wsbase = a.wsf;  // its weight scales
  uint32_t aoff[4], woff0 = 0, wsl = 0, asl = 0;  // (A4 uses aoff[0..1])
  auto set_scale_loads = [&](const Item& it, int mine) __attribute__((always_inline)) {
    wsbase = a.wsf + (size_t)it.e * N * (size_t)(K >> 5);
    // (GEMM layout: the row block's groups are 8 KB images of wsc)
    wsl = PREP ? it.nb * (K >> 9) * 8192 + (128 * wave + lane) * 16 : wrow(it.nb, 128 * wave + lane) * (K >> 5);
    asl = mine * (K >> 5);
  };
  auto set_operand_loads = [&](const Item& it, int mine) __attribute__((always_inline)) {
    wbase = a.w + (size_t)it.e * N * (size_t)(K >> 1);
#pragma unroll
    for (int i = 0; i < kActOps; ++i) {
      if (!A4) {
        const int S = 256 * wave + 64 * i + lane;
        const int t = S >> 3, p = (S & 7) ^ ((t >> 1) & 7);
        aoff[i] = __shfl(mine, t - 32 * wave, 64) * K + 16 * p;
      } else {
        const int S = 128 * wave + 64 * i + lane;
        const int t = S >> 2, p = (S & 3) ^ ((t >> 2) & 3);
        aoff[i] = __shfl(mine, t - 32 * wave, 64) * (K >> 1) + 16 * p;
      }
    }
    const int r = 128 * wave + (lane >> 2), pw = (lane & 3) ^ ((lane >> 4) & 3);
    // (GEMM layout: the row block's stages are 32 KB images of the LDS weight
    // area, instruction i of wave w its KB 8 w + i)
    woff0 = PREP ? it.nb * (K >> 7) * 32768 + (512 * wave + lane) * 16 : wrow(it.nb, r) * (K >> 1) + 16 * pw;
  };
  // (uniform 64-bit base + 32-bit lane offset: the scalar-base address form)
  // Load instruction j (0 .. kOps - 1) of a stage: activations first, then
  // weights.  (The LDS destinations are written as element addresses of the
  // shared array itself, which keeps them in the LDS address space.)
  auto issue_one = [&](uint32_t b, uint32_t k0, int j) __attribute__((always_inline)) {
    const uint32_t st = b * kStage;
    if (j < kActOps) {
      if (!A4)
        __builtin_amdgcn_global_load_lds(act + (aoff[j] + k0), &ring.d[st + (256 * wave + 64 * j) * 16], 16, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(act + (aoff[j] + (k0 >> 1)), &ring.d[st + (128 * wave + 64 * j) * 16], 16,
                                         0, 0);
    } else {
      const int i = j - kActOps;
      const uint32_t wo = PREP ? woff0 + 1024 * i + 256 * k0 : woff0 + 8 * K * i + (k0 >> 1);
      __builtin_amdgcn_global_load_lds(wbase + wo, &ring.d[st + kW + (512 * wave + 64 * i) * 16], 16, 0, 0);
    }
  };
  auto issue = [&](uint32_t b, uint32_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kOps; ++j) issue_one(b, k0, j);
  };
  auto issue_scales = [&](uint32_t kb0) __attribute__((always_inline)) {
    // (kb0: the group's byte offset in a RAW scale row, 16 per group)
    const uint32_t w0 = PREP ? wsl + 512 * kb0 : wsl + kb0;
    const uint32_t w1 = PREP ? w0 + 1024 : w0 + 64 * (K >> 5);
    __builtin_amdgcn_global_load_lds(wsbase + w0, &side.wsc[128 * wave * 16], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(wsbase + w1, &side.wsc[(128 * wave + 64) * 16], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(a.act_sf + (asl + kb0), &side.asc[wave][0], 16, 0, 0);
  };

  // The lane's scale bytes for a group: stage gs uses byte 4 gs + q of its
  // row's (token's) 16, so it keeps bytes q, 4 + q, 8 + q, 12 + q in one
  // word and the MFMA picks byte gs of it.
  struct LaneScales { uint32_t w[8], a[8]; };
  const uint32_t sel_lo = (uint32_t)q | ((uint32_t)(4 + q) << 8) | 0x0C0C0000u;
  auto lane_bytes = [&](const v4i& v) __attribute__((always_inline)) {
    const uint32_t l = __builtin_amdgcn_perm((uint32_t)v.y, (uint32_t)v.x, sel_lo);
    const uint32_t h = __builtin_amdgcn_perm((uint32_t)v.w, (uint32_t)v.z, sel_lo);
    return __builtin_amdgcn_perm(h, l, 0x05040100u);
  };
  // per-lane LDS bases of the scale reads (row r16 of the wave's first row
  // group, tile row r16); the row groups' offsets are compile-time
  const uint32_t ws_base = lds_addr(&side.wsc[0]) + (wrow0 + r16) * 16;
  const uint32_t as_base = lds_addr(&side.asc[0][0]) + r16 * 16;
  // A group's scales in two halves: the reads (into 16 line registers), and
  // the wait and the byte selection.  Between them the reads complete under
  // other work (the last MFMAs of the group before).
  struct ScaleLines { v4i t[16]; };
  auto issue_scale_reads = [&](ScaleLines& L) __attribute__((always_inline)) {
    auto rw = [&](auto rgi) __attribute__((always_inline)) {
      constexpr int rg = decltype(rgi)::value;
      L.t[rg] = lds_read16o<16 * roff<FC1>(rg)>(ws_base);
    };
    auto ra = [&](auto tgi) __attribute__((always_inline)) {
      constexpr int tg = decltype(tgi)::value;
      // tile row 16 tg + r16 sits in region (tg >> 1), lane (tg & 1) * 16 + r16
      L.t[8 + tg] = lds_read16o<(tg >> 1) * 1024 + (tg & 1) * 256>(as_base);
    };
    static_for<8>(rw);
    static_for<8>(ra);
  };
  auto finish_scales = [&](ScaleLines& L, LaneScales& d) __attribute__((always_inline)) {
    lds_wait(L.t[0], L.t[1], L.t[2], L.t[3], L.t[4], L.t[5], L.t[6], L.t[7]);
    lds_wait(L.t[8], L.t[9], L.t[10], L.t[11], L.t[12], L.t[13], L.t[14], L.t[15]);
    // (the empty asm statements keep the byte selection here: sunk to the
    // MFMAs, it would keep all 16 lines alive through the group)
#pragma unroll
    for (int rg = 0; rg < 8; ++rg) {
      d.w[rg] = lane_bytes(L.t[rg]);
      asm volatile("" : "+v"(d.w[rg]));
    }
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) {
      d.a[tg] = lane_bytes(L.t[8 + tg]);
      asm volatile("" : "+v"(d.a[tg]));
    }
  };

  // ---- MFMA over one stage ------------------------------------------------
  v4f acc[8][8];
  auto zero_acc = [&]() __attribute__((always_inline)) {
    // (an opaque zero: a hoisted constant would keep a second accumulator
    // set alive across the loop)
    float z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
    for (int rg = 0; rg < 8; ++rg)
#pragma unroll
      for (int tg = 0; tg < 8; ++tg) acc[rg][tg] = v4f{z, z, z, z};
  };
  zero_acc();

  // Per-lane LDS offsets (bytes): the swizzle terms depend only on the lane
  // (row and token group bases are multiples of 16), so every operand read
  // of a stage is one of these plus a wave-uniform offset.
  const int lw = 16 * (4 * r16 + (q ^ ((r16 >> 2) & 3)));     // weight row r16, piece q
  const int xr = (r16 >> 1) & 7;
  const int la0 = 16 * (8 * r16 + (q ^ xr));                  // token r16, piece q
  const int la1 = 16 * (8 * r16 + ((q + 4) ^ xr));            // token r16, piece q + 4

  // Stage in buffer b; g holds the stage's scale bytes in the low byte of
  // each word.  Every token group is multiplied, also the rows past the
  // tile's valid ones (their results are never stored).  Reads: token
  // groups 0 and 1, then the weight fragments in order, so that the first
  // MFMAs wait only for the fragments they use; then each pair of token
  // groups' MFMAs runs while the next pair's activation fragments are read.
  // hook(j), j = 0..15, runs after every 4 MFMAs (it issues the loads of a
  // later stage).
  constexpr int NX = A4 ? 1 : 2;  // LDS reads per activation fragment
  auto compute = [&](uint32_t b, const LaneScales& g, auto&& hook, auto&& before_last)
      __attribute__((always_inline)) {
    const uint32_t sb = lds_addr(&ring.d[0]) + b * kStage;
    const uint32_t bw = sb + kW + 64 * wrow0 + lw;       // weight row group 0's fragment
    const uint32_t bx0 = sb + (A4 ? lw : la0);           // token group 0's fragment (FP8: first half)
    const uint32_t bx1 = sb + la1;                       // (FP8: second half)
    v4i c[8], x0[8], x1[8];
    auto read_w = [&](auto rgi) __attribute__((always_inline)) {
      constexpr int rg = decltype(rgi)::value;
      c[rg] = lds_read16o<64 * roff<FC1>(rg)>(bw);
    };
    auto read_x = [&](auto tgi) __attribute__((always_inline)) {
      constexpr int tg = decltype(tgi)::value;
      if (A4) {
        x0[tg] = lds_read16o<64 * 16 * tg>(bx0);
      } else {
        x0[tg] = lds_read16o<128 * 16 * tg>(bx0);
        x1[tg] = lds_read16o<128 * 16 * tg>(bx1);
      }
    };
    auto touch_x = [&](int tg) __attribute__((always_inline)) {
      touch(x0[tg]);
      if (!A4) touch(x1[tg]);
    };
    auto wait_x = [&](int tg) __attribute__((always_inline)) {
      if (A4) lds_wait(x0[tg], x0[tg + 1]);
      else lds_wait(x0[tg], x1[tg], x0[tg + 1], x1[tg + 1]);
    };
    auto mfma = [&](int tg, int rg) __attribute__((always_inline)) {
      const v8i B = A4 ? v8i{(int)x0[tg].x, (int)x0[tg].y, (int)x0[tg].z, (int)x0[tg].w, 0, 0, 0, 0}
                       : v8i{(int)x0[tg].x, (int)x0[tg].y, (int)x0[tg].z, (int)x0[tg].w, (int)x1[tg].x,
                             (int)x1[tg].y, (int)x1[tg].z, (int)x1[tg].w};
      const v8i A = v8i{(int)c[rg].x, (int)c[rg].y, (int)c[rg].z, (int)c[rg].w, 0, 0, 0, 0};
      acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[rg][tg], 4, A4 ? 4 : 0, 0,
                                                                    (int)g.w[rg], 0, (int)g.a[tg]);
      // (an empty asm statement that reads the result keeps the MFMA here:
      // otherwise it is sunk to the end of the stage, after every load)
      asm volatile("" ::"a"(acc[rg][tg]));
    };
    auto hook_at = [&](int j) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      hook(j);
      __builtin_amdgcn_sched_barrier(0);
    };
    // token group tg's 8 MFMAs, hooks 2 tg and 2 tg + 1
    auto group = [&](auto tgi, auto&& before) __attribute__((always_inline)) {
      constexpr int tg = decltype(tgi)::value;
#pragma unroll
      for (int rg = 0; rg < 8; ++rg) {
        before(rg);
        mfma(tg, rg);
        if (rg == 3 || rg == 7) hook_at(2 * tg + (rg >> 2));
      }
    };
    auto none = [&](int) __attribute__((always_inline)) {};
    read_x(std::integral_constant<int, 0>{});
    read_x(std::integral_constant<int, 1>{});
    static_for<8>(read_w);
    read_x(std::integral_constant<int, 2>{});
    read_x(std::integral_constant<int, 3>{});
    // token group 0: weight fragment rg is done once at most its 7 - rg
    // successors and the 2 prefetched groups' reads are in flight
    group(std::integral_constant<int, 0>{}, [&](int rg) __attribute__((always_inline)) {
      switch (rg) {
        case 0: lgkm_wait_n<7 + 2 * NX>(); touch_x(0); touch_x(1); break;
        case 1: lgkm_wait_n<6 + 2 * NX>(); break;
        case 2: lgkm_wait_n<5 + 2 * NX>(); break;
        case 3: lgkm_wait_n<4 + 2 * NX>(); break;
        case 4: lgkm_wait_n<3 + 2 * NX>(); break;
        case 5: lgkm_wait_n<2 + 2 * NX>(); break;
        case 6: lgkm_wait_n<1 + 2 * NX>(); break;
        default: lgkm_wait_n<0 + 2 * NX>(); break;
      }
      touch(c[rg]);
    });
    group(std::integral_constant<int, 1>{}, none);
    auto pair = [&](auto pri) __attribute__((always_inline)) {
      constexpr int pr = decltype(pri)::value;  // 1..3
      __builtin_amdgcn_sched_barrier(0);
      wait_x(2 * pr);
      if constexpr (pr < 3) {
        read_x(std::integral_constant<int, 2 * pr + 2>{});
        read_x(std::integral_constant<int, 2 * pr + 3>{});
      } else {
        before_last();
      }
      __builtin_amdgcn_sched_barrier(0);
      group(std::integral_constant<int, 2 * pr>{}, none);
      group(std::integral_constant<int, 2 * pr + 1>{}, none);
    };
    pair(std::integral_constant<int, 1>{});
    pair(std::integral_constant<int, 2>{});
    pair(std::integral_constant<int, 3>{});
  };

  // ---- epilogue of one item ------------------------------------------------
  // lane holds, for row group rg and token group tg, weight rows 4q..4q+3 of
  // the 16-row group and token r16 of the 16-token group
  auto epilogue = [&](const Item& it) __attribute__((always_inline)) {
    const int m0 = it.m0, ne = it.ne, oe = it.oe, nb = it.nb;
    const float gsc = it.gs;
    // the last MFMA's results: 32 wait states (an MFMA of 16 passes needs 19)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int tg = 0; tg < 8; ++tg) {
      __builtin_amdgcn_sched_barrier(0);
      const int m = m0 + 16 * tg + r16;
      const bool valid = m < ne;
      const int slot = oe + m;
      if (FC1) {
        // 32-wide h blocks j = 0, 1 of this wave: gate groups 2j, 2j+1 with up
        // groups 4+2j, 5+2j; outputs nb*256 + 64 w + 32 j + [0, 32)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float h[2][4];
          float amax = 0.0f;
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              h[u][i] = swiglu_fast(acc_read(acc[2 * j + u][tg][i]) * gsc, acc_read(acc[4 + 2 * j + u][tg][i]) * gsc);
              amax = fmaxf(amax, fabsf(h[u][i]));
            }
          amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
          amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
          int ex = amax > 0.0f ? (A4 ? ceil_log2_over_6(amax) : ceil_log2_over_448(amax)) : -127;
          ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
          const float inv = __builtin_ldexpf(1.0f, -ex);
          if (valid) {
            const int ob = nb * 256 + 64 * wave + 32 * j;
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
        float* y = a.y_out + (size_t)slot * a.H + nb * 512 + 128 * wave + 4 * q;
#pragma unroll
        for (int rg = 0; rg < 8; ++rg)
          *reinterpret_cast<float4*>(y + 16 * rg) =
              float4{acc_read(acc[rg][tg][0]) * gsc, acc_read(acc[rg][tg][1]) * gsc,
                     acc_read(acc[rg][tg][2]) * gsc, acc_read(acc[rg][tg][3]) * gsc};
      }
    }
  };

  // ---- pipeline ------------------------------------------------------------
  // The workgroup streams the stages of its items back to back through a
  // ring of 3 stage buffers: the loads of a stage are issued two stages
  // ahead, into the buffer the stage before the current one used, so the
  // first stages of the next item load during the last stages and the
  // epilogue of the current one.  The scales of group g + 1 go to LDS during
  // group g (after every wave has taken group g's into registers).  Step c:
  // wait until this wave's loads of stage c (and of its scale group) have
  // landed -- the loads of the next stage stay in flight --, barrier (every
  // wave's loads visible, every wave done with stage c - 1), load stage
  // c + 2, multiply stage c.  The waits are static: a step waits until no
  // more memory operations are outstanding than those issued at later steps
  // (kOps operand loads per step, plus kIdx index loads at a group's first
  // step, before its operand loads, and kScaleOps scale loads at its second).  The stores of an
  // epilogue only make the next group's first waits count more operations
  // than they need to.
  auto barrier = [&]() __attribute__((always_inline)) {
    // plain s_barrier (__syncthreads() would also wait for the loads in
    // flight); the asm statements keep LDS accesses on their side
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // the current item k and the next one (its loads start in the current
  // item's last group)
  fill_desc(0);
  int k = 0;
  Item cur = describe(0);
  bool has_next = n_items > 1;
  Item nxt = has_next ? describe(1) : cur;
  int next_assign = 0;  // (FC1) the next item's sorted assignment of tile row 32 w + (lane & 31)
  {
    const int mine = token_of(cur, FC1 ? a.sorted_assign[row_of(cur)] : 0);
    set_scale_loads(cur, mine);
    set_operand_loads(cur, mine);
  }
  issue_scales(0);
  issue(0, 0);
  issue(1, GK);
  uint32_t bcur = 0;  // ring buffer of the stage being multiplied

  LaneScales gcur;
  bool first = true;
  int cs = 0;        // stage of the current item
  int next_mine = 0; // the next item's source row of tile row 32 w + (lane & 31)
  for (;;) {
    // stage P of its scale group (the group's first stage is cs - P)
    const int P = cs & (GS - 1);
    const bool last_group = cs >= ns - GS;
    if (P >= 2 && last_group && !has_next) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // draining: wait for all
    } else if (P == 0 || P == 3) {
      WAIT_VM(kOps);
    } else if (P == 1) {
      if (FC1 && last_group) WAIT_VM(kOps);  // and the next item's assignments
      else WAIT_VM(kOps + kIdx);
    } else {
      WAIT_VM(kOps + kScaleOps);
    }
    barrier();
    // (a group's scales are read at the previous group's last step; the
    // first group's here)
    if (first) {
      ScaleLines l0;
      issue_scale_reads(l0);
      finish_scales(l0, gcur);
      first = false;
    }
    if (P == 1) {
      if (!last_group) {
        issue_scales((cs - 1 + GS) * 4);
      } else if (has_next) {
        // the next item: its source rows, its first scale group
        if (FC1) {
          next_assign = lds_read4(lds_addr(&side.idx[wave][lane]));
          lds_wait(next_assign);
        }
        next_mine = token_of(nxt, next_assign);
        set_scale_loads(nxt, next_mine);
        issue_scales(0);
      }
    }
    // every operand load of the current item is issued: switch to the next one
    if (P == 2 && last_group && has_next) set_operand_loads(nxt, next_mine);
    // (the copy of the next item's assignments precedes the stage loads, so
    // that the next step's wait covers it)
    if (P == 0 && FC1) __builtin_amdgcn_global_load_lds(a.sorted_assign + row_of(nxt), &side.idx[wave][0], 4, 0, 0);
    // stage cs + 2's loads, one between every 4 MFMAs of stage cs (branch
    // free: past the last stage of the last item they reload the item's
    // first stages into the buffer no stage reads any more, and the
    // draining waits cover them)
    const uint32_t bnext = bcur == 0 ? 2 : bcur - 1;  // (bcur + 2) % 3
    const uint32_t k2 = cs + 2 < ns ? (cs + 2) * GK : (cs + 2 - ns) * GK;
    // at a group's last step the next group's scales (landed with the next
    // stage) are read under the last MFMAs
    const bool next_scales = P == GS - 1 && (!last_group || has_next);
    ScaleLines sl;
    compute(bcur, gcur, [&](int j) __attribute__((always_inline)) {
      if (j < kOps) issue_one(bnext, k2, j);
    }, [&]() __attribute__((always_inline)) {
      if (next_scales) issue_scale_reads(sl);
    });
    // the next stage's scale bytes to the low byte of each word (or the
    // next group's words)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gcur.w[i] >>= 8;
      gcur.a[i] >>= 8;
    }
    if (next_scales) finish_scales(sl, gcur);
    bcur = bcur == 2 ? 0 : bcur + 1;
    if (++cs < ns) continue;
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
    cs = 0;
  }
}

template <bool FC1, bool A4, bool PREP>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int nblk = FC1 ? a.I / 256 : a.H / 512;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  // one workgroup per CU (the ring takes 144 KB of LDS), a multiple of the 8
  // XCDs; each walks its items
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  const long long items = (long long)max_tiles * nblk;
  const long long grid = std::min<long long>(cus / 8 * 8, (items + 7) / 8 * 8);
  hipLaunchKernelGGL((fc_gemm_a8_kernel<FC1, A4, PREP>), dim3((unsigned)grid), dim3(256), 0, s, a, nblk);
  return hipGetLastError();
}

// GEMM weight layout (moe_fp4_prepare_gemm_weights): one 16-byte piece per
// lane, read and written whole.  Codes: piece c of expert e, c = (nb * K/128
// + s) * 2048 + j; scales: piece c = (nb * K/512 + g) * 512 + i.
__global__ __launch_bounds__(256) void prepare_gemm_kernel(const uint8_t* __restrict__ src,
                                                           const uint8_t* __restrict__ src_sf,
                                                           uint8_t* __restrict__ dst, uint8_t* __restrict__ dst_sf,
                                                           int N, int K, int w13, int w13_order, int ncode,
                                                           int nscale) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= ncode + nscale) return;
  // src row of row i of 512-row block nb
  auto row = [&](int nb, int i) {
    if (!w13) return nb * 512 + i;
    const int i0 = nb * 256 + (i & 255);
    return ((i >= 256) != (w13_order != 0)) ? N / 2 + i0 : i0;
  };
  const size_t ecode = (size_t)e * N * (size_t)(K >> 1), escale = (size_t)e * N * (size_t)(K >> 5);
  if (c < ncode) {
    const int ns = K >> 7;
    const int j = c & 2047, bs = c >> 11;  // slot, (block, stage)
    const int nb = bs / ns, st = bs - nb * ns;
    const int piece = (j & 3) ^ ((j >> 4) & 3);
    const uint4 v = *reinterpret_cast<const uint4*>(src + ecode + (size_t)row(nb, j >> 2) * (K >> 1) + 64 * st +
                                                    16 * piece);
    *reinterpret_cast<uint4*>(dst + ecode + (size_t)c * 16) = v;
  } else {
    const int cs = c - ncode;
    const int ng = K >> 9;
    const int i = cs & 511, bg = cs >> 9;  // row, (block, group)
    const int nb = bg / ng, g = bg - nb * ng;
    const uint4 v = *reinterpret_cast<const uint4*>(src_sf + escale + (size_t)row(nb, i) * (K >> 5) + 16 * g);
    *reinterpret_cast<uint4*>(dst_sf + escale + (size_t)cs * 16) = v;
  }
}

}  // namespace

hipError_t launch_fc_gemm_a8(const FcArgs& a, bool fc1, bool a4, bool prep, int max_tiles, hipStream_t s) {
  if (prep) {
    if (a4) return fc1 ? launch_one<true, true, true>(a, max_tiles, s) : launch_one<false, true, true>(a, max_tiles, s);
    return fc1 ? launch_one<true, false, true>(a, max_tiles, s) : launch_one<false, false, true>(a, max_tiles, s);
  }
  if (a4) return fc1 ? launch_one<true, true, false>(a, max_tiles, s) : launch_one<false, true, false>(a, max_tiles, s);
  return fc1 ? launch_one<true, false, false>(a, max_tiles, s) : launch_one<false, false, false>(a, max_tiles, s);
}

hipError_t launch_prepare_gemm(const uint8_t* src, const uint8_t* src_sf, uint8_t* dst, uint8_t* dst_sf,
                               int64_t E, int64_t N, int64_t K, bool w13, int w13_order, hipStream_t s) {
  const int64_t ncode = N * K / 32, nscale = N * K / 512;  // 16-byte pieces per expert
  if (E <= 0 || ncode <= 0) return hipSuccess;
  const int64_t gx = (ncode + nscale + 255) / 256;
  hipLaunchKernelGGL(prepare_gemm_kernel, dim3((unsigned)gx, (unsigned)E), dim3(256), 0, s, src, src_sf, dst, dst_sf,
                     (int)N, (int)K, w13 ? 1 : 0, w13_order, (int)ncode, (int)nscale);
  return hipGetLastError();
}

}  // namespace moefp4
