// Decode-shaped grouped GEMMs: FC1 + SwiGLU (+ h quantisation) and FC2 for
// expert tiles of at most 16 activation rows.
//   MODE 0  bf16 activations, group16 E4M3 weights   -> fp16 MFMA
//   MODE 1  bf16 activations, group32 UE8M0 weights  -> bf16 MFMA
//   MODE 2  FP8 + UE8M0 activations, group32 weights -> block-scaled MFMA
//   MODE 3  MXFP4 activations (A4), group32 weights  -> block-scaled MFMA,
//           both operands FP4
// (the W4A16 forms of b12x moe/fused/w4a16/prepare.py and the FP8xFP4
// recipe (1, 1, 32) of the GLM-5.2 NVFP4 group16 MegaMoE notes, Context).
//
// Decode is a weight stream, so the kernel is built around how the weight
// bytes leave HBM.  A workgroup owns 128 weight rows of one expert (FC1: 64
// gate + the matching 64 up rows; FC2: 128 output rows) and walks K in
// 256-element chunks (128 code bytes per row).  Each chunk's 16 KB of codes
// goes straight to LDS with 16-byte direct-to-LDS loads marked non-temporal,
// every load instruction covering eight whole 128-byte rows (measured on the
// decode16 FC1 geometry: 6.8 TB/s for this form against 6.1 TB/s for
// register loads in the MFMA lane layout, which can only ask for 64 bytes
// of each row per instruction).  The block scales stream the same way, one
// 128-byte line per row per scale group (8 chunks of group16 scales or 16
// chunks of group32 scales): the next group's lines arrive a slice per
// chunk, and at the start of a group every lane copies its own scale bytes
// of all the group's chunks into registers, which frees the buffer.
// Activation rows that hold a token are loaded into registers one chunk
// ahead and staged in LDS once for the 4 waves; for group16 FC1 the route
// launch has already written x as fp16 x 2**-p (exact), and those rows go
// straight to LDS with direct-to-LDS loads beside the weights (the register
// staging sat on the critical path of every chunk: 530 -> 513 us on the
// decode16 FC1).
//
// Per chunk: stage the activations, barrier, read every operand of the
// chunk into registers, issue the next chunk's loads (into a second set of
// buffers, or into the same ones after a second barrier), MFMAs.  Two or
// three workgroups per CU keep loads in flight while others read and
// compute.
//
// K index permutation inside a chunk (identical for both MFMA operands):
// lane group q (= lane / 16) holds code bytes [32 q, 32 q + 32) of a row,
// i.e. K [64 q, 64 q + 64):
//   16-bit MFMA j = 0..7 takes K [64 q + 8 j, + 8) (code dword j);
//   scaled MFMA step st = 0, 1: hardware K block b of the step is memory K
//   block 2 b + st (32 elements), so the FP4 operand of lane group q is code
//   bytes [32 q + 16 st, + 16) and the FP8 operand lane group q takes the
//   16-element halves of memory blocks 2 (q / 2) + st and 4 + 2 (q / 2) + st
//   selected by q % 2 (the FP8 lane layout of common.h).
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace moefp4 {

namespace {

constexpr int KC = 256;   // K elements per chunk
constexpr int WR = 128;   // weight rows per workgroup
constexpr int kNT = 2;    // cache policy of the weight / scale loads: non-temporal

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled
template <int N, int I = 0, typename F>
__device__ __forceinline__ void unroll_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    unroll_for<N, I + 1>(f);
  }
}

// A wave-uniform pointer held as one scalar register pair, so that a load
// from it plus a 32-bit per-lane offset is selected as one instruction with
// a scalar base (rather than 64-bit vector adds of its parts per load).
__device__ __forceinline__ const uint8_t* sbase(const uint8_t* p) {
  uint64_t v = reinterpret_cast<uint64_t>(p);
  asm volatile("" : "+s"(v));
  return reinterpret_cast<const uint8_t*>(v);
}

__device__ __forceinline__ uint32_t dw(const uint4& v, int r) {
  return r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w;
}

// 16-byte segment swizzle of a staged scale line: row lr keeps logical
// segment s at s ^ sc_swz(lr), so the 16 lanes reading one dword of 16
// consecutive rows hit 16 distinct bank groups
__device__ __forceinline__ int sc_swz(int lr) { return (lr >> 1) & 7; }

// One item: expert tile `tile` (<= 16 activation rows of one expert) x weight
// row block `rb` (FC1: gate rows [64 rb, 64 rb + 64) and the matching up
// rows; FC2: output rows [128 rb, 128 rb + 128)), the whole K.  The LDS
// arrays are the calling kernel's own __shared__ arrays, passed in (distinct
// objects, so the compiler keeps the loads into one buffer apart from the
// reads of another).
template <int MODE, bool FC1>
__device__ __forceinline__ void decode_item(const FcArgs& a, const int tile, const int rb, uint8_t* s_w0,
                                            uint8_t* s_w1, uint8_t* s_sc, uint8_t* s_b0, uint8_t* s_b1,
                                            uint8_t* s_bsf0, uint8_t* s_bsf1, int* s_src, float* s_rs,
                                            float (*s_amax)[16]) {
  constexpr bool RING2 = MODE == 0 && FC1;
  // ADMA: the activation rows are fp16 already (converted by the route
  // launch) and go straight to LDS like the weights, with no register staging
  constexpr bool ADMA = MODE == 0 && FC1;
  constexpr bool SCALED = MODE >= 2;                   // block-scaled activations (FP8 or FP4)
  constexpr int ACB = MODE == 3 ? KC / 2 : MODE == 2 ? KC : 2 * KC;  // activation bytes per row per chunk
  constexpr int AROW = ADMA ? ACB : ACB + 16;          // staged activation row stride
  constexpr int SEGB = ACB / 16;                       // activation bytes per thread (32, 16 or 8)
  constexpr int SCB = MODE == 0 ? KC / 16 : KC / 32;   // weight-scale bytes per row per chunk
  constexpr int SG = 128 / SCB;                        // chunks per scale group
  constexpr int RPC = WR / SG;                         // scale lines staged per chunk (16 or 8)

  // (wave-uniform by construction; readfirstlane states it for the
  // persistent kernel, whose item index the compiler cannot prove uniform)
  const int e = __builtin_amdgcn_readfirstlane(a.tiles[2 * tile]);
  const int m0 = __builtin_amdgcn_readfirstlane(a.tiles[2 * tile + 1]);
  const int ne = __builtin_amdgcn_readfirstlane(a.counts[e]), oe = __builtin_amdgcn_readfirstlane(a.offsets[e]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int nchunks = K / KC;
  const int ngroups = (nchunks + SG - 1) / SG;
  const size_t rowb = (size_t)(K >> 1);          // code bytes per weight row
  const int sb = K / (MODE == 0 ? 16 : 32);       // scale bytes per weight row
  const uint8_t* wexp = a.w + (size_t)e * N * rowb;
  const uint8_t* sexp = a.wsf + (size_t)e * N * sb;

  // workgroup-local weight row (0..127) -> row of the expert's matrix
  auto wrow = [&](int lr) __attribute__((always_inline)) -> int {
    if (FC1) {
      const int i0 = rb * 64 + (lr & 63);
      return ((lr >= 64) != (a.w13_order != 0)) ? a.I + i0 : i0;
    }
    return rb * 128 + lr;
  };

  // weight loads: instruction i of a wave covers rows 32 wave + 8 i .. + 8;
  // lane -> row + lane / 8, LDS slot lane % 8 holding the row's 16-byte
  // segment (lane % 8) ^ (row % 8).  Addresses are a wave-uniform base (the
  // expert's weights plus the chunk) and a 32-bit per-lane offset (the
  // forward rejects experts of 2 GB or more), so each load is one
  // instruction with no 64-bit address arithmetic per chunk.
  uint32_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = 32 * wave + 8 * i + (lane >> 3);
    woff[i] = (uint32_t)wrow(lr) * (uint32_t)rowb + 16u * ((lane & 7) ^ (lr & 7));
  }
  auto issue_w = [&](int c, uint8_t* sw) __attribute__((always_inline)) {
    const uint8_t* base = sbase(wexp + (size_t)c * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(base + woff[i], sw + (32 * wave + 8 * i) * 128, 16, 0, kNT);
  };
  // scale loads: this wave's rows [rb0, rb0 + nrows) of group g's 128-byte
  // lines, 16 bytes per lane (8 rows per instruction) when the scale rows
  // are 16-byte aligned, else 4 bytes (2 rows); bytes past a row's scales
  // are not read
  const bool sc16 = (sb & 15) == 0;
  auto issue_sc = [&](int g, int rb0, int nrows) __attribute__((always_inline)) {
    if (sc16) {
      for (int r = rb0; r < rb0 + nrows; r += 8) {
        const int lr = r + (lane >> 3);
        const int off = 128 * g + 16 * ((lane & 7) ^ sc_swz(lr));
        if (off < sb)
          __builtin_amdgcn_global_load_lds(sexp + (size_t)wrow(lr) * sb + off, &s_sc[r * 128], 16, 0, kNT);
      }
    } else {
      for (int r = rb0; r < rb0 + nrows; r += 2) {
        const int lr = r + (lane >> 5);
        const int off = 128 * g + 4 * ((lane & 31) ^ (4 * sc_swz(lr)));
        if (off < sb)
          __builtin_amdgcn_global_load_lds(sexp + (size_t)wrow(lr) * sb + off, &s_sc[r * 128], 4, 0, kNT);
      }
    }
  };
  // slice j (0..SG-1) of group g's lines: rows [j RPC, (j + 1) RPC), split
  // over the waves
  auto issue_sc_slice = [&](int g, int j) __attribute__((always_inline)) {
    if (sc16) {
      if (8 * wave < RPC) issue_sc(g, j * RPC + 8 * wave, 8);
    } else {
      issue_sc(g, j * RPC + wave * (RPC / 4), RPC / 4);
    }
  };
  // The same for group16 scales (always 16-byte rows of lines, RPC = 16:
  // waves 0 and 1 load 8 rows each): the lane's row of slice 0 and its
  // swizzled segment are fixed per lane, slice j adds a wave-uniform row step.
  const int sc_lr = 8 * wave + (lane >> 3);
  const uint32_t sc_seg = 16u * ((lane & 7) ^ sc_swz(sc_lr));
  const uint32_t sc_off = MODE == 0 ? (uint32_t)wrow(sc_lr) * (uint32_t)sb + sc_seg : 0u;
  const bool sc_full = (sb & 127) == 0;  // every line whole: no per-lane check
  auto issue_sc_slice0 = [&](int g, int j) __attribute__((always_inline)) {
    if (wave < 2) {
      int rstep = 16 * j;
      if (FC1) {
        const bool up0 = a.w13_order != 0, upj = (j >= 4) != up0;
        rstep = 16 * (j & 3) + (upj ? a.I : 0) - (up0 ? a.I : 0);
      }
      const uint8_t* base = sbase(sexp + (ptrdiff_t)rstep * sb + 128 * g);
      if (sc_full || 128 * g + (int)sc_seg < sb)
        __builtin_amdgcn_global_load_lds(base + sc_off, &s_sc[(j * RPC + 8 * wave) * 128], 16, 0, kNT);
    }
  };

  if (tid < 16) {
    const int m = m0 + tid;
    int src = -1;
    float sc = 1.0f;
    if (m < ne) {
      const int slot = oe + m;
      src = FC1 ? a.sorted_assign[slot] / a.top_k : slot;
      if (MODE == 0) {
        if (FC1) {
          sc = a.act_scale[src];
        } else {
          // (an atomic load: FC1 publishes the maxima with atomics, in the
          // single-launch form during this same launch)
          const uint32_t hm = __hip_atomic_load(a.hmax_in + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          sc = __builtin_ldexpf(1.0f, hm ? (int)(hm >> 23) - 127 - 14 : 0);
        }
      }
    }
    s_src[tid] = src;
    s_rs[tid] = sc;
  }
  // Activation rows that hold no token are zero for the whole item (only
  // rows with a token are written below).  Their MFMA columns are never
  // stored either way, but multiplying zeros draws less power than stale
  // LDS contents: measured on decode16, the shader clock then stays ~50 MHz
  // higher while the GPU ramps up after an idle period (steps 0.5-2% faster).
  {
    constexpr int BYTES = 16 * AROW;
    for (int o = 16 * tid; o < BYTES; o += 16 * 256) {
      *reinterpret_cast<uint4*>(s_b0 + o) = uint4{0u, 0u, 0u, 0u};
      if (RING2) *reinterpret_cast<uint4*>(s_b1 + o) = uint4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();

  // ADMA loads: instruction i = wave, wave + 4 fills LDS rows 2 i, 2 i + 1 (1
  // KB); lane -> row 2 i + lane / 32, slot lane % 32 holding the row's
  // 16-byte segment (lane % 32) ^ (row % 16), so that the 16 rows' reads of
  // one segment hit distinct banks.  Instructions whose two rows are both
  // past the tile's tokens are not issued, and in a partly valid pair the
  // lanes of the row past them load nothing (the row stays zero).
  // (32-bit per-lane offsets from a wave-uniform base: the forward rejects
  // decode batches whose fp16 rows reach 4 GB)
  uint32_t adma_off[2] = {0u, 0u};
  bool adma_on[2] = {false, false};
  bool adma_row[2] = {false, false};  // this lane's row holds a token
  if (ADMA) {
    const int nvr = min(16, ne - m0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = wave + 4 * u, row = 2 * i + (lane >> 5);
      adma_on[u] = 2 * i < nvr;
      adma_row[u] = row < nvr;
      const int src = s_src[row < nvr ? row : 0];
      adma_off[u] = (uint32_t)src * (uint32_t)((K / KC) * ACB) + 16u * ((lane & 31) ^ (row & 15));
    }
  }
  auto issue_a = [&](int c, uint8_t* sbuf) __attribute__((always_inline)) {
    if (ADMA) {
      const uint8_t* base = sbase(static_cast<const uint8_t*>(a.act) + (size_t)c * ACB);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (adma_on[u] && adma_row[u])
          __builtin_amdgcn_global_load_lds(base + adma_off[u], sbuf + (wave + 4 * u) * 1024, 16, 0, 0);
    }
  };

  // activation staging role: row sr, segment ss (rows past the expert's
  // token count are not loaded; their MFMA columns are never stored)
  const int sr = tid >> 4, ss = tid & 15;
  const int ssrc = s_src[sr];
  const float sinv = 1.0f / s_rs[sr];
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const uint8_t* arow_p = act + (size_t)(ssrc >= 0 ? ssrc : 0) * ((size_t)(K / KC) * ACB) + ss * SEGB;
  const uint8_t* asf_p = SCALED ? a.act_sf + (size_t)(ssrc >= 0 ? ssrc : 0) * (K >> 5) : nullptr;
  uint4 av0 = {0u, 0u, 0u, 0u}, av1 = {0u, 0u, 0u, 0u};
  uint2 avs = {0u, 0u};
  auto load_act = [&](int c) __attribute__((always_inline)) {
    if (!ADMA && ssrc >= 0) {
      if (SEGB == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(arow_p + (size_t)c * ACB);
        av0 = uint4{v.x, v.y, 0u, 0u};
      } else {
        av0 = *reinterpret_cast<const uint4*>(arow_p + (size_t)c * ACB);
      }
      if (SEGB == 32) av1 = *reinterpret_cast<const uint4*>(arow_p + (size_t)c * ACB + 16);
      if (SCALED && ss == 0) avs = *reinterpret_cast<const uint2*>(asf_p + c * (KC / 32));
    }
  };

  // this lane's weight rows (workgroup-local)
  const int lrow0 = FC1 ? wave * 16 + r16 : wave * 32 + r16;
  const int lrow1 = FC1 ? 64 + wave * 16 + r16 : wave * 32 + 16 + r16;
  int obase = FC1 ? rb * 64 + wave * 16 : rb * 128 + wave * 32;

  // LDS byte offsets of this lane's operand reads within a buffer, computed
  // once (the empty asm makes them opaque, so the compiler keeps them in
  // registers and puts the buffer's own address in each read's offset field
  // instead of rebuilding every address each chunk)
  uint32_t lw[4] = {(uint32_t)(lrow0 * 128 + 16 * ((2 * q) ^ (lrow0 & 7))),
                    (uint32_t)(lrow0 * 128 + 16 * ((2 * q + 1) ^ (lrow0 & 7))),
                    (uint32_t)(lrow1 * 128 + 16 * ((2 * q) ^ (lrow1 & 7))),
                    (uint32_t)(lrow1 * 128 + 16 * ((2 * q + 1) ^ (lrow1 & 7)))};
  asm volatile("" : "+v"(lw[0]), "+v"(lw[1]), "+v"(lw[2]), "+v"(lw[3]));
  // activation reads: ADMA rows keep segment 8 q + jj of row r16 in slot
  // (8 q + jj) ^ r16; staged rows are plain (segment 8 q + jj at 16 jj past
  // 128 q)
  uint32_t la[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj)
    la[jj] = (uint32_t)(r16 * AROW + (ADMA ? 16 * ((8 * q + jj) ^ r16) : 128 * q + 16 * jj));
  if (ADMA)
    asm volatile("" : "+v"(la[0]), "+v"(la[1]), "+v"(la[2]), "+v"(la[3]), "+v"(la[4]), "+v"(la[5]), "+v"(la[6]),
                 "+v"(la[7]));
  else
    asm volatile("" : "+v"(la[0]));

  // the lane's weight-scale bytes of the current group, one entry per chunk
  // (group16: the 4 scales of K [64 q, 64 q + 64) for each of the two rows;
  // group32: the 2 scales of each row, row 0 in the low half).  Group16
  // chunks are unrolled over the group, so entry j is read by chunk j;
  // otherwise the entries are consumed from 0 and shifted down each chunk.
  constexpr int NSR = MODE == 0 ? 2 * SG : SG;
  uint32_t sreg[NSR];
#pragma unroll
  for (int i = 0; i < NSR; ++i) sreg[i] = 0;

  // prologue: group 0's scale lines, chunk 0's activations and weights
  issue_sc(0, 32 * wave, 32);
  load_act(0);
  issue_a(0, s_b0);
  issue_w(0, s_w0);

  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // one chunk: its weights (sw) and activations (sb, sbsf) were loaded
  // during the previous chunk; RING2 loads the next chunk into the other
  // buffers (sw_next).  JJ: integral_constant of the chunk's index in its
  // scale group g (group16), or -1 (index taken from c at run time)
  auto step = [&](auto JJ, int g, int c, const uint8_t* sw, uint8_t* sw_next, uint8_t* sb, uint8_t* sb_next,
                  uint8_t* sbsf) __attribute__((always_inline)) {
    constexpr int JS = decltype(JJ)::value;
    // stage chunk c's activations
    if (!ADMA && ssrc >= 0) {
      uint4 v0 = av0, v1 = av1;
      if (MODE == 0) {
        // bf16 x or h -> fp16 * 2**-p (exact: 8 significant bits, in range)
        uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const _Float16 lo = (_Float16)(bf16_to_f32(w[j] & 0xFFFFu) * sinv);
          const _Float16 hi = (_Float16)(bf16_to_f32(w[j] >> 16) * sinv);
          w[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        v0 = uint4{w[0], w[1], w[2], w[3]};
        v1 = uint4{w[4], w[5], w[6], w[7]};
      }
      uint8_t* d = sb + sr * AROW + ss * SEGB;
      if (SEGB == 8) *reinterpret_cast<uint2*>(d) = uint2{v0.x, v0.y};
      else *reinterpret_cast<uint4*>(d) = v0;
      if (SEGB == 32) *reinterpret_cast<uint4*>(d + 16) = v1;
      if (SCALED && ss == 0) *reinterpret_cast<uint2*>(sbsf + sr * 8) = avs;
    }
    // also waits for this chunk's weight and scale loads; every wave is past
    // the previous chunk, so the other buffers and the scale lines read at
    // the last group start may be refilled
    __syncthreads();

    const int j = JS >= 0 ? JS : c % SG;
    if (j == 0) {
      // a new scale group: this lane's scales of all its chunks
      const int x0 = 4 * sc_swz(lrow0), x1 = 4 * sc_swz(lrow1);
      const uint8_t* p0 = s_sc + lrow0 * 128;
      const uint8_t* p1 = s_sc + lrow1 * 128;
#pragma unroll
      for (int jj = 0; jj < SG; ++jj) {
        if (MODE == 0) {
          const int d = 4 * jj + q;
          sreg[2 * jj] = *reinterpret_cast<const uint32_t*>(p0 + 4 * (d ^ x0));
          sreg[2 * jj + 1] = *reinterpret_cast<const uint32_t*>(p1 + 4 * (d ^ x1));
        } else {
          const int d = 2 * jj + (q >> 1), h = 2 * (q & 1);
          sreg[jj] = (uint32_t)*reinterpret_cast<const uint16_t*>(p0 + 4 * (d ^ x0) + h) |
                     ((uint32_t)*reinterpret_cast<const uint16_t*>(p1 + 4 * (d ^ x1) + h) << 16);
        }
      }
    }
    uint32_t s0, s1;
    if constexpr (JS >= 0) {
      s0 = MODE == 0 ? sreg[2 * JS] : (sreg[JS] & 0xFFFFu);
      s1 = MODE == 0 ? sreg[2 * JS + 1] : (sreg[JS] >> 16);
    } else {
      s0 = MODE == 0 ? sreg[0] : (sreg[0] & 0xFFFFu);
      s1 = MODE == 0 ? sreg[1] : (sreg[0] >> 16);
      constexpr int SSH = MODE == 0 ? 2 : 1;
#pragma unroll
      for (int i = 0; i + SSH < NSR; ++i) sreg[i] = sreg[i + SSH];
    }

    // RING2: the next chunk's loads now.  The next group's scale lines
    // arrive a slice per chunk from the group's second chunk on (the group
    // start above has just read the buffer; every wave is past it one
    // barrier later), the last chunk of the group taking the last two slices.
    if (RING2) {
      if (c + 1 < nchunks) {
        load_act(c + 1);
        issue_a(c + 1, sb_next);
        issue_w(c + 1, sw_next);
      }
      if (g + 1 < ngroups && j > 0) {
        if (MODE == 0) {
          issue_sc_slice0(g + 1, j - 1);
          if (j == SG - 1) issue_sc_slice0(g + 1, SG - 1);
        } else {
          issue_sc_slice(g + 1, j - 1);
          if (j == SG - 1) issue_sc_slice(g + 1, SG - 1);
        }
      }
    }

    // this chunk's operands, then its MFMAs
    const uint4 w0a = *reinterpret_cast<const uint4*>(sw + lw[0]);
    const uint4 w0b = *reinterpret_cast<const uint4*>(sw + lw[1]);
    const uint4 w1a = *reinterpret_cast<const uint4*>(sw + lw[2]);
    const uint4 w1b = *reinterpret_cast<const uint4*>(sw + lw[3]);
    const uint8_t* brow = sb + r16 * AROW;
    uint4 bv[8];
    int sbb0 = 0, sbb1 = 0;
    if (SCALED) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (MODE == 3) {
          // FP4 operand: hardware block q of step st = memory block 2 q + st
          bv[2 * st] = *reinterpret_cast<const uint4*>(brow + 16 * (2 * q + st));
        } else {
          const int o = 64 * (q >> 1) + 32 * st + 16 * (q & 1);
          bv[2 * st] = *reinterpret_cast<const uint4*>(brow + o);
          bv[2 * st + 1] = *reinterpret_cast<const uint4*>(brow + 128 + o);
        }
      }
      const uint32_t sbb = *reinterpret_cast<const uint16_t*>(sbsf + r16 * 8 + 2 * q);
      sbb0 = (int)(sbb & 0xFFu);
      sbb1 = (int)(sbb >> 8);
    } else if (ADMA) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) bv[jj] = *reinterpret_cast<const uint4*>(sb + la[jj]);
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) bv[jj] = *reinterpret_cast<const uint4*>(sb + la[0] + 16 * jj);
    }
    if (!RING2) {
      __syncthreads();  // operands read: the buffers may be refilled
      if (c + 1 < nchunks) {
        load_act(c + 1);
        issue_w(c + 1, s_w0);
      }
      if (g + 1 < ngroups) {
        if (MODE == 0) issue_sc_slice0(g + 1, j);
        else issue_sc_slice(g + 1, j);
      }
    }
    if (SCALED) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint4& ca = st ? w0b : w0a;
        const uint4& cb = st ? w1b : w1a;
        const v8i B = MODE == 3 ? v8i{(int)bv[2 * st].x, (int)bv[2 * st].y, (int)bv[2 * st].z,
                                      (int)bv[2 * st].w, 0, 0, 0, 0}
                                : v8i{(int)bv[2 * st].x, (int)bv[2 * st].y, (int)bv[2 * st].z,
                                      (int)bv[2 * st].w, (int)bv[2 * st + 1].x, (int)bv[2 * st + 1].y,
                                      (int)bv[2 * st + 1].z, (int)bv[2 * st + 1].w};
        const v8i A0 = {(int)ca.x, (int)ca.y, (int)ca.z, (int)ca.w, 0, 0, 0, 0};
        const v8i A1 = {(int)cb.x, (int)cb.y, (int)cb.z, (int)cb.w, 0, 0, 0, 0};
        const int sa0 = (int)((s0 >> (8 * st)) & 0xFFu);
        const int sa1 = (int)((s1 >> (8 * st)) & 0xFFu);
        const int sbv = st ? sbb1 : sbb0;
        acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, B, acc0, 4, MODE == 3 ? 4 : 0, 0, sa0, 0,
                                                                sbv);
        acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, B, acc1, 4, MODE == 3 ? 4 : 0, 0, sa1, 0,
                                                                sbv);
      }
    } else if (MODE == 0) {
      // group16 scale of MFMA j: byte j / 2 of s0 / s1
      const v2h p0l = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s0, 1.0f, false);
      const v2h p0h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s0, 1.0f, true);
      const v2h p1l = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s1, 1.0f, false);
      const v2h p1h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s1, 1.0f, true);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const _Float16 h0 = jj < 2 ? p0l[0] : jj < 4 ? p0l[1] : jj < 6 ? p0h[0] : p0h[1];
        const _Float16 h1 = jj < 2 ? p1l[0] : jj < 4 ? p1l[1] : jj < 6 ? p1h[0] : p1h[1];
        const uint32_t c0 = jj < 4 ? dw(w0a, jj) : dw(w0b, jj - 4);
        const uint32_t c1 = jj < 4 ? dw(w1a, jj) : dw(w1b, jj - 4);
        const v8h B = __builtin_bit_cast(v8h, bv[jj]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(c0, v2h{h0, h0}), B, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(c1, v2h{h1, h1}), B, acc1, 0, 0, 0);
      }
    } else {
      // group32 scale of MFMA j: byte j / 4 of s0 / s1
      const float x0l = ue8m0_to_f32(s0 & 0xFFu), x0h = ue8m0_to_f32(s0 >> 8);
      const float x1l = ue8m0_to_f32(s1 & 0xFFu), x1h = ue8m0_to_f32(s1 >> 8);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint32_t c0 = jj < 4 ? dw(w0a, jj) : dw(w0b, jj - 4);
        const uint32_t c1 = jj < 4 ? dw(w1a, jj) : dw(w1b, jj - 4);
        const v8bf B = __builtin_bit_cast(v8bf, bv[jj]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(c0, jj < 4 ? x0l : x0h), B, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(c1, jj < 4 ? x1l : x1h), B, acc1, 0, 0, 0);
      }
    }
  };
  if constexpr (MODE == 0) {
    // group16: the chunks of a scale group unrolled (SG = 8, even, so a
    // chunk's RING2 buffer pair is fixed by its index in the group)
    for (int g = 0; g < ngroups; ++g) {
      unroll_for<SG>([&](auto J) __attribute__((always_inline)) {
        constexpr int jc = decltype(J)::value;
        const int c = g * SG + jc;
        if (c < nchunks) {
          if (RING2 && (jc & 1)) step(J, g, c, s_w1, s_w0, s_b1, s_b0, s_bsf1);
          else if (RING2) step(J, g, c, s_w0, s_w1, s_b0, s_b1, s_bsf0);
          else step(J, g, c, s_w0, s_w0, s_b0, s_b0, s_bsf0);
        }
      });
    }
  } else if (RING2) {
    constexpr std::integral_constant<int, -1> JR{};
    for (int c = 0; c < nchunks; c += 2) {
      step(JR, c / SG, c, s_w0, s_w1, s_b0, s_b1, s_bsf0);
      if (c + 1 < nchunks) step(JR, (c + 1) / SG, c + 1, s_w1, s_w0, s_b1, s_b0, s_bsf1);
    }
  } else {
    constexpr std::integral_constant<int, -1> JR{};
    for (int c = 0; c < nchunks; ++c) step(JR, c / SG, c, s_w0, s_w0, s_b0, s_b0, s_bsf0);
  }

  // epilogue: lane holds rows 4q..4q+3 of each 16-row tile, column r16
  const int m = m0 + r16;
  const bool valid = m < ne;
  const int slot = oe + m;
  const float cs = s_rs[r16] * (a.gs ? a.gs[e] : 1.0f);
  if (FC1) {
    float h[4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = swiglu(acc0[i] * cs, acc1[i] * cs);
      amax = fmaxf(amax, fabsf(h[i]));
    }
    if (SCALED) {
      // the 32-wide quantisation block spans this wave and its partner
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      if (q == 0) s_amax[wave][r16] = amax;
      __syncthreads();
      amax = fmaxf(s_amax[wave][r16], s_amax[wave ^ 1][r16]);
      int ex = amax > 0.0f ? (MODE == 3 ? ceil_log2_over_6(amax) : ceil_log2_over_448(amax)) : -127;
      ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
      const float inv = __builtin_ldexpf(1.0f, -ex);
      if (valid) {
        if (MODE == 3) {
          // E2M1 RNE (hardware conversion, unit scale), two per byte
          uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, h[0] * inv, h[1] * inv, 1.0f, 0);
          d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, h[2] * inv, h[3] * inv, 1.0f, 1);
          uint8_t* hrow = static_cast<uint8_t*>(a.h_out) + (size_t)slot * (a.I >> 1);
          *reinterpret_cast<uint16_t*>(hrow + ((obase + 4 * q) >> 1)) = (uint16_t)d;
        } else {
          uint32_t wv = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) wv |= f32_to_e4m3_rne(h[i] * inv) << (8 * i);
          uint8_t* hrow = static_cast<uint8_t*>(a.h_out) + (size_t)slot * a.I;
          *reinterpret_cast<uint32_t*>(hrow + obase + 4 * q) = wv;
        }
        if (q == 0 && (wave & 1) == 0)
          a.h_sf_out[(size_t)slot * (a.I >> 5) + (obase >> 5)] = (uint8_t)(ex + 127);
      }
    } else {
      uint32_t hb[4];
      uint32_t hmax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = f32_to_bf16_rne(h[i]);
        const uint32_t mag = (hb[i] & 0x7FFFu) << 16;
        hmax = mag > hmax ? mag : hmax;
      }
      if (valid) {
        uint16_t* hp = static_cast<uint16_t*>(a.h_out) + (size_t)slot * a.I + obase + 4 * q;
        *reinterpret_cast<uint2*>(hp) = uint2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
      }
      if (MODE == 0) {
        uint32_t o = __shfl_xor(hmax, 16, 64);
        hmax = o > hmax ? o : hmax;
        o = __shfl_xor(hmax, 32, 64);
        hmax = o > hmax ? o : hmax;
        if (valid && q == 0 && hmax) atomicMax(a.hmax_out + slot, hmax);
      }
    }
  } else if (valid) {
    float* y = a.y_out + (size_t)slot * a.H + obase + 4 * q;
    *reinterpret_cast<float4*>(y) = float4{acc0[0] * cs, acc0[1] * cs, acc0[2] * cs, acc0[3] * cs};
    *reinterpret_cast<float4*>(y + 16) = float4{acc1[0] * cs, acc1[1] * cs, acc1[2] * cs, acc1[3] * cs};
  }
}

// The LDS arrays of an item (AROWV: the staged activation row stride the
// items use; RING: the paired buffers).
#define DECODE_LDS(AROWV, RING)                                                   \
  constexpr int NB1_ = (RING) ? 1 : 0;                                            \
  __shared__ __attribute__((aligned(16))) uint8_t s_w0[WR * 128];                 \
  __shared__ __attribute__((aligned(16))) uint8_t s_w1[NB1_ * WR * 128 + 16];     \
  __shared__ __attribute__((aligned(16))) uint8_t s_sc[WR * 128];                 \
  __shared__ __attribute__((aligned(16))) uint8_t s_b0[16 * (AROWV)];             \
  __shared__ __attribute__((aligned(16))) uint8_t s_b1[NB1_ * 16 * (AROWV) + 16]; \
  __shared__ __attribute__((aligned(16))) uint8_t s_bsf0[16 * 8];                 \
  __shared__ __attribute__((aligned(16))) uint8_t s_bsf1[NB1_ * 16 * 8 + 16];     \
  __shared__ int s_src[16];                                                       \
  __shared__ float s_rs[16];                                                      \
  __shared__ float s_amax[4][16]
#define DECODE_LDS_ARGS s_w0, s_w1, s_sc, s_b0, s_b1, s_bsf0, s_bsf1, s_src, s_rs, s_amax

// activation bytes per row per chunk, and the staged row stride of an item
template <int MODE>
constexpr int decode_acb() { return MODE == 3 ? KC / 2 : MODE == 2 ? KC : 2 * KC; }
template <int MODE, bool FC1>
constexpr int decode_arow() { return decode_acb<MODE>() + ((MODE == 0 && FC1) ? 0 : 16); }

// RING2: chunk buffers in pairs, so the next chunk's loads are issued right
// after the chunk's barrier (two workgroups per CU, one barrier per chunk);
// otherwise one set of buffers, refilled after a second barrier once every
// wave has read its operands (three workgroups per CU).  Measured per kernel
// on the decode16 geometry: the pair wins only where the MFMA phase is
// longest (group16 FC1, 512 vs 545 us); elsewhere the extra workgroup per
// CU wins (e.g. group16 FC2 268 vs 277 us, FP8 FC1 471 vs 486 us).
template <int MODE, bool FC1>
__global__ __launch_bounds__(256, (MODE == 0 && FC1) ? 2 : 3) void fc_decode_kernel(FcArgs a) {
  DECODE_LDS((decode_arow<MODE, FC1>()), MODE == 0 && FC1);
  const int tile = blockIdx.y;
  if (tile >= a.ntiles[0]) return;
  decode_item<MODE, FC1>(a, tile, blockIdx.x, DECODE_LDS_ARGS);
}

// The XCD (accelerator complex die) this wave runs on.
__device__ __forceinline__ int xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & 0xFu);
}

// Longest wait of an FC2 item for its tile's FC1 items, in ticks of the
// 100 MHz real-time counter (50 ms, far beyond any real wait).
constexpr uint64_t kMaxWaitTicks = 5000000;

// Single-launch decode: FC1 items, then FC2 items, of the tiles of this
// workgroup's XCD (see DecodeSync).  Within an XCD the L2 is shared and the
// vector L1 is per CU and write-through, so a store is visible to the other
// CUs of the XCD once it has completed; the FC2 side invalidates its L1
// before reading h.  No agent-scope release is needed (it would write back
// the whole L2).
template <int MODE>
__global__ __launch_bounds__(256, 2) void fc_decode_fused_kernel(FcArgs a1, FcArgs a2, DecodeSync y) {
  // (one set of arrays for both item kinds: FC1's pairs, the wider row stride)
  DECODE_LDS((decode_arow<MODE, false>()), MODE == 0);
  __shared__ int s_item;
  // Every branch and loop bound below is wave-uniform (scalar), and the
  // claim, the release and the wait are done by all of wave 0: with a
  // per-lane condition (thread 0 only) around them, the compiler may route
  // the other lanes straight back to the loop's barriers, past the claim,
  // and the waves then no longer pass through the items together.
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int x = xcc_id() % y.nx;
  const int ntiles = __builtin_amdgcn_readfirstlane(a1.ntiles[0]);
  const int ntx = ntiles > x ? (ntiles - x + y.nx - 1) / y.nx : 0;
  const int n1 = ntx * y.nblk1, n = n1 + ntx * y.nblk2;
  // Items are claimed one ahead: the next claim's round trip runs under the
  // current item.  A workgroup's next item always comes later in the queue
  // than its current one, so an FC1 item held as a next item belongs to a
  // workgroup whose current item is an FC1 item too (which never waits):
  // every wait ends.
  auto claim = [&]() __attribute__((always_inline)) {
    // one atomic for the wave (lane 0 adds 1), the old value in every lane
    return __hip_atomic_fetch_add(y.queue + x, lane == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (wave == 0) s_item = __builtin_amdgcn_readfirstlane(claim());
  __syncthreads();
  int it = __builtin_amdgcn_readfirstlane(s_item);
  for (;;) {
    __syncthreads();  // (every wave has read s_item)
    if (it >= n) break;
    int next = 0;
    if (wave == 0) next = claim();
    if (it < n1) {
      const int lt = it / y.nblk1;
      const int t = lt * y.nx + x;
      decode_item<MODE, true>(a1, t, it - lt * y.nblk1, DECODE_LDS_ARGS);
      // this wave's stores of h (and of its maxima) have completed
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (wave == 0)
        __hip_atomic_fetch_add(y.done + t, lane == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const int j = it - n1, lt = j / y.nblk2;
      const int t = lt * y.nx + x;
      if (wave == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
          const int d = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(y.done + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          if (d >= y.nblk1) break;
          if (__builtin_amdgcn_s_memrealtime() - t0 > kMaxWaitTicks) {
            __hip_atomic_fetch_add(y.err, lane == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      __syncthreads();
      // lines of h this CU's L1 may hold from before the wait
      asm volatile("buffer_inv sc0" ::: "memory");
      decode_item<MODE, false>(a2, t, j - lt * y.nblk2, DECODE_LDS_ARGS);
    }
    __syncthreads();  // (every wave is past the item: s_item may be rewritten)
    if (wave == 0) s_item = __builtin_amdgcn_readfirstlane(next);
    __syncthreads();
    it = __builtin_amdgcn_readfirstlane(s_item);
  }
}

template <int MODE>
hipError_t launch_fused(const FcArgs& a1, const FcArgs& a2, const DecodeSync& y, hipStream_t s) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  // two workgroups per CU, every one resident at once (three would not fit
  // the registers of both item kinds without spilling)
  const int grid = cus * 2;
  hipLaunchKernelGGL((fc_decode_fused_kernel<MODE>), dim3(grid), dim3(256), 0, s, a1, a2, y);
  return hipGetLastError();
}

template <int MODE, bool FC1>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int nblk = FC1 ? a.I / 64 : a.H / 128;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  // x = weight-row block (fast), y = expert tile: concurrently resident
  // workgroups stream whole experts
  hipLaunchKernelGGL((fc_decode_kernel<MODE, FC1>), dim3(nblk, max_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc_decode(const FcArgs& a, int mode, bool fc1, int max_tiles, hipStream_t s) {
  if (fc1) {
    if (mode == 0) return launch_one<0, true>(a, max_tiles, s);
    if (mode == 1) return launch_one<1, true>(a, max_tiles, s);
    if (mode == 2) return launch_one<2, true>(a, max_tiles, s);
    return launch_one<3, true>(a, max_tiles, s);
  }
  if (mode == 0) return launch_one<0, false>(a, max_tiles, s);
  if (mode == 1) return launch_one<1, false>(a, max_tiles, s);
  if (mode == 2) return launch_one<2, false>(a, max_tiles, s);
  return launch_one<3, false>(a, max_tiles, s);
}

int xcd_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 32)
    return 1;
  return cus / 32 > 8 ? 8 : cus / 32;
}

hipError_t launch_fc_decode_fused(const FcArgs& a1, const FcArgs& a2, int mode, const DecodeSync& y,
                                  hipStream_t s) {
  if (mode == 0) return launch_fused<0>(a1, a2, y, s);
  if (mode == 1) return launch_fused<1>(a1, a2, y, s);
  if (mode == 2) return launch_fused<2>(a1, a2, y, s);
  return launch_fused<3>(a1, a2, y, s);
}

}  // namespace moefp4
