// Decode-shaped grouped GEMMs (at most 16 activation rows per expert tile):
// FC1 + SwiGLU (+ h quantisation) and FC2, for all three operand formats
//   MODE 0  bf16 activations, group16 E4M3 weights   -> fp16 MFMA
//   MODE 1  bf16 activations, group32 UE8M0 weights  -> bf16 MFMA
//   MODE 2  FP8 + UE8M0 activations, group32 weights -> block-scaled MFMA
// (the W4A16 forms of b12x moe/fused/w4a16/prepare.py and the FP8xFP4
// recipe (1, 1, 32) of the GLM-5.2 NVFP4 group16 MegaMoE notes, Context).
//
// Decode is a weight stream: each FP4 weight byte is read once and used by
// a handful of tokens.  The kernel is built to keep HBM busy:
//  * one workgroup = 4 independent wavefronts over 64 (FC1: 16 gate + 16 up
//    rows each) or 128 (FC2: 32 rows each) weight rows of one expert tile;
//  * the K loop runs in 512-element chunks; the next chunk's codes and scales
//    (64 contiguous bytes per lane per 16-row tile) are loaded into registers
//    while the current chunk is multiplied;
//  * the activation chunk of the tile (16 rows) is double-buffered in LDS --
//    each thread stages one 64-byte (32-byte for FP8) segment, one barrier
//    per chunk -- so the waves share it instead of each re-reading it;
//  * rows of the tile past the expert's token count are zero and never read.
// K index permutation inside a chunk (identical for both MFMA operands):
//  16-bit MFMA: MFMA j = 0..15 of lane group q takes chunk elements
//    [128 (j / 4) + 32 q + 8 (j % 4), + 8) -- so that the 4 lanes of a row read
//    64 contiguous code bytes per load instruction;
//  scaled MFMA: K-step st = 0..3 covers [128 st, 128 st + 128) in the
//    measured FP4 / FP8 lane layouts (see common.h).
#include "common.h"
#include "kernels.h"

namespace moefp4 {

namespace {

constexpr int KC = 512;

template <int MODE>
struct Frag {
  uint4 c[4];  // 64 code bytes: piece i = 16 bytes at row offset 16 q + 64 i of the chunk
  uint4 s;     // MODE 1/2: the chunk's 16 UE8M0 bytes (MODE 0 scales are staged in LDS)
};

// Codes: the 4 lanes of a row read 64 contiguous bytes per load instruction
// (cached loads: the next instruction reads the other half of the same
// 128-byte lines); piece i of lane group q holds chunk elements
// [128 i + 32 q, + 32).
template <int MODE>
__device__ __forceinline__ void load_frag(Frag<MODE>& f, const uint8_t* rc, const uint8_t* rs,
                                          int k0, int q) {
  const uint8_t* p = rc + (k0 >> 1) + 16 * q;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.c[i] = *reinterpret_cast<const uint4*>(p + 64 * i);
  if (MODE != 0) f.s = *reinterpret_cast<const uint4*>(rs + (k0 >> 5));
}

__device__ __forceinline__ uint32_t dw(const uint4& v, int r) {
  return r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w;
}

// E4M3 (fn) RNE encode of |y| <= 448, sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float y) {
  const uint32_t u = f2u(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t ua = u & 0x7FFFFFFFu;
  uint32_t code;
  if (ua >= 0x3C800000u) {
    const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    code = (uint32_t)__builtin_rintf(u2f(ua) * 512.0f);
  }
  return sign | code;
}

template <int MODE, bool FC1>
__global__ __launch_bounds__(256) void fc_skinny_kernel(FcArgs a) {
  constexpr int ESZ = MODE == 2 ? 1 : 2;          // activation element bytes
  constexpr int ROWB = KC * ESZ + 16;             // staged row stride (bytes)
  constexpr int SEGB = KC * ESZ / 16;             // bytes staged per thread
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2][16 * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t s_bsf[2][16 * 16];
  __shared__ int s_src[16];
  __shared__ float s_rs[16];
  __shared__ float s_amax[4][16];
  // MODE 0: the workgroup's 128 rows x 32 group16 scale bytes of a chunk
  __shared__ __attribute__((aligned(16))) uint8_t s_sc[2][MODE == 0 ? 128 * 32 : 16];

  const int tile = blockIdx.x;
  if (tile >= a.ntiles[0]) return;
  const int e = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const int ne = a.counts[e], oe = a.offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;

  int obase, row0, row1;
  if (FC1) {
    obase = blockIdx.y * 64 + wave * 16;
    row0 = a.w13_order == 0 ? obase + r16 : a.I + obase + r16;  // gate
    row1 = a.w13_order == 0 ? a.I + obase + r16 : obase + r16;  // up
  } else {
    obase = blockIdx.y * 128 + wave * 32;
    row0 = obase + r16;
    row1 = obase + 16 + r16;
  }
  const size_t rb = (size_t)(K >> 1), sb = (size_t)(K / (MODE == 0 ? 16 : 32));
  const uint8_t* wc0 = a.w + ((size_t)e * N + row0) * rb;
  const uint8_t* wc1 = a.w + ((size_t)e * N + row1) * rb;
  const uint8_t* ws0 = a.wsf + ((size_t)e * N + row0) * sb;
  const uint8_t* ws1 = a.wsf + ((size_t)e * N + row1) * sb;

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
          const uint32_t hm = a.hmax_in[slot];
          sc = __builtin_ldexpf(1.0f, hm ? (int)(hm >> 23) - 127 - 14 : 0);
        }
      }
    }
    s_src[tid] = src;
    s_rs[tid] = sc;
  }
  __syncthreads();

  // staging role: row sr, segment ss
  const int sr = tid >> 4, ss = tid & 15;
  const int ssrc = s_src[sr];
  const float sinv = 1.0f / s_rs[sr];
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const size_t arow = (size_t)K * ESZ;

  // Activation staging.  Rows of the tile past the expert's token count load
  // row 0 instead (no lane-divergent branch around the loads): their MFMA
  // output columns are never stored.
  const uint8_t* arow_p = act + (size_t)(ssrc >= 0 ? ssrc : 0) * arow + ss * SEGB;
  const uint8_t* asf_p =
      MODE == 2 ? a.act_sf + (size_t)(ssrc >= 0 ? ssrc : 0) * (K >> 5) : nullptr;
  // MODE 0 scale staging: thread t stages 16 of the 32 scale bytes of WG-local
  // row t / 2 (FC1: local rows 0..63 gate, 64..127 up; FC2: 128 consecutive)
  const uint8_t* sc_p = nullptr;
  if (MODE == 0) {
    const int lr = tid >> 1;
    int grow;
    if (FC1) {
      const int i0 = blockIdx.y * 64 + (lr & 63);
      const bool up = lr >= 64;
      grow = (up != (a.w13_order != 0)) ? a.I + i0 : i0;
    } else {
      grow = blockIdx.y * 128 + lr;
    }
    sc_p = a.wsf + ((size_t)e * N + grow) * (size_t)(K >> 4) + 16 * (tid & 1);
  }
  // WG-local rows of this lane's two tiles (for reading the staged scales)
  const int lrow0 = FC1 ? wave * 16 + r16 : wave * 32 + r16;
  const int lrow1 = FC1 ? 64 + wave * 16 + r16 : wave * 32 + 16 + r16;
  // vs: MODE 2 the row's 16 UE8M0 activation scales of the chunk; MODE 0 the
  // 16 weight-scale bytes this thread stages
  auto load_b = [&](int k0, uint4 (&v)[4], uint4& vs) {
    const uint8_t* p = arow_p + (size_t)k0 * ESZ;
#pragma unroll
    for (int i = 0; i < SEGB / 16; ++i) v[i] = *reinterpret_cast<const uint4*>(p + 16 * i);
    if (MODE == 2) vs = *reinterpret_cast<const uint4*>(asf_p + (k0 >> 5));
    if (MODE == 0) vs = *reinterpret_cast<const uint4*>(sc_p + (k0 >> 4));
  };
  auto store_b = [&](int buf, uint4 (&v)[4], const uint4& vs) {
    if (MODE == 0 && !FC1) {
      // bf16 h -> fp16 * 2**-p (exact: 8 significant bits, in range)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const _Float16 lo = (_Float16)(bf16_to_f32(w[j] & 0xFFFFu) * sinv);
          const _Float16 hi = (_Float16)(bf16_to_f32(w[j] >> 16) * sinv);
          w[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        v[i] = uint4{w[0], w[1], w[2], w[3]};
      }
    }
    uint8_t* d = s_b[buf] + sr * ROWB + ss * SEGB;
#pragma unroll
    for (int i = 0; i < SEGB / 16; ++i) *reinterpret_cast<uint4*>(d + 16 * i) = v[i];
    if (MODE == 2 && ss == 0) *reinterpret_cast<uint4*>(s_bsf[buf] + sr * 16) = vs;
    if (MODE == 0) *reinterpret_cast<uint4*>(s_sc[buf] + 16 * tid) = vs;
  };

  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Frag<MODE>& g0, const Frag<MODE>& g1, int cur) {
    const uint8_t* brow = s_b[cur] + r16 * ROWB;
    if (MODE == 2) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(brow + 128 * st + 16 * q);
        const uint4 b1 = *reinterpret_cast<const uint4*>(brow + 128 * st + 64 + 16 * q);
        const v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                       (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        const int sbb = s_bsf[cur][r16 * 16 + 4 * st + q];
        const int sa0 = (int)((dw(g0.s, st) >> (8 * q)) & 0xFFu);
        const int sa1 = (int)((dw(g1.s, st) >> (8 * q)) & 0xFFu);
        const v8i A0 = {(int)g0.c[st].x, (int)g0.c[st].y, (int)g0.c[st].z, (int)g0.c[st].w, 0, 0, 0, 0};
        const v8i A1 = {(int)g1.c[st].x, (int)g1.c[st].y, (int)g1.c[st].z, (int)g1.c[st].w, 0, 0, 0, 0};
        acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, B, acc0, 4, 0, 0, sa0, 0, sbb);
        acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, B, acc1, 4, 0, 0, sa1, 0, sbb);
      }
    } else {
      // MODE 0: piece i of lane group q uses the group16 scales 8 i + 2 q, + 1
      const uint8_t* sc0 = s_sc[cur] + lrow0 * 32 + 2 * q;
      const uint8_t* sc1 = s_sc[cur] + lrow1 * 32 + 2 * q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v2h sp0, sp1;
        if (MODE == 0) {
          sp0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
              *reinterpret_cast<const uint16_t*>(sc0 + 8 * i), 1.0f, false);
          sp1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
              *reinterpret_cast<const uint16_t*>(sc1 + 8 * i), 1.0f, false);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint4 braw =
              *reinterpret_cast<const uint4*>(brow + (128 * i + 32 * q + 8 * jj) * 2);
          const uint32_t c0 = dw(g0.c[i], jj), c1 = dw(g1.c[i], jj);
          if (MODE == 0) {
            const v2h s0 = jj < 2 ? v2h{sp0[0], sp0[0]} : v2h{sp0[1], sp0[1]};
            const v2h s1 = jj < 2 ? v2h{sp1[0], sp1[0]} : v2h{sp1[1], sp1[1]};
            const v8h A0 = dq8_f16(c0, s0);
            const v8h A1 = dq8_f16(c1, s1);
            const v8h B = __builtin_bit_cast(v8h, braw);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B, acc1, 0, 0, 0);
          } else {
            const v8bf A0 = dq8_bf16(c0, ue8m0_to_f32((dw(g0.s, i) >> (8 * q)) & 0xFFu));
            const v8bf A1 = dq8_bf16(c1, ue8m0_to_f32((dw(g1.s, i) >> (8 * q)) & 0xFFu));
            const v8bf B = __builtin_bit_cast(v8bf, braw);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc1, 0, 0, 0);
          }
        }
      }
    }
  };

  // one chunk ahead: the next chunk's weights and activations are loaded
  // into registers while the current chunk (in LDS) is multiplied
  Frag<MODE> f0, f1, g0, g1;
  uint4 bv[4];
  uint4 bvs = {0u, 0u, 0u, 0u};
  load_b(0, bv, bvs);
  load_frag<MODE>(f0, wc0, ws0, 0, q);
  load_frag<MODE>(f1, wc1, ws1, 0, q);
  store_b(0, bv, bvs);
  __syncthreads();
  const int nchunks = K / KC;
  for (int c = 0; c < nchunks; ++c) {
    const int cur = c & 1;
    const bool more = c + 1 < nchunks;
    g0 = f0;
    g1 = f1;
    if (more) {
      load_b((c + 1) * KC, bv, bvs);
      load_frag<MODE>(f0, wc0, ws0, (c + 1) * KC, q);
      load_frag<MODE>(f1, wc1, ws1, (c + 1) * KC, q);
    }
    compute(g0, g1, cur);
    if (more) store_b(cur ^ 1, bv, bvs);
    __syncthreads();
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
    if (MODE == 2) {
      // the 32-wide quantisation block spans this wave and its partner
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      if (q == 0) s_amax[wave][r16] = amax;
      __syncthreads();
      amax = fmaxf(s_amax[wave][r16], s_amax[wave ^ 1][r16]);
      int ex = amax > 0.0f ? ceil_log2_over_448(amax) : -127;
      ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
      const float inv = __builtin_ldexpf(1.0f, -ex);
      if (valid) {
        uint32_t wv = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) wv |= f32_to_e4m3_rne(h[i] * inv) << (8 * i);
        uint8_t* hrow = static_cast<uint8_t*>(a.h_out) + (size_t)slot * a.I;
        *reinterpret_cast<uint32_t*>(hrow + obase + 4 * q) = wv;
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

template <int MODE, bool FC1>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int nblk = FC1 ? a.I / 64 : a.H / 128;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((fc_skinny_kernel<MODE, FC1>), dim3(max_tiles, nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc_skinny(const FcArgs& a, int mode, bool fc1, int max_tiles, hipStream_t s) {
  if (fc1) {
    if (mode == 0) return launch_one<0, true>(a, max_tiles, s);
    if (mode == 1) return launch_one<1, true>(a, max_tiles, s);
    return launch_one<2, true>(a, max_tiles, s);
  }
  if (mode == 0) return launch_one<0, false>(a, max_tiles, s);
  if (mode == 1) return launch_one<1, false>(a, max_tiles, s);
  return launch_one<2, false>(a, max_tiles, s);
}

}  // namespace moefp4
