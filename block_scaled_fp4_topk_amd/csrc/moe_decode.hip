// Decode-shaped grouped GEMMs, occupancy-driven form: FC1 + SwiGLU (+ h
// quantisation) and FC2 for tiles of at most 16 activation rows per expert.
//   MODE 0  bf16 activations, group16 E4M3 weights   -> fp16 MFMA
//   MODE 1  bf16 activations, group32 UE8M0 weights  -> bf16 MFMA
//   MODE 2  FP8 + UE8M0 activations, group32 weights -> block-scaled MFMA
// (the W4A16 forms of b12x moe/fused/w4a16/prepare.py and the FP8xFP4
// recipe (1, 1, 32) of the GLM-5.2 NVFP4 group16 MegaMoE notes, Context).
//
// Decode is a weight stream.  This kernel keeps HBM busy by residency rather
// than by software pipelining: each wave holds only one 256-element K chunk
// (32 code bytes per lane per 16-row tile) and few registers, so 8 waves
// per SIMD are resident and the memory latency of one wave is covered by
// the others.  Per chunk: every thread issues its share of the activation
// tile (16 rows, staged once in LDS for the 4 waves) and its weight loads,
// one barrier, the MFMAs, one barrier.
//
// Load shapes: the 4 lanes of a weight row read 64 contiguous bytes per
// instruction and two instructions cover the row's 128-byte chunk (cached
// loads, so the second hits the line the first brought in).  Rows of a tile
// past the expert's token count read activation row 0 (their MFMA columns
// are never stored).
// K index permutation inside a chunk (identical for both MFMA operands):
//  16-bit MFMA j = 0..7 of lane group q takes chunk elements
//    [128 (j / 4) + 32 q + 8 (j % 4), + 8);
//  scaled MFMA step st = 0, 1 covers [128 st, 128 st + 128) in the measured
//    FP4 / FP8 lane layouts (see common.h).
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace moefp4 {

namespace {

constexpr int KC = 256;
// chunks per weight-scale staging group: one full 128-byte line of a row's
// scales at a time (group16: 16 B per row per chunk -> 8 chunks; group32:
// 8 B -> 16 chunks); half-line groups measured 3-12% slower

__device__ __forceinline__ uint32_t dw(const uint4& v, int r) {
  return r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w;
}


template <int MODE, bool FC1>
__global__ __launch_bounds__(256, 8) void fc_decode_kernel(FcArgs a) {
  constexpr int ESZ = MODE == 2 ? 1 : 2;          // activation element bytes
  constexpr int ROWB = KC * ESZ + 16;             // staged row stride (bytes)
  constexpr int SEGB = KC * ESZ / 16;             // bytes staged per thread (32 or 16)
  constexpr int SCB = MODE == 0 ? KC / 16 : KC / 32;  // weight-scale bytes per row per chunk
  constexpr int SG = MODE == 0 ? 8 : 16;
  constexpr int SCROW = SG * SCB + (MODE == 0 ? 16 : 8);  // staged scale row stride (bytes)
  using ScPiece = typename std::conditional<MODE == 0, uint4, uint2>::type;
  __shared__ __attribute__((aligned(16))) uint8_t s_b[16 * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t s_bsf[16 * 8];
  // weight scales of 4 chunks for the workgroup's 128 rows (padded rows)
  __shared__ __attribute__((aligned(16))) uint8_t s_sc[128 * SCROW];
  __shared__ int s_src[16];
  __shared__ float s_rs[16];
  __shared__ float s_amax[4][16];

  const int tile = blockIdx.y;
  if (tile >= a.ntiles[0]) return;
  const int e = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const int ne = a.counts[e], oe = a.offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;

  int obase, row0, row1;
  if (FC1) {
    obase = blockIdx.x * 64 + wave * 16;
    row0 = a.w13_order == 0 ? obase + r16 : a.I + obase + r16;  // gate
    row1 = a.w13_order == 0 ? a.I + obase + r16 : obase + r16;  // up
  } else {
    obase = blockIdx.x * 128 + wave * 32;
    row0 = obase + r16;
    row1 = obase + 16 + r16;
  }
  const size_t rb = (size_t)(K >> 1), sb = (size_t)(K / (MODE == 0 ? 16 : 32));
  const uint8_t* wc0 = a.w + ((size_t)e * N + row0) * rb + 16 * q;
  const uint8_t* wc1 = a.w + ((size_t)e * N + row1) * rb + 16 * q;

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

  // staging role: row sr, segment ss.  Rows past the expert's token count are
  // not loaded: their LDS contents only reach MFMA output columns that are
  // never stored.
  const int sr = tid >> 4, ss = tid & 15;
  const int ssrc = s_src[sr];
  const float sinv = 1.0f / s_rs[sr];
  const uint8_t* act = static_cast<const uint8_t*>(a.act);
  const uint8_t* arow_p = act + (size_t)(ssrc >= 0 ? ssrc : 0) * ((size_t)K * ESZ) + ss * SEGB;
  const uint8_t* asf_p = MODE == 2 ? a.act_sf + (size_t)(ssrc >= 0 ? ssrc : 0) * (K >> 5) : nullptr;

  // Weight-scale staging: once per group of SG chunks the workgroup's 128
  // rows x SG chunks of scale bytes go to LDS.  Thread t loads the chunk
  // (t % SG) piece of WG-local rows t / SG + (256 / SG) h, h < SG / 2, so the
  // SG threads of a row read its SG * SCB contiguous bytes.  WG-local rows:
  // FC1 0..63 gate and 64..127 up of the 64 outputs; FC2 128 consecutive rows.
  constexpr int NH = SG / 2;  // rows staged per thread
  const int sq = tid % SG, slr = tid / SG;
  const uint8_t* sc_src[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int lr = slr + (256 / SG) * h;
    int grow;
    if (FC1) {
      const int i0 = blockIdx.x * 64 + (lr & 63);
      grow = ((lr >= 64) != (a.w13_order != 0)) ? a.I + i0 : i0;
    } else {
      grow = blockIdx.x * 128 + lr;
    }
    sc_src[h] = a.wsf + ((size_t)e * N + grow) * sb + sq * SCB;
  }
  // this lane's rows in the staged scales
  const int lrow0 = FC1 ? wave * 16 + r16 : wave * 32 + r16;
  const int lrow1 = FC1 ? 64 + wave * 16 + r16 : wave * 32 + 16 + r16;

  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int nchunks = K / KC;
  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * KC;
    // activation segment of this thread
    uint4 bv0 = {0u, 0u, 0u, 0u}, bv1 = {0u, 0u, 0u, 0u};
    uint2 bsf = {0u, 0u};
    if (ssrc >= 0) {
      bv0 = *reinterpret_cast<const uint4*>(arow_p + (size_t)k0 * ESZ);
      if (SEGB == 32) bv1 = *reinterpret_cast<const uint4*>(arow_p + (size_t)k0 * ESZ + 16);
      if (MODE == 2) bsf = *reinterpret_cast<const uint2*>(asf_p + (k0 >> 5));
    }
    // weight scales of the next 4 chunks
    const bool sgroup = (c % SG) == 0;
    ScPiece sp[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) sp[h] = ScPiece{};
    if (sgroup && c + sq < nchunks) {
      const size_t off = (size_t)(k0 / KC) * SCB;
#pragma unroll
      for (int h = 0; h < NH; ++h) sp[h] = *reinterpret_cast<const ScPiece*>(sc_src[h] + off);
    }
    // weights: pieces i = 0, 1 of 16 bytes at row offset 16 q + 64 i
    const uint4 c00 = *reinterpret_cast<const uint4*>(wc0 + (k0 >> 1));
    const uint4 c01 = *reinterpret_cast<const uint4*>(wc0 + (k0 >> 1) + 64);
    const uint4 c10 = *reinterpret_cast<const uint4*>(wc1 + (k0 >> 1));
    const uint4 c11 = *reinterpret_cast<const uint4*>(wc1 + (k0 >> 1) + 64);
    if (MODE == 0) {
      // bf16 x or h -> fp16 * 2**-p (exact: 8 significant bits, in range)
      uint32_t w[8] = {bv0.x, bv0.y, bv0.z, bv0.w, bv1.x, bv1.y, bv1.z, bv1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const _Float16 lo = (_Float16)(bf16_to_f32(w[j] & 0xFFFFu) * sinv);
        const _Float16 hi = (_Float16)(bf16_to_f32(w[j] >> 16) * sinv);
        w[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      bv0 = uint4{w[0], w[1], w[2], w[3]};
      bv1 = uint4{w[4], w[5], w[6], w[7]};
    }
    uint8_t* d = s_b + sr * ROWB + ss * SEGB;
    *reinterpret_cast<uint4*>(d) = bv0;
    if (SEGB == 32) *reinterpret_cast<uint4*>(d + 16) = bv1;
    if (MODE == 2 && ss == 0) *reinterpret_cast<uint2*>(s_bsf + sr * 8) = bsf;
    if (sgroup) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
        *reinterpret_cast<ScPiece*>(s_sc + (slr + (256 / SG) * h) * SCROW + sq * SCB) = sp[h];
    }
    __syncthreads();

    // scales of the two pieces of the two tiles
    uint32_t s0a, s0b, s1a, s1b;
    {
      const uint8_t* p0 = s_sc + lrow0 * SCROW + (c % SG) * SCB;
      const uint8_t* p1 = s_sc + lrow1 * SCROW + (c % SG) * SCB;
      if (MODE == 0) {
        // piece i needs the group16 scales 8 i + 2 q and + 1
        s0a = *reinterpret_cast<const uint16_t*>(p0 + 2 * q);
        s0b = *reinterpret_cast<const uint16_t*>(p0 + 8 + 2 * q);
        s1a = *reinterpret_cast<const uint16_t*>(p1 + 2 * q);
        s1b = *reinterpret_cast<const uint16_t*>(p1 + 8 + 2 * q);
      } else {
        // the chunk's 8 UE8M0 bytes (piece / step i uses byte 4 i + q)
        const uint2 v0 = *reinterpret_cast<const uint2*>(p0);
        const uint2 v1 = *reinterpret_cast<const uint2*>(p1);
        s0a = v0.x; s0b = v0.y; s1a = v1.x; s1b = v1.y;
      }
    }

    const uint8_t* brow = s_b + r16 * ROWB;
    if (MODE == 2) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint4 b0 = *reinterpret_cast<const uint4*>(brow + 128 * st + 16 * q);
        const uint4 b1 = *reinterpret_cast<const uint4*>(brow + 128 * st + 64 + 16 * q);
        const v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        const int sbb = s_bsf[r16 * 8 + 4 * st + q];
        const uint4& ca = st ? c01 : c00;
        const uint4& cb = st ? c11 : c10;
        const int sa0 = (int)(((st ? s0b : s0a) >> (8 * q)) & 0xFFu);
        const int sa1 = (int)(((st ? s1b : s1a) >> (8 * q)) & 0xFFu);
        const v8i A0 = {(int)ca.x, (int)ca.y, (int)ca.z, (int)ca.w, 0, 0, 0, 0};
        const v8i A1 = {(int)cb.x, (int)cb.y, (int)cb.z, (int)cb.w, 0, 0, 0, 0};
        acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A0, B, acc0, 4, 0, 0, sa0, 0, sbb);
        acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, B, acc1, 4, 0, 0, sa1, 0, sbb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4& ca = i ? c01 : c00;
        const uint4& cb = i ? c11 : c10;
        v2h sp0, sp1;
        if (MODE == 0) {
          sp0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(i ? s0b : s0a, 1.0f, false);
          sp1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(i ? s1b : s1a, 1.0f, false);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint4 braw = *reinterpret_cast<const uint4*>(brow + (128 * i + 32 * q + 8 * jj) * 2);
          if (MODE == 0) {
            const v2h x0 = jj < 2 ? v2h{sp0[0], sp0[0]} : v2h{sp0[1], sp0[1]};
            const v2h x1 = jj < 2 ? v2h{sp1[0], sp1[0]} : v2h{sp1[1], sp1[1]};
            const v8h B = __builtin_bit_cast(v8h, braw);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(dw(ca, jj), x0), B, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8_f16(dw(cb, jj), x1), B, acc1, 0, 0, 0);
          } else {
            const float x0 = ue8m0_to_f32(((i ? s0b : s0a) >> (8 * q)) & 0xFFu);
            const float x1 = ue8m0_to_f32(((i ? s1b : s1a) >> (8 * q)) & 0xFFu);
            const v8bf B = __builtin_bit_cast(v8bf, braw);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(dw(ca, jj), x0), B, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8_bf16(dw(cb, jj), x1), B, acc1, 0, 0, 0);
          }
        }
      }
    }
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
    return launch_one<2, true>(a, max_tiles, s);
  }
  if (mode == 0) return launch_one<0, false>(a, max_tiles, s);
  if (mode == 1) return launch_one<1, false>(a, max_tiles, s);
  return launch_one<2, false>(a, max_tiles, s);
}

}  // namespace moefp4
