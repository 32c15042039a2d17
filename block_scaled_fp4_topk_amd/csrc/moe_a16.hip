// Grouped FC1 (+SwiGLU) and FC2 GEMMs for 16-bit activations over
// block-scaled FP4 weights (the W4A16 form of b12x moe/fused/w4a16/prepare.py:
// prepare_w4a16_modelopt_nvfp4_weights for K/16 E4M3 scales with a
// per-expert global scale, prepare_w4a16_fp4_e8m0_k32_weights for K/32 E8M0
// scales).
//
// Work decomposition: one workgroup = one (expert, 16*NT activation rows)
// tile x one block of weight rows; 4 wavefronts, each owning two 16-row MFMA
// tiles of weight rows (FC1: the gate rows i and the up rows I + i of the
// same 16 output columns, so SwiGLU is fused in registers; FC2: 32
// consecutive output rows).  The K loop streams the FP4 codes straight from
// HBM into registers (each lane: 32 contiguous bytes of one row per 256-K
// chunk) and stages the activation tile in LDS, shared by the 4 waves.
//
// Dequantisation (exact in both variants):
//  * gran 32 (UE8M0): v_cvt_scalef32_pk_bf16_fp4 with the power-of-two scale
//    -> bf16 weights, bf16 activations, bf16 MFMA.
//  * gran 16 (E4M3):  v_cvt_scalef32_pk_f16_fp4 then a packed fp16 multiply
//    by the E4M3 scale -> fp16 weights; activations enter as fp16 with an
//    exact per-row power-of-two scale (x: rows_to_f16 pre-pass; h: scaled by
//    its per-slot maximum while staged), fp16 MFMA; the row scale and the
//    global scale multiply the FP32 accumulator.
//
// The K index inside a 256-element chunk is permuted identically for both
// MFMA operands: lane group q (= lane / 16) owns chunk elements
// [64 q, 64 q + 64), fed to the 8 MFMAs j = 0..7 as [64 q + 8 j, + 8).
#include "common.h"
#include "kernels.h"

namespace moefp4 {

namespace {

constexpr int kChunk = 256;
constexpr int kLdsStride = kChunk + 8;  // 16-bit elements per staged row (+16 B pad)

template <int GRAN>
struct Wfrag {
  uint4 c[2];   // 32 bytes = 64 codes
  uint32_t s;   // GRAN 16: 4 E4M3 bytes; GRAN 32: 2 UE8M0 bytes
};

template <int GRAN>
__device__ __forceinline__ void load_wfrag(Wfrag<GRAN>& f, const uint8_t* row_codes,
                                           const uint8_t* row_sf, int k0, int q) {
  const uint8_t* p = row_codes + (k0 >> 1) + q * 32;
  f.c[0] = ld_nt(p);
  f.c[1] = ld_nt(p + 16);
  if (GRAN == 16) {
    f.s = *reinterpret_cast<const uint32_t*>(row_sf + (k0 >> 4) + q * 4);
  } else {
    f.s = *reinterpret_cast<const uint16_t*>(row_sf + (k0 >> 5) + q * 2);
  }
}

template <int GRAN>
__device__ __forceinline__ uint32_t code_dword(const Wfrag<GRAN>& f, int j) {
  const uint4& v = f.c[j >> 2];
  const int r = j & 3;
  return r == 0 ? v.x : r == 1 ? v.y : r == 2 ? v.z : v.w;
}

// Per-block (expert tile, weight-row block) kernel.
//  FC1: A-tiles = gate rows / up rows; output h (bf16) [A, I].
//  FC2: A-tiles = rows n0 .. n0+31;     output y (f32)  [A, H].
template <int GRAN, int NT, bool FC1>
__global__ __launch_bounds__(256) void fc_a16_kernel(FcArgs a) {
  constexpr int BN = NT * 16;
  __shared__ __attribute__((aligned(16))) uint16_t s_act[BN * kLdsStride];
  __shared__ int s_rowsrc[BN];
  __shared__ float s_rowscale[BN];

  const int tile = blockIdx.x;
  if (tile >= a.ntiles[0]) return;
  const int e = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const int ne = a.counts[e], oe = a.offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;

  int row0, row1, obase;
  if (FC1) {
    obase = blockIdx.y * 64 + wave * 16;  // output column i0 of this wave
    // row0 feeds acc[0] (gate), row1 feeds acc[1] (up)
    row0 = a.w13_order == 0 ? obase + r16 : a.I + obase + r16;
    row1 = a.w13_order == 0 ? a.I + obase + r16 : obase + r16;
  } else {
    obase = blockIdx.y * 128 + wave * 32;
    row0 = obase + r16;
    row1 = obase + 16 + r16;
  }
  const size_t rowbytes = (size_t)(K >> 1);
  const size_t sfbytes = (size_t)(K / GRAN);
  const uint8_t* wc0 = a.w + ((size_t)e * N + row0) * rowbytes;
  const uint8_t* wc1 = a.w + ((size_t)e * N + row1) * rowbytes;
  const uint8_t* ws0 = a.wsf + ((size_t)e * N + row0) * sfbytes;
  const uint8_t* ws1 = a.wsf + ((size_t)e * N + row1) * sfbytes;

  // activation source row and its power-of-two scale per staged row
  if (tid < BN) {
    const int m = m0 + tid;
    int src = -1;
    float sc = 1.0f;
    if (m < ne) {
      const int slot = oe + m;
      if (FC1) {
        src = a.sorted_assign[slot] / a.top_k;
        if (GRAN == 16) sc = a.act_scale[src];
      } else {
        src = slot;
        if (GRAN == 16) {
          const uint32_t hm = a.hmax_in[slot];
          const int p = hm ? (int)(hm >> 23) - 127 - 14 : 0;
          sc = __builtin_ldexpf(1.0f, p);
        }
      }
    }
    s_rowsrc[tid] = src;
    s_rowscale[tid] = sc;
  }
  __syncthreads();

  v4f acc[2][NT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[t][n] = v4f{0.f, 0.f, 0.f, 0.f};

  Wfrag<GRAN> f0, f1;
  load_wfrag<GRAN>(f0, wc0, ws0, 0, q);
  load_wfrag<GRAN>(f1, wc1, ws1, 0, q);

  const uint16_t* act = reinterpret_cast<const uint16_t*>(a.act);
  for (int k0 = 0; k0 < K; k0 += kChunk) {
    // stage the activation chunk: thread -> (row, 16-element segment)
#pragma unroll
    for (int rr = 0; rr < NT; ++rr) {
      const int r = rr * 16 + (tid >> 4), seg = tid & 15;
      const int src = s_rowsrc[r];
      uint4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
      if (src >= 0) {
        const uint4* p = reinterpret_cast<const uint4*>(act + (size_t)src * K + k0 + seg * 16);
        v0 = p[0];
        v1 = p[1];
        if (!FC1 && GRAN == 16) {
          // bf16 h -> fp16 * 2**-p (exact: 8 significant bits, in range)
          const float inv = 1.0f / s_rowscale[r];
          uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float lo = bf16_to_f32(w[i] & 0xFFFF) * inv;
            const float hi = bf16_to_f32(w[i] >> 16) * inv;
            const _Float16 hl = (_Float16)lo, hh = (_Float16)hi;
            w[i] = (uint32_t)__builtin_bit_cast(uint16_t, hl) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hh) << 16);
          }
          v0 = uint4{w[0], w[1], w[2], w[3]};
          v1 = uint4{w[4], w[5], w[6], w[7]};
        }
      }
      uint4* d = reinterpret_cast<uint4*>(s_act + r * kLdsStride + seg * 16);
      d[0] = v0;
      d[1] = v1;
    }
    __syncthreads();

    // prefetch the next chunk's weights while this one is consumed
    Wfrag<GRAN> g0 = f0, g1 = f1;
    if (k0 + kChunk < K) {
      load_wfrag<GRAN>(f0, wc0, ws0, k0 + kChunk, q);
      load_wfrag<GRAN>(f1, wc1, ws1, k0 + kChunk, q);
    }

#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kk = q * 64 + j * 8;
      if (GRAN == 16) {
        const v2h s0 = e4m3_to_h2((g0.s >> (8 * (j >> 1))) & 0xFF);
        const v2h s1 = e4m3_to_h2((g1.s >> (8 * (j >> 1))) & 0xFF);
        const v8h A0 = dq8_f16(code_dword(g0, j), s0);
        const v8h A1 = dq8_f16(code_dword(g1, j), s1);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const v8h B = *reinterpret_cast<const v8h*>(s_act + (n * 16 + r16) * kLdsStride + kk);
          acc[0][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, B, acc[0][n], 0, 0, 0);
          acc[1][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, B, acc[1][n], 0, 0, 0);
        }
      } else {
        const float s0 = ue8m0_to_f32((g0.s >> (8 * (j >> 2))) & 0xFF);
        const float s1 = ue8m0_to_f32((g1.s >> (8 * (j >> 2))) & 0xFF);
        const v8bf A0 = dq8_bf16(code_dword(g0, j), s0);
        const v8bf A1 = dq8_bf16(code_dword(g1, j), s1);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const v8bf B = *reinterpret_cast<const v8bf*>(s_act + (n * 16 + r16) * kLdsStride + kk);
          acc[0][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc[0][n], 0, 0, 0);
          acc[1][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc[1][n], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds rows 4q..4q+3 of each 16-row tile, column r16
  const float gsc = a.gs ? a.gs[e] : 1.0f;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int m = m0 + n * 16 + r16;
    const bool valid = m < ne;
    const int slot = oe + m;
    const float cs = s_rowscale[n * 16 + r16] * gsc;
    if (FC1) {
      uint32_t hb[4];
      uint32_t hmax = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[0][n][i] * cs, u = acc[1][n][i] * cs;
        hb[i] = f32_to_bf16_rne(swiglu(g, u));
        const uint32_t mag = (hb[i] & 0x7FFFu) << 16;
        hmax = mag > hmax ? mag : hmax;
      }
      if (valid) {
        uint16_t* h = reinterpret_cast<uint16_t*>(a.h_out) + (size_t)slot * a.I + obase + 4 * q;
        *reinterpret_cast<uint2*>(h) = uint2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
      }
      if (GRAN == 16) {
        uint32_t o = __shfl_xor(hmax, 16, 64);
        hmax = o > hmax ? o : hmax;
        o = __shfl_xor(hmax, 32, 64);
        hmax = o > hmax ? o : hmax;
        if (valid && q == 0 && hmax) atomicMax(a.hmax_out + slot, hmax);
      }
    } else if (valid) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float* y = a.y_out + (size_t)slot * a.H + obase + 16 * t + 4 * q;
        *reinterpret_cast<float4*>(y) =
            float4{acc[t][n][0] * cs, acc[t][n][1] * cs, acc[t][n][2] * cs, acc[t][n][3] * cs};
      }
    }
  }
}

template <int GRAN, int NT, bool FC1>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int rows_per_block = FC1 ? 64 : 128;
  const int nblk = FC1 ? a.I / rows_per_block : a.H / rows_per_block;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((fc_a16_kernel<GRAN, NT, FC1>), dim3(max_tiles, nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1_a16(const FcArgs& a, int gran, int max_tiles, hipStream_t s) {
  return gran == 16 ? launch_one<16, 4, true>(a, max_tiles, s) : launch_one<32, 4, true>(a, max_tiles, s);
}

hipError_t launch_fc2_a16(const FcArgs& a, int gran, int max_tiles, hipStream_t s) {
  return gran == 16 ? launch_one<16, 4, false>(a, max_tiles, s) : launch_one<32, 4, false>(a, max_tiles, s);
}

}  // namespace moefp4
