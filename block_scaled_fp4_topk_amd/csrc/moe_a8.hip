// Grouped FC1 (+SwiGLU + FP8 requantisation of h) and FC2 GEMMs for FP8
// activations with per-32 UE8M0 scales over FP4 weights with per-32 UE8M0
// scales: the FP8xFP4 recipe (1, 1, 32) of the GLM-5.2 NVFP4 group16
// MegaMoE notes (Context), computed with the CDNA4 block-scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 (A = FP4 weights, B = FP8 activations;
// each lane passes the UE8M0 byte of its row/column for its 32-wide K block).
//
// One workgroup = one (expert, 16*NT activation rows) tile x one block of
// weight rows; 4 wavefronts.  FC1 waves own 32 gate rows and the matching 32
// up rows (four 16-row MFMA tiles), so every 32-element block of h of a row
// is produced inside one wavefront and can be quantised there: UE8M0
// e = ceil(log2(amax / 448)), E4M3 codes = RNE(h / 2**e).  FC2 waves own 32
// output rows.  Codes and scales of the weights go HBM -> registers; the
// activation chunk (256 K bytes per row + its 8 scale bytes) is staged in LDS.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace moefp4 {

namespace {

constexpr int kChunk = 256;          // K elements per loop iteration (2 MFMA K-steps)
constexpr int kActStride = kChunk + 16;


struct W4frag {
  uint4 c[2];    // MFMA step 0 / 1: 16 bytes = 32 codes each
  uint2 s;       // 8 UE8M0 bytes of the chunk
};

__device__ __forceinline__ void load_w4(W4frag& f, const uint8_t* rc, const uint8_t* rs, int k0,
                                        int q) {
  const uint8_t* p = rc + (k0 >> 1) + 16 * q;
  f.c[0] = ld_nt(p);
  f.c[1] = ld_nt(p + 64);
  f.s = *reinterpret_cast<const uint2*>(rs + (k0 >> 5));
}

__device__ __forceinline__ int sbyte(const uint2& s, int idx) {
  const uint32_t w = idx < 4 ? s.x : s.y;
  return (int)((w >> (8 * (idx & 3))) & 0xFFu);
}

__device__ __forceinline__ v8i a_op(const uint4& c) {
  v8i r = {(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  return r;
}

template <int NT, int TILES>
__device__ __forceinline__ void stage_and_mma(const uint8_t* act, const uint8_t* act_sf, int K,
                                              const int* s_rowsrc, uint8_t* s_act, uint8_t* s_sf,
                                              int k0, int tid, int r16, int q,
                                              const W4frag (&f)[TILES], v4f (&acc)[TILES][NT]) {
#pragma unroll
  for (int rr = 0; rr < NT; ++rr) {
    const int r = rr * 16 + (tid >> 4), seg = tid & 15;
    const int src = s_rowsrc[r];
    uint4 v = {0, 0, 0, 0};
    if (src >= 0) v = *reinterpret_cast<const uint4*>(act + (size_t)src * K + k0 + seg * 16);
    *reinterpret_cast<uint4*>(s_act + r * kActStride + seg * 16) = v;
  }
  if (tid < NT * 16) {
    const int src = s_rowsrc[tid];
    uint2 v = {0, 0};
    if (src >= 0) v = *reinterpret_cast<const uint2*>(act_sf + (size_t)src * (K >> 5) + (k0 >> 5));
    *reinterpret_cast<uint2*>(s_sf + tid * 8) = v;
  }
  __syncthreads();
#pragma unroll
  for (int st = 0; st < 2; ++st) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint8_t* rowp = s_act + (n * 16 + r16) * kActStride + st * 128 + 16 * q;
      const uint4 b0 = *reinterpret_cast<const uint4*>(rowp);
      const uint4 b1 = *reinterpret_cast<const uint4*>(rowp + 64);
      const v8i B = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                     (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      const int sb = s_sf[(n * 16 + r16) * 8 + st * 4 + q];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int sa = sbyte(f[t].s, st * 4 + q);
        acc[t][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_op(f[t].c[st]), B, acc[t][n],
                                                                    4, 0, 0, sa, 0, sb);
      }
    }
  }
  __syncthreads();
}

template <int NT, bool FC1>
__global__ __launch_bounds__(256) void fc_a8_kernel(FcArgs a) {
  constexpr int BN = NT * 16;
  constexpr int TILES = FC1 ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t s_act[BN * kActStride];
  __shared__ __attribute__((aligned(16))) uint8_t s_sf[BN * 8];
  __shared__ int s_rowsrc[BN];

  const int tile = blockIdx.x;
  if (tile >= a.ntiles[0]) return;
  const int e = a.tiles[2 * tile], m0 = a.tiles[2 * tile + 1];
  const int ne = a.counts[e], oe = a.offsets[e];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;

  int obase;
  int rows[TILES];
  if (FC1) {
    obase = blockIdx.y * 128 + wave * 32;
    const int g = a.w13_order == 0 ? 0 : a.I, u = a.w13_order == 0 ? a.I : 0;
    rows[0] = g + obase + r16;
    rows[1] = g + obase + 16 + r16;
    rows[2 % TILES] = u + obase + r16;
    rows[3 % TILES] = u + obase + 16 + r16;
  } else {
    obase = blockIdx.y * 128 + wave * 32;
    rows[0] = obase + r16;
    rows[1 % TILES] = obase + 16 + r16;
  }
  const uint8_t* wc[TILES];
  const uint8_t* ws[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    wc[t] = a.w + ((size_t)e * N + rows[t]) * (size_t)(K >> 1);
    ws[t] = a.wsf + ((size_t)e * N + rows[t]) * (size_t)(K >> 5);
  }

  if (tid < BN) {
    const int m = m0 + tid;
    int src = -1;
    if (m < ne) src = FC1 ? a.sorted_assign[oe + m] / a.top_k : oe + m;
    s_rowsrc[tid] = src;
  }
  __syncthreads();

  v4f acc[TILES][NT];
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[t][n] = v4f{0.f, 0.f, 0.f, 0.f};

  W4frag f[TILES], g[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) load_w4(f[t], wc[t], ws[t], 0, q);

  const uint8_t* act = reinterpret_cast<const uint8_t*>(a.act);
  for (int k0 = 0; k0 < K; k0 += kChunk) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) g[t] = f[t];
    if (k0 + kChunk < K) {
#pragma unroll
      for (int t = 0; t < TILES; ++t) load_w4(f[t], wc[t], ws[t], k0 + kChunk, q);
    }
    stage_and_mma<NT, TILES>(act, a.act_sf, K, s_rowsrc, s_act, s_sf, k0, tid, r16, q, g, acc);
  }

  const float gsc = a.gs ? a.gs[e] : 1.0f;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int m = m0 + n * 16 + r16;
    const bool valid = m < ne;
    const int slot = oe + m;
    if (FC1) {
      float h[2][4];
      float amax = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[t][i] = swiglu(acc[t][n][i] * gsc, acc[t + 2][n][i] * gsc);
          amax = fmaxf(amax, fabsf(h[t][i]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      int ex = amax > 0.0f ? ceil_log2_over_448(amax) : -127;
      ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
      const float inv = __builtin_ldexpf(1.0f, -ex);
      if (valid) {
        uint8_t* hrow = reinterpret_cast<uint8_t*>(a.h_out) + (size_t)slot * a.I;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint32_t w = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) w |= f32_to_e4m3_rne(h[t][i] * inv) << (8 * i);
          *reinterpret_cast<uint32_t*>(hrow + obase + 16 * t + 4 * q) = w;
        }
        if (q == 0) a.h_sf_out[(size_t)slot * (a.I >> 5) + (obase >> 5)] = (uint8_t)(ex + 127);
      }
    } else if (valid) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float* y = a.y_out + (size_t)slot * a.H + obase + 16 * t + 4 * q;
        *reinterpret_cast<float4*>(y) = float4{acc[t][n][0] * gsc, acc[t][n][1] * gsc,
                                               acc[t][n][2] * gsc, acc[t][n][3] * gsc};
      }
    }
  }
}

template <int NT, bool FC1>
hipError_t launch_one(const FcArgs& a, int max_tiles, hipStream_t s) {
  const int nblk = (FC1 ? a.I : a.H) / 128;
  if (max_tiles <= 0 || nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((fc_a8_kernel<NT, FC1>), dim3(max_tiles, nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ w, int T, int k,
                                                      int H, void* __restrict__ out) {
  // Work item b = (token t, column chunk c) in token-major order, so that
  // consecutive workgroups read consecutive 4 KB pieces of the same Y rows;
  // the grid strides over the items (it is capped below 2^32 work-items).
  const int nch = (H / 4 + 255) / 256;
  const long long items = (long long)T * nch;
  for (long long b = blockIdx.x; b < items; b += gridDim.x) {
    const int t = (int)(b / nch);
    const int n = ((int)(b - (long long)t * nch) * 256 + threadIdx.x) * 4;
    if (n >= H) continue;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    // Y is read once: non-temporal (whole 4 KB row pieces per workgroup).
    // The rows of 8 picks are loaded before any is summed (8 loads in flight
    // per lane instead of one), then summed in pick order.
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    for (int j0 = 0; j0 < k; j0 += 8) {
      f32x4 v[8];
      float wj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int s = j < k ? slot_of[(size_t)t * k + j] : -1;
        wj[u] = s >= 0 ? w[(size_t)t * k + j] : 0.f;
        v[u] = s >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + (size_t)s * H + n))
                      : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u >= k || slot_of[(size_t)t * k + j0 + u] < 0) continue;
        acc.x += wj[u] * v[u].x;
        acc.y += wj[u] * v[u].y;
        acc.z += wj[u] * v[u].z;
        acc.w += wj[u] * v[u].w;
      }
    }
    if (F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + (size_t)t * H + n) = acc;
    } else {
      const uint32_t b0 = f32_to_bf16_rne(acc.x), b1 = f32_to_bf16_rne(acc.y);
      const uint32_t b2 = f32_to_bf16_rne(acc.z), b3 = f32_to_bf16_rne(acc.w);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (size_t)t * H + n) =
          uint2{b0 | (b1 << 16), b2 | (b3 << 16)};
    }
  }
}

}  // namespace

hipError_t launch_fc1_a8(const FcArgs& a, int max_tiles, hipStream_t s) {
  return launch_one<4, true>(a, max_tiles, s);
}

hipError_t launch_fc2_a8(const FcArgs& a, int max_tiles, hipStream_t s) {
  return launch_one<4, false>(a, max_tiles, s);
}

hipError_t launch_combine(const float* y, const int32_t* slot_of, const float* topk_w, int T,
                          int k, int H, void* out, bool out_f32, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  // one workgroup per (token, column chunk), at most 2^22 (the kernel strides)
  const long long items = (long long)T * ((H / 4 + 255) / 256);
  const dim3 grid((unsigned)std::min<long long>(items, 1LL << 22));
  if (out_f32)
    hipLaunchKernelGGL(combine_kernel<true>, grid, dim3(256), 0, s, y, slot_of, topk_w, T, k, H, out);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, dim3(256), 0, s, y, slot_of, topk_w, T, k, H, out);
  return hipGetLastError();
}

}  // namespace moefp4
