// Routing: stable counting sort of the T*k assignments by expert id, the
// per-expert tile list of the grouped GEMMs, and the fp16 row preparation
// used by the group16 (E4M3-scaled) path.
//
// The grouping is the "top-k routed tokens gathered per expert" step of the
// fused MoE (GLM-5.2 NVFP4 group16 MegaMoE notes, Context; b12x W4A16
// prepare.py, make_w4a16_packed_buffers sizes its buffers by tokens and
// top-k).  The order inside an expert is the assignment order a = t*k + j,
// made deterministic without atomics on positions: within a wavefront the
// rank of a lane among lanes with the same expert comes from ballots over
// the bits of the expert id; across wavefronts from per-wave counts in LDS.
#include "common.h"
#include "kernels.h"

namespace moefp4 {

namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// Exclusive scan of v over the whole block (one value per thread);
// returns the exclusive prefix, *total gets the block sum.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kRouteWaves ? s_tmp[lane] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      int y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < kRouteWaves) s_tmp[64 + lane] = w;  // inclusive wave prefix
  }
  __syncthreads();
  const int before = wave ? s_tmp[64 + wave - 1] : 0;
  *total = s_tmp[64 + kRouteWaves - 1];
  __syncthreads();
  return before + x - v;
}

// Power-of-two fp16 staging exponent of a bf16 row: p = floor(log2(max |x|))
// - 14, so that max * 2**-p lies in [2**14, 2**15) (bf16's 8 significant bits
// then fit fp16 exactly down to 2**-24 of the scaled range).
__device__ __forceinline__ int row_exponent(uint32_t maxbits) {
  const int p = maxbits ? (int)(maxbits >> 23) - 127 - 14 : 0;
  return p < -110 ? -110 : p;
}

// One workgroup per row (rows b, b + nb, ...): the row's largest |x|
// (compared as bit patterns), its scale 2**p, and (x16) the row converted to
// fp16 with that scale, each thread taking 8 elements every 8 * 1024.
__device__ void row_scales_from(const RouteOut& o, int b, int nb) {
  __shared__ uint32_t s_red[kRouteWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = b; t < o.T; t += nb) {
    const uint16_t* row = o.x + (size_t)t * o.H;
    uint32_t m = 0;
    for (int i = tid * 8; i < o.H; i += 8 * kRouteThreads) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + i);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (w[j] & 0x7FFFu) << 16, hi = (w[j] & 0x7FFF0000u);
        m = lo > m ? lo : m;
        m = hi > m ? hi : m;
      }
    }
    for (int d = 32; d >= 1; d >>= 1) {
      const uint32_t y = __shfl_xor(m, d, 64);
      m = y > m ? y : m;
    }
    if (lane == 0) s_red[wave] = m;
    __syncthreads();
    m = s_red[0];
    for (int w = 1; w < kRouteWaves; ++w) m = s_red[w] > m ? s_red[w] : m;
    const int pt = row_exponent(m);
    if (tid == 0) o.row_scale[t] = __builtin_ldexpf(1.0f, pt);
    if (o.x16) {
      // the row again (cache-resident), times 2**-p, to fp16
      const float inv = __builtin_ldexpf(1.0f, -pt);
      uint16_t* orow = o.x16 + (size_t)t * o.H;
      for (int i = tid * 8; i < o.H; i += 8 * kRouteThreads) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + i);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const _Float16 lo = (_Float16)(bf16_to_f32(w[j] & 0xFFFFu) * inv);
          const _Float16 hi = (_Float16)(bf16_to_f32(w[j] >> 16) * inv);
          w[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint4*>(orow + i) = uint4{w[0], w[1], w[2], w[3]};
      }
    }
    __syncthreads();  // s_red is reused by the next row
  }
}

// Stable scatter of assignments [a0, a1), 1024 per pass, to s_base[e] +
// (rank among earlier assignments of expert e); s_base advances per pass.
// Within a wavefront the rank comes from ballots over the bits of the expert
// id, across wavefronts from per-wave counts in LDS.
__device__ void scatter_range(const int32_t* __restrict__ ids, int a0, int a1, int E, int* s_base,
                              int* s_wc, const RouteOut& o) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int c0 = a0; c0 < a1; c0 += kRouteThreads) {
    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) s_wc[i] = 0;
    const int a = c0 + tid;
    const int e = a < a1 ? ids[a] : -1;
    const bool valid = a < a1 && (unsigned)e < (unsigned)E;
    uint64_t peers = ballot(valid);
    const int key = valid ? e : 0;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    __syncthreads();  // s_wc cleared
    if (valid && rank == 0) s_wc[wave * E + e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = s_base[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wc[w * E + e];
      o.sorted_assign[pos] = a;
      o.slot_of[a] = pos;
    } else if (a < a1) {
      o.slot_of[a] = -1;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kRouteThreads) {
      int s = 0;
      for (int w = 0; w < kRouteWaves; ++w) s += s_wc[w * E + ee];
      s_base[ee] += s;
    }
    __syncthreads();
  }
}

// Counts and scans shared by both forms: expert counts c (thread e), their
// exclusive offsets, the tile list, the dropped count.  Returns the number
// of valid assignments.
__device__ int finish_counts(int c, int E, int tile_m, int drops, int* s_tmp, int* s_base,
                             const RouteOut& o) {
  const int tid = threadIdx.x;
  int valid_total;
  const int base = block_exclusive_scan(c, s_tmp, &valid_total);
  const int nt = (c + tile_m - 1) / tile_m;
  int tiles_total;
  const int tbase = block_exclusive_scan(nt, s_tmp, &tiles_total);
  if (tid < E) {
    o.counts[tid] = c;
    o.offsets[tid] = base;
    s_base[tid] = base;
    for (int i = 0; i < nt; ++i) {
      o.tiles[2 * (tbase + i)] = tid;
      o.tiles[2 * (tbase + i) + 1] = i * tile_m;
    }
  }
  if (tid == 0) {
    o.offsets[E] = valid_total;
    o.ntiles[0] = tiles_total;
    o.flags[0] = drops;
    o.flags[1] = 0;  // synchronisation timeouts of the single-launch decode kernel
  }
  return valid_total;
}

// Single-workgroup route (small T * k): histogram, scans, stable scatter.
// FP8 quantisation of one 32-element block of a bf16 row (the activation
// side of recipe (1, 1, 32)): UE8M0 e = smallest with 448 * 2**e >= amax,
// E4M3 RNE of x / 2**e (x / 2**e is exact in FP32: x has 8 significant bits
// and |x / 2**e| <= 448; values too small for FP32 normals round to zero
// in E4M3 either way).
__device__ __forceinline__ void quantize_block32(const uint16_t* __restrict__ src, uint8_t* dst,
                                                 uint8_t* sf) {
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const uint4*>(src)[i];
  uint32_t m = 0;  // largest magnitude, as bf16 bits (monotone in the value)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
      m = lo > m ? lo : m;
      m = hi > m ? hi : m;
    }
  }
  int ex = m ? ceil_log2_over_448(bf16_to_f32(m)) : -127;
  ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
  const float inv = __builtin_ldexpf(1.0f, -ex);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const uint32_t c0 = f32_to_e4m3_rne(bf16_to_f32(w[j] & 0xFFFFu) * inv);
      const uint32_t c1 = f32_to_e4m3_rne(bf16_to_f32(w[j] >> 16) * inv);
      const uint32_t c2 = f32_to_e4m3_rne(bf16_to_f32(w[j + 1] & 0xFFFFu) * inv);
      const uint32_t c3 = f32_to_e4m3_rne(bf16_to_f32(w[j + 1] >> 16) * inv);
      q[2 * i + j / 2] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
  }
  reinterpret_cast<uint4*>(dst)[0] = uint4{q[0], q[1], q[2], q[3]};
  reinterpret_cast<uint4*>(dst)[1] = uint4{q[4], q[5], q[6], q[7]};
  *sf = (uint8_t)(ex + 127);
}

// MXFP4 quantisation of one 32-element block of a bf16 row (the A4 form,
// the block rule of the group32 requantisation applied to activations):
// UE8M0 e = smallest with 6 * 2**e >= amax, clamped to [-127, 127] (amax
// == 0: -127), E2M1 RNE of x / 2**e with the sign kept.  x / 2**e is exact
// in FP32 (8 significant bits; a bf16 amax below 2**-126 clamps e to -127,
// which keeps every x / 2**e a finite FP32 value <= 6).  The RNE encode is
// the hardware conversion with a unit scale; codes are packed two per byte,
// element 2j in the low nibble.
__device__ __forceinline__ void quantize_block32_fp4(const uint16_t* __restrict__ src, uint8_t* dst,
                                                     uint8_t* sf) {
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const uint4*>(src)[i];
  uint32_t m = 0;  // largest magnitude, as bf16 bits (monotone in the value)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
      m = lo > m ? lo : m;
      m = hi > m ? hi : m;
    }
  }
  // amax = M * 2**E, M in [1, 2): 6 = 1.5 * 2**2, so e = E - 2 + (M > 1.5);
  // subnormal (and zero) maxima clamp to -127
  int ex = -127;
  if (m >= 0x0080u) {
    const int E = (int)(m >> 7) - 127;
    ex = E - 2 + ((m & 0x7Fu) > 0x40u ? 1 : 0);
    ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
  }
  const float inv = __builtin_ldexpf(1.0f, -ex);
  uint32_t q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf16_to_f32(w[j] & 0xFFFFu) * inv;
      f[2 * j + 1] = bf16_to_f32(w[j] >> 16) * inv;
    }
    uint32_t d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0], f[1], 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[2], f[3], 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[4], f[5], 1.0f, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[6], f[7], 1.0f, 3);
    q[i] = d;
  }
  *reinterpret_cast<uint4*>(dst) = uint4{q[0], q[1], q[2], q[3]};
  *sf = (uint8_t)(ex + 127);
}

// Workgroup b of nb quantises 32-element blocks b * 1024 + tid, then every
// nb * 1024 further; FP4: MXFP4 (16 code bytes per block), else E4M3 (32).
template <bool FP4>
__device__ __forceinline__ void quantize_rows_from(const uint16_t* __restrict__ x, long long T, int H,
                                   uint8_t* __restrict__ xq, uint8_t* __restrict__ xsf, int b,
                                   int nb) {
  const long long nblk = T * (H / 32);
  for (long long i = (long long)b * kRouteThreads + threadIdx.x; i < nblk;
       i += (long long)nb * kRouteThreads) {
    if (FP4) quantize_block32_fp4(x + i * 32, xq + i * 16, xsf + i);
    else quantize_block32(x + i * 32, xq + i * 32, xsf + i);
  }
}

template <bool FP4>
__global__ __launch_bounds__(kRouteThreads) void quantize_act_kernel(const uint16_t* __restrict__ x,
                                                                     long long T, int H,
                                                                     uint8_t* __restrict__ xq,
                                                                     uint8_t* __restrict__ xsf) {
  quantize_rows_from<FP4>(x, T, H, xq, xsf, blockIdx.x, gridDim.x);
}

// Activation preparation done by the extra workgroups of a route launch.
__device__ void row_prep(const RouteOut& o, int b, int nb) {
  if (o.row_scale) row_scales_from(o, b, nb);
  if (o.x8) {
    if (o.x_fp4) quantize_rows_from<true>(o.x, o.T, o.H, o.x8, o.xsf, b, nb);
    else quantize_rows_from<false>(o.x, o.T, o.H, o.x8, o.xsf, b, nb);
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ ids,
                                                              int A, int E, int tile_m,
                                                              RouteOut o) {
  extern __shared__ int smem[];
  int* s_base = smem;                 // [E] running start of each expert
  int* s_wc = s_base + E;             // [kRouteWaves][E] per-wave counts of a chunk
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_tmp[128];
  __shared__ int s_drop;
  const int tid = threadIdx.x;
  // workgroups past the first compute the per-row staging scales instead
  if (blockIdx.x > 0) {
    row_prep(o, blockIdx.x - 1, gridDim.x - 1);
    return;
  }

  for (int i = tid; i < o.n_zero; i += kRouteThreads) o.zero_words[i] = 0u;
  for (int e = tid; e < E; e += kRouteThreads) s_cnt[e] = 0;
  if (tid == 0) s_drop = 0;
  __syncthreads();

  // 1. histogram (LDS atomics: the counts do not depend on their order)
  int drop = 0;
  for (int a = tid; a < A; a += kRouteThreads) {
    const int e = ids[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
    else ++drop;
  }
  if (drop) atomicAdd(&s_drop, drop);
  __syncthreads();

  // 2. exclusive scans: expert offsets and tile offsets (E <= 1024 = threads)
  const int valid_total = finish_counts(tid < E ? s_cnt[tid] : 0, E, tile_m, s_drop, s_tmp, s_base, o);
  // 3. stable scatter
  scatter_range(ids, 0, A, E, s_base, s_wc, o);
  for (int i = valid_total + tid; i < A; i += kRouteThreads) o.sorted_assign[i] = -1;
}

// Multi-workgroup route (large T * k), three launches over chunks of
// o.chunk assignments: per-chunk histograms, one workgroup that scans them
// (chunk g of expert e starts at offsets[e] + the counts of e in chunks
// before g), and per-chunk stable scatters.  Same result as the single
// workgroup form.
__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(const int32_t* __restrict__ ids,
                                                                   int A, int E, RouteOut o) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_drop;
  const int tid = threadIdx.x;
  if (blockIdx.x >= o.nchunks) {
    row_prep(o, blockIdx.x - o.nchunks, gridDim.x - o.nchunks);
    return;
  }
  for (int e = tid; e < E; e += kRouteThreads) s_cnt[e] = 0;
  if (tid == 0) s_drop = 0;
  __syncthreads();
  const int a0 = blockIdx.x * o.chunk, a1 = min(A, a0 + o.chunk);
  int drop = 0;
  for (int a = a0 + tid; a < a1; a += kRouteThreads) {
    const int e = ids[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
    else ++drop;
  }
  if (drop) atomicAdd(&s_drop, drop);
  __syncthreads();
  int32_t* h = o.hist + (size_t)blockIdx.x * (E + 1);
  for (int e = tid; e < E; e += kRouteThreads) h[e] = s_cnt[e];
  if (tid == 0) h[E] = s_drop;
}

__global__ __launch_bounds__(kRouteThreads) void route_scan_kernel(int A, int E, int tile_m,
                                                                   RouteOut o) {
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_tmp[128];
  const int tid = threadIdx.x;
  for (int i = tid; i < o.n_zero; i += kRouteThreads) o.zero_words[i] = 0u;
  int c = 0, drops = 0;
  if (tid < E)
    for (int g = 0; g < o.nchunks; ++g) c += o.hist[(size_t)g * (E + 1) + tid];
  if (tid == 0)
    for (int g = 0; g < o.nchunks; ++g) drops += o.hist[(size_t)g * (E + 1) + E];
  const int valid_total = finish_counts(c, E, tile_m, drops, s_tmp, s_base, o);
  __syncthreads();
  // per-chunk starts, in place
  if (tid < E) {
    int run = s_base[tid];
    for (int g = 0; g < o.nchunks; ++g) {
      int32_t* h = o.hist + (size_t)g * (E + 1) + tid;
      const int n = *h;
      *h = run;
      run += n;
    }
  }
  for (int i = valid_total + tid; i < A; i += kRouteThreads) o.sorted_assign[i] = -1;
}

__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(const int32_t* __restrict__ ids,
                                                                      int A, int E, RouteOut o) {
  extern __shared__ int smem[];
  int* s_base = smem;       // [E]
  int* s_wc = s_base + E;   // [kRouteWaves][E]
  const int g = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kRouteThreads) s_base[e] = o.hist[(size_t)g * (E + 1) + e];
  __syncthreads();
  const int a0 = g * o.chunk, a1 = min(A, a0 + o.chunk);
  scatter_range(ids, a0, a1, E, s_base, s_wc, o);
}

__global__ __launch_bounds__(256) void rows_to_f16_kernel(const uint16_t* __restrict__ x, int T,
                                                          int H, uint16_t* __restrict__ x16,
                                                          float* __restrict__ scale) {
  __shared__ uint32_t s_max[4];
  const int t = blockIdx.x;
  if (t >= T) return;
  const uint16_t* row = x + (size_t)t * H;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < H; i += 256) {
    const uint32_t b = (uint32_t)(row[i] & 0x7FFF) << 16;
    m = b > m ? b : m;
  }
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t y = __shfl_xor(m, d, 64);
    m = y > m ? y : m;
  }
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  m = s_max[0];
  for (int w = 1; w < 4; ++w) m = s_max[w] > m ? s_max[w] : m;
  const int p = row_exponent(m);
  const float inv = __builtin_ldexpf(1.0f, -p);
  uint16_t* orow = x16 + (size_t)t * H;
  for (int i = threadIdx.x; i < H; i += 256) {
    const _Float16 h = (_Float16)(bf16_to_f32(row[i]) * inv);
    orow[i] = __builtin_bit_cast(uint16_t, h);
  }
  if (threadIdx.x == 0) scale[t] = __builtin_ldexpf(1.0f, p);
}

}  // namespace

hipError_t launch_route(const int32_t* topk_ids, int A, int E, int tile_m, const RouteOut& o,
                        hipStream_t s) {
  const size_t lds = (size_t)(E + kRouteWaves * E) * sizeof(int);
  int scale_blocks = 0;
  if (o.row_scale && o.T > 0) scale_blocks = o.T > 256 ? 256 : o.T;  // a row per workgroup
  if (o.x8 && o.T > 0) {
    const long long nb = ((long long)o.T * (o.H / 32) + kRouteThreads - 1) / kRouteThreads;
    scale_blocks = (int)(nb > 256 ? 256 : nb);
  }
  if (o.nchunks <= 0) {
    hipLaunchKernelGGL(route_kernel, dim3(1 + scale_blocks), dim3(kRouteThreads), lds, s, topk_ids, A,
                       E, tile_m, o);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_hist_kernel, dim3(o.nchunks + scale_blocks), dim3(kRouteThreads), 0, s,
                     topk_ids, A, E, o);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, s, A, E, tile_m, o);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(o.nchunks), dim3(kRouteThreads), lds, s, topk_ids, A,
                     E, o);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, long long T, int H, uint8_t* xq, uint8_t* xsf,
                               bool fp4, hipStream_t s) {
  if (T <= 0 || H <= 0) return hipSuccess;
  long long nb = (T * (H / 32) + kRouteThreads - 1) / kRouteThreads;
  nb = nb > 1024 ? 1024 : nb;
  if (fp4)
    hipLaunchKernelGGL(quantize_act_kernel<true>, dim3((unsigned)nb), dim3(kRouteThreads), 0, s, x, T, H,
                       xq, xsf);
  else
    hipLaunchKernelGGL(quantize_act_kernel<false>, dim3((unsigned)nb), dim3(kRouteThreads), 0, s, x, T, H,
                       xq, xsf);
  return hipGetLastError();
}

hipError_t launch_rows_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, float* scale,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(rows_to_f16_kernel, dim3(T), dim3(256), 0, s, x, T, H, x16, scale);
  return hipGetLastError();
}

}  // namespace moefp4
