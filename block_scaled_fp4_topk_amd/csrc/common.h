// Device helpers shared by the moefp4 kernels (gfx950 / CDNA4).
//
// Lane layouts of the matrix instructions used here, as measured on gfx950:
//  * v_mfma_f32_16x16x32_{bf16,f16}: lane l supplies row (A) / column (B)
//    l % 16 and the 8 K values 8*(l/16) .. 8*(l/16)+7; the 4 accumulator
//    values of lane l are rows 4*(l/16) + i, column l % 16.
//  * v_mfma_scale_f32_16x16x128_f8f6f4: an FP4 operand lane supplies the 32
//    K values 32*(l/16) .. +31 (16 bytes, low nibble first); an FP8 operand
//    lane supplies K 16*(l/16) .. +15 in bytes 0..15 and 64 + 16*(l/16) .. +15
//    in bytes 16..31.  The scale operand of lane l is the UE8M0 scale of row
//    / column l % 16 for the K block [32*(l/16), 32*(l/16) + 32).
//  * v_cvt_scalef32_pk_{bf16,f16}_fp4 decode one byte (two E2M1 codes, low
//    nibble first) exactly and multiply by 2**exponent(scale) -- only the
//    exponent of the f32 scale is used.
//  * v_cvt_f32_fp8 decodes OCP E4M3 (fn).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moefp4 {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming (non-temporal) load / store.
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void st_nt(void* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// E4M3 (fn) byte -> float, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// UE8M0 byte b -> 2**(b - 127) as f32 bits (valid for b in 1..254).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) { return u2f(b << 23); }

// Eight E2M1 codes (one dword, element 0 in the low nibble) -> eight bf16
// values times 2**exponent(scale).  Exact.
__device__ __forceinline__ v8bf dq8_bf16(uint32_t codes, float pow2_scale) {
  v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 0);
  v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 1);
  v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 2);
  v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, pow2_scale, 3);
  v8bf r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Eight E2M1 codes -> eight fp16 values times an fp16 block scale (the
// scale broadcast in both halves of s2).  E2M1 x E4M3 has at most 6
// significant bits and lies in [2**-10, 2688]: exact in fp16.
__device__ __forceinline__ v8h dq8_f16(uint32_t codes, v2h s2) {
  v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  v8h r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ v2h e4m3_to_h2(uint32_t byte) {
  _Float16 h = (_Float16)e4m3_to_f32(byte);
  v2h r = {h, h};
  return r;
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = f2u(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return u2f(bits16 << 16); }

// silu(z) * u in f32.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}
// The same with the hardware reciprocal (1 ulp) in place of the IEEE
// division, for epilogues where SwiGLU is a visible share of the VALU work;
// the result differs from swiglu() by a few ulp, far below the rounding to
// FP8 / FP4 that follows.
__device__ __forceinline__ float swiglu_fast(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Smallest e with 448 * 2**e >= a (a > 0 normal): a = M * 2**E, M in [1, 2):
// 448 = 1.75 * 2**8, so e = E - 8 + (M > 1.75).
__device__ __forceinline__ int ceil_log2_over_448(float a) {
  uint32_t b = f2u(a);
  int E = (int)(b >> 23) - 127;
  return E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
}

// Smallest e with 6 * 2**e >= a (a > 0): a = M * 2**E, M in [1, 2): 6 =
// 1.5 * 2**2, so e = E - 2 + (M > 1.5).  FP32 subnormal a gives e <= -128
// (callers clamp to -127).
__device__ __forceinline__ int ceil_log2_over_6(float a) {
  uint32_t b = f2u(a);
  int E = (int)(b >> 23) - 127;
  return E - 2 + ((b & 0x7FFFFFu) > 0x400000u ? 1 : 0);
}

// E4M3 (fn) round-to-nearest-even encode of |y| <= 448, sign kept: normals
// (|y| >= 2**-6) round the 23-bit mantissa to 3 bits, subnormals round to a
// multiple of 2**-9.
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

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

}  // namespace moefp4
