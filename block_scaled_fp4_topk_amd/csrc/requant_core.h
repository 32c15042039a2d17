// Arithmetic core of the group16 -> group32 FP4 requantisation, written so
// that it compiles both for gfx950 (the kernel in requant.hip) and for the
// host (a CPU build used to check the arithmetic without a GPU).
//
// What is computed (GLM-5.2 NVFP4 group16 MegaMoE notes, Requantization
// path): restored values v = E2M1(code) * E4M3(scale16) * gs; per block of
// 32, UE8M0 e = smallest integer with 6 * 2**e >= max|v|; codes =
// RNE(|v| / 2**e) on the E2M1 grid, ties to the even code, sign of v kept.
//
// Exactness in FP32.  E2M1 * E4M3 is exact (<= 6 significant bits); the
// product with gs is not, so it is rounded to odd (round toward zero, then
// set the last bit when inexact): with 24 >= 2 + 2 bits of precision a
// round-to-odd value followed by a round-to-nearest-even to the 2-bit E2M1
// grid gives the same result as rounding the exact value, and the odd
// result can never land on a grid midpoint or on 6 * 2**e unless the exact
// value does, so the choice of e is exact too.  Powers of two then scale
// the values without error.
//
// Per 16-element half-block only 7 distinct magnitudes occur, so the codes
// are mapped through a per-half lookup table of the 8 source magnitudes
// (applied to 4 codes at a time with a byte permute).
#pragma once

#include <stdint.h>
#include <string.h>
#include <math.h>

#if defined(__HIPCC__)
#define MOEFP4_HD __host__ __device__ __forceinline__
#else
#define MOEFP4_HD inline
#endif

namespace moefp4 {
namespace rq {

MOEFP4_HD uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
MOEFP4_HD float fbits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

// Byte permute: byte i of the result is byte sel_i of the 8-byte value
// {hi:lo} (selector values 0..7 only).
MOEFP4_HD uint32_t perm8(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(hi, lo, sel);
#else
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) r |= (uint32_t)((v >> (8 * ((sel >> (8 * i)) & 7))) & 0xFF) << (8 * i);
  return r;
#endif
}

MOEFP4_HD int clz32(uint32_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_clz(x);
#else
  return x ? __builtin_clz(x) : 32;
#endif
}

// E4M3 (fn) byte -> f32 (finite bytes), exact.
MOEFP4_HD float e4m3_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15, m = b & 7;
  const float mag = e ? fbits(((e + 120) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (b & 0x80) ? -mag : mag;
}

// Magnitude of E2M1 code m (0..7) as f32.
MOEFP4_HD float e2m1_f32(uint32_t m) {
  return m < 2 ? (float)m * 0.5f : fbits(((126 + (m >> 1)) << 23) | ((m & 1) << 22));
}

// a * b rounded to odd (a, b >= 0, finite, product normal or zero).
MOEFP4_HD float mul_ro(float a, float b) {
  const float hi = a * b;
  const float lo = fmaf(a, b, -hi);
  uint32_t u = bits(hi);
  if (lo != 0.0f) u = (u - (lo < 0.0f ? 1u : 0u)) | 1u;
  return fbits(u);
}

// RNE of x in [0, 6] onto the E2M1 grid -> magnitude code 0..7.  The grid
// quantum at x is 2**(k-1), k = max(0, floor(log2 x)); adding 2**(22+k) (a
// float whose ulp is that quantum) rounds x to the grid and the bit
// distance counts quanta.
MOEFP4_HD uint32_t e2m1_code(float x) {
  const int ex = (int)(bits(x) >> 23) - 127;
  const uint32_t k = ex < 0 ? 0u : (uint32_t)ex;
  const float c = fbits(0x4A800000u + (k << 23));
  const float t = x + c;
  return bits(t) - bits(c) + 2u * k;
}

// Max magnitude code (0..7) among the 8 codes of each dword of a half.
MOEFP4_HD uint32_t max_mag(uint32_t w0, uint32_t w1) {
  // one-hot byte 1 << m per code, OR-reduced
  const uint32_t lo = 0x08040201u, hi = 0x80402010u;
  uint32_t o = perm8(hi, lo, w0 & 0x07070707u) | perm8(hi, lo, (w0 >> 4) & 0x07070707u) |
               perm8(hi, lo, w1 & 0x07070707u) | perm8(hi, lo, (w1 >> 4) & 0x07070707u);
  o |= o >> 16;
  o |= o >> 8;
  o &= 0xFFu;
  return 31u - (uint32_t)clz32(o | 1u);
}

// Byte lookup table (two dwords) mapping source magnitude m to the new
// magnitude code, for a half with E4M3 scale s (f32, >= 0), |gs| = ag and
// block exponent e: value of magnitude m = E2M1(m) * s * ag / 2**e.
MOEFP4_HD void half_lut(float s, float ag, int e, uint32_t& lut_lo, uint32_t& lut_hi) {
  // E2M1 magnitudes are {1,2,4,8} * 0.5 and {3,6,12} * 0.5: two odd-rounded
  // products, then exact power-of-two multiples.
  const float p1 = ldexpf(mul_ro(s, ag), -e - 1);
  const float p3 = ldexpf(mul_ro(3.0f * s, ag), -e - 1);
  const uint32_t c1 = e2m1_code(fminf(p1, 6.0f));
  const uint32_t c2 = e2m1_code(fminf(2.0f * p1, 6.0f));
  const uint32_t c3 = e2m1_code(fminf(p3, 6.0f));
  const uint32_t c4 = e2m1_code(fminf(4.0f * p1, 6.0f));
  const uint32_t c5 = e2m1_code(fminf(2.0f * p3, 6.0f));
  const uint32_t c6 = e2m1_code(fminf(8.0f * p1, 6.0f));
  const uint32_t c7 = e2m1_code(fminf(4.0f * p3, 6.0f));
  lut_lo = (c1 << 8) | (c2 << 16) | (c3 << 24);
  lut_hi = c4 | (c5 << 8) | (c6 << 16) | (c7 << 24);
}

MOEFP4_HD uint32_t apply_lut(uint32_t w, uint32_t lut_lo, uint32_t lut_hi, uint32_t signflip) {
  const uint32_t nlo = perm8(lut_hi, lut_lo, w & 0x07070707u);
  const uint32_t nhi = perm8(lut_hi, lut_lo, (w >> 4) & 0x07070707u);
  return ((w & 0x88888888u) ^ signflip) | nlo | (nhi << 4);
}

// One 32-element block: c[4] packed codes (elements 8i..8i+7 in c[i]),
// sf16 = two E4M3 bytes (half 0 in the low byte), gs = global scale.
// Writes the new codes and returns the UE8M0 byte.
MOEFP4_HD uint32_t requant_block(const uint32_t c[4], uint32_t sf16, float gs, uint32_t out[4]) {
  const float s0 = fabsf(e4m3_f32(sf16 & 0xFF));
  const float s1 = fabsf(e4m3_f32((sf16 >> 8) & 0xFF));
  const uint32_t gneg = bits(gs) >> 31;
  // a negative block scale flips the sign of its half, like a negative gs
  const uint32_t flip0 = ((sf16 >> 7) & 1) ^ gneg, flip1 = ((sf16 >> 15) & 1) ^ gneg;
  const float ag = fabsf(gs);
  const float a0 = mul_ro(e2m1_f32(max_mag(c[0], c[1])) * s0, ag);
  const float a1 = mul_ro(e2m1_f32(max_mag(c[2], c[3])) * s1, ag);
  const uint32_t am = bits(fmaxf(a0, a1));
  // amax = M * 2**E: smallest e with 6 * 2**e >= amax is E - 2 + (M > 1.5)
  int b = (int)(am >> 23) - 2 + ((am & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  b = am == 0 ? 0 : b;
  b = b < 0 ? 0 : (b > 254 ? 254 : b);
  const int e = b - 127;
  uint32_t l0, h0, l1, h1;
  half_lut(s0, ag, e, l0, h0);
  half_lut(s1, ag, e, l1, h1);
  out[0] = apply_lut(c[0], l0, h0, flip0 ? 0x88888888u : 0u);
  out[1] = apply_lut(c[1], l0, h0, flip0 ? 0x88888888u : 0u);
  out[2] = apply_lut(c[2], l1, h1, flip1 ? 0x88888888u : 0u);
  out[3] = apply_lut(c[3], l1, h1, flip1 ? 0x88888888u : 0u);
  return (uint32_t)b;
}

// ---------------------------------------------------------------------------
// Table-driven form used by the kernel.  Per expert, for every E4M3 byte b:
//   P1[b] = RO(|E4M3(b)| * |gs|),  P3[b] = RO(3 * |E4M3(b)| * |gs|)
// (RO = round to odd).  The odd-rounded value of E2M1(m) * |s| * |gs| is then
// a power-of-two multiple of P1 (m = 1, 2, 4, 6 -> 0.5, 1, 2, 4 x) or of P3
// (m = 3, 5, 7 -> 0.5, 1, 2 x), so the block maximum and every lookup-table
// entry come from two table reads and exact scalings.

MOEFP4_HD void ro_pair(uint32_t b, float ag, float& p1, float& p3) {
  const float s = fabsf(e4m3_f32(b));
  p1 = mul_ro(s, ag);
  p3 = mul_ro(3.0f * s, ag);
}

// odd-rounded E2M1(m) * |s| * |gs| for magnitude code m (0..7), branch-free:
// m = 1..7 -> {P1/2, P1, P3/2, 2 P1, P3, 4 P1, 2 P3}; m = 0 -> 0
MOEFP4_HD float ladder(uint32_t m, float p1, float p3) {
  const uint32_t use3 = (0xA8u >> m) & 1u;                       // m = 3, 5, 7
  const int k = (int)((0x23120101u >> (4 * m)) & 0xFu) - 1;      // exponent offset
  const float v = ldexpf(use3 ? p3 : p1, k);
  return m ? v : 0.0f;
}

// RNE code of x / 2**(e+1) on the E2M1 grid with saturation at 6 (the
// semantics of v_cvt_scalef32_pk_fp4_f32 with a power-of-two scale, which
// the kernel uses; this is the host equivalent).
MOEFP4_HD uint32_t code_scaled(float x, int e) { return e2m1_code(fminf(ldexpf(x, -e - 1), 6.0f)); }

MOEFP4_HD uint32_t requant_block_tab(const uint32_t c[4], uint32_t sf16, float p1a, float p3a,
                                     float p1b, float p3b, uint32_t gneg, uint32_t out[4]) {
  uint32_t lo[4], hi[4];
  for (int i = 0; i < 4; ++i) {
    lo[i] = c[i] & 0x07070707u;
    hi[i] = (c[i] >> 4) & 0x07070707u;
  }
  const uint32_t ohl = 0x08040201u, ohh = 0x80402010u;  // one-hot byte 1 << m
  uint32_t oa = perm8(ohh, ohl, lo[0]) | perm8(ohh, ohl, hi[0]) | perm8(ohh, ohl, lo[1]) |
                perm8(ohh, ohl, hi[1]);
  uint32_t ob = perm8(ohh, ohl, lo[2]) | perm8(ohh, ohl, hi[2]) | perm8(ohh, ohl, lo[3]) |
                perm8(ohh, ohl, hi[3]);
  oa |= oa >> 16;
  oa |= oa >> 8;
  ob |= ob >> 16;
  ob |= ob >> 8;
  const uint32_t ma = 31u - (uint32_t)clz32((oa & 0xFFu) | 1u);
  const uint32_t mb = 31u - (uint32_t)clz32((ob & 0xFFu) | 1u);
  const uint32_t am = bits(fmaxf(ladder(ma, p1a, p3a), ladder(mb, p1b, p3b)));
  int b = (int)(am >> 23) - 2 + ((am & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  b = am == 0 ? 0 : b;
  b = b < 0 ? 0 : (b > 254 ? 254 : b);
  const int e = b - 127;
  const int es = e > 126 ? 126 : e;  // the lookup tables' scaling exponent
  uint32_t la = 0, ha = 0, lb = 0, hb = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  const float sc = fbits((uint32_t)(es + 1 + 127) << 23);
  la = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(la, p1a, 0.0f, sc, 1);
  la = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(la, 2.0f * p1a, 0.0f, sc, 2);
  la = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(la, p3a, 0.0f, sc, 3);
  ha = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ha, 4.0f * p1a, 0.0f, sc, 0);
  ha = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ha, 2.0f * p3a, 0.0f, sc, 1);
  ha = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ha, 8.0f * p1a, 0.0f, sc, 2);
  ha = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(ha, 4.0f * p3a, 0.0f, sc, 3);
  lb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lb, p1b, 0.0f, sc, 1);
  lb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lb, 2.0f * p1b, 0.0f, sc, 2);
  lb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lb, p3b, 0.0f, sc, 3);
  hb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hb, 4.0f * p1b, 0.0f, sc, 0);
  hb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hb, 2.0f * p3b, 0.0f, sc, 1);
  hb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hb, 8.0f * p1b, 0.0f, sc, 2);
  hb = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hb, 4.0f * p3b, 0.0f, sc, 3);
#else
  la = (code_scaled(p1a, es) << 8) | (code_scaled(2.0f * p1a, es) << 16) | (code_scaled(p3a, es) << 24);
  ha = code_scaled(4.0f * p1a, es) | (code_scaled(2.0f * p3a, es) << 8) |
       (code_scaled(8.0f * p1a, es) << 16) | (code_scaled(4.0f * p3a, es) << 24);
  lb = (code_scaled(p1b, es) << 8) | (code_scaled(2.0f * p1b, es) << 16) | (code_scaled(p3b, es) << 24);
  hb = code_scaled(4.0f * p1b, es) | (code_scaled(2.0f * p3b, es) << 8) |
       (code_scaled(8.0f * p1b, es) << 16) | (code_scaled(4.0f * p3b, es) << 24);
#endif
  // sign: a negative block scale flips its half, a negative gs the block
  const uint32_t fa = ((((sf16 >> 7) & 1u) ^ gneg) ? 0x88888888u : 0u);
  const uint32_t fb = ((((sf16 >> 15) & 1u) ^ gneg) ? 0x88888888u : 0u);
  out[0] = ((c[0] & 0x88888888u) ^ fa) | perm8(ha, la, lo[0]) | (perm8(ha, la, hi[0]) << 4);
  out[1] = ((c[1] & 0x88888888u) ^ fa) | perm8(ha, la, lo[1]) | (perm8(ha, la, hi[1]) << 4);
  out[2] = ((c[2] & 0x88888888u) ^ fb) | perm8(hb, lb, lo[2]) | (perm8(hb, lb, hi[2]) << 4);
  out[3] = ((c[3] & 0x88888888u) ^ fb) | perm8(hb, lb, lo[3]) | (perm8(hb, lb, hi[3]) << 4);
  return (uint32_t)b;
}

}  // namespace rq
}  // namespace moefp4
