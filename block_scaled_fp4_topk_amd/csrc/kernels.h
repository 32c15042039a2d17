// Internal launcher interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moefp4 {

constexpr int kMaxExperts = 512;

// Tile of activation rows processed by one grouped-GEMM workgroup.
struct RouteOut {
  int32_t* counts;         // [E]
  int32_t* offsets;        // [E+1]
  int32_t* sorted_assign;  // [A]
  int32_t* slot_of;        // [A]
  int32_t* tiles;          // [2 * max_tiles] (expert, first row)
  int32_t* ntiles;         // [1]
  int32_t* flags;          // [1] dropped assignments
  uint32_t* zero_words;    // optional [n_zero] words cleared by the route kernel
  int n_zero;
  // optional: per-token fp16 staging scale of bf16 rows x [T, H] (row_scale
  // null: not computed); row_scale[t] = 2**p_t with p_t chosen so the row
  // maximum times 2**-p_t lies in [2**14, 2**15)
  const uint16_t* x;
  int T, H;
  float* row_scale;
  // optional (with row_scale): the rows themselves converted, fp16(x * 2**-p_t)
  // [T, H] (exact: 8 significant bits inside the fp16 range)
  uint16_t* x16;
  // optional: FP8 + UE8M0 per 32 quantisation of bf16 rows x [T, H] into
  // x8 [T, H] and xsf [T, H/32] (x8 null: not computed); x_fp4: MXFP4
  // (E2M1 + UE8M0 per 32) instead, x8 [T, H/2]
  uint8_t* x8;
  uint8_t* xsf;
  bool x_fp4;
  // multi-workgroup form (nchunks > 0): chunks of `chunk` assignments and a
  // [nchunks][E + 1] int32 scratch for their histograms / starts
  int nchunks, chunk;
  int32_t* hist;
};

// Assignments per chunk of the multi-workgroup route (T * k above
// kRouteSingleMax uses it).
constexpr int kRouteSingleMax = 8192;
inline int route_chunk(long long A) {
  long long c = (A + 63) / 64;
  c = (c + 1023) / 1024 * 1024;
  return (int)(c < 4096 ? 4096 : c);
}

hipError_t launch_route(const int32_t* topk_ids, int A, int E, int tile_m, const RouteOut& o,
                        hipStream_t s);

// bf16 [T, H] -> E4M3 [T, H] + UE8M0 [T, H/32]: per 32 elements e =
// ceil(log2(amax / 448)) (amax == 0: e = -127), clamped to [-127, 127],
// codes RNE(x / 2**e), sign kept.  fp4: MXFP4 instead, E2M1 [T, H/2] (two
// per byte, even element low) with e = ceil(log2(amax / 6)).  H % 32 == 0.
hipError_t launch_quantize_act(const uint16_t* x, long long T, int H, uint8_t* xq, uint8_t* xsf,
                               bool fp4, hipStream_t s);

// bf16 [T, H] -> fp16 [T, H] * 2**-p_t with p_t chosen per row so the row
// maximum lands in [2**14, 2**15); scale[t] = 2**p_t.
hipError_t launch_rows_to_f16(const uint16_t* x, int T, int H, uint16_t* x16, float* scale,
                              hipStream_t s);

struct FcArgs {
  const uint8_t* w;          // [E, N, K/2]
  const uint8_t* wsf;        // [E, N, K/gran]
  const float* gs;           // [E] or null
  const void* act;           // FC1: x or x16 [T, K]; FC2: h [A, K]
  const uint8_t* act_sf;     // A8: [rows, K/32] UE8M0
  const float* act_scale;    // A16 group16 FC1: per token 2**p
  const uint32_t* hmax_in;   // A16 group16 FC2: per slot max |h| bits
  const int32_t* tiles;
  const int32_t* ntiles;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* sorted_assign;
  int K, N, I, H, top_k, w13_order;
  void* h_out;               // FC1: h [A, I] (bf16 or fp8)
  uint8_t* h_sf_out;         // FC1 A8: [A, I/32]
  uint32_t* hmax_out;        // FC1 A16 group16: per slot max |h| bits
  float* y_out;              // FC2: [A, H]
};

// 64-row expert tiles (bf16 activations with more than 16 assignments per
// active expert, and FP8 activations at shapes the prefill GEMM does not take)
hipError_t launch_fc1_a16(const FcArgs& a, int gran, int max_tiles, hipStream_t s);
hipError_t launch_fc2_a16(const FcArgs& a, int gran, int max_tiles, hipStream_t s);
hipError_t launch_fc1_a8(const FcArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_fc2_a8(const FcArgs& a, int max_tiles, hipStream_t s);

// Decode-shaped FC kernels (expert tiles of <= 16 activation rows); mode 0:
// bf16 x group16, 1: bf16 x group32, 2: FP8 x group32, 3: MXFP4 x group32
// (act [rows, K/2], h written as MXFP4).  Needs K % 256 == 0,
// I % 64 == 0 (FC1) and H % 128 == 0 (FC2).
hipError_t launch_fc_decode(const FcArgs& a, int mode, bool fc1, int max_tiles, hipStream_t s);

// Single-launch decode (FC1 + SwiGLU + h quantisation, then FC2) in one
// persistent kernel.  Each expert tile's FC1 and FC2 items run on one XCD
// (tile t on XCD t % nx), taken from that XCD's queue in order (every FC1
// item before any FC2 item), so h passes from FC1 to FC2 through the XCD's
// own L2: an FC1 item waits for its stores and bumps done[t]; an FC2 item
// waits until done[t] counts every FC1 row block of its tile, then drops its
// CU's L1 lines.  queue [nx] and done [max_tiles] are zeroed by the route
// launch (which also clears *err); err counts waits that exceeded their
// time limit (the kernel then finishes with wrong results instead of
// hanging).
struct DecodeSync {
  int32_t* queue;
  int32_t* done;
  int32_t* err;
  int nx;            // XCDs (workgroups read their XCD id from the hardware)
  int nblk1, nblk2;  // FC1 / FC2 row blocks per tile
};
hipError_t launch_fc_decode_fused(const FcArgs& a1, const FcArgs& a2, int mode, const DecodeSync& y,
                                  hipStream_t s);
// words of the DecodeSync queue + done counters for max_tiles tiles
inline int decode_sync_words(int max_tiles) { return 8 + max_tiles; }
// XCDs of the current device (32 CUs each on MI355X), 1..8
int xcd_count();

// Prefill-shaped FP8 x FP4 grouped GEMMs on 128-row expert tiles (direct-
// to-LDS pipelined, 512 weight rows per work item); a4: MXFP4 activations
// (act [rows, K/2], h written as MXFP4).  Needs H % 512 == 0, I % 512 == 0
// and 32-bit row offsets.  prep: weights in the GEMM layout of
// launch_prepare_gemm.
hipError_t launch_fc_gemm_a8(const FcArgs& a, bool fc1, bool a4, bool prep, int max_tiles, hipStream_t s);

// RAW group32 weights [E, N, K/2] + [E, N, K/32] -> the GEMM layout of the
// prefill kernels (moe_fp4_prepare_gemm_weights); N, K multiples of 512,
// N * K / 32 < 2^31.
hipError_t launch_prepare_gemm(const uint8_t* src, const uint8_t* src_sf, uint8_t* dst, uint8_t* dst_sf,
                               int64_t E, int64_t N, int64_t K, bool w13, int w13_order, hipStream_t s);

// Group16 weights (E2M1 + E4M3 [E, N, K/16] + global scale gs [E] or null)
// -> the same GEMM layout with group32 UE8M0 scales, gs folded in
// (moe_fp4_prepare_gemm_weights_g16): bit-identical to launch_requant_g16_g32
// followed by launch_prepare_gemm.  N, K multiples of 512, N * K / 32 < 2^31.
hipError_t launch_requant_prepare_gemm(const uint8_t* src, const uint8_t* src_sf, const float* gs, uint8_t* dst,
                                       uint8_t* dst_sf, int64_t E, int64_t N, int64_t K, bool w13, int w13_order,
                                       hipStream_t s);

// out[t, :] = sum_j w[t, j] * y[slot_of[t*k + j], :]  (f32, or rounded to bf16)
hipError_t launch_combine(const float* y, const int32_t* slot_of, const float* topk_w, int T,
                          int k, int H, void* out, bool out_f32, hipStream_t s);

// Register-only loop of the block-scaled MFMA (FP4 x FP8, or FP4 x FP4 with
// a4): blocks x 4 waves x iters x 32 instructions of 2*16*16*128 flops.
hipError_t launch_mfma_peak(bool a4, int iters, int blocks, float* sink, hipStream_t s);

hipError_t launch_requant_g16_g32(const uint8_t* src, const uint8_t* src_sf, const float* gs,
                                  uint8_t* dst, uint8_t* dst_sf, int64_t E, int64_t N, int64_t K,
                                  hipStream_t s);

}  // namespace moefp4
