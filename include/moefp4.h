/*
 * moefp4 -- block-scaled FP4 top-k mixture-of-experts forward and
 * group16 -> group32 FP4 requantisation for AMD MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named as device memory must point to memory
 * allocated on the current HIP device; the library never allocates, frees or
 * synchronises on these calls, and all work is enqueued on the caller's
 * stream in order.  Host-side validation runs before any launch: a call that
 * returns an error status has enqueued nothing, and moefp4_last_error()
 * returns a message for it (thread-local, valid until the next call on the
 * same thread).
 *
 * Sources (the pages this library implements; cited by title and section):
 *  [P1] DeepGEMM commit log, branch "cch/deepgemm-glm52-nvfp4-group16":
 *       requant_fp4_to_gran_k with separate source/destination scale packing
 *       that recomputes UE8M0 scales; the explicit group16 capability gate of
 *       the fused FP8xFP4 compute.
 *  [P2] "GLM-5.2 NVFP4 group16 MegaMoE notes": sections Context (recipe
 *       (1, 1, 32), group_size=16 checkpoints), Current patch scope,
 *       Requantization path, Validation target.
 *  [P3] b12x moe/fused/w4a16/prepare.py: raw [E, N, K/2] packed FP4 weights,
 *       K/16 E4M3 block scales with a per-expert FP32 global scale
 *       (prepare_w4a16_modelopt_nvfp4_weights), K/32 E8M0 scales
 *       (prepare_w4a16_fp4_e8m0_k32_weights, _validate_e8m0_k32_scales),
 *       gate/up order of the fused W13 rows (_normalize_w13_layout), per-call
 *       buffers sized by tokens and top-k (make_w4a16_packed_buffers).
 *
 * Data layouts (row-major, K contiguous):
 *  FP4 tensor  [E, N, K/2] uint8, two E2M1 codes per byte, element 2j in the
 *              low nibble of byte j ([P3] _repack_4bit_no_perm reads a row as
 *              little-endian int32 words, element pos at shift 4*pos).
 *  scales      [E, N, K/gran] uint8: E4M3 (fn) for gran 16, UE8M0 for gran 32.
 *  global      [E] float32 multiplier per expert per tensor, or NULL.
 *              (compressed-tensors checkpoints store 1/gs: pass its inverse.)
 */
#ifndef MOEFP4_H
#define MOEFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moefp4_status {
  MOEFP4_OK = 0,
  MOEFP4_EINVAL = 1,        /* bad shape, pointer or argument */
  MOEFP4_EUNSUPPORTED = 2,  /* valid request this library does not compute */
  MOEFP4_EWORKSPACE = 3,    /* workspace missing or too small */
  MOEFP4_EHIP = 4           /* a HIP launch reported an error */
} moefp4_status;

/* Activation formats.
 * BF16: x [T, H] bfloat16.
 * FP8_UE8M0_K32: x [T, H] E4M3 (fn) bytes and x_sf [T, H/32] UE8M0 bytes,
 *   value = fp8 * 2**(sf - 127) -- the activation side of the FP8xFP4
 *   recipe (1, 1, 32) of [P2] Context.
 * BF16_QUANT_FP8_K32: x [T, H] bfloat16, quantised by the library to the
 *   FP8_UE8M0_K32 format (as moe_fp4_quantize_act) before the FP8xFP4
 *   computation; x_sf must be NULL.
 * FP4_UE8M0_K32 ("A4"): x [T, H/2] E2M1 codes, two per byte, element 2j in
 *   the low nibble of byte j, and x_sf [T, H/32] UE8M0 bytes, value = e2m1 *
 *   2**(sf - 127): MXFP4 activations for the FP4xFP4 path (the "A4 prefill"
 *   of [P3] prepare_w4a16_modelopt_native_weights, in the block-scaled form
 *   the matrix instruction consumes).  h is quantised the same way between
 *   FC1 and FC2.
 * BF16_QUANT_FP4_K32: x [T, H] bfloat16, quantised by the library to
 *   FP4_UE8M0_K32 (as moe_fp4_quantize_act_fp4); x_sf must be NULL. */
typedef enum moefp4_act_fmt {
  MOEFP4_ACT_BF16 = 0,
  MOEFP4_ACT_FP8_UE8M0_K32 = 1,
  MOEFP4_ACT_BF16_QUANT_FP8_K32 = 2,
  MOEFP4_ACT_FP4_UE8M0_K32 = 3,
  MOEFP4_ACT_BF16_QUANT_FP4_K32 = 4
} moefp4_act_fmt;

/* Order of the 2I rows of w13.  GATE_UP: rows [0, I) are the gate projection
 * (the kernel-native "w31"/"gate_up" of [P3] _normalize_w13_layout).
 * UP_GATE: rows [0, I) are the up projection ("w13"/"up_gate" checkpoint
 * order, which [P3] _prepare_w4a16_packed_weights handles as a row rotation
 * by I). */
typedef enum moefp4_w13_order { MOEFP4_GATE_UP = 0, MOEFP4_UP_GATE = 1 } moefp4_w13_order;

/* Output formats.  BF16: out [T, H] bfloat16, the FP32 result rounded to
 * nearest even.  F32: out [T, H] float32, the FP32-accumulated result itself
 * (the same value the BF16 output is rounded from). */
typedef enum moefp4_out_fmt { MOEFP4_OUT_BF16 = 0, MOEFP4_OUT_F32 = 1 } moefp4_out_fmt;

/* Weight layouts.  RAW: the [E, N, K/2] codes and [E, N, K/gran] scales
 * described at the top (the checkpoint layout of [P3]).  GEMM: the layout
 * moe_fp4_prepare_gemm_weights writes from RAW group32 weights: the same
 * bytes ordered as the prefill GEMM stages them, so that it reads every
 * weight stage with contiguous 1 KB loads.  The layout itself is this
 * library's (it follows its prefill kernel); the step is the counterpart of
 * the weight preparation of [P1] (prepare_fp4_weights_for_mega_moe turning
 * raw grouped FP4 weights and scales into the fused kernel's layouts, the
 * benchmark feeding both forms from the same raw tensors) and of [P3]
 * _repack_weight. */
typedef enum moefp4_w_layout { MOEFP4_W_RAW = 0, MOEFP4_W_GEMM = 1 } moefp4_w_layout;

/* Problem description.  T tokens, E experts, top_k experts per token,
 * H hidden size, I intermediate size (w13 has 2I rows), gran_k 16 or 32,
 * act_fmt (moefp4_act_fmt), w13_order (moefp4_w13_order), out_fmt
 * (moefp4_out_fmt), w_layout (moefp4_w_layout) of w13/w13_sf and w2/w2_sf. */
typedef struct moefp4_problem {
  int32_t T, E, top_k, H, I, gran_k, act_fmt, w13_order, out_fmt, w_layout;
} moefp4_problem;

/* Workspace size for moe_fp4_route / moe_fp4_forward on problem p.
 * Returns OK and writes *bytes, or EINVAL/EUNSUPPORTED for an invalid or
 * unsupported problem.  The workspace is caller-owned device memory (the
 * analogue of [P3] make_w4a16_packed_buffers and _make_workspace); its
 * first 4 bytes hold, after a call completes, the number of assignments
 * whose expert id was outside [0, E) and was therefore dropped. */
moefp4_status moe_fp4_workspace_bytes(const moefp4_problem* p, size_t* bytes);

/* Where a forward on problem p keeps, in its workspace, the intermediate h
 * that FC2 consumes (byte offsets from the workspace start): *h: h [A, I] in
 * expert-slot order, A = T * top_k -- bfloat16 for BF16 activations, E4M3
 * bytes for FP8 activations, two E2M1 codes per byte ([A, I/2], element 2j in
 * the low nibble of byte j) for FP4 activations; *h_sf: its UE8M0 scales
 * [A, I/32] (FP8 / FP4 activations; 0 otherwise); *slot_of: the int32 [A]
 * map from assignment t * top_k + j to its slot (-1: dropped).  After a
 * forward completes these regions hold the values of that call (the h
 * quantisation of SwiGLU's output: bf16 RNE, or E4M3 / E2M1 + UE8M0 per 32).
 * For tests and debugging of the quantisation decisions; EINVAL / EUNSUPPORTED
 * as moe_fp4_workspace_bytes. */
moefp4_status moe_fp4_workspace_offsets(const moefp4_problem* p, size_t* h, size_t* h_sf,
                                        size_t* slot_of);

/* Routing: groups the T*k assignments a = t*k + j by expert id, stably (ties
 * in a-order).  Device outputs: counts [E], offsets [E+1] (exclusive prefix,
 * offsets[E] = number of valid assignments), sorted_assign [T*k] (assignment
 * ids in expert order, -1 past offsets[E]), slot_of [T*k] (inverse: position
 * of assignment a in sorted_assign, -1 if dropped).  Ids outside [0, E) are
 * dropped and counted in the workspace's first word.
 * [P3] make_w4a16_packed_buffers sizes per-call buffers by tokens and top-k;
 * the grouping itself is the "top-k routed tokens gathered per expert" step
 * of the fused MoE. */
moefp4_status moe_fp4_route(const moefp4_problem* p, const int32_t* topk_ids,
                            int32_t* counts, int32_t* offsets,
                            int32_t* sorted_assign, int32_t* slot_of,
                            void* workspace, size_t ws_bytes, hipStream_t stream);

/* MoE forward: out[t] = sum_j topk_w[t, j] * FC2_e(SwiGLU(FC1_e(x[t]))),
 * e = topk_ids[t, j]; FC1 uses w13 [E, 2I, H/2] + w13_sf [E, 2I, H/gran]
 * (+ w13_gs [E]), FC2 uses w2 [E, H, I/2] + w2_sf [E, H, I/gran] (+ w2_gs),
 * SwiGLU h = silu(gate) * up; h is rounded to bfloat16 (BF16 activations) or
 * quantised per 32 elements to E4M3 + UE8M0 (FP8 activations) or to E2M1 +
 * UE8M0 (FP4 activations) before FC2; FP32 accumulation; out [T, H]
 * bfloat16 or float32 (p->out_fmt).
 * Supported: (BF16, gran 16), (BF16, gran 32), (FP8, gran 32), (FP4, gran
 * 32; H and I multiples of 512, the shapes of the FP8 / FP4 GEMM tiles).  FP8 or FP4 activations with group16 weights return
 * EUNSUPPORTED, like the capability gate on recipe (1, 1, 16) in [P1] / [P2]
 * Current patch scope.  Decode-shaped problems (at most 16 assignments per
 * active expert, run on 16-row tiles) need I*H below 2^31 and, for BF16
 * activations with group16 weights, T*H below 2^31 (the decode kernels
 * address an expert's weights and the fp16 copy of x with 32-bit offsets);
 * EUNSUPPORTED otherwise.
 * x_sf must be NULL for BF16 and non-NULL for FP8 / FP4.  All pointers device
 * memory; topk_ids [T, k] int32, topk_w [T, k] float32; x, x_sf, the weight
 * and scale tensors and out 16-byte aligned, the workspace 256-byte aligned
 * (EINVAL otherwise). */
moefp4_status moe_fp4_forward(const moefp4_problem* p,
                              const void* x, const uint8_t* x_sf,
                              const int32_t* topk_ids, const float* topk_w,
                              const uint8_t* w13, const uint8_t* w13_sf, const float* w13_gs,
                              const uint8_t* w2, const uint8_t* w2_sf, const float* w2_gs,
                              void* out, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* moe_fp4_forward with FC1 and FC2 in one persistent launch: the fused
 * form the pages set beside the baseline grouped GEMM ([P1] the commit that
 * updates the MegaMoE synthetic benchmark: baseline grouped GEMM and fused
 * MegaMoE fed from the same raw source tensors; [P2] Context: the fused
 * FP8xFP4 MegaMoE compute path).  Each expert tile's FC2 work waits, inside
 * the launch, for that tile's FC1 work on the same XCD (per-tile counters in
 * the workspace; h passes through the XCD's own L2).  Same arguments,
 * workspace size, arithmetic and result as moe_fp4_forward (bit-identical
 * output); runs only problems of the 16-row decode tiles (at most 16
 * assignments per active expert) and returns EUNSUPPORTED with a message
 * otherwise.  Slower than moe_fp4_forward on the measured decode shapes; it
 * exists as the single-launch form, not as the default.  If a wait of the
 * fused kernel ever exceeded its 50 ms limit, the workspace's second word is
 * nonzero and the result is not valid. */
moefp4_status moe_fp4_forward_fused(const moefp4_problem* p,
                                    const void* x, const uint8_t* x_sf,
                                    const int32_t* topk_ids, const float* topk_w,
                                    const uint8_t* w13, const uint8_t* w13_sf, const float* w13_gs,
                                    const uint8_t* w2, const uint8_t* w2_sf, const float* w2_gs,
                                    void* out, void* workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* moe_fp4_forward without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the workspace is a static device
 * array inside the library, 64 MiB per GPU (held from the library's load
 * until the process ends), which covers decode-sized problems (e.g. 256
 * tokens, top-8, H = 6144, I = 2048 needs 52 MiB with FP8 activations, 59
 * MiB with bf16 activations and group16 weights); a problem whose
 * workspace (moe_fp4_workspace_bytes) exceeds it returns MOEFP4_EWORKSPACE
 * with a message and enqueues nothing.  Arguments, layouts, supported
 * problems and errors otherwise as moe_fp4_forward; the result is bit-
 * identical to moe_fp4_forward's.  No allocation, no synchronisation.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (concurrent streams, or threads) race and must be serialised by the
 * caller; stream-ordered calls on one stream are safe.  The dropped-id count
 * of moe_fp4_workspace_bytes lands in the static array and is not reported. */
moefp4_status moe_fp4_forward_static(const moefp4_problem* p,
                                     const void* x, const uint8_t* x_sf,
                                     const int32_t* topk_ids, const float* topk_w,
                                     const uint8_t* w13, const uint8_t* w13_sf, const float* w13_gs,
                                     const uint8_t* w2, const uint8_t* w2_sf, const float* w2_gs,
                                     void* out, hipStream_t stream);

/* Reorder group32 weights (RAW layout, UE8M0 scales) into the GEMM layout
 * of the prefill kernels.  which = 0: w13 (N = 2I rows in w13_order, K =
 * H); which = 1: w2 (N = H, K = I).  The GEMM's weight rows are taken in
 * blocks of 512: block nb of w13 is gate rows [256 nb, 256 nb + 256) then
 * the matching up rows (w13_order says where in src they are); block nb of
 * w2 is rows [512 nb, 512 nb + 512).  With r(nb, i) the src row of the
 * block's i-th row:
 *   codes  dst[e][((nb * K/128 + s) * 2048 + j) * 16 + b] =
 *            src[e][r(nb, j >> 2)][64 s + 16 ((j & 3) ^ ((j >> 4) & 3)) + b]
 *          for K stage s (128 elements), slot j in [0, 2048), byte b < 16;
 *   scales dst_sf[e][((nb * K/512 + g) * 512 + i) * 16 + b] =
 *            src_sf[e][r(nb, i)][16 g + b]   for group g (512 elements).
 * dst and dst_sf have the sizes of src and src_sf.  Device memory, 16-byte
 * aligned, disjoint from each other and from src / src_sf (EINVAL
 * otherwise); N and K multiples of 512 (EINVAL otherwise).  A forward with
 * w_layout = GEMM reads these buffers where it runs the prefill GEMM (FP8 or
 * FP4 activations, group32, H and I multiples of 512, more than 16
 * assignments per active expert on average: T * top_k > 16 * min(T * top_k,
 * E)) and returns EUNSUPPORTED for other problems. */
moefp4_status moe_fp4_prepare_gemm_weights(int64_t E, int64_t N, int64_t K, int32_t which,
                                           int32_t w13_order, const uint8_t* src,
                                           const uint8_t* src_sf, uint8_t* dst, uint8_t* dst_sf,
                                           hipStream_t stream);

/* Group16 NVFP4 weights straight into the GEMM layout, in one pass: the
 * requantisation of fp4_requant_gran_k (dequantise with the group16 E4M3
 * scales and the per-expert global scale, UE8M0 e = ceil(log2(amax / 6)) per
 * block of 32, E2M1 RNE codes; the global scale folded in) written in the
 * layout of moe_fp4_prepare_gemm_weights.  The counterpart of the weight
 * preparation of [P1] that accepts raw grouped FP4 weights and scales and
 * performs the optional requantisation and the layout transform in one call
 * (prepare_fp4_weights_for_mega_moe).  Output bit-identical to
 * fp4_requant_gran_k followed by moe_fp4_prepare_gemm_weights.
 * src [E, N, K/2] uint8, src_sf [E, N, K/16] E4M3 bytes, src_gs [E] float32 or
 * NULL (1), dst [E, N, K/2] uint8, dst_sf [E, N, K/32] uint8 (UE8M0, GEMM
 * layout); which / w13_order as for moe_fp4_prepare_gemm_weights.  Device
 * memory, 16-byte aligned, pairwise disjoint (EINVAL otherwise); N and K
 * multiples of 512 (EINVAL otherwise).  The forward then takes dst / dst_sf
 * with gran_k = 32, w_layout = GEMM and no global scale. */
moefp4_status moe_fp4_prepare_gemm_weights_g16(int64_t E, int64_t N, int64_t K, int32_t which,
                                               int32_t w13_order, const uint8_t* src,
                                               const uint8_t* src_sf, const float* src_gs,
                                               uint8_t* dst, uint8_t* dst_sf, hipStream_t stream);

/* Requantise E x [N, K] FP4 from src_gran to dst_gran ([P2] Requantization
 * path; [P1] requant_fp4_to_gran_k): dequantise with the group16 E4M3 scales
 * and the optional per-expert global scale (src_gs [E] or NULL), then per
 * block of 32 K elements choose UE8M0 e = ceil(log2(amax / 6)) (the smallest
 * e with 6 * 2**e >= amax; byte 0 for an all-zero block) and round each value
 * / 2**e to the nearest E2M1 code, ties to the even code, sign kept.  The
 * global scale is folded into the result.  Bit-exact with the FP64
 * definition whenever |gs| * 2688 and the smallest nonzero |gs| * 2**-10 are
 * normal FP32 numbers.
 * src [E, N, K/2], src_sf [E, N, K/16], dst [E, N, K/2], dst_sf [E, N, K/32],
 * all device memory.  dst may equal src (in place); any other overlap among
 * the four buffers is EINVAL.  Only src_gran 16 -> dst_gran 32 is computed
 * (EUNSUPPORTED otherwise); K must be a multiple of 32. */
moefp4_status fp4_requant_gran_k(int64_t E, int64_t N, int64_t K,
                                 const uint8_t* src, const uint8_t* src_sf,
                                 int32_t src_gran, const float* src_gs,
                                 uint8_t* dst, uint8_t* dst_sf, int32_t dst_gran,
                                 hipStream_t stream);

/* Quantise bfloat16 activation rows to the FP8 activation format of recipe
 * (1, 1, 32) ([P2] Context): per row, per 32 consecutive elements, UE8M0
 * scale byte e + 127 with e the smallest integer such that 448 * 2**e >=
 * max |x| (a block of zeros gets byte 0; e clamped to [-127, 127]), and
 * E4M3 (fn) codes round-to-nearest-even of x / 2**e, the sign kept (also on
 * zero).  The same rule quantises h between FC1 and FC2 on the FP8 path.
 * x [T, H] bfloat16, x_fp8 [T, H] uint8, x_sf [T, H/32] uint8, all device
 * memory owned by the caller, x and x_fp8 16-byte aligned; H a positive
 * multiple of 32 (EINVAL otherwise).  Enqueued on `stream`.  NaN and
 * infinite inputs are outside the contract. */
moefp4_status moe_fp4_quantize_act(int64_t T, int64_t H, const void* x, uint8_t* x_fp8,
                                   uint8_t* x_sf, hipStream_t stream);

/* Quantise bfloat16 activation rows to the MXFP4 activation format
 * (FP4_UE8M0_K32): per row, per 32 consecutive elements, UE8M0 scale byte e
 * + 127 with e the smallest integer such that 6 * 2**e >= max |x| (a block
 * of zeros gets byte 0; e clamped to [-127, 127]), and E2M1 codes
 * round-to-nearest-even of x / 2**e, ties to the even code, the sign kept
 * (also on zero) -- the block rule of fp4_requant_gran_k ([P2]
 * Requantization path) applied to activations.  x [T, H] bfloat16, x_fp4
 * [T, H/2] uint8 (element 2j in the low nibble of byte j), x_sf [T, H/32]
 * uint8, all device memory owned by the caller, x and x_fp4 16-byte
 * aligned; H a positive multiple of 32 (EINVAL otherwise).  Enqueued on
 * `stream`.  NaN and infinite inputs are outside the contract. */
moefp4_status moe_fp4_quantize_act_fp4(int64_t T, int64_t H, const void* x, uint8_t* x_fp4,
                                       uint8_t* x_sf, hipStream_t stream);

/* Profiling hook.  With events non-NULL and n >= 6, each later
 * moe_fp4_forward call on this thread records, on its stream, events[0]
 * before routing, [1] after routing, [2] after the activation preparation
 * (group16 bf16 path; otherwise right after [1]), [3] after FC1 + SwiGLU,
 * [4] after FC2 and [5] after the combine -- the caller owns the events
 * (hipEventCreate) and may change the array between calls.  events = NULL
 * turns recording off.  n in 1..5 is EINVAL. */
moefp4_status moefp4_set_stage_events(hipEvent_t* events, int32_t n);

/* Measurement helper (not part of the forward): enqueues a register-only
 * loop of the block-scaled matrix instruction the prefill kernels issue
 * (v_mfma_scale_f32_16x16x128_f8f6f4; FP4 x FP8 operands, or FP4 x FP4 with
 * a4 != 0) on `blocks` workgroups of 4 waves (one per CU at a time), `iters`
 * x 64 instructions per wave (64 independent accumulators, the prefill
 * GEMM's stage), and writes the flop count it performs to *flops
 * (host); time it
 * with events on `stream` to get the instruction's delivered rate on this
 * GPU, the practical ceiling beside the published peak.  sink: device
 * memory of blocks * 256 floats (never written for valid operands). */
moefp4_status moefp4_mfma_peak_probe(int32_t a4, int32_t iters, int32_t blocks, float* sink, double* flops,
                                     hipStream_t stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* moefp4_last_error(void);

/* Library version string. */
const char* moefp4_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOEFP4_H */
