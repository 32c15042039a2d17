// C-ABI entry points of libmoefp4: argument validation, workspace planning
// and the launch sequence on the caller's stream.  No allocation, no
// synchronisation; every check runs before the first launch.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/moefp4.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t* g_stage_events = nullptr;


moefp4_status fail(moefp4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moefp4_status ok() {
  g_err.clear();
  return MOEFP4_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t flags, counts, offsets, sorted, slot_of, tiles, ntiles;
  size_t act_scale, x16, x8, x8_sf, sync, hmax, h, h_sf, y, route_hist, total;
  int sync_words, zero_words;  // decode: queue + done counters; + hmax words (all cleared by the route launch)
  int route_chunks, route_chunk;
  int tile_m, nt, max_tiles;
  bool a8, a4, quant_x, g16_a16;
};

moefp4_status check_problem(const moefp4_problem* p) {
  if (!p) return fail(MOEFP4_EINVAL, "problem is NULL");
  if (p->T < 0) return fail(MOEFP4_EINVAL, "T must be >= 0, got %d", p->T);
  if (p->E < 1 || p->E > moefp4::kMaxExperts)
    return fail(p->E < 1 ? MOEFP4_EINVAL : MOEFP4_EUNSUPPORTED, "E must be in [1, %d], got %d",
                moefp4::kMaxExperts, p->E);
  if (p->top_k < 1 || p->top_k > p->E)
    return fail(MOEFP4_EINVAL, "top_k must be in [1, E=%d], got %d", p->E, p->top_k);
  if (p->H <= 0 || p->I <= 0) return fail(MOEFP4_EINVAL, "H and I must be positive");
  if (p->gran_k != 16 && p->gran_k != 32)
    return fail(MOEFP4_EINVAL, "gran_k must be 16 or 32, got %d", p->gran_k);
  if (p->act_fmt < MOEFP4_ACT_BF16 || p->act_fmt > MOEFP4_ACT_BF16_QUANT_FP4_K32)
    return fail(MOEFP4_EINVAL, "unknown act_fmt %d", p->act_fmt);
  if (p->w13_order != MOEFP4_GATE_UP && p->w13_order != MOEFP4_UP_GATE)
    return fail(MOEFP4_EINVAL, "unknown w13_order %d", p->w13_order);
  if (p->out_fmt != MOEFP4_OUT_BF16 && p->out_fmt != MOEFP4_OUT_F32)
    return fail(MOEFP4_EINVAL, "unknown out_fmt %d", p->out_fmt);
  if (p->w_layout != MOEFP4_W_RAW && p->w_layout != MOEFP4_W_GEMM)
    return fail(MOEFP4_EINVAL, "unknown w_layout %d", p->w_layout);
  if (p->H % 32 || p->I % 32)
    return fail(MOEFP4_EINVAL, "H and I must be multiples of 32 (K blocks of the scale grid), got H=%d I=%d",
                p->H, p->I);
  if (p->act_fmt != MOEFP4_ACT_BF16 && p->gran_k == 16)
    return fail(MOEFP4_EUNSUPPORTED,
                "FP8 / FP4 activations with group16 weights (recipe (1,1,16)) are not computed: requantise "
                "the weights to group32 with fp4_requant_gran_k");
  if (p->H % 256 || p->I % 256)
    return fail(MOEFP4_EUNSUPPORTED, "this build tiles K in chunks of 256: H and I must be multiples of 256, got H=%d I=%d",
                p->H, p->I);
  const long long A = (long long)p->T * p->top_k;
  if (A > (1LL << 26)) return fail(MOEFP4_EUNSUPPORTED, "T*top_k = %lld exceeds 2^26", A);
  if (p->act_fmt == MOEFP4_ACT_FP4_UE8M0_K32 || p->act_fmt == MOEFP4_ACT_BF16_QUANT_FP4_K32) {
    // FP4 activations beyond decode sizes run on the 128-row GEMM tiles only
    if (p->H % 512 || p->I % 512)
      return fail(MOEFP4_EUNSUPPORTED, "FP4 activations need H and I multiples of 512, got H=%d I=%d", p->H,
                  p->I);
    if ((long long)p->T * p->H >= (1LL << 31) || A * p->I >= (1LL << 31) ||
        (long long)p->I * p->H >= (1LL << 31))
      return fail(MOEFP4_EUNSUPPORTED, "FP4 activations need T*H, T*top_k*I and I*H below 2^31");
  }
  return MOEFP4_OK;
}

moefp4_status plan(const moefp4_problem* p, Layout* L) {
  moefp4_status st = check_problem(p);
  if (st != MOEFP4_OK) return st;
  const size_t A = (size_t)p->T * p->top_k, E = p->E, T = p->T, H = p->H, I = p->I;
  L->a4 = p->act_fmt == MOEFP4_ACT_FP4_UE8M0_K32 || p->act_fmt == MOEFP4_ACT_BF16_QUANT_FP4_K32;
  L->quant_x = p->act_fmt == MOEFP4_ACT_BF16_QUANT_FP8_K32 || p->act_fmt == MOEFP4_ACT_BF16_QUANT_FP4_K32;
  // a8: block-scaled activations (FP8 or FP4) with h quantised the same way
  L->a8 = p->act_fmt != MOEFP4_ACT_BF16;
  L->g16_a16 = !L->a8 && p->gran_k == 16;
  const size_t active = A < E ? A : E;
  const double avg = active ? (double)A / (double)active : 0.0;
  // 16-row tiles for decode-shaped routing; 128-row tiles for the FP8 x FP4
  // prefill GEMM (needs 32-bit row offsets and its row-block shapes); else
  // 64-row tiles
  const bool gemm_ok = L->a8 && I % 512 == 0 && H % 512 == 0 &&
                       T * H < (1ull << 31) &&
                       A * I < (1ull << 31) && I * H < (1ull << 31);
  L->nt = avg > 16.0 ? (gemm_ok ? 8 : 4) : 1;
  // the decode kernels address an expert's weights and the fp16 rows of x
  // with 32-bit offsets
  if (L->nt == 1 && (I * H >= (1ull << 31) || (L->g16_a16 && T * H >= (1ull << 31))))
    return fail(MOEFP4_EUNSUPPORTED,
                "decode-shaped problem too large for the 16-row tiles: needs I*H and (16-bit activations with "
                "group16 weights) T*H below 2^31, got I*H=%zu T*H=%zu",
                I * H, T * H);
  if (p->w_layout == MOEFP4_W_GEMM && L->nt != 8)
    return fail(MOEFP4_EUNSUPPORTED,
                "GEMM-layout weights are read by the prefill GEMM only (FP8 / FP4 activations, group32, H and "
                "I multiples of 512, more than 16 assignments per active expert); this problem runs on the %s "
                "tiles: pass RAW weights",
                L->nt == 1 ? "16-row decode" : "64-row");
  L->tile_m = 16 * L->nt;
  L->max_tiles = (int)(A / L->tile_m + active);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
  L->flags = take(64);
  L->counts = take(E * 4);
  L->offsets = take((E + 1) * 4);
  L->sorted = take(A * 4);
  L->slot_of = take(A * 4);
  L->tiles = take((size_t)L->max_tiles * 8);
  L->ntiles = take(4);
  L->act_scale = take(L->g16_a16 ? T * 4 : 0);
  L->x16 = take(L->g16_a16 ? T * H * 2 : 0);
  L->x8 = take(L->quant_x ? (L->a4 ? T * H / 2 : T * H) : 0);
  L->x8_sf = take(L->quant_x ? T * (H / 32) : 0);
  // the single-launch decode kernel's counters, then the per-slot h maxima
  // (group16 with bf16 x): one region the route launch clears
  L->sync_words = L->nt == 1 ? moefp4::decode_sync_words(L->max_tiles) : 0;
  L->zero_words = L->sync_words + (L->g16_a16 ? (int)A : 0);
  L->sync = take((size_t)L->zero_words * 4);
  L->hmax = L->sync + (size_t)L->sync_words * 4;
  L->h = take(L->a4 ? A * I / 2 : L->a8 ? A * I : A * I * 2);
  L->h_sf = take(L->a8 ? A * (I / 32) : 0);
  L->y = take(A * H * 4);
  L->route_chunks = 0;
  L->route_chunk = 0;
  if ((long long)A > moefp4::kRouteSingleMax) {
    L->route_chunk = moefp4::route_chunk((long long)A);
    L->route_chunks = (int)((A + L->route_chunk - 1) / L->route_chunk);
  }
  L->route_hist = take((size_t)L->route_chunks * (E + 1) * 4);
  L->total = o;
  return MOEFP4_OK;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

bool misaligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; }

moefp4_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOEFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MOEFP4_OK;
}

// stage boundary events of moefp4_set_stage_events (timing only)
moefp4_status stage_mark(int i, hipStream_t s) {
  return g_stage_events ? hip_status(hipEventRecord(g_stage_events[i], s), "stage event")
                        : MOEFP4_OK;
}

moefp4_status route_into(const moefp4_problem* p, const Layout& L, const int32_t* ids,
                         int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* slot_of,
                         void* ws, uint32_t* zero_words, int n_zero, const void* x, float* row_scale,
                         uint16_t* x16, uint8_t* x8, uint8_t* x8_sf, hipStream_t s) {
  moefp4::RouteOut o;
  o.counts = counts;
  o.offsets = offsets;
  o.sorted_assign = sorted;
  o.slot_of = slot_of;
  o.tiles = at<int32_t>(ws, L.tiles);
  o.ntiles = at<int32_t>(ws, L.ntiles);
  o.flags = at<int32_t>(ws, L.flags);
  o.zero_words = zero_words;
  o.n_zero = n_zero;
  o.x = static_cast<const uint16_t*>(x);
  o.T = p->T;
  o.H = p->H;
  o.row_scale = row_scale;
  o.x16 = x16;
  o.x8 = x8;
  o.xsf = x8_sf;
  o.x_fp4 = L.a4;
  o.nchunks = L.route_chunks;
  o.chunk = L.route_chunk;
  o.hist = L.route_chunks ? at<int32_t>(ws, L.route_hist) : nullptr;
  return hip_status(moefp4::launch_route(ids, p->T * p->top_k, p->E, L.tile_m, o, s), "route");
}

// The scratch of moe_fp4_forward_static: a file-scope device array, one copy
// per GPU, that holds the forward's workspace for callers that cannot
// allocate.  Host code uses only the per-device address hipGetSymbolAddress
// returns for it (the array's name is not a device address on the host).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the scratch array (resolved once per device, with
// that device current).
moefp4_status static_scratch(void** ptr) {
  int dev = -1;
  moefp4_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != MOEFP4_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(MOEFP4_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != MOEFP4_OK) return st;
    if (!p) return fail(MOEFP4_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOEFP4_OK;
}

}  // namespace

namespace {

// The forward; fused: FC1 and FC2 in one persistent launch (16-row decode
// tiles only, checked by the caller).
moefp4_status forward_impl(const moefp4_problem* p, const Layout& L, const void* x, const uint8_t* x_sf,
                           const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                           const uint8_t* w13_sf, const float* w13_gs, const uint8_t* w2,
                           const uint8_t* w2_sf, const float* w2_gs, void* out, void* workspace,
                           size_t ws_bytes, bool fused, hipStream_t stream) {
  moefp4_status st = MOEFP4_OK;
  if (p->T == 0) return ok();
  if (!x || !topk_ids || !topk_w || !w13 || !w13_sf || !w2 || !w2_sf || !out)
    return fail(MOEFP4_EINVAL, "x, topk_ids, topk_w, w13, w13_sf, w2, w2_sf and out must be non-NULL");
  if (L.a8 && !L.quant_x && !x_sf) return fail(MOEFP4_EINVAL, "FP8 / FP4 activations need x_sf");
  if ((!L.a8 || L.quant_x) && x_sf)
    return fail(MOEFP4_EINVAL, "x_sf must be NULL for bfloat16 activations");
  if (misaligned(x, 16) || misaligned(w13, 16) || misaligned(w2, 16) || misaligned(out, 16) ||
      misaligned(w13_sf, 16) || misaligned(w2_sf, 16) || (x_sf && misaligned(x_sf, 16)))
    return fail(MOEFP4_EINVAL, "x, x_sf, w13, w13_sf, w2, w2_sf and out must be 16-byte aligned");
  if (!workspace || ws_bytes < L.total)
    return fail(MOEFP4_EWORKSPACE, "workspace of %zu bytes needed, got %zu", L.total,
                workspace ? ws_bytes : (size_t)0);
  if (misaligned(workspace, 256)) return fail(MOEFP4_EINVAL, "workspace must be 256-byte aligned");

  const int A = p->T * p->top_k;
  int32_t* counts = at<int32_t>(workspace, L.counts);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted = at<int32_t>(workspace, L.sorted);
  int32_t* slot_of = at<int32_t>(workspace, L.slot_of);
  uint32_t* hmax = L.g16_a16 ? at<uint32_t>(workspace, L.hmax) : nullptr;
  uint32_t* zero = L.zero_words ? at<uint32_t>(workspace, L.sync) : nullptr;
  if ((st = stage_mark(0, stream)) != MOEFP4_OK) return st;
  // group16 weights with bf16 x on 16-row tiles: the route launch also
  // computes the per-token fp16 staging scales and writes the rows converted
  // with them, which FC1 copies straight to LDS
  const bool stage_f16 = L.g16_a16 && L.nt == 1;
  float* xs = L.g16_a16 ? at<float>(workspace, L.act_scale) : nullptr;
  uint16_t* x16 = L.g16_a16 ? at<uint16_t>(workspace, L.x16) : nullptr;
  // bf16 x to be quantised to FP8 or MXFP4 (+ UE8M0 per 32): also done by
  // the route launch, into the workspace
  uint8_t* x8 = L.quant_x ? at<uint8_t>(workspace, L.x8) : nullptr;
  uint8_t* x8_sf = L.quant_x ? at<uint8_t>(workspace, L.x8_sf) : nullptr;
  st = route_into(p, L, topk_ids, counts, offsets, sorted, slot_of, workspace, zero,
                  L.zero_words, (stage_f16 || L.quant_x) ? x : nullptr,
                  stage_f16 ? xs : nullptr, stage_f16 ? x16 : nullptr, x8, x8_sf, stream);
  if (st != MOEFP4_OK) return st;
  if ((st = stage_mark(1, stream)) != MOEFP4_OK) return st;

  moefp4::FcArgs a;
  memset(&a, 0, sizeof a);
  a.tiles = at<int32_t>(workspace, L.tiles);
  a.ntiles = at<int32_t>(workspace, L.ntiles);
  a.counts = counts;
  a.offsets = offsets;
  a.sorted_assign = sorted;
  a.I = p->I;
  a.H = p->H;
  a.top_k = p->top_k;
  a.w13_order = p->w13_order;

  // FC1 + SwiGLU (+ h quantisation)
  a.w = w13;
  a.wsf = w13_sf;
  a.gs = w13_gs;
  a.K = p->H;
  a.N = 2 * p->I;
  a.h_out = at<void>(workspace, L.h);
  if (L.a8) {
    a.act = L.quant_x ? x8 : x;
    a.act_sf = L.quant_x ? x8_sf : x_sf;
    a.h_sf_out = at<uint8_t>(workspace, L.h_sf);
  } else if (stage_f16) {
    a.act = x16;
    a.act_scale = xs;
    a.hmax_out = hmax;
  } else if (L.g16_a16) {
    st = hip_status(moefp4::launch_rows_to_f16(static_cast<const uint16_t*>(x), p->T, p->H, x16, xs, stream),
                    "rows_to_f16");
    if (st != MOEFP4_OK) return st;
    a.act = x16;
    a.act_scale = xs;
    a.hmax_out = hmax;
  } else {
    a.act = x;
  }
  // FC2
  moefp4::FcArgs b = a;
  b.w = w2;
  b.wsf = w2_sf;
  b.gs = w2_gs;
  b.K = p->I;
  b.N = p->H;
  b.act = at<void>(workspace, L.h);
  b.act_sf = L.a8 ? at<uint8_t>(workspace, L.h_sf) : nullptr;
  b.act_scale = nullptr;
  b.hmax_in = hmax;
  b.hmax_out = nullptr;
  b.h_out = nullptr;
  b.h_sf_out = nullptr;
  b.y_out = at<float>(workspace, L.y);
  const int mode = L.a4 ? 3 : L.a8 ? 2 : (p->gran_k == 16 ? 0 : 1);
  if ((st = stage_mark(2, stream)) != MOEFP4_OK) return st;
  if (fused) {
    // FC1 and FC2 in one persistent launch (16-row decode tiles)
    moefp4::DecodeSync y;
    y.queue = at<int32_t>(workspace, L.sync);
    y.done = y.queue + 8;
    y.err = at<int32_t>(workspace, L.flags) + 1;
    y.nx = moefp4::xcd_count();
    y.nblk1 = p->I / 64;
    y.nblk2 = p->H / 128;
    st = hip_status(moefp4::launch_fc_decode_fused(a, b, mode, y, stream), "fc1+fc2");
    if (st != MOEFP4_OK) return st;
    if ((st = stage_mark(3, stream)) != MOEFP4_OK) return st;
  } else {
    st = hip_status(L.nt == 1   ? moefp4::launch_fc_decode(a, mode, true, L.max_tiles, stream)
                    : L.nt == 8 ? moefp4::launch_fc_gemm_a8(a, true, L.a4, p->w_layout == MOEFP4_W_GEMM,
                                                            L.max_tiles, stream)
                    : L.a8      ? moefp4::launch_fc1_a8(a, L.max_tiles, stream)
                                : moefp4::launch_fc1_a16(a, p->gran_k, L.max_tiles, stream),
                    "fc1");
    if (st != MOEFP4_OK) return st;
    if ((st = stage_mark(3, stream)) != MOEFP4_OK) return st;
    st = hip_status(L.nt == 1   ? moefp4::launch_fc_decode(b, mode, false, L.max_tiles, stream)
                    : L.nt == 8 ? moefp4::launch_fc_gemm_a8(b, false, L.a4, p->w_layout == MOEFP4_W_GEMM,
                                                            L.max_tiles, stream)
                    : L.a8      ? moefp4::launch_fc2_a8(b, L.max_tiles, stream)
                                : moefp4::launch_fc2_a16(b, p->gran_k, L.max_tiles, stream),
                    "fc2");
    if (st != MOEFP4_OK) return st;
  }
  if ((st = stage_mark(4, stream)) != MOEFP4_OK) return st;

  st = hip_status(moefp4::launch_combine(b.y_out, slot_of, topk_w, p->T, p->top_k, p->H, out,
                                         p->out_fmt == MOEFP4_OUT_F32, stream),
                  "combine");
  if (st != MOEFP4_OK) return st;
  if ((st = stage_mark(5, stream)) != MOEFP4_OK) return st;
  return ok();
}

}  // namespace

extern "C" {

moefp4_status moe_fp4_workspace_bytes(const moefp4_problem* p, size_t* bytes) {
  if (!bytes) return fail(MOEFP4_EINVAL, "bytes is NULL");
  Layout L;
  moefp4_status st = plan(p, &L);
  if (st != MOEFP4_OK) return st;
  *bytes = L.total;
  return ok();
}

moefp4_status moe_fp4_workspace_offsets(const moefp4_problem* p, size_t* h, size_t* h_sf, size_t* slot_of) {
  if (!h || !h_sf || !slot_of) return fail(MOEFP4_EINVAL, "h, h_sf and slot_of must be non-NULL");
  Layout L;
  moefp4_status st = plan(p, &L);
  if (st != MOEFP4_OK) return st;
  *h = L.h;
  *h_sf = L.a8 ? L.h_sf : 0;
  *slot_of = L.slot_of;
  return ok();
}

moefp4_status moe_fp4_route(const moefp4_problem* p, const int32_t* topk_ids, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_assign, int32_t* slot_of,
                            void* workspace, size_t ws_bytes, hipStream_t stream) {
  Layout L;
  moefp4_status st = plan(p, &L);
  if (st != MOEFP4_OK) return st;
  if (p->T > 0 && (!topk_ids || !sorted_assign || !slot_of))
    return fail(MOEFP4_EINVAL, "topk_ids, sorted_assign and slot_of must be non-NULL");
  if (!counts || !offsets) return fail(MOEFP4_EINVAL, "counts and offsets must be non-NULL");
  if (!workspace || ws_bytes < L.total)
    return fail(MOEFP4_EWORKSPACE, "workspace of %zu bytes needed, got %zu", L.total,
                workspace ? ws_bytes : (size_t)0);
  st = route_into(p, L, topk_ids, counts, offsets, sorted_assign, slot_of, workspace, nullptr, 0,
                  nullptr, nullptr, nullptr, nullptr, nullptr, stream);
  return st == MOEFP4_OK ? ok() : st;
}

moefp4_status moe_fp4_forward(const moefp4_problem* p, const void* x, const uint8_t* x_sf,
                              const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                              const uint8_t* w13_sf, const float* w13_gs, const uint8_t* w2,
                              const uint8_t* w2_sf, const float* w2_gs, void* out,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  Layout L;
  moefp4_status st = plan(p, &L);
  if (st != MOEFP4_OK) return st;
  return forward_impl(p, L, x, x_sf, topk_ids, topk_w, w13, w13_sf, w13_gs, w2, w2_sf, w2_gs, out, workspace,
                      ws_bytes, false, stream);
}

moefp4_status moe_fp4_forward_fused(const moefp4_problem* p, const void* x, const uint8_t* x_sf,
                                    const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                                    const uint8_t* w13_sf, const float* w13_gs, const uint8_t* w2,
                                    const uint8_t* w2_sf, const float* w2_gs, void* out, void* workspace,
                                    size_t ws_bytes, hipStream_t stream) {
  Layout L;
  moefp4_status st = plan(p, &L);
  if (st != MOEFP4_OK) return st;
  if (L.nt != 1)
    return fail(MOEFP4_EUNSUPPORTED,
                "the single-launch forward runs the 16-row decode tiles only (at most 16 assignments per active "
                "expert); this problem runs on the %s tiles: use moe_fp4_forward",
                L.nt == 8 ? "128-row GEMM" : "64-row");
  return forward_impl(p, L, x, x_sf, topk_ids, topk_w, w13, w13_sf, w13_gs, w2, w2_sf, w2_gs, out, workspace,
                      ws_bytes, true, stream);
}

moefp4_status moe_fp4_forward_static(const moefp4_problem* p, const void* x, const uint8_t* x_sf,
                                     const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                                     const uint8_t* w13_sf, const float* w13_gs, const uint8_t* w2,
                                     const uint8_t* w2_sf, const float* w2_gs, void* out, hipStream_t stream) {
  Layout L;
  moefp4_status st = plan(p, &L);
  if (st != MOEFP4_OK) return st;
  if (L.total > kStaticScratchBytes)
    return fail(MOEFP4_EWORKSPACE,
                "this problem needs %zu bytes of scratch; the static scratch of moe_fp4_forward_static holds %zu "
                "(use moe_fp4_forward with a caller workspace)",
                L.total, kStaticScratchBytes);
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != MOEFP4_OK) return st;
  return moe_fp4_forward(p, x, x_sf, topk_ids, topk_w, w13, w13_sf, w13_gs, w2, w2_sf, w2_gs, out, ws,
                         kStaticScratchBytes, stream);
}

moefp4_status fp4_requant_gran_k(int64_t E, int64_t N, int64_t K, const uint8_t* src,
                                 const uint8_t* src_sf, int32_t src_gran, const float* src_gs,
                                 uint8_t* dst, uint8_t* dst_sf, int32_t dst_gran,
                                 hipStream_t stream) {
  if (E < 0 || N < 0 || K < 0) return fail(MOEFP4_EINVAL, "E, N, K must be >= 0");
  if ((src_gran != 16 && src_gran != 32) || (dst_gran != 16 && dst_gran != 32))
    return fail(MOEFP4_EINVAL, "granularities must be 16 or 32, got %d -> %d", src_gran, dst_gran);
  if (src_gran != 16 || dst_gran != 32)
    return fail(MOEFP4_EUNSUPPORTED, "only group16 -> group32 requantisation is computed, got %d -> %d",
                src_gran, dst_gran);
  if (K % 32) return fail(MOEFP4_EINVAL, "K must be a multiple of 32, got %lld", (long long)K);
  if (N * (K / 32) > (int64_t)1 << 30 || E > 65535)
    return fail(MOEFP4_EUNSUPPORTED, "N*K/32 must be <= 2^30 and E <= 65535");
  const int64_t n = E * N * K;
  if (n == 0) return ok();
  if (!src || !src_sf || !dst || !dst_sf)
    return fail(MOEFP4_EINVAL, "src, src_sf, dst and dst_sf must be non-NULL");
  if (misaligned(src, 16) || misaligned(dst, 16) || misaligned(src_sf, 8) || misaligned(dst_sf, 4))
    return fail(MOEFP4_EINVAL, "src/dst must be 16-byte aligned, src_sf 8-byte, dst_sf 4-byte");
  // overlap rules: dst == src allowed; everything else disjoint
  struct R { uintptr_t b, e; } r[4] = {
      {(uintptr_t)src, (uintptr_t)src + (uintptr_t)(n / 2)},
      {(uintptr_t)src_sf, (uintptr_t)src_sf + (uintptr_t)(n / 16)},
      {(uintptr_t)dst, (uintptr_t)dst + (uintptr_t)(n / 2)},
      {(uintptr_t)dst_sf, (uintptr_t)dst_sf + (uintptr_t)(n / 32)}};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j) {
      if (i == 0 && j == 2 && src == dst) continue;
      if (r[i].b < r[j].e && r[j].b < r[i].e)
        return fail(MOEFP4_EINVAL, "buffers overlap (only dst == src is allowed)");
    }
  moefp4_status st = hip_status(
      moefp4::launch_requant_g16_g32(src, src_sf, src_gs, dst, dst_sf, E, N, K, stream), "requant");
  return st == MOEFP4_OK ? ok() : st;
}

moefp4_status moe_fp4_prepare_gemm_weights(int64_t E, int64_t N, int64_t K, int32_t which,
                                           int32_t w13_order, const uint8_t* src, const uint8_t* src_sf,
                                           uint8_t* dst, uint8_t* dst_sf, hipStream_t stream) {
  if (E < 0 || N < 0 || K < 0) return fail(MOEFP4_EINVAL, "E, N, K must be >= 0");
  if (which != 0 && which != 1) return fail(MOEFP4_EINVAL, "which must be 0 (w13) or 1 (w2), got %d", which);
  if (w13_order != MOEFP4_GATE_UP && w13_order != MOEFP4_UP_GATE)
    return fail(MOEFP4_EINVAL, "unknown w13_order %d", w13_order);
  if (N % 512 || K % 512)
    return fail(MOEFP4_EINVAL, "N and K must be multiples of 512, got N=%lld K=%lld", (long long)N,
                (long long)K);
  if (N * K / 32 >= ((int64_t)1 << 31) || E > 65535)
    return fail(MOEFP4_EUNSUPPORTED, "N*K/32 must be below 2^31 and E <= 65535");
  const int64_t n = E * N * K;
  if (n == 0) return ok();
  if (!src || !src_sf || !dst || !dst_sf)
    return fail(MOEFP4_EINVAL, "src, src_sf, dst and dst_sf must be non-NULL");
  if (misaligned(src, 16) || misaligned(dst, 16) || misaligned(src_sf, 16) || misaligned(dst_sf, 16))
    return fail(MOEFP4_EINVAL, "src, src_sf, dst and dst_sf must be 16-byte aligned");
  struct R { uintptr_t b, e; } r[4] = {
      {(uintptr_t)src, (uintptr_t)src + (uintptr_t)(n / 2)},
      {(uintptr_t)src_sf, (uintptr_t)src_sf + (uintptr_t)(n / 32)},
      {(uintptr_t)dst, (uintptr_t)dst + (uintptr_t)(n / 2)},
      {(uintptr_t)dst_sf, (uintptr_t)dst_sf + (uintptr_t)(n / 32)}};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (r[i].b < r[j].e && r[j].b < r[i].e) return fail(MOEFP4_EINVAL, "buffers overlap");
  moefp4_status st = hip_status(
      moefp4::launch_prepare_gemm(src, src_sf, dst, dst_sf, E, N, K, which == 0, w13_order, stream),
      "prepare_gemm_weights");
  return st == MOEFP4_OK ? ok() : st;
}

moefp4_status moe_fp4_prepare_gemm_weights_g16(int64_t E, int64_t N, int64_t K, int32_t which,
                                               int32_t w13_order, const uint8_t* src, const uint8_t* src_sf,
                                               const float* src_gs, uint8_t* dst, uint8_t* dst_sf,
                                               hipStream_t stream) {
  if (E < 0 || N < 0 || K < 0) return fail(MOEFP4_EINVAL, "E, N, K must be >= 0");
  if (which != 0 && which != 1) return fail(MOEFP4_EINVAL, "which must be 0 (w13) or 1 (w2), got %d", which);
  if (w13_order != MOEFP4_GATE_UP && w13_order != MOEFP4_UP_GATE)
    return fail(MOEFP4_EINVAL, "unknown w13_order %d", w13_order);
  if (N % 512 || K % 512)
    return fail(MOEFP4_EINVAL, "N and K must be multiples of 512, got N=%lld K=%lld", (long long)N,
                (long long)K);
  if (N * K / 32 >= ((int64_t)1 << 31) || E > 65535)
    return fail(MOEFP4_EUNSUPPORTED, "N*K/32 must be below 2^31 and E <= 65535");
  const int64_t n = E * N * K;
  if (n == 0) return ok();
  if (!src || !src_sf || !dst || !dst_sf)
    return fail(MOEFP4_EINVAL, "src, src_sf, dst and dst_sf must be non-NULL");
  if (misaligned(src, 16) || misaligned(dst, 16) || misaligned(src_sf, 16) || misaligned(dst_sf, 16))
    return fail(MOEFP4_EINVAL, "src, src_sf, dst and dst_sf must be 16-byte aligned");
  struct R { uintptr_t b, e; } r[4] = {
      {(uintptr_t)src, (uintptr_t)src + (uintptr_t)(n / 2)},
      {(uintptr_t)src_sf, (uintptr_t)src_sf + (uintptr_t)(n / 16)},
      {(uintptr_t)dst, (uintptr_t)dst + (uintptr_t)(n / 2)},
      {(uintptr_t)dst_sf, (uintptr_t)dst_sf + (uintptr_t)(n / 32)}};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (r[i].b < r[j].e && r[j].b < r[i].e) return fail(MOEFP4_EINVAL, "buffers overlap");
  moefp4_status st = hip_status(moefp4::launch_requant_prepare_gemm(src, src_sf, src_gs, dst, dst_sf, E, N, K,
                                                                    which == 0, w13_order, stream),
                                "prepare_gemm_weights_g16");
  return st == MOEFP4_OK ? ok() : st;
}

moefp4_status moe_fp4_quantize_act(int64_t T, int64_t H, const void* x, uint8_t* x_fp8,
                                   uint8_t* x_sf, hipStream_t stream) {
  if (T < 0 || H <= 0 || H % 32) return fail(MOEFP4_EINVAL, "need T >= 0 and H a positive multiple of 32, got T=%lld H=%lld", (long long)T, (long long)H);
  if (H > (1 << 30) || T > (1ll << 40) / H) return fail(MOEFP4_EUNSUPPORTED, "T*H too large");
  if (T == 0) return ok();
  if (!x || !x_fp8 || !x_sf) return fail(MOEFP4_EINVAL, "x, x_fp8 and x_sf must be non-NULL");
  if (misaligned(x, 16) || misaligned(x_fp8, 16))
    return fail(MOEFP4_EINVAL, "x and x_fp8 must be 16-byte aligned");
  moefp4_status st = hip_status(moefp4::launch_quantize_act(static_cast<const uint16_t*>(x), T, (int)H,
                                                            x_fp8, x_sf, false, stream),
                                "quantize_act");
  return st == MOEFP4_OK ? ok() : st;
}

moefp4_status moe_fp4_quantize_act_fp4(int64_t T, int64_t H, const void* x, uint8_t* x_fp4,
                                       uint8_t* x_sf, hipStream_t stream) {
  if (T < 0 || H <= 0 || H % 32) return fail(MOEFP4_EINVAL, "need T >= 0 and H a positive multiple of 32, got T=%lld H=%lld", (long long)T, (long long)H);
  if (H > (1 << 30) || T > (1ll << 40) / H) return fail(MOEFP4_EUNSUPPORTED, "T*H too large");
  if (T == 0) return ok();
  if (!x || !x_fp4 || !x_sf) return fail(MOEFP4_EINVAL, "x, x_fp4 and x_sf must be non-NULL");
  if (misaligned(x, 16) || misaligned(x_fp4, 16))
    return fail(MOEFP4_EINVAL, "x and x_fp4 must be 16-byte aligned");
  moefp4_status st = hip_status(moefp4::launch_quantize_act(static_cast<const uint16_t*>(x), T, (int)H,
                                                            x_fp4, x_sf, true, stream),
                                "quantize_act_fp4");
  return st == MOEFP4_OK ? ok() : st;
}

moefp4_status moefp4_mfma_peak_probe(int32_t a4, int32_t iters, int32_t blocks, float* sink, double* flops,
                                     hipStream_t stream) {
  if (iters < 1 || blocks < 1 || !flops) return fail(MOEFP4_EINVAL, "iters, blocks >= 1 and flops non-NULL needed");
  if (!sink) return fail(MOEFP4_EINVAL, "sink must be non-NULL (blocks * 256 floats)");
  *flops = (double)blocks * 4 * (double)iters * 64 * 2.0 * 16 * 16 * 128;
  moefp4_status st = hip_status(moefp4::launch_mfma_peak(a4 != 0, iters, blocks, sink, stream), "mfma_peak");
  return st == MOEFP4_OK ? ok() : st;
}

moefp4_status moefp4_set_stage_events(hipEvent_t* events, int32_t n) {
  if (events && n < 6) return fail(MOEFP4_EINVAL, "stage events need an array of 6, got %d", n);
  g_stage_events = events;
  return ok();
}

const char* moefp4_last_error(void) { return g_err.c_str(); }

const char* moefp4_version(void) { return "moefp4 0.1 gfx950"; }

}  // extern "C"
