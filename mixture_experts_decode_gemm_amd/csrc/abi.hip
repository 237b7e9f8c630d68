// abi.hip -- the C ABI of libmoedecode (include/moedecode.h): host-side argument
// checks, workspace layout, and the layer's launch sequence.  Nothing here allocates
// device memory, frees or synchronises; moe_layer keeps one side stream and two events
// per device (created on its first call on that device) to run the shared expert beside
// the routed path.
#include <algorithm>
#include <mutex>
#include <string.h>

#include "moedecode.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int kMaxTokens = 4096;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
// the GPU share the shared expert's GEMMs are planned for: they run beside the routing
// kernels (gate/up) and the expert passes (down), so fewer, longer splits (fewer partial
// bytes) serve better than filling every CU (measured for both at once: 0.5 best of
// 0.3 .. 1; 547 -> 521 us per layer)
constexpr double kSideShareGu = 0.5;
constexpr double kSideShareDown = 0.5;
// up to this many tokens the routed path is short and the shared expert's chain weighs
// more: its GEMMs are planned for the whole GPU (measured per layer: -15 us at 8 tokens,
// -24 at 64, -27 at 96, -3.6 at 130; +3.5 at 1 token, +6 at 192 and +8 at 256)
constexpr int kNarrowSideTokens = 160;
inline double side_share(int T, double share) { return T <= kNarrowSideTokens ? 1.0 : share; }
// the front GEMM (router + latent down rows) runs beside the side stream's gate/up GEMM:
// planned for three quarters of the GPU it takes 4 splits of 128-token chunks, not 5
// (measured 495.7 -> 487.2 us per layer at 256 tokens)
constexpr double kFrontShare = 0.75;
// past this many tokens the shared expert is forked after the routing lists (see moe_layer)
constexpr int kLateForkTokens = 256;

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t up256(size_t b) { return (b + 255) / 256 * 256; }

moe_status launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// checks shared by every call that takes moe_dims
moe_status check_dims(const moe_dims* d) {
    if (!d) return MOE_ERR_NULL;
    if (d->tokens < 1 || d->max_tokens < d->tokens || d->max_tokens > kMaxTokens)
        return MOE_ERR_SHAPE;
    if (d->hidden < 64 || d->hidden % 64 || d->latent < 64 || d->latent % 64) return MOE_ERR_SHAPE;
    if (d->shared_inter < 64 || d->shared_inter % 64) return MOE_ERR_SHAPE;
    if (d->experts < 1 || d->experts > kMaxExperts) return MOE_ERR_SHAPE;
    if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->experts) return MOE_ERR_SHAPE;
    if (d->unit_tokens != 8 && d->unit_tokens != 16) return MOE_ERR_SHAPE;
    if (d->expert_inter < 32 || d->expert_inter % 32) return MOE_ERR_SHAPE;
    if (!(d->rms_eps >= 0.0f)) return MOE_ERR_SHAPE;
    if (d->expert_format == MOE_FMT_MXFP4_MXFP8) {
        if (d->latent % 256 || d->expert_inter % 128) return MOE_ERR_SHAPE;
    } else if (d->expert_format == MOE_FMT_MXFP4_MXFP8_PACKED) {
        const int is = d->expert_inter / 128;
        if (d->latent % 512 || d->latent > 3584 || d->expert_inter % 128 ||
            (is != 1 && is != 2 && is != 4))
            return MOE_ERR_SHAPE;
    } else if (d->expert_format == MOE_FMT_BF16) {
        if (d->expert_inter > 4096) return MOE_ERR_SHAPE;
    } else {
        return MOE_ERR_FORMAT;
    }
    return MOE_OK;
}

struct Layout {
    size_t off[MOE_WS_FIELDS];
    size_t act, uni, uni_side, parts, sync, total;
};

Layout layout(const moe_dims* d) {
    const size_t T = d->max_tokens, H = d->hidden, L = d->latent, E = d->experts, K = d->top_k;
    const size_t S = d->shared_inter, P = T * K;
    const size_t U = (P + d->unit_tokens - 1) / d->unit_tokens + E;
    const size_t I = d->expert_inter;
    const size_t sizes[17] = {T * E * 4, P * 4, P * 4, E * 4, (E + 1) * 4, P * 4, U * 16, 16,
                              T * L * 2, T * L, T * (L / 32), P * L * 2, T * L * 2, T * H * 2,
                              T * L * 2, P * I, P * (I / 32)};
    Layout lo;
    size_t at = 0;
    for (int i = 0; i < 17; ++i) {
        lo.off[i] = at;
        at += up256(sizes[i]);
    }
    lo.off[17] = at;
    lo.act = at;
    at += up256(T * S * 2);
    // scratch of the routed path (list bitmaps; the tiled GEMMs' split partials), of the
    // shared expert's GEMMs on the side stream (their split partials), and the partials of
    // the front GEMM (router + latent down), later of the up-projection
    const int Tm = d->max_tokens;
    const int Hi = d->hidden, Li = d->latent, Ei = d->experts, S2 = 2 * d->shared_inter;
    lo.uni = at;
    size_t u = 0;
    const size_t g[4] = {gemm_scratch_bytes(Tm, Ei, Hi), gemm_scratch_bytes(Tm, Li, Hi),
                         gemm_scratch_bytes(Tm, Hi, Li), lists_scratch_bytes(Tm, Ei)};
    for (size_t v : g) u = v > u ? v : u;
    at += up256(u);
    lo.uni_side = at;
    size_t us = 0;
    const size_t g2[4] = {gemm_parts_bytes(Tm, S2, Hi), gemm_scratch_bytes(Tm, Hi, d->shared_inter),
                          std::max(wgemm_parts_bytes(Tm, S2, Hi, kSideShareGu),
                                   wgemm_parts_bytes(std::min(Tm, kNarrowSideTokens), S2, Hi, 1.0)),
                          std::max(wgemm_parts_bytes(Tm, Hi, d->shared_inter, kSideShareDown),
                                   wgemm_parts_bytes(std::min(Tm, kNarrowSideTokens), Hi,
                                                     d->shared_inter, 1.0))};
    for (size_t v : g2) us = v > us ? v : us;
    at += up256(us);
    lo.parts = at;
    const size_t p1 = std::max(wgemm_parts_bytes(Tm, Ei + Li, Hi, kFrontShare),
                               wgemm_parts_bytes(Tm, Ei + Li, Hi, 1.0)),
                 p2 = std::max(wgemm_parts_bytes(Tm, Hi, Li),
                               wgemm_parts_bytes(Tm, Hi, Li, 1.0, true));
    at += up256(p1 > p2 ? p1 : p2);
    lo.sync = at;  // the expert passes' work counters
    at += 256;
    lo.total = at;
    return lo;
}

// One side stream and a fork/join event pair per device, created on first use and kept
// until the process ends.  The mutex serialises the enqueue sequence of concurrent
// moe_layer calls on one device (an event must be waited for before it is re-recorded).
constexpr int kMaxDevices = 64;
struct SideStream {
    std::mutex mu;
    bool tried = false, ok = false;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[kMaxDevices];
// The events only order the two streams of one device (kernel boundaries already make
// each kernel's writes visible device-wide), so they skip the system-scope fence, whose
// cache writeback delays the next kernel on the stream (measured: 489.1 -> 486.8 us per
// layer at 256 tokens)
constexpr unsigned kEventFlags = hipEventDisableTiming | hipEventDisableSystemFence;

SideStream* side_stream() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream& ss = g_side[dev];
    std::lock_guard<std::mutex> lock(ss.mu);
    if (!ss.tried) {
        ss.tried = true;
        ss.ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess &&
                hipEventCreateWithFlags(&ss.fork, kEventFlags) == hipSuccess &&
                hipEventCreateWithFlags(&ss.join, kEventFlags) == hipSuccess;
    }
    return ss.ok ? &ss : nullptr;
}

// ---- the allocation-free grouped FFN -----------------------------------------------------
// The grouped FFN's scratch (the MXFP8 hidden of every listed pair and the passes' work
// counters) in a file-scope device array, for callers that cannot allocate.  Every GPU the
// library runs on holds its own copy until the process ends.  In host code the array's
// name is only a host-side stand-in: its device address, per device, comes from
// hipGetSymbolAddress (taken on the entry point's first call on that device, with that
// device current), and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = 9u << 20;  // 9 MiB: 1020 tokens x top-16 at I = 512
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

struct ScratchAddr {
    std::once_flag once;
    hipError_t err = hipErrorNotInitialized;
    void* ptr = nullptr;
};
ScratchAddr g_scratch[kMaxDevices];

// the device address of `scratch` on the current device (nullptr if it cannot be had)
void* scratch_addr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    ScratchAddr& sa = g_scratch[dev];
    std::call_once(sa.once, [&] { sa.err = hipGetSymbolAddress(&sa.ptr, HIP_SYMBOL(scratch)); });
    return sa.err == hipSuccess ? sa.ptr : nullptr;
}

// the router GEMM: the weight-streaming kernel when the shape allows it
bool router_fast(const moe_dims* d) {
    return wgemm_fits(d->max_tokens, d->experts, d->experts, d->experts, d->hidden, false);
}

size_t router_scratch(const moe_dims* d, int M) {
    return router_fast(d) ? wgemm_parts_bytes(M, d->experts, d->hidden)
                          : gemm_scratch_bytes(M, d->experts, d->hidden);
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "libmoedecode 0.1 (gfx950)"; }

size_t moe_router_workspace_size(const moe_dims* d) {
    if (check_dims(d) != MOE_OK) return 0;
    return router_scratch(d, d->max_tokens);
}

moe_status moe_router_topk(const moe_dims* d, const void* x, const void* w_gate,
                           const float* bias, float* logits, int32_t* ids, float* weights,
                           int32_t flags, void* workspace, size_t ws_bytes, void* stream) {
    moe_status st = check_dims(d);
    if (st != MOE_OK) return st;
    if (flags & ~(MOE_LOGITS_GIVEN | MOE_GATE_PACKED)) return MOE_ERR_FORMAT;
    const bool given = flags & MOE_LOGITS_GIVEN;
    const bool packed = !given && (flags & MOE_GATE_PACKED);
    if (packed && !wgemm_fits(d->max_tokens, d->experts, d->experts, d->experts, d->hidden, true))
        return MOE_ERR_FORMAT;
    if (!bias || !logits || !ids || !weights) return MOE_ERR_NULL;
    if (!given && (!x || !w_gate)) return MOE_ERR_NULL;
    if (!al16(bias) || !al16(logits) || !al16(ids) || !al16(weights)) return MOE_ERR_ALIGN;
    if (!given && (!al16(x) || !al16(w_gate))) return MOE_ERR_ALIGN;
    const size_t need = given ? 0 : router_scratch(d, d->tokens);
    if (need && (!workspace || ws_bytes < need)) return MOE_ERR_WORKSPACE;
    if (workspace && !al16(workspace)) return MOE_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (!given && (packed || router_fast(d))) {
        // the split partials are added (in split order) into each token's logits inside the
        // top-K launch, as in the layer's front: no separate reduce, no logits round trip
        int S = 1;
        if (launch_wgemm(d->tokens, d->experts, d->experts, d->experts, d->hidden, x, w_gate,
                         nullptr, nullptr, packed, (float*)workspace, s, false, &S) != hipSuccess)
            return MOE_ERR_LAUNCH;
        return launch_status(launch_front_topk(d->tokens, d->experts, d->experts, 0, S,
                                               (const float*)workspace, logits, bias, d->top_k,
                                               d->renormalize, d->routed_scale, ids, weights,
                                               nullptr, nullptr, nullptr, nullptr, s));
    } else if (!given) {
        hipError_t e = launch_gemm(d->tokens, d->experts, d->hidden, x, w_gate, logits, nullptr, 0,
                                   workspace, s);
        if (e != hipSuccess) return MOE_ERR_LAUNCH;
    }
    return launch_status(launch_topk(d->tokens, d->experts, d->top_k, logits, bias,
                                     d->renormalize, d->routed_scale, ids, weights, nullptr, s));
}

size_t moe_lists_workspace_size(const moe_dims* d) {
    if (check_dims(d) != MOE_OK) return 0;
    return lists_scratch_bytes(d->max_tokens, d->experts);
}

moe_status moe_build_lists(const moe_dims* d, const int32_t* ids, int32_t* counts,
                           int32_t* offsets, int32_t* pairs, moe_unit* units,
                           int32_t* num_units, void* workspace, size_t ws_bytes, void* stream) {
    moe_status st = check_dims(d);
    if (st != MOE_OK) return st;
    if (!ids || !counts || !offsets || !pairs || !units || !num_units || !workspace)
        return MOE_ERR_NULL;
    if (!al16(ids) || !al16(counts) || !al16(offsets) || !al16(pairs) || !al16(units) ||
        !al16(num_units) || !al16(workspace))
        return MOE_ERR_ALIGN;
    if (ws_bytes < lists_scratch_bytes(d->tokens, d->experts)) return MOE_ERR_WORKSPACE;
    return launch_status(launch_lists(d->tokens, d->top_k, d->experts, d->unit_tokens, ids, counts,
                                      offsets, pairs, (int32_t*)units, num_units, workspace,
                                      nullptr, (hipStream_t)stream));
}

moe_status moe_quant_mxfp8(int32_t rows, int32_t cols, const void* x, uint8_t* codes,
                           uint8_t* scales, void* stream) {
    if (rows < 1 || cols < 32 || cols % 32 || (long)rows * cols > (1L << 34)) return MOE_ERR_SHAPE;
    if (!x || !codes || !scales) return MOE_ERR_NULL;
    if (!al16(x) || !al16(codes) || !al16(scales)) return MOE_ERR_ALIGN;
    return launch_status(launch_quant_mxfp8(rows, cols, x, codes, scales, (hipStream_t)stream));
}

size_t moe_ffn_workspace_size(const moe_dims* d) {
    if (check_dims(d) != MOE_OK) return 0;
    if (d->expert_format == MOE_FMT_BF16) return 256;
    return ffn_scratch_bytes(d->max_tokens * d->top_k, d->expert_inter);
}

moe_status moe_grouped_ffn_stages(const moe_dims* d, const moe_expert_weights* w,
                                  const void* act, const uint8_t* act_scales,
                                  const int32_t* pairs, const moe_unit* units,
                                  const int32_t* num_units, void* rows, void* workspace,
                                  size_t ws_bytes, int32_t stages, void* stream) {
    moe_status st = check_dims(d);
    if (st != MOE_OK) return st;
    if (stages < 1 || stages > 3) return MOE_ERR_FORMAT;
    const bool packed = d->expert_format == MOE_FMT_MXFP4_MXFP8_PACKED;
    const bool mx = d->expert_format == MOE_FMT_MXFP4_MXFP8 || packed;
    if (!mx && stages != 3) return MOE_ERR_FORMAT;
    const bool up = stages & MOE_FFN_UP, down = stages & MOE_FFN_DOWN;
    if (!w || !pairs || !units || !num_units) return MOE_ERR_NULL;
    if ((up && (!w->w13 || !act)) || (down && (!w->w2 || !rows))) return MOE_ERR_NULL;
    if (!al16(pairs) || !al16(units) || !al16(num_units)) return MOE_ERR_ALIGN;
    if ((up && (!al16(w->w13) || !al16(act))) || (down && (!al16(w->w2) || !al16(rows))))
        return MOE_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (mx) {
        if ((up && (!w->s13 || !act_scales)) || (down && !w->s2) || !workspace)
            return MOE_ERR_NULL;
        if ((up && (!al16(w->s13) || !al16(act_scales))) || (down && !al16(w->s2)) ||
            !al16(workspace))
            return MOE_ERR_ALIGN;
        if (ws_bytes < ffn_scratch_bytes(d->tokens * d->top_k, d->expert_inter))
            return MOE_ERR_WORKSPACE;
        uint8_t* hid = (uint8_t*)workspace;
        uint8_t* hsc = hid + up256((size_t)d->tokens * d->top_k * d->expert_inter);
        unsigned* counters =
            (unsigned*)(hid + ffn_counter_offset(d->tokens * d->top_k, d->expert_inter));
        return launch_status(launch_ffn_mx(
            d->tokens, d->top_k, d->experts, d->latent, d->expert_inter, d->unit_tokens,
            (const uint8_t*)w->w13, (const uint8_t*)w->s13, (const uint8_t*)w->w2,
            (const uint8_t*)w->s2, (const uint8_t*)act, act_scales, pairs, (const int32_t*)units,
            num_units, rows, hid, hsc, stages, packed, counters, false, s));
    }
    return launch_status(launch_ffn_bf16(d->tokens, d->top_k, d->experts, d->latent,
                                         d->expert_inter, d->unit_tokens, w->w13, w->w2, act,
                                         pairs, (const int32_t*)units, num_units, rows, s));
}

moe_status moe_grouped_ffn(const moe_dims* d, const moe_expert_weights* w, const void* act,
                           const uint8_t* act_scales, const int32_t* pairs,
                           const moe_unit* units, const int32_t* num_units, void* rows,
                           void* workspace, size_t ws_bytes, void* stream) {
    return moe_grouped_ffn_stages(d, w, act, act_scales, pairs, units, num_units, rows,
                                  workspace, ws_bytes, MOE_FFN_UP | MOE_FFN_DOWN, stream);
}

size_t moe_grouped_ffn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

moe_status moe_grouped_ffn_noalloc(const moe_dims* d, const moe_expert_weights* w,
                                   const void* act, const uint8_t* act_scales,
                                   const int32_t* pairs, const moe_unit* units,
                                   const int32_t* num_units, void* rows, void* stream) {
    const moe_status st = check_dims(d);
    if (st != MOE_OK) return st;
    // what this call uses: the MXFP8 hidden of its T*K pairs and the counters
    if (d->expert_format != MOE_FMT_BF16 &&
        ffn_scratch_bytes(d->tokens * d->top_k, d->expert_inter) > kNoAllocScratchBytes)
        return MOE_ERR_WORKSPACE;
    void* ws = scratch_addr();
    if (!ws) return MOE_ERR_LAUNCH;
    return moe_grouped_ffn_stages(d, w, act, act_scales, pairs, units, num_units, rows, ws,
                                  kNoAllocScratchBytes, MOE_FFN_UP | MOE_FFN_DOWN, stream);
}

moe_status moe_pack_expert_weights(const moe_dims* d, const moe_expert_weights* src,
                                   const moe_expert_weights* dst, void* stream) {
    if (!d || !src || !dst) return MOE_ERR_NULL;
    moe_dims pd = *d;
    pd.expert_format = MOE_FMT_MXFP4_MXFP8_PACKED;
    const moe_status st = check_dims(&pd);
    if (st != MOE_OK) return st;
    const void* ptrs[] = {src->w13, src->s13, src->w2, src->s2, dst->w13, dst->s13, dst->w2,
                          dst->s2};
    for (const void* p : ptrs) {
        if (!p) return MOE_ERR_NULL;
        if (!al16(p)) return MOE_ERR_ALIGN;
    }
    return launch_status(launch_pack_experts(
        d->experts, d->latent, d->expert_inter, (const uint8_t*)src->w13,
        (const uint8_t*)src->s13, (const uint8_t*)src->w2, (const uint8_t*)src->s2,
        (uint8_t*)dst->w13, (uint8_t*)dst->s13, (uint8_t*)dst->w2, (uint8_t*)dst->s2,
        (hipStream_t)stream));
}

moe_status moe_finalize(int32_t tokens, int32_t top_k, int32_t cols, const void* rows,
                        const float* weights, const int32_t* ids, void* out, void* stream) {
    if (tokens < 1 || top_k < 1 || top_k > kMaxTopK || cols < 8 || cols % 8) return MOE_ERR_SHAPE;
    if ((long)tokens * (cols / 8) >= (1L << 31) - 256) return MOE_ERR_SHAPE;
    if (!rows || !weights || !out) return MOE_ERR_NULL;
    if (!al16(rows) || !al16(weights) || !al16(out) || (ids && !al16(ids))) return MOE_ERR_ALIGN;
    return launch_status(
        launch_finalize(tokens, top_k, cols, rows, weights, ids, out, (hipStream_t)stream));
}

moe_status moe_rmsnorm(int32_t rows, int32_t cols, const void* r, const void* g, float eps,
                       void* out, void* stream) {
    if (rows < 1 || cols < 8 || cols % 8 || !(eps >= 0.0f)) return MOE_ERR_SHAPE;
    if (!r || !g || !out) return MOE_ERR_NULL;
    if (!al16(r) || !al16(g) || !al16(out)) return MOE_ERR_ALIGN;
    return launch_status(launch_rmsnorm(rows, cols, r, g, eps, out, (hipStream_t)stream));
}

size_t moe_linear_workspace_size(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || N < 1 || K < 64 || K % 64) return 0;
    return wgemm_fits(M, N, N, N, K, false) ? wgemm_parts_bytes(M, N, K)
                                            : gemm_scratch_bytes(M, N, K);
}

moe_status moe_linear(int32_t M, int32_t N, int32_t K, const void* x, const void* w, void* out,
                      const void* add, int32_t mode, void* workspace, size_t ws_bytes,
                      void* stream) {
    if (M < 1 || M > 65536 || N < 1 || N > (1 << 20) || K < 64 || K % 64) return MOE_ERR_SHAPE;
    if (mode < MOE_LINEAR_F32 || mode > MOE_LINEAR_ADD_BF16) return MOE_ERR_FORMAT;
    if (!x || !w || !out || (mode == MOE_LINEAR_ADD_BF16 && !add)) return MOE_ERR_NULL;
    if (!al16(x) || !al16(w) || !al16(out) || (add && !al16(add))) return MOE_ERR_ALIGN;
    const bool fast = wgemm_fits(M, N, N, N, K, false);
    const size_t need = fast ? wgemm_parts_bytes(M, N, K) : gemm_scratch_bytes(M, N, K);
    if (need && (!workspace || ws_bytes < need)) return MOE_ERR_WORKSPACE;
    if (workspace && !al16(workspace)) return MOE_ERR_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (fast) {
        int S = 1;
        if (launch_wgemm(M, N, N, N, K, x, w, nullptr, nullptr, false, (float*)workspace, s, false,
                         &S) != hipSuccess)
            return MOE_ERR_LAUNCH;
        return launch_status(launch_wg_reduce(M, N, 0, N, S, (const float*)workspace, nullptr, mode,
                                              out, add, s, false));
    }
    return launch_status(launch_gemm(M, N, K, x, w, out, add, mode, workspace, s));
}

moe_status moe_pack_dense_weight(int32_t N, int32_t K, const void* w, void* out, void* stream) {
    if (N < 64 || N % 64 || K < 128 || K % 128 || (long)N * K > (1L << 34)) return MOE_ERR_SHAPE;
    if (!w || !out) return MOE_ERR_NULL;
    if (!al16(w) || !al16(out)) return MOE_ERR_ALIGN;
    const uintptr_t a = (uintptr_t)w, b = (uintptr_t)out, n = (uintptr_t)N * K * 2;
    if (a < b + n && b < a + n) return MOE_ERR_SHAPE;  // overlapping buffers
    return launch_status(launch_pack_dense(N, K, w, out, (hipStream_t)stream));
}

moe_status moe_silu_mul(int32_t M, int32_t S, const void* gu, void* out, void* stream) {
    if (M < 1 || S < 8 || S % 8) return MOE_ERR_SHAPE;
    if (!gu || !out) return MOE_ERR_NULL;
    if (!al16(gu) || !al16(out)) return MOE_ERR_ALIGN;
    return launch_status(launch_silu_mul(M, S, gu, out, (hipStream_t)stream));
}

size_t moe_workspace_size(const moe_dims* d) {
    if (check_dims(d) != MOE_OK) return 0;
    return layout(d).total;
}

moe_status moe_workspace_layout(const moe_dims* d, size_t offsets[MOE_WS_FIELDS]) {
    moe_status st = check_dims(d);
    if (st != MOE_OK) return st;
    if (!offsets) return MOE_ERR_NULL;
    const Layout lo = layout(d);
    memcpy(offsets, lo.off, sizeof(lo.off));
    return MOE_OK;
}

moe_status moe_layer(const moe_dims* d, const moe_layer_weights* w, const void* x, void* out,
                     void* workspace, size_t ws_bytes, void* stream) {
    moe_status st = check_dims(d);
    if (st != MOE_OK) return st;
    if (!w || !x || !out || !workspace) return MOE_ERR_NULL;
    if (!w->w_gate || !w->bias || !w->w_down || !w->w_shared_gu || !w->w_shared_down ||
        !w->norm_w || !w->w_up || !w->experts.w13 || !w->experts.w2)
        return MOE_ERR_NULL;
    const bool packed = d->expert_format == MOE_FMT_MXFP4_MXFP8_PACKED;
    const bool mx = d->expert_format == MOE_FMT_MXFP4_MXFP8 || packed;
    if (mx && (!w->experts.s13 || !w->experts.s2)) return MOE_ERR_NULL;
    const void* ptrs[] = {w->w_gate, w->bias, w->w_down, w->w_shared_gu, w->w_shared_down,
                          w->norm_w, w->w_up, w->experts.w13, w->experts.w2, x, out, workspace};
    for (const void* p : ptrs)
        if (!al16(p)) return MOE_ERR_ALIGN;
    if (mx && (!al16(w->experts.s13) || !al16(w->experts.s2))) return MOE_ERR_ALIGN;
    if (w->dense_format != MOE_DENSE_ROWMAJOR && w->dense_format != MOE_DENSE_PACKED)
        return MOE_ERR_FORMAT;
    const bool dpack = w->dense_format == MOE_DENSE_PACKED;
    // the weight-streaming GEMMs for every dense projection, else (row-major weights of
    // shapes they do not take) the tiled GEMM
    const int S2 = 2 * d->shared_inter;
    const int H_ = d->hidden, L_ = d->latent;
    const int Tm = d->max_tokens;
    const bool fast = wgemm_fits(Tm, d->experts + L_, d->experts, d->experts + L_, H_, dpack) &&
                      wgemm_fits(Tm, S2, S2, S2, H_, dpack) &&
                      wgemm_fits(Tm, H_, H_, H_, d->shared_inter, dpack) &&
                      wgemm_fits(Tm, H_, H_, H_, L_, dpack);
    if (dpack && !fast) return MOE_ERR_SHAPE;
    const Layout lo = layout(d);
    if (ws_bytes < lo.total) return MOE_ERR_WORKSPACE;

    char* ws = (char*)workspace;
    float* logits = (float*)(ws + lo.off[0]);
    int32_t* ids = (int32_t*)(ws + lo.off[1]);
    float* wts = (float*)(ws + lo.off[2]);
    int32_t* counts = (int32_t*)(ws + lo.off[3]);
    int32_t* offs = (int32_t*)(ws + lo.off[4]);
    int32_t* pairs = (int32_t*)(ws + lo.off[5]);
    int32_t* units = (int32_t*)(ws + lo.off[6]);
    int32_t* nu = (int32_t*)(ws + lo.off[7]);
    void* latent = ws + lo.off[8];
    uint8_t* codes = (uint8_t*)(ws + lo.off[9]);
    uint8_t* scales = (uint8_t*)(ws + lo.off[10]);
    void* rows = ws + lo.off[11];
    void* routed = ws + lo.off[12];
    void* shared = ws + lo.off[13];
    void* normed = ws + lo.off[14];
    uint8_t* hid = (uint8_t*)(ws + lo.off[15]);
    uint8_t* hid_scales = (uint8_t*)(ws + lo.off[16]);
    void* act = ws + lo.act;
    void* uni = ws + lo.uni;
    void* uni_side = ws + lo.uni_side;

    const int T = d->tokens, H = d->hidden, L = d->latent, E = d->experts, K = d->top_k;
    const int S = d->shared_inter, I = d->expert_inter;
    hipStream_t s = (hipStream_t)stream;
#define MOE_TRY(call)                                   \
    do {                                                \
        if ((call) != hipSuccess) return MOE_ERR_LAUNCH; \
    } while (0)
    SideStream* ss = side_stream();
    std::unique_lock<std::mutex> side_lock;
    if (ss) side_lock = std::unique_lock<std::mutex>(ss->mu);
    hipStream_t sh = ss ? ss->s : s;
    int s_fr = 1, s_gu = 1, s_sd = 1, s_up = 1;
    unsigned* counters = (unsigned*)(ws + lo.sync);  // the expert passes' work counters
    float* parts = (float*)(ws + lo.parts);
    float* parts_side = (float*)uni_side;
    // The shared expert depends on x only: its gate/up GEMM, activation, down GEMM and
    // rounding run on the side stream ([wide] and [ep] module summaries: the shared
    // expert beside the routed path), joined before the up-projection adds into it.  Up to
    // kLateForkTokens tokens it is forked at the start, beside the routing kernels; past
    // that its GEMMs would fill every CU and starve them, so it is forked after the lists,
    // beside the expert passes.
    const bool late_fork = T > kLateForkTokens;
    auto launch_side = [&]() -> bool {
        if (ss) {
            if (hipEventRecord(ss->fork, s) != hipSuccess) return false;
            if (hipStreamWaitEvent(sh, ss->fork, 0) != hipSuccess) return false;
        }
        if (late_fork) {  // unsplit: the BF16 gate/up values in the side scratch
            if (launch_wgemm(T, 2 * S, 2 * S, 2 * S, H, x, w->w_shared_gu, nullptr, nullptr,
                             dpack, parts_side, sh, false, &s_gu, kSideShareGu, nullptr, false,
                             parts_side) != hipSuccess)
                return false;
            if (launch_silu_mul(T, S, parts_side, act, sh) != hipSuccess) return false;
        } else {
            if (launch_wgemm(T, 2 * S, 2 * S, 2 * S, H, x, w->w_shared_gu, nullptr, nullptr,
                             dpack, parts_side, sh, false, &s_gu,
                             side_share(T, kSideShareGu)) != hipSuccess)
                return false;
            if (launch_silu_mul_parts(T, S, s_gu, parts_side, 2 * S, act, sh) != hipSuccess)
                return false;
        }
        // the down GEMM into the shared expert's BF16 output (one rounding), which the
        // up-projection's reduce adds to: forked late (beside the expert passes, which
        // leave it time to spare) unsplit and written directly, else as split partials
        // reduced on the side stream
        if (late_fork) {
            if (launch_wgemm(T, H, H, H, S, act, w->w_shared_down, nullptr, nullptr, dpack,
                             parts_side, sh, false, &s_sd, kSideShareDown, nullptr, false,
                             shared) != hipSuccess)
                return false;
        } else {
            if (launch_wgemm(T, H, H, H, S, act, w->w_shared_down, nullptr, nullptr, dpack,
                             parts_side, sh, false, &s_sd,
                             side_share(T, kSideShareDown)) != hipSuccess)
                return false;
            if (launch_wg_reduce(T, H, 0, H, s_sd, parts_side, nullptr, 1, shared, nullptr, sh,
                                 false) != hipSuccess)
                return false;
        }
        return !ss || hipEventRecord(ss->join, sh) == hipSuccess;
    };
    // the routing slot map (for the list build past one workgroup), filled by the top-K
    uint8_t* slot_of = lists_fused_fits(T, E) ? nullptr : lists_slot_map(uni, T, E);
    if (fast) {
        if (!late_fork && !launch_side()) return MOE_ERR_LAUNCH;
        // [wide] front: the router rows and the latent down rows as one FP32-out GEMM over
        // x; FP32 logits and the latent rounded once to BF16 from the same partials
        // (the GEMM also zeroes the expert passes' two work counters)
        MOE_TRY(launch_wgemm(T, E + L, E, E + L, H, x, w->w_gate, w->w_down, nullptr, dpack, parts,
                             s, true, &s_fr, late_fork ? 1.0 : kFrontShare, counters));
        // FP32 logits; the latent rounded once to BF16 and, for MXFP4 experts, its MXFP8
        // codes in the same pass, with the sigmoid top-K of each token taken from its
        // logits in LDS
        if (mx)
            MOE_TRY(launch_front_topk(T, E + L, E, L, s_fr, parts, logits, w->bias, K,
                                      d->renormalize, d->routed_scale, ids, wts, slot_of, latent,
                                      codes, scales, s));
        else
            MOE_TRY(launch_wg_reduce(T, E + L, E, E + L, s_fr, parts, logits, 1, latent, nullptr,
                                     s, true));
    } else {
        // The shared expert depends on x only: it runs on the side stream beside the whole
        // routed path; gate/up as split-K partials, whose sum the activation rounds (the
        // gate/up BF16 values) before SiLU-and-mul
        if (ss) {
            MOE_TRY(hipEventRecord(ss->fork, s));
            MOE_TRY(hipStreamWaitEvent(sh, ss->fork, 0));
        }
        MOE_TRY(launch_gemm_parts(T, 2 * S, H, x, w->w_shared_gu, parts_side, sh, false, &s_gu));
        MOE_TRY(launch_silu_mul_parts(T, S, s_gu, parts_side, 2 * S, act, sh));
        MOE_TRY(launch_gemm(T, H, S, act, w->w_shared_down, shared, nullptr, 1, uni_side, sh));
        if (ss) MOE_TRY(hipEventRecord(ss->join, sh));
        // routing: FP32 router GEMM, the latent down GEMM (one BF16 rounding)
        MOE_TRY(launch_gemm(T, E, H, x, w->w_gate, logits, nullptr, 0, uni, s, 0, true));
        MOE_TRY(launch_gemm(T, L, H, x, w->w_down, latent, nullptr, 1, uni, s, 0, true));
    }
    // sigmoid top-K (already taken with the front reduce on the fast MXFP4 path), lists
    // and unit windows
    if (!(fast && mx))
        MOE_TRY(launch_topk(T, E, K, logits, w->bias, d->renormalize, d->routed_scale, ids, wts,
                            slot_of, s));
    MOE_TRY(launch_lists(T, K, E, d->unit_tokens, ids, counts, offs, pairs, units, nu, uni, slot_of,
                         s));
    if (fast && late_fork && !launch_side()) return MOE_ERR_LAUNCH;
    // MXFP8 latent, grouped experts, Finalize
    if (mx) {
        if (!fast) MOE_TRY(launch_quant_mxfp8(T, L, latent, codes, scales, s));
        MOE_TRY(launch_ffn_mx(T, K, E, L, I, d->unit_tokens, (const uint8_t*)w->experts.w13,
                              (const uint8_t*)w->experts.s13, (const uint8_t*)w->experts.w2,
                              (const uint8_t*)w->experts.s2, codes, scales, pairs, units, nu,
                              rows, hid, hid_scales, 3, packed, counters, fast, s));
    } else {
        MOE_TRY(launch_ffn_bf16(T, K, E, L, I, d->unit_tokens, w->experts.w13, w->experts.w2,
                                latent, pairs, units, nu, rows, s));
    }
    if (finalize_rmsnorm_fits(L)) {
        MOE_TRY(launch_finalize_rmsnorm(T, K, L, rows, wts, w->norm_w, d->rms_eps, routed, normed,
                                        s));
    } else {
        MOE_TRY(launch_finalize(T, K, L, rows, wts, nullptr, routed, s));
        MOE_TRY(launch_rmsnorm(T, L, routed, w->norm_w, d->rms_eps, normed, s));
    }
    // the up-projection added into the shared partial (one rounding); only its reduce
    // needs the side stream's results.  With the shared expert forked early, the side
    // stream is done by now and the GEMM has the GPU to itself (its plan counts its
    // partials once); forked late, the side GEMMs may still run beside it.
    if (fast) {
        MOE_TRY(launch_wgemm(T, H, H, H, L, normed, w->w_up, nullptr, nullptr, dpack, parts, s,
                             false, &s_up, 1.0, nullptr, !late_fork));
        if (ss) MOE_TRY(hipStreamWaitEvent(s, ss->join, 0));
        // out = BF16(FP32(shared) + the up-projection's partials in split order)
        MOE_TRY(launch_wg_reduce(T, H, 0, H, s_up, parts, nullptr, 2, out, shared, s, false));
    } else {
        if (ss) MOE_TRY(hipStreamWaitEvent(s, ss->join, 0));
        MOE_TRY(launch_gemm(T, H, L, normed, w->w_up, out, shared, 2, uni, s));
    }
#undef MOE_TRY
    return MOE_OK;
}

}  // extern "C"
