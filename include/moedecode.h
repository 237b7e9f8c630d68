/*
 * moedecode.h -- C ABI of libmoedecode: one wide-batch decode step of a latent
 * mixture-of-experts layer on one MI355X (gfx950), TP1.
 *
 * The layer, as the pages state it (citations name the page and section):
 *   [wide] "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.wide", module
 *          summary (the listed data flow and the precision paragraph), Finalize,
 *          WideRoute, WideScratch, WideMoE.tail;
 *   [ep]   "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.ep.layer",
 *          module summary, EpMoeLayer (topk, gate_up, stock_order), EpRouted.prepare;
 *   [fp]   "vllm.models.glm5next.nvidia.specialized_decode.cutedsl.finalize_publish",
 *          _QuadFinalizePublishDeviceKernel (the invalid-slot rule).
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers unless stated; arrays are row-major with the
 *     last dimension contiguous; BF16 is IEEE bfloat16 bits; every pointer to a tensor
 *     must be 16-byte aligned (MOE_ERR_ALIGN otherwise).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call
 *     only enqueues work: it never allocates device memory, frees or synchronises
 *     (concurrent calls on different streams must not share output or workspace
 *     buffers).  The one piece of state: moe_layer creates, on its first call on a
 *     device, one non-blocking side stream and two events there (kept until the process
 *     ends) and runs the shared expert on that stream, forked from and joined back into
 *     `stream` with the events; if they cannot be created it runs everything on
 *     `stream`.  Its enqueue sequence holds a per-device lock.
 *   - The caller owns every buffer.  Weights and inputs are read-only.
 *   - All argument checks happen on the host before any launch; a failing check
 *     returns its status and writes nothing.  MOE_ERR_LAUNCH reports a failed launch
 *     (hipGetLastError); work enqueued before the failure may have run.
 *   - Model-size limits: tokens <= max_tokens <= 4096, experts <= 1024, top_k <= 16,
 *     unit_tokens in {8, 16}.
 */
#ifndef MOEDECODE_H
#define MOEDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,      /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,     /* a size is out of range (cf. [ep] EpRouted.prepare:
                              ValueError unless 0 < tokens <= capacity; [fp]: ValueError
                              when the hidden size is not a multiple of the vector) */
    MOE_ERR_ALIGN = 3,     /* a tensor pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 4, /* workspace smaller than required (cf. [wide] WideScratch.reserve:
                              RuntimeError when rows must grow after being bound) */
    MOE_ERR_FORMAT = 5,    /* unsupported expert format or flag */
    MOE_ERR_LAUNCH = 6     /* a kernel launch failed */
} moe_status;

/* expert weight / activation format */
enum { MOE_FMT_MXFP4_MXFP8 = 0, /* MXFP4 (E2M1 + E8M0 per 32) weights x MXFP8 (E4M3 + E8M0
                                   per 32) activations, MXFP8 hidden ([wide] precision) */
       MOE_FMT_BF16 = 1,        /* BF16 weights and activations (small test models) */
       MOE_FMT_MXFP4_MXFP8_PACKED = 2 }; /* the same arithmetic with the expert weights in
                                   the packed layout of moe_pack_expert_weights */

/* moe_router_topk flags */
enum {
    MOE_LOGITS_GIVEN = 1, /* skip the router GEMM and read `logits` as input */
    MOE_GATE_PACKED = 2   /* w_gate in the packed layout of moe_pack_dense_weight */
};

/* Host struct describing the layer.  tokens = T of this call; max_tokens sizes the
   workspace (the widest batch, as [wide] WideScratch sizes its buffers).
   hidden H, latent L, experts E, top_k K, expert_inter I, shared_inter S. */
typedef struct {
    int32_t tokens, max_tokens, hidden, latent, experts, top_k, expert_inter, shared_inter,
        unit_tokens, expert_format, renormalize;
    float routed_scale, rms_eps;
} moe_dims;

/* One unit window: `count` (1..unit_tokens) consecutive entries pairs[begin ..] of one
   expert's routing list ([wide] module summary: the grouped engine's unit windows, one
   pass over a touched expert's weights per 8 of its tokens).  expert_total is the expert's whole list length on its first window
   and 0 on its later windows (the grouped FFN streams an expert once for all of its
   windows). */
typedef struct {
    int32_t expert, begin, count, expert_total;
} moe_unit;

/* Expert weights (device).  MXFP4: w13 [E, 2I, L/2] bytes (element 2j in the low
   nibble of byte j), s13 [E, 2I, L/32] E8M0; w2 [E, L, I/2], s2 [E, L, I/32].  Rows
   [0, I) of w13 are the gate, rows [I, 2I) the up projection.  BF16: w13 [E, 2I, L],
   w2 [E, L, I], s13 = s2 = NULL. */
typedef struct {
    const void *w13, *s13, *w2, *s2;
} moe_expert_weights;

/* dense weight format of moe_layer_weights */
enum { MOE_DENSE_ROWMAJOR = 0, /* BF16 [N, K] row-major, as the pages state the weights */
       MOE_DENSE_PACKED = 1 }; /* the same values reordered by moe_pack_dense_weight */

/* Layer weights (device): w_gate BF16 [E, H]; bias FP32 [E] (the e_score correction
   bias); w_down BF16 [L, H]; w_shared_gu BF16 [2S, H] (gate rows first);
   w_shared_down BF16 [H, S]; norm_w BF16 [L]; w_up BF16 [H, L].  dense_format tells the
   layout of the five BF16 matrices: all row-major, or all packed (each matrix packed on
   its own by moe_pack_dense_weight; needs E, L, 2S and H multiples of 64 and H, S, L
   multiples of 128).  The results are identical in both layouts. */
typedef struct {
    const void* w_gate;
    const float* bias;
    const void* w_down;
    const void* w_shared_gu;
    const void* w_shared_down;
    const void* norm_w;
    const void* w_up;
    moe_expert_weights experts;
    int32_t dense_format;
} moe_layer_weights;

/* Router GEMM and sigmoid top-K ([ep] EpMoeLayer.topk and stock_order; [wide] WideRoute).
   logits[t,e] = sum_h x[t,h] Wg[e,h] in FP32 (unless MOE_LOGITS_GIVEN: logits is read).
   score s = sigmoid(logit) with the library's defined exponential (Cody-Waite reduction,
   degree-7 Taylor polynomial, IEEE FP32 steps); key = s + bias[e]; the top_k largest keys
   in descending order, ties to the lower expert id -> ids [T,K] int32; weights [T,K] FP32
   = the chosen unbiased scores, divided by their slot-order FP32 sum when renormalize,
   times routed_scale.  workspace: >= moe_router_workspace_size(d) bytes (split-K
   partials of the GEMM; may be NULL when MOE_LOGITS_GIVEN).  MOE_GATE_PACKED: w_gate
   holds the packed layout of moe_pack_dense_weight (as the layer's dense weights may;
   needs experts % 64 == 0 and hidden % 128 == 0, else MOE_ERR_FORMAT); the logits are
   the same bits as from the row-major W_gate. */
moe_status moe_router_topk(const moe_dims* d, const void* x, const void* w_gate,
                           const float* bias, float* logits, int32_t* ids, float* weights,
                           int32_t flags, void* workspace, size_t ws_bytes, void* stream);
size_t moe_router_workspace_size(const moe_dims* d);

/* Routing lists and unit windows ([wide] WideRoute: each (token, slot) pair appended to
   its expert's list as token*K + slot; module summary: unit windows of 8).  Built without
   atomic list claims, deterministically: counts[E]; offsets[E+1] (exclusive prefix sum);
   pairs [T*K] by expert ascending, ascending pair id inside a list; units: windows of
   unit_tokens consecutive list entries -- first the first window of every touched
   expert (experts ascending), then every later window (experts ascending, list order);
   num_units[4] = (number of units, dropped pairs (id outside [0,E) or repeated within a
   token; such pairs are in no list), touched experts D, 0).  units must hold
   ceil(T*K/unit_tokens) + E entries.  workspace: >= moe_lists_workspace_size(d) bytes. */
moe_status moe_build_lists(const moe_dims* d, const int32_t* ids, int32_t* counts,
                           int32_t* offsets, int32_t* pairs, moe_unit* units,
                           int32_t* num_units, void* workspace, size_t ws_bytes, void* stream);
size_t moe_lists_workspace_size(const moe_dims* d);

/* MXFP8 quantisation of BF16 rows ([wide] module summary: the latent row becomes the
   experts' MXFP8 input; WideRoute's plan rows).  Per 32-element block: X =
   floor(log2 amax) - 8 clamped to [-127, 127], scale byte X + 127 (0 for an all-zero
   block), codes = E4M3 round-to-nearest-even of v / 2^X, saturating at +-448, zero
   sign kept.  codes [rows, cols] u8, scales [rows, cols/32] u8; cols % 32 == 0. */
moe_status moe_quant_mxfp8(int32_t rows, int32_t cols, const void* x, uint8_t* codes,
                           uint8_t* scales, void* stream);

/* Grouped expert FFN over the unit windows ([wide] module summary: the listed grouped
   engine; [ep] EpRouted: MXFP4 x MXFP8 experts with the gated activation).  For each
   listed pair p = pairs[i] of expert e: h = A W13e^T with A = the MXFP8 latent row of
   token p/K (FP32 accumulation); act = silu(h[:I]) * h[I:] in FP32; act -> MXFP8 (the
   moe_quant_mxfp8 rule); y = act_q W2e^T (FP32) rounded to BF16 into rows[p] [T*K, L].
   BF16 format: act = BF16 latent [T, L] (act_scales NULL), h and act rounded to BF16.
   Rows of pairs in no list are not written.  units and num_units are moe_build_lists'
   output, read on the device: each touched expert is streamed once, for all of its
   windows (the first D units name the touched experts and their list lengths).
   workspace: >= moe_ffn_workspace_size(d) bytes; on return it holds the MXFP8 hidden of
   every listed pair: codes u8 [T*K, I] at offset 0 and E8M0 scales u8 [T*K, I/32] at
   offset round_up(T*K*I, 256), indexed by pair id; the 256 bytes after the scales hold
   the two passes' work counters, which each call zeroes on its stream before use. */
moe_status moe_grouped_ffn(const moe_dims* d, const moe_expert_weights* w, const void* act,
                           const uint8_t* act_scales, const int32_t* pairs,
                           const moe_unit* units, const int32_t* num_units, void* rows,
                           void* workspace, size_t ws_bytes, void* stream);
size_t moe_ffn_workspace_size(const moe_dims* d);

/* The grouped FFN above without a caller workspace, for callers that cannot allocate
   device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
   allocation).  Same arguments, arithmetic and rows as moe_grouped_ffn; the MXFP8 hidden
   and the work counters live in a device array of the library, of
   moe_grouped_ffn_noalloc_max_bytes() bytes (9 MiB: 1020 tokens x top-16 at expert_inter
   512), that every GPU the library runs on holds until the process ends.  The call
   allocates nothing (no hipMalloc, no allocating library routine); on its first call on
   a device it looks up the array's address there.  MOE_ERR_WORKSPACE when the call's
   scratch (moe_ffn_workspace_size of these dims with max_tokens = tokens) exceeds the
   array.  Every call on one
   GPU shares that GPU's array: calls that overlap in time on one GPU (on different
   streams, or from different host threads) race and must not be issued; calls on one
   stream are ordered and safe.  The hidden left in the array is not part of the
   interface. */
moe_status moe_grouped_ffn_noalloc(const moe_dims* d, const moe_expert_weights* w,
                                   const void* act, const uint8_t* act_scales,
                                   const int32_t* pairs, const moe_unit* units,
                                   const int32_t* num_units, void* rows, void* stream);
size_t moe_grouped_ffn_noalloc_max_bytes(void);

/* Load-time preparation of MXFP4 expert weights for the grouped FFN's loads (the pages
   prepare weights ahead of the decode step too: [wide] WideMoE prepares the layer's
   persistent experts for the wide batches, and [ep] pack_front packs the front GEMM's
   weights).  src holds the row-major tensors described at
   moe_expert_weights; dst receives the same bytes reordered, buffers of the same sizes,
   for use with expert_format = MOE_FMT_MXFP4_MXFP8_PACKED:
     W13 of expert e: 1 KiB blocks (j, w, m, i) for j < I/32, w < 4, m < 4, i < L/512; lane
       l = r + 16 g of a block holds the 16 bytes of row (m / 2) I + 32 j + 16 (m % 2) + r,
       K elements 32 (4 (L/512 w + i) + g) .. +31;
     S13 of expert e: for (j, w, m, r) the L/512 scale dwords of that row starting at
       byte 4 (L/512) w;
     W2 of expert e: 1 KiB blocks (jd, w, m, s) for jd < L/512, w < 4, m < 8, s < I/128;
       lane l = r + 16 g holds row 512 jd + 128 w + 16 m + r, K elements 32 (4 s + g) .. +31;
     S2: unchanged.
   The arithmetic of every call is unchanged; only the weight loads differ.  Requires
   latent % 512 == 0 (latent <= 3584) and expert_inter / 128 in {1, 2, 4}; src and dst
   must not overlap.  d->tokens is ignored beyond the dims check. */
moe_status moe_pack_expert_weights(const moe_dims* d, const moe_expert_weights* src,
                                   const moe_expert_weights* dst, void* stream);

/* One pass of the grouped FFN above (MXFP4 x MXFP8 experts only), for callers that time
   or schedule the two expert passes apart.  stages = MOE_FFN_UP: steps (1)-(3) of the
   expert computation (gate/up product, SiLU-and-mul, MXFP8 hidden into the workspace at
   the offsets stated above; rows untouched, may be NULL); MOE_FFN_DOWN: step (4), rows
   from the hidden a previous MOE_FFN_UP call left in the same workspace with the same
   lists (act and act_scales unused, may be NULL); MOE_FFN_UP | MOE_FFN_DOWN: the same as
   moe_grouped_ffn.  Other values, or the BF16 format with a single stage: MOE_ERR_FORMAT. */
enum { MOE_FFN_UP = 1, MOE_FFN_DOWN = 2 };
moe_status moe_grouped_ffn_stages(const moe_dims* d, const moe_expert_weights* w,
                                  const void* act, const uint8_t* act_scales,
                                  const int32_t* pairs, const moe_unit* units,
                                  const int32_t* num_units, void* rows, void* workspace,
                                  size_t ws_bytes, int32_t stages, void* stream);

/* Finalize ([wide] Finalize): out[t,c] = BF16_RNE(acc), acc = +0 then
   acc = fma(w[t,k], rows[K t + k, c], acc) for k = 0..K-1 in order, FP32.  ids may be
   NULL; when given, a slot with ids[t,k] < 0 is skipped and its row never read ([fp]:
   row index -1 gets weight 0).  rows [T*K, cols] BF16, weights [T,K] FP32, out [T, cols]
   BF16; cols % 8 == 0, 1 <= top_k <= 16. */
moe_status moe_finalize(int32_t tokens, int32_t top_k, int32_t cols, const void* rows,
                        const float* weights, const int32_t* ids, void* out, void* stream);

/* RMSNorm ([ep] EpMoeLayer: ops.rms_norm(normed, routed, norm, eps)):
   out = BF16(r / sqrt(mean(r^2) + eps) * g), FP32 arithmetic; r, out [rows, cols] BF16,
   g [cols] BF16; cols % 8 == 0. */
moe_status moe_rmsnorm(int32_t rows, int32_t cols, const void* r, const void* g, float eps,
                       void* out, void* stream);

/* Dense BF16 linear out = x W^T with FP32 accumulation ([wide] precision paragraph: the
   dense projections are BF16; [ep] stock_order).  x [M, K], W [N, K] BF16.  mode MOE_LINEAR_F32: out FP32
   [M, N]; MOE_LINEAR_BF16: out BF16 = one rounding; MOE_LINEAR_ADD_BF16: out BF16 =
   BF16(FP32(add) + acc), add [M, N] BF16 (may alias out) -- the shared.addmm_ of [ep].
   K % 64 == 0, N % 8 == 0.  workspace >= moe_linear_workspace_size(M, N, K) bytes. */
enum { MOE_LINEAR_F32 = 0, MOE_LINEAR_BF16 = 1, MOE_LINEAR_ADD_BF16 = 2 };
moe_status moe_linear(int32_t M, int32_t N, int32_t K, const void* x, const void* w, void* out,
                      const void* add, int32_t mode, void* workspace, size_t ws_bytes,
                      void* stream);
size_t moe_linear_workspace_size(int32_t M, int32_t N, int32_t K);

/* Load-time reordering of one dense BF16 weight W [N, K] into the packed layout
   (MOE_DENSE_PACKED; [wide] WideMoE prepares its front weights once, ahead of the steps,
   and [ep] packs the front the same way).  The output holds the same N*K values as 1 KiB
   blocks [N/64 row groups][K/64 K stages][tile 2][K step 4][lane 64][8 BF16]: lane l of
   block (g, s, i, q) holds row 64g + 32i + l%32, columns 64s + 16q + 8(l/32) .. +8 -- the
   A operand of one 32x32x16 BF16 MFMA, so that every weight load of the dense kernels is
   a contiguous 1 KiB block per wavefront.  N % 64 == 0, K % 128 == 0; out (N*K BF16,
   caller-owned) must not overlap w.  Enqueued on `stream`. */
moe_status moe_pack_dense_weight(int32_t N, int32_t K, const void* w, void* out, void* stream);

/* Shared-expert gated activation ([ep] EpMoeLayer.gate_up; SiLU-and-mul stands in for
   the pages' undefined SiTU): out[m,j] = BF16(silu(gu[m,j]) * gu[m,S+j]), FP32 math;
   gu [M, 2S], out [M, S] BF16; S % 8 == 0. */
moe_status moe_silu_mul(int32_t M, int32_t S, const void* gu, void* out, void* stream);

/* The whole layer, the stock order of [ep] EpMoeLayer.stock_order at TP1 with the
   precision chain of the [wide] module summary: router GEMM -> top-K -> lists/units ->
   latent down (BF16) -> MXFP8 latent -> grouped experts -> Finalize -> RMSNorm ->
   shared expert (gate_up, SiLU-and-mul, down) -> out = BF16(shared + normed W_up^T).
   The shared expert runs on an internal side stream beside the routed path (see the
   conventions above); the result does not depend on the overlap.
   x [T, H] BF16 -> out [T, H] BF16.  workspace >= moe_workspace_size(d) bytes; its layout
   (moe_workspace_layout) exposes every intermediate for inspection. */
moe_status moe_layer(const moe_dims* d, const moe_layer_weights* w, const void* x, void* out,
                     void* workspace, size_t ws_bytes, void* stream);

size_t moe_workspace_size(const moe_dims* d); /* bytes at d->max_tokens; 0 if d invalid */

/* Byte offsets inside the moe_layer workspace of: 0 logits f32 [T,E], 1 ids [T,K],
   2 weights f32 [T,K], 3 counts [E], 4 offsets [E+1], 5 pairs [T*K], 6 units,
   7 num_units [4], 8 latent bf16 [T,L], 9 codes u8 [T,L], 10 scales u8 [T,L/32],
   11 rows bf16 [T*K,L], 12 routed bf16 [T,L], 13 shared bf16 [T,H], 14 normed bf16 [T,L],
   15 hidden codes u8 [T*K,I] (MXFP8 hidden of the experts, by pair id), 16 hidden scales
   u8 [T*K,I/32], 17 scratch (shared-expert intermediates, GEMM split partials, list
   bitmaps, the expert passes' work counters).  Sizes are at d->max_tokens; the row-major
   tensors of a call with T tokens occupy their first T rows. */
#define MOE_WS_FIELDS 18
moe_status moe_workspace_layout(const moe_dims* d, size_t offsets[MOE_WS_FIELDS]);

/* Library version string (static storage). */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif
