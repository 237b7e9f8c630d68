/*
 * oracle.h -- the plain CPU oracle of one wide-batch decode step of a latent
 * mixture-of-experts layer.  TEST INFRASTRUCTURE ONLY: only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  The GPU library
 * never includes, links or calls anything declared here, and this file includes
 * nothing from the GPU library.
 *
 * Sources (the three vLLM API pages the method is stated on):
 *   [wide]     "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.wide"
 *   [ep]       "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.ep.layer"
 *   [finalize] "vllm.models.glm5next.nvidia.specialized_decode.cutedsl.finalize_publish"
 *
 * Conventions: BF16 values travel as uint16_t bit patterns; every dot product is
 * accumulated in double and rounded once to FP32 where the method keeps an FP32
 * accumulator; every rounding is round-to-nearest-even.  Arrays are row-major.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codecs ---------------------------------------------------------------- */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);          /* RNE; NaN -> 0x7FC0 */
double   orc_e4m3_value(uint8_t code);      /* NaN for 0x7F / 0xFF */
uint8_t  orc_e4m3_encode(double v);         /* nearest finite, ties to even code, saturating */
double   orc_e2m1_value(uint8_t nibble);    /* low 4 bits used */
double   orc_e8m0_value(uint8_t byte);      /* 2^(byte-127); NaN for 0xFF */

/* ---- routing ----------------------------------------------------------------- */
float orc_exp_defined(float z);             /* Cody-Waite + degree-7 Taylor */
float orc_sigmoid(float logit);             /* 1 / (1 + exp_defined(-logit)) */
void  orc_sigmoid_constants(float out[11]); /* log2e, ln2_hi, ln2_lo, c0..c7 */

void orc_linear_f32(int M, int N, int K, const uint16_t* x, const uint16_t* w, float* out);
void orc_topk(int T, int E, int K, const float* logits, const float* bias, int renormalize,
              float scale, int32_t* ids, float* weights);
/* returns the number of dropped pairs (expert id outside [0,E) or repeated in a token);
   units [n,4] = (expert, first list entry, window length, list length on the first
   window of an expert else 0), first windows first; num_units[4] = (units, dropped,
   touched experts, 0) */
int  orc_build_lists(int T, int K, int E, int unit_tokens, const int32_t* ids, int32_t* counts,
                     int32_t* offsets, int32_t* pairs, int32_t* units, int32_t* num_units);

/* ---- MX quantisation ----------------------------------------------------------- */
void orc_quant_mxfp8_bf16(int rows, int cols, const uint16_t* x, uint8_t* codes, uint8_t* scales);
void orc_quant_mxfp8_f32(int rows, int cols, const float* x, uint8_t* codes, uint8_t* scales);

/* ---- grouped expert FFN (per listed pair) --------------------------------------- */
void orc_ffn_up_mx(int n, const int32_t* pair_ids, const int32_t* pair_experts, int K, int L, int I,
                   const uint8_t* codes, const uint8_t* scales, const uint8_t* w13,
                   const uint8_t* s13, uint8_t* hid_codes, uint8_t* hid_scales, float* hid_f32);
void orc_ffn_down_mx(int n, const int32_t* pair_experts, int L, int I, const uint8_t* hid_codes,
                     const uint8_t* hid_scales, const uint8_t* w2, const uint8_t* s2,
                     uint16_t* rows);
void orc_ffn_bf16(int n, const int32_t* pair_ids, const int32_t* pair_experts, int K, int L, int I,
                  const uint16_t* latent, const uint16_t* w13, const uint16_t* w2, uint16_t* rows);

/* ---- combine ---------------------------------------------------------------------- */
void orc_finalize(int T, int K, int cols, const uint16_t* rows, const float* weights,
                  const int32_t* ids, uint16_t* out);
void orc_rmsnorm(int T, int cols, const uint16_t* r, const uint16_t* g, float eps, uint16_t* out);

/* ---- dense BF16 linears and the shared expert ---------------------------------------- */
void orc_linear_bf16(int M, int N, int K, const uint16_t* x, const uint16_t* w, uint16_t* out);
void orc_linear_add_bf16(int M, int N, int K, const uint16_t* x, const uint16_t* w,
                         const uint16_t* add, uint16_t* out);
void orc_silu_mul_bf16(int M, int S, const uint16_t* gu, uint16_t* out);

/* ---- the whole layer, stock order at TP1 --------------------------------------------- */
typedef struct {
    int T, H, L, E, K, I, S, unit_tokens, expert_format /* 0 MXFP4xMXFP8, 1 BF16 */, renormalize;
    float routed_scale, rms_eps;
} orc_dims;

typedef struct {
    const uint16_t *w_gate;      /* [E,H]   */
    const float    *bias;        /* [E]     */
    const uint16_t *w_down;      /* [L,H]   */
    const uint16_t *w_shared_gu; /* [2S,H]  */
    const uint16_t *w_shared_dn; /* [H,S]   */
    const uint16_t *norm_w;      /* [L]     */
    const uint16_t *w_up;        /* [H,L]   */
    const void *w13, *s13, *w2, *s2; /* experts: MXFP4 bytes + E8M0, or BF16 (s* unused) */
} orc_weights;

/* intermediates (any may be NULL): logits [T,E] f32, ids [T,K], w [T,K], latent [T,L],
   codes [T,L], scales [T,L/32], rows [T*K,L], routed [T,L], normed [T,L], shared [T,H] */
typedef struct {
    float *logits; int32_t *ids; float *weights; uint16_t *latent; uint8_t *codes, *scales;
    uint16_t *rows, *routed, *normed, *shared;
} orc_trace;

void orc_layer(const orc_dims* d, const orc_weights* w, const uint16_t* x, uint16_t* out,
               orc_trace* trace);

int orc_threads(void);
void orc_set_threads(int n); /* thread count of the parallel loops; results do not depend on it */

#ifdef __cplusplus
}
#endif
#endif
