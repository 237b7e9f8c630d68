/*
 * oracle.c -- plain, slow, obviously correct CPU oracle of one wide-batch decode
 * step of a latent mixture-of-experts layer (TP1, one device).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, header,
 * table or constant with the GPU library; the two meet only in the seeded input
 * generator, which holds none of the method's arithmetic.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math).  Every dot product is
 * accumulated in double and rounded once; every rounding is round-to-nearest-even.
 *
 * Sources (the pages):
 *   [wide]     vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.wide
 *   [ep]       vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.moe.ep.layer
 *   [finalize] vllm.models.glm5next.nvidia.specialized_decode.cutedsl.finalize_publish
 *
 * Parity status: every function here is pinned by a CPU test against a closed form,
 * a brute force, or an independent library routine, except where a header comment
 * says "parity unpinned" (the readings the pages leave open: the gated activation,
 * the MXFP8 scale rule, the defined exponential).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* thread count of the parallel loops (timing only: results do not depend on it) */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ============================ codecs ============================================= */

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* magnitude of a BF16 pattern as a double, treating the all-ones exponent as 2^128
   (the value an unbounded exponent would give); used only to compare distances */
static double bf16_mag_unbounded(uint16_t b) {
    int e = (b >> 7) & 0xFF, m = b & 0x7F;
    if (e == 0) return ldexp((double)m, -133);
    return ldexp((double)(128 + m), e - 134);
}

/* Round-to-nearest-even by brute force: the two BF16 neighbours of f that share its
   sign are the truncation and the next pattern up; pick the nearer, ties to even. */
uint16_t orc_f32_to_bf16(float f) {
    if (isnan(f)) return 0x7FC0;
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t lo = (uint16_t)(u >> 16);
    if (orc_bf16_to_f32(lo) == f) return lo; /* exact, or +-inf */
    uint16_t hi = (uint16_t)(lo + 1);
    double a = fabs((double)f);
    double dlo = a - bf16_mag_unbounded(lo);
    double dhi = bf16_mag_unbounded(hi) - a;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi; /* 0x7F80 / 0xFF80 = +-inf on overflow */
    return (lo & 1) ? hi : lo;
}

static uint16_t bf16_of(double v) { return orc_f32_to_bf16((float)v); }

/* OCP MX v1.0 element formats: E4M3 and E2M1 elements, one E8M0 scale per 32.  The
   pages name MXFP8 activations and MXFP4 expert weights ([wide] module summary,
   precision paragraph) but print no codec. */
double orc_e4m3_value(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* nearest finite E4M3 value by exhaustive search, ties to the even code, saturating
   at +-448; the sign of a zero result is kept */
uint8_t orc_e4m3_encode(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int best = 0;
    double bestd = a;
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - orc_e4m3_value((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(sign | best);
}

double orc_e2m1_value(uint8_t nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

double orc_e8m0_value(uint8_t b) {
    if (b == 0xFF) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* ============================ routing ============================================ */

/* The pages route with the stock sigmoid top-16 ([ep] EpMoeLayer.topk: one group, a
   sigmoid score, the correction bias, renormalisation, the routed scale) but never
   state the exponential.
   Routing ids must be bit-exact across implementations, so the exponential is
   defined here from a textbook method (Cody and Waite's argument reduction
   z = n ln2 + r with ln2 split into a 16-significant-bit head and a tail, then the
   degree-7 Taylor polynomial of e^r by Horner's rule, then a scaling by 2^n), each
   step one IEEE FP32 operation.  Parity unpinned against the pages (they print no
   sigmoid); pinned against exp() by an ulp bound. */
static float C_LOG2E, C_LN2_HI, C_LN2_LO, C_TAYLOR[8];
static int c_ready = 0;

static void init_constants(void) {
    if (c_ready) return;
    C_LOG2E = (float)M_LOG2E;
    C_LN2_HI = (float)(nearbyint(M_LN2 * 65536.0) / 65536.0);
    C_LN2_LO = (float)(M_LN2 - (double)C_LN2_HI);
    double f = 1.0;
    for (int k = 0; k < 8; ++k) {
        if (k > 0) f *= k;
        C_TAYLOR[k] = (float)(1.0 / f);
    }
    c_ready = 1;
}

void orc_sigmoid_constants(float out[11]) {
    init_constants();
    out[0] = C_LOG2E;
    out[1] = C_LN2_HI;
    out[2] = C_LN2_LO;
    for (int k = 0; k < 8; ++k) out[3 + k] = C_TAYLOR[k];
}

float orc_exp_defined(float z) {
    init_constants();
    float nf = rintf(z * C_LOG2E);
    float r = fmaf(-nf, C_LN2_HI, z);
    r = fmaf(-nf, C_LN2_LO, r);
    float p = C_TAYLOR[7];
    for (int k = 6; k >= 0; --k) p = fmaf(p, r, C_TAYLOR[k]);
    return ldexpf(p, (int)nf);
}

float orc_sigmoid(float logit) {
    float z = -logit;
    if (z > 88.0f) return 0.0f;
    if (z < -87.0f) return 1.0f;
    float e = orc_exp_defined(z);
    float den = 1.0f + e;
    return 1.0f / den;
}

/* router logits with an FP32 output ([wide] module summary, precision paragraph;
   [ep] stock_order, where the router product is taken straight to FP32) */
void orc_linear_f32(int M, int N, int K, const uint16_t* x, const uint16_t* w, float* out) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)orc_bf16_to_f32(x[(size_t)m * K + k]) *
                       (double)orc_bf16_to_f32(w[(size_t)n * K + k]);
            out[(size_t)m * N + n] = (float)acc;
        }
}

typedef struct {
    float key;
    int e;
} key_id;

static int by_key_desc_then_id(const void* pa, const void* pb) {
    const key_id* a = (const key_id*)pa;
    const key_id* b = (const key_id*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->e < b->e) ? -1 : (a->e > b->e);
}

/* [ep] EpMoeLayer.topk / stock_order; [wide] WideRoute ("exact top16 and
   renormalized weights").  Score s = sigmoid(logit); selection key = s + bias (one
   FP32 add); the K largest keys, descending, ties to the lower expert id; weights
   are the unbiased scores of the chosen experts, summed in slot order in FP32,
   divided by the sum when renormalising, then multiplied by the routed scale. */
void orc_topk(int T, int E, int K, const float* logits, const float* bias, int renormalize,
              float scale, int32_t* ids, float* weights) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        key_id* ks = (key_id*)malloc(sizeof(key_id) * (size_t)E);
        float* s = (float*)malloc(sizeof(float) * (size_t)E);
        for (int e = 0; e < E; ++e) {
            s[e] = orc_sigmoid(logits[(size_t)t * E + e]);
            ks[e].key = s[e] + bias[e];
            ks[e].e = e;
        }
        qsort(ks, (size_t)E, sizeof(key_id), by_key_desc_then_id);
        float sum = 0.0f;
        for (int k = 0; k < K; ++k) {
            ids[(size_t)t * K + k] = ks[k].e;
            weights[(size_t)t * K + k] = s[ks[k].e];
            sum = sum + s[ks[k].e];
        }
        for (int k = 0; k < K; ++k) {
            float w = weights[(size_t)t * K + k];
            if (renormalize) w = w / sum;
            weights[(size_t)t * K + k] = w * scale;
        }
        free(ks);
        free(s);
    }
}

/* [wide] WideRoute (each (token, slot) pair appended to its expert's list, encoded
   token*16 + slot) and the module summary (the routing lists are cut into windows of 8
   tokens, and the grouped engine passes over a touched expert's weights once per such
   window).  The pages fill
   lists with atomic claims, so the order inside a list is theirs to choose; here a
   list holds its pairs in ascending pair id.  A unit is a window of unit_tokens
   consecutive entries of one list: (expert, first list entry, window length, the
   expert's list length on its first window and 0 on later ones).  The units list the
   first window of every touched expert (experts ascending), then every later window
   (experts ascending, windows in list order).  num_units = (units, dropped pairs,
   touched experts, 0).
   A pair whose id lies outside [0,E), or whose expert already appeared at an earlier
   slot of the same token, is dropped and counted. */
int orc_build_lists(int T, int K, int E, int unit_tokens, const int32_t* ids, int32_t* counts,
                    int32_t* offsets, int32_t* pairs, int32_t* units, int32_t* num_units) {
    int P = T * K;
    char* listed = (char*)calloc((size_t)(P > 0 ? P : 1), 1);
    int dropped = 0;
    for (int p = 0; p < P; ++p) {
        int e = ids[p];
        int ok = (e >= 0 && e < E);
        int t = p / K;
        for (int q = t * K; ok && q < p; ++q)
            if (ids[q] == e) ok = 0;
        listed[p] = (char)ok;
        if (!ok) ++dropped;
    }
    for (int e = 0; e < E; ++e) {
        counts[e] = 0;
        for (int p = 0; p < P; ++p)
            if (listed[p] && ids[p] == e) ++counts[e];
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int n = 0;
    for (int e = 0; e < E; ++e)
        for (int p = 0; p < P; ++p)
            if (listed[p] && ids[p] == e) pairs[n++] = p;
    /* the first window of every touched expert, experts ascending, then every later
       window, experts ascending and windows in list order */
    int u = 0, touched = 0;
    for (int e = 0; e < E; ++e)
        if (counts[e] > 0) {
            units[4 * u + 0] = e;
            units[4 * u + 1] = offsets[e];
            units[4 * u + 2] = counts[e] < unit_tokens ? counts[e] : unit_tokens;
            units[4 * u + 3] = counts[e];
            ++u;
            ++touched;
        }
    for (int e = 0; e < E; ++e)
        for (int j = 1; j * unit_tokens < counts[e]; ++j) {
            int rest = counts[e] - j * unit_tokens;
            units[4 * u + 0] = e;
            units[4 * u + 1] = offsets[e] + j * unit_tokens;
            units[4 * u + 2] = rest < unit_tokens ? rest : unit_tokens;
            units[4 * u + 3] = 0;
            ++u;
        }
    num_units[0] = u;
    num_units[1] = dropped;
    num_units[2] = touched;
    num_units[3] = 0;
    free(listed);
    return dropped;
}

/* ============================ MXFP8 quantisation ================================== */

/* One 32-element block ([wide] module summary: the latent becomes the experts' MXFP8
   input, and the expert hidden is MXFP8 as well).  The pages name the
   quantiser but not its scale rule; this is the OCP MX v1.0 rule: shared exponent
   X = floor(log2(amax)) - 8 (8 = the largest E4M3 exponent), clamped to the E8M0
   range, elements v / 2^X rounded to the nearest E4M3 value with saturation.  An
   all-zero block gets scale byte 0 and signed-zero codes.  Parity unpinned against
   the pages' quantiser (not printed); pinned against brute force and the OCP
   definition. */
static void quant_block(const double* v, uint8_t* codes, uint8_t* scale) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i)
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) {
        *scale = 0;
        for (int i = 0; i < 32; ++i) codes[i] = signbit(v[i]) ? 0x80 : 0x00;
        return;
    }
    int ex;
    frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5,1): floor(log2 amax) = ex - 1 */
    int x = (ex - 1) - 8;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    *scale = (uint8_t)(x + 127);
    for (int i = 0; i < 32; ++i) codes[i] = orc_e4m3_encode(ldexp(v[i], -x));
}

void orc_quant_mxfp8_bf16(int rows, int cols, const uint16_t* x, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < cols / 32; ++b) {
            double v[32];
            for (int i = 0; i < 32; ++i) v[i] = orc_bf16_to_f32(x[(size_t)r * cols + 32 * b + i]);
            quant_block(v, codes + (size_t)r * cols + 32 * b, scales + (size_t)r * (cols / 32) + b);
        }
}

void orc_quant_mxfp8_f32(int rows, int cols, const float* x, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < cols / 32; ++b) {
            double v[32];
            for (int i = 0; i < 32; ++i) v[i] = x[(size_t)r * cols + 32 * b + i];
            quant_block(v, codes + (size_t)r * cols + 32 * b, scales + (size_t)r * (cols / 32) + b);
        }
}

/* ============================ grouped expert FFN ================================== */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* MXFP4 weight row: element j sits in byte j/2, the even element in the low nibble;
   one E8M0 scale per 32 elements along the row (the fan-in axis). */
static void dequant_mxfp4_row(const uint8_t* bytes, const uint8_t* sc, int n, double* out) {
    for (int j = 0; j < n; ++j) {
        uint8_t b = bytes[j / 2];
        uint8_t nib = (j & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
        out[j] = orc_e2m1_value(nib) * orc_e8m0_value(sc[j / 32]);
    }
}

static void dequant_mxfp8_row(const uint8_t* codes, const uint8_t* sc, int n, double* out) {
    for (int j = 0; j < n; ++j) out[j] = orc_e4m3_value(codes[j]) * orc_e8m0_value(sc[j / 32]);
}

/* First half of one expert on one pair ([wide] module summary, the grouped expert
   engine over the routing lists; [ep] EpRouted, the stock MXFP4 x MXFP8 routed MoE with
   its gated activation): h = A W13^T over the dequantised MXFP8 latent row of token p/K
   (FP32 from a double sum), act = silu(gate) * up on the two halves (gate first),
   then act is quantised to MXFP8 from FP32.  The pages' gated activation (SiTU) is
   never defined; SiLU-and-mul is used -- parity unpinned against the pages. */
void orc_ffn_up_mx(int n, const int32_t* pair_ids, const int32_t* pair_experts, int K, int L, int I,
                   const uint8_t* codes, const uint8_t* scales, const uint8_t* w13,
                   const uint8_t* s13, uint8_t* hid_codes, uint8_t* hid_scales, float* hid_f32) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
        int t = pair_ids[i] / K, e = pair_experts[i];
        double* a = (double*)malloc(sizeof(double) * (size_t)L);
        double* w = (double*)malloc(sizeof(double) * (size_t)L);
        float* h = (float*)malloc(sizeof(float) * (size_t)(2 * I));
        float* act = (float*)malloc(sizeof(float) * (size_t)I);
        dequant_mxfp8_row(codes + (size_t)t * L, scales + (size_t)t * (L / 32), L, a);
        for (int r = 0; r < 2 * I; ++r) {
            size_t row = (size_t)e * 2 * I + r;
            dequant_mxfp4_row(w13 + row * (L / 2), s13 + row * (L / 32), L, w);
            double acc = 0.0;
            for (int j = 0; j < L; ++j) acc += a[j] * w[j];
            h[r] = (float)acc;
        }
        for (int j = 0; j < I; ++j) act[j] = (float)(silu((double)h[j]) * (double)h[I + j]);
        if (hid_f32) memcpy(hid_f32 + (size_t)i * I, act, sizeof(float) * (size_t)I);
        orc_quant_mxfp8_f32(1, I, act, hid_codes + (size_t)i * I, hid_scales + (size_t)i * (I / 32));
        free(a);
        free(w);
        free(h);
        free(act);
    }
}

/* Second half: y = act_q W2^T (FP32 from a double sum), rounded to BF16 into the
   pair's expanded row ([wide] module summary: "FP32 accumulation of the BF16 top16
   rows" -- the rows are BF16). */
void orc_ffn_down_mx(int n, const int32_t* pair_experts, int L, int I, const uint8_t* hid_codes,
                     const uint8_t* hid_scales, const uint8_t* w2, const uint8_t* s2,
                     uint16_t* rows) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
        int e = pair_experts[i];
        double* a = (double*)malloc(sizeof(double) * (size_t)I);
        double* w = (double*)malloc(sizeof(double) * (size_t)I);
        dequant_mxfp8_row(hid_codes + (size_t)i * I, hid_scales + (size_t)i * (I / 32), I, a);
        for (int r = 0; r < L; ++r) {
            size_t row = (size_t)e * L + r;
            dequant_mxfp4_row(w2 + row * (I / 2), s2 + row * (I / 32), I, w);
            double acc = 0.0;
            for (int j = 0; j < I; ++j) acc += a[j] * w[j];
            rows[(size_t)i * L + r] = bf16_of((float)acc);
        }
        free(a);
        free(w);
    }
}

/* BF16-weight expert (the toy configuration: "all weights BF16 ... no
   quantisation"): every linear rounds its output to BF16 once. */
void orc_ffn_bf16(int n, const int32_t* pair_ids, const int32_t* pair_experts, int K, int L, int I,
                  const uint16_t* latent, const uint16_t* w13, const uint16_t* w2, uint16_t* rows) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
        int t = pair_ids[i] / K, e = pair_experts[i];
        float* h = (float*)malloc(sizeof(float) * (size_t)(2 * I));
        float* act = (float*)malloc(sizeof(float) * (size_t)I);
        for (int r = 0; r < 2 * I; ++r) {
            double acc = 0.0;
            for (int j = 0; j < L; ++j)
                acc += (double)orc_bf16_to_f32(latent[(size_t)t * L + j]) *
                       (double)orc_bf16_to_f32(w13[((size_t)e * 2 * I + r) * L + j]);
            h[r] = orc_bf16_to_f32(bf16_of((float)acc));
        }
        for (int j = 0; j < I; ++j)
            act[j] = orc_bf16_to_f32(bf16_of(silu((double)h[j]) * (double)h[I + j]));
        for (int r = 0; r < L; ++r) {
            double acc = 0.0;
            for (int j = 0; j < I; ++j)
                acc += (double)act[j] * (double)orc_bf16_to_f32(w2[((size_t)e * L + r) * I + j]);
            rows[(size_t)i * L + r] = bf16_of((float)acc);
        }
        free(h);
        free(act);
    }
}

/* ============================ combine ============================================ */

/* [wide] Finalize: out[t] = sum_k w[t,k] * rows[K t + k], FP32 with k in order (one
   fused multiply-add per slot), one BF16 rounding at the end.  [finalize]
   _QuadFinalizePublishDeviceKernel: a slot whose row index is -1 has weight zero and
   its row is not read; here any negative id marks such a slot. */
void orc_finalize(int T, int K, int cols, const uint16_t* rows, const float* weights,
                  const int32_t* ids, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < cols; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                if (ids && ids[(size_t)t * K + k] < 0) continue;
                float v = orc_bf16_to_f32(rows[((size_t)t * K + k) * cols + c]);
                acc = fmaf(weights[(size_t)t * K + k], v, acc);
            }
            out[(size_t)t * cols + c] = orc_f32_to_bf16(acc);
        }
}

/* [ep] EpMoeLayer: ops.rms_norm(normed, routed, norm, eps=1e-5) on the routed
   latent.  n = r / sqrt(mean(r^2) + eps) * g in double, one BF16 rounding (the
   stock kernel's internal rounding points are not on the pages). */
void orc_rmsnorm(int T, int cols, const uint16_t* r, const uint16_t* g, float eps, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int c = 0; c < cols; ++c) {
            double v = orc_bf16_to_f32(r[(size_t)t * cols + c]);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / cols + (double)eps);
        for (int c = 0; c < cols; ++c)
            out[(size_t)t * cols + c] = bf16_of((double)orc_bf16_to_f32(r[(size_t)t * cols + c]) *
                                                inv * (double)orc_bf16_to_f32(g[c]));
    }
}

/* ============================ dense linears ====================================== */

/* BF16 linear with FP32 accumulation and one BF16 rounding ([wide] module summary,
   precision paragraph: the dense projections are BF16, and the latent is rounded to
   BF16 once) */
void orc_linear_bf16(int M, int N, int K, const uint16_t* x, const uint16_t* w, uint16_t* out) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)orc_bf16_to_f32(x[(size_t)m * K + k]) *
                       (double)orc_bf16_to_f32(w[(size_t)n * K + k]);
            out[(size_t)m * N + n] = orc_f32_to_bf16((float)acc);
        }
}

/* [ep] EpMoeLayer: shared.addmm_(normed, up.T) -- the up-projection added into the
   BF16 shared partial with one rounding, as the stock path does (the [ep] module
   summary notes the single rounding of the library addmm). */
void orc_linear_add_bf16(int M, int N, int K, const uint16_t* x, const uint16_t* w,
                         const uint16_t* add, uint16_t* out) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)orc_bf16_to_f32(x[(size_t)m * K + k]) *
                       (double)orc_bf16_to_f32(w[(size_t)n * K + k]);
            float sum = orc_bf16_to_f32(add[(size_t)m * N + n]) + (float)acc;
            out[(size_t)m * N + n] = orc_f32_to_bf16(sum);
        }
}

/* [ep] EpMoeLayer.gate_up / stock_order: the stock gated activation on the [T, 2S]
   gate_up rows, gate in the first half.  SiLU-and-mul stands in for the undefined
   SiTU (parity unpinned against the pages). */
void orc_silu_mul_bf16(int M, int S, const uint16_t* gu, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int j = 0; j < S; ++j) {
            double g = orc_bf16_to_f32(gu[(size_t)m * 2 * S + j]);
            double u = orc_bf16_to_f32(gu[(size_t)m * 2 * S + S + j]);
            out[(size_t)m * S + j] = bf16_of(silu(g) * u);
        }
}

/* ============================ the layer ========================================== */

/* [ep] EpMoeLayer.stock_order at TP1 with the [wide] precision chain: router logits
   -> sigmoid top-K -> lists and units -> latent down (BF16) -> MXFP8 latent ->
   grouped experts -> Finalize -> RMSNorm -> shared expert -> up-projection added
   into the shared partial.  No all-reduce (one device). */
void orc_layer(const orc_dims* d, const orc_weights* w, const uint16_t* x, uint16_t* out,
               orc_trace* tr) {
    int T = d->T, H = d->H, L = d->L, E = d->E, K = d->K, I = d->I, S = d->S;
    size_t P = (size_t)T * K;
    float* logits = (float*)malloc(sizeof(float) * (size_t)T * E);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * P);
    float* wts = (float*)malloc(sizeof(float) * P);
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* pairs = (int32_t*)malloc(sizeof(int32_t) * (P > 0 ? P : 1));
    int32_t* units = (int32_t*)malloc(sizeof(int32_t) * 4 * (P + (size_t)E + 1));
    int32_t nu[4];
    int32_t* pexp = (int32_t*)malloc(sizeof(int32_t) * (P > 0 ? P : 1));
    uint16_t* latent = (uint16_t*)malloc(2 * (size_t)T * L);
    uint8_t* codes = (uint8_t*)malloc((size_t)T * L);
    uint8_t* scales = (uint8_t*)malloc((size_t)T * L / 32 + 1);
    uint16_t* rows_listed = (uint16_t*)malloc(2 * P * L);
    uint16_t* rows = (uint16_t*)malloc(2 * P * L);
    uint16_t* routed = (uint16_t*)malloc(2 * (size_t)T * L);
    uint16_t* normed = (uint16_t*)malloc(2 * (size_t)T * L);
    uint16_t* gu = (uint16_t*)malloc(2 * (size_t)T * 2 * S);
    uint16_t* act = (uint16_t*)malloc(2 * (size_t)T * S);
    uint16_t* shared = (uint16_t*)malloc(2 * (size_t)T * H);

    orc_linear_f32(T, E, H, x, w->w_gate, logits);
    orc_topk(T, E, K, logits, w->bias, d->renormalize, d->routed_scale, ids, wts);
    orc_build_lists(T, K, E, d->unit_tokens, ids, counts, offsets, pairs, units, nu);
    for (size_t i = 0; i < (size_t)offsets[E]; ++i) pexp[i] = ids[pairs[i]];
    orc_linear_bf16(T, L, H, x, w->w_down, latent);
    int n = offsets[E];
    if (d->expert_format == 0) {
        orc_quant_mxfp8_bf16(T, L, latent, codes, scales);
        uint8_t* hc = (uint8_t*)malloc((size_t)n * I + 1);
        uint8_t* hs = (uint8_t*)malloc((size_t)n * I / 32 + 1);
        orc_ffn_up_mx(n, pairs, pexp, K, L, I, codes, scales, (const uint8_t*)w->w13,
                      (const uint8_t*)w->s13, hc, hs, NULL);
        orc_ffn_down_mx(n, pexp, L, I, hc, hs, (const uint8_t*)w->w2, (const uint8_t*)w->s2,
                        rows_listed);
        free(hc);
        free(hs);
    } else {
        orc_ffn_bf16(n, pairs, pexp, K, L, I, latent, (const uint16_t*)w->w13,
                     (const uint16_t*)w->w2, rows_listed);
    }
    memset(rows, 0, 2 * P * L);
    for (int i = 0; i < n; ++i)
        memcpy(rows + (size_t)pairs[i] * L, rows_listed + (size_t)i * L, 2 * (size_t)L);
    orc_finalize(T, K, L, rows, wts, NULL, routed);
    orc_rmsnorm(T, L, routed, w->norm_w, d->rms_eps, normed);
    orc_linear_bf16(T, 2 * S, H, x, w->w_shared_gu, gu);
    orc_silu_mul_bf16(T, S, gu, act);
    orc_linear_bf16(T, H, S, act, w->w_shared_dn, shared);
    orc_linear_add_bf16(T, H, L, normed, w->w_up, shared, out);

    if (tr) {
        if (tr->logits) memcpy(tr->logits, logits, sizeof(float) * (size_t)T * E);
        if (tr->ids) memcpy(tr->ids, ids, sizeof(int32_t) * P);
        if (tr->weights) memcpy(tr->weights, wts, sizeof(float) * P);
        if (tr->latent) memcpy(tr->latent, latent, 2 * (size_t)T * L);
        if (tr->codes && d->expert_format == 0) memcpy(tr->codes, codes, (size_t)T * L);
        if (tr->scales && d->expert_format == 0) memcpy(tr->scales, scales, (size_t)T * L / 32);
        if (tr->rows) memcpy(tr->rows, rows, 2 * P * L);
        if (tr->routed) memcpy(tr->routed, routed, 2 * (size_t)T * L);
        if (tr->normed) memcpy(tr->normed, normed, 2 * (size_t)T * L);
        if (tr->shared) memcpy(tr->shared, shared, 2 * (size_t)T * H);
    }
    free(logits); free(ids); free(wts); free(counts); free(offsets); free(pairs); free(units);
    free(pexp); free(latent); free(codes); free(scales); free(rows_listed); free(rows);
    free(routed); free(normed); free(gu); free(act); free(shared);
}
