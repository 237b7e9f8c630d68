/*
 * sanitize_main.c -- drives every function of the CPU oracle (oracle.c) once on small
 * inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer.  TEST
 * INFRASTRUCTURE ONLY (the CPU test tier builds and runs it); it checks no numerics
 * (the pins do that), only that every access stays in bounds and no operation is
 * undefined, including the edge cases: an expert id outside [0, E), a repeated id, an
 * invalid Finalize slot, an all-zero MXFP8 block, saturating and subnormal values, a
 * single token, and both expert formats of the whole layer.
 *
 * Build: gcc -std=c11 -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all
 *        -ffp-contract=off oracle.c sanitize_main.c -lm
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* SplitMix64: a test driver's source of arbitrary bytes */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform(void) { return (double)(next_u64() >> 11) * 0x1.0p-53; }

/* BF16 bits of a value of about the given spread (truncation) */
static uint16_t bf16_rand(double scale) {
    float f = (float)((uniform() * 2.0 - 1.0) * scale);
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static uint16_t* bf16_array(size_t n, double scale) {
    uint16_t* a = xmalloc(2 * n);
    for (size_t i = 0; i < n; ++i) a[i] = bf16_rand(scale);
    return a;
}

static uint8_t* byte_array(size_t n, int lo, int hi) {
    uint8_t* a = xmalloc(n);
    for (size_t i = 0; i < n; ++i) a[i] = (uint8_t)(lo + (int)(next_u64() % (uint64_t)(hi - lo + 1)));
    return a;
}

static double checksum = 0.0;

static void mix_f32(const float* a, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (isfinite(a[i])) checksum += a[i];
}

static void mix_u16(const uint16_t* a, size_t n) {
    for (size_t i = 0; i < n; ++i) checksum += a[i];
}

static void mix_u8(const uint8_t* a, size_t n) {
    for (size_t i = 0; i < n; ++i) checksum += a[i];
}

static void codecs(void) {
    for (int c = 0; c < 256; ++c) {
        checksum += isnan(orc_e4m3_value((uint8_t)c)) ? 0 : orc_e4m3_value((uint8_t)c);
        checksum += orc_e4m3_encode((double)(c - 128) * 3.7);
        checksum += orc_e2m1_value((uint8_t)c);
        if (c != 255) checksum += orc_e8m0_value((uint8_t)c) > 0;
    }
    for (uint32_t b = 0; b < 65536; b += 7) {
        float f = orc_bf16_to_f32((uint16_t)b);
        if (!isnan(f)) checksum += orc_f32_to_bf16(f * 1.001f);
    }
    checksum += orc_e4m3_encode(1e9) + orc_e4m3_encode(-1e9) + orc_e4m3_encode(-0.0);
    float c11[11];
    orc_sigmoid_constants(c11);
    mix_f32(c11, 11);
    const float zs[] = {-100.f, -87.5f, -87.f, -1.f, 0.f, 1e-8f, 1.f, 88.f, 88.5f, 100.f};
    for (size_t i = 0; i < sizeof zs / sizeof zs[0]; ++i)
        checksum += orc_sigmoid(zs[i]) + (fabsf(zs[i]) < 88.f ? orc_exp_defined(zs[i]) : 0.f);
}

static void routing_and_lists(void) {
    const int T = 13, E = 40, K = 6, H = 64;
    uint16_t* x = bf16_array((size_t)T * H, 2.0);
    uint16_t* wg = bf16_array((size_t)E * H, 0.2);
    float* logits = xmalloc(sizeof(float) * T * E);
    float* bias = xmalloc(sizeof(float) * E);
    for (int e = 0; e < E; ++e) bias[e] = (float)(uniform() * 0.1);
    orc_linear_f32(T, E, H, x, wg, logits);
    int32_t* ids = xmalloc(sizeof(int32_t) * T * K);
    float* w = xmalloc(sizeof(float) * T * K);
    orc_topk(T, E, K, logits, bias, 1, 2.5f, ids, w);
    orc_topk(T, E, K, logits, bias, 0, 1.0f, ids, w);
    mix_f32(w, (size_t)T * K);
    /* out-of-range and repeated ids are dropped and counted */
    ids[0] = -3;
    ids[1] = E + 5;
    ids[3] = ids[2];
    for (int unit = 8; unit <= 16; unit += 8) {
        int32_t* counts = xmalloc(sizeof(int32_t) * E);
        int32_t* offsets = xmalloc(sizeof(int32_t) * (E + 1));
        int32_t* pairs = xmalloc(sizeof(int32_t) * T * K);
        int32_t* units = xmalloc(sizeof(int32_t) * 4 * ((size_t)T * K / unit + 1 + E));
        int32_t nu[4];
        checksum += orc_build_lists(T, K, E, unit, ids, counts, offsets, pairs, units, nu);
        checksum += nu[0] + nu[1] + nu[2] + offsets[E];
        free(counts), free(offsets), free(pairs), free(units);
    }
    /* one expert chosen by every token: several windows of one list */
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) ids[t * K + k] = k == 0 ? 7 : (t + k) % E;
    {
        int32_t counts[40], offsets[41], pairs[13 * 6], units[4 * (13 * 6 / 8 + 1 + 40)], nu[4];
        orc_build_lists(T, K, E, 8, ids, counts, offsets, pairs, units, nu);
        checksum += nu[0];
    }
    free(x), free(wg), free(logits), free(bias), free(ids), free(w);
}

static void quant(void) {
    const int R = 5, C = 96;
    uint16_t* x = bf16_array((size_t)R * C, 100.0);
    for (int i = 0; i < 32; ++i) x[i] = (i & 1) ? 0x8000 : 0x0000; /* an all-zero block */
    for (int i = 32; i < 64; ++i) x[i] = (uint16_t)(0x0001 + i);    /* BF16 subnormals */
    uint8_t* codes = xmalloc((size_t)R * C);
    uint8_t* sc = xmalloc((size_t)R * C / 32);
    orc_quant_mxfp8_bf16(R, C, x, codes, sc);
    mix_u8(codes, (size_t)R * C), mix_u8(sc, (size_t)R * C / 32);
    float* f = xmalloc(sizeof(float) * R * C);
    for (int i = 0; i < R * C; ++i) f[i] = (float)((uniform() - 0.5) * 1e6);
    f[5] = 3e38f;
    f[6] = 1e-42f;
    orc_quant_mxfp8_f32(R, C, f, codes, sc);
    mix_u8(codes, (size_t)R * C), mix_u8(sc, (size_t)R * C / 32);
    free(x), free(codes), free(sc), free(f);
}

static void experts_and_combine(void) {
    const int T = 7, K = 3, L = 64, I = 64, E = 5, n = T * K;
    int32_t pid[21], pex[21];
    for (int i = 0; i < n; ++i) pid[i] = i, pex[i] = (i * 3) % E;
    uint8_t* codes = byte_array((size_t)T * L, 0, 0x7E);
    uint8_t* sc = byte_array((size_t)T * L / 32, 110, 130);
    uint8_t* w13 = byte_array((size_t)E * 2 * I * L / 2, 0, 255);
    uint8_t* s13 = byte_array((size_t)E * 2 * I * L / 32, 115, 125);
    uint8_t* w2 = byte_array((size_t)E * L * I / 2, 0, 255);
    uint8_t* s2 = byte_array((size_t)E * L * I / 32, 115, 125);
    uint8_t* hc = xmalloc((size_t)n * I);
    uint8_t* hs = xmalloc((size_t)n * I / 32);
    float* hf = xmalloc(sizeof(float) * n * I);
    uint16_t* rows = xmalloc(2 * (size_t)n * L);
    orc_ffn_up_mx(n, pid, pex, K, L, I, codes, sc, w13, s13, hc, hs, hf);
    orc_ffn_up_mx(n, pid, pex, K, L, I, codes, sc, w13, s13, hc, hs, NULL);
    orc_ffn_down_mx(n, pex, L, I, hc, hs, w2, s2, rows);
    mix_u16(rows, (size_t)n * L);
    uint16_t* lat = bf16_array((size_t)T * L, 1.0);
    uint16_t* b13 = bf16_array((size_t)E * 2 * I * L, 0.1);
    uint16_t* b2 = bf16_array((size_t)E * L * I, 0.1);
    orc_ffn_bf16(n, pid, pex, K, L, I, lat, b13, b2, rows);
    mix_u16(rows, (size_t)n * L);
    float* w = xmalloc(sizeof(float) * n);
    int32_t ids[21];
    for (int i = 0; i < n; ++i) w[i] = (float)uniform(), ids[i] = (i % 4 == 1) ? -1 : i % E;
    uint16_t* out = xmalloc(2 * (size_t)T * L);
    orc_finalize(T, K, L, rows, w, NULL, out);
    orc_finalize(T, K, L, rows, w, ids, out);
    uint16_t* g = bf16_array(L, 1.0);
    uint16_t* nrm = xmalloc(2 * (size_t)T * L);
    orc_rmsnorm(T, L, out, g, 1e-5f, nrm);
    mix_u16(nrm, (size_t)T * L);
    uint16_t* wl = bf16_array((size_t)L * L, 0.1);
    uint16_t* lo = xmalloc(2 * (size_t)T * L);
    orc_linear_bf16(T, L, L, nrm, wl, lo);
    orc_linear_add_bf16(T, L, L, nrm, wl, lo, out);
    uint16_t* act = xmalloc(2 * (size_t)T * (L / 2));
    orc_silu_mul_bf16(T, L / 2, out, act);
    mix_u16(act, (size_t)T * (L / 2));
    free(codes), free(sc), free(w13), free(s13), free(w2), free(s2), free(hc), free(hs), free(hf);
    free(rows), free(lat), free(b13), free(b2), free(w), free(out), free(g), free(nrm), free(wl);
    free(lo), free(act);
}

static void layer(int fmt, int T) {
    orc_dims d = {T, 128, 64, 16, 4, 64, 64, 8, fmt, 1, 2.5f, 1e-5f};
    const int H = d.H, L = d.L, E = d.E, I = d.I, S = d.S, K = d.K;
    uint16_t* x = bf16_array((size_t)T * H, 2.0);
    orc_weights w;
    w.w_gate = bf16_array((size_t)E * H, 0.1);
    float* bias = xmalloc(sizeof(float) * E);
    for (int e = 0; e < E; ++e) bias[e] = (float)(uniform() * 0.02);
    w.bias = bias;
    w.w_down = bf16_array((size_t)L * H, 0.1);
    w.w_shared_gu = bf16_array((size_t)2 * S * H, 0.1);
    w.w_shared_dn = bf16_array((size_t)H * S, 0.1);
    w.norm_w = bf16_array(L, 1.0);
    w.w_up = bf16_array((size_t)H * L, 0.1);
    void *w13, *s13 = NULL, *w2, *s2 = NULL;
    if (fmt == 0) {
        w13 = byte_array((size_t)E * 2 * I * L / 2, 0, 255);
        s13 = byte_array((size_t)E * 2 * I * L / 32, 118, 124);
        w2 = byte_array((size_t)E * L * I / 2, 0, 255);
        s2 = byte_array((size_t)E * L * I / 32, 118, 124);
    } else {
        w13 = bf16_array((size_t)E * 2 * I * L, 0.1);
        w2 = bf16_array((size_t)E * L * I, 0.1);
    }
    w.w13 = w13, w.s13 = s13, w.w2 = w2, w.s2 = s2;
    uint16_t* out = xmalloc(2 * (size_t)T * H);
    orc_trace tr;
    tr.logits = xmalloc(sizeof(float) * T * E);
    tr.ids = xmalloc(sizeof(int32_t) * T * K);
    tr.weights = xmalloc(sizeof(float) * T * K);
    tr.latent = xmalloc(2 * (size_t)T * L);
    tr.codes = xmalloc((size_t)T * L);
    tr.scales = xmalloc((size_t)T * L / 32);
    tr.rows = xmalloc(2 * (size_t)T * K * L);
    tr.routed = xmalloc(2 * (size_t)T * L);
    tr.normed = xmalloc(2 * (size_t)T * L);
    tr.shared = xmalloc(2 * (size_t)T * H);
    orc_layer(&d, &w, x, out, &tr);
    orc_layer(&d, &w, x, out, NULL);
    mix_u16(out, (size_t)T * H);
    free(x), free((void*)w.w_gate), free(bias), free((void*)w.w_down), free((void*)w.w_shared_gu);
    free((void*)w.w_shared_dn), free((void*)w.norm_w), free((void*)w.w_up);
    free(w13), free(s13), free(w2), free(s2), free(out);
    free(tr.logits), free(tr.ids), free(tr.weights), free(tr.latent), free(tr.codes);
    free(tr.scales), free(tr.rows), free(tr.routed), free(tr.normed), free(tr.shared);
}

int main(void) {
    codecs();
    routing_and_lists();
    quant();
    experts_and_combine();
    layer(0, 1);
    layer(0, 19);
    layer(1, 9);
    printf("oracle sanitizer run ok (checksum %.6g)\n", checksum);
    return 0;
}
