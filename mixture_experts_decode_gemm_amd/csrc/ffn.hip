// ffn.hip -- the grouped expert FFN over unit windows (wide page, module summary: the
// grouped expert engine over the routing lists, whose cost is one pass over each touched
// expert's weights per window of 8 of its tokens; precision paragraph: MXFP8 activations,
// MXFP4 experts, an MXFP8 hidden; ep/layer page, EpRouted: MXFP4 x MXFP8 experts with
// the gated activation).
//
// CDNA4 path: V_MFMA_SCALE_F32_16X16X128_F8F6F4 with the weights as the A operand
// (16 weight rows x 128 K, E2M1, E8M0 per 32) and the unit's tokens as the B operand
// (128 K x 16 tokens, E4M3, E8M0 per 32).  A unit holds <= 8 tokens, so half of B's
// columns are zero; the work is bound by streaming the expert's weights from HBM.
// Operand lane layout (gfx950, measured): lane l carries row/column r = l % 16 of its
// operand and, with g = l / 16, the scale byte of K block g (elements 32g..32g+31).  An
// FP4 operand lane holds K 32g..32g+31 (16 bytes, element 2j in the low nibble of byte
// j); an FP8 operand lane holds K 16g..16g+15 in bytes 0-15 and K 64+16g..64+16g+15 in
// bytes 16-31.
//
// Two launches:
//   up   -- item = (touched expert, 32 columns j of the expert intermediate).  The four
//           wavefronts split the L/128 K-steps; each computes gate rows 32j..32j+31 and
//           up rows I+32j..I+32j+31 (four 16-row tiles) for all of the expert's tokens,
//           partial sums are added across wavefronts in LDS in a fixed order, then
//           silu(gate)*up in FP32 and the 32-column block is quantised to MXFP8 (one E8M0
//           scale per token).
//   down -- item = (touched expert, 64*MT rows of W2).  Each wavefront owns 16*MT rows
//           (MT tiles) over all I/128 K-steps; outputs are rounded to BF16 into the pairs'
//           rows.
// Both are persistent grid-stride loops over items (items i, i + G, i + 2G, ... of a
// workgroup, so that at any time the CUs read one compact window of expert weights); the
// item count comes from the device-side unit count, so every workgroup reaches the same
// exit.
#include "device.h"
#include "kernels.h"

namespace moe {

size_t ffn_scratch_bytes(int P, int I) {
    size_t codes = (size_t)P * I;
    size_t scales = (size_t)P * (I / 32);
    return ((codes + 255) / 256) * 256 + ((scales + 255) / 256) * 256 + 256;
}

// the expert passes' work counters (gate/up: 8 words, down: 8 words) in the last 256
// bytes of that scratch
size_t ffn_counter_offset(int P, int I) { return ffn_scratch_bytes(P, I) - 256; }

__global__ void k_zero_words(unsigned* p, int n) {
    if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

__device__ __forceinline__ v8i load_fp4x32(const uint8_t* p) {
    const uint4 a = *(const uint4*)p;
    v8i r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

// the FP8 operand of lane group g for the 128-element K step at `step`
__device__ __forceinline__ v8i load_fp8x32(const uint8_t* step, int g) {
    const uint4 a = *(const uint4*)(step + 16 * g);
    const uint4 b = *(const uint4*)(step + 64 + 16 * g);
    v8i r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
    return r;
}

__device__ __forceinline__ v4f mfma_fp4_fp8(v8i a, v8i b, v4f c, int sa, int sb) {
    // A format 4 = E2M1 (FP4), B format 0 = E4M3 (FP8); scale bytes in bits 7:0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, sb);
}

constexpr int UP_COLS = 32;     // intermediate columns per up item
constexpr int DOWN_ROWS = 256;  // W2 rows per down item

__device__ __forceinline__ v8i as_fp4_operand(uint4 a) {
    v8i r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
    return r;
}

// Reduce the four wavefronts' partial H tiles (K split across wavefronts, added in a
// fixed order), then act = silu(gate) * up in FP32 and one MXFP8 block of 32 columns
// per token, written by pair id.  `red` and `hbuf` are LDS; called by all 256 threads.
// `pair` is the pair id of token n0 + (lane % 16) (valid where that token exists); it
// is exchanged by lane shuffles, so the epilogue issues no global load (a load here
// would have to wait behind every prefetch still in flight).
__device__ __forceinline__ void up_epilogue_lds(const v4f (&acc)[4], float (*red)[4][4][64],
                                            float (*hbuf)[17], int total, int n0, int pair,
                                            int j, int I, uint8_t* __restrict__ hid,
                                            uint8_t* __restrict__ hid_scales) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][m][i][lane] = acc[m][i];
    lds_barrier();
    {
        const int m = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = ((red[0][m][i][l] + red[1][m][i][l]) + red[2][m][i][l]) +
                            red[3][m][i][l];
            hbuf[m * 16 + 4 * (l >> 4) + i][l & 15] = v;
        }
    }
    lds_barrier();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int nn = h * 8 + (threadIdx.x >> 5);
        const int c = threadIdx.x & 31;
        const float gt = hbuf[c][nn];
        const float up = hbuf[32 + c][nn];
        const float a = gt / (1.0f + expf(-gt)) * up;
        uint32_t mag = __float_as_uint(a) & 0x7FFFFFFFu;
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)mag, off, 64);
            mag = mag > o ? mag : o;
        }
        const int X = mx_block_exponent(mag);
        const uint32_t code = e4m3_rne_sat(ldexpf(a, -X));
        const int p = __shfl(pair, nn, 64);
        if (n0 + nn < total) {
            hid[(size_t)p * I + j * UP_COLS + c] = (uint8_t)code;
            if (c == 0) hid_scales[(size_t)p * (I / 32) + j] = (uint8_t)(X + 127);
        }
    }
    lds_barrier();
}

// dword loads at 4-byte alignment (scale bytes of one row, a wavefront's share): one
// dwordx4 per 4 dwords and one x3/x2/x1 load for the rest
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef u32x4 __attribute__((aligned(4))) u32x4_a4;
typedef u32x3 __attribute__((aligned(4))) u32x3_a4;
typedef u32x2 __attribute__((aligned(4))) u32x2_a4;
template <int N>
__device__ __forceinline__ void load_dwords(const uint8_t* p, uint32_t (&out)[N]) {
#pragma unroll
    for (int k = 0; k + 4 <= N; k += 4) {
        const u32x4 v = *(const u32x4_a4*)(p + 4 * k);
        out[k] = v.x; out[k + 1] = v.y; out[k + 2] = v.z; out[k + 3] = v.w;
    }
    constexpr int k = N & ~3;
    if (N % 4 == 3) {
        const u32x3 v = *(const u32x3_a4*)(p + 4 * k);
        out[k] = v.x; out[k + 1 < N ? k + 1 : 0] = v.y; out[k + 2 < N ? k + 2 : 0] = v.z;
    } else if (N % 4 == 2) {
        const u32x2 v = *(const u32x2_a4*)(p + 4 * k);
        out[k] = v.x; out[k + 1 < N ? k + 1 : 0] = v.y;
    } else if (N % 4 == 1) {
        out[k < N ? k : 0] = *(const uint32_t*)(p + 4 * k);
    }
}

// Up projection, latent L = 512 * SPW.  Item = (touched expert u < D, 32 columns j): the
// expert's tile (gate rows 32j.., up rows I+32j.., 64 x L FP4, 112 KiB at L = 3584) is
// streamed ONCE into registers -- wavefront w holds K steps SPW*w .. SPW*w+SPW-1 of the
// four 16-row tiles, with those steps' E8M0 scale bytes as dwords -- and applied to all
// of the expert's tokens, 16 per MFMA column tile.  One workgroup per CU runs a software
// pipeline: while item i is computed, the weights (and then the first activations) of
// item i + gridDim are already in flight.  The activations of a token group go through
// LDS (see up_issue_acts); their scale dwords are loaded into registers.
template <int SPW>
struct UpStage {
    uint4 w[4][SPW];        // FP4 weight fragments
    uint32_t ws[4][SPW];    // their scale dwords (byte g = K block 4s+g)
    uint32_t bs[SPW];       // the activations' scale dwords
    uint32_t bs1[SPW];      // those of the second token group (tokens 16..31)
    int4 un;                // (expert, list begin, -, list length)
    int j, pair, pair1;     // pair ids of tokens r and 16 + r of the expert's list
};

// Every load below is issued unconditionally (indices are clamped, unused lanes load a
// valid address and discard it) so that the same number of loads is outstanding on every
// path: the compiler can then wait for exactly the current item's data (s_waitcnt
// vmcnt(N)) and leave the next item's loads in flight.
// un3: the first D units as (expert, list begin, list length) in LDS; DUAL: the second
// token group's pair ids too (the two-area build, see up_issue_acts)
template <int SPW, bool PACKED, bool DUAL>
__device__ __forceinline__ void up_issue_weights(UpStage<SPW>& st, int item, int nt, int I,
                                                 const uint8_t* __restrict__ w13,
                                                 const uint8_t* __restrict__ s13,
                                                 const int32_t* __restrict__ pairs,
                                                 const int* un3) {
    constexpr int L = SPW * 512, SROW = L / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int u = item / nt;
    st.j = item - u * nt;
    st.un = make_int4(un3[3 * u], un3[3 * u + 1], 0, un3[3 * u + 2]);
    const int e = st.un.x;
    // the first two token groups' pair ids, issued before the weights so that the
    // activation addresses can wait on them without waiting on the weights
    st.pair = pairs[st.un.y + min(r16, st.un.w - 1)];
    if (DUAL) st.pair1 = pairs[st.un.y + min(16 + r16, st.un.w - 1)];
    if (PACKED) {
        // packed layout: this wavefront's fragments are 4*SPW consecutive 1 KiB blocks
        // (tile-major, then step), each in lane order; the scale dwords of tile m, row r16
        // are SPW consecutive dwords
        const size_t blk = (size_t)st.j * 4 + wave;
        const uint8_t* wb = w13 + (size_t)e * I * L + blk * (4 * SPW * 1024) + lane * 16;
        const uint8_t* sbase = s13 + (size_t)e * I * (L / 16) + blk * (4 * 16 * 4 * SPW);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int i = 0; i < SPW; ++i) st.w[m][i] = load_stream16(wb + (m * SPW + i) * 1024);
            load_dwords<SPW>(sbase + (m * 16 + r16) * (4 * SPW), st.ws[m]);
        }
        return;
    }
    const size_t ebase = (size_t)e * 2 * I;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const size_t R = ebase + (m >> 1) * I + st.j * UP_COLS + (m & 1) * 16 + r16;
        const uint8_t* base = w13 + R * (L / 2) + (SPW * wave) * 64 + 16 * g;
#pragma unroll
        for (int i = 0; i < SPW; ++i) st.w[m][i] = load_stream16(base + i * 64);
        load_dwords<SPW>(s13 + R * SROW + 4 * SPW * wave, st.ws[m]);
    }
}

// The wavefront's activations for token group n0 (its SPW K steps of the group's 16
// tokens) go to its own LDS area `act` (SPW x 2 KiB: step i at 2048 i, token r at 128 r,
// its 16-byte chunk c at position c ^ (r & 7), so that the fragment reads of eight
// consecutive tokens fall in distinct banks).  Direct loads bring eight whole 128-byte
// token rows of a step per instruction (lane l: token l / 8, position l % 8), instead of
// gathering the MFMA operand layout from sixteen half rows per instruction; the second
// eight tokens are skipped when the group has at most eight.  A lane past the group's last
// token holds a copy of a valid token: MFMA output column n depends on B column n only,
// and such columns are never stored.  The scale dwords are register loads, issued last.
//
// act1 (the first group's call only): an expert of more than 16 tokens also gets its
// second group's activations, into the wavefront's second area act1, and their scale
// dwords (bs1) -- issued BEFORE the first group's loads.  Loads complete in issue order,
// so the first group's exact wait covers the second group's loads as well, and the second
// group is computed without a wait of its own: the next item's weights stay in flight.
template <int SPW, bool DUAL>
__device__ __forceinline__ void up_issue_acts(UpStage<SPW>& st, int K, int n0,
                                              const uint8_t* __restrict__ codes, int cbytes,
                                              const uint8_t* __restrict__ scales,
                                              uint8_t* act, bool dma = true,
                                              uint8_t* act1 = nullptr) {
    constexpr int L = SPW * 512, SROW = L / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int q = lane >> 3, pos = lane & 7;
    // every address first (lane r < 16 holds the pair of the group's token r): the one
    // wait for the pair ids then comes before any branch, the same on every path (a wait
    // placed after a branch covers the path that skipped it and here would also wait for
    // part of the next item's weights)
    const uint32_t t0 = (uint32_t)(__shfl(st.pair, q, 64) / K);
    const uint32_t t1 = (uint32_t)(__shfl(st.pair, 8 + q, 64) / K);
    const int pr1 = DUAL ? st.pair1 : 0;
    const uint32_t v0 = (uint32_t)(__shfl(pr1, q, 64) / K);
    const uint32_t v1 = (uint32_t)(__shfl(pr1, 8 + q, 64) / K);
    const size_t srow0 = (size_t)(st.pair / K) * SROW + 4 * SPW * wave;
    const size_t srow1 = (size_t)(pr1 / K) * SROW + 4 * SPW * wave;
    const uint32_t chunk = (uint32_t)((SPW * wave) * 128 + ((pos ^ q) << 4));
    if (DUAL && act1 && st.un.w > 16) {  // (uniform)
        if (dma) {
#pragma unroll
            for (int i = 0; i < SPW; ++i)
                dma16(codes, cbytes, v0 * L + chunk + i * 128, (lds_ptr)(act1 + i * 2048));
            if (st.un.w > 24) {  // (uniform)
#pragma unroll
                for (int i = 0; i < SPW; ++i)
                    dma16(codes, cbytes, v1 * L + chunk + i * 128,
                          (lds_ptr)(act1 + i * 2048 + 1024));
            }
        }
        load_dwords<SPW>(scales + srow1, st.bs1);
    }
    if (dma) {  // (uniform) else the area already holds this group
#pragma unroll
        for (int i = 0; i < SPW; ++i)
            dma16(codes, cbytes, t0 * L + chunk + i * 128, (lds_ptr)(act + i * 2048));
        if (st.un.w - n0 > 8) {  // (uniform)
#pragma unroll
            for (int i = 0; i < SPW; ++i)
                dma16(codes, cbytes, t1 * L + chunk + i * 128, (lds_ptr)(act + i * 2048 + 1024));
        }
    }
    load_dwords<SPW>(scales + srow0, st.bs);
}

// VMEM instructions of up_issue_weights (the pair id, SPW fragments and the scale dwords
// of four tiles): a compute that follows the next item's weight issue waits with this
// count for its own activations
template <int SPW, bool DUAL>
constexpr int up_weight_loads() { return (DUAL ? 2 : 1) + 4 * (SPW + SPW / 4 + (SPW % 4 ? 1 : 0)); }

// Partial H tiles of the four wavefronts (each summed over its quarter of K), one buffer:
// [wave][tile][token][row] FP32, tiles padded to 272 floats so that the gate and up reads
// of one token fall in different LDS banks.
constexpr int RED_TILE = 16 * 16 + 16;
constexpr int RED_FLOATS = 16 * RED_TILE;

// Epilogue of one token group: the K-split partials meet in LDS (one barrier; the buffer
// alternates between groups, so a wavefront that runs ahead writes the other buffer).
// Thread t then owns token n = t / 16 and columns c, c+1 (c = 2 (t mod 16)) of the
// 32-column block: the four partials are added in wavefront order, act = silu(gate) * up
// in FP32, the block's amax is a max over the 16 lanes of that token (lane shuffles), and
// the two E4M3 codes go out as one 16-bit store, the E8M0 scale from the lane holding c=0.
// one thread's share of a token group's MXFP8 hidden, computed but not yet stored
struct UpOut {
    uint32_t code2;  // two E4M3 codes (columns c, c+1)
    uint32_t scale;  // the E8M0 byte (stored by the lane with c = 0)
    size_t at;       // byte offset of the codes in hid (p * I + 32 j + c)
    size_t sat;      // byte offset of the scale in hid_scales
    bool ok, first;  // store at all; this lane holds c = 0
    int ticket;      // the value thread 0 published through the epilogue's barrier
};

__device__ __forceinline__ void up_store(const UpOut& o, uint8_t* __restrict__ hid,
                                         uint8_t* __restrict__ hid_scales) {
    if (o.ok) {
        *(uint16_t*)(hid + o.at) = (uint16_t)o.code2;
        if (o.first) hid_scales[o.sat] = (uint8_t)o.scale;
    }
}

__device__ __forceinline__ UpOut up_epilogue(const v4f (&acc)[4], float* __restrict__ red,
                                             bool store, int total, int n0, int pair, int j,
                                             int I, int* tick, int publish) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int m = 0; m < 4; ++m)
        *(v4f*)(red + (wave * 4 + m) * RED_TILE + r16 * 16 + 4 * g) = acc[m];
    if (tick && threadIdx.x == 0) *tick = publish;
    lds_barrier();
    const int ticket = tick ? *tick : 0;
    const int n = threadIdx.x >> 4, c = 2 * (threadIdx.x & 15);
    const int mg = c >> 4, cr = c & 15;
    float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float2 gv = *(const float2*)(red + (w * 4 + mg) * RED_TILE + n * 16 + cr);
        const float2 uv = *(const float2*)(red + (w * 4 + mg + 2) * RED_TILE + n * 16 + cr);
        if (w == 0) {
            g0 = gv.x; g1 = gv.y; u0 = uv.x; u1 = uv.y;
        } else {
            g0 += gv.x; g1 += gv.y; u0 += uv.x; u1 += uv.y;
        }
    }
    const float a0 = g0 / (1.0f + expf(-g0)) * u0;
    const float a1 = g1 / (1.0f + expf(-g1)) * u1;
    uint32_t m0 = __float_as_uint(a0) & 0x7FFFFFFFu, m1 = __float_as_uint(a1) & 0x7FFFFFFFu;
    uint32_t mag = m0 > m1 ? m0 : m1;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mag, off, 64);
        mag = mag > o ? mag : o;
    }
    const int X = mx_block_exponent(mag);
    const uint32_t q0 = e4m3_rne_sat(ldexpf(a0, -X)), q1 = e4m3_rne_sat(ldexpf(a1, -X));
    const int p = __shfl(pair, n, 64);  // lane n of every wavefront holds token n's pair
    UpOut o;
    o.code2 = q0 | (q1 << 8);
    o.scale = (uint32_t)(X + 127);
    o.at = (size_t)p * I + j * UP_COLS + c;
    o.sat = (size_t)p * (I / 32) + j;
    o.ok = store && n0 + n < total;
    o.first = c == 0;
    o.ticket = ticket;
    return o;
}

// NV: the VMEM instructions issued after the group's activations (their direct loads
// are not tracked by the compiler, so the wait for them is explicit)
template <int SPW, int NV>
__device__ __forceinline__ UpOut up_group(UpStage<SPW>& st, const uint8_t* act, int n0, int I,
                                          bool store, float* red, int* tick = nullptr,
                                          int publish = 0) {
    const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
    wait_vmcnt<NV>();
    __builtin_amdgcn_sched_barrier(0);  // no fragment read moves above the wait
    // B fragment of step i: token r16's bytes 16g.. and 64+16g.. of the step
    const uint8_t* row = act + r16 * 128;
    const int sw = r16 & 7;
    v8i b[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const uint4 lo = *(const uint4*)(row + i * 2048 + ((g ^ sw) << 4));
        const uint4 hi = *(const uint4*)(row + i * 2048 + (((4 + g) ^ sw) << 4));
        b[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    v4f acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
    // the MFMA reads its scales from bits 7:0 of the scale operands
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int sb = (int)(st.bs[i] >> (8 * g));
#pragma unroll
        for (int m = 0; m < 4; ++m)
            acc[m] = mfma_fp4_fp8(as_fp4_operand(st.w[m][i]), b[i], acc[m],
                                  (int)(st.ws[m][i] >> (8 * g)), sb);
    }
    return up_epilogue(acc, red, store, st.un.w, n0, st.pair, st.j, I, tick, publish);
}

// All token groups of one item.  The first group's result is returned unstored (the
// caller stores it, before the next activation loads); later groups of a hot expert are
// stored at once, and then the first group's too.
// The first group's activations are followed by the next item's weight issue (and at
// most the conditional ticket, which is older and completes with them).  The second
// group's loads went out before the first group's (see up_issue_acts), so the second
// group needs no wait; a third and later group (an expert of more than 32 tokens) loads
// its activations into the second area and waits for every load in flight.
template <int SPW, bool DUAL, int NV0 = up_weight_loads<SPW, DUAL>()>
__device__ __forceinline__ UpOut up_compute(UpStage<SPW>& st, int K, int I, bool store,
                                            const uint8_t* __restrict__ codes, int cbytes,
                                            const uint8_t* __restrict__ scales,
                                            const int32_t* __restrict__ pairs,
                                            uint8_t* __restrict__ hid,
                                            uint8_t* __restrict__ hid_scales, float* red,
                                            int& rb, uint8_t* act, uint8_t* act1,
                                            int* tick = nullptr, int publish = 0) {
    const int r16 = threadIdx.x & 15;
    UpOut first = up_group<SPW, NV0>(
        st, act, 0, I, store, red + rb * RED_FLOATS, tick ? tick + rb : nullptr, publish);
    rb ^= 1;
    if (st.un.w <= 16) return first;
    up_store(first, hid, hid_scales);
    first.ok = false;
    int n0 = 16;
    if (DUAL) {  // the second group is in act1 already
        st.pair = st.pair1;
#pragma unroll
        for (int i = 0; i < SPW; ++i) st.bs[i] = st.bs1[i];
        up_store(up_group<SPW, 63>(st, act1, 16, I, store, red + rb * RED_FLOATS), hid,
                 hid_scales);
        rb ^= 1;
        n0 = 32;
    }
    for (; n0 < st.un.w; n0 += 16) {  // later token groups of a hot expert
        st.pair = pairs[st.un.y + min(n0 + r16, st.un.w - 1)];
        up_issue_acts<SPW, DUAL>(st, K, n0, codes, cbytes, scales, act1);
        up_store(up_group<SPW, 0>(st, act1, n0, I, store, red + rb * RED_FLOATS), hid,
                 hid_scales);
        rb ^= 1;
    }
    return first;
}

// Work order of both persistent passes: workgroup w takes the static items w, w + G, ...,
// w + (2R - 1) G (R passes of two), then items from tickets as it frees up, so that
// workgroups starting late (their CU still busy with the side stream's GEMMs) or drawing
// costlier items (experts of more token groups) take fewer of the last items instead of
// finishing late.  The dynamic tail is the last quarter of
// the passes (at least two): the tickets' cost (an LDS round between a compute and the
// next loads) is paid only there.  Items still go out in ascending order: the CUs sweep
// one compact window of weights together.  Thread 0 takes each ticket one stage ahead --
// just before the loads of the stage after the one it will name -- and publishes it
// through the barrier of a later compute, so that neither a compute's wait for its own
// loads nor the publishing waits for an atomic still in flight.  Tickets only grow, so a
// workgroup's items ascend and the loop ends once one passes the count.
// (at least two static passes before any ticket: the first tickets are taken in pass 0
// for the items of pass 2; up to four passes everything is static)
__device__ __forceinline__ int static_passes(int items, int G) {
    const int passes = ((items + G - 1) / G + 1) / 2;
    if (passes <= 4) return passes;
    return passes - (passes / 4 > 2 ? passes / 4 : 2);
}
// One counter per XCD (workgroup w counts on counter w % 8, the XCD it is placed on), so
// that each counter serves 1/8 of the workgroups; ticket t of counter x names item
// base + 8t + x, base = 2RG (all counters together cover every item past the static ones
// once).  With G < 8 some counters have no workgroup; callers launch G = min(items, CUs),
// so then items = G and every item is static.
__device__ __forceinline__ int take_ticket(unsigned* counters) {
    return threadIdx.x == 0 ? (int)atomicAdd(counters + (blockIdx.x & 7), 1u) : 0;
}
__device__ __forceinline__ int ticket_item(int base, int t) { return base + 8 * t + (blockIdx.x & 7); }

// DUAL: two activation areas a wavefront (the second token group's loads issued ahead);
// else one (LDS then leaves room for a side-stream GEMM's workgroup on the same CU)
template <int SPW, bool PACKED, bool DUAL>
__global__ __launch_bounds__(256, 1) void k_ffn_up_fast(
    int K, int I, const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const uint8_t* __restrict__ codes, int cbytes, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ pairs, const int4* __restrict__ units,
    const int32_t* __restrict__ num_units, uint8_t* __restrict__ hid,
    uint8_t* __restrict__ hid_scales, unsigned* __restrict__ counter, int dyn) {
    __shared__ __attribute__((aligned(16))) float red[2 * RED_FLOATS];
    __shared__ int tick[2];
    // the first D units (one per touched expert, E <= 1024) as (expert, begin, length)
    __shared__ int un_lds[3 * 1024];
    // each wavefront's activation areas (one token group each; see up_issue_acts); with
    // one area, later groups reuse the first
    __shared__ __attribute__((aligned(1024))) uint8_t act_all[DUAL ? 2 : 1][4][SPW * 2048];
    uint8_t* act = act_all[0][threadIdx.x >> 6];
    uint8_t* act1 = act_all[DUAL ? 1 : 0][threadIdx.x >> 6];
    const int nt = I / UP_COLS;
    const int D = num_units[2];
    const int items = D * nt;  // touched experts x column tiles
    const int G = gridDim.x;
    // the units in LDS: an item's unit is then an LDS read, not a global round trip
    // between learning the item and issuing its weight loads
    for (int i = threadIdx.x; i < D; i += 256) {
        const int4 u = units[i];
        un_lds[3 * i] = u.x;
        un_lds[3 * i + 1] = u.y;
        un_lds[3 * i + 2] = u.w;
    }
    __syncthreads();
    int a = blockIdx.x;  // the item in stage A
    if (a >= items) return;
    int b = a + G;        // the item in stage B
    // dyn = 0: every pass static (no counter is touched)
    const int R = dyn ? static_passes(items, G) : 0x7fffffff, base = dyn ? 2 * R * G : 0;
    // Within the whole static blocks of 2G items, the two stages of a pass take two
    // neighbouring column tiles of one expert (a pass still covers one compact window of
    // 2G items): for an expert of at most 16 tokens (32 with two areas) stage B then finds
    // the groups' activations already in LDS and loads none.  (Four tiles over two passes would skip
    // more loads, but hand a hot expert's heavy tiles to one workgroup four at a time:
    // measured slower with skewed routing.)  Items past those blocks (the dynamic tail, a
    // last partial block) keep their own order.
    const int full = min(items, dyn ? 2 * R * G : items) / (2 * G) * (2 * G);
    auto item_of = [&](int i) {
        if (i >= full) return i;
        const int k = i / (2 * G), r = i - k * 2 * G;  // pass, place in it
        return 2 * (G * k + (r < G ? r : r - G)) + (r < G ? 0 : 1);
    };
    int t_prev = 0;       // the ticket naming the next A (taken last pass, if dynamic)
    int rb = 0;
    UpStage<SPW> A, B;
    // (B of A's expert: its groups are still in the areas up to this many tokens)
    constexpr int REUSE = DUAL ? 32 : 16;
    if (items <= G) {  // (uniform) one item a workgroup: no second stage, no tickets; the
                       // item's first group waits for every load (none follows them)
        up_issue_weights<SPW, PACKED, DUAL>(A, a, nt, I, w13, s13, pairs, un_lds);
        up_issue_acts<SPW, DUAL>(A, K, 0, codes, cbytes, scales, act, true, act1);
        const UpOut o = up_compute<SPW, DUAL, 0>(A, K, I, true, codes, cbytes, scales, pairs,
                                                 hid, hid_scales, red, rb, act, act1);
        up_store(o, hid, hid_scales);
        wait_vmcnt<0>();
        return;
    }
    up_issue_weights<SPW, PACKED, DUAL>(A, item_of(a), nt, I, w13, s13, pairs, un_lds);
    up_issue_acts<SPW, DUAL>(A, K, 0, codes, cbytes, scales, act, true, act1);
    // Items in pairs (stages A and B), pass k holding a_k and b_k.  Nothing between a
    // stage's loads and its compute is conditional: a conditional exit there would let the
    // compiler sink the loads below it, losing the prefetch.  Past the last item a stage
    // repeats an item, computes it and stores nothing.
    // A stage's stores (conditional per lane) go out right after its compute, before the
    // other stage's activation loads: a compute waits for its activations with a vmcnt
    // that the compiler counts on the path without the stores, so stores issued after the
    // activations would make that wait cover the first loads of the next item as well.
    for (int k = 0;; ++k) {
        const bool b_real = b < items;
        const int t_b = k + 1 < R ? 0 : take_ticket(counter);  // names b_{k+1} if dynamic
        // tickets go through LDS only in the tail (a static pass reads none: its next items'
        // addresses then wait for nothing)
        int* const tk = k + 1 < R ? nullptr : tick;
        // (the scheduling barriers keep each stage's loads ahead of the other stage's
        // compute; otherwise the scheduler interleaves them into it)
        up_issue_weights<SPW, PACKED, DUAL>(B, item_of(b_real ? b : a), nt, I, w13, s13, pairs,
                                            un_lds);
        __builtin_amdgcn_sched_barrier(0);
        const UpOut oa = up_compute<SPW, DUAL>(A, K, I, true, codes, cbytes, scales, pairs, hid,
                                               hid_scales, red, rb, act, act1, tk, t_prev);
        const int a_next = k + 1 < R ? a + 2 * G : ticket_item(base, oa.ticket);
        up_store(oa, hid, hid_scales);
        __builtin_amdgcn_sched_barrier(0);
        up_issue_acts<SPW, DUAL>(B, K, 0, codes, cbytes, scales, act,
                                 !(B.un.x == A.un.x && A.un.w <= REUSE), act1);
        t_prev = k + 2 < R ? 0 : take_ticket(counter);  // names a_{k+2} if dynamic
        const int e_b = B.un.x;
        up_issue_weights<SPW, PACKED, DUAL>(A, item_of(a_next < items ? a_next : a), nt, I, w13,
                                            s13, pairs, un_lds);
        __builtin_amdgcn_sched_barrier(0);
        const UpOut ob = up_compute<SPW, DUAL>(B, K, I, b_real, codes, cbytes, scales, pairs,
                                               hid, hid_scales, red, rb, act, act1, tk, t_b);
        up_store(ob, hid, hid_scales);
        __builtin_amdgcn_sched_barrier(0);
        up_issue_acts<SPW, DUAL>(A, K, 0, codes, cbytes, scales, act,
                                 !(A.un.x == e_b && A.un.w <= REUSE), act1);
        __builtin_amdgcn_sched_barrier(0);
        if (a_next >= items) break;  // (every later item is larger)
        b = k + 1 < R ? b + 2 * G : ticket_item(base, ob.ticket);
        a = a_next;
    }
    wait_vmcnt<0>();  // no direct load may still target LDS when the workgroup ends
}

// Up projection for any L % 128 == 0: wavefronts take K steps round-robin, weights are
// loaded per step (fewer bytes in flight than the fast path).
__global__ __launch_bounds__(256) void k_ffn_up_generic(
    int K, int L, int I, const uint8_t* __restrict__ w13, const uint8_t* __restrict__ s13,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ pairs, const int4* __restrict__ units,
    const int32_t* __restrict__ num_units, uint8_t* __restrict__ hid,
    uint8_t* __restrict__ hid_scales) {
    __shared__ float red[4][4][4][64];
    __shared__ float hbuf[64][17];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int nt = I / UP_COLS;
    const int items = num_units[2] * nt;
    const int steps = L / 128;
    const size_t wrow = (size_t)L / 2, srow = (size_t)L / 32;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int u = item / nt, j = item - u * nt;
        const int4 un = units[u];
        if (un.w == 0) continue;
        const int e = un.x, begin = un.y, total = un.w;
        for (int n0 = 0; n0 < total; n0 += 16) {
            const int n = n0 + r16;
            const bool tok = n < total;
            const int pair = tok ? pairs[begin + n] : 0;
            const int t = pair / K;
            v4f acc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
            for (int st = wave; st < steps; st += 4) {
                v8i b = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
                int sb = 127;
                if (tok) {
                    b = load_fp8x32(codes + (size_t)t * L + st * 128, g);
                    sb = scales[(size_t)t * srow + st * 4 + g];
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const size_t R = (size_t)e * 2 * I + (m >> 1) * I + j * UP_COLS +
                                     (m & 1) * 16 + r16;
                    const v8i a = load_fp4x32(w13 + R * wrow + st * 64 + g * 16);
                    const int sa = s13[R * srow + st * 4 + g];
                    acc[m] = mfma_fp4_fp8(a, b, acc[m], sa, sb);
                }
            }
            up_epilogue_lds(acc, red, hbuf, total, n0, pair, j, I, hid, hid_scales);
        }
    }
}

// Down projection, intermediate I = 128 * IS.  Item = (touched expert u < D, 64*MT rows
// of W2): wavefront w streams MT 16-row tiles (all IS K steps, plus the rows' scale
// words) ONCE and applies them to all of the expert's pairs, 16 per MFMA column tile;
// BF16 rows out.  Same one-workgroup-per-CU pipeline as the up projection: the next
// item's weights are in flight while the current one is computed.
template <int IS, int MT>
struct DownStage {
    uint4 w[MT][IS];
    uint32_t sw[MT][IS];  // scale dwords of each row (byte g = K block 4s+g)
    uint32_t bs[IS];      // the hidden's scale dwords (the hidden itself goes through LDS)
    uint32_t bs1[IS];     // those of the second token group (pairs 16..31 of the list)
    int4 un;
    int j, pair, pair1;   // pair ids of entries r and 16 + r of the expert's list
};

template <int IS, int MT, bool PACKED>
__device__ __forceinline__ void down_issue_weights(DownStage<IS, MT>& st, int item, int nt, int L,
                                                   const uint8_t* __restrict__ w2,
                                                   const uint8_t* __restrict__ s2,
                                                   const int32_t* __restrict__ pairs,
                                                   const int4* __restrict__ units) {
    constexpr int I = IS * 128, WROW = I / 2, SROW = I / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int u = item / nt;
    st.j = item - u * nt;
    st.un = units[u];
    st.pair = pairs[st.un.y + min(r16, st.un.w - 1)];
    st.pair1 = pairs[st.un.y + min(16 + r16, st.un.w - 1)];
    const size_t R0 = (size_t)st.un.x * L + st.j * (64 * MT) + wave * (16 * MT) + r16;
    // packed layout: this wavefront's fragments are MT*IS consecutive 1 KiB blocks in
    // lane order (the scale rows keep their order)
    const uint8_t* wb = w2 + (size_t)st.un.x * L * WROW +
                        ((size_t)st.j * 4 + wave) * (MT * IS * 1024) + lane * 16;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const size_t R = R0 + m * 16;
#pragma unroll
        for (int s = 0; s < IS; ++s)
            st.w[m][s] = PACKED ? load_stream16(wb + (m * IS + s) * 1024)
                                : load_stream16(w2 + R * WROW + s * 64 + 16 * g);
        load_dwords<IS>(s2 + R * SROW, st.sw[m]);
    }
}

// The MXFP8 hidden of a token group, shared by the four wavefronts (each takes all K
// steps of its own rows): wavefront s brings K step s of the group's tokens into the
// stage's LDS buffer `hb` (IS x 2 KiB: step s at 2048 s, token r at 128 r, its 16-byte
// chunk c at position c ^ (r & 7), as in the up projection), eight whole 128-byte rows
// per direct load, the second eight skipped for groups of at most eight tokens.  Rows past
// the group's last token hold its last token.  The scale dwords are register loads.
// hb1 (the first group's call only): an expert of more than 16 pairs also gets its second
// group's hidden, into the stage's second buffer hb1, and its scale dwords (bs1) -- issued
// BEFORE the first group's loads, so that the first group's exact wait (and barrier)
// covers them and the second group is computed without draining the next item's weights.
// Every address is computed before any branch (one wait for the pair ids on every path).
template <int IS, int MT>
__device__ __forceinline__ void down_issue_acts(DownStage<IS, MT>& st, int n0,
                                                const uint8_t* __restrict__ hid, int hbytes,
                                                const uint8_t* __restrict__ hid_scales,
                                                uint8_t* hb, uint8_t* hb1 = nullptr) {
    constexpr int I = IS * 128, SROW = I / 32;
    const int lane = threadIdx.x & 63;
    // the wavefront index as a scalar: the branch and the LDS base are then uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 3, pos = lane & 7;
    const uint32_t chunk = (uint32_t)(wave * 128 + ((pos ^ q) << 4));
    const uint32_t p0 = (uint32_t)__shfl(st.pair, q, 64);
    const uint32_t p1 = (uint32_t)__shfl(st.pair, 8 + q, 64);
    const uint32_t r0 = (uint32_t)__shfl(st.pair1, q, 64);
    const uint32_t r1 = (uint32_t)__shfl(st.pair1, 8 + q, 64);
    const size_t srow0 = (size_t)st.pair * SROW, srow1 = (size_t)st.pair1 * SROW;
    if (hb1 && st.un.w > 16) {  // (uniform)
        if (wave < IS) {
            dma16(hid, hbytes, r0 * I + chunk, (lds_ptr)(hb1 + wave * 2048));
            if (st.un.w > 24)  // (uniform)
                dma16(hid, hbytes, r1 * I + chunk, (lds_ptr)(hb1 + wave * 2048 + 1024));
        }
        load_dwords<IS>(hid_scales + srow1, st.bs1);
    }
    if (wave < IS) {
        dma16(hid, hbytes, p0 * I + chunk, (lds_ptr)(hb + wave * 2048));
        if (st.un.w - n0 > 8)  // (uniform)
            dma16(hid, hbytes, p1 * I + chunk, (lds_ptr)(hb + wave * 2048 + 1024));
    }
    load_dwords<IS>(hid_scales + srow0, st.bs);
}

// VMEM instructions of down_issue_weights (the pair id, MT*IS fragments and MT rows of
// scale dwords): a compute that follows the next item's weight issue waits with this count
template <int IS, int MT>
constexpr int down_weight_loads() { return 2 + MT * IS + MT * (IS / 4 + (IS % 4 ? 1 : 0)); }

// The wavefront's output block is 16 tokens x 16*MT columns of BF16.  It is staged in
// the wavefront's own LDS area ([token][column], rows padded by 16 bytes) and written
// back so that each store instruction covers whole 128-byte lines: lane l takes token
// 4q + l/16 and the 16 bytes at column 8 (l mod 16) .. of the block (MT = 8: 256 bytes a
// token, two full lines).  No other wavefront touches the area, so no barrier is needed.
template <int MT>
constexpr int down_stage_row() { return 32 * MT + 16; }

// NV: the VMEM instructions issued after the group's hidden (its direct loads are not
// tracked by the compiler, so each wavefront waits for its own explicitly, then the
// barrier makes every wavefront's share visible).  cnt: the group's tokens (1..16);
// column r16 takes token min(r16, cnt - 1), the token whose pair id the lane holds.
template <int IS, int MT, int NV>
__device__ __forceinline__ void down_mfma_stage(DownStage<IS, MT>& st, const uint8_t* hb,
                                                int cnt, uint8_t* stage) {
    constexpr int ROWB = down_stage_row<MT>();
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, g = lane >> 4;
    wait_vmcnt<NV>();
    lds_sync();  // every wavefront's K step landed (no fragment read moves above it)
    const int tr = min(r16, cnt - 1), sw = tr & 7;
    const uint8_t* row = hb + tr * 128;
    v8i b[IS];
#pragma unroll
    for (int s = 0; s < IS; ++s) {
        const uint4 lo = *(const uint4*)(row + s * 2048 + ((g ^ sw) << 4));
        const uint4 hi = *(const uint4*)(row + s * 2048 + (((4 + g) ^ sw) << 4));
        b[s] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    v4f acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < IS; ++s)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[m] = mfma_fp4_fp8(as_fp4_operand(st.w[m][s]), b[s], acc[m],
                                  (int)(st.sw[m][s] >> (8 * g)), (int)(st.bs[s] >> (8 * g)));
    // acc[m][i] = out[token r16][column m*16 + 4g + i]
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        uint2 o;
        o.x = pack_bf16x2(acc[m][0], acc[m][1]);
        o.y = pack_bf16x2(acc[m][2], acc[m][3]);
        *(uint2*)(stage + r16 * ROWB + (m * 16 + 4 * g) * 2) = o;
    }
}

// write the staged block of token group n0 (pair ids in st.pair) to the rows
template <int IS, int MT>
__device__ __forceinline__ void down_store(const DownStage<IS, MT>& st, int n0, int L, bool store,
                                           uint16_t* __restrict__ rows, const uint8_t* stage) {
    constexpr int ROWB = down_stage_row<MT>();
    constexpr int LANES_PER_TOKEN = 2 * MT;  // 16-byte pieces per token
    constexpr int TOKENS_PER_STORE = 64 / LANES_PER_TOKEN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col0 = st.j * (64 * MT) + wave * (16 * MT);
#pragma unroll
    for (int q = 0; q < 16 / TOKENS_PER_STORE; ++q) {
        const int tk = q * TOKENS_PER_STORE + lane / LANES_PER_TOKEN;
        const int piece = lane % LANES_PER_TOKEN;
        const uint4 v = *(const uint4*)(stage + tk * ROWB + piece * 16);
        const int p = __shfl(st.pair, tk, 64);  // lane tk holds token tk's pair
        if (store && n0 + tk < st.un.w)
            *(uint4*)(rows + (size_t)p * L + col0 + piece * 8) = v;
    }
}

// The item's first token group is computed and left staged (the caller stores it, before
// the next activation loads); later groups of a hot expert are stored at once.
// The first group's hidden is followed by the next item's weight issue (and at most the
// conditional ticket, older).  The second group's hidden is already in hb1 (see
// down_issue_acts); a third and later group reuses hb1 once every wavefront is done
// reading it (a barrier ahead of its loads) and waits for every load in flight.
template <int IS, int MT, int NV0 = down_weight_loads<IS, MT>()>
__device__ __forceinline__ void down_compute(DownStage<IS, MT>& st, int L, bool store,
                                             const uint8_t* __restrict__ hid, int hbytes,
                                             const uint8_t* __restrict__ hid_scales,
                                             const int32_t* __restrict__ pairs,
                                             uint16_t* __restrict__ rows, uint8_t* hb,
                                             uint8_t* hb1, uint8_t* stage) {
    const int r16 = threadIdx.x & 15;
    down_mfma_stage<IS, MT, NV0>(st, hb, min(st.un.w, 16), stage);
    if (st.un.w <= 16) return;
    down_store(st, 0, L, store, rows, stage);
    st.pair = st.pair1;
#pragma unroll
    for (int i = 0; i < IS; ++i) st.bs[i] = st.bs1[i];
    down_mfma_stage<IS, MT, 63>(st, hb1, min(st.un.w - 16, 16), stage);
    down_store(st, 16, L, store, rows, stage);
    for (int n0 = 32; n0 < st.un.w; n0 += 16) {  // later pair groups of a hot expert
        st.pair = pairs[st.un.y + min(n0 + r16, st.un.w - 1)];
        lds_sync();
        down_issue_acts(st, n0, hid, hbytes, hid_scales, hb1);
        down_mfma_stage<IS, MT, 0>(st, hb1, min(st.un.w - n0, 16), stage);
        down_store(st, n0, L, store, rows, stage);
    }
}

template <int IS, int MT, bool PACKED>
__global__ __launch_bounds__(256, 1) void k_ffn_down_fast(
    int L, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const uint8_t* __restrict__ hid, const uint8_t* __restrict__ hid_scales,
    const int32_t* __restrict__ pairs, const int4* __restrict__ units,
    const int32_t* __restrict__ num_units, uint16_t* __restrict__ rows,
    unsigned* __restrict__ counter, int dyn, int hbytes) {
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[4][16 * (32 * MT + 16)];
    // the hidden of stage A's and stage B's first and second token groups (see
    // down_issue_acts)
    __shared__ __attribute__((aligned(1024))) uint8_t hbuf[2][IS * 2048];
    __shared__ __attribute__((aligned(1024))) uint8_t hbuf1[2][IS * 2048];
    __shared__ int tick[2];
    __shared__ int4 un_lds[1024];  // the first D units, as in the up projection
    uint8_t* stage = stage_all[threadIdx.x >> 6];
    const int nt = L / (64 * MT);
    const int D = num_units[2];
    const int items = D * nt;
    const int G = gridDim.x;
    for (int i = threadIdx.x; i < D; i += 256) un_lds[i] = units[i];
    __syncthreads();
    int a = blockIdx.x;
    if (a >= items) return;
    int b = a + G;
    // dyn = 0: every pass static (no counter is touched)
    const int R = dyn ? static_passes(items, G) : 0x7fffffff, base = dyn ? 2 * R * G : 0;
    int t_prev = 0;
    DownStage<IS, MT> A, B;
    if (items <= G) {  // (uniform) one item a workgroup, as in the up projection
        down_issue_weights<IS, MT, PACKED>(A, a, nt, L, w2, s2, pairs, un_lds);
        down_issue_acts(A, 0, hid, hbytes, hid_scales, hbuf[0], hbuf1[0]);
        down_compute<IS, MT, 0>(A, L, true, hid, hbytes, hid_scales, pairs, rows, hbuf[0],
                                hbuf1[0], stage);
        if (A.un.w <= 16) down_store(A, 0, L, true, rows, stage);
        wait_vmcnt<0>();
        return;
    }
    down_issue_weights<IS, MT, PACKED>(A, a, nt, L, w2, s2, pairs, un_lds);
    down_issue_acts(A, 0, hid, hbytes, hid_scales, hbuf[0], hbuf1[0]);
    // items in pairs, nothing conditional between a stage's loads and its compute, each
    // stage's stores right after its compute (see the up projection); the dynamic tail's
    // tickets as there, published through one barrier a stage
    for (int k = 0;; ++k) {
        const bool b_real = b < items;
        const int t_b = k + 1 < R ? 0 : take_ticket(counter);
        down_issue_weights<IS, MT, PACKED>(B, b_real ? b : a, nt, L, w2, s2, pairs, un_lds);
        __builtin_amdgcn_sched_barrier(0);
        down_compute(A, L, true, hid, hbytes, hid_scales, pairs, rows, hbuf[0], hbuf1[0], stage);
        int a_next = a + 2 * G;
        if (k + 1 >= R) {  // uniform
            if (threadIdx.x == 0) tick[0] = t_prev;
            lds_barrier();
            a_next = ticket_item(base, tick[0]);
        }
        if (A.un.w <= 16) down_store(A, 0, L, true, rows, stage);
        __builtin_amdgcn_sched_barrier(0);
        down_issue_acts(B, 0, hid, hbytes, hid_scales, hbuf[1], hbuf1[1]);
        t_prev = k + 2 < R ? 0 : take_ticket(counter);
        down_issue_weights<IS, MT, PACKED>(A, a_next < items ? a_next : a, nt, L, w2, s2, pairs,
                                           un_lds);
        __builtin_amdgcn_sched_barrier(0);
        down_compute(B, L, b_real, hid, hbytes, hid_scales, pairs, rows, hbuf[1], hbuf1[1],
                     stage);
        int b_next = b + 2 * G;
        if (k + 1 >= R) {
            if (threadIdx.x == 0) tick[1] = t_b;
            lds_barrier();
            b_next = ticket_item(base, tick[1]);
        }
        if (B.un.w <= 16) down_store(B, 0, L, b_real, rows, stage);
        __builtin_amdgcn_sched_barrier(0);
        down_issue_acts(A, 0, hid, hbytes, hid_scales, hbuf[0], hbuf1[0]);
        __builtin_amdgcn_sched_barrier(0);
        if (a_next >= items) break;
        a = a_next;
        b = b_next;
    }
    wait_vmcnt<0>();  // no direct load may still target LDS when the workgroup ends
}

// Down projection for any I % 128 == 0 (weights loaded per K step)
__global__ __launch_bounds__(256) void k_ffn_down_generic(
    int L, int I, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2,
    const uint8_t* __restrict__ hid, const uint8_t* __restrict__ hid_scales,
    const int32_t* __restrict__ pairs, const int4* __restrict__ units,
    const int32_t* __restrict__ num_units, uint16_t* __restrict__ rows) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int nt = L / DOWN_ROWS;
    const int items = num_units[2] * nt;
    const int steps = I / 128;
    const size_t wrow = (size_t)I / 2, srow = (size_t)I / 32;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int u = item / nt, j = item - u * nt;
        const int4 un = units[u];
        if (un.w == 0) continue;
        const int e = un.x, begin = un.y, total = un.w;
        for (int n0 = 0; n0 < total; n0 += 16) {
            const int n = n0 + r16;
            const bool tok = n < total;
            const int p = tok ? pairs[begin + n] : 0;
            v4f acc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m] = (v4f){0.f, 0.f, 0.f, 0.f};
            for (int st = 0; st < steps; ++st) {
                v8i b = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
                int sb = 127;
                if (tok) {
                    b = load_fp8x32(hid + (size_t)p * I + st * 128, g);
                    sb = hid_scales[(size_t)p * srow + st * 4 + g];
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const size_t R = (size_t)e * L + j * DOWN_ROWS + wave * 64 + m * 16 + r16;
                    const v8i a = load_fp4x32(w2 + R * wrow + st * 64 + g * 16);
                    const int sa = s2[R * srow + st * 4 + g];
                    acc[m] = mfma_fp4_fp8(a, b, acc[m], sa, sb);
                }
            }
            if (tok) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int row = j * DOWN_ROWS + wave * 64 + m * 16 + 4 * g;
                    uint2 o;
                    o.x = pack_bf16x2(acc[m][0], acc[m][1]);
                    o.y = pack_bf16x2(acc[m][2], acc[m][3]);
                    *(uint2*)(rows + (size_t)p * L + row) = o;
                }
            }
        }
    }
}

// compute units of the current device (queried once; 256 on MI355X)
static int num_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            cus = n;
        else
            cus = 256;
    }
    return cus;
}

static int persistent_blocks(int max_items, int per_cu) {
    const int cap = num_cus() * per_cu;
    return max_items < cap ? (max_items > 0 ? max_items : 1) : cap;
}

hipError_t launch_ffn_mx(int T, int K, int E, int L, int I, int unit, const uint8_t* w13,
                         const uint8_t* s13, const uint8_t* w2, const uint8_t* s2,
                         const uint8_t* codes, const uint8_t* scales, const int32_t* pairs,
                         const int32_t* units, const int32_t* num_units, void* rows,
                         uint8_t* hid, uint8_t* hsc, int stages, bool packed, unsigned* counters,
                         bool counters_zeroed, hipStream_t s) {
    (void)unit;
    // the dynamic tail at every batch size: up to 256 tokens the side stream's GEMMs hold
    // some CUs at the start; past 256 the items' costs differ (experts of one to several
    // token groups, hot experts under skewed routing): measured per layer -20 us at 1020
    // tokens, -44 with a Zipf-skewed bias, -43 at 510 with Zipf, +3..+6 at 510 uniform
    const int dyn = 1;
    const bool dual = T >= kUpTwoAreaTokens;
    if (dyn && !counters_zeroed)
        hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, s, counters, 16);
    const int4* un = (const int4*)units;
    const int cbytes = T * L;  // the MXFP8 latent's codes (< 2^31: T <= 4096, L <= 3584)
    const int hbytes = T * K * I;  // the MXFP8 hidden (< 2^31: T K <= 65536, I <= 512)
    const int up_items = E * (I / UP_COLS);  // an upper bound: the kernels read D on the device
    const int cus = num_cus();
    const dim3 blk(256);
    const dim3 ugrid(up_items < cus ? up_items : cus);
    // packed weights exist only for L % 512 == 0 and I / 128 in {1, 2, 4} (checked by the
    // callers), which the fast kernels cover
    switch ((stages & 1) ? (L % 512 == 0 ? L / 512 : 0) : -1) {
#define MOE_UP_L(SPW, DUAL)                                                                  \
    if (packed)                                                                              \
        hipLaunchKernelGGL((k_ffn_up_fast<SPW, true, DUAL>), ugrid, blk, 0, s, K, I, w13,    \
                           s13, codes, cbytes, scales, pairs, un, num_units, hid, hsc,       \
                           counters, dyn);                                                   \
    else                                                                                     \
        hipLaunchKernelGGL((k_ffn_up_fast<SPW, false, DUAL>), ugrid, blk, 0, s, K, I, w13,   \
                           s13, codes, cbytes, scales, pairs, un, num_units, hid, hsc,       \
                           counters, dyn);
#define MOE_UP(SPW)                                                                          \
    case SPW:                                                                                \
        if (dual) {                                                                          \
            MOE_UP_L(SPW, true)                                                              \
        } else {                                                                             \
            MOE_UP_L(SPW, false)                                                             \
        }                                                                                    \
        break;
        MOE_UP(1) MOE_UP(2) MOE_UP(3) MOE_UP(4) MOE_UP(5) MOE_UP(6) MOE_UP(7)
#undef MOE_UP_L
#undef MOE_UP
        case -1:
            break;
        default:
            hipLaunchKernelGGL(k_ffn_up_generic, dim3(persistent_blocks(up_items, 8)), blk, 0, s,
                               K, L, I, w13, s13, codes, scales, pairs, un, num_units, hid, hsc);
    }
    const int MTsel = L % 512 == 0 ? 8 : (L % 256 == 0 ? 4 : 0);
    const int down_items = MTsel ? E * (L / (64 * MTsel)) : E * (L / DOWN_ROWS);
    const dim3 dgrid(down_items < cus ? down_items : cus);
    switch ((stages & 2) ? MTsel * 10 + I / 128 : -1) {
#define MOE_DOWN(MT, IS)                                                                     \
    case MT * 10 + IS:                                                                       \
        if (packed && MT == 8)                                                               \
            hipLaunchKernelGGL((k_ffn_down_fast<IS, MT, true>), dgrid, blk, 0, s, L, w2, s2, \
                               hid, hsc, pairs, un, num_units, (uint16_t*)rows,              \
                               counters + 8, dyn, hbytes);                                   \
        else                                                                                 \
            hipLaunchKernelGGL((k_ffn_down_fast<IS, MT, false>), dgrid, blk, 0, s, L, w2, s2,\
                               hid, hsc, pairs, un, num_units, (uint16_t*)rows,              \
                               counters + 8, dyn, hbytes);                                   \
        break;
        MOE_DOWN(8, 1) MOE_DOWN(8, 2) MOE_DOWN(8, 4) MOE_DOWN(4, 1) MOE_DOWN(4, 2)
        MOE_DOWN(4, 4)
#undef MOE_DOWN
        case -1:
            break;
        default:
            hipLaunchKernelGGL(k_ffn_down_generic, dim3(persistent_blocks(down_items, 8)), blk, 0,
                               s, L, I, w2, s2, hid, hsc, pairs, un, num_units, (uint16_t*)rows);
    }
    return hipGetLastError();
}

// ---- the packed expert layout (load-time preparation of MXFP4 weights) -----------------
// W13 of expert e: blocks (j, w, m, i) of 1 KiB, j < I/32 the 32-column item, w < 4 the
// wavefront, m < 4 the 16-row tile (gate 0-15, gate 16-31, up 0-15, up 16-31 of the item's
// columns), i < L/512 the wavefront's K step; lane l = r + 16 g of a block holds the 16
// bytes of row r of tile m, K block g of step L/512*w + i.  S13 of expert e: for (j, w, m, r)
// the L/512 scale dwords of that row covering the wavefront's steps.  W2 of expert e:
// blocks (jd, w, m, s), jd < L/512 the 512-row item, w < 4, m < 8 the 16-row tile (rows
// 512 jd + 128 w + 16 m ..), s < I/128 the K step, lanes as above.  S2 is unchanged.
__global__ __launch_bounds__(256) void k_pack_w13(long total, int I, int L,
                                                  const uint4* __restrict__ src,
                                                  uint4* __restrict__ dst) {
    const int SPW = L / 512;
    const long per_e = (long)I * L / 16;
    for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < total; c += (long)gridDim.x * 256) {
        const long e = c / per_e;
        long r = c - e * per_e;
        const int lane = (int)(r % 64); r /= 64;
        const int i = (int)(r % SPW); r /= SPW;
        const int m = (int)(r % 4); r /= 4;
        const int w = (int)(r % 4);
        const int j = (int)(r / 4);
        const long row = (long)(m >> 1) * I + j * UP_COLS + (m & 1) * 16 + (lane & 15);
        const long col16 = (long)(SPW * w + i) * 4 + (lane >> 4);  // 16-byte unit in the row
        dst[c] = src[e * per_e + row * (L / 32) + col16];
    }
}

__global__ __launch_bounds__(256) void k_pack_s13(long total, int I, int L,
                                                  const uint32_t* __restrict__ src,
                                                  uint32_t* __restrict__ dst) {
    const int SPW = L / 512;
    const long per_e = (long)I * L / 64;  // dwords per expert
    for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < total; c += (long)gridDim.x * 256) {
        const long e = c / per_e;
        long r = c - e * per_e;
        const int k = (int)(r % SPW); r /= SPW;
        const int r16 = (int)(r % 16); r /= 16;
        const int m = (int)(r % 4); r /= 4;
        const int w = (int)(r % 4);
        const int j = (int)(r / 4);
        const long row = (long)(m >> 1) * I + j * UP_COLS + (m & 1) * 16 + r16;
        dst[c] = src[e * per_e + row * (L / 128) + SPW * w + k];
    }
}

__global__ __launch_bounds__(256) void k_pack_w2(long total, int I, int L,
                                                 const uint4* __restrict__ src,
                                                 uint4* __restrict__ dst) {
    const int IS = I / 128;
    const long per_e = (long)I * L / 32;
    for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < total; c += (long)gridDim.x * 256) {
        const long e = c / per_e;
        long r = c - e * per_e;
        const int lane = (int)(r % 64); r /= 64;
        const int s = (int)(r % IS); r /= IS;
        const int m = (int)(r % 8); r /= 8;
        const int w = (int)(r % 4);
        const int jd = (int)(r / 4);
        const long row = (long)jd * 512 + w * 128 + m * 16 + (lane & 15);
        dst[c] = src[e * per_e + row * (I / 32) + s * 4 + (lane >> 4)];
    }
}

__global__ __launch_bounds__(256) void k_copy_u32(long total, const uint32_t* __restrict__ src,
                                                  uint32_t* __restrict__ dst) {
    for (long c = (long)blockIdx.x * 256 + threadIdx.x; c < total; c += (long)gridDim.x * 256)
        dst[c] = src[c];
}

hipError_t launch_pack_experts(int E, int L, int I, const uint8_t* w13, const uint8_t* s13,
                               const uint8_t* w2, const uint8_t* s2, uint8_t* pw13, uint8_t* ps13,
                               uint8_t* pw2, uint8_t* ps2, hipStream_t s) {
    const dim3 blk(256), grid(8 * num_cus());
    hipLaunchKernelGGL(k_pack_w13, grid, blk, 0, s, (long)E * I * L / 16, I, L,
                       (const uint4*)w13, (uint4*)pw13);
    hipLaunchKernelGGL(k_pack_s13, grid, blk, 0, s, (long)E * I * L / 64, I, L,
                       (const uint32_t*)s13, (uint32_t*)ps13);
    hipLaunchKernelGGL(k_pack_w2, grid, blk, 0, s, (long)E * I * L / 32, I, L,
                       (const uint4*)w2, (uint4*)pw2);
    hipLaunchKernelGGL(k_copy_u32, grid, blk, 0, s, (long)E * I * L / 128, (const uint32_t*)s2,
                       (uint32_t*)ps2);
    return hipGetLastError();
}

// ---- BF16-weight experts (small test models): plain FP32 FMA, one unit per item ------
__global__ __launch_bounds__(256) void k_ffn_bf16(int K, int L, int I,
                                                  const uint16_t* __restrict__ w13,
                                                  const uint16_t* __restrict__ w2,
                                                  const uint16_t* __restrict__ latent,
                                                  const int32_t* __restrict__ pairs,
                                                  const int4* __restrict__ units,
                                                  const int32_t* __restrict__ num_units,
                                                  uint16_t* __restrict__ rows) {
    extern __shared__ float sm[];
    float* h = sm;           // [2I]
    float* act = sm + 2 * I; // [I]
    const int nunits = num_units[0];
    for (int u = blockIdx.x; u < nunits; u += gridDim.x) {
        const int4 un = units[u];
        const int e = un.x, begin = un.y, count = un.z;
        for (int n = 0; n < count; ++n) {
            const int p = pairs[begin + n];
            const uint16_t* a = latent + (size_t)(p / K) * L;
            for (int r = threadIdx.x; r < 2 * I; r += 256) {
                const uint16_t* wr = w13 + ((size_t)e * 2 * I + r) * L;
                float acc = 0.f;
                for (int k = 0; k < L; ++k) acc = __builtin_fmaf(bf16_to_f(a[k]), bf16_to_f(wr[k]), acc);
                h[r] = bf16_to_f((uint16_t)f_to_bf16(acc));
            }
            __syncthreads();
            for (int c = threadIdx.x; c < I; c += 256) {
                const float gt = h[c];
                act[c] = bf16_to_f((uint16_t)f_to_bf16(gt / (1.0f + __expf(-gt)) * h[I + c]));
            }
            __syncthreads();
            for (int r = threadIdx.x; r < L; r += 256) {
                const uint16_t* wr = w2 + ((size_t)e * L + r) * I;
                float acc = 0.f;
                for (int k = 0; k < I; ++k) acc = __builtin_fmaf(act[k], bf16_to_f(wr[k]), acc);
                rows[(size_t)p * L + r] = (uint16_t)f_to_bf16(acc);
            }
            __syncthreads();
        }
    }
}

hipError_t launch_ffn_bf16(int T, int K, int E, int L, int I, int unit, const void* w13,
                           const void* w2, const void* latent, const int32_t* pairs,
                           const int32_t* units, const int32_t* num_units, void* rows,
                           hipStream_t s) {
    const int max_units = (T * K + unit - 1) / unit + E;
    hipLaunchKernelGGL(k_ffn_bf16, dim3(persistent_blocks(max_units, 8)), dim3(256),
                       (size_t)3 * I * sizeof(float), s, K, L, I, (const uint16_t*)w13,
                       (const uint16_t*)w2, (const uint16_t*)latent, pairs, (const int4*)units,
                       num_units, (uint16_t*)rows);
    return hipGetLastError();
}

}  // namespace moe
