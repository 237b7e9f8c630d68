// wgemm.hip -- the dense BF16 projections of a decode step, out = x W^T with FP32
// accumulation (wide page, module summary and precision paragraph: BF16 dense
// projections, FP32 router logits, the latent rounded to BF16 once; ep/layer page,
// stock_order: the shared expert's gate_up and down, the up-projection added into the
// shared partial with one rounding).  The router rows and the latent down rows form one
// GEMM over x, as the wide page's front does (one FP32-out GEMM over the router rows and
// the latent down rows, packed ahead of the step).
//
// Decode batches are short (M = 65 .. 1020 tokens) and the weights long (N x K up to
// 12288 x 7168), so at M ~ 256 a projection is near the MFMA/HBM balance point: both
// the weight stream and the matrix cores must run close to their limits.  Design:
//  * one workgroup per CU (8 wavefronts); its tile is 256 weight rows x up to 256 tokens
//    over a K range (split-K), the largest FP32 accumulator tile the register file holds
//    (each wavefront: 32 rows x 256 tokens = 128 accumulators per lane);
//  * weights go straight from HBM into VGPRs as the A operands of
//    v_mfma_f32_32x32x16_bf16 (each wavefront streams its own 32 rows, so nothing is
//    shared and nothing goes through LDS); packed weights make each of these loads one
//    contiguous 1 KiB block per wavefront;
//  * activations go global -> LDS by direct loads (two 64-deep K stages, rows
//    XOR-swizzled in 16-byte chunks) and are read by all eight wavefronts as B operands;
//  * the LDS reads of the next group of token tiles are issued ahead of the current
//    group's MFMAs (scheduling groups pin that order), the next K stage's weights and
//    activations are in flight during the current stage's MFMAs;
//  * split-K partials go to an FP32 buffer [S][M][N]; a reduce kernel adds them in split
//    order and applies the epilogue (FP32 out, BF16 out, BF16 out of an added BF16
//    tensor plus the sum), or the consumer adds them itself (SiLU-and-mul).  The split
//    count balances filling the CUs against the partial traffic it costs.
#include "device.h"
#include "kernels.h"

namespace moe {

typedef float v16f __attribute__((ext_vector_type(16)));

// blocks b, b + 8, b + 16, ... run on one XCD (round-robin placement); give each XCD a
// contiguous run of work items so the workgroups sharing an activation K range share
// that XCD's L2
__device__ __forceinline__ int wg_xcd_item(int b, int G) {
    const int x = b & 7, j = b >> 3, q = G >> 3, r = G & 7;
    return x * q + (x < r ? x : r) + j;
}

struct WgArgs {
    const uint16_t* x;     // [M, K] BF16
    const uint16_t* w[3];  // row segments [0, N0), [N0, N1), [N1, N): row-major or packed
    float* part;           // [S][M][N] FP32
    unsigned* zero;        // optional: 16 words workgroup 0 sets to 0 (for a later launch)
    uint16_t* out;         // optional, with S = 1: BF16 [M, N] written directly, no partials
    int M, K, N, N0, N1, S, NX, MCH, prio;  // M chunks of 32 * MT32 tokens
};

// MT32: 32-token tiles computed per token chunk (1..8); KS: K depth of one LDS stage (64
// or 128); PACKED: weights in the packed layout of launch_pack_dense.
template <int MT32, int KS, bool PACKED>
__global__ __launch_bounds__(512, 1) void k_wgemm(const WgArgs a) {
    constexpr int CPR = KS / 8;   // 16-byte chunks of one token row of a stage
    constexpr int RB = KS * 2;    // bytes of one token row of a stage
    // token rows staged: whole rounds of direct loads (512 threads x 16 bytes)
    constexpr int ROWS = KS == 64 ? (MT32 + 1) / 2 * 64 : MT32 * 32;
    constexpr int LA = ROWS * CPR / 512;  // direct loads per thread per stage
    constexpr int SLOT = ROWS * RB;       // bytes of one LDS stage
    constexpr int NQ = KS / 16;           // MFMA K steps per stage
    constexpr int TSTR = 32 * RB;         // bytes between 32-token tiles in a stage
    // LDS fragments read ahead per group (a divisor of MT32; smaller where the registers of
    // 128-deep stages run short)
    constexpr int LOOK = (KS == 128 && MT32 >= 7)
                             ? (MT32 == 8 ? 2 : 1)
                             : (MT32 % 4 == 0 ? 4 : (MT32 % 3 == 0 ? 3 : (MT32 % 2 == 0 ? 2 : MT32)));
    constexpr int NG = MT32 / LOOK;  // LDS read groups per K step
    static_assert(LA * 512 == ROWS * CPR, "direct-load rounds");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * SLOT];
    if (a.prio) wave_priority_high();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (a.zero && blockIdx.x == 0 && tid < 16) a.zero[tid] = 0u;
    const int r32 = lane & 31, h = lane >> 5;
    // items: token chunk fastest, then weight tile, then K split -- the chunks of one
    // weight tile are neighbours on one XCD and share its weights through L2
    const int item = wg_xcd_item(blockIdx.x, a.NX * a.S * a.MCH);
    const int mc = item % a.MCH, rest = item / a.MCH;
    const int nt = rest % a.NX, z = rest / a.NX;
    const int Q = a.K / (2 * KS);  // K in pairs of stages
    const int q0 = z * Q / a.S, q1 = (z + 1) * Q / a.S;
    const int kb = q0 * 2 * KS, nst = (q1 - q0) * 2;
    const int n0 = nt * 256 + wave * 32;  // this wavefront's 32 output rows
    const int m0 = mc * 32 * MT32;

    // weight rows of this wavefront (past N: a valid tile, loaded but never stored)
    const int nrow = min(n0, a.N - 32);
    const int seg = nrow >= a.N1 ? 2 : (nrow >= a.N0 ? 1 : 0);
    const int wr = nrow - (seg == 2 ? a.N1 : (seg == 1 ? a.N0 : 0));
    const uint16_t* wm = a.w[seg];
    const uint16_t* wsrc =
        PACKED ? wm + (size_t)(wr / 64) * (a.K / 64) * 4096 + ((wr % 64) / 32) * 2048 + lane * 8
               : wm + (size_t)(wr + r32) * a.K + 8 * h;
    // Activation stage layout: token row r at r * RB, its 16-byte chunk c at position
    // c ^ sw(r), sw(r) = ((r >> 1) & 7) for 128-byte rows, (r & 15) for 256-byte rows, so
    // that the fragment reads of 16 consecutive rows hit 16 distinct bank groups.  The
    // direct loads fill LDS chunk p = i * 512 + tid with the global chunk that belongs there.
    uint32_t asrc[LA];  // element offsets into x (M * K < 2^31)
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int p = i * 512 + tid, r = p / CPR;
        const int c = (p % CPR) ^ (KS == 64 ? ((r >> 1) & 7) : (r & 15));
        asrc[i] = (uint32_t)(min(m0 + r, a.M - 1) * a.K + 8 * c);
    }
    // stages past the end repeat the last one (never used), so every thread always has
    // the same loads in flight
    uint4 wf[2][NQ];
    auto issue_w = [&](int slot, int st) {
        const int k0 = kb + min(st, nst - 1) * KS;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            wf[slot][q] = load_stream16(
                PACKED ? wsrc + (size_t)(k0 / 64 + q / 4) * 4096 + (q % 4) * 512
                       : wsrc + k0 + 16 * q);
    };
    // activations through a raw buffer resource: the MUBUF form of the direct LDS load
    // is counted on vmcnt alone (the FLAT form also counts as a pending LDS access, and
    // the compiler then waits lgkmcnt(0) at every fragment read, exposing the LDS latency
    // of the reads issued ahead)
    const int xbytes = (int)min((long)a.M * a.K * 2, 0x7fffffffL);
    auto issue_a = [&](int slot, int st) {
        const int k0 = kb + min(st, nst - 1) * KS;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            dma16(a.x, xbytes, (asrc[i] + k0) * 2,
                  (lds_ptr)(lds + slot * SLOT + (i * 512 + wave * 64) * 16));
    };
    v16f acc[MT32];
#pragma unroll
    for (int t = 0; t < MT32; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;

    // B operand of token tile t, K step q: row 32 t + r32, chunk 2 q + h (the swizzle term
    // depends on r32 only)
    const int sw = KS == 64 ? ((r32 >> 1) & 7) : (r32 & 15);
    int boff[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) boff[q] = r32 * RB + (((2 * q + h) ^ sw) << 4);

    issue_w(0, 0);
    issue_a(0, 0);
    issue_w(1, 1);
    for (int s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            // in flight in issue order: ... W(s) A(s) W(s+1): at most the NQ loads of
            // W(s + 1) may still be outstanding
            wait_vmcnt<NQ>();
            lds_sync();  // everyone's A(s) landed; everyone is done reading A(s - 1)
            issue_a(j ^ 1, s0 + j + 1);
            __builtin_amdgcn_sched_barrier(0);  // keeps A(s+1) ahead of W(s+2) in issue order
            const uint8_t* At = lds + j * SLOT;
            bf16x8 bc[LOOK], bn[LOOK];
#pragma unroll
            for (int u = 0; u < LOOK; ++u) bc[u] = *(const bf16x8*)(At + boff[0] + u * TSTR);
#pragma unroll
            for (int gq = 0; gq < NQ * NG; ++gq) {
                const int q = gq / NG, tg = gq % NG;
                if (gq + 1 < NQ * NG) {
                    const int qn = (gq + 1) / NG, tn = (gq + 1) % NG;
#pragma unroll
                    for (int u = 0; u < LOOK; ++u)
                        bn[u] = *(const bf16x8*)(At + boff[qn] + (tn * LOOK + u) * TSTR);
                }
                bf16x8 wa;
                __builtin_memcpy(&wa, &wf[j][q], 16);
#pragma unroll
                for (int u = 0; u < LOOK; ++u)
                    acc[tg * LOOK + u] =
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, bc[u], acc[tg * LOOK + u], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < LOOK; ++u) bc[u] = bn[u];
            }
            // the reads of group g + 1 go out before the MFMAs of group g
            __builtin_amdgcn_sched_group_barrier(0x100, LOOK, 0);
#pragma unroll
            for (int gq = 0; gq < NQ * NG; ++gq) {
                if (gq + 1 < NQ * NG) __builtin_amdgcn_sched_group_barrier(0x100, LOOK, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, LOOK, 0);
            }
            issue_w(j, s0 + j + 2);
        }
    }
    wait_vmcnt<0>();  // no direct load may still target LDS when the workgroup ends
    if (n0 >= a.N) return;
    // D layout: lane holds token column r32 of the tile, rows 8 (v / 4) + 4 h + v % 4
    if (a.out) {  // one split: the sum is final, rounded once to BF16
#pragma unroll
        for (int t = 0; t < MT32; ++t) {
            const int m = m0 + t * 32 + r32;
            if (m >= a.M) continue;
            uint16_t* dst = a.out + (size_t)m * a.N + n0 + 4 * h;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *(uint2*)(dst + 8 * jj) =
                    make_uint2(pack_bf16x2(acc[t][4 * jj], acc[t][4 * jj + 1]),
                               pack_bf16x2(acc[t][4 * jj + 2], acc[t][4 * jj + 3]));
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < MT32; ++t) {
        const int m = m0 + t * 32 + r32;
        if (m >= a.M) continue;
        float* dst = a.part + ((size_t)z * a.M + m) * a.N + n0 + 4 * h;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            *(v4f*)(dst + 8 * jj) = (v4f){acc[t][4 * jj], acc[t][4 * jj + 1], acc[t][4 * jj + 2],
                                          acc[t][4 * jj + 3]};
    }
}

// ---- plan ------------------------------------------------------------------------------
// Split count from a cost model: the time is the larger of the MFMA time of the busiest
// CU (rounds of workgroups) and the HBM time of the weights plus the split partials
// (written, then read back by the reduce; counted once with parts_once, for a GEMM at the
// end of the step whose reduce reads them right away with nothing else running: measured
// on the up-projection at 256 tokens, 4 splits of 128-token chunks instead of 3 gain
// 2 us a layer).  Rates are measured ones of this kernel on
// MI355X: ~5 TFLOP/s per CU in its MFMA loop, ~5.5 TB/s of HBM traffic.  `share` is the
// fraction of the GPU the GEMM is planned for (below 1 for a GEMM that runs beside
// other work: fewer splits, fewer partial bytes).
struct WgPlan {
    int S, NX, MCH, MT32, KS;
};

// Token chunks: 256 tokens (MT32 = 8; fewer for M < 256) or 128 (MT32 = 4, twice the
// workgroups for the same split count); the chunks of one weight tile read its weights
// once from HBM (neighbouring items on one XCD).  Token counts fall in classes (32-token
// steps up to 256, 128-token steps past it) with one plan each.
static int wg_class(int M) { return M <= 256 ? (M + 31) / 32 * 32 : (M + 127) / 128 * 128; }

static WgPlan wg_plan(int M, int N, int K, double share, bool parts_once, int smax = 64) {
    const int KS = 64;  // (128-deep stages measured no faster at the layer's shapes)
    const int NX = (N + 255) / 256;
    const int Q = K / (2 * KS);
    const double cus = gemm_device_cus() * share, rate = 5.0e12, bw = 5.5e12 * share;
    // one workgroup streams weights at ~32 GB/s (the loads it keeps in flight over the
    // loaded latency; measured on 36..48 workgroups at 8 tokens), so a plan with few
    // workgroups cannot reach the HBM rate however small its partials are
    const double bw_wg = 32e9;
    const double wbytes = (double)N * K * 2;
    // the class end bounds the partials: the plan is the same for every M of a class
    const double Mc = wg_class(M);
    WgPlan best_p{1, NX, 1, 1, KS};
    double best = 1e30;
    for (int chunk = 256; chunk >= 128; chunk /= 2) {
        if (chunk == 128 && M <= 128) break;
        const int mch = (M + chunk - 1) / chunk;
        const int mt32 = M < chunk ? (M + 31) / 32 : chunk / 32;
        for (int S = 1; S <= Q && S <= smax; ++S) {
            const double wgs = (double)NX * mch * S;
            const double rounds = (double)(long)((wgs + cus - 1) / cus);
            const double kz = (double)((Q + S - 1) / S) * 2 * KS;  // the longest K range
            const double t_mfma = rounds * 2.0 * 256 * (32.0 * mt32) * kz / rate;
            const double active = wgs < cus ? wgs : cus;
            const double rate_hbm = bw < active * bw_wg ? bw : active * bw_wg;
            const double t_parts = (parts_once ? 1.0 : 2.0) * S * Mc * N * 4 / rate_hbm;
            // up to 256 tokens the partials' traffic overlaps the MFMA time; past 256 the
            // GEMM is MFMA-bound and its partials add to it (the stores follow each
            // workgroup's main loop, the reads are a launch of their own): measured at 1020
            // tokens, 3 splits of the front GEMM instead of 7 gain 34 us a layer
            const double t_w = wbytes / rate_hbm;
            const double t = M > 256 ? (t_mfma > t_w ? t_mfma : t_w) + t_parts
                                     : (t_mfma > t_w + t_parts ? t_mfma : t_w + t_parts);
            if (t < best * 0.995) {
                best = t;
                best_p = WgPlan{S, NX, mch, mt32, KS};
            }
        }
    }
    return best_p;
}

bool wgemm_fits(int M, int N, int N0, int N1, int K, bool packed) {
    const int q = packed ? 64 : 32;
    if (K < 128 || K % 128 || N < 32 || N0 < 0 || N1 < N0 || N1 > N) return false;
    if (M < 1 || (long)M * K >= (1L << 31)) return false;  // 32-bit activation offsets
    return N0 % q == 0 && (N1 - N0) % q == 0 && (N - N1) % q == 0;
}

int wgemm_splits(int M, int N, int K, double share, bool parts_once) {
    return wg_plan(M, N, K, share, parts_once).S;
}

size_t wgemm_parts_bytes(int M, int N, int K, double share, bool parts_once) {
    // the plan depends on M through the 32-token tile count and the 256-token chunks:
    // the largest M of each class bounds its partial buffer
    size_t best = 0;
    for (int m = 32;; m += (m < 256 ? 32 : 128)) {
        const int mm = m < M ? m : M;
        const size_t b = (size_t)wg_plan(mm, N, K, share, parts_once).S * mm * N * sizeof(float);
        if (b > best) best = b;
        if (m >= M) break;
    }
    return best;
}

template <int MT32, int KS>
static hipError_t launch_mt(const WgArgs& a, bool packed, int G, hipStream_t s) {
    if (packed)
        hipLaunchKernelGGL((k_wgemm<MT32, KS, true>), dim3(G), dim3(512), 0, s, a);
    else
        hipLaunchKernelGGL((k_wgemm<MT32, KS, false>), dim3(G), dim3(512), 0, s, a);
    return hipGetLastError();
}

template <int KS>
static hipError_t launch_ks(const WgArgs& a, int mt32, bool packed, int G, hipStream_t s) {
    switch (mt32) {
        case 1: return launch_mt<1, KS>(a, packed, G, s);
        case 2: return launch_mt<2, KS>(a, packed, G, s);
        case 3: return launch_mt<3, KS>(a, packed, G, s);
        case 4: return launch_mt<4, KS>(a, packed, G, s);
        case 5: return launch_mt<5, KS>(a, packed, G, s);
        case 6: return launch_mt<6, KS>(a, packed, G, s);
        case 7: return launch_mt<7, KS>(a, packed, G, s);
        default: return launch_mt<8, KS>(a, packed, G, s);
    }
}

hipError_t launch_wgemm(int M, int N, int N0, int N1, int K, const void* x, const void* w0,
                        const void* w1, const void* w2, bool packed, float* parts, hipStream_t s,
                        bool prio, int* S, double share, unsigned* zero, bool parts_once,
                        void* out_bf16) {
    const WgPlan p = wg_plan(M, N, K, share, parts_once, out_bf16 ? 1 : 64);
    WgArgs a;
    a.zero = zero;
    a.out = (uint16_t*)out_bf16;
    a.x = (const uint16_t*)x;
    a.w[0] = (const uint16_t*)w0;
    a.w[1] = (const uint16_t*)(w1 ? w1 : w0);
    a.w[2] = (const uint16_t*)(w2 ? w2 : a.w[1]);
    a.part = parts;
    a.M = M;
    a.K = K;
    a.N = N;
    a.N0 = N0;
    a.N1 = N1;
    a.S = p.S;
    a.NX = p.NX;
    a.MCH = p.MCH;
    a.prio = prio ? 1 : 0;
    *S = p.S;
    const int G = p.NX * p.S * p.MCH;
    return launch_ks<64>(a, p.MT32, packed, G, s);
}

// ---- split reduce + epilogue -----------------------------------------------------------
// Of the partial rows (stride N), columns [0, N0) -> out0 as FP32 (the router logits of
// the front GEMM), columns [N0, N1) -> out1 (row stride N1 - N0) with MODE 0 FP32, 1 BF16
// (one rounding), 2 BF16 of FP32(add1) + sum; columns from N1 on are left to another
// consumer.  Four columns per thread; the S partials are added in split order.
// q: the four BF16 values of the added tensor at idx (MODE 2), loaded by the caller
template <int MODE>
__device__ __forceinline__ void store4(void* out, uint2 q, size_t idx, v4f v) {
    if (MODE == 0) {
        *(v4f*)((float*)out + idx) = v;
    } else {
        if (MODE == 2) {
            v[0] += bf16_lo(q.x);
            v[1] += bf16_hi(q.x);
            v[2] += bf16_lo(q.y);
            v[3] += bf16_hi(q.y);
        }
        *(uint2*)((uint16_t*)out + idx) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
}

template <int MODE1>
__global__ __launch_bounds__(256) void k_wg_reduce(int M, int N, int N0, int N1, int S,
                                                   const float* __restrict__ part, float* out0,
                                                   void* out1, const void* add1, int prio) {
    if (prio) wave_priority_high();
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int n4 = N1 / 4;
    if (idx >= (long)M * n4) return;
    const int m = (int)(idx / n4), c = (int)(idx - (long)m * n4) * 4;
    const size_t i1 = (size_t)m * (N1 - N0) + (c >= N0 ? c - N0 : 0);
    // the added values go out with the partials' loads (unconditionally, from a clamped
    // index: a load behind a branch would be waited for on its own)
    const uint2 q = MODE1 == 2 ? *(const uint2*)((const uint16_t*)add1 + i1) : make_uint2(0, 0);
    const v4f v = sum_splits(part + (size_t)m * N + c, (size_t)M * N, S);
    if (c < N0)
        store4<0>(out0, q, (size_t)m * N0 + c, v);
    else
        store4<MODE1>(out1, q, i1, v);
}

hipError_t launch_wg_reduce(int M, int N, int N0, int N1, int S, const float* parts, float* out0,
                            int mode1, void* out1, const void* add1, hipStream_t s, bool prio) {
    const long n = (long)M * (N1 / 4);
    const dim3 grid((unsigned)((n + 255) / 256)), blk(256);
    const int pr = prio ? 1 : 0;
    if (mode1 == 0)
        hipLaunchKernelGGL(k_wg_reduce<0>, grid, blk, 0, s, M, N, N0, N1, S, parts, out0, out1, add1, pr);
    else if (mode1 == 1)
        hipLaunchKernelGGL(k_wg_reduce<1>, grid, blk, 0, s, M, N, N0, N1, S, parts, out0, out1, add1, pr);
    else
        hipLaunchKernelGGL(k_wg_reduce<2>, grid, blk, 0, s, M, N, N0, N1, S, parts, out0, out1, add1, pr);
    return hipGetLastError();
}

// ---- packed dense layout ---------------------------------------------------------------
// W [N, K] BF16 row-major -> blocks of 1 KiB: [N/64 row groups][K/64 K stages][tile 2]
// [K step 4][lane 64][8 BF16], lane l of (group g, stage s, tile i, step q) holding row
// 64 g + 32 i + l % 32, columns 64 s + 16 q + 8 (l / 32) .. + 8: the A operand of one
// 32x32x16 MFMA.  A wavefront's loads for one K stage are 4 KiB in a row.
__global__ __launch_bounds__(256) void k_pack_dense(int N, int K, const uint4* __restrict__ w,
                                                    uint4* __restrict__ p) {
    const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;  // one 16-byte chunk
    if (id >= (size_t)N * K / 8) return;
    const int lane = (int)(id & 63), q = (int)((id >> 6) & 3), i = (int)((id >> 8) & 1);
    const size_t rest = id >> 9;
    const int ks = (int)(rest % (K / 64)), g = (int)(rest / (K / 64));
    const int row = g * 64 + 32 * i + (lane & 31);
    const int col = ks * 64 + 16 * q + 8 * (lane >> 5);
    p[id] = w[((size_t)row * K + col) / 8];
}

hipError_t launch_pack_dense(int N, int K, const void* w, void* out, hipStream_t s) {
    const size_t n = (size_t)N * K / 8;
    hipLaunchKernelGGL(k_pack_dense, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, N, K,
                       (const uint4*)w, (uint4*)out);
    return hipGetLastError();
}

}  // namespace moe
