// gemm.hip -- dense BF16 linears out = x W^T with FP32 accumulation (wide page, module
// summary, precision paragraph: BF16 dense projections, router logits in FP32, the
// latent rounded to BF16 once; ep/layer page, stock_order, and the single rounding of
// the up-projection added into the shared partial).
//
// Decode shapes are skinny (M = tokens, 65..1020) and wide (N up to 12288, K up to 7168):
// the weights must stream from HBM at full rate, which takes many bytes in flight per CU.
// Tiles are 128 x 64 with BK = 64; both operand tiles go global -> LDS by direct loads
// (no register staging), rows XOR-swizzled in 16-byte chunks so that the MFMA fragment
// reads of 16 rows hit distinct LDS bank groups; NS LDS stages with NS - 1 K-steps in
// flight.  Small stages (24 KB each) let three workgroups share a CU, and it is that
// occupancy, more than pipeline depth, which keeps HBM busy.  Four wavefronts as 2 x 2,
// each 64 x 32 (4 x 2 MFMA 16x16x32 BF16 tiles); FP32 accumulation.  When the tile grid
// is too small to fill the CUs the K range is split; split partials go to an FP32 scratch
// and a second kernel adds them in split order and applies the epilogue (FP32 out, BF16
// out, or BF16 out of FP32(add) + acc).
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int GEMM_BM = 128, GEMM_BN = 64, BK = 64;
constexpr int GEMM_NS = 2;                                    // LDS stages
constexpr int GEMM_LDS = GEMM_NS * (GEMM_BM + GEMM_BN) * BK * 2;  // bytes per workgroup
constexpr int GEMM_WG_PER_CU = (160 * 1024 / GEMM_LDS) < 4 ? (160 * 1024 / GEMM_LDS) : 4;

struct Split {
    int S, kchunk;
};

static int gemm_cus() {
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

static Split choose_split(int M, int N, int K) {
    const int tiles = ((M + GEMM_BM - 1) / GEMM_BM) * ((N + GEMM_BN - 1) / GEMM_BN);
    const int target = gemm_cus() * GEMM_WG_PER_CU;  // one round of resident workgroups
    int S = (target + tiles - 1) / tiles;
    const int maxS = K / 512 > 0 ? K / 512 : 1;  // keep at least 8 K-steps per split
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    int kchunk = ((K / S + BK - 1) / BK) * BK;
    S = (K + kchunk - 1) / kchunk;
    return {S, kchunk};
}

size_t gemm_scratch_bytes(int M, int N, int K) {
    // the largest split partial buffer over every token count up to M
    size_t best = 0;
    for (int mt = 1; mt <= (M + GEMM_BM - 1) / GEMM_BM; ++mt) {
        const int m = mt * GEMM_BM < M ? mt * GEMM_BM : M;
        const Split sp = choose_split(m, N, K);
        if (sp.S > 1) {
            const size_t b = (size_t)sp.S * m * N * sizeof(float);
            if (b > best) best = b;
        }
    }
    return best;
}

template <int MODE>
__device__ __forceinline__ void store_out(void* out, const void* add, size_t idx, float v) {
    if (MODE == 0) {
        ((float*)out)[idx] = v;
    } else if (MODE == 1) {
        ((uint16_t*)out)[idx] = (uint16_t)f_to_bf16(v);
    } else {
        const float a = bf16_to_f(((const uint16_t*)add)[idx]);
        ((uint16_t*)out)[idx] = (uint16_t)f_to_bf16(a + v);
    }
}

// MODE: 0 FP32 out, 1 BF16 out, 2 BF16 out + add; 3 FP32 split partial (out = scratch)
// One output tile (m0, n0) over K range [kb, ke) of split z.
template <int MODE, int NS>
__device__ __forceinline__ void gemm_tile(int M, int N, int K, int m0, int n0, int z, int kb,
                                          int ke, const uint16_t* __restrict__ x,
                                          const uint16_t* __restrict__ w, void* out,
                                          const void* add) {
    constexpr int BM = GEMM_BM, BN = GEMM_BN;
    constexpr int LA = BM * 8 / 256, LB = BN * 8 / 256;  // 16-byte chunks per thread per step
    // stage s: [BM rows of x][BN rows of w], 128 bytes a row; row r's chunk c at c ^ ((r>>1)&7)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NS][(BM + BN) * BK * 2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int nsteps = (ke - kb) / BK;

    // the direct loads of a wavefront fill 64 consecutive 16-byte LDS chunks, so LDS chunk
    // p = i*256 + tid receives the global chunk that belongs there after the swizzle.
    // Rows past M or N read a valid row (clamped); their results are never stored.
    const uint16_t* srcA[LA];
    const uint16_t* srcB[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int p = i * 256 + tid, r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
        srcA[i] = x + (size_t)min(m0 + r, M - 1) * K + 8 * c;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int p = i * 256 + tid, r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
        srcB[i] = w + (size_t)min(n0 + r, N - 1) * K + 8 * c;
    }
    auto issue = [&](int slot, int k0) {
#pragma unroll
        for (int i = 0; i < LA; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(srcA[i] + k0),
                                             (lds_ptr)(lds[slot] + (i * 256 + wave * 64) * 16),
                                             16, 0, 0);
#pragma unroll
        for (int i = 0; i < LB; ++i)
            __builtin_amdgcn_global_load_lds(
                (const void*)(srcB[i] + k0),
                (lds_ptr)(lds[slot] + BM * BK * 2 + (i * 256 + wave * 64) * 16), 16, 0, 0);
    };
    v4f acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

    // prologue: NS - 1 steps in flight (past the end: a repeat of the first step, unused,
    // so that every thread always has the same number of loads outstanding)
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, st < nsteps ? kb + st * BK : kb);
    for (int ks = 0; ks < nsteps; ++ks) {
        wait_vmcnt<(NS - 2) * (LA + LB)>();  // this thread's loads of step ks have landed
        lds_barrier();                       // ... everyone's; step ks - 1 fully consumed
        const int nk = ks + NS - 1;
        issue(nk % NS, nk < nsteps ? kb + nk * BK : kb);
        const uint8_t* At = lds[ks % NS];
        const uint8_t* Bt = At + BM * BK * 2;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c = kk * 4 + g;
            bf16x8 fb[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int rb = wn * 32 + b * 16 + r16;
                fb[b] = *(const bf16x8*)(Bt + rb * 128 + ((c ^ ((rb >> 1) & 7)) << 4));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int ra = wm * 64 + a * 16 + r16;
                const bf16x8 fa = *(const bf16x8*)(At + ra * 128 + ((c ^ ((ra >> 1) & 7)) << 4));
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb[b], acc[a][b], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();  // no load may still target LDS when the workgroup ends
    // D tile layout: lane l holds rows 4*(l/16)+i, column l%16
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int col = n0 + wn * 32 + b * 16 + r16;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + wm * 64 + a * 16 + 4 * g + i;
                if (row >= M) continue;
                if (MODE == 3) {
                    ((float*)out)[((size_t)z * M + row) * N + col] = acc[a][b][i];
                } else {
                    store_out<MODE>(out, add, (size_t)row * N + col, acc[a][b][i]);
                }
            }
        }
}

// Work item t = (n tile fastest, then m tile, then split); a workgroup takes items
// blockIdx.x, blockIdx.x + gridDim.x, ... (one item each when the grid covers them all; a
// narrower persistent grid leaves room on every CU for kernels running beside it).
template <int MODE, int NS>
__global__ __launch_bounds__(256) void k_gemm(int M, int N, int K, int kchunk, int S, int prio,
                                              const uint16_t* __restrict__ x,
                                              const uint16_t* __restrict__ w, void* out,
                                              const void* add) {
    if (prio) wave_priority_high();
    const int NX = (N + GEMM_BN - 1) / GEMM_BN, MY = (M + GEMM_BM - 1) / GEMM_BM;
    const int items = NX * MY * S;
    for (int t = blockIdx.x; t < items; t += gridDim.x) {
        const int nt = t % NX, mt = (t / NX) % MY, z = t / (NX * MY);
        const int kb = z * kchunk;
        gemm_tile<MODE, NS>(M, N, K, mt * GEMM_BM, nt * GEMM_BN, z, kb, min(K, kb + kchunk), x,
                            w, out, add);
        if (t + gridDim.x < items) __syncthreads();  // the next item's loads reuse the LDS
    }
}

template <int MODE>
__global__ __launch_bounds__(256) void k_splitk_reduce(int M, int N, int S,
                                                       const float* __restrict__ part,
                                                       void* out, const void* add) {
    wave_priority_high();
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)M * N;
    if (idx >= total) return;
    float v = part[idx];
    for (int z = 1; z < S; ++z) v += part[(size_t)z * total + idx];
    store_out<MODE>(out, add, idx, v);
}

hipError_t launch_gemm(int M, int N, int K, const void* x, const void* w, void* out,
                       const void* add, int mode, void* scratch, hipStream_t s, int max_wg,
                       bool prio) {
    const Split sp = choose_split(M, N, K);
    const uint16_t* xa = (const uint16_t*)x;
    const uint16_t* wa = (const uint16_t*)w;
    const int items = ((N + GEMM_BN - 1) / GEMM_BN) * ((M + GEMM_BM - 1) / GEMM_BM) * sp.S;
    const dim3 grid(max_wg > 0 && max_wg < items ? max_wg : items);
    const dim3 blk(256);
    if (sp.S == 1) {
        if (mode == 0)
            hipLaunchKernelGGL((k_gemm<0, GEMM_NS>), grid, blk, 0, s, M, N, K, sp.kchunk, 1, prio, xa, wa, out, add);
        else if (mode == 1)
            hipLaunchKernelGGL((k_gemm<1, GEMM_NS>), grid, blk, 0, s, M, N, K, sp.kchunk, 1, prio, xa, wa, out, add);
        else
            hipLaunchKernelGGL((k_gemm<2, GEMM_NS>), grid, blk, 0, s, M, N, K, sp.kchunk, 1, prio, xa, wa, out, add);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_gemm<3, GEMM_NS>), grid, blk, 0, s, M, N, K, sp.kchunk, sp.S, prio, xa,
                       wa, scratch, (const void*)nullptr);
    const size_t total = (size_t)M * N;
    const int blocks = (int)((total + 255) / 256);
    const float* part = (const float*)scratch;
    if (mode == 0)
        hipLaunchKernelGGL(k_splitk_reduce<0>, dim3(blocks), blk, 0, s, M, N, sp.S, part, out, add);
    else if (mode == 1)
        hipLaunchKernelGGL(k_splitk_reduce<1>, dim3(blocks), blk, 0, s, M, N, sp.S, part, out, add);
    else
        hipLaunchKernelGGL(k_splitk_reduce<2>, dim3(blocks), blk, 0, s, M, N, sp.S, part, out, add);
    return hipGetLastError();
}

int gemm_device_cus() { return gemm_cus(); }

int gemm_splits(int M, int N, int K) { return choose_split(M, N, K).S; }

size_t gemm_parts_bytes(int M, int N, int K) {
    size_t best = 0;
    for (int mt = 1; mt <= (M + GEMM_BM - 1) / GEMM_BM; ++mt) {
        const int m = mt * GEMM_BM < M ? mt * GEMM_BM : M;
        const size_t b = (size_t)choose_split(m, N, K).S * m * N * sizeof(float);
        if (b > best) best = b;
    }
    return best;
}

hipError_t launch_gemm_parts(int M, int N, int K, const void* x, const void* w, float* parts,
                             hipStream_t s, bool prio, int* S) {
    const Split sp = choose_split(M, N, K);
    const int items = ((N + GEMM_BN - 1) / GEMM_BN) * ((M + GEMM_BM - 1) / GEMM_BM) * sp.S;
    hipLaunchKernelGGL((k_gemm<3, GEMM_NS>), dim3(items), dim3(256), 0, s, M, N, K, sp.kchunk,
                       sp.S, prio ? 1 : 0, (const uint16_t*)x, (const uint16_t*)w, (void*)parts,
                       (const void*)nullptr);
    *S = sp.S;
    return hipGetLastError();
}

}  // namespace moe
