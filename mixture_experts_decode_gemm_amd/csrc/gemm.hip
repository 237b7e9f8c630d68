// gemm.hip -- dense BF16 linears out = x W^T with FP32 accumulation (wide page, module
// summary: "BF16 linears", "FP32 router logits", "the latent rounded once to BF16";
// ep/layer page, stock_order and the "cuBLAS addmm: one rounding" of the up-projection).
//
// Decode shapes are skinny (M = tokens, 65..1020) and wide (N up to 12288, K up to 7168):
// the weights are streamed once, the activations re-read from L2.  Tiles are 128 x 128
// with BK = 64, 256 threads as 2 x 2 wavefronts of 64 x 64 (4 x 4 MFMA 16x16x32 BF16
// tiles), LDS single-buffered with the next K-step prefetched into registers.  When the
// tile grid is too small to fill the 256 CUs the K range is split; the split partials go
// to an FP32 scratch and a second kernel adds them in split order and applies the
// epilogue (FP32 out, BF16 out, or BF16 out of FP32(add) + acc).
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int BM = 128, BN = 128, BK = 64, LDSK = BK + 8;  // +8: rows 144 B apart

struct Split {
    int S, kchunk;
};

static Split choose_split(int M, int N, int K) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    int S = (512 + tiles - 1) / tiles;
    const int maxS = K / 256 > 0 ? K / 256 : 1;
    if (S > maxS) S = maxS;
    if (S < 1) S = 1;
    int kchunk = ((K / S + BK - 1) / BK) * BK;
    S = (K + kchunk - 1) / kchunk;
    return {S, kchunk};
}

size_t gemm_scratch_bytes(int M, int N, int K) {
    // the largest split partial buffer over every token count up to M
    size_t best = 0;
    for (int mt = 1; mt <= (M + BM - 1) / BM; ++mt) {
        const int m = mt * BM < M ? mt * BM : M;
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
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm(int M, int N, int K, int kchunk,
                                              const uint16_t* __restrict__ x,
                                              const uint16_t* __restrict__ w, void* out,
                                              const void* add) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDSK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDSK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int kb = blockIdx.z * kchunk;
    const int ke = min(K, kb + kchunk);

    uint4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            const int r = q >> 3, c = (q & 7) * 8;
            ra[i] = (m0 + r < M) ? *(const uint4*)(x + (size_t)(m0 + r) * K + k0 + c)
                                 : make_uint4(0, 0, 0, 0);
            rb[i] = (n0 + r < N) ? *(const uint4*)(w + (size_t)(n0 + r) * K + k0 + c)
                                 : make_uint4(0, 0, 0, 0);
        }
    };
    v4f acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (v4f){0.f, 0.f, 0.f, 0.f};

    gload(kb);
    for (int k0 = kb; k0 < ke; k0 += BK) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i;
            const int r = q >> 3, c = (q & 7) * 8;
            *(uint4*)(As + r * LDSK + c) = ra[i];
            *(uint4*)(Bs + r * LDSK + c) = rb[i];
        }
        __syncthreads();
        if (k0 + BK < ke) gload(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = *(const bf16x8*)(As + (wm * 64 + i * 16 + (lane & 15)) * LDSK + kk +
                                         8 * (lane >> 4));
                fb[i] = *(const bf16x8*)(Bs + (wn * 64 + i * 16 + (lane & 15)) * LDSK + kk +
                                         8 * (lane >> 4));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fb[b], acc[a][b], 0,
                                                                        0, 0);
        }
    }
    // D tile layout: lane l holds rows 4*(l/16)+i, column l%16
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = n0 + wn * 64 + b * 16 + (lane & 15);
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + wm * 64 + a * 16 + 4 * (lane >> 4) + i;
                if (row >= M) continue;
                if (MODE == 3) {
                    ((float*)out)[((size_t)blockIdx.z * M + row) * N + col] = acc[a][b][i];
                } else {
                    store_out<MODE>(out, add, (size_t)row * N + col, acc[a][b][i]);
                }
            }
        }
}

template <int MODE>
__global__ __launch_bounds__(256) void k_splitk_reduce(int M, int N, int S,
                                                       const float* __restrict__ part,
                                                       void* out, const void* add) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)M * N;
    if (idx >= total) return;
    float v = part[idx];
    for (int z = 1; z < S; ++z) v += part[(size_t)z * total + idx];
    store_out<MODE>(out, add, idx, v);
}

hipError_t launch_gemm(int M, int N, int K, const void* x, const void* w, void* out,
                       const void* add, int mode, void* scratch, hipStream_t s) {
    const Split sp = choose_split(M, N, K);
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, sp.S);
    const uint16_t* xa = (const uint16_t*)x;
    const uint16_t* wa = (const uint16_t*)w;
    if (sp.S == 1) {
        if (mode == 0) hipLaunchKernelGGL(k_gemm<0>, grid, dim3(256), 0, s, M, N, K, sp.kchunk, xa, wa, out, add);
        else if (mode == 1) hipLaunchKernelGGL(k_gemm<1>, grid, dim3(256), 0, s, M, N, K, sp.kchunk, xa, wa, out, add);
        else hipLaunchKernelGGL(k_gemm<2>, grid, dim3(256), 0, s, M, N, K, sp.kchunk, xa, wa, out, add);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_gemm<3>, grid, dim3(256), 0, s, M, N, K, sp.kchunk, xa, wa, scratch,
                       (const void*)nullptr);
    const size_t total = (size_t)M * N;
    const int blocks = (int)((total + 255) / 256);
    const float* part = (const float*)scratch;
    if (mode == 0) hipLaunchKernelGGL(k_splitk_reduce<0>, dim3(blocks), dim3(256), 0, s, M, N, sp.S, part, out, add);
    else if (mode == 1) hipLaunchKernelGGL(k_splitk_reduce<1>, dim3(blocks), dim3(256), 0, s, M, N, sp.S, part, out, add);
    else hipLaunchKernelGGL(k_splitk_reduce<2>, dim3(blocks), dim3(256), 0, s, M, N, sp.S, part, out, add);
    return hipGetLastError();
}

}  // namespace moe
