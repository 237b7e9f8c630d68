// router.hip -- sigmoid top-K routing (ep/layer page, EpMoeLayer.topk: the stock
// router's sigmoid top-16 over one group with the correction bias, renormalize and
// scale; wide page, WideRoute: an exact top-16 with renormalised weights).
//
// One wavefront per token.  Each lane owns experts lane, lane+64, ... (<= 16 per lane,
// E <= 1024) and builds 64-bit selection keys (order-preserving bits of the FP32 key
// s + bias, then the complemented expert id so that equal keys prefer the lower id).
// K rounds of a wave-wide maximum (xor shuffles) pick the winners in descending order;
// the winner's lane clears its key.  Lane k keeps slot k's score; the slot-order FP32
// sum, the divide and the routed scale follow.
//
// The sigmoid is 1/(1 + E(-x)) with E a defined exponential (Cody-Waite reduction with a
// 16-significant-bit head of ln 2, degree-7 Taylor polynomial by Horner's rule, scaling
// by 2^n), each step one IEEE FP32 operation, so any correct implementation of the same
// steps gives the same bits.  This file is compiled with -ffp-contract=off.
#include "device.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr float kLog2e = 0x1.715476p+0f;
constexpr float kLn2Hi = 0x1.62e4p-1f;    // ln 2 to 16 significant bits
constexpr float kLn2Lo = 0x1.7f7d1cp-20f; // FP32(ln 2 - kLn2Hi)
constexpr float kC[8] = {0x1p+0f,        0x1p+0f,        0x1p-1f,        0x1.555556p-3f,
                         0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f};
}  // namespace

__device__ __forceinline__ float exp_defined(float z) {
    const float nf = rintf(__fmul_rn(z, kLog2e));
    float r = __builtin_fmaf(-nf, kLn2Hi, z);
    r = __builtin_fmaf(-nf, kLn2Lo, r);
    float p = kC[7];
#pragma unroll
    for (int k = 6; k >= 0; --k) p = __builtin_fmaf(p, r, kC[k]);
    return ldexpf(p, (int)nf);
}

__device__ __forceinline__ float sigmoid_defined(float logit) {
    const float z = -logit;
    if (z > 88.0f) return 0.0f;
    if (z < -87.0f) return 1.0f;
    const float den = __fadd_rn(1.0f, exp_defined(z));
    return 1.0f / den;  // IEEE division (correctly rounded by default on gfx950)
}

__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;  // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(256) void k_topk(int T, int E, int K, const float* __restrict__ logits,
                                              const float* __restrict__ bias, int renorm,
                                              float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ weights) {
    wave_priority_high();
    constexpr int PER = 16;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wavefront
    const float* lg = logits + (size_t)t * E;
    uint32_t khi[PER], klo[PER];
    float sc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = j * 64 + lane;
        if (e < E) {
            const float s = sigmoid_defined(lg[e]);
            sc[j] = s;
            khi[j] = order_bits(__fadd_rn(s, bias[e]));
            klo[j] = ~(uint32_t)e;
        } else {
            sc[j] = 0.0f;
            khi[j] = 0;
            klo[j] = 0;
        }
    }
    float mine = 0.0f;  // lane k holds the score chosen for slot k
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
        uint32_t bh = 0, bl = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const bool gt = khi[j] > bh || (khi[j] == bh && klo[j] > bl);
            bh = gt ? khi[j] : bh;
            bl = gt ? klo[j] : bl;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const uint32_t oh = (uint32_t)__shfl_xor((int)bh, off, 64);
            const uint32_t ol = (uint32_t)__shfl_xor((int)bl, off, 64);
            const bool gt = oh > bh || (oh == bh && ol > bl);
            bh = gt ? oh : bh;
            bl = gt ? ol : bl;
        }
        const int win = (int)(~bl);
        const int owner = win & 63;
        float s_own = 0.0f;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (j * 64 + lane == win) {
                s_own = sc[j];
                khi[j] = 0;
                klo[j] = 0;
            }
        }
        const float s_win = __shfl(s_own, owner, 64);
        if (lane == k) {
            mine = s_win;
            my_id = win;
        }
    }
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum = __fadd_rn(sum, __shfl(mine, k, 64));
    if (lane < K) {
        float w = renorm ? mine / sum : mine;
        w = __fmul_rn(w, scale);
        ids[(size_t)t * K + lane] = my_id;
        weights[(size_t)t * K + lane] = w;
    }
}

hipError_t launch_topk(int T, int E, int K, const float* logits, const float* bias, int renorm,
                       float scale, int32_t* ids, float* w, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, T, E, K, logits, bias, renorm,
                       scale, ids, w);
    return hipGetLastError();
}

}  // namespace moe
