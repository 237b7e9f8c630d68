// router.hip -- sigmoid top-K routing (ep/layer page, EpMoeLayer.topk: the stock
// router's sigmoid top-16 over one group with the correction bias, renormalize and
// scale; wide page, WideRoute: an exact top-16 with renormalised weights).
//
// One wavefront per token.  Each lane owns experts lane, lane+64, ... (<= 16 per lane,
// E <= 1024) and builds 64-bit selection keys (order-preserving bits of the FP32 key
// s + bias, then the complemented expert id so that equal keys prefer the lower id).
// K rounds of a wave-wide maximum (DPP, then readlane) pick the winners in descending
// order; the winner's lane clears its key.  Lane k keeps slot k's score; the slot-order
// FP32 sum, the divide and the routed scale follow.
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

// Wave-wide maximum of 64-bit keys (hi, lo), returned in every lane: DPP row shifts by
// 1, 2, 4, 8 leave each row's maximum in its lane 15, row broadcasts 15 and 31 carry them
// to lane 63, and a readlane makes it uniform.  Lanes outside a shift's reach combine
// with 0, the identity (every live key is nonzero).
__device__ __forceinline__ void dpp_step(uint32_t& h, uint32_t& l, uint32_t oh, uint32_t ol) {
    const bool gt = oh > h || (oh == h && ol > l);
    h = gt ? oh : h;
    l = gt ? ol : l;
}
#define MOE_DPP(ctrl, rmask)                                                                   \
    dpp_step(h, l, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, ctrl, rmask, 0xf, false), \
             (uint32_t)__builtin_amdgcn_update_dpp(0, (int)l, ctrl, rmask, 0xf, false))
__device__ __forceinline__ void wave_max64(uint32_t& h, uint32_t& l) {
    MOE_DPP(0x111, 0xf);  // row_shr:1
    MOE_DPP(0x112, 0xf);  // row_shr:2
    MOE_DPP(0x114, 0xf);  // row_shr:4
    MOE_DPP(0x118, 0xf);  // row_shr:8
    MOE_DPP(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    MOE_DPP(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
    h = (uint32_t)__builtin_amdgcn_readlane((int)h, 63);
    l = (uint32_t)__builtin_amdgcn_readlane((int)l, 63);
}
#undef MOE_DPP

// One wavefront per token.
// slot_of (optional, [T][E] bytes): slot_of[t][e] = the slot that chose expert e, for
// the list build (entries of experts a token did not choose are left as they are).
__global__ __launch_bounds__(256) void k_topk(int T, int E, int K, const float* __restrict__ src,
                                              const float* __restrict__ bias, int renorm,
                                              float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ weights,
                                              uint8_t* __restrict__ slot_of) {
    wave_priority_high();
    constexpr int PER = 16;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wavefront
    uint32_t khi[PER], klo[PER];
    float sc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = j * 64 + lane;
        if (e < E) {
            const float s = sigmoid_defined(src[(size_t)t * E + e]);
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
        for (int j = 0; j < PER; ++j) dpp_step(bh, bl, khi[j], klo[j]);
        wave_max64(bh, bl);
        const int win = (int)(~bl);  // uniform
        const int owner = win & 63, jw = win >> 6;
        float sel = 0.0f;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (j == jw) {
                sel = sc[j];
                if (lane == owner) {
                    khi[j] = 0;
                    klo[j] = 0;
                }
            }
        }
        const float s_win = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel), owner));
        if (lane == k) {
            mine = s_win;
            my_id = win;
        }
    }
    float sum = 0.0f;
    for (int k = 0; k < K; ++k)
        sum = __fadd_rn(sum, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), k)));
    if (lane < K) {
        float w = renorm ? mine / sum : mine;
        w = __fmul_rn(w, scale);
        ids[(size_t)t * K + lane] = my_id;
        weights[(size_t)t * K + lane] = w;
        if (slot_of) slot_of[(size_t)t * E + my_id] = (uint8_t)lane;
    }
}

hipError_t launch_topk(int T, int E, int K, const float* logits, const float* bias, int renorm,
                       float scale, int32_t* ids, float* w, uint8_t* slot_of, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, T, E, K, logits, bias, renorm,
                       scale, ids, w, slot_of);
    return hipGetLastError();
}

}  // namespace moe
