// router.hip -- sigmoid top-K routing (ep/layer page, EpMoeLayer.topk: the stock
// router's sigmoid top-16 over one group with the correction bias, renormalize and
// scale; wide page, WideRoute: an exact top-16 with renormalised weights).
//
// One workgroup of four wavefronts per token.  Each lane owns four experts (E <= 1024)
// and their 32-bit selection keys (order-preserving bits of the FP32 key s + bias).
// Rounds of a wave-wide maximum (DPP, then readlane) pick winners in descending order,
// first within each wavefront, then among the wavefronts' winners; a ballot names the
// winner's lane, equal keys going to the lower expert id, and that lane clears its key.
// Lane k keeps slot k's score; the slot-order FP32 sum, the divide and the routed scale
// follow.
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

// (branch-free: the in-range value is computed for every input and the two clamps are
// selects, so a wavefront never splits here)
__device__ __forceinline__ float sigmoid_defined(float logit) {
    const float z = -logit;
    const float den = __fadd_rn(1.0f, exp_defined(fminf(fmaxf(z, -87.0f), 88.0f)));
    const float s = 1.0f / den;  // IEEE division (correctly rounded by default on gfx950)
    return z > 88.0f ? 0.0f : (z < -87.0f ? 1.0f : s);
}

__device__ __forceinline__ uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;  // -0 and +0 compare equal
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave-wide maximum of 32-bit keys, uniform in every lane: DPP row shifts by 1, 2, 4, 8
// leave each row's maximum in its lane 15, row broadcasts 15 and 31 carry them to lane 63,
// and a readlane makes it uniform.  Lanes outside a shift's reach combine with 0, the
// identity (every live key is nonzero).
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t k) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, CTRL, RMASK, 0xf, false);
    return o > k ? o : k;
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t k) {
    k = dpp_max_u32<0x111, 0xf>(k);  // row_shr:1
    k = dpp_max_u32<0x112, 0xf>(k);  // row_shr:2
    k = dpp_max_u32<0x114, 0xf>(k);  // row_shr:4
    k = dpp_max_u32<0x118, 0xf>(k);  // row_shr:8
    k = dpp_max_u32<0x142, 0xa>(k);  // row_bcast:15 into rows 1 and 3
    k = dpp_max_u32<0x143, 0xc>(k);  // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)k, 63);
}

// The lane that wins a round: of the lanes whose candidate key equals the wave maximum,
// the only one, or -- equal FP32 keys, rare -- the one whose candidate has the lowest
// expert id (the maximum of ~e over the tied lanes; ids are unique).
__device__ __forceinline__ int winner_lane(bool hit, int cand_e) {
    const uint64_t bal = __ballot(hit);
    if (__popcll(bal) == 1) return (int)__builtin_ctzll(bal);  // (uniform)
    const uint32_t ne = hit ? ~(uint32_t)cand_e : 0u;
    const uint32_t m = wave_max_u32_dpp(ne);
    return (int)__builtin_ctzll(__ballot(hit && ne == m));
}

// this lane's four bias values (experts j*256 + wave*64 + lane, clamped to E - 1)
__device__ __forceinline__ void load_bias4(int E, const float* __restrict__ bias, float (&bi)[4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) bi[j] = bias[min(j * 256 + wave * 64 + lane, E - 1)];
}

// One 256-thread workgroup per token.  Wavefront w owns experts w*64 + lane + 256 j
// (j < 4, E <= 1024) with keys = order bits of the FP32 s + bias (0 where the lane has no
// expert).  It finds its own top-K in K rounds: each lane offers its best remaining key
// (the lowest j among equal ones), a 32-bit wave maximum names the winning key, a ballot
// its lane (ties between lanes go to the lowest expert id), and the winner drops it.  Its K
// winners (key, id, score) go to LDS; wavefront 0 then takes the 4K candidates, one a lane,
// and picks the token's top-K from them the same way.  The order is that of one top-K over
// all E keys: descending key, equal keys by ascending expert id.
// lg: token t's E logits (global memory or LDS); bi: this lane's four bias values (experts
// j*256 + wave*64 + lane, clamped to E - 1), loaded by the caller; cand_*: 64-entry LDS
// arrays.
// slot_of (optional, [T][E] bytes): slot_of[t][e] = the slot that chose expert e, for
// the list build (entries of experts a token did not choose are left as they are).
__device__ __forceinline__ void topk_token(int t, int E, int K, const float* lg,
                                           const float (&bi)[4], int renorm,
                                           float scale, int32_t* __restrict__ ids,
                                           float* __restrict__ weights,
                                           uint8_t* __restrict__ slot_of, uint32_t* cand_key,
                                           int* cand_e, float* cand_sc) {
    constexpr int PER = 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t key[PER];
    float sc[PER];
    // every logit of this lane is loaded before the first use (clamped indices, no
    // branches), so the wavefront waits for one round trip, not one per expert
    float lgv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) lgv[j] = lg[min(j * 256 + wave * 64 + lane, E - 1)];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = j * 256 + wave * 64 + lane;
        const float s = sigmoid_defined(lgv[j]);
        const bool live = e < E;
        sc[j] = live ? s : 0.0f;
        key[j] = live ? order_bits(__fadd_rn(s, bi[j])) : 0u;
    }
    // K rounds over this wavefront's keys: lane k ends with its slot-k winner
    uint32_t mine_key = 0;
    int mine_e = 0;
    float mine = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint32_t c = key[0];
        int jc = 0;
        float cs = sc[0];
#pragma unroll
        for (int j = 1; j < PER; ++j) {
            const bool better = key[j] > c;  // strict: equal keys keep the lower j
            c = better ? key[j] : c;
            jc = better ? j : jc;
            cs = better ? sc[j] : cs;
        }
        const uint32_t M = wave_max_u32_dpp(c);
        if (M == 0u) break;  // (uniform) the wavefront has no keys left
        const int ce = jc * 256 + wave * 64 + lane;
        const int wl = winner_lane(c == M, ce);
#pragma unroll
        for (int j = 0; j < PER; ++j) key[j] = (lane == wl && j == jc) ? 0u : key[j];
        const float s_win = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), wl));
        const int e_win = __builtin_amdgcn_readlane(ce, wl);
        if (lane == k) {
            mine_key = M;
            mine_e = e_win;
            mine = s_win;
        }
    }
    if (lane < 16) {
        cand_key[wave * 16 + lane] = lane < K ? mine_key : 0u;
        cand_e[wave * 16 + lane] = mine_e;
        cand_sc[wave * 16 + lane] = mine;
    }
    __syncthreads();
    if (wave != 0) return;
    // the token's top-K among the 4K candidates (one a lane)
    uint32_t ck = cand_key[lane];
    const int ce = cand_e[lane];
    const float cs = cand_sc[lane];
    int my_id = 0;
    mine = 0.0f;
    for (int k = 0; k < K; ++k) {
        const uint32_t M = wave_max_u32_dpp(ck);
        const int wl = winner_lane(ck == M, ce);
        ck = lane == wl ? 0u : ck;
        const float s_win = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs), wl));
        const int e_win = __builtin_amdgcn_readlane(ce, wl);
        if (lane == k) {
            mine = s_win;
            my_id = e_win;
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

__global__ __launch_bounds__(256) void k_topk(int T, int E, int K, const float* __restrict__ src,
                                              const float* __restrict__ bias, int renorm,
                                              float scale, int32_t* __restrict__ ids,
                                              float* __restrict__ weights,
                                              uint8_t* __restrict__ slot_of) {
    wave_priority_high();
    __shared__ uint32_t cand_key[64];
    __shared__ int cand_e[64];
    __shared__ float cand_sc[64];
    float bi[4];
    load_bias4(E, bias, bi);
    topk_token(blockIdx.x, E, K, src + (size_t)blockIdx.x * E, bi, renorm, scale, ids, weights,
               slot_of, cand_key, cand_e, cand_sc);
}

// The front GEMM's split partials [S][T][N] (router rows [0, E), latent rows [E, E + L))
// to routing and MXFP8 latent in one launch.  Workgroups [0, T): token t's E logits are
// added over the splits in split order into LDS (and the logits array), then its top-K is
// selected from LDS as k_topk does; the rest take the latent, eight columns a thread (see
// front_latent8).  Saves the logits' round trip and a launch between the two steps.
__global__ __launch_bounds__(256) void k_front_topk(int T, int N, int E, int L, int S,
                                                    const float* __restrict__ part,
                                                    float* __restrict__ logits,
                                                    const float* __restrict__ bias, int K,
                                                    int renorm, float scale,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ weights,
                                                    uint8_t* __restrict__ slot_of,
                                                    uint4* __restrict__ latent,
                                                    uint2* __restrict__ codes,
                                                    uint8_t* __restrict__ scales) {
    wave_priority_high();
    __shared__ __attribute__((aligned(16))) float lg[1024];
    __shared__ uint32_t cand_key[64];
    __shared__ int cand_e[64];
    __shared__ float cand_sc[64];
    if ((int)blockIdx.x < T) {
        const int t = blockIdx.x;
        float bi[4];
        load_bias4(E, bias, bi);  // (in flight with the partials' loads)
        for (int c = threadIdx.x * 4; c < E; c += 1024) {
            const v4f v = sum_splits(part + (size_t)t * N + c, (size_t)T * N, S);
            *(v4f*)(lg + c) = v;
            *(v4f*)(logits + (size_t)t * E + c) = v;
        }
        __syncthreads();
        topk_token(t, E, K, lg, bi, renorm, scale, ids, weights, slot_of, cand_key, cand_e,
                   cand_sc);
        return;
    }
    const long b = (long)(blockIdx.x - T) * 256 + threadIdx.x;
    if (b >= (long)T * (L / 8)) return;
    front_latent8(b, T, N, E, E + L, S, part, latent, codes, scales);
}

hipError_t launch_front_topk(int T, int N, int E, int L, int S, const float* parts, float* logits,
                             const float* bias, int K, int renorm, float scale, int32_t* ids,
                             float* w, uint8_t* slot_of, void* latent, uint8_t* codes,
                             uint8_t* scales, hipStream_t s) {
    const long lat = ((long)T * (L / 8) + 255) / 256;
    hipLaunchKernelGGL(k_front_topk, dim3((unsigned)(T + lat)), dim3(256), 0, s, T, N, E, L, S,
                       parts, logits, bias, K, renorm, scale, ids, w, slot_of, (uint4*)latent,
                       (uint2*)codes, scales);
    return hipGetLastError();
}

hipError_t launch_topk(int T, int E, int K, const float* logits, const float* bias, int renorm,
                       float scale, int32_t* ids, float* w, uint8_t* slot_of, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3(T), dim3(256), 0, s, T, E, K, logits, bias, renorm, scale, ids,
                       w, slot_of);
    return hipGetLastError();
}

}  // namespace moe
