// finalize.hip -- top-K weighted Finalize (wide MoE page, class Finalize):
// out[t] = BF16_RNE(sum_k w[t,k] * rows[K t + k]) with one FP32 fused multiply-add per
// slot in slot order.  Invalid slots (finalize_publish page, the -1 row rule) are skipped.
//
// MI355X layout: one workgroup per token (blockDim = cols/8 rounded up to a wavefront, at
// most 1024; wider rows loop), one thread per 8 consecutive columns (16-byte loads and
// stores).  The token's K weights (and ids) are fetched first as 16-byte loads of the same
// addresses in every thread (one cache line, broadcast); then all of a thread's K row
// fragments are loaded before the first FMA, so each lane keeps K 16-byte loads in flight
// (the Finalize section issues all of its loads before the first multiply-add).
#include "device.h"
#include "kernels.h"

namespace moe {

// the K (<= 16) weights and ids of token t; ids may be null (every slot valid)
__device__ __forceinline__ void load_slots(int t, int K, const float* __restrict__ w,
                                           const int32_t* __restrict__ ids, float (&wk)[16],
                                           bool (&ok)[16]) {
    int32_t id[16];
    if (K == 16) {  // 64-byte rows, 16-byte aligned (the ABI aligns w and ids)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 q = ((const float4*)(w + (size_t)t * 16))[i];
            wk[4 * i] = q.x, wk[4 * i + 1] = q.y, wk[4 * i + 2] = q.z, wk[4 * i + 3] = q.w;
            const int4 d = ids ? ((const int4*)(ids + (size_t)t * 16))[i] : make_int4(0, 0, 0, 0);
            id[4 * i] = d.x, id[4 * i + 1] = d.y, id[4 * i + 2] = d.z, id[4 * i + 3] = d.w;
        }
    } else {  // unconditional loads of a clamped slot, batched; slots past K dropped below
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const size_t i = (size_t)t * K + (k < K ? k : K - 1);
            wk[k] = w[i];
            id[k] = ids ? ids[i] : 0;
        }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) ok[k] = k < K && id[k] >= 0;
}

__global__ __launch_bounds__(1024) void k_finalize(int K, int cols8, const uint4* __restrict__ rows,
                                                   const float* __restrict__ w,
                                                   const int32_t* __restrict__ ids,
                                                   uint4* __restrict__ out) {
    const int t = blockIdx.x;
    float wk[16];
    bool ok[16];
    load_slots(t, K, w, ids, wk, ok);
    // An invalid slot loads the first valid slot's row instead (and drops it), so every
    // row load is unconditional and the K of them go out as one batch, while the row of
    // an invalid slot is still never read.  A token with no valid slot reads no row.
    int first = -1;
#pragma unroll
    for (int k = 15; k >= 0; --k) first = ok[k] ? k : first;
    if (first < 0) {
        for (int c = threadIdx.x; c < cols8; c += blockDim.x)
            out[(size_t)t * cols8 + c] = make_uint4(0, 0, 0, 0);
        return;
    }
    int src[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) src[k] = ok[k] ? k : first;
    for (int c = threadIdx.x; c < cols8; c += blockDim.x) {
        uint4 v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = rows[((size_t)t * K + src[k]) * cols8 + c];
        __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first multiply-add
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (!ok[k]) continue;
            const uint32_t q[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = __builtin_fmaf(wk[k], bf16_lo(q[i]), acc[2 * i]);
                acc[2 * i + 1] = __builtin_fmaf(wk[k], bf16_hi(q[i]), acc[2 * i + 1]);
            }
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        out[(size_t)t * cols8 + c] = o;
    }
}

hipError_t launch_finalize(int T, int K, int cols, const void* rows, const float* w,
                           const int32_t* ids, void* out, hipStream_t s) {
    const int cols8 = cols / 8;
    const int threads = cols8 >= 1024 ? 1024 : (cols8 + 63) / 64 * 64;
    hipLaunchKernelGGL(k_finalize, dim3(T), dim3(threads), 0, s, K, cols8, (const uint4*)rows, w,
                       ids, (uint4*)out);
    return hipGetLastError();
}

}  // namespace moe
