// finalize.hip -- top-K weighted Finalize (wide MoE page, class Finalize):
// out[t] = BF16_RNE(sum_k w[t,k] * rows[K t + k]) with one FP32 fused multiply-add per
// slot in slot order.  Invalid slots (finalize_publish page, the -1 row rule) are skipped.
//
// MI355X layout: one thread per 8 consecutive columns of one token (16-byte loads and
// stores); all K row fragments of a thread are loaded before the first FMA, so each
// lane keeps K 16-byte loads in flight (the Finalize section issues all of its loads
// before the first multiply-add).
// Threads are numbered token-major so a wavefront streams 64 x 16 B = 1 KiB of one row.
#include "device.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void k_finalize(int T, int K, int cols8,
                                                  const uint4* __restrict__ rows,
                                                  const float* __restrict__ w,
                                                  const int32_t* __restrict__ ids,
                                                  uint4* __restrict__ out) {
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int t = gid / cols8;
    const int c = gid - t * cols8;
    if (t >= T) return;
    uint4 v[16];
    float wk[16];
    bool ok[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        ok[k] = k < K;
        if (ok[k] && ids) ok[k] = ids[t * K + k] >= 0;
        wk[k] = ok[k] ? w[t * K + k] : 0.0f;
        if (ok[k]) v[k] = rows[(size_t)(t * K + k) * cols8 + c];
        else v[k] = make_uint4(0, 0, 0, 0);
    }
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

hipError_t launch_finalize(int T, int K, int cols, const void* rows, const float* w,
                           const int32_t* ids, void* out, hipStream_t s) {
    const int cols8 = cols / 8;
    const long threads = (long)T * cols8;
    const int blocks = (int)((threads + 255) / 256);
    hipLaunchKernelGGL(k_finalize, dim3(blocks), dim3(256), 0, s, T, K, cols8,
                       (const uint4*)rows, w, ids, (uint4*)out);
    return hipGetLastError();
}

}  // namespace moe
