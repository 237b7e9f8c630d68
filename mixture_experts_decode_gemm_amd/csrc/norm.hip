// norm.hip -- latent RMSNorm (ep/layer page, EpMoeLayer: ops.rms_norm(normed, routed,
// norm, eps); wide page, WideMoE.tail: the RMSNorm fused into the latent all-reduce) and
// the shared expert's gated activation (ep/layer page, EpMoeLayer.gate_up: the [T, 2S]
// gate_up rows; SiLU-and-mul stands in for the pages' undefined SiTU).
#include "device.h"
#include "kernels.h"

namespace moe {

// one workgroup of 256 threads per row; 16-byte loads; FP32 sum of squares reduced
// across the wavefront by xor shuffles and across the four wavefronts in LDS
__global__ __launch_bounds__(256) void k_rmsnorm(int cols8, const uint4* __restrict__ r,
                                                 const uint4* __restrict__ g, float eps,
                                                 uint4* __restrict__ out) {
    __shared__ float part[4];
    const int row = blockIdx.x;
    const uint4* src = r + (size_t)row * cols8;
    float ss = 0.f;
    for (int c = threadIdx.x; c < cols8; c += 256) {
        const uint4 v = src[c];
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = bf16_lo(q[i]), b = bf16_hi(q[i]);
            ss = __builtin_fmaf(a, a, ss);
            ss = __builtin_fmaf(b, b, ss);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = 1.0f / sqrtf(tot / (float)(cols8 * 8) + eps);
    for (int c = threadIdx.x; c < cols8; c += 256) {
        const uint4 v = src[c], gw = g[c];
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
        const uint32_t h[4] = {gw.x, gw.y, gw.z, gw.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = pack_bf16x2(bf16_lo(q[i]) * inv * bf16_lo(h[i]),
                               bf16_hi(q[i]) * inv * bf16_hi(h[i]));
        out[(size_t)row * cols8 + c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Finalize and RMSNorm of one token in one workgroup (the layer's own path; the two
// stand-alone kernels stay for moe_finalize and moe_rmsnorm).  Thread c owns columns
// 8c .. 8c+7: the top-K weighted sum of its row fragments (one FMA per slot in slot order,
// as in k_finalize) rounded once to BF16 is the routed latent (written out), then the
// row's FP32 sum of squares of those BF16 values (per-thread partials, xor shuffles in the
// wavefront, the wavefronts' partials added in order) gives the RMS scaling of the same
// registers.  blockDim.x = cols8 rounded up to a wavefront (<= 1024).
__global__ __launch_bounds__(1024) void k_finalize_rmsnorm(int K, int cols8,
                                                           const uint4* __restrict__ rows,
                                                           const float* __restrict__ w,
                                                           const uint4* __restrict__ g,
                                                           float eps,
                                                           uint4* __restrict__ routed,
                                                           uint4* __restrict__ normed) {
    __shared__ float part[16];
    const int t = blockIdx.x, c = threadIdx.x;
    const bool live = c < cols8;
    // Every load is unconditional, from a clamped slot and column, so the K row fragments
    // and the norm weights go out as one batch with no branch between them (a load behind
    // a branch can get a wait of its own: one more round trip).  Slots past K and lanes
    // past the row end load a valid address and their values are dropped below.
    const int cc = live ? c : cols8 - 1;
    const uint4 gw = g[cc];
    uint4 v[16];
    float wk[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int kk = k < K ? k : K - 1;
        wk[k] = w[t * K + kk];
        v[k] = rows[(size_t)(t * K + kk) * cols8 + cc];
    }
    __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first multiply-add
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // slots past K keep the sum as it was (a select, not a branch: behind a branch the
    // compiler sinks each weight's scalar load there and waits for it one slot at a time)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const bool use = k < K;
        const uint32_t q[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = __builtin_fmaf(wk[k], bf16_lo(q[i]), acc[2 * i]);
            const float b = __builtin_fmaf(wk[k], bf16_hi(q[i]), acc[2 * i + 1]);
            acc[2 * i] = use ? a : acc[2 * i];
            acc[2 * i + 1] = use ? b : acc[2 * i + 1];
        }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = bf16_lo(o[i]), b = bf16_hi(o[i]);
        ss = __builtin_fmaf(a, a, ss);
        ss = __builtin_fmaf(b, b, ss);
    }
    ss = live ? ss : 0.f;
    if (live) routed[(size_t)t * cols8 + c] = make_uint4(o[0], o[1], o[2], o[3]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((c & 63) == 0) part[c >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += part[i];
    const float inv = 1.0f / sqrtf(tot / (float)(cols8 * 8) + eps);
    if (!live) return;
    const uint32_t h[4] = {gw.x, gw.y, gw.z, gw.w};
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        n[i] = pack_bf16x2(bf16_lo(o[i]) * inv * bf16_lo(h[i]), bf16_hi(o[i]) * inv * bf16_hi(h[i]));
    normed[(size_t)t * cols8 + c] = make_uint4(n[0], n[1], n[2], n[3]);
}

bool finalize_rmsnorm_fits(int cols) { return cols % 8 == 0 && cols / 8 <= 1024; }

hipError_t launch_finalize_rmsnorm(int T, int K, int cols, const void* rows, const float* w,
                                   const void* g, float eps, void* routed, void* normed,
                                   hipStream_t s) {
    const int cols8 = cols / 8;
    const int threads = (cols8 + 63) / 64 * 64;
    hipLaunchKernelGGL(k_finalize_rmsnorm, dim3(T), dim3(threads), 0, s, K, cols8,
                       (const uint4*)rows, w, (const uint4*)g, eps, (uint4*)routed,
                       (uint4*)normed);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int rows, int cols, const void* r, const void* g, float eps, void* out,
                          hipStream_t s) {
    hipLaunchKernelGGL(k_rmsnorm, dim3(rows), dim3(256), 0, s, cols / 8, (const uint4*)r,
                       (const uint4*)g, eps, (uint4*)out);
    return hipGetLastError();
}

// out[m, j] = BF16(silu(gu[m, j]) * gu[m, S + j]); one thread per 8 columns
__global__ __launch_bounds__(256) void k_silu_mul(int M, int S8, const uint4* __restrict__ gu,
                                                  uint4* __restrict__ out) {
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (long)M * S8) return;
    const long m = gid / S8, c = gid - m * S8;
    const uint4 gv = gu[m * 2 * S8 + c], uv = gu[m * 2 * S8 + S8 + c];
    const uint32_t gq[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uq[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float g0 = bf16_lo(gq[i]), g1 = bf16_hi(gq[i]);
        o[i] = pack_bf16x2(g0 / (1.0f + __expf(-g0)) * bf16_lo(uq[i]),
                           g1 / (1.0f + __expf(-g1)) * bf16_hi(uq[i]));
    }
    out[gid] = make_uint4(o[0], o[1], o[2], o[3]);
}

// The same from the gate/up GEMM's nsplit FP32 split-K partials: slab z holds M rows of
// stride ld floats, gate values in columns [0, S), up values in [S, 2S).  Each gate and up
// value is the split-order sum rounded once to BF16 (the GEMM's output), then as above.
__global__ __launch_bounds__(256) void k_silu_mul_parts(int M, int S8, int nsplit, int ld4,
                                                        const float4* __restrict__ parts,
                                                        uint4* __restrict__ out) {
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (long)M * S8) return;
    const long m = gid / S8, c = gid - m * S8;
    const long zs = (long)M * ld4;                  // float4s per split
    const float4* gp = parts + m * ld4 + c * 2;     // 8 gate floats of this thread
    const float4* up = gp + S8 * 2;                 // 8 up floats
    float gv[8], uv[8];
    // the loads of up to four splits go out together (one round trip, not one a split)
    constexpr int MAXS = 4;
    float4 ga[MAXS][2], ua[MAXS][2];
#pragma unroll
    for (int z = 0; z < MAXS; ++z)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ga[z][h] = z < nsplit ? gp[z * zs + h] : make_float4(0.f, 0.f, 0.f, 0.f);
            ua[z][h] = z < nsplit ? up[z * zs + h] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float4 a = ga[0][h], b = ua[0][h];
#pragma unroll
        for (int z = 1; z < MAXS; ++z) {
            if (z >= nsplit) break;
            const float4 a2 = ga[z][h], b2 = ua[z][h];
            a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
            b.x += b2.x; b.y += b2.y; b.z += b2.z; b.w += b2.w;
        }
        for (int z = MAXS; z < nsplit; ++z) {
            const float4 a2 = gp[z * zs + h], b2 = up[z * zs + h];
            a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
            b.x += b2.x; b.y += b2.y; b.z += b2.z; b.w += b2.w;
        }
        gv[4 * h] = a.x; gv[4 * h + 1] = a.y; gv[4 * h + 2] = a.z; gv[4 * h + 3] = a.w;
        uv[4 * h] = b.x; uv[4 * h + 1] = b.y; uv[4 * h + 2] = b.z; uv[4 * h + 3] = b.w;
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t gq = pack_bf16x2(gv[2 * i], gv[2 * i + 1]);
        const uint32_t uq = pack_bf16x2(uv[2 * i], uv[2 * i + 1]);
        const float g0 = bf16_lo(gq), g1 = bf16_hi(gq);
        o[i] = pack_bf16x2(g0 / (1.0f + __expf(-g0)) * bf16_lo(uq),
                           g1 / (1.0f + __expf(-g1)) * bf16_hi(uq));
    }
    out[gid] = make_uint4(o[0], o[1], o[2], o[3]);
}

hipError_t launch_silu_mul_parts(int M, int S, int nsplit, const float* parts, int ld, void* out,
                                 hipStream_t s) {
    const long n = (long)M * (S / 8);
    hipLaunchKernelGGL(k_silu_mul_parts, dim3((int)((n + 255) / 256)), dim3(256), 0, s, M, S / 8,
                       nsplit, ld / 4, (const float4*)parts, (uint4*)out);
    return hipGetLastError();
}

hipError_t launch_silu_mul(int M, int S, const void* gu, void* out, hipStream_t s) {
    const long n = (long)M * (S / 8);
    hipLaunchKernelGGL(k_silu_mul, dim3((int)((n + 255) / 256)), dim3(256), 0, s, M, S / 8,
                       (const uint4*)gu, (uint4*)out);
    return hipGetLastError();
}

}  // namespace moe
