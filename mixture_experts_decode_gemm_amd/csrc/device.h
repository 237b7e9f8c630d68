// device.h -- small device helpers shared by the libmoedecode kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

// ---- BF16 -------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round-to-nearest-even FP32 -> BF16 bits (NaN -> quiet NaN; overflow -> inf)
__device__ __forceinline__ uint32_t f_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f_to_bf16(lo) | (f_to_bf16(hi) << 16);
}

// ---- MXFP8 (OCP MX: E4M3 elements, E8M0 block scale) --------------------------------
// floor(log2 |v|) of a nonzero finite FP32 magnitude given as bits (subnormals included)
__device__ __forceinline__ int ilog2_f32_bits(uint32_t mag) {
    int e = (int)(mag >> 23);
    if (e) return e - 127;
    return (31 - __clz((int)mag)) - 149;
}

// block exponent X = floor(log2 amax) - 8 (8 = largest E4M3 exponent), clamped to the
// E8M0 range; the all-zero block returns the smallest scale (byte 0)
__device__ __forceinline__ int mx_block_exponent(uint32_t amax_f32_bits) {
    if (amax_f32_bits == 0) return -127;
    int x = ilog2_f32_bits(amax_f32_bits) - 8;
    return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// E4M3 code of v (already divided by the block scale): round to nearest even,
// saturating to +-448, the sign of zero kept.  v is finite.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t mag = u & 0x7FFFFFFFu;
    float a = __uint_as_float(mag);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (mag < 0x3C800000u) {  // a < 2^-6: subnormal grid of step 2^-9
        code = (uint32_t)rintf(a * 512.0f);  // 0..8 (8 = the smallest normal, 0x08)
    } else {
        uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);  // keep 3 mantissa bits, RNE
        int e = (int)(r >> 23) - 127;
        code = ((uint32_t)(e + 7) << 3) | ((r >> 20) & 7u);
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return sign | code;
}

// One MXFP8 block of 32 BF16 values given as 16 words of BF16 pairs (element 2i in the low
// half of word i): the E8M0 exponent X (returned) from the block's largest magnitude and
// the 32 E4M3 codes of v / 2^X, four to a word in element order.
__device__ __forceinline__ int mxfp8_encode_block(const uint32_t (&q)[16], uint32_t (&out)[8]) {
    uint32_t amax = 0;  // magnitude bits order like magnitudes for finite BF16
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t lo = q[i] & 0x7FFFu, hi = (q[i] >> 16) & 0x7FFFu;
        amax = amax > lo ? amax : lo;
        amax = amax > hi ? amax : hi;
    }
    const int X = mx_block_exponent(amax << 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t c0 = e4m3_rne_sat(ldexpf(bf16_lo(q[2 * i]), -X));
        const uint32_t c1 = e4m3_rne_sat(ldexpf(bf16_hi(q[2 * i]), -X));
        const uint32_t c2 = e4m3_rne_sat(ldexpf(bf16_lo(q[2 * i + 1]), -X));
        const uint32_t c3 = e4m3_rne_sat(ldexpf(bf16_hi(q[2 * i + 1]), -X));
        out[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    return X;
}

// Four columns of the S split partials (split stride zs floats) added in split order.  The
// loads of up to eight splits are issued together, so the thread waits for one round
// trip, not one per split.
__device__ __forceinline__ v4f sum_splits(const float* __restrict__ p, size_t zs, int S) {
    constexpr int MAXS = 8;
    v4f q[MAXS];
#pragma unroll
    for (int zz = 0; zz < MAXS; ++zz)
        q[zz] = zz < S ? *(const v4f*)(p + zz * zs) : (v4f){0.f, 0.f, 0.f, 0.f};
    v4f v = q[0];
#pragma unroll
    for (int zz = 1; zz < MAXS; ++zz)
        if (zz < S) v += q[zz];
    for (int zz = MAXS; zz < S; ++zz) v += *(const v4f*)(p + zz * zs);
    return v;
}

// One thread's share of the front GEMM's latent columns: eight consecutive columns b of
// the M x (N1 - N0) latent (four threads per 32-column MXFP8 block) summed over the S split
// partials in split order, rounded once to BF16 (latent), and the block's E4M3 codes and
// E8M0 scale (the lanes of one block exchange their maxima; the first writes the scale).
__device__ __forceinline__ void front_latent8(long b, int M, int N, int N0, int N1, int S,
                                              const float* __restrict__ part,
                                              uint4* __restrict__ latent,
                                              uint2* __restrict__ codes,
                                              uint8_t* __restrict__ scales) {
    const int c8s = (N1 - N0) / 8;
    const size_t zs = (size_t)M * N;
    const int m = (int)(b / c8s), c8 = (int)(b - (long)m * c8s);
    const float* p = part + (size_t)m * N + N0 + c8 * 8;
    const v4f v0 = sum_splits(p, zs, S), v1 = sum_splits(p + 4, zs, S);
    const uint32_t q[4] = {pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                           pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
    latent[b] = make_uint4(q[0], q[1], q[2], q[3]);
    uint32_t amax = 0;  // magnitude bits order like magnitudes for finite BF16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = q[i] & 0x7FFFu, hi = (q[i] >> 16) & 0x7FFFu;
        amax = amax > lo ? amax : lo;
        amax = amax > hi ? amax : hi;
    }
#pragma unroll
    for (int off = 1; off < 4; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)amax, off, 64);
        amax = amax > o ? amax : o;
    }
    const int X = mx_block_exponent(amax << 16);
    uint32_t out[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t c0 = e4m3_rne_sat(ldexpf(bf16_lo(q[2 * i]), -X));
        const uint32_t c1 = e4m3_rne_sat(ldexpf(bf16_hi(q[2 * i]), -X));
        const uint32_t c2 = e4m3_rne_sat(ldexpf(bf16_lo(q[2 * i + 1]), -X));
        const uint32_t c3 = e4m3_rne_sat(ldexpf(bf16_hi(q[2 * i + 1]), -X));
        out[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    codes[b] = make_uint2(out[0], out[1]);
    if ((b & 3) == 0) scales[b >> 2] = (uint8_t)(X + 127);
}

// ---- workgroup barrier over LDS only ----------------------------------------------------
// __syncthreads() fences global memory too, which makes every wavefront wait for all of
// its outstanding global loads (s_waitcnt vmcnt(0)) -- fatal to a software pipeline that
// keeps the next tile's loads in flight across the barrier.  This barrier orders LDS only.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for code that also has direct global-to-LDS loads in flight: waits
// for this wavefront's own LDS reads and writes (lgkmcnt) and nothing else.  A release
// fence (lds_barrier) would make the compiler wait for every outstanding direct load
// (they write LDS), draining a prefetch; here completion of direct loads is the caller's
// business (wait_vmcnt before the barrier).  The asm statement is also a compiler-level
// memory barrier, so no memory access moves across it.
__device__ __forceinline__ void lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14; expcnt and lgkmcnt left at their maxima).  Direct global-to-LDS loads are not
// tracked by the compiler's own waits: code that reads what they wrote waits with this,
// then crosses an LDS barrier.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// One 16-byte-per-lane direct load into LDS (the wavefront's 64 pieces land at dst +
// 16 lane) from a raw buffer over [base, base + bytes); reads past the end return zeros.
__device__ __forceinline__ void dma16(const void* base, int bytes, uint32_t off, lds_ptr dst) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}

// 16-byte load marked non-temporal (the nt bit: the lines are streamed through the caches
// with the lowest retention).  For weights that are read once per step: without it they
// evict the small, re-read activations from L2 and those go back to HBM.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    const u32x4_nt v = __builtin_nontemporal_load((const u32x4_nt*)p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Raise this wavefront's issue priority (s_setprio 3).  The routing kernels are short and
// latency-bound and run while the shared expert's GEMMs occupy every CU from another
// stream; priority lets their waves issue first on a shared SIMD.  Stream priorities are
// not involved.
__device__ __forceinline__ void wave_priority_high() { __builtin_amdgcn_s_setprio(3); }

// ---- wave helpers ---------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, WAVE);
        v = v > o ? v : o;
    }
    return v;
}

}  // namespace moe
