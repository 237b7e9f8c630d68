// quant.hip -- MXFP8 quantisation of BF16 rows (the wide MoE page's module summary:
// the latent written as the experts' MXFP8 plan).  Per 32-element block: E8M0 scale
// X = floor(log2 amax) - 8 clamped to [-127, 127], E4M3 codes = RNE(v / 2^X) saturating
// at 448.  One thread per block: four 16-byte loads, two 16-byte code stores, one scale
// byte; consecutive threads cover consecutive blocks, so loads and stores are coalesced.
#include "device.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void k_quant_mxfp8(long nblocks, const uint4* __restrict__ x,
                                                     uint4* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
    wave_priority_high();
    const long b = (long)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    uint32_t q[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 v = x[b * 4 + i];
        q[4 * i] = v.x;
        q[4 * i + 1] = v.y;
        q[4 * i + 2] = v.z;
        q[4 * i + 3] = v.w;
    }
    uint32_t out[8];
    const int X = mxfp8_encode_block(q, out);
    codes[b * 2] = make_uint4(out[0], out[1], out[2], out[3]);
    codes[b * 2 + 1] = make_uint4(out[4], out[5], out[6], out[7]);
    scales[b] = (uint8_t)(X + 127);
}

hipError_t launch_quant_mxfp8(int rows, int cols, const void* x, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
    const long nb = (long)rows * (cols / 32);
    const int blocks = (int)((nb + 255) / 256);
    hipLaunchKernelGGL(k_quant_mxfp8, dim3(blocks), dim3(256), 0, s, nb, (const uint4*)x,
                       (uint4*)codes, scales);
    return hipGetLastError();
}

}  // namespace moe
