// kernels.h -- host-side launchers of the libmoedecode kernels (internal; the public
// ABI is include/moedecode.h).  Every launcher only enqueues work on `stream` and
// returns hipGetLastError().  Arguments are validated by the callers in abi.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_finalize(int T, int K, int cols, const void* rows, const float* w,
                           const int32_t* ids, void* out, hipStream_t s);

hipError_t launch_quant_mxfp8(int rows, int cols, const void* x, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);

// slot_of (optional, [T][E] bytes): the slot that chose each chosen expert, for the lists
hipError_t launch_topk(int T, int E, int K, const float* logits, const float* bias, int renorm,
                       float scale, int32_t* ids, float* w, uint8_t* slot_of, hipStream_t s);

// the front GEMM's split partials [S][T][N] (router rows [0, E), latent rows [E, E + L)):
// FP32 logits, sigmoid top-K as launch_topk, and the latent rounded once to BF16 with its
// MXFP8 codes and scales (E % 4 == 0, E <= 1024, L % 32 == 0)
hipError_t launch_front_topk(int T, int N, int E, int L, int S, const float* parts, float* logits,
                             const float* bias, int K, int renorm, float scale, int32_t* ids,
                             float* w, uint8_t* slot_of, void* latent, uint8_t* codes,
                             uint8_t* scales, hipStream_t s);

// routing lists: scratch of lists_scratch_bytes(T, E) bytes, which ends with the slot map
// (lists_slot_map) that launch_topk fills; slot_of null: the mark launch fills it
size_t lists_scratch_bytes(int T, int E);
uint8_t* lists_slot_map(void* scratch, int T, int E);
// whether launch_lists builds the lists in one workgroup (no slot map needed then)
bool lists_fused_fits(int T, int E);
hipError_t launch_lists(int T, int K, int E, int unit, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* pairs, int32_t* units, int32_t* num_units,
                        void* scratch, const uint8_t* slot_of, hipStream_t s);

// grouped FFN: MXFP4 x MXFP8; the MXFP8 hidden goes to hid [T*K, I] and hid_scales
// [T*K, I/32] (by pair id); ffn_scratch_bytes(P, I) covers both, 256-aligned.
// stages: bit 0 the gate/up pass, bit 1 the down pass
size_t ffn_scratch_bytes(int P, int I);
hipError_t launch_ffn_mx(int T, int K, int E, int L, int I, int unit, const uint8_t* w13,
                         const uint8_t* s13, const uint8_t* w2, const uint8_t* s2,
                         const uint8_t* codes, const uint8_t* scales, const int32_t* pairs,
                         const int32_t* units, const int32_t* num_units, void* rows,
                         uint8_t* hid, uint8_t* hid_scales, int stages, bool packed,
                         unsigned* counters, bool counters_zeroed, hipStream_t s);
// The passes end with a dynamic tail of work tickets.  counters: the two passes' work
// counters (16 words); counters_zeroed: the caller's stream zeroed them since their last
// use (else the launcher zeroes them first with a small kernel).  In moe_grouped_ffn's
// workspace they sit at ffn_counter_offset.
size_t ffn_counter_offset(int P, int I);
// From kUpTwoAreaTokens tokens the gate/up pass keeps two activation areas a wavefront
// (an expert's second token group loaded ahead with its first); below, one (less LDS, so
// that its workgroups share CUs with the side stream's GEMMs)
constexpr int kUpTwoAreaTokens = 128;
// the packed expert layout (see ffn.hip); L % 512 == 0, I / 128 in {1, 2, 4}
hipError_t launch_pack_experts(int E, int L, int I, const uint8_t* w13, const uint8_t* s13,
                               const uint8_t* w2, const uint8_t* s2, uint8_t* pw13, uint8_t* ps13,
                               uint8_t* pw2, uint8_t* ps2, hipStream_t s);
hipError_t launch_ffn_bf16(int T, int K, int E, int L, int I, int unit, const void* w13,
                           const void* w2, const void* latent, const int32_t* pairs,
                           const int32_t* units, const int32_t* num_units, void* rows,
                           hipStream_t s);

// dense BF16 GEMM out = x W^T (mode 0 FP32 out, 1 BF16 out, 2 BF16 out with BF16 add);
// max_wg > 0 caps the grid (a persistent grid looping over the tiles); prio raises the
// waves' issue priority (for the routed path while the shared expert runs beside it)
size_t gemm_scratch_bytes(int M, int N, int K);
hipError_t launch_gemm(int M, int N, int K, const void* x, const void* w, void* out,
                       const void* add, int mode, void* scratch, hipStream_t s, int max_wg = 0,
                       bool prio = false);
int gemm_device_cus();
// the GEMM's FP32 split-K partials [S][M][N] only (S >= 1 returned), for a consumer that
// adds them in split order itself; gemm_parts_bytes(M, N, K) covers every token count <= M
int gemm_splits(int M, int N, int K);
size_t gemm_parts_bytes(int M, int N, int K);
hipError_t launch_gemm_parts(int M, int N, int K, const void* x, const void* w, float* parts,
                             hipStream_t s, bool prio, int* S);
// SiLU-and-mul of the gate/up GEMM's split partials: gate columns [0, S) and up columns
// [S, 2S) of rows with stride ld floats, nsplit slabs of M rows
hipError_t launch_silu_mul_parts(int M, int S, int nsplit, const float* parts, int ld, void* out,
                                 hipStream_t s);

// weight-streaming dense GEMM (wgemm.hip): FP32 split partials [S][M][N] of x W^T where W
// is three row segments stacked: rows [0, N0) from w0, [N0, N1) from w1, [N1, N) from w2
// (row-major, or packed by launch_pack_dense; empty segments may pass null); *S receives
// the split count.  wgemm_fits tells whether the shape is supported (K % 128 == 0, every
// segment a multiple of 32 rows, of 64 when packed, M * K < 2^31).  zero (optional): 16
// words the launch sets to 0, for the counters of a later launch on the same stream.
// out_bf16 (optional, N0 = N1 = N): one split, the result rounded once to BF16 and written
// to out_bf16 [M, N] directly (no partials, no reduce; parts unused).
bool wgemm_fits(int M, int N, int N0, int N1, int K, bool packed);
// share: the fraction of the GPU the split plan assumes (1 when the GEMM runs alone);
// parts_once: the plan counts the partials' bytes once, not written and read back (for a
// GEMM on an otherwise idle GPU whose reduce follows at once)
int wgemm_splits(int M, int N, int K, double share = 1.0, bool parts_once = false);
size_t wgemm_parts_bytes(int M, int N, int K, double share = 1.0, bool parts_once = false);
hipError_t launch_wgemm(int M, int N, int N0, int N1, int K, const void* x, const void* w0,
                        const void* w1, const void* w2, bool packed, float* parts, hipStream_t s,
                        bool prio, int* S, double share = 1.0, unsigned* zero = nullptr,
                        bool parts_once = false, void* out_bf16 = nullptr);
// adds the S partials (rows of stride N) in split order: columns [0, N0) to out0 (FP32),
// [N0, N1) to out1 with mode1 0 FP32, 1 BF16, 2 BF16 of add1 + sum; columns past N1 untouched
hipError_t launch_wg_reduce(int M, int N, int N0, int N1, int S, const float* parts, float* out0,
                            int mode1, void* out1, const void* add1, hipStream_t s, bool prio);
// W [N, K] BF16 -> the packed layout (N % 64 == 0, K % 64 == 0)
hipError_t launch_pack_dense(int N, int K, const void* w, void* out, hipStream_t s);

hipError_t launch_rmsnorm(int rows, int cols, const void* r, const void* g, float eps, void* out,
                          hipStream_t s);
// Finalize (no invalid slots) and RMSNorm of each token in one workgroup: routed and normed
// [T, cols] BF16; cols % 8 == 0 and cols / 8 <= 1024 (finalize_rmsnorm_fits)
bool finalize_rmsnorm_fits(int cols);
hipError_t launch_finalize_rmsnorm(int T, int K, int cols, const void* rows, const float* w,
                                   const void* g, float eps, void* routed, void* normed,
                                   hipStream_t s);
hipError_t launch_silu_mul(int M, int S, const void* gu, void* out, hipStream_t s);

}  // namespace moe
