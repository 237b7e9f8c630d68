// lists.hip -- per-expert routing lists and unit windows (wide page, WideRoute: each
// (token, slot) pair appended to its expert's list as token*K + slot; module summary:
// unit windows of 8 tokens per touched expert).
//
// The pages claim list slots with relaxed atomic counters, so a list's order depends on
// timing.  Here the build is deterministic, in three small launches:
//   mark  -- one workgroup per 32-token column w: bm[w][e] = bitmask of the column's
//            tokens that chose expert e (LDS bit-ORs, whose result is order-free; an id
//            outside [0,E) sets nothing, a repeated id sets the same bit once);
//   scan  -- one workgroup, one thread per expert: counts, per-word running offsets,
//            exclusive prefix sums over experts (offsets, window indices), the units
//            (the first window of every touched expert first, then the later windows);
//   fill  -- one thread per (word, expert): the set bits in ascending token order give
//            the list entries; the slot k comes from the slot map, recorded by the top-K
//            (the layer's path) or by the mark launch (the first slot of the token
//            holding e).
// Lists therefore hold ascending pair ids.  Batches whose bitmaps fit in LDS take one
// launch instead (k_lists_fused).
#include "device.h"
#include "kernels.h"

namespace moe {

// scratch: bitmaps [W][E] and word offsets [W][E] (u32), then the slot map [T][E] (u8)
size_t lists_scratch_bytes(int T, int E) {
    const size_t W = (size_t)(T + 31) / 32;
    return 2 * W * (size_t)E * sizeof(uint32_t) + ((size_t)T * E + 255) / 256 * 256;
}

uint8_t* lists_slot_map(void* scratch, int T, int E) {
    const size_t W = (size_t)(T + 31) / 32;
    return (uint8_t*)scratch + 2 * W * (size_t)E * sizeof(uint32_t);
}

// slot_map (optional): also records the slot map the fill reads -- one thread per token,
// slots written last to first, so that an expert a token names twice keeps its first slot
// (the list holds one pair per token and expert)
__global__ __launch_bounds__(256) void k_lists_mark(int T, int K, int E,
                                                    const int32_t* __restrict__ ids,
                                                    uint32_t* __restrict__ bm,
                                                    uint8_t* __restrict__ slot_map) {
    wave_priority_high();
    __shared__ uint32_t words[1024];
    const int w = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 256) words[e] = 0;
    __syncthreads();
    const int t0 = w * 32;
    const int n = min(32, T - t0) * K;
    for (int q = threadIdx.x; q < n; q += 256) {
        const int e = ids[(size_t)t0 * K + q];
        if (e >= 0 && e < E) atomicOr(&words[e], 1u << (q / K));
    }
    if (slot_map && (int)threadIdx.x < min(32, T - t0)) {
        const int t = t0 + threadIdx.x;
        int32_t v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = ids[(size_t)t * K + min(k, K - 1)];  // (together)
#pragma unroll
        for (int k = 15; k >= 0; --k)
            if (k < K && v[k] >= 0 && v[k] < E) slot_map[(size_t)t * E + v[k]] = (uint8_t)k;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) bm[(size_t)w * E + e] = words[e];
}

__device__ int3 block_exclusive_scan3_1024(int3 v, int3* smem, int3* total);

// popcounts of expert e's bitmap words w0 .. w0 + 15 (0 past W), their loads issued together
// (unconditionally, past W from the last word: a load under a branch would be waited for
// on its own)
__device__ __forceinline__ void word_popcounts(const uint32_t* __restrict__ bm, int W, int E,
                                               int e, int w0, int (&pc)[16]) {
    uint32_t b[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = bm[(size_t)min(w0 + i, W - 1) * E + e];
#pragma unroll
    for (int i = 0; i < 16; ++i) pc[i] = w0 + i < W ? __popc(b[i]) : 0;
}

// One thread per expert: its count (the words' popcounts, sixteen loads in flight; the
// first 32 kept in registers), one three-value block scan (list offsets, first windows,
// later windows), then each word's list position (words past 32 loaded again, from L2 by
// then) and the units.
__global__ __launch_bounds__(1024) void k_lists_scan(int T, int K, int E, int unit,
                                                     const uint32_t* __restrict__ bm,
                                                     int32_t* __restrict__ wordoff,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets,
                                                     int4* __restrict__ units,
                                                     int32_t* __restrict__ num_units) {
    wave_priority_high();
    __shared__ int3 smem[17];
    const int W = (T + 31) / 32;
    const int e = threadIdx.x;
    int c = 0;
    int pa[16] = {}, pb[16] = {};  // the first 32 words' popcounts, kept for the offsets
    if (e < E) {
        word_popcounts(bm, W, E, e, 0, pa);
        word_popcounts(bm, W, E, e, 16, pb);
#pragma unroll
        for (int i = 0; i < 16; ++i) c += pa[i] + pb[i];
        for (int w0 = 32; w0 < W; w0 += 16) {
            int pc[16];
            word_popcounts(bm, W, E, e, w0, pc);
#pragma unroll
            for (int i = 0; i < 16; ++i) c += pc[i];
        }
    }
    const int nu = (c + unit - 1) / unit;
    // the first window of every touched expert, then every later window
    int3 tot;
    const int3 ex = block_exclusive_scan3_1024(make_int3(c, c > 0 ? 1 : 0, nu > 1 ? nu - 1 : 0),
                                               smem, &tot);
    const int off = ex.x, fi = ex.y, li = ex.z;
    const int total_pairs = tot.x, touched = tot.y, later_total = tot.z;
    if (e < E) {
        int run = off;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            if (i < W) wordoff[(size_t)i * E + e] = run;
            run += i < 16 ? pa[i] : pb[i - 16];
        }
        for (int w0 = 32; w0 < W; w0 += 16) {
            int pc[16];
            word_popcounts(bm, W, E, e, w0, pc);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (w0 + i < W) wordoff[(size_t)(w0 + i) * E + e] = run;
                run += pc[i];
            }
        }
        counts[e] = c;
        offsets[e] = off;
        if (c > 0) units[fi] = make_int4(e, off, c < unit ? c : unit, c);
        for (int j = 1; j < nu; ++j) {
            const int rest = c - j * unit;
            units[touched + li + j - 1] = make_int4(e, off + j * unit, rest < unit ? rest : unit, 0);
        }
    }
    if (threadIdx.x == 0) {
        offsets[E] = total_pairs;
        num_units[0] = touched + later_total;
        num_units[1] = T * K - total_pairs;
        num_units[2] = touched;
        num_units[3] = 0;
    }
}

__global__ __launch_bounds__(256) void k_lists_fill(int T, int K, int E,
                                                    const uint32_t* __restrict__ bm,
                                                    const int32_t* __restrict__ wordoff,
                                                    const uint8_t* __restrict__ slot_of,
                                                    int32_t* __restrict__ pairs) {
    wave_priority_high();
    const int W = (T + 31) / 32;
    const int gid = blockIdx.x * 256 + threadIdx.x;
    if (gid >= W * E) return;
    const int w = gid / E, e = gid - w * E;
    uint32_t word = bm[gid];
    int pos = wordoff[gid];
    while (word) {
        const int j = __ffs((int)word) - 1;
        word &= word - 1;
        const int t = w * 32 + j;
        pairs[pos++] = t * K + slot_of[(size_t)t * E + e];  // the slot that chose (t, e)
    }
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP moves (no LDS round
// trips): shifts by 1, 2, 4 and 8 lanes within each 16-lane row (lanes shifted in from
// outside the row read 0), then the last lane of row 0 added into row 1 and of row 2 into
// row 3 (row broadcast 15), then the last lane of row 1 into rows 2 and 3 (row broadcast
// 31).  Lanes a masked row does not write read the old value, 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
    return x;
}

// Exclusive prefix sums of three values at once over a 1024-thread block (one pass: wave
// scans by DPP moves, the 16 wave totals scanned by one wavefront); totals returned.
__device__ int3 block_exclusive_scan3_1024(int3 v, int3* smem, int3* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int3 x = make_int3(wave_incl_scan(v.x), wave_incl_scan(v.y), wave_incl_scan(v.z));
    if (lane == 63) smem[wave] = x;
    __syncthreads();
    if (wave == 0) {
        const int3 w = lane < 16 ? smem[lane] : make_int3(0, 0, 0);
        const int3 y = make_int3(wave_incl_scan(w.x), wave_incl_scan(w.y), wave_incl_scan(w.z));
        if (lane < 16) smem[lane] = make_int3(y.x - w.x, y.y - w.y, y.z - w.z);
        if (lane == 15) smem[16] = y;
    }
    __syncthreads();
    const int3 base = smem[wave];
    *total = smem[16];
    return make_int3(base.x + x.x - v.x, base.y + x.y - v.y, base.z + x.z - v.z);
}

// the K ids of token t (-1 past K), loaded together
__device__ __forceinline__ void load_token_ids(const int32_t* __restrict__ ids, int t, int K,
                                               int32_t v[16]) {
    const int32_t* row = ids + (size_t)t * K;
    if (K == 16) {  // 64-byte rows: four 16-byte loads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int4 q = ((const int4*)row)[i];
            v[4 * i] = q.x;
            v[4 * i + 1] = q.y;
            v[4 * i + 2] = q.z;
            v[4 * i + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = row[min(k, K - 1)];  // (unconditional loads)
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = k < K ? v[k] : -1;
    }
}

// The whole build in one workgroup when the bitmaps fit in LDS (decode batches up to a
// few hundred tokens): the three steps above with the bitmaps and list offsets in LDS and
// block barriers between them, and a scatter fill -- a token's pair (t, k) goes to
// offsets[e] + (the tokens before t that chose e: set bits of e's bitmap below t).  A slot
// repeating an earlier slot's id is dropped, as in the marking.  Four threads share a
// token, each taking four of its slots.
// LDS of the one-workgroup build: bitmaps [W][E] u32, list offsets [E] u32, and -- when
// the whole stays within kListsLds -- the per-word list positions [W][E] u16
constexpr size_t kListsLds = 61440;
__host__ __device__ inline size_t lists_base_lds(int T, int E) {
    return ((size_t)(T + 31) / 32 * E + E) * sizeof(uint32_t);
}
__host__ __device__ inline bool lists_prefix_fits(int T, int E) {
    return lists_base_lds(T, E) + (size_t)(T + 31) / 32 * E * sizeof(uint16_t) <= kListsLds;
}
static size_t lists_fused_lds(int T, int E) {
    return lists_base_lds(T, E) +
           (lists_prefix_fits(T, E) ? (size_t)(T + 31) / 32 * E * sizeof(uint16_t) : 0);
}

__global__ __launch_bounds__(1024) void k_lists_fused(int T, int K, int E, int unit,
                                                      const int32_t* __restrict__ ids,
                                                      int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets,
                                                      int4* __restrict__ units,
                                                      int32_t* __restrict__ num_units,
                                                      int32_t* __restrict__ pairs) {
    wave_priority_high();
    extern __shared__ uint32_t lds_lists[];
    __shared__ int3 smem[17];
    const int W = (T + 31) / 32;
    uint32_t* bm = lds_lists;                // [W][E]
    int* offl = (int*)(lds_lists + W * E);   // [E]
    // with room for it, the list position of each (word, expert) before its own bits:
    // pre[w][e] = offsets[e] + the set bits of e's words below w (< 2^16: T*K <= 65536)
    uint16_t* pre = (uint16_t*)(offl + E);   // [W][E]
    const bool use_pre = lists_prefix_fits(T, E);
    // four threads a token (tokens t0, t0 + 256, ...), thread q of a token taking its slots
    // 4 q .. 4 q + 3; the ids of the first token stay in registers from the marking to the
    // fill
    const int q = threadIdx.x & 3, t0 = threadIdx.x >> 2;
    int32_t v0[16];
    if (t0 < T) load_token_ids(ids, t0, K, v0);
    for (int i = threadIdx.x; i < W * E; i += 1024) bm[i] = 0;
    __syncthreads();
    // slot 4 q + j of a token's ids (a select chain: no dynamically indexed registers)
    auto slot_id = [&](const int32_t v[16], int j) {
        int ek = -1;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) ek = kk == 4 * q + j ? v[kk] : ek;
        return ek;
    };
    auto mark = [&](int t, const int32_t v[16]) {
        const uint32_t bit = 1u << (t & 31);
        uint32_t* row = bm + (t >> 5) * E;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ek = slot_id(v, j);
            if (4 * q + j < K && ek >= 0 && ek < E) atomicOr(&row[ek], bit);
        }
    };
    if (t0 < T) mark(t0, v0);
    for (int t = t0 + 256; t < T; t += 256) {
        int32_t v[16];
        load_token_ids(ids, t, K, v);
        mark(t, v);
    }
    __syncthreads();
    const int e = threadIdx.x;
    int c = 0;
    if (e < E)
        for (int w = 0; w < W; ++w) c += __popc(bm[w * E + e]);
    const int nu = (c + unit - 1) / unit;
    // list offsets; the first window of every touched expert first, then every later window
    int3 tot;
    const int3 ex = block_exclusive_scan3_1024(make_int3(c, c > 0 ? 1 : 0, nu > 1 ? nu - 1 : 0),
                                               smem, &tot);
    const int off = ex.x, fi = ex.y, li = ex.z;
    const int total_pairs = tot.x, touched = tot.y, later_total = tot.z;
    if (e < E) {
        offl[e] = off;
        if (use_pre) {
            int run = off;
            for (int w = 0; w < W; ++w) {
                pre[w * E + e] = (uint16_t)run;
                run += __popc(bm[w * E + e]);
            }
        }
        counts[e] = c;
        offsets[e] = off;
        if (c > 0) units[fi] = make_int4(e, off, c < unit ? c : unit, c);
        for (int j = 1; j < nu; ++j) {
            const int rest = c - j * unit;
            units[touched + li + j - 1] = make_int4(e, off + j * unit, rest < unit ? rest : unit, 0);
        }
    }
    if (threadIdx.x == 0) {
        offsets[E] = total_pairs;
        num_units[0] = touched + later_total;
        num_units[1] = T * K - total_pairs;
        num_units[2] = touched;
        num_units[3] = 0;
    }
    __syncthreads();  // offl complete
    // the fill, in the marking's layout (the repeat check looks at every earlier slot of
    // the token): all the workgroup's threads take part and each one's LDS reads go out
    // together
    auto fill = [&](int t, const int32_t v[16]) {
        const int w = t >> 5;
        const uint32_t below = (1u << (t & 31)) - 1u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = 4 * q + j, ek = slot_id(v, j);
            bool first = k < K && ek >= 0 && ek < E;
#pragma unroll
            for (int k2 = 0; k2 < 15; ++k2) first = first && !(k2 < k && v[k2] == ek);
            if (!first) continue;
            int pos = __popc(bm[w * E + ek] & below);
            if (use_pre) {
                pos += pre[w * E + ek];
            } else {
                pos += offl[ek];
                for (int w2 = 0; w2 < w; ++w2) pos += __popc(bm[w2 * E + ek]);
            }
            pairs[pos] = t * K + k;
        }
    };
    if (t0 < T) fill(t0, v0);
    for (int t = t0 + 256; t < T; t += 256) {
        int32_t v[16];
        load_token_ids(ids, t, K, v);
        fill(t, v);
    }
}

// the one-workgroup build runs when its bitmaps and offsets fit in kListsLds, E <= 1024
bool lists_fused_fits(int T, int E) { return E <= 1024 && lists_base_lds(T, E) <= kListsLds; }

hipError_t launch_lists(int T, int K, int E, int unit, const int32_t* ids, int32_t* counts,
                        int32_t* offsets, int32_t* pairs, int32_t* units, int32_t* num_units,
                        void* scratch, const uint8_t* slot_of, hipStream_t s) {
    if (lists_fused_fits(T, E)) {
        hipLaunchKernelGGL(k_lists_fused, dim3(1), dim3(1024), lists_fused_lds(T, E), s, T, K, E,
                           unit, ids, counts, offsets, (int4*)units, num_units, pairs);
        return hipGetLastError();
    }
    const int W = (T + 31) / 32;
    uint32_t* bm = (uint32_t*)scratch;
    int32_t* wordoff = (int32_t*)(bm + (size_t)W * E);
    // without the top-K's slot map the mark launch writes one into the scratch, so that the
    // fill reads one byte a pair instead of the token's K ids
    uint8_t* map = slot_of ? nullptr : lists_slot_map(scratch, T, E);
    hipLaunchKernelGGL(k_lists_mark, dim3(W), dim3(256), 0, s, T, K, E, ids, bm, map);
    hipLaunchKernelGGL(k_lists_scan, dim3(1), dim3(1024), 0, s, T, K, E, unit, bm, wordoff,
                       counts, offsets, (int4*)units, num_units);
    hipLaunchKernelGGL(k_lists_fill, dim3((W * E + 255) / 256), dim3(256), 0, s, T, K, E, bm,
                       wordoff, slot_of ? slot_of : map, pairs);
    return hipGetLastError();
}

}  // namespace moe
