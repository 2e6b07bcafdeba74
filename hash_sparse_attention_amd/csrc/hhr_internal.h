// Internal definitions of libhhr (HIP, gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/hhr.h"

namespace hhr {

// Resolved dimensions of one call.
struct Shape {
    int B, Hq, Hkv, G, D, P, NB, NW, T;
    int64_t NPmax;  // pages of a full-capacity sequence
    int64_t NPB;    // 64-page blocks of meta per (b, h)
    bool bf16;
};

// Attention keys handled by one block (one split) of the attend kernel.
constexpr int kAttnChunk = 256;

// Region offsets of the decode workspace (bytes, 256-aligned).
struct WsLayout {
    size_t q_rot, code_q, q_split, score, pages, n_pages, ham, sel, k_eff, partial, counters, total;
    int n_splits;
};

WsLayout ws_layout(const Shape& s, int max_keep, int top_k);

// Kernel launchers (defined in the .hip files); each returns the hipError_t of its launch.
hipError_t launch_encode(const Shape& s, const void* K, const float* R, const float* W, const int32_t* start,
                         const int32_t* count, int max_count, float* meta, uint64_t* codes,
                         hipStream_t stream);

struct DecodeArgs {
    Shape s;
    int max_keep, top_k;
    float scale;
    const void *Q, *K, *V;
    const float *R, *W, *meta;
    const uint64_t* codes;
    const int32_t *seq_len, *keep_pages;
    float* out;
    int32_t* sel;  // user sel_idx or the workspace region
    char* ws;
    WsLayout lay;
};

// Projection of a few vectors (appended keys and/or the queries) by [R_h; W_h].
struct ProjectArgs {
    bool keys, queries;
    const void *Q, *K;
    const float *R, *W;
    const int32_t *start, *count;
    int max_count;
    float* meta;
    uint64_t* codes;
    float* q_rot;
    uint64_t* code_q;
    double* q_split;
    uint32_t* counters;
    int n_counters;
};
// Appends of at most this many keys per sequence go through the projection kernel.
constexpr int kAppendMax = 64;

hipError_t launch_project(const Shape& s, const ProjectArgs& a, hipStream_t stream);
hipError_t launch_qprep(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_page_bounds(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_select(const DecodeArgs& a, hipStream_t stream);  // pages, then keys, one launch
hipError_t launch_select_pages(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_select_keys(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_attend(const DecodeArgs& a, bool zero_counters, hipStream_t stream);

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ int clamp_len(int L, int T) { return L < 0 ? 0 : (L > T ? T : L); }

__device__ __forceinline__ int64_t n_pages_of(int64_t L, int P) { return (L + P - 1) / P; }

// Exclusive prefix sum of v over the whole block (blockDim.x a multiple of 64,
// at most 1024).  `scratch` holds >= 17 ints of LDS.  Returns the prefix and
// the block total; every thread of the block must call it.
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int n = __shfl_up(x, off, 64);
        if (lane >= off) x += n;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int w = lane < nw ? scratch[lane] : 0;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            int n = __shfl_up(w, off, 64);
            if (lane >= off) w += n;
        }
        if (lane < nw) scratch[lane] = w;
    }
    __syncthreads();
    const int base = wave ? scratch[wave - 1] : 0;
    total = scratch[nw - 1];
    __syncthreads();
    return base + x - v;
}

}  // namespace hhr
