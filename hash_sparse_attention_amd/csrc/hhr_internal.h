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
    bool bf16;      // Q, K, V are bf16
    bool meta16;    // page metadata is bf16 (outward-rounded)
    bool msplit;    // page metadata is dimension-major with max and min sides apart (sign-split)
    int nsink, window;  // keys always attended: the first nsink and the last window
    bool pg_min;        // page score = min over the group (else max)
    bool ham_mean;      // Hamming against the group's mean-query code (else summed over the group)
    int Gh;             // query codes per KV head in the Hamming stage: 1 with ham_mean, else G
    int share;          // selection units per data head: 1, or G with per-query-head selection
                        // (then Hkv counts units, G = 1, and a unit's data head is unit / share)
    bool per_head;      // per-query-head selection was asked for
};

// The shape the selection stages run on: with per-query-head selection one
// unit per query head (Hkv := Hq, G := 1), reading data head unit / share.
inline Shape selection_shape(const Shape& d) {
    if (!d.per_head || d.G == 1) return d;
    Shape s = d;
    s.share = d.G;
    s.Hkv = d.Hq;
    s.G = 1;
    s.Gh = 1;
    s.ham_mean = false;  // the mean of one query is that query
    s.pg_min = false;    // the min over one head is that head's bound
    return s;
}

// Attention keys handled by one block (one split) of the attend kernel.
constexpr int kAttnChunk = 128;

// Key select: candidate slots per block-local chunk, the kept pages the
// select kernel holds in LDS, and the candidate slots one compact+attend
// block owns (8 per thread).
constexpr int kSelChunk = 16384;
constexpr int kSelListLds = 8192;
constexpr int kCompactSlots = 2048;

// Bit pattern of a split attention partial not yet written in this step (a
// NaN payload that arithmetic never produces).
constexpr uint32_t kPartSentinel = 0x7fbadbadu;

// Region offsets of the decode workspace (bytes, 256-aligned).  counters:
// [0, B*Hkv) attention-split counters, then (sel_splits > 1) the per-(b, h)
// Hamming histograms of the head, ghist_off u32 entries in; both are cleared
// by the query prep of every step.  kcum (private, sel_splits > 1): per
// (b, h) and select block, the block's cumulative Hamming histogram.
// part_splits: split stride of the attention partials.
struct WsLayout {
    size_t q_rot, code_q, q_split, score, pages, n_pages, ham, sel, k_eff, partial, counters, kcum, total;
    size_t code_qm;  // the group's mean-query code [B][Hkv][NW] (ham_mean)
    int n_splits, sel_splits, part_splits, nbins;
    bool sel_pages_apart;  // split select: the page select runs once per head in a launch of its own
    size_t ghist_off;  // u32 entries from counters to the head histograms
    int n_clear;       // u32 entries the query prep clears from counters
};

WsLayout ws_layout(const Shape& s, int max_keep, int top_k);

// Kernel launchers (defined in the .hip files); each returns the hipError_t of its launch.
hipError_t launch_encode(const Shape& s, const void* K, const float* R, const float* W, const int32_t* start,
                         const int32_t* count, int max_count, float* meta, uint64_t* codes,
                         hipStream_t stream);

struct DecodeArgs {
    Shape s;   // selection shape (units)
    Shape sd;  // data shape (the KV heads of the cache): projection and append
    int max_keep, top_k;
    int sel_cap;  // entries per (b, h) row of sel: top_k plus the forced keys' room
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

// TopK (Oracle) path: 12-bit histogram digits of the exact logits, keys per
// collect / write block, the largest boundary bucket ranked in registers,
// and the most collect blocks one (b, h) can have (max_ctx <= 2^26).
constexpr int kTopkBins = 4096;
constexpr int kTopkBlk = 4096;
constexpr int kTopkCap = 16384;
constexpr int kTopkMaxBlk = (1 << 26) / kTopkBlk;

// Workspace regions of the TopK (Oracle) step beyond those it shares with
// the decode step's layout (sel, k_eff, partial, counters: counters holds
// B*Hkv attention tickets, then B*Hkv bucket fill counts).
struct TopkLayout {
    size_t score, q64, hist, info, bkey, bidx, ocnt, off;
    int nblk;  // collect / write blocks per (b, h)
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
    uint64_t* code_qm;  // with ham_mean: the group's mean-query code
    double* q_split;
    uint32_t* counters;
    int n_counters;
    bool qmean;    // also code the group's mean query into code_qm (queries only)
};
// Appends of at most this many keys per sequence go through the projection kernel.
constexpr int kAppendMax = 64;

hipError_t launch_project(const Shape& s, const ProjectArgs& a, hipStream_t stream);
hipError_t launch_qprep(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_page_bounds(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_select(const DecodeArgs& a, hipStream_t stream);  // pages, then keys, one launch
hipError_t launch_select_pages(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_hamming(const DecodeArgs& a, hipStream_t stream);  // ham only
hipError_t launch_select_keys(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_attend(const DecodeArgs& a, bool zero_counters, hipStream_t stream);
// Threshold, ordered compaction and attention of the split key select (the decode step when sel_splits > 1).
hipError_t launch_compact_attend(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream);

struct TopkArgs {
    DecodeArgs d;  // Q, K, V, seq_len, top_k, scale, out, sel, ws and the shared layout
    TopkLayout tl;
};
void topk_layout(const Shape& s, int top_k, WsLayout& lay, TopkLayout& tl);
hipError_t launch_topk_prep(const TopkArgs& a, hipStream_t stream);
hipError_t launch_topk_logits(const TopkArgs& a, hipStream_t stream);
hipError_t launch_topk_select(const TopkArgs& a, hipStream_t stream);  // collect, threshold, ordered write

// ---------------------------------------------------------------- device helpers

// A native vector of four 32-bit words: the compiler keeps it in registers
// (the HIP struct vector types can go to scratch when indexed in a rolled loop).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the nontemporal hint, for data a step reads exactly once:
// the page metadata of the bound pass, the keys of the exact-logit pass, the
// candidates' codes, the gathered K/V rows and the projection rows.  Measured
// on gfx950 at 128K context: the bound stream ran 4.7 TB/s with it against
// 4.2 TB/s with plain loads, the logit stream 4.8 against 4.4, and the hinted
// code loads and row gathers took the decode step from 53.4 to 51.4 us per
// layer.  Data the previous launch wrote is read with plain loads (hinting
// the select outputs that compaction reads back made the step slower); the
// page scores are the one exception, measured slightly faster hinted.
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Outward rounding of page statistics to bf16 (bit patterns): the smallest
// bf16 >= x for a max, the largest bf16 <= x for a min.  Dropping the low
// half of the bits moves x toward zero, so a positive max (negative min)
// with a nonzero low half goes one bf16 step further out.  Finite inputs,
// -0 already read as +0.
__device__ __forceinline__ uint32_t bf16_up(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u >> 16) + ((u & 0xffffu) != 0 && !(u >> 31) ? 1u : 0u);
}
__device__ __forceinline__ uint32_t bf16_down(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u >> 16) + ((u & 0xffffu) != 0 && (u >> 31) ? 1u : 0u);
}
// (max, min) of one dimension as the two bf16 of a 32-bit word, max first.
__device__ __forceinline__ uint32_t bf16_pair_out(float mx, float mn) { return bf16_up(mx) | (bf16_down(mn) << 16); }

// 12-bit digit of a logit for the TopK (Oracle) histogram: the top bits of
// the order-preserving 32-bit key of its fp32 rounding (a monotone map, so a
// higher digit means a larger logit).
__device__ __forceinline__ uint32_t topk_bin(double z) {
    const uint32_t u = __float_as_uint((float)z);
    return ((u >> 31) ? ~u : (u | 0x80000000u)) >> 20;
}

__device__ __forceinline__ int clamp_len(int L, int T) { return L < 0 ? 0 : (L > T ? T : L); }

// P is a power of two (validated on the host): a shift, not a 64-bit division.
__device__ __forceinline__ int64_t n_pages_of(int64_t L, int P) { return (L + P - 1) >> __builtin_ctz((unsigned)P); }

// Data head of selection unit h of sequence b (share > 1 only with per-query-head selection).
__device__ __forceinline__ int64_t data_head(int b, int h, int Hunits, int share) {
    return share == 1 ? (int64_t)b * Hunits + h : (int64_t)b * (Hunits / share) + h / share;
}

// ---- wave64 primitives on DPP (row shifts within 16-lane rows, then row
// broadcasts across rows).  A DPP step is a VALU op: far cheaper than a
// cross-lane permute through LDS, which is what __shfl compiles to.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int old, int x) {
    return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += dpp_i<kRowShr1, 0xf>(0, x);
    x += dpp_i<kRowShr2, 0xf>(0, x);
    x += dpp_i<kRowShr4, 0xf>(0, x);
    x += dpp_i<kRowShr8, 0xf>(0, x);
    x += dpp_i<kRowBcast15, 0xa>(0, x);
    x += dpp_i<kRowBcast31, 0xc>(0, x);
    return x;
}

// Wave-wide max / sum / OR, returned to every lane (a fixed combination
// order, so float sums are reproducible bit for bit).
__device__ __forceinline__ float wave_max(float x) {
    const int id = __float_as_int(-__builtin_inff());
    x = fmaxf(x, __int_as_float(dpp_i<kRowShr1, 0xf>(id, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowShr2, 0xf>(id, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowShr4, 0xf>(id, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowShr8, 0xf>(id, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowBcast15, 0xa>(id, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowBcast31, 0xc>(id, __float_as_int(x))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += __int_as_float(dpp_i<kRowShr1, 0xf>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowShr2, 0xf>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowShr4, 0xf>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowShr8, 0xf>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowBcast15, 0xa>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowBcast31, 0xc>(0, __float_as_int(x)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
    x |= (uint32_t)dpp_i<kRowShr1, 0xf>(0, (int)x);
    x |= (uint32_t)dpp_i<kRowShr2, 0xf>(0, (int)x);
    x |= (uint32_t)dpp_i<kRowShr4, 0xf>(0, (int)x);
    x |= (uint32_t)dpp_i<kRowShr8, 0xf>(0, (int)x);
    x |= (uint32_t)dpp_i<kRowBcast15, 0xa>(0, (int)x);
    x |= (uint32_t)dpp_i<kRowBcast31, 0xc>(0, (int)x);
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_and(uint32_t x) {
    x &= (uint32_t)dpp_i<kRowShr1, 0xf>(-1, (int)x);
    x &= (uint32_t)dpp_i<kRowShr2, 0xf>(-1, (int)x);
    x &= (uint32_t)dpp_i<kRowShr4, 0xf>(-1, (int)x);
    x &= (uint32_t)dpp_i<kRowShr8, 0xf>(-1, (int)x);
    x &= (uint32_t)dpp_i<kRowBcast15, 0xa>(-1, (int)x);
    x &= (uint32_t)dpp_i<kRowBcast31, 0xc>(-1, (int)x);
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Lanes below this one whose bit is set in the wave mask m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum of v over a block of NT threads (a multiple of 64, at
// most 1024; a constant, since blockDim.x is a load from the dispatch packet).
// `scratch` holds >= 16 ints of LDS.  Returns the prefix and the block total;
// every thread of the block must call it.
template <int NT, bool TAIL = true>
__device__ __forceinline__ int block_excl_scan(int v, int* scratch, int& total) {
    static_assert(NT % 64 == 0 && NT <= 1024, "block size");
    constexpr int nw = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < nw; ++w) {
        const int t = scratch[w];
        base += w < wave ? t : 0;
        tot += t;
    }
    total = tot;
    if (TAIL) __syncthreads();  // scratch may be rewritten next (TAIL = false: the caller passes a barrier first)
    return base + x - v;
}

}  // namespace hhr
