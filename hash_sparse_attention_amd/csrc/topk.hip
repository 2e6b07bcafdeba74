// TopK (Oracle) selection of one decode step on gfx950: the comparison row
// of the HHR evaluation that keeps, for every (sequence, KV head), the keys
// with the largest exact attention logit instead of routing through page
// bounds and hash codes ("TopK (Oracle)" rows of Table 1 and Table 2 and
// "TopK-1.5%" in Appendix Table 4 on the thelatestinai.com page for arXiv
// 2610.01230; rit.work HHR blog post, section "Когда HHR меняет планы запуска
// модели": the evaluation includes selection by exact scores).
//
// This file holds the front of that path:
//  - prep: the group's queries widened to fp64, [D][G] per (b, h), which the
//    logit kernel reads with uniform (scalar) loads, and the per-step
//    counters cleared;
//  - logits: z(t) = max over the G query heads of sum_d q_i,d k_t,d in fp64,
//    d ascending from +0 (each product of two fp32 values is exact in fp64,
//    so the result is reproducible bit for bit), plus a histogram of the top
//    12 bits of an order key of fp32(z) that the key select starts from.
// The key select and the attention run in select.hip and attend.hip.
#include "hhr_internal.h"

namespace hhr {
namespace {

__global__ __launch_bounds__(256) void topk_prep_kernel(const void* __restrict__ Q, double* __restrict__ q64,
                                                        uint32_t* __restrict__ hist, uint32_t* __restrict__ counters,
                                                        int Hq, int Hkv, int G, int D, int bf16) {
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h, q0 = (int64_t)b * Hq + (int64_t)h * G;
    for (int x = tid; x < D * G; x += 256) {
        const int d = x / G, i = x % G;
        const int64_t e = (q0 + i) * D + d;
        const float v = bf16 ? bf16_to_f32(static_cast<const uint16_t*>(Q)[e]) : static_cast<const float*>(Q)[e];
        q64[bh * D * G + x] = (double)v;
    }
    for (int x = tid; x < kTopkBins; x += 256) hist[bh * kTopkBins + x] = 0u;
    if (tid == 0) {
        counters[bh] = 0u;                             // attention split tickets
        counters[(int64_t)gridDim.x * gridDim.y + bh] = 0u;  // boundary-bucket fill
    }
}

// One block: 4 waves, each wave 64 keys per tile (one lane per key, which
// fixes the order of its sums), `tiles` tiles per wave, chosen on the host so
// the whole grid is resident at once (no tail wave of blocks).  A tile's rows
// arrive with 1 KiB-contiguous loads (8 lanes per 128-byte row chunk) and go
// through a wave-private LDS tile (16-byte slots XOR-swizzled by row) so each
// lane can read its own row.  The next chunk's loads are in flight while the
// current one is summed.
constexpr int kLogitResident = 4 * 256;  // blocks the GPU holds at once (LDS: 4 per CU)


// The 8 16-byte pieces this lane loads of one 64-row tile chunk: rows
// t0 + 8j + lrow, bytes [c*128 + lslot*16, +16) of each row.  `filler`: the
// loop's last refill, whose data is never used; it keeps the load count fixed
// (so the waits stay exact) but every lane reads the same 16 bytes, one cache
// line per instruction instead of a whole chunk (at 128K a wave has only 8
// chunks, so re-reading one was 12% of the stream's bytes).
template <int RB>
__device__ __forceinline__ void tile_load(u32x4 (&v)[8], const char* __restrict__ kbase, int t0, int T, int c,
                                          int lrow, int lslot, bool filler = false) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int t = filler ? t0 : t0 + 8 * j + lrow;
        t = t < T ? t : T - 1;  // rows past the capacity are never used
        const int off = filler ? 0 : c * 128 + lslot * 16;
        v[j] = load_stream16(kbase + (int64_t)t * RB + off);  // K is read once
    }
}

// Stage one tile chunk through the wave's LDS tile and add it to the lane's
// G running sums (d ascending within the chunk; chunks arrive in order).
__device__ __forceinline__ void stage_chunk(const u32x4 (&v)[8], u32x4* st, int lrow, int lslot) {
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 8 * j + lrow;
        st[r * 8 + (lslot ^ (r & 7))] = v[j];
    }
    __syncthreads();
}

template <int D, bool BF16, int G>
__device__ __forceinline__ void logit_chunk(const u32x4* st, int lane, const double* __restrict__ qc, bool first,
                                            double (&acc)[G]) {
    constexpr int EPS = BF16 ? 8 : 4;  // elements per 16-byte slot
    if (first) {
#pragma unroll
        for (int i = 0; i < G; ++i) acc[i] = 0.0;
    }
    // Slots one per iteration (not unrolled): each iteration holds one slot's
    // queries (EPS * G doubles, uniform loads) instead of the whole chunk's.
#pragma unroll 1
    for (int s = 0; s < 8; ++s) {
        const double* __restrict__ qd = qc + s * EPS * G;
        const u32x4 w = st[lane * 8 + (s ^ (lane & 7))];
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
            float kf;
            if constexpr (BF16) kf = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
            else kf = __uint_as_float(w[e]);
            const double kd = (double)kf;
#pragma unroll
            for (int i = 0; i < G; ++i) acc[i] = __builtin_fma(qd[e * G + i], kd, acc[i]);
        }
    }
}

// z of the lane's key: the group max, -0 read as +0; counted in the block
// histogram (two 16-bit bins per word) when inside the sequence.  The store
// is unconditional, so the compiler can count outstanding memory operations
// exactly and keep the next chunk's loads in flight: a key in [L, T) leaves
// an unspecified entry, and a lane past the capacity (its row clamped to
// T - 1) writes z(T - 1) itself to entry T - 1.
template <int G>
__device__ __forceinline__ void logit_finish(const double (&acc)[G], int t, int L, int T, double* __restrict__ sc,
                                             uint32_t* lh) {
    double z = acc[0];
#pragma unroll
    for (int i = 1; i < G; ++i) z = acc[i] > z ? acc[i] : z;
    if (z == 0.0) z = 0.0;
    sc[t < T ? t : T - 1] = z;
    if (t < L) {
        const uint32_t bin = topk_bin(z);
        atomicAdd(&lh[bin >> 1], 1u << (16 * (bin & 1)));
    }
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void topk_logit_kernel(const void* __restrict__ K, const double* __restrict__ q64,
                                                         const int32_t* __restrict__ seq_len,
                                                         double* __restrict__ score, uint32_t* __restrict__ hist,
                                                         int Hkv, int T, int tiles) {
    constexpr int ES = BF16 ? 2 : 4;        // bytes per element
    constexpr int NC = D * ES / 128;        // 128-byte chunks per row
    constexpr int CD = 128 / ES;            // dimensions per chunk
    static_assert(NC >= 1, "row chunks");
    const int NS = tiles * NC;              // (tile, chunk) steps per wave; even (the host rounds tiles)
    __shared__ u32x4 stage[4][64 * 8];
    __shared__ uint32_t lh[kTopkBins / 2];  // a block counts at most 65535 keys per bin

    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int tb = blockIdx.x * 256 * tiles;
    if (tb >= L) return;  // block-uniform
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int x = tid; x < kTopkBins / 2; x += 256) lh[x] = 0u;
    const double* __restrict__ qh = q64 + bh * D * G;

    const char* kbase = static_cast<const char*>(K) + bh * (int64_t)T * (D * ES);
    double* __restrict__ sc = score + bh * T;
    u32x4* st = stage[wave];
    const int lrow = lane >> 3, lslot = lane & 7;
    const int tw = tb + wave * 64;  // tile k of this wave starts at tw + k * 256

    // Steps (tile, chunk) in order, two at a time with fixed buffers: the
    // loads of the next step are in flight while this one is summed.
    // Steps (tile, chunk) in order, two per iteration with fixed register
    // buffers A and B: B's loads go out at the top of the iteration and A is
    // refilled (two steps ahead) as soon as it is in LDS, so loads stay in
    // flight while a chunk is summed.  Every load is unconditional (the last
    // ones re-load a chunk already read) and A's loads are always older than
    // B's, so the compiler can wait for exactly the buffer it needs.
    u32x4 A[8], B[8];
    double acc[G];
    auto t_of = [&](int step) { return tw + (step / NC) * 256; };
    tile_load<D * ES>(A, kbase, t_of(0), T, 0, lrow, lslot);
#pragma unroll 1
    for (int step = 0; step < NS; step += 2) {
        const int ca = step % NC, cb = (step + 1) % NC;
        if (tb + (step / NC) * 256 >= L) break;  // block-uniform: the rest of the block is past the sequence
        const int na = step + 2 < NS ? step + 2 : step;
        tile_load<D * ES>(B, kbase, t_of(step + 1), T, cb, lrow, lslot);
        stage_chunk(A, st, lrow, lslot);
        tile_load<D * ES>(A, kbase, t_of(na), T, na % NC, lrow, lslot, na == step);
        logit_chunk<D, BF16, G>(st, lane, qh + ca * CD * G, ca == 0, acc);
        if constexpr (NC == 1) logit_finish<G>(acc, t_of(step) + lane, L, T, sc, lh);
        else if constexpr (NC > 2) {
            if (ca == NC - 1) logit_finish<G>(acc, t_of(step) + lane, L, T, sc, lh);
        }
        stage_chunk(B, st, lrow, lslot);
        logit_chunk<D, BF16, G>(st, lane, qh + cb * CD * G, cb == 0, acc);
        if constexpr (NC <= 2) logit_finish<G>(acc, t_of(step + 1) + lane, L, T, sc, lh);
        else if (cb == NC - 1) logit_finish<G>(acc, t_of(step + 1) + lane, L, T, sc, lh);
    }
    __syncthreads();
    uint32_t* gh = hist + bh * kTopkBins;
    for (int x = tid; x < kTopkBins / 2; x += 256) {
        const uint32_t n = lh[x];
        if (n & 0xffffu) atomicAdd(&gh[2 * x], n & 0xffffu);
        if (n >> 16) atomicAdd(&gh[2 * x + 1], n >> 16);
    }
}

template <int D, bool BF16, int G>
hipError_t logits_g(const TopkArgs& a, hipStream_t st) {
    const Shape& s = a.d.s;
    // Tiles per wave: enough that the grid fits the resident block slots, even.
    const int64_t heads = (int64_t)s.B * s.Hkv;
    const int64_t per_head = kLogitResident / heads > 0 ? kLogitResident / heads : 1;
    int tiles = (int)((s.T + 256 * per_head - 1) / (256 * per_head));
    tiles = tiles < 2 ? 2 : tiles + (tiles & 1);
    const dim3 grid((unsigned)((s.T + 256 * tiles - 1) / (256 * tiles)), s.Hkv, s.B);
    hipLaunchKernelGGL((topk_logit_kernel<D, BF16, G>), grid, dim3(256), 0, st, a.d.K,
                       reinterpret_cast<const double*>(a.d.ws + a.tl.q64), a.d.seq_len,
                       reinterpret_cast<double*>(a.d.ws + a.tl.score),
                       reinterpret_cast<uint32_t*>(a.d.ws + a.tl.hist), s.Hkv, s.T, tiles);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t logits_dt(const TopkArgs& a, hipStream_t st) {
    switch (a.d.s.G) {
        case 1: return logits_g<D, BF16, 1>(a, st);
        case 2: return logits_g<D, BF16, 2>(a, st);
        case 3: return logits_g<D, BF16, 3>(a, st);
        case 4: return logits_g<D, BF16, 4>(a, st);
        case 5: return logits_g<D, BF16, 5>(a, st);
        case 6: return logits_g<D, BF16, 6>(a, st);
        case 7: return logits_g<D, BF16, 7>(a, st);
        default: return logits_g<D, BF16, 8>(a, st);
    }
}

}  // namespace

hipError_t launch_topk_prep(const TopkArgs& a, hipStream_t st) {
    const Shape& s = a.d.s;
    hipLaunchKernelGGL(topk_prep_kernel, dim3(s.Hkv, s.B), dim3(256), 0, st, a.d.Q,
                       reinterpret_cast<double*>(a.d.ws + a.tl.q64), reinterpret_cast<uint32_t*>(a.d.ws + a.tl.hist),
                       reinterpret_cast<uint32_t*>(a.d.ws + a.d.lay.counters), s.Hq, s.Hkv, s.G, s.D, s.bf16 ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_topk_logits(const TopkArgs& a, hipStream_t st) {
    const Shape& s = a.d.s;
    if (s.D == 64) return s.bf16 ? logits_dt<64, true>(a, st) : logits_dt<64, false>(a, st);
    return s.bf16 ? logits_dt<128, true>(a, st) : logits_dt<128, false>(a, st);
}

}  // namespace hhr
