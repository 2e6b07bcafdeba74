// GKR page bounds of the HHR decode step on gfx950 (and the query-prep
// launcher, which runs the projection kernel).
// ("HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", Abstract;
// rit.work HHR blog post, sections "Почему расстояние Хэмминга пропускает
// важные ключи" and "Два уровня маршрутизации решают разные ошибки";
// top-k selection as in Appendix Table 4 of the thelatestinai.com page.)
#include <type_traits>

#include "hhr_internal.h"

namespace hhr {
namespace {

// ============================================================== page bounds
// One lane per page; a wave covers one 64-page block of meta, so each
// float4 load of a dimension pair is one contiguous 1 KiB span per wave.  The
// lane sums in fp64, dimensions ascending, exactly the definition's order:
// per dimension fma(max(q,0), kmax, acc) then fma(min(q,0), kmin, acc) -- one
// of the two products is zero, the other is the larger of q*kmax and q*kmin,
// and every such product is exact in fp64.
//
// The order of the sum ties each page to one lane, so a launch has one wave
// per SIMD at 64K pages; the stream stays busy because every lane keeps the
// next batch of U 16-byte loads in flight while it sums the current one.
// (Measured on gfx950: spreading a page over 2, 4 or 8 waves, each summing
// part of the dimensions, streams no faster than one lane per page, and
// issuing the first batches before the query terms are staged gains nothing.)  The
// loads carry the nontemporal hint: every metadata line is read once.
//
// The query terms are block-uniform (a block covers pages of one head).  For
// G <= 4 they reach the FMAs as scalar loads, an SGPR operand each, so the
// stream issues no LDS reads at all; a 16-byte LDS broadcast still returns
// 16 bytes per lane, and at G = 4 a page block needs 512 of them.  The block
// first pulls its terms into the XCD's L2 with one coalesced round trip: the
// projection launch has just written them, and scalar misses issued a slot
// or two ahead would otherwise serialise.  Larger groups, and bf16 metadata
// (a 16-byte slot then holds 4 dimensions: 64 SGPRs of terms per slot at
// G = 4), need more SGPRs per slot than the scalar file holds without
// stalling or spilling, so they stage the terms once per block in LDS and read
// them as broadcasts (measured: bf16 metadata at G = 4 ran 17.6 us per launch
// on scalar terms against 11.6 us on LDS).
template <int G, int U>
__device__ __forceinline__ void bound_batch(const float4 (&v)[U], const double2* __restrict__ qs, int j0,
                                            double (&acc)[G]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int d = 2 * (j0 + u);
        const double a0 = v[u].x, c0 = v[u].y, a1 = v[u].z, c1 = v[u].w;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const double2 q0 = qs[d * G + i], q1 = qs[(d + 1) * G + i];
            acc[i] = __builtin_fma(q0.x, a0, acc[i]);
            acc[i] = __builtin_fma(q0.y, c0, acc[i]);
            acc[i] = __builtin_fma(q1.x, a1, acc[i]);
            acc[i] = __builtin_fma(q1.y, c1, acc[i]);
        }
    }
}

// The same for bf16 metadata: one 16-byte slot holds a dimension quad
// (max, min) x 4 as bf16, widened exactly to fp64.
template <int G, int U>
__device__ __forceinline__ void bound_batch16(const uint4 (&v)[U], const double2* __restrict__ qs, int j0,
                                              double (&acc)[G]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int d = 4 * (j0 + u);
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double a = __uint_as_float(w[e] << 16), c = __uint_as_float(w[e] & 0xffff0000u);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const double2 q = qs[(d + e) * G + i];
                acc[i] = __builtin_fma(q.x, a, acc[i]);
                acc[i] = __builtin_fma(q.y, c, acc[i]);
            }
        }
    }
}

// Every lane of the block loads its share of the head's D * G query terms
// (all loads issued, then waited for), so the lines sit in this XCD's L2
// before the waves read them as scalar loads.
template <int D, int G, int NT>
__device__ __forceinline__ void warm_query_terms(const double2* __restrict__ qg) {
    constexpr int NQ = (D * G + NT - 1) / NT;
    double2 t[NQ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        const int x = threadIdx.x + r * NT;
        t[r] = qg[x < D * G ? x : 0];
    }
#pragma unroll
    for (int r = 0; r < NQ; ++r) asm volatile("" ::"v"(t[r].x), "v"(t[r].y));  // wait for every load
}

// Pages (lanes) per block: 128 when the query terms are scalar loads -- at
// batch 8 and 32K the finer blocks spread the stream more evenly over the
// compute units (measured: the launch 7-8% shorter, the same at 128K) --
// and 256 when each block stages the terms in LDS first (G > 4 or bf16
// metadata), where halving the blocks would double the staging.
template <int D, int G, bool M16>
constexpr int bound_block_pages() { return (G <= 4 && !M16) ? 128 : 256; }

// PU (per-query-head selection with interleaved metadata): the launch runs
// over data heads, and each of the group's G sums is written as its own
// unit's score (unit = data head * G + i) instead of their max, so a KV
// head's metadata is streamed once for its G selection units.
template <int D, int G, int U, bool M16, bool PGMIN, int BP = bound_block_pages<D, G, M16>(), bool PU = false>
__global__ __launch_bounds__(BP) void page_bound_kernel(const float* __restrict__ meta,
                                                         const double* __restrict__ q_split,
                                                         const int32_t* __restrict__ seq_len,
                                                         double* __restrict__ score, int Hkv, int T, int P,
                                                         int64_t NPB, int64_t NPmax, int share, int nbatch) {
    constexpr int NJ = M16 ? D / 4 : D / 2;  // 16-byte slots per page
    static_assert(NJ % U == 0, "batches");
    constexpr bool SQ = G <= 4 && !M16;       // query terms as scalar loads (else LDS broadcasts)
    using V4 = typename std::conditional<M16, uint4, float4>::type;
    __shared__ double2 qs_lds[SQ ? 1 : D * G];  // (max(q,0), min(q,0)) per dimension and query head
    // One-dimensional grid in (head, sequence, page block) order, head fastest: the workgroups of a
    // (sequence, head) share an XCD with the projection blocks that wrote its query terms and the select
    // blocks that read its scores (workgroups go to the XCDs in turn by linear index).
    // (Per-query-head selection runs this kernel over KV heads with PU set.)
    const int h = (int)(blockIdx.x % (unsigned)Hkv);
    const int b = (int)((blockIdx.x / (unsigned)Hkv) % (unsigned)nbatch);
    const int64_t pb = blockIdx.x / ((unsigned)Hkv * (unsigned)nbatch);
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int64_t NP = n_pages_of(L, P);
    const int64_t p = pb * BP + threadIdx.x;
    if (pb * BP >= NP) return;  // block-uniform

    const double2* qg = reinterpret_cast<const double2*>(q_split) + bh * D * G;
    if constexpr (SQ) {
        warm_query_terms<D, G, BP>(qg);
    } else {
        for (int x = threadIdx.x; x < D * G; x += BP) qs_lds[x] = qg[x];
    }
    __syncthreads();
    if (p >= NP) return;
    const double2* qs = SQ ? qg : qs_lds;

    const int64_t bhd = data_head(b, h, Hkv, share);  // the unit's data head
    const V4* mp = reinterpret_cast<const V4*>(meta) + (bhd * NPB + p / 64) * NJ * 64 + (p & 63);
    double acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = 0.0;

    // Double buffering, fully unrolled: batch k + 1 is in flight while batch k
    // is summed.  The empty asm statements are compiler barriers for memory
    // operations, so the loads stay where they are written.
    constexpr int NBT = NJ / U;
    V4 A[U], B[U];
    auto load = [&](V4 (&v)[U], int k) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4 r = load_stream16(mp + (int64_t)(k * U + u) * 64);
            if constexpr (M16) v[u] = make_uint4(r.x, r.y, r.z, r.w);
            else v[u] = make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w));
        }
    };
    load(A, 0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < NBT; k += 2) {
        if (k + 1 < NBT) load(B, k + 1);
        asm volatile("" ::: "memory");
        if constexpr (M16) bound_batch16<G, U>(A, qs, k * U, acc);
        else bound_batch<G, U>(A, qs, k * U, acc);
        asm volatile("" ::: "memory");
        if (k + 2 < NBT) load(A, k + 2);
        asm volatile("" ::: "memory");
        if constexpr (M16) {
            if (k + 1 < NBT) bound_batch16<G, U>(B, qs, (k + 1) * U, acc);
        } else {
            if (k + 1 < NBT) bound_batch<G, U>(B, qs, (k + 1) * U, acc);
        }
        asm volatile("" ::: "memory");
    }
    if constexpr (PU) {
#pragma unroll
        for (int i = 0; i < G; ++i) score[(bh * G + i) * NPmax + p] = acc[i] == 0.0 ? 0.0 : acc[i];
        return;
    }
    double S = acc[0];  // the group's max, or its min (a variant)
#pragma unroll
    for (int i = 1; i < G; ++i) S = PGMIN ? (acc[i] < S ? acc[i] : S) : (acc[i] > S ? acc[i] : S);
    if (S == 0.0) S = 0.0;
    score[bh * NPmax + p] = S;
}

// Sign-split metadata (dimension-major per 64-page block: the 64 pages' max
// values of a dimension, then their min values; fp32 or bf16).  With one
// query head per selection (G = 1) only the side the sign of the rotated
// query coordinate picks is read: kmax where q >= 0 (q_split's min term is
// zero), kmin where q < 0.  The side not read would add an exact zero, so the
// fp64 sum, dimensions ascending, is the interleaved kernel's bit for bit
// (the sign of a zero score aside, which is normalised).  The side of each
// dimension is a bit of a wave-uniform mask built by ballots, so every load
// address is uniform plus the lane: one contiguous 256-byte (fp32) or
// 128-byte (bf16) run per wave and dimension.  With G > 1 both sides are read.
// For G = 1 every wave loads the D query terms itself (coalesced, two per
// lane at D = 128) for the ballots, which also brings them into the XCD's L2,
// and the sums read them as scalar loads: no LDS and no block barrier.
// PU: as in page_bound_kernel, one pass per data head writes each of the G
// sums as its own unit's score (per-query-head selection).  Each sum adds
// both sides of every dimension; the side a head's sign does not pick adds
// an exact zero, so the bits are those of that head's one-side sum.
template <int D, int G, int U, bool M16, bool PGMIN, bool PU = false>
__global__ __launch_bounds__(256) void page_bound_split_kernel(const float* __restrict__ meta,
                                                               const double* __restrict__ q_split,
                                                               const int32_t* __restrict__ seq_len,
                                                               double* __restrict__ score, int Hkv, int T, int P,
                                                               int64_t NPB, int64_t NPmax, int share, int nbatch) {
    using E = typename std::conditional<M16, uint16_t, float>::type;
    constexpr int NS = G == 1 ? 1 : 2;  // sides read per dimension
    constexpr int NBT = D / U;          // batches of U dimensions
    static_assert(D % U == 0 && NBT % 2 == 0, "batches");
    __shared__ double2 qs_lds[G == 1 ? 1 : D * G];  // (max(q,0), min(q,0)) per dimension and query head
    // One-dimensional grid in (head, sequence, page block) order, head fastest: the workgroups of a
    // (sequence, head) share an XCD with the projection blocks that wrote its query terms and the select
    // blocks that read its scores (workgroups go to the XCDs in turn by linear index).
    // (Per-query-head selection runs this kernel over KV heads with PU set.)
    const int h = (int)(blockIdx.x % (unsigned)Hkv);
    const int b = (int)((blockIdx.x / (unsigned)Hkv) % (unsigned)nbatch);
    const int64_t pb = blockIdx.x / ((unsigned)Hkv * (unsigned)nbatch);
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int64_t NP = n_pages_of(L, P);
    const int64_t p = pb * 256 + threadIdx.x;
    if (pb * 256 >= NP) return;  // block-uniform

    const double2* qg = reinterpret_cast<const double2*>(q_split) + bh * D * G;
    // G = 1: bit d set when q_d < 0 (the min side is read).  Built while every
    // lane of the wave is active: a ballot leaves out lanes that have exited.
    const int lane = threadIdx.x & 63;
    uint64_t neg[D / 64];
    if constexpr (G == 1) {
        double qn[D / 64];
#pragma unroll
        for (int w = 0; w < D / 64; ++w) qn[w] = qg[w * 64 + lane].y;
#pragma unroll
        for (int w = 0; w < D / 64; ++w) neg[w] = __ballot(qn[w] != 0.0);
    } else {
        for (int x = threadIdx.x; x < D * G; x += 256) qs_lds[x] = qg[x];
        __syncthreads();
#pragma unroll
        for (int w = 0; w < D / 64; ++w) neg[w] = 0ull;
    }
    if (p >= NP) return;
    const double2* qs = G == 1 ? qg : qs_lds;

    const int64_t bhd = data_head(b, h, Hkv, share);  // the unit's data head
    const E* mp = reinterpret_cast<const E*>(meta) + ((bhd * NPB + p / 64) * D) * 128 + (p & 63);
    auto side = [&](int d) { return (int)((neg[d >> 6] >> (d & 63)) & 1u); };
    auto widen = [](E v) -> double {
        if constexpr (M16) return (double)__uint_as_float((uint32_t)v << 16);
        else return (double)v;
    };
    double acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = 0.0;
    E A[U][NS], B[U][NS];
    auto load = [&](E (&v)[U][NS], int k) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int d = k * U + u;
            if constexpr (G == 1) {
                v[u][0] = __builtin_nontemporal_load(mp + d * 128 + side(d) * 64);
            } else {
                v[u][0] = __builtin_nontemporal_load(mp + d * 128);
                v[u][1] = __builtin_nontemporal_load(mp + d * 128 + 64);
            }
        }
    };
    auto sum = [&](const E (&v)[U][NS], int k) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int d = k * U + u;
            if constexpr (G == 1) {  // the sign-selected term only: one scalar load of 8 bytes
                const double q = reinterpret_cast<const double*>(qs)[2 * d + side(d)];
                acc[0] = __builtin_fma(q, widen(v[u][0]), acc[0]);
            } else {
                const double a = widen(v[u][0]), c = widen(v[u][1]);
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const double2 q = qs[d * G + i];
                    acc[i] = __builtin_fma(q.x, a, acc[i]);
                    acc[i] = __builtin_fma(q.y, c, acc[i]);
                }
            }
        }
    };
    // Double buffering, fully unrolled; the empty asm statements keep the
    // loads where they are written.
    load(A, 0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < NBT; k += 2) {
        load(B, k + 1);
        asm volatile("" ::: "memory");
        sum(A, k);
        asm volatile("" ::: "memory");
        if (k + 2 < NBT) load(A, k + 2);
        asm volatile("" ::: "memory");
        sum(B, k + 1);
        asm volatile("" ::: "memory");
    }
    if constexpr (PU) {
#pragma unroll
        for (int i = 0; i < G; ++i) score[(bh * G + i) * NPmax + p] = acc[i] == 0.0 ? 0.0 : acc[i];
        return;
    }
    double S = acc[0];  // the group's max, or its min (a variant)
#pragma unroll
    for (int i = 1; i < G; ++i) S = PGMIN ? (acc[i] < S ? acc[i] : S) : (acc[i] > S ? acc[i] : S);
    if (S == 0.0) S = 0.0;
    score[bh * NPmax + p] = S;
}

// ------------------------------------------------------------------ dispatch helpers
template <int D, int G>
hipError_t bounds_g(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    // Pages per block: the interleaved kernel's choice, or 256 for the sign-split kernel.
    const int bp = s.msplit ? 256 : (s.meta16 ? bound_block_pages<D, G, true>() : bound_block_pages<D, G, false>());
    const dim3 grid((unsigned)(((s.NPmax + bp - 1) / bp) * s.Hkv * s.B));
    // Loads per lane per batch (two batches in flight), measured best per metadata type.
    auto kern = s.meta16 ? (s.pg_min ? page_bound_kernel<D, G, 8, true, true> : page_bound_kernel<D, G, 8, true, false>)
                         : (s.pg_min ? page_bound_kernel<D, G, 4, false, true> : page_bound_kernel<D, G, 4, false, false>);
    if (s.msplit) {  // dimensions per batch: 16 single-side loads for G = 1, else 8 dimensions of two loads
        constexpr int US = G == 1 ? 16 : 8;
        kern = s.meta16 ? (s.pg_min ? page_bound_split_kernel<D, G, US, true, true>
                                    : page_bound_split_kernel<D, G, US, true, false>)
                        : (s.pg_min ? page_bound_split_kernel<D, G, US, false, true>
                                    : page_bound_split_kernel<D, G, US, false, false>);
    }
    hipLaunchKernelGGL(kern, grid, dim3(bp), 0, st, a.meta,
                       reinterpret_cast<const double*>(a.ws + a.lay.q_split), a.seq_len,
                       reinterpret_cast<double*>(a.ws + a.lay.score), s.Hkv, s.T, s.P, s.NPB, s.NPmax,
                       s.share, s.B);
    return hipGetLastError();
}

// Per-query-head selection: one pass per data head (G = the units per data
// head), each unit's score written separately.
template <int D, int G>
hipError_t bounds_units(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    const int Hd = s.Hkv / G;  // data heads (s.Hkv counts the units)
    constexpr int BP16 = bound_block_pages<D, G, true>(), BP32 = bound_block_pages<D, G, false>();
    const int bp = s.msplit ? 256 : (s.meta16 ? BP16 : BP32);
    const dim3 grid((unsigned)(((s.NPmax + bp - 1) / bp) * Hd * s.B));
    auto kern = s.meta16 ? page_bound_kernel<D, G, 8, true, false, BP16, true>
                         : page_bound_kernel<D, G, 4, false, false, BP32, true>;
    if (s.msplit)  // both sides of 8 dimensions a batch, as for a shared selection
        kern = s.meta16 ? page_bound_split_kernel<D, G, 8, true, false, true>
                        : page_bound_split_kernel<D, G, 8, false, false, true>;
    hipLaunchKernelGGL(kern, grid, dim3(bp), 0, st, a.meta, reinterpret_cast<const double*>(a.ws + a.lay.q_split),
                       a.seq_len, reinterpret_cast<double*>(a.ws + a.lay.score), Hd, s.T, s.P, s.NPB, s.NPmax, 1,
                       s.B);
    return hipGetLastError();
}

template <int D>
hipError_t bounds_d(const DecodeArgs& a, hipStream_t st) {
    if (a.s.share > 1) {
        switch (a.s.share) {
            case 2: return bounds_units<D, 2>(a, st);
            case 3: return bounds_units<D, 3>(a, st);
            case 4: return bounds_units<D, 4>(a, st);
            case 5: return bounds_units<D, 5>(a, st);
            case 6: return bounds_units<D, 6>(a, st);
            case 7: return bounds_units<D, 7>(a, st);
            default: return bounds_units<D, 8>(a, st);
        }
    }
    switch (a.s.G) {
        case 1: return bounds_g<D, 1>(a, st);
        case 2: return bounds_g<D, 2>(a, st);
        case 3: return bounds_g<D, 3>(a, st);
        case 4: return bounds_g<D, 4>(a, st);
        case 5: return bounds_g<D, 5>(a, st);
        case 6: return bounds_g<D, 6>(a, st);
        case 7: return bounds_g<D, 7>(a, st);
        default: return bounds_g<D, 8>(a, st);
    }
}

}  // namespace

hipError_t launch_qprep(const DecodeArgs& a, hipStream_t st) {
    ProjectArgs p{};
    p.queries = true;
    p.Q = a.Q;
    p.R = a.R;
    p.W = a.W;
    p.q_rot = reinterpret_cast<float*>(a.ws + a.lay.q_rot);
    p.code_q = reinterpret_cast<uint64_t*>(a.ws + a.lay.code_q);
    p.code_qm = reinterpret_cast<uint64_t*>(a.ws + a.lay.code_qm);
    p.q_split = reinterpret_cast<double*>(a.ws + a.lay.q_split);
    p.counters = reinterpret_cast<uint32_t*>(a.ws + a.lay.counters);
    p.n_counters = a.lay.n_clear;
    p.qmean = a.s.ham_mean;
    return launch_project(a.sd, p, st);  // per KV head of the cache
}

hipError_t launch_page_bounds(const DecodeArgs& a, hipStream_t st) {
    return a.s.D == 64 ? bounds_d<64>(a, st) : bounds_d<128>(a, st);
}

}  // namespace hhr
