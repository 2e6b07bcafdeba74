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
// and every such product is exact in fp64.  q_split is uniform across the
// block (scalar loads).
//
// The order of the sum ties each page to one lane, so a launch has one wave
// per SIMD at 64K pages; the stream stays busy because every lane keeps the
// next batch of U 16-byte loads in flight while it sums the current one.  The
// loads carry the nontemporal hint: every metadata line is read once.  The
// query terms are staged once per block in LDS and read as broadcasts.
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

template <int D, int G, int U, bool M16, bool PGMIN>
__global__ __launch_bounds__(256) void page_bound_kernel(const float* __restrict__ meta,
                                                         const double* __restrict__ q_split,
                                                         const int32_t* __restrict__ seq_len,
                                                         double* __restrict__ score, int Hkv, int T, int P,
                                                         int64_t NPB, int64_t NPmax, int share) {
    constexpr int NJ = M16 ? D / 4 : D / 2;  // 16-byte slots per page
    static_assert(NJ % U == 0, "batches");
    using V4 = typename std::conditional<M16, uint4, float4>::type;
    __shared__ double2 qs[D * G];  // (max(q,0), min(q,0)) per dimension and query head
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int64_t NP = n_pages_of(L, P);
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if ((int64_t)blockIdx.x * 256 >= NP) return;  // block-uniform

    const double2* qg = reinterpret_cast<const double2*>(q_split) + bh * D * G;
    for (int x = threadIdx.x; x < D * G; x += 256) qs[x] = qg[x];
    __syncthreads();
    if (p >= NP) return;

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
    const dim3 grid((unsigned)((s.NPmax + 255) / 256), s.Hkv, s.B);
    // Loads per lane per batch (two batches in flight), measured best per metadata type.
    auto kern = s.meta16 ? (s.pg_min ? page_bound_kernel<D, G, 8, true, true> : page_bound_kernel<D, G, 8, true, false>)
                         : (s.pg_min ? page_bound_kernel<D, G, 4, false, true> : page_bound_kernel<D, G, 4, false, false>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a.meta,
                       reinterpret_cast<const double*>(a.ws + a.lay.q_split), a.seq_len,
                       reinterpret_cast<double*>(a.ws + a.lay.score), s.Hkv, s.T, s.P, s.NPB, s.NPmax,
                       s.share);
    return hipGetLastError();
}

template <int D>
hipError_t bounds_d(const DecodeArgs& a, hipStream_t st) {
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
    p.qs_unit = a.s.share > 1;
    return launch_project(a.sd, p, st);  // per KV head of the cache
}

hipError_t launch_page_bounds(const DecodeArgs& a, hipStream_t st) {
    return a.s.D == 64 ? bounds_d<64>(a, st) : bounds_d<128>(a, st);
}

}  // namespace hhr
