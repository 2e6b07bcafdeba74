// Gather attention over the keys HHR kept: for every query head i of a KV
// head's group, out_i = sum_t softmax_t(scale * q_i . k_t) v_t over the
// selected t ("HHR: Hierarchical Hash Retrieval for Efficient LLM
// Generation", Abstract: hash-based sparse attention computes exact
// attention on the retrieved keys).
//
// gfx950 mapping, built for latency at batch 1: grid (splits, Hkv, B); a
// block owns 128 consecutive entries of the KV head's selected list, each of
// its 4 waves 32 of them, and each 16-lane row of a wave 8 entries (entries
// e, e + 4, ..., e + 28).  A row reads a whole K or V row with one 16-byte
// load per lane (a wave instruction fetches 4 rows, fully coalesced), and
// every K and V load of the block is issued before any arithmetic.
//  scores: each lane dots its D/16 dimensions with the G queries, and four
//    DPP rotations within the row leave the full dot product in every lane;
//  softmax per row over its 8 keys, then the row accumulates p * v for its
//    D/16 dimensions;
//  the 16 row partials (o, m, l) of the block merge in LDS with a log-sum-exp
//    into the split's partial, and the last block of the KV head
//    (device-scope counter) merges all splits -- every partial load of a
//    round in flight at once, online rescaling across rounds -- writes out
//    and resets the counter.
#include "hhr_internal.h"

namespace hhr {
namespace {

constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Sum over the 16 lanes of a DPP row, returned to every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
    x += __int_as_float(dpp_i<kRowRor8, 0xf>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowRor4, 0xf>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowRor2, 0xf>(0, __float_as_int(x)));
    x += __int_as_float(dpp_i<kRowRor1, 0xf>(0, __float_as_int(x)));
    return x;
}

// Load this lane's D/16 elements of a K/V/Q row as raw 32-bit words.
template <int D, bool BF16>
__device__ __forceinline__ void load_slice(const void* base, int64_t row, int sub, uint32_t (&w)[BF16 ? D / 32 : D / 16]) {
    constexpr int NWD = BF16 ? D / 32 : D / 16;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(base) + row * (BF16 ? D / 2 : D) + sub * NWD;
    if constexpr (NWD == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x; w[1] = v.y;
    } else {
#pragma unroll
        for (int x = 0; x < NWD; x += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(p + x);
            w[x] = v.x; w[x + 1] = v.y; w[x + 2] = v.z; w[x + 3] = v.w;
        }
    }
}

template <int D, bool BF16>
__device__ __forceinline__ float slice_elem(const uint32_t* w, int d) {
    if (BF16) return __uint_as_float((d & 1) ? (w[d >> 1] & 0xffff0000u) : (w[d >> 1] << 16));
    return __uint_as_float(w[d]);
}

// Split partials cross XCDs, whose L2s are not coherent with each other.  They
// are written and read with relaxed agent-scope atomics (coherent per access)
// and each block waits for its own stores before it bumps the split counter,
// so no agent-scope fence -- a full L2 write-back per block -- is needed.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_agent2(const float* p) {
    const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
__device__ __forceinline__ float4 ld_agent4(const float* p) {
    const float2 a = ld_agent2(p), b = ld_agent2(p + 2);
    return make_float4(a.x, a.y, b.x, b.y);
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void attend_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                     const void* __restrict__ V, const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ k_eff, float* __restrict__ part_o,
                                                     float* __restrict__ part_ml, uint32_t* __restrict__ counters,
                                                     float* __restrict__ out, int Hq, int Hkv, int T, int top_k,
                                                     int n_splits, float scale) {
    constexpr int NI = 8;                     // entries per row
    constexpr int CH = 16 * NI;               // entries per block (4 waves x 4 rows)
    static_assert(CH == kAttnChunk, "split size");
    constexpr int DPL = D / 16;               // dimensions per lane
    constexpr int NWD = BF16 ? DPL / 2 : DPL; // 32-bit words per lane per row
    constexpr int NP = 16;                    // row partials per block
    constexpr int MAXS = 32;                  // splits merged per round by the last block
    __shared__ float wo[NP][G][D];
    __shared__ float wml[NP][G][2];
    __shared__ float cml[G][MAXS][2];
    __shared__ float lred[256];
    __shared__ int last_flag;

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, sub = lane & 15;
    const int rw = tid >> 4;                  // row of the block, 0..15
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;
    int keff = k_eff[bh];
    keff = keff < 0 ? 0 : (keff > top_k ? top_k : keff);
    const int e0 = split * CH + (rw >> 2) * (4 * NI) + (rw & 3);  // entries e0 + 4j

    // Indices, then every K and V load of the row.
    int t[NI];
    bool ok[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int e = e0 + 4 * j;
        ok[j] = e < keff;
        int tj = ok[j] ? sel[bh * top_k + e] : 0;
        tj = (tj < 0 || tj >= T) ? 0 : tj;
        t[j] = tj;
    }
    const int64_t kvb = bh * T;
    uint32_t kw[NI][NWD], vw[NI][NWD];
#pragma unroll
    for (int j = 0; j < NI; ++j) load_slice<D, BF16>(K, kvb + t[j], sub, kw[j]);
#pragma unroll
    for (int j = 0; j < NI; ++j) load_slice<D, BF16>(V, kvb + t[j], sub, vw[j]);
    float qv[G][DPL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        uint32_t qw[NWD];
        load_slice<D, BF16>(Q, q0 + i, sub, qw);
#pragma unroll
        for (int d = 0; d < DPL; ++d) qv[i][d] = slice_elem<D, BF16>(qw, d);
    }

    // Scores of the row's entries for the G heads.
    float sc[NI][G];
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float a = 0.f;
#pragma unroll
            for (int d = 0; d < DPL; ++d) a = __builtin_fmaf(qv[i][d], slice_elem<D, BF16>(kw[j], d), a);
            sc[j][i] = a;
        }
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int i = 0; i < G; ++i) sc[j][i] = row_sum16(sc[j][i]);

    // Row softmax and p * v over the row's entries.
    float m_i[G], l_i[G], o[G][DPL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < NI; ++j)
            if (ok[j]) mx = fmaxf(mx, sc[j][i] * scale);
        float l = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[i][d] = 0.f;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const float p = ok[j] ? __expf(sc[j][i] * scale - mx) : 0.f;
            l += p;
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[i][d] = __builtin_fmaf(p, slice_elem<D, BF16>(vw[j], d), o[i][d]);
        }
        m_i[i] = mx;
        l_i[i] = l;
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) wo[rw][i][sub * DPL + d] = o[i][d];
        if (sub == 0) {
            wml[rw][i][0] = m_i[i];
            wml[rw][i][1] = l_i[i];
        }
    }
    __syncthreads();

    // Merge the block's rows into this split's partial.
    const int blk_keys = keff - split * CH;
    if (blk_keys > 0) {
        for (int x = tid; x < G * D; x += 256) {
            const int i = x / D, d = x % D;
            float M = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < NP; ++r) M = fmaxf(M, wml[r][i][0]);
            float acc = 0.f, L = 0.f;
#pragma unroll
            for (int r = 0; r < NP; ++r) {
                const float f = wml[r][i][1] > 0.f ? __expf(wml[r][i][0] - M) : 0.f;
                acc = __builtin_fmaf(wo[r][i][d], f, acc);
                L = __builtin_fmaf(wml[r][i][1], f, L);
            }
            st_agent(part_o + ((q0 + i) * n_splits + split) * D + d, acc);
            if (d == 0) {
                st_agent(part_ml + ((q0 + i) * n_splits + split) * 2, M);
                st_agent(part_ml + ((q0 + i) * n_splits + split) * 2 + 1, L);
            }
        }
    }

    // The last block of this KV head merges the splits.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0)
        last_flag = __hip_atomic_fetch_add(&counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    (uint32_t)(n_splits - 1);
    __syncthreads();
    if (!last_flag) return;

    // Columns of 4 output floats; NGR groups of threads split the splits.
    const int used = (keff + CH - 1) / CH;
    constexpr int NC = G * D / 4, NGR = 256 / NC, NB = 16;  // NB: loads in flight per batch
    const int c = tid % NC, g = tid / NC, qi = c / (D / 4);
    const bool act = g < NGR;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float Lacc = 0.f, Mrun = -__builtin_inff();
    for (int s0 = 0; s0 < used; s0 += MAXS) {
        const int ns = used - s0 < MAXS ? used - s0 : MAXS;
        for (int x = tid; x < G * ns; x += 256) {
            const int i = x / ns, sI = x % ns;
            const float2 ml = ld_agent2(part_ml + ((q0 + i) * n_splits + s0 + sI) * 2);
            cml[i][sI][0] = ml.x;
            cml[i][sI][1] = ml.y;
        }
        __syncthreads();
        if (act) {
            float Mr = Mrun;
            for (int sI = 0; sI < ns; ++sI) Mr = fmaxf(Mr, cml[qi][sI][0]);
            const float f = Mrun == -__builtin_inff() ? 0.f : __expf(Mrun - Mr);
            acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
            Lacc *= f;
            Mrun = Mr;
            const float* po = part_o + ((q0 + qi) * n_splits + s0) * D + (c % (D / 4)) * 4;
            for (int b0 = g; b0 < ns; b0 += NB * NGR) {
                float4 v[NB];
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    const int sI = b0 + u * NGR;
                    v[u] = sI < ns ? ld_agent4(po + (int64_t)sI * D) : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    const int sI = b0 + u * NGR;
                    if (sI < ns && cml[qi][sI][1] > 0.f) {
                        const float w = __expf(cml[qi][sI][0] - Mr);
                        acc.x = __builtin_fmaf(v[u].x, w, acc.x);
                        acc.y = __builtin_fmaf(v[u].y, w, acc.y);
                        acc.z = __builtin_fmaf(v[u].z, w, acc.z);
                        acc.w = __builtin_fmaf(v[u].w, w, acc.w);
                        Lacc = __builtin_fmaf(cml[qi][sI][1], w, Lacc);
                    }
                }
            }
        }
        __syncthreads();
    }
    // Sum the groups and normalise.
    float4* red = reinterpret_cast<float4*>(&wo[0][0][0]);  // NGR * NC <= 16 * G * D / 4 float4
    if (act) {
        red[g * NC + c] = acc;
        lred[g * NC + c] = Lacc;
    }
    __syncthreads();
    if (act && g == 0) {
        for (int r = 1; r < NGR; ++r) {
            const float4 a = red[r * NC + c];
            acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
            Lacc += lred[r * NC + c];
        }
        const float inv = Lacc > 0.f ? 1.f / Lacc : 0.f;
        *reinterpret_cast<float4*>(out + (q0 + qi) * D + (c % (D / 4)) * 4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (tid == 0) __hip_atomic_store(&counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <int D, bool BF16, int G>
hipError_t attend_g(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    const dim3 grid(a.lay.n_splits, s.Hkv, s.B);
    float* po = reinterpret_cast<float*>(a.ws + a.lay.partial);
    float* pml = po + (size_t)s.B * s.Hq * a.lay.n_splits * s.D;
    hipLaunchKernelGGL((attend_kernel<D, BF16, G>), grid, dim3(256), 0, st, a.Q, a.K, a.V, a.sel,
                       reinterpret_cast<const int32_t*>(a.ws + a.lay.k_eff), po, pml,
                       reinterpret_cast<uint32_t*>(a.ws + a.lay.counters), a.out, s.Hq, s.Hkv, s.T, a.top_k,
                       a.lay.n_splits, a.scale);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t attend_dt(const DecodeArgs& a, hipStream_t st) {
    switch (a.s.G) {
        case 1: return attend_g<D, BF16, 1>(a, st);
        case 2: return attend_g<D, BF16, 2>(a, st);
        case 3: return attend_g<D, BF16, 3>(a, st);
        case 4: return attend_g<D, BF16, 4>(a, st);
        case 5: return attend_g<D, BF16, 5>(a, st);
        case 6: return attend_g<D, BF16, 6>(a, st);
        case 7: return attend_g<D, BF16, 7>(a, st);
        default: return attend_g<D, BF16, 8>(a, st);
    }
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t st) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_attend(const DecodeArgs& a, bool zero_counters, hipStream_t st) {
    if (zero_counters) {
        const hipError_t e = launch_zero_u32(reinterpret_cast<uint32_t*>(a.ws + a.lay.counters), a.s.B * a.s.Hkv, st);
        if (e != hipSuccess) return e;
    }
    const Shape& s = a.s;
    if (s.D == 64) return s.bf16 ? attend_dt<64, true>(a, st) : attend_dt<64, false>(a, st);
    return s.bf16 ? attend_dt<128, true>(a, st) : attend_dt<128, false>(a, st);
}

}  // namespace hhr
