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

// Max over the 16 lanes of a DPP row, returned to every lane of the row.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, __int_as_float(dpp_i<kRowRor8, 0xf>(0, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowRor4, 0xf>(0, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowRor2, 0xf>(0, __float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kRowRor1, 0xf>(0, __float_as_int(x))));
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
            const u32x4 v = load_stream16(p + x);  // a gathered row is read once
            w[x] = v.x; w[x + 1] = v.y; w[x + 2] = v.z; w[x + 3] = v.w;
        }
    }
}

typedef __bf16 __attribute__((ext_vector_type(2))) bf16x2;
typedef __bf16 __attribute__((ext_vector_type(8))) bf16x8;
typedef float __attribute__((ext_vector_type(4))) f32x4;

// Dot product of this lane's slices of a query and a key: bf16 pairs through
// the packed bf16 dot instruction with fp32 accumulation, fp32 by FMAs.
template <int D, bool BF16>
__device__ __forceinline__ float slice_dot(const uint32_t (&q)[BF16 ? D / 32 : D / 16],
                                           const uint32_t (&k)[BF16 ? D / 32 : D / 16]) {
    float a = 0.f;
    if constexpr (BF16) {
#pragma unroll
        for (int w = 0; w < D / 32; ++w)
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q[w]), __builtin_bit_cast(bf16x2, k[w]), a,
                                                false);
    } else {
#pragma unroll
        for (int d = 0; d < D / 16; ++d) a = __builtin_fmaf(__uint_as_float(q[d]), __uint_as_float(k[d]), a);
    }
    return a;
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

constexpr int kMergeRound = 32;  // split partials merged per round by the last block

// NR partials (16-lane rows, or waves) of a block of NT threads.
template <int D, int G, int NR = 16, int NT = NR * 16>
struct alignas(16) AttnShared {
    static constexpr int kWo = NR * G * D > 4 * NT ? NR * G * D : 4 * NT;
    float wo_[kWo];         // partials (o) [NR][G][D], reused by the final reduction (NT float4)
    float wml[NR][G][2];    // partials (m, l)
    float cml[G][kMergeRound][2];
    float lred[NT];
    __device__ __forceinline__ float* wo(int r, int i) { return wo_ + (r * G + i) * D; }
    float fr[NR][G];        // row weights exp(m_r - M) of the block combine
    float bml[G][2];        // block (M, L) per query head
    int last_flag;
};

// A row's partial o of query head i into sh.wo[rw][i]: lane `sub` owns the
// DPL = D / 16 dimensions [sub * DPL, sub * DPL + DPL).  With DPL = 8 a lane's
// 32 bytes go out as two 16-byte stores; written in the same order by every
// lane, lanes 4 (and 8) apart -- and the rows of a wave, 2 KB apart at G = 4 --
// would hit the same LDS banks in each store.  Lanes whose bit 2 of `sub`
// differs from bit 3 store their upper half first, so within every 8 and every
// 16 consecutive lanes a store's addresses cover distinct banks.  The stored
// layout is unchanged; only which store carries which half differs.
template <int D, int G, int NR, int NT, int DPL>
__device__ __forceinline__ void store_row_o(AttnShared<D, G, NR, NT>& sh, int rw, int sub, const float (&o)[G][DPL]) {
    if constexpr (DPL == 8) {
        const bool hi_first = ((sub >> 2) ^ (sub >> 3)) & 1;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float a[4], c[4];  // the first and the second store's values, selected per component
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                a[d] = hi_first ? o[i][4 + d] : o[i][d];
                c[d] = hi_first ? o[i][d] : o[i][4 + d];
            }
            float* base = sh.wo(rw, i) + sub * DPL;
            *reinterpret_cast<float4*>(base + (hi_first ? 4 : 0)) = make_float4(a[0], a[1], a[2], a[3]);
            *reinterpret_cast<float4*>(base + (hi_first ? 0 : 4)) = make_float4(c[0], c[1], c[2], c[3]);
        }
    } else if constexpr (DPL == 4) {  // 16 bytes a lane: consecutive lanes, consecutive 16-byte slots
#pragma unroll
        for (int i = 0; i < G; ++i)
            *reinterpret_cast<float4*>(sh.wo(rw, i) + sub * DPL) = make_float4(o[i][0], o[i][1], o[i][2], o[i][3]);
    } else {
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int d = 0; d < DPL; ++d) sh.wo(rw, i)[sub * DPL + d] = o[i][d];
    }
}

// Log-sum-exp weights of the block's NR row partials: per query head i,
// M_i = max_r m_r, f_r = exp(m_r - M_i) (0 for a row without keys) and
// L_i = sum_r f_r l_r, one thread per (i, r) with butterflies over the rows
// (NR is a power of two, so a row group never straddles a wave).  Every
// thread of the block calls it, after a barrier that follows the row writes.
template <int D, int G, int NR, int NT>
__device__ __forceinline__ void row_weights(AttnShared<D, G, NR, NT>& sh) {
    static_assert((NR & (NR - 1)) == 0 && NR <= 64, "row groups within a wave");
    const int tid = threadIdx.x;
    if (tid < G * NR) {
        const int i = tid / NR, r = tid % NR;
        const float m = sh.wml[r][i][0], l = sh.wml[r][i][1];
        float M = m;
#pragma unroll
        for (int o = NR / 2; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float f = l > 0.f ? __expf(m - M) : 0.f;
        float L = f * l;
#pragma unroll
        for (int o = NR / 2; o > 0; o >>= 1) L += __shfl_xor(L, o);
        sh.fr[r][i] = f;
        if (r == 0) {
            sh.bml[i][0] = M;
            sh.bml[i][1] = L;
        }
    }
    __syncthreads();
}

// The NT / 16 row partials of a block (m, l, o per query head, in LDS) merge
// with a log-sum-exp into the block's split partial, published with
// agent-scope stores; the last block of the (b, h) to finish merges the
// `used` splits and writes out.  `stride`: splits per query head in the
// partial arrays; `nblocks`: blocks that report to the counter.  Every thread
// of the block calls it, after a barrier that follows the row writes.
template <int D, int G, int NT = 256>
__device__ __forceinline__ void merge_splits(AttnShared<D, G, NT / 16>& sh, bool has_keys, int split, int stride,
                                             int nblocks, int used, int64_t q0, float* __restrict__ part_o,
                                             float* __restrict__ part_ml, uint32_t* __restrict__ counter,
                                             float* __restrict__ out) {
    constexpr int NP = NT / 16;
    const int tid = threadIdx.x;
    row_weights(sh);
    if (has_keys) {
        for (int x = tid; x < G * D; x += NT) {
            const int i = x / D, d = x % D;
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < NP; ++r) acc = __builtin_fmaf(sh.wo(r, i)[d], sh.fr[r][i], acc);
            st_agent(part_o + ((q0 + i) * stride + split) * D + d, acc);
            if (d == 0) {
                st_agent(part_ml + ((q0 + i) * stride + split) * 2, sh.bml[i][0]);
                st_agent(part_ml + ((q0 + i) * stride + split) * 2 + 1, sh.bml[i][1]);
            }
        }
    }

    // The last block of this KV head merges the splits.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0)
        sh.last_flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                       (uint32_t)(nblocks - 1);
    __syncthreads();
    if (!sh.last_flag) return;

    // Columns of 4 output floats; NGR groups of threads split the splits.
    constexpr int NC = G * D / 4, NGR = NT / NC, NB = 16;  // NB: loads in flight per batch
    const int c = tid % NC, g = tid / NC, qi = c / (D / 4);
    const bool act = g < NGR;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float Lacc = 0.f, Mrun = -__builtin_inff();
    for (int s0 = 0; s0 < used; s0 += kMergeRound) {
        const int ns = used - s0 < kMergeRound ? used - s0 : kMergeRound;
        const float* po = part_o + ((q0 + qi) * stride + s0) * D + (c % (D / 4)) * 4;
        // The round's (m, l) and the first batch of partials are loaded together.
        float2 ml[(G * kMergeRound + NT - 1) / NT];
#pragma unroll
        for (int r = 0; r < (G * kMergeRound + NT - 1) / NT; ++r) {
            const int x = tid + r * NT;
            const int i = x / ns, sI = x % ns;
            ml[r] = x < G * ns ? ld_agent2(part_ml + ((q0 + i) * stride + s0 + sI) * 2) : make_float2(0.f, 0.f);
        }
        float4 v[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int sI = g + u * NGR;
            v[u] = act && sI < ns ? ld_agent4(po + (int64_t)sI * D) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int r = 0; r < (G * kMergeRound + NT - 1) / NT; ++r) {
            const int x = tid + r * NT;
            if (x < G * ns) {
                sh.cml[x / ns][x % ns][0] = ml[r].x;
                sh.cml[x / ns][x % ns][1] = ml[r].y;
            }
        }
        __syncthreads();
        if (act) {
            float Mr = Mrun;
            for (int sI = 0; sI < ns; ++sI) Mr = fmaxf(Mr, sh.cml[qi][sI][0]);
            const float f = Mrun == -__builtin_inff() ? 0.f : __expf(Mrun - Mr);
            acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
            Lacc *= f;
            Mrun = Mr;
            for (int b0 = g; b0 < ns; b0 += NB * NGR) {
                if (b0 != g) {  // later batches (more splits per thread than NB)
#pragma unroll
                    for (int u = 0; u < NB; ++u) {
                        const int sI = b0 + u * NGR;
                        v[u] = sI < ns ? ld_agent4(po + (int64_t)sI * D) : make_float4(0.f, 0.f, 0.f, 0.f);
                    }
                }
#pragma unroll
                for (int u = 0; u < NB; ++u) {
                    const int sI = b0 + u * NGR;
                    if (sI < ns && sh.cml[qi][sI][1] > 0.f) {
                        const float w = __expf(sh.cml[qi][sI][0] - Mr);
                        acc.x = __builtin_fmaf(v[u].x, w, acc.x);
                        acc.y = __builtin_fmaf(v[u].y, w, acc.y);
                        acc.z = __builtin_fmaf(v[u].z, w, acc.z);
                        acc.w = __builtin_fmaf(v[u].w, w, acc.w);
                        Lacc = __builtin_fmaf(sh.cml[qi][sI][1], w, Lacc);
                    }
                }
            }
        }
        __syncthreads();
    }
    // Sum the groups and normalise.
    float4* red = reinterpret_cast<float4*>(sh.wo_);  // NGR * NC <= NT float4
    if (act) {
        red[g * NC + c] = acc;
        sh.lred[g * NC + c] = Lacc;
    }
    __syncthreads();
    if (act && g == 0) {
        for (int r = 1; r < NGR; ++r) {
            const float4 a = red[r * NC + c];
            acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
            Lacc += sh.lred[r * NC + c];
        }
        const float inv = Lacc > 0.f ? 1.f / Lacc : 0.f;
        *reinterpret_cast<float4*>(out + (q0 + qi) * D + (c % (D / 4)) * 4) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
}

// Split merge of the compact+attend kernel.  Every block publishes its
// split partial with agent-scope stores and, unless it is the merger, is
// done: no store wait, no counter round trip.  The merger is the block that
// took the head's last start ticket, so every block it waits for has
// already started.  It loads all S partials and repeats the loads until none
// still holds the sentinel the select kernel wrote for this step (each
// 32-bit word is written once, so a word that is not the sentinel is final),
// then merges them as merge_splits does.  The wait is bounded: after
// kMaxPolls rounds the head's outputs are set to NaN rather than hang.
constexpr int kMaxPolls = 1 << 20;

template <int D, int G, int NT, int NP>
__device__ __forceinline__ void merge_polled(AttnShared<D, G, NP, NT>& sh, int split, int stride, int S,
                                             int64_t q0, float* __restrict__ part_o, float* __restrict__ part_ml,
                                             float* __restrict__ out) {
    const int tid = threadIdx.x;
    row_weights(sh);
    for (int x = tid; x < G * D; x += NT) {
        const int i = x / D, d = x % D;
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < NP; ++r) acc = __builtin_fmaf(sh.wo(r, i)[d], sh.fr[r][i], acc);
        st_agent(part_o + ((q0 + i) * stride + split) * D + d, acc);
        if (d == 0) {
            st_agent(part_ml + ((q0 + i) * stride + split) * 2, sh.bml[i][0]);
            st_agent(part_ml + ((q0 + i) * stride + split) * 2 + 1, sh.bml[i][1]);
        }
    }
    if (!sh.last_flag) return;

    // Columns of 4 output floats; NGR groups of threads split the splits, NB
    // loads each per round, so one batch covers a round of RND splits.  At
    // most 8 loads a thread keep the polling loop's addresses in registers.
    constexpr int NC = G * D / 4, NGR = NT / NC;
    constexpr int NB = (kMergeRound + NGR - 1) / NGR < 8 ? (kMergeRound + NGR - 1) / NGR : 8;
    constexpr int RND = NB * NGR < kMergeRound ? NB * NGR : kMergeRound;
    static_assert(NGR >= 1 && NB * NGR >= RND, "one batch per merge round");
    constexpr int NML = (G * RND + NT - 1) / NT;
    const int c = tid % NC, g = tid / NC, qi = c / (D / 4);
    const bool act = g < NGR;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float Lacc = 0.f, Mrun = -__builtin_inff();
    bool failed = false;
    for (int s0 = 0; s0 < S && !failed; s0 += RND) {
        const int ns = S - s0 < RND ? S - s0 : RND;
        const float* po = part_o + ((q0 + qi) * stride + s0) * D + (c % (D / 4)) * 4;
        float2 ml[NML];
        float4 v[NB];
        for (int poll = 0;; ++poll) {
            bool pending = false;
#pragma unroll
            for (int r = 0; r < NML; ++r) {
                const int x = tid + r * NT;
                const int i = x / ns, sI = x % ns;
                ml[r] = x < G * ns ? ld_agent2(part_ml + ((q0 + i) * stride + s0 + sI) * 2) : make_float2(0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int sI = g + u * NGR;
                v[u] = act && sI < ns ? ld_agent4(po + (int64_t)sI * D) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int r = 0; r < NML; ++r)
                pending |= __float_as_uint(ml[r].x) == kPartSentinel || __float_as_uint(ml[r].y) == kPartSentinel;
#pragma unroll
            for (int u = 0; u < NB; ++u)
                pending |= __float_as_uint(v[u].x) == kPartSentinel || __float_as_uint(v[u].y) == kPartSentinel ||
                           __float_as_uint(v[u].z) == kPartSentinel || __float_as_uint(v[u].w) == kPartSentinel;
            if (!__syncthreads_or(pending)) break;
            if (poll >= kMaxPolls) {
                failed = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (failed) break;
#pragma unroll
        for (int r = 0; r < NML; ++r) {
            const int x = tid + r * NT;
            if (x < G * ns) {
                sh.cml[x / ns][x % ns][0] = ml[r].x;
                sh.cml[x / ns][x % ns][1] = ml[r].y;
            }
        }
        __syncthreads();
        if (act) {
            float Mr = Mrun;
            for (int sI = 0; sI < ns; ++sI) Mr = fmaxf(Mr, sh.cml[qi][sI][0]);
            const float f = Mrun == -__builtin_inff() ? 0.f : __expf(Mrun - Mr);
            acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
            Lacc *= f;
            Mrun = Mr;
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int sI = g + u * NGR;
                if (sI < ns && sh.cml[qi][sI][1] > 0.f) {
                    const float w = __expf(sh.cml[qi][sI][0] - Mr);
                    acc.x = __builtin_fmaf(v[u].x, w, acc.x);
                    acc.y = __builtin_fmaf(v[u].y, w, acc.y);
                    acc.z = __builtin_fmaf(v[u].z, w, acc.z);
                    acc.w = __builtin_fmaf(v[u].w, w, acc.w);
                    Lacc = __builtin_fmaf(sh.cml[qi][sI][1], w, Lacc);
                }
            }
        }
        __syncthreads();
    }
    // Sum the groups and normalise.
    float4* red = reinterpret_cast<float4*>(sh.wo_);  // NGR * NC <= NT float4
    if (act) {
        red[g * NC + c] = acc;
        sh.lred[g * NC + c] = Lacc;
    }
    __syncthreads();
    if (act && g == 0) {
        for (int r = 1; r < NGR; ++r) {
            const float4 a = red[r * NC + c];
            acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
            Lacc += sh.lred[r * NC + c];
        }
        const float inv = Lacc > 0.f ? 1.f / Lacc : 0.f;
        const float nan = __builtin_nanf("");
        *reinterpret_cast<float4*>(out + (q0 + qi) * D + (c % (D / 4)) * 4) =
            failed ? make_float4(nan, nan, nan, nan)
                   : make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void attend_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                     const void* __restrict__ V, const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ k_eff, float* __restrict__ part_o,
                                                     float* __restrict__ part_ml, uint32_t* __restrict__ counters,
                                                     float* __restrict__ out, int Hq, int Hkv, int T, int top_k,
                                                     int n_splits, int stride, float scale, int share) {
    constexpr int NI = 8;                     // entries per row
    constexpr int CH = 16 * NI;               // entries per block (4 waves x 4 rows)
    static_assert(CH == kAttnChunk, "split size");
    constexpr int DPL = D / 16;               // dimensions per lane
    constexpr int NWD = BF16 ? DPL / 2 : DPL; // 32-bit words per lane per row
    __shared__ AttnShared<D, G> sh;

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
    const int64_t kvb = data_head(b, h, Hkv, share) * T;  // rows of the unit's data head
    uint32_t kw[NI][NWD], vw[NI][NWD];
#pragma unroll
    for (int j = 0; j < NI; ++j) load_slice<D, BF16>(K, kvb + t[j], sub, kw[j]);
#pragma unroll
    for (int j = 0; j < NI; ++j) load_slice<D, BF16>(V, kvb + t[j], sub, vw[j]);
    uint32_t qw[G][NWD];  // this lane's slice of each query, raw
#pragma unroll
    for (int i = 0; i < G; ++i) load_slice<D, BF16>(Q, q0 + i, sub, qw[i]);

    // Scores of the row's entries for the G heads.
    float sc[NI][G];
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int i = 0; i < G; ++i) {
            sc[j][i] = slice_dot<D, BF16>(qw[i], kw[j]);
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
    store_row_o(sh, rw, sub, o);
    if (sub == 0) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            sh.wml[rw][i][0] = m_i[i];
            sh.wml[rw][i][1] = l_i[i];
        }
    }
    __syncthreads();

    merge_splits<D, G>(sh, keff - split * CH > 0, split, stride, n_splits, (keff + CH - 1) / CH, q0, part_o,
                       part_ml, counters + bh, out);
}

// ------------------------------------------------------------------ compact + attend
// The decode step's tail when the Hamming scan ran as S blocks per (b, h):
// block j owns candidate slots [j*per, (j+1)*per) and
//  - finds the head's threshold h* (the k_eff-th smallest distance) from the
//    head histogram, and how many of the keys at h* earlier blocks take (the
//    first `need` in slot order win ties) from their cumulative histograms;
//  - compacts its own selected keys, in slot order (ascending key index),
//    into sel at its offset and into an LDS list;
//  - runs gather attention over that list and merges with the other blocks
//    as above.  bf16 K/V: the scores come from the matrix cores, 16 keys per
//    wave per instruction group, the weights reach half-wave rows through
//    LDS for the fp32 weight x V sums, and each wave leaves one partial;
//    fp32 K/V: 16-lane rows with online softmax over batches of 16 * NI
//    keys, one partial per row.
constexpr int kCompactThreads = 512;

template <int D, bool BF16, int G>
__global__ __launch_bounds__(kCompactThreads) __attribute__((amdgpu_waves_per_eu(BF16 ? 4 : 2))) void compact_attend_kernel(
    const void* __restrict__ Q, const void* __restrict__ K, const void* __restrict__ V,
    const int32_t* __restrict__ pages, const int32_t* __restrict__ n_pages, const uint16_t* __restrict__ ham,
    const uint32_t* __restrict__ cum, const uint32_t* __restrict__ ghist, const int32_t* __restrict__ seq_len,
    int32_t* __restrict__ sel, int32_t* __restrict__ k_eff_out, float* __restrict__ part_o,
    float* __restrict__ part_ml, uint32_t* __restrict__ counters, float* __restrict__ out, int Hq, int Hkv, int T,
    int P, int max_keep, int top_k, int S, int stride, int nbins, float scale, int share, int nsink, int window) {
    constexpr int NT = kCompactThreads;
    constexpr int NR = NT / 16;               // 16-lane rows
    constexpr int SPT = kCompactSlots / NT;   // slots per thread
    constexpr int BPT = (1025 + NT - 1) / NT; // histogram bins per thread (nbins <= 1025)
    constexpr int NI = G <= 4 ? 8 : 4;        // entries per row per batch
    constexpr int DPL = D / 16;
    constexpr int NWD = BF16 ? DPL / 2 : DPL;
    constexpr uint16_t kNoKey = 0xFFFF;
    // Partials per wave with bf16 K/V (the rows of a wave share its running max), else per 16-lane row.
    __shared__ AttnShared<D, G, (BF16 ? NT / 64 : NR), NT> sh;
    __shared__ alignas(16) uint16_t hs[kCompactSlots];
    __shared__ alignas(16) int ts[kCompactSlots];
    __shared__ int list[kCompactSlots];
    __shared__ int scan[16];
    __shared__ int thr[2];
    __shared__ int offs[3];

    // Same grid order as the select kernels, (Hkv, B, S): a block lands on the XCD whose L2 holds the
    // slots and histograms the select block of the same (head, split) wrote.
    const int b = blockIdx.y, split = blockIdx.z;
    // Per-query-head selection: the units of one data head take the grid
    // slots of that head's XCD (workgroups go to the XCDs in turn), where its
    // page-bound pass left their scores.
    int h = blockIdx.x;
    if (share > 1) {  // block-uniform
        const unsigned Hd = (unsigned)(Hkv / share);
        h = (int)((blockIdx.x % Hd) * (unsigned)share + blockIdx.x / Hd);
    }
    const int tid = threadIdx.x, lane = tid & 63, sub = lane & 15, rw = tid >> 4;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;
    int np = n_pages[bh];
    np = np < 0 ? 0 : (np > max_keep ? max_keep : np);
    const int nslots = np * P, lp = 31 - __clz(P);
    const int per = (nslots + S - 1) / S;
    const int lo = split * per < nslots ? split * per : nslots;
    const int hi = lo + per < nslots ? lo + per : nslots;
    const int nmine = hi - lo;  // <= kCompactSlots (the split count is chosen so)
    const uint16_t* hm = ham + bh * (int64_t)max_keep * P;
    const int32_t* pl = pages + bh * (int64_t)max_keep;

    // Every load of the head histogram and of this block's slots, then use.
    uint32_t gh[BPT];
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
        const int bn = tid * BPT + r;
        gh[r] = ghist[bh * nbins + (bn < nbins ? bn : 0)];
    }
    uint16_t hk[SPT];
    int pk[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int s = lo + k * NT + tid;
        const int ss = s < hi ? s : 0;
        hk[k] = hm[ss];
        pk[k] = pl[ss >> lp];
    }
    // Start ticket of the head (the count is cleared by the step's query
    // prep); the block that draws S - 1 merges the splits.  The result is
    // only used at the end: the address carries the lane's mbcnt (0 for lane
    // 0) so the compiler does not turn it into a wave-aggregated atomic whose
    // result it reads back at once, which would stall the wave for the whole
    // device-scope round trip here.  The last wave takes it: its next wait on
    // memory is the K/V gather, by when the atomic has returned (wave 0 waits
    // earlier, on the cumulative histograms).
    uint32_t ticket = 0;
    if (tid == NT - 64)
        ticket = __hip_atomic_fetch_add(counters + bh + __builtin_amdgcn_mbcnt_lo(~0u, 0u), 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
        thr[0] = nbins;
        thr[1] = 0;
    }
    int sum = 0;
#pragma unroll
    for (int r = 0; r < BPT; ++r)
        if (tid * BPT + r < nbins) sum += (int)gh[r];
    int nvalid;
    int run = block_excl_scan<NT, false>(sum, scan, nvalid);
    const int keff = nvalid < top_k ? nvalid : top_k;
#pragma unroll
    for (int r = 0; r < BPT; ++r) {
        const int bn = tid * BPT + r;
        const int c = bn < nbins ? (int)gh[r] : 0;
        if (keff > 0 && run < keff && run + c >= keff) {
            thr[0] = bn;
            thr[1] = keff - run;
        }
        run += c;
    }
    // Stage this block's slots (distance, key) in slot order.
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        const int s = lo + k * NT + tid;
        if (s < hi) {
            hs[s - lo] = hk[k];
            ts[s - lo] = pk[k] * P + (s & (P - 1));
        }
    }
    __syncthreads();
    const int hstar = thr[0], need = thr[1];

    // Earlier blocks' counts below and at h* (one lane per block, S <= 64):
    // both loads of every lane issued before either is used.
    if (tid < 64) {
        const int i = tid <= split ? tid : split;
        const uint32_t* ci = cum + (bh * S + i) * (int64_t)nbins;
        const int ib = hstar <= 0 ? 0 : (hstar < nbins ? hstar - 1 : nbins - 1), ia = hstar < nbins ? hstar : 0;
        const uint32_t c_at = ci[ia], c_below = ci[ib];
        const int below = hstar > 0 ? (int)c_below : 0;
        const int at = hstar < nbins ? (int)c_at - below : 0;
        int lt = 0, eq = 0, own_eq = 0;
        if (tid < split) {
            lt = below;
            eq = at;
        } else if (tid == split) {
            own_eq = at;
        }
        lt = wave_incl_scan(lt);
        eq = wave_incl_scan(eq);
        own_eq = wave_incl_scan(own_eq);
        if (tid == 63) {
            offs[0] = lt;
            offs[1] = eq;
            offs[2] = own_eq;
        }
    }
    __syncthreads();
    const int E = offs[1], own_eq = offs[2];
    const int offset = offs[0] + (need < E ? need : E);
    int incl = need - E;
    incl = incl < 0 ? 0 : (incl > own_eq ? own_eq : incl);

    // Ordered compaction of this block's slots (thread tid: slots [tid*SPT, tid*SPT + SPT)),
    // read as one 8-byte and one 16-byte LDS load per thread (consecutive threads, consecutive
    // addresses: no bank conflicts, where per-slot loads would be 8 and 16 bytes apart).
    static_assert(SPT == 4, "slot reads sized for 4 slots per thread");
    uint16_t hv[SPT];
    int tv[SPT];
    int n_lt = 0, n_eq = 0;
    {
        const uint2 hw = *reinterpret_cast<const uint2*>(&hs[tid * SPT]);
        const int4 tw = *reinterpret_cast<const int4*>(&ts[tid * SPT]);
        hv[0] = (uint16_t)hw.x;
        hv[1] = (uint16_t)(hw.x >> 16);
        hv[2] = (uint16_t)hw.y;
        hv[3] = (uint16_t)(hw.y >> 16);
        tv[0] = tw.x;
        tv[1] = tw.y;
        tv[2] = tw.z;
        tv[3] = tw.w;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const bool mine = tid * SPT + k < nmine;
            hv[k] = mine ? hv[k] : kNoKey;
            tv[k] = mine ? tv[k] : 0;
            n_lt += hv[k] < hstar;
            n_eq += hv[k] == hstar;
        }
    }
    int tot;
    const int packed = block_excl_scan<NT, false>((n_lt << 16) | n_eq, scan, tot);
    int eq_rank = packed & 0xffff;
    int pos = (packed >> 16) + (eq_rank < incl ? eq_rank : incl);
    // Forced keys (sink tokens, local window): [0, s_end) and [w_start, L),
    // listed around the ranked ones; block 0 also attends them.
    const int L = clamp_len(seq_len[b], T);
    const int s_end = nsink < L ? nsink : L;
    const int w_start = L - window > s_end ? L - window : s_end;
    const int nforced = s_end + (L - w_start);
    int32_t* so = sel + bh * ((int64_t)top_k + nsink + window);
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
        bool in = hv[k] < hstar;
        if (hv[k] == hstar) {
            in = eq_rank < incl;
            ++eq_rank;
        }
        if (in) {
            if (offset + pos < top_k) so[s_end + offset + pos] = tv[k];
            list[pos] = tv[k];
            ++pos;
        }
    }
    int cnt = (tot >> 16) + ((tot & 0xffff) < incl ? (tot & 0xffff) : incl);
    if (split == 0) {
        const int listed = keff + nforced;
        for (int j = tid; j < s_end; j += NT) so[j] = j;
        for (int j = tid; j < L - w_start; j += NT) so[s_end + keff + j] = w_start + j;
        for (int j = listed + tid; j < top_k + nsink + window; j += NT) so[j] = -1;
        for (int j = tid; j < nforced && cnt + j < kCompactSlots; j += NT)
            list[cnt + j] = j < s_end ? j : w_start + (j - s_end);
        cnt = cnt + nforced < kCompactSlots ? cnt + nforced : kCompactSlots;  // the layout keeps it in range
        if (tid == 0) k_eff_out[bh] = listed;
    }
    __syncthreads();

    const int64_t kvb = data_head(b, h, Hkv, share) * T;  // rows of the unit's data head
    float m_i[G], l_i[G], o[G][DPL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        m_i[i] = -__builtin_inff();
        l_i[i] = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[i][d] = 0.f;
    }
    if constexpr (BF16) {
        // Scores on the matrix cores.  Each wave takes groups of 16 consecutive entries; one
        // v_mfma_f32_16x16x32_bf16 per 32 dimensions multiplies the queries (A: row i = head i, zero rows
        // past G) by the gathered keys (B: column j = key j) into S[head 4 (l / 16) + r][key l % 16], held
        // in component r of lane l.  Lane l supplies dimensions 32 s + 8 (l / 16) + [0, 8) of slice s, so
        // the four lanes of a key read 64 contiguous bytes per slice; the queries use the same permutation
        // of the dimensions, which leaves every dot product unchanged.  bf16 products are exact and the
        // sums fp32, as in the dot-product path.  The online softmax runs in that layout (row maxima and
        // sums over the 16 keys by DPP).  The weights go through a per-wave LDS tile [key][head] -- the
        // slot staging array, free after the compaction -- to the weight x V sums, where each half-wave
        // covers a V row (D / 32 dimensions a lane) and takes 8 of the group's keys: half h takes keys
        // h, h + 2, ..., h + 14.  A lane thus holds G x D / 32 accumulators, which leaves room for two
        // blocks per compute unit.
        constexpr int KS = D / 32;
        constexpr int DPW = D / 32;                  // dimensions per lane in the weight x V sums
        constexpr int NGRP = 1;                      // groups per wave per batch
        constexpr int STEP = (NT / 64) * 16 * NGRP;  // entries per block per batch
        static_assert(D % 32 == 0 && G <= 8, "score tiles hold 8 heads");
        static_assert(sizeof(ts) >= (NT / 64) * NGRP * 16 * 8 * sizeof(float), "weight tiles fit the staging array");
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const int wv = tid >> 6, gq = lane >> 4, ln = lane & 15, hw = lane >> 5, hl = lane & 31;
        float* pt = reinterpret_cast<float*>(ts) + wv * (NGRP * 16 * 8);  // [group][key][8 heads]
        bf16x8 qa[KS];
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
            u32x4 w = {0u, 0u, 0u, 0u};
            if (ln < G)
                w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(Q) + (q0 + ln) * D + sl * 32 + 8 * gq);
            qa[sl] = __builtin_bit_cast(bf16x8, w);
        }
        float mr[4], lr[4];  // running max and (per-lane part of the) weight sum of heads 4 gq + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            mr[r] = -__builtin_inff();
            lr[r] = 0.f;
        }
        float ow[G][DPW];  // this lane's dimensions [hl * DPW, hl * DPW + DPW) of the half-wave's outputs
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int d = 0; d < DPW; ++d) ow[i][d] = 0.f;
        for (int e0 = 0; e0 < cnt; e0 += STEP) {
            int tk[NGRP], tv[NGRP][8];
            bool okk[NGRP];
#pragma unroll
            for (int g = 0; g < NGRP; ++g) {
                const int eb = e0 + (g * (NT / 64) + wv) * 16;
                okk[g] = eb + ln < cnt;
                const int t = list[okk[g] ? eb + ln : 0];
                tk[g] = (t < 0 || t >= L) ? 0 : t;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int ev = eb + hw + 2 * q;
                    const int u = list[ev < cnt ? ev : 0];
                    tv[g][q] = (u < 0 || u >= L) ? 0 : u;
                }
            }
            u32x4 kb[NGRP][KS];
            uint32_t vw[NGRP][8][DPW / 2];
#pragma unroll
            for (int g = 0; g < NGRP; ++g)
#pragma unroll
                for (int sl = 0; sl < KS; ++sl)
                    kb[g][sl] = load_stream16(static_cast<const uint16_t*>(K) + (kvb + tk[g]) * D + sl * 32 + 8 * gq);
#pragma unroll
            for (int g = 0; g < NGRP; ++g)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t* vp = static_cast<const uint32_t*>(V) + (kvb + tv[g][q]) * (D / 2) + hl * (DPW / 2);
                    if constexpr (DPW == 4) {
                        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vp));
                        vw[g][q][0] = v.x;
                        vw[g][q][1] = v.y;
                    } else {
                        vw[g][q][0] = __builtin_nontemporal_load(vp);
                    }
                }
            f32x4 c[NGRP];
#pragma unroll
            for (int g = 0; g < NGRP; ++g) {
                c[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sl = 0; sl < KS; ++sl)
                    c[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[sl], __builtin_bit_cast(bf16x8, kb[g][sl]), c[g],
                                                                  0, 0, 0);
            }
            float fr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float sv[NGRP];
                float bm = -__builtin_inff();
#pragma unroll
                for (int g = 0; g < NGRP; ++g) {
                    sv[g] = okk[g] ? c[g][r] * scale : -__builtin_inff();
                    bm = fmaxf(bm, sv[g]);
                }
                const float mn = fmaxf(mr[r], row_max16(bm));
                fr[r] = mr[r] == -__builtin_inff() ? 0.f : __expf(mr[r] - mn);
                float ls = lr[r] * fr[r];
#pragma unroll
                for (int g = 0; g < NGRP; ++g) {
                    sv[g] = sv[g] == -__builtin_inff() ? 0.f : __expf(sv[g] - mn);
                    ls += sv[g];
                    c[g][r] = sv[g];  // the weight replaces the score
                }
                lr[r] = ls;
                mr[r] = mn;
            }
            if (4 * gq < G) {
#pragma unroll
                for (int g = 0; g < NGRP; ++g)
                    *reinterpret_cast<float4*>(pt + (g * 16 + ln) * 8 + 4 * gq) = make_float4(c[g][0], c[g][1], c[g][2], c[g][3]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // Rescale the accumulators (head i's factor is in lane 16 (i / 4), component i % 4), then add the
            // half-wave's keys' weight x V.
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fr[i % 4]), 16 * (i / 4)));
#pragma unroll
                for (int d = 0; d < DPW; ++d) ow[i][d] *= f;
            }
#pragma unroll
            for (int g = 0; g < NGRP; ++g)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float* wq = pt + (g * 16 + hw + 2 * q) * 8;
                    float wgt[8];
#pragma unroll
                    for (int i4 = 0; i4 < (G + 3) / 4; ++i4) {
                        const float4 w4 = *reinterpret_cast<const float4*>(wq + 4 * i4);
                        wgt[4 * i4] = w4.x;
                        wgt[4 * i4 + 1] = w4.y;
                        wgt[4 * i4 + 2] = w4.z;
                        wgt[4 * i4 + 3] = w4.w;
                    }
#pragma unroll
                    for (int i = 0; i < G; ++i)
#pragma unroll
                        for (int d = 0; d < DPW; ++d)
                            ow[i][d] = __builtin_fmaf(wgt[i], slice_elem<D, BF16>(vw[g][q], d), ow[i][d]);
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        // The wave's partial: its (max, weight sum) per head, and the sum of its two halves' outputs, which
        // the first half stores.
#pragma unroll
        for (int r = 0; r < 4; ++r) lr[r] = row_sum16(lr[r]);
#pragma unroll
        for (int i = 0; i < G; ++i) {
            m_i[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mr[i % 4]), 16 * (i / 4)));
            l_i[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lr[i % 4]), 16 * (i / 4)));
        }
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int d = 0; d < DPW; ++d) ow[i][d] += __shfl_xor(ow[i][d], 32);
        if (hw == 0) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                float* dst = sh.wo(wv, i) + hl * DPW;
                if constexpr (DPW == 4)
                    *reinterpret_cast<float4*>(dst) = make_float4(ow[i][0], ow[i][1], ow[i][2], ow[i][3]);
                else
                    *reinterpret_cast<float2*>(dst) = make_float2(ow[i][0], ow[i][1]);
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                sh.wml[wv][i][0] = m_i[i];
                sh.wml[wv][i][1] = l_i[i];
            }
        }
    } else {
    // Attention over list[0, cnt): row rw takes entries e0 + rw + NR j.
    uint32_t qw[G][NWD];  // this lane's slice of each query, raw
#pragma unroll
    for (int i = 0; i < G; ++i) load_slice<D, BF16>(Q, q0 + i, sub, qw[i]);
    for (int e0 = 0; e0 < cnt; e0 += NR * NI) {
        int t[NI];
        bool ok[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int e = e0 + rw + NR * j;
            ok[j] = e < cnt;
            int tj = list[ok[j] ? e : 0];
            tj = (tj < 0 || tj >= L) ? 0 : tj;
            t[j] = tj;
        }
        uint32_t kw[NI][NWD], vw[NI][NWD];
#pragma unroll
        for (int j = 0; j < NI; ++j) load_slice<D, BF16>(K, kvb + t[j], sub, kw[j]);
#pragma unroll
        for (int j = 0; j < NI; ++j) load_slice<D, BF16>(V, kvb + t[j], sub, vw[j]);
        float sc[NI][G];
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int i = 0; i < G; ++i) {
                sc[j][i] = slice_dot<D, BF16>(qw[i], kw[j]);
            }
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int i = 0; i < G; ++i) sc[j][i] = row_sum16(sc[j][i]) * scale;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float mb = m_i[i];
#pragma unroll
            for (int j = 0; j < NI; ++j)
                if (ok[j]) mb = fmaxf(mb, sc[j][i]);
            const float f = m_i[i] == -__builtin_inff() ? 0.f : __expf(m_i[i] - mb);
            float l = l_i[i] * f;
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[i][d] *= f;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const float p = ok[j] ? __expf(sc[j][i] - mb) : 0.f;
                l += p;
#pragma unroll
                for (int d = 0; d < DPL; ++d) o[i][d] = __builtin_fmaf(p, slice_elem<D, BF16>(vw[j], d), o[i][d]);
            }
            m_i[i] = mb;
            l_i[i] = l;
        }
    }
    store_row_o(sh, rw, sub, o);
    if (sub == 0) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            sh.wml[rw][i][0] = m_i[i];
            sh.wml[rw][i][1] = l_i[i];
        }
    }
    }
    if (tid == NT - 64) sh.last_flag = ticket == (uint32_t)(S - 1);
    __syncthreads();
    merge_polled<D, G, NT>(sh, split, stride, S, q0, part_o, part_ml, out);
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
    float* pml = po + (size_t)s.B * s.Hq * a.lay.part_splits * s.D;
    hipLaunchKernelGGL((attend_kernel<D, BF16, G>), grid, dim3(256), 0, st, a.Q, a.K, a.V, a.sel,
                       reinterpret_cast<const int32_t*>(a.ws + a.lay.k_eff), po, pml,
                       reinterpret_cast<uint32_t*>(a.ws + a.lay.counters), a.out, s.Hq, s.Hkv, s.T, a.sel_cap,
                       a.lay.n_splits, a.lay.part_splits, a.scale, s.share);
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

template <int D, bool BF16, int G>
hipError_t compact_g(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    const int S = a.lay.sel_splits;
    if (S < 2 || S > 64) return hipErrorInvalidValue;  // one lane per split in the offset scan
    float* po = reinterpret_cast<float*>(a.ws + a.lay.partial);
    float* pml = po + (size_t)s.B * s.Hq * a.lay.part_splits * s.D;
    uint32_t* counters = reinterpret_cast<uint32_t*>(a.ws + a.lay.counters);
    hipLaunchKernelGGL((compact_attend_kernel<D, BF16, G>), dim3(s.Hkv, s.B, S), dim3(kCompactThreads), 0, st, a.Q,
                       a.K, a.V,
                       reinterpret_cast<const int32_t*>(a.ws + a.lay.pages),
                       reinterpret_cast<const int32_t*>(a.ws + a.lay.n_pages),
                       reinterpret_cast<const uint16_t*>(a.ws + a.lay.ham),
                       reinterpret_cast<const uint32_t*>(a.ws + a.lay.kcum), counters + a.lay.ghist_off, a.seq_len,
                       a.sel, reinterpret_cast<int32_t*>(a.ws + a.lay.k_eff), po, pml, counters, a.out, s.Hq, s.Hkv,
                       s.T, s.P, a.max_keep, a.top_k, S, a.lay.part_splits, a.lay.nbins, a.scale, s.share, s.nsink,
                       s.window);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t compact_dt(const DecodeArgs& a, hipStream_t st) {
    switch (a.s.G) {
        case 1: return compact_g<D, BF16, 1>(a, st);
        case 2: return compact_g<D, BF16, 2>(a, st);
        case 3: return compact_g<D, BF16, 3>(a, st);
        case 4: return compact_g<D, BF16, 4>(a, st);
        case 5: return compact_g<D, BF16, 5>(a, st);
        case 6: return compact_g<D, BF16, 6>(a, st);
        case 7: return compact_g<D, BF16, 7>(a, st);
        default: return compact_g<D, BF16, 8>(a, st);
    }
}

}  // namespace

hipError_t launch_compact_attend(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    if (s.D == 64) return s.bf16 ? compact_dt<64, true>(a, st) : compact_dt<64, false>(a, st);
    return s.bf16 ? compact_dt<128, true>(a, st) : compact_dt<128, false>(a, st);
}

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
