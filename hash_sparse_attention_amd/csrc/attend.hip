// Gather attention over the keys HHR kept: for every query head i of a KV
// head's group, out_i = sum_t softmax_t(scale * q_i . k_t) v_t over the
// selected t ("HHR: Hierarchical Hash Retrieval for Efficient LLM
// Generation", Abstract: hash-based sparse attention computes exact
// attention on the retrieved keys).
//
// gfx950 mapping, built for latency at batch 1: grid (splits, Hkv, B); a
// block owns 256 consecutive entries of the KV head's selected list and each
// of its 4 waves owns 64 of them.
//  phase A (lane = key): the lane loads its whole K row in one batch and
//    runs G independent fp32 FMA chains q_i . k; the queries are
//    wave-uniform, so they arrive through scalar loads as SGPR operands;
//  wave softmax per head over its 64 keys (butterfly max and sum);
//  phase B (lane = dimension slice): all 64 V rows of the wave are loaded
//    up front; the weights move from the key lanes with v_readlane;
//  the 4 waves merge in LDS into the block's (o, m, l) per query head, and
//    the last block of the KV head (device-scope counter) merges all splits
//    with a log-sum-exp, writes out and resets the counter.
#include "hhr_internal.h"

namespace hhr {
namespace {

template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void attend_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                     const void* __restrict__ V, const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ k_eff, float* __restrict__ part_o,
                                                     float* __restrict__ part_ml, uint32_t* __restrict__ counters,
                                                     float* __restrict__ out, int Hq, int Hkv, int T, int top_k,
                                                     int n_splits, float scale) {
    constexpr int CH = kAttnChunk;            // keys per block (4 waves x 64)
    constexpr int DPL = D / 64;               // dims per lane in phase B
    constexpr int VB = BF16 ? 64 : 32;        // V rows in flight per batch
    constexpr int MAXS = 64;                  // splits merged per round by the last block
    __shared__ float wo[4][G][D];
    __shared__ float wml[4][G][2];
    __shared__ float cml[G][MAXS][2];
    __shared__ int last_flag;

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;
    int keff = k_eff[bh];
    keff = keff < 0 ? 0 : (keff > top_k ? top_k : keff);
    const int c0 = split * CH + wv * 64;                     // this wave's first list entry
    const int n = keff - c0 < 0 ? 0 : (keff - c0 > 64 ? 64 : keff - c0);  // its keys (wave-uniform)

    float m_i[G], l_i[G], o[G][DPL];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        m_i[i] = -__builtin_inff();
        l_i[i] = 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) o[i][k] = 0.f;
    }

    if (n > 0) {
        int t = lane < n ? sel[bh * top_k + c0 + lane] : 0;
        t = (t < 0 || t >= T) ? 0 : t;
        const int64_t kvb = bh * T;

        // Phase A: logits of key `lane` for the G heads.
        float s[G];
#pragma unroll
        for (int i = 0; i < G; ++i) s[i] = 0.f;
        if (BF16) {
            const uint4* kr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(K) + (kvb + t) * D);
            uint4 u[D / 8];
#pragma unroll
            for (int x = 0; x < D / 8; ++x) u[x] = kr[x];
            const uint32_t* qw = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(Q) + q0 * D);
#pragma unroll
            for (int x = 0; x < D / 8; ++x) {
                const uint32_t w4[4] = {u[x].x, u[x].y, u[x].z, u[x].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float k0 = __uint_as_float(w4[q] << 16), k1 = __uint_as_float(w4[q] & 0xffff0000u);
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        const uint32_t qq = qw[(i * D + 8 * x + 2 * q) / 2];
                        s[i] = __builtin_fmaf(__uint_as_float(qq << 16), k0, s[i]);
                        s[i] = __builtin_fmaf(__uint_as_float(qq & 0xffff0000u), k1, s[i]);
                    }
                }
            }
        } else {
            const float4* kr = reinterpret_cast<const float4*>(static_cast<const float*>(K) + (kvb + t) * D);
            float4 f[D / 4];
#pragma unroll
            for (int x = 0; x < D / 4; ++x) f[x] = kr[x];
            const float* qf = static_cast<const float*>(Q) + q0 * D;
#pragma unroll
            for (int x = 0; x < D / 4; ++x) {
                const float kv[4] = {f[x].x, f[x].y, f[x].z, f[x].w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < G; ++i) s[i] = __builtin_fmaf(qf[i * D + 4 * x + q], kv[q], s[i]);
            }
        }

        // Wave softmax over the wave's keys.
        float p[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float si = lane < n ? s[i] * scale : -__builtin_inff();
            const float mx = wave_max(si);
            p[i] = lane < n ? __expf(si - mx) : 0.f;
            m_i[i] = mx;
            l_i[i] = wave_sum(p[i]);
        }

        // Phase B: o_i[lane slice] = sum_j p_i[j] * v_j, rows loaded VB at a time.
        for (int j0 = 0; j0 < n; j0 += VB) {
            uint32_t vraw[VB][BF16 ? 1 : DPL];
#pragma unroll
            for (int j = 0; j < VB; ++j) {
                const int tj = __builtin_amdgcn_readlane(t, (j0 + j) & 63);  // rows >= n are harmless, weight 0
                if (BF16) {
                    const uint16_t* vp = static_cast<const uint16_t*>(V) + (kvb + tj) * D + lane * DPL;
                    vraw[j][0] = DPL == 2 ? *reinterpret_cast<const uint32_t*>(vp) : (uint32_t)vp[0] << 16;
                } else {
                    const float* vp = static_cast<const float*>(V) + (kvb + tj) * D + lane * DPL;
#pragma unroll
                    for (int k = 0; k < DPL; ++k) vraw[j][BF16 ? 0 : k] = __float_as_uint(vp[k]);
                }
            }
#pragma unroll
            for (int j = 0; j < VB; ++j) {
                float vv[DPL];
                if (BF16) {
                    vv[0] = __uint_as_float(DPL == 2 ? vraw[j][0] << 16 : vraw[j][0]);
                    if (DPL == 2) vv[DPL - 1] = __uint_as_float(vraw[j][0] & 0xffff0000u);
                } else {
#pragma unroll
                    for (int k = 0; k < DPL; ++k) vv[k] = __uint_as_float(vraw[j][BF16 ? 0 : k]);
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                    __builtin_bit_cast(int, p[i]), (j0 + j) & 63));
#pragma unroll
                    for (int k = 0; k < DPL; ++k) o[i][k] = __builtin_fmaf(pj, vv[k], o[i][k]);
                }
            }
        }
    }

    // Merge the 4 waves of the block.
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
        for (int k = 0; k < DPL; ++k) wo[wv][i][lane * DPL + k] = o[i][k];
        if (lane == 0) {
            wml[wv][i][0] = m_i[i];
            wml[wv][i][1] = l_i[i];
        }
    }
    __syncthreads();
    const int blk_keys = keff - split * CH;
    if (blk_keys > 0) {
        for (int x = tid; x < G * D; x += 256) {
            const int i = x / D, d = x % D;
            float M = wml[0][i][0];
#pragma unroll
            for (int w = 1; w < 4; ++w) M = fmaxf(M, wml[w][i][0]);
            float acc = 0.f, L = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float sc = wml[w][i][1] > 0.f ? __expf(wml[w][i][0] - M) : 0.f;
                acc = __builtin_fmaf(wo[w][i][d], sc, acc);
                L = __builtin_fmaf(wml[w][i][1], sc, L);
            }
            part_o[((q0 + i) * n_splits + split) * D + d] = acc;
            if (d == 0) {
                part_ml[((q0 + i) * n_splits + split) * 2] = M;
                part_ml[((q0 + i) * n_splits + split) * 2 + 1] = L;
            }
        }
    }

    // The last block of this KV head merges the splits.
    __threadfence();
    __syncthreads();
    if (tid == 0) last_flag = atomicAdd(&counters[bh], 1u) == (uint32_t)(n_splits - 1);
    __syncthreads();
    if (!last_flag) return;
    __threadfence();

    const int used = (keff + CH - 1) / CH;
    constexpr int R = (G * D + 255) / 256;
    float acc[R], Mx[R], Ls[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
        Ls[r] = 0.f;
        Mx[r] = -__builtin_inff();
    }
    // Split maxima first (all splits), then weighted sums in rounds of MAXS.
    for (int s0 = 0; s0 < used; s0 += MAXS) {
        const int ns = used - s0 < MAXS ? used - s0 : MAXS;
        for (int x = tid; x < G * ns; x += 256) {
            const int i = x / ns, sI = x % ns;
            const float* ml = part_ml + ((q0 + i) * n_splits + s0 + sI) * 2;
            cml[i][sI][0] = ml[0];
            cml[i][sI][1] = ml[1];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int x = tid + r * 256;
            if (x < G * D) {
                const int i = x / D;
                for (int sI = 0; sI < ns; ++sI) Mx[r] = fmaxf(Mx[r], cml[i][sI][0]);
            }
        }
        __syncthreads();
    }
    for (int s0 = 0; s0 < used; s0 += MAXS) {
        const int ns = used - s0 < MAXS ? used - s0 : MAXS;
        for (int x = tid; x < G * ns; x += 256) {
            const int i = x / ns, sI = x % ns;
            const float* ml = part_ml + ((q0 + i) * n_splits + s0 + sI) * 2;
            cml[i][sI][0] = ml[0];
            cml[i][sI][1] = ml[1];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int x = tid + r * 256;
            if (x < G * D) {
                const int i = x / D, d = x % D;
                const float* po = part_o + ((q0 + i) * n_splits + s0) * D + d;
                int sI = 0;
                for (; sI + 8 <= ns; sI += 8) {
                    float v8[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) v8[u] = po[(int64_t)(sI + u) * D];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float w = __expf(cml[i][sI + u][0] - Mx[r]);
                        acc[r] = __builtin_fmaf(v8[u], w, acc[r]);
                        Ls[r] = __builtin_fmaf(cml[i][sI + u][1], w, Ls[r]);
                    }
                }
                for (; sI < ns; ++sI) {
                    const float w = __expf(cml[i][sI][0] - Mx[r]);
                    acc[r] = __builtin_fmaf(po[(int64_t)sI * D], w, acc[r]);
                    Ls[r] = __builtin_fmaf(cml[i][sI][1], w, Ls[r]);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int x = tid + r * 256;
        if (x < G * D) out[(q0 + x / D) * D + x % D] = used > 0 ? acc[r] / Ls[r] : 0.f;
    }
    if (tid == 0) counters[bh] = 0u;  // ready for the next call
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

hipError_t launch_attend(const DecodeArgs& a, bool zero_counters, hipStream_t st) {
    if (zero_counters) {
        const int n = a.s.B * a.s.Hkv;
        hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, st,
                           reinterpret_cast<uint32_t*>(a.ws + a.lay.counters), n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const Shape& s = a.s;
    if (s.D == 64) return s.bf16 ? attend_dt<64, true>(a, st) : attend_dt<64, false>(a, st);
    return s.bf16 ? attend_dt<128, true>(a, st) : attend_dt<128, false>(a, st);
}

}  // namespace hhr
