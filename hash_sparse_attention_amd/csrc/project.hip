// Projection of a few vectors by a KV head's [R_h; W_h] -- the per-token
// work of HHR: the rotated query and its LHP code for the GKR bound and the
// Hamming ranking, and the append of newly generated keys (their codes and
// the GKR statistics of the page they land in).  "HHR: Hierarchical Hash
// Retrieval for Efficient LLM Generation", Abstract; rit.work HHR blog post,
// section "Два уровня маршрутизации решают разные ошибки".
//
// gfx950 mapping for batch-1 latency: grid (Hkv, B, key blocks + query
// block).  A key block owns one page touched by the append: it recomputes
// the page's rotated keys (for its max/min) and the new keys' codes.  The
// query block projects the G queries of the KV head.  A block stages its
// vectors in LDS as fp32 with one round of loads; each wave keeps 64 rows of
// [R_h; W_h] in VGPRs (one row per lane) and runs four vectors at a time as
// independent canonical chains (acc = fma(row[c], x[c], acc), c ascending
// from +0), so the FMA latency of one chain hides behind the others.  Hash
// waves ballot 64 sign bits into a code word; rotation waves keep running
// max/min over the page's keys and meet in LDS.
#include "hhr_internal.h"

namespace hhr {
namespace {

constexpr int kProjWaves = 8;
constexpr int kChains = 4;  // vectors in flight per wave

template <int D, int NB, bool BF16, bool KEYS, bool QUERIES>
__global__ __launch_bounds__(kProjWaves * 64) void project_kernel(
    const void* __restrict__ Q, const void* __restrict__ K, const float* __restrict__ R,
    const float* __restrict__ W, const int32_t* __restrict__ start, const int32_t* __restrict__ count,
    int max_count, int key_blocks, float* __restrict__ meta, uint64_t* __restrict__ codes,
    float* __restrict__ q_rot, uint64_t* __restrict__ code_q, double* __restrict__ q_split,
    uint32_t* __restrict__ counters, int n_counters, int Hq, int Hkv, int G, int T, int P, int64_t NPB) {
    constexpr int RR = D / 64, HR = NB / 64;  // rotation / hash row groups (waves per vector group)
    constexpr int NW = NB / 64;
    constexpr int RVG = (kProjWaves - HR) / RR;  // rotation vector groups
    extern __shared__ float lds[];
    float* xs = lds;                          // [nvec][D] staged vectors
    float* red = lds + 64 * D;                // [RVG][D][2] max/min partials

    const int h = blockIdx.x, b = blockIdx.y, z = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;
    const bool qblock = QUERIES && z == (KEYS ? key_blocks : 0);

    if (QUERIES && counters && qblock && blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = tid; i < n_counters; i += kProjWaves * 64) counters[i] = 0u;

    // This block's vectors: n_rot for the rotation rows (first ones), of which
    // the last n_hash also go through the hash rows.
    int s = 0, lo = 0, p = 0, n_rot = 0, hfirst = 0;
    int64_t xrow0 = 0;
    if (qblock) {
        n_rot = G;
        hfirst = 0;
        xrow0 = q0;
    } else if (KEYS) {
        s = start[b];
        s = s < 0 ? 0 : (s > T ? T : s);
        int c = count[b];
        c = c < 0 ? 0 : c;
        c = c > max_count ? max_count : c;
        c = c > T - s ? T - s : c;
        const int e = s + c;
        p = s / P + z;
        lo = p * P;
        n_rot = (c > 0 && lo < e) ? (lo + P < e ? lo + P : e) - lo : 0;
        hfirst = s - lo > 0 ? s - lo : 0;
        xrow0 = bh * T + lo;
    }
    if (n_rot == 0) return;  // block-uniform
    const int n_hash = n_rot - hfirst;

    // Stage the vectors (rows xrow0 .. xrow0 + n_rot - 1 of Q or K) as fp32.
    const void* src = qblock ? Q : K;
    if (BF16) {
        const uint32_t* x2 = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(src) + xrow0 * D);
        for (int i = tid; i < n_rot * D / 2; i += kProjWaves * 64) {
            const uint32_t u = x2[i];
            xs[2 * i] = __uint_as_float(u << 16);
            xs[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
        }
    } else {
        const float* xf = static_cast<const float*>(src) + xrow0 * D;
        for (int i = tid; i < n_rot * D; i += kProjWaves * 64) xs[i] = xf[i];
    }

    // Roles: waves [0, RR*RVG) rotation rows, the next HR waves hash rows.
    const bool rot = w < RR * RVG;
    const bool hashw = !rot && w < RR * RVG + HR;
    const int row = rot ? (w % RR) * 64 + lane : D + (w - RR * RVG) * 64 + lane;
    const int vg = rot ? w / RR : 0, nvg = rot ? RVG : 1;
    const int v0 = rot ? 0 : hfirst;
    const int nv = rot ? n_rot : n_hash;
    float m[D];
    if (rot || hashw) {
        const float* mrow = rot ? R + ((int64_t)h * D + row) * D : W + ((int64_t)h * NB + (row - D)) * D;
#pragma unroll
        for (int i = 0; i < D; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(mrow + i);
            m[i] = v.x; m[i + 1] = v.y; m[i + 2] = v.z; m[i + 3] = v.w;
        }
    }
    __syncthreads();

    float mx = -__builtin_inff(), mn = __builtin_inff();
    if (rot || hashw) {
        // vectors v0 + vg, v0 + vg + nvg, ... in groups of kChains
        for (int j0 = vg; j0 < nv; j0 += nvg * kChains) {
            float acc[kChains];
            int vi[kChains];
#pragma unroll
            for (int u = 0; u < kChains; ++u) {
                acc[u] = 0.f;
                const int j = j0 + u * nvg;
                vi[u] = v0 + (j < nv ? j : vg);  // out-of-range chains recompute a valid vector; discarded
            }
#pragma unroll
            for (int c = 0; c < D; c += 4) {
                float4 x[kChains];
#pragma unroll
                for (int u = 0; u < kChains; ++u) x[u] = *reinterpret_cast<const float4*>(xs + vi[u] * D + c);
#pragma unroll
                for (int u = 0; u < kChains; ++u) {
                    acc[u] = __builtin_fmaf(m[c], x[u].x, acc[u]);
                    acc[u] = __builtin_fmaf(m[c + 1], x[u].y, acc[u]);
                    acc[u] = __builtin_fmaf(m[c + 2], x[u].z, acc[u]);
                    acc[u] = __builtin_fmaf(m[c + 3], x[u].w, acc[u]);
                }
                // Pin the four chains to this step: left alone, the compiler
                // finishes one chain before the next and keeps every loaded
                // vector of the others live, which spills.
                asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])::"memory");
            }
#pragma unroll
            for (int u = 0; u < kChains; ++u) {
                const int j = j0 + u * nvg;
                if (j >= nv) continue;  // wave-uniform
                const int v = v0 + j;
                if (qblock) {
                    const int64_t qi = q0 + v;
                    if (rot) {
                        q_rot[qi * D + row] = acc[u];
                        double* qsp = q_split + ((bh * D + row) * G + v) * 2;
                        qsp[0] = acc[u] >= 0.f ? (double)acc[u] : 0.0;
                        qsp[1] = acc[u] < 0.f ? (double)acc[u] : 0.0;
                    } else {
                        const uint64_t word = __ballot(acc[u] > 0.f);
                        if (lane == 0) code_q[qi * NW + (row - D) / 64] = word;
                    }
                } else if (rot) {
                    const float vk = acc[u] == 0.f ? 0.f : acc[u];
                    mx = fmaxf(mx, vk);
                    mn = fminf(mn, vk);
                } else {
                    const uint64_t word = __ballot(acc[u] > 0.f);
                    if (lane == 0) codes[(bh * T + lo + v) * NW + (row - D) / 64] = word;
                }
            }
        }
    }
    if (KEYS && !qblock) {
        if (rot) {
            red[(vg * D + row) * 2] = mx;
            red[(vg * D + row) * 2 + 1] = mn;
        }
        __syncthreads();
        if (rot && vg == 0) {
#pragma unroll
            for (int g = 1; g < RVG; ++g) {
                mx = fmaxf(mx, red[(g * D + row) * 2]);
                mn = fminf(mn, red[(g * D + row) * 2 + 1]);
            }
            float* mp = meta + (((bh * NPB + p / 64) * (D / 2) + row / 2) * 64 + (p & 63)) * 4 + (row & 1) * 2;
            *reinterpret_cast<float2*>(mp) = make_float2(mx, mn);
        }
    }
}

template <int D, int NB, bool BF16, bool KEYS, bool QUERIES>
hipError_t project_t(const Shape& s, const ProjectArgs& a, hipStream_t st) {
    constexpr int RR = D / 64, HR = NB / 64, RVG = (kProjWaves - HR) / RR;
    const int key_blocks = KEYS ? (a.max_count - 1) / s.P + 2 : 0;
    const int blocks = key_blocks + (QUERIES ? 1 : 0);
    const size_t lds = (size_t)(64 * D + RVG * D * 2) * sizeof(float);
    hipLaunchKernelGGL((project_kernel<D, NB, BF16, KEYS, QUERIES>), dim3(s.Hkv, s.B, blocks), dim3(kProjWaves * 64),
                       lds, st, a.Q, a.K, a.R, a.W, a.start, a.count, a.max_count, key_blocks, a.meta, a.codes,
                       a.q_rot, a.code_q, a.q_split, a.counters, a.n_counters, s.Hq, s.Hkv, s.G, s.T, s.P, s.NPB);
    return hipGetLastError();
}

template <int D, int NB, bool BF16>
hipError_t project_mode(const Shape& s, const ProjectArgs& a, hipStream_t st) {
    if (a.keys && a.queries) return project_t<D, NB, BF16, true, true>(s, a, st);
    if (a.keys) return project_t<D, NB, BF16, true, false>(s, a, st);
    return project_t<D, NB, BF16, false, true>(s, a, st);
}

template <int D, int NB>
hipError_t project_dt(const Shape& s, const ProjectArgs& a, hipStream_t st) {
    return s.bf16 ? project_mode<D, NB, true>(s, a, st) : project_mode<D, NB, false>(s, a, st);
}

}  // namespace

hipError_t launch_project(const Shape& s, const ProjectArgs& a, hipStream_t st) {
    if (s.D == 64 && s.NB == 64) return project_dt<64, 64>(s, a, st);
    if (s.D == 64 && s.NB == 128) return project_dt<64, 128>(s, a, st);
    if (s.D == 128 && s.NB == 64) return project_dt<128, 64>(s, a, st);
    return project_dt<128, 128>(s, a, st);
}

}  // namespace hhr
