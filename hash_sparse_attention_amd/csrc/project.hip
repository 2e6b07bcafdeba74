// Projection of a few vectors by a KV head's [R_h; W_h] -- the per-token
// work of HHR: the rotated query and its LHP code for the GKR bound and the
// Hamming ranking, and the append of newly generated keys (their codes and
// the GKR statistics of the page they land in).  "HHR: Hierarchical Hash
// Retrieval for Efficient LLM Generation", Abstract; rit.work HHR blog post,
// section "Два уровня маршрутизации решают разные ошибки".
//
// gfx950 mapping: a block per (sequence, KV head[, touched page]); wave w
// owns 64 rows of [R_h; W_h] (one row per lane, held in VGPRs) and walks a
// strided subset of the vectors.  A vector is wave-uniform, so its elements
// arrive through scalar loads and enter v_fma as SGPR operands: no LDS and no
// cross-lane traffic in the FMA chains.  Each chain is the canonical one
// (acc = fma(row[c], x[c], acc), c ascending from +0), bit-identical to any
// other IEEE evaluation of it.  Rotation waves keep running max/min over the
// page's keys, meeting in LDS; hash waves ballot 64 sign bits into a word.
#include "hhr_internal.h"

namespace hhr {
namespace {

constexpr int kProjWaves = 8;

template <int D, int NB, bool BF16, bool KEYS, bool QUERIES>
__global__ __launch_bounds__(kProjWaves * 64) void project_kernel(
    const void* __restrict__ Q, const void* __restrict__ K, const float* __restrict__ R,
    const float* __restrict__ W, const int32_t* __restrict__ start, const int32_t* __restrict__ count,
    int max_count, float* __restrict__ meta, uint64_t* __restrict__ codes, float* __restrict__ q_rot,
    uint64_t* __restrict__ code_q, double* __restrict__ q_split, uint32_t* __restrict__ counters, int n_counters,
    int Hq, int Hkv, int G, int T, int P, int64_t NPB) {
    constexpr int NRW = (D + NB) / 64;       // row waves
    constexpr int VG = kProjWaves / NRW;     // vector groups
    constexpr int NW = NB / 64;
    __shared__ float red[VG][D][2];

    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool active = w < NRW * VG;
    const int rw = w % NRW, vg = w / NRW;
    const int row = rw * 64 + lane;
    const bool rot = row < D;  // wave-uniform
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;

    if (QUERIES && counters && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
        for (int i = tid; i < n_counters; i += blockDim.x) counters[i] = 0u;

    // Keys of this block: page p's keys [lo, lo + n); codes only for keys >= s.
    int s = 0, e = 0, lo = 0, n = 0, p = 0;
    if (KEYS) {
        s = start[b];
        s = s < 0 ? 0 : (s > T ? T : s);
        int c = count[b];
        c = c < 0 ? 0 : c;
        c = c > max_count ? max_count : c;
        c = c > T - s ? T - s : c;
        e = s + c;
        p = s / P + blockIdx.z;
        lo = p * P;
        n = (c > 0 && lo < e) ? (lo + P < e ? lo + P : e) - lo : 0;
    }
    const bool do_q = QUERIES && blockIdx.z == 0;
    if (KEYS && n == 0 && !do_q) return;  // block-uniform

    const int jfirst = rot ? 0 : (s - lo > 0 ? s - lo : 0);  // hash rows: only keys >= s
    const int nk = KEYS ? (n > jfirst ? n - jfirst : 0) : 0;  // key vectors of this wave's rows
    const int nv = nk + (do_q ? G : 0);

    float mx = -__builtin_inff(), mn = __builtin_inff();
    if (active) {
        const float* src = rot ? R + ((int64_t)h * D + row) * D : W + ((int64_t)h * NB + (row - D)) * D;
        float m[D];
#pragma unroll
        for (int i = 0; i < D; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(src + i);
            m[i] = v.x; m[i + 1] = v.y; m[i + 2] = v.z; m[i + 3] = v.w;
        }
        for (int v = vg; v < nv; v += VG) {
            const bool is_key = v < nk;
            const int64_t xrow = is_key ? (bh * T + lo + jfirst + v) : (q0 + (v - nk));
            const void* base = is_key ? K : Q;
            float acc = 0.f;
            if (BF16) {
                const uint32_t* x = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + xrow * D);
#pragma unroll
                for (int c = 0; c < D; c += 2) {
                    const uint32_t u = x[c / 2];
                    acc = __builtin_fmaf(m[c], __uint_as_float(u << 16), acc);
                    acc = __builtin_fmaf(m[c + 1], __uint_as_float(u & 0xffff0000u), acc);
                }
            } else {
                const float* x = static_cast<const float*>(base) + xrow * D;
#pragma unroll
                for (int c = 0; c < D; ++c) acc = __builtin_fmaf(m[c], x[c], acc);
            }
            if (is_key) {
                if (rot) {
                    const float vk = acc == 0.f ? 0.f : acc;
                    mx = fmaxf(mx, vk);
                    mn = fminf(mn, vk);
                } else {
                    const uint64_t word = __ballot(acc > 0.f);
                    if (lane == 0) codes[(bh * T + lo + jfirst + v) * NW + (row - D) / 64] = word;
                }
            } else {
                const int64_t qi = q0 + (v - nk);
                if (rot) {
                    q_rot[qi * D + row] = acc;
                    double* qsp = q_split + ((bh * D + row) * G + (v - nk)) * 2;
                    qsp[0] = acc >= 0.f ? (double)acc : 0.0;
                    qsp[1] = acc < 0.f ? (double)acc : 0.0;
                } else {
                    const uint64_t word = __ballot(acc > 0.f);
                    if (lane == 0) code_q[qi * NW + (row - D) / 64] = word;
                }
            }
        }
    }
    if (KEYS && n > 0) {
        if (active && rot) {
            red[vg][row][0] = mx;
            red[vg][row][1] = mn;
        }
        __syncthreads();
        if (active && rot && vg == 0) {
#pragma unroll
            for (int g = 1; g < VG; ++g) {
                mx = fmaxf(mx, red[g][row][0]);
                mn = fminf(mn, red[g][row][1]);
            }
            float* mp = meta + (((bh * NPB + p / 64) * (D / 2) + row / 2) * 64 + (p & 63)) * 4 + (row & 1) * 2;
            *reinterpret_cast<float2*>(mp) = make_float2(mx, mn);
        }
    }
}

template <int D, int NB, bool BF16, bool KEYS, bool QUERIES>
hipError_t project_t(const Shape& s, const ProjectArgs& a, hipStream_t st) {
    const int pages = KEYS ? (a.max_count - 1) / s.P + 2 : 1;
    hipLaunchKernelGGL((project_kernel<D, NB, BF16, KEYS, QUERIES>), dim3(s.Hkv, s.B, pages), dim3(kProjWaves * 64), 0,
                       st, a.Q, a.K, a.R, a.W, a.start, a.count, a.max_count, a.meta, a.codes, a.q_rot, a.code_q,
                       a.q_split, a.counters, a.n_counters, s.Hq, s.Hkv, s.G, s.T, s.P, s.NPB);
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
