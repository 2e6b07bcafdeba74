// Projection of a few vectors by a KV head's [R_h; W_h] -- the per-token
// work of HHR: the rotated query and its LHP code for the GKR bound and the
// Hamming ranking, and the append of newly generated keys (their codes and
// the GKR statistics of the page they land in).  "HHR: Hierarchical Hash
// Retrieval for Efficient LLM Generation", Abstract; rit.work HHR blog post,
// section "Два уровня маршрутизации решают разные ошибки".
//
// gfx950 mapping for batch-1 latency: a block owns one 64-row group of the
// KV head's stacked [R_h; W_h] (rows of R_h first) and one vector block: a
// page touched by the append (its keys feed the page's max/min; the new keys
// also feed the codes) or the G queries.  The block loads its 64 x D rows
// with coalesced 16-byte loads into an LDS tile padded to D + 4 floats per
// row (so a lane reading its own row hits distinct banks) and its vectors as
// fp32; every wave loads its lane's row into registers and runs its share of
// the vectors, two at a time, as independent canonical chains, lane = row:
// acc = fma(row[c], x[c], acc), c ascending from +0.
// With the mean-query variant the query block adds one vector, the group's
// mean qm_d = (sum_i q_i,d) / G in fp32 (heads ascending, one division),
// which only goes through the hash rows; its code goes to code_qm.
// Rows are independent (one rotated dimension, or one code bit), so no
// result crosses blocks: hash rows ballot 64 sign bits into a code word and
// rotation rows keep max/min over the page's keys, merged across waves in
// LDS.
#include "hhr_internal.h"

namespace hhr {
namespace {

constexpr int kProjWaves = 8;
constexpr int kMaxVec = 64;  // vectors a block stages (P <= 64 keys, or G <= 8 queries)

template <int D, int NB, bool BF16, bool KEYS, bool QUERIES>
__global__ __launch_bounds__(kProjWaves * 64) void project_kernel(
    const void* __restrict__ Q, const void* __restrict__ K, const float* __restrict__ R,
    const float* __restrict__ W, const int32_t* __restrict__ start, const int32_t* __restrict__ count,
    int max_count, int key_blocks, float* __restrict__ meta, uint64_t* __restrict__ codes,
    float* __restrict__ q_rot, uint64_t* __restrict__ code_q, uint64_t* __restrict__ code_qm,
    double* __restrict__ q_split, uint32_t* __restrict__ counters, int n_counters, int Hq, int Hkv, int G, int T,
    int P, int64_t NPB, bool meta16, bool msplit, bool qmean) {
    constexpr int RG = (D + NB) / 64;  // row groups of [R_h; W_h]
    constexpr int NW = NB / 64;
    constexpr int LDM = D + 4;         // padded row stride of the tile (floats)
    __shared__ float mt[64 * LDM];
    __shared__ float xs[kMaxVec * D];
    __shared__ float red[kProjWaves][64][2];

    const int h = blockIdx.x, b = blockIdx.y, vb = blockIdx.z / RG, rg = blockIdx.z % RG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;
    const bool qblock = QUERIES && vb == (KEYS ? key_blocks : 0);
    const bool rot = rg < D / 64;

    if (QUERIES && counters && qblock && rg == 0 && h == 0 && b == 0)
        for (int i = tid; i < n_counters; i += kProjWaves * 64) counters[i] = 0u;

    // This block's vectors: n_rot through the rotation rows, of which the
    // last ones (from hfirst) also through the hash rows.
    int lo = 0, p = 0, n_rot = 0, hfirst = 0, n_load = 0, n_vec = 0;
    int64_t xrow0 = 0;
    if (qblock) {
        n_rot = G;
        n_load = G;
        n_vec = G + (qmean ? 1 : 0);  // the mean query goes through the hash rows only
        xrow0 = q0;
    } else if (KEYS) {
        int s = start[b];
        s = s < 0 ? 0 : (s > T ? T : s);
        int c = count[b];
        c = c < 0 ? 0 : c;
        c = c > max_count ? max_count : c;
        c = c > T - s ? T - s : c;
        const int e = s + c;
        p = s / P + vb;
        lo = p * P;
        n_rot = (c > 0 && lo < e) ? (lo + P < e ? lo + P : e) - lo : 0;
        hfirst = s - lo > 0 ? s - lo : 0;
        xrow0 = bh * T + lo;
        n_load = n_vec = n_rot;
    }
    const int v0 = rot ? 0 : hfirst;
    const int nv = (rot ? n_rot : n_vec) - v0;
    if (nv <= 0) return;  // block-uniform

    // The 64 rows of this group (coalesced) and the vectors (as fp32).
    const float4* mg = reinterpret_cast<const float4*>(
        rot ? R + ((int64_t)h * D + 64 * rg) * D : W + ((int64_t)h * NB + 64 * (rg - D / 64)) * D);
    constexpr int F4PT = 64 * D / 4 / (kProjWaves * 64);
    float4 mv[F4PT];
#pragma unroll
    for (int k = 0; k < F4PT; ++k) {  // the rows are read once per step
        const u32x4 r = load_stream16(mg + tid + k * kProjWaves * 64);
        mv[k] = make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w));
    }
    const void* src = qblock ? Q : K;
    if (BF16) {
        const uint32_t* x2 = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(src) + xrow0 * D);
        for (int i = tid; i < n_load * D / 2; i += kProjWaves * 64) {
            const uint32_t u = x2[i];
            xs[2 * i] = __uint_as_float(u << 16);
            xs[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
        }
    } else {
        const float* xf = static_cast<const float*>(src) + xrow0 * D;
        for (int i = tid; i < n_load * D; i += kProjWaves * 64) xs[i] = xf[i];
    }
#pragma unroll
    for (int k = 0; k < F4PT; ++k) {
        const int f = tid + k * kProjWaves * 64;  // float4 index within the 64 x D group
        *reinterpret_cast<float4*>(&mt[(f / (D / 4)) * LDM + (f % (D / 4)) * 4]) = mv[k];
    }
    __syncthreads();
    if (n_vec > n_load) {  // block-uniform: the group's mean query, after the staged queries
        for (int d = tid; d < D; d += kProjWaves * 64) {
            float acc = 0.f;
            for (int i = 0; i < G; ++i) acc += xs[i * D + d];
            xs[G * D + d] = acc / (float)G;
        }
        __syncthreads();
    }

    // Wave w runs vectors w, w + kProjWaves, ... two chains at a time.  The
    // lane's row of the group goes into registers in halves of up to 64
    // columns (independent LDS reads, so their latency overlaps), and the
    // chains run from registers, columns ascending.
    const int row = 64 * rg + lane;  // row of [R_h; W_h]
    constexpr int HC = D < 64 ? D : 64;  // columns per half
    float mx = -__builtin_inff(), mn = __builtin_inff();
    auto emit = [&](int j, float a) {
        const int v = v0 + j;
        if (qblock) {
            const int64_t qi = q0 + v;
            if (rot) {
                q_rot[qi * D + row] = a;
                double* qsp = q_split + ((bh * D + row) * G + v) * 2;
                qsp[0] = a >= 0.f ? (double)a : 0.0;
                qsp[1] = a < 0.f ? (double)a : 0.0;
            } else {
                const uint64_t word = __ballot(a > 0.f);
                if (lane == 0) {
                    if (v < G) code_q[qi * NW + (row - D) / 64] = word;
                    else code_qm[bh * NW + (row - D) / 64] = word;
                }
            }
        } else if (rot) {
            const float vk = a == 0.f ? 0.f : a;
            mx = fmaxf(mx, vk);
            mn = fminf(mn, vk);
        } else {
            const uint64_t word = __ballot(a > 0.f);
            if (lane == 0) codes[(bh * T + lo + v) * NW + (row - D) / 64] = word;
        }
    };
    for (int ja = w; ja < nv; ja += 2 * kProjWaves) {  // wave-uniform
        const int jb = ja + kProjWaves;
        const bool two = jb < nv;  // wave-uniform
        const float4* xa = reinterpret_cast<const float4*>(xs + (v0 + ja) * D);
        const float4* xb = reinterpret_cast<const float4*>(xs + (v0 + (two ? jb : ja)) * D);
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 1
        for (int c0 = 0; c0 < D; c0 += HC) {
            float4 mrow[HC / 4];
#pragma unroll
            for (int k = 0; k < HC / 4; ++k)
                mrow[k] = *reinterpret_cast<const float4*>(&mt[lane * LDM + c0 + 4 * k]);
#pragma unroll
            for (int k = 0; k < HC / 4; ++k) {
                const float4 x = xa[c0 / 4 + k], y = xb[c0 / 4 + k];
                acc0 = __builtin_fmaf(mrow[k].x, x.x, acc0);
                acc0 = __builtin_fmaf(mrow[k].y, x.y, acc0);
                acc0 = __builtin_fmaf(mrow[k].z, x.z, acc0);
                acc0 = __builtin_fmaf(mrow[k].w, x.w, acc0);
                acc1 = __builtin_fmaf(mrow[k].x, y.x, acc1);
                acc1 = __builtin_fmaf(mrow[k].y, y.y, acc1);
                acc1 = __builtin_fmaf(mrow[k].z, y.z, acc1);
                acc1 = __builtin_fmaf(mrow[k].w, y.w, acc1);
            }
        }
        emit(ja, acc0);
        if (two) emit(jb, acc1);
    }
    if (KEYS && !qblock && rot) {  // block-uniform
        red[w][lane][0] = mx;
        red[w][lane][1] = mn;
        __syncthreads();
        if (w == 0) {
#pragma unroll
            for (int g = 1; g < kProjWaves; ++g) {
                mx = fmaxf(mx, red[g][lane][0]);
                mn = fminf(mn, red[g][lane][1]);
            }
            if (msplit) {  // sign-split: (dimension row, max side) run, then its min side, 64 pages each
                const int64_t e0 = ((bh * NPB + p / 64) * D + row) * 128 + (p & 63);
                if (meta16) {
                    uint16_t* mp = reinterpret_cast<uint16_t*>(meta) + e0;
                    mp[0] = (uint16_t)bf16_up(mx);
                    mp[64] = (uint16_t)bf16_down(mn);
                } else {
                    meta[e0] = mx;
                    meta[e0 + 64] = mn;
                }
            } else if (meta16) {  // bf16 slot (dimension quad row / 4, page p), word row % 4
                uint32_t* mp = reinterpret_cast<uint32_t*>(meta) +
                               (((bh * NPB + p / 64) * (D / 4) + row / 4) * 64 + (p & 63)) * 4 + (row & 3);
                *mp = bf16_pair_out(mx, mn);
            } else {
                float* mp = meta + (((bh * NPB + p / 64) * (D / 2) + row / 2) * 64 + (p & 63)) * 4 + (row & 1) * 2;
                *reinterpret_cast<float2*>(mp) = make_float2(mx, mn);
            }
        }
    }
}

template <int D, int NB, bool BF16, bool KEYS, bool QUERIES>
hipError_t project_t(const Shape& s, const ProjectArgs& a, hipStream_t st) {
    constexpr int RG = (D + NB) / 64;
    // Pages that max_count consecutive tokens can touch: floor((c + 2P - 2) / P)
    // (one for a single token, where (c - 1) / P + 2 launched an idle second
    // page's blocks).
    const int key_pages = (a.max_count + 2 * s.P - 2) / s.P;
    const int key_blocks = KEYS ? (key_pages > 1 ? key_pages : 1) : 0;
    const int blocks = (key_blocks + (QUERIES ? 1 : 0)) * RG;
    hipLaunchKernelGGL((project_kernel<D, NB, BF16, KEYS, QUERIES>), dim3(s.Hkv, s.B, blocks),
                       dim3(kProjWaves * 64), 0, st, a.Q, a.K, a.R, a.W, a.start, a.count, a.max_count, key_blocks,
                       a.meta, a.codes, a.q_rot, a.code_q, a.code_qm, a.q_split, a.counters, a.n_counters, s.Hq,
                       s.Hkv, s.G, s.T, s.P, s.NPB, s.meta16, s.msplit, a.queries && a.qmean);
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
