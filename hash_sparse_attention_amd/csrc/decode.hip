// HHR decode step on gfx950: query prep, GKR page bounds, page selection,
// LHP Hamming ranking with top-k, and gather attention over the kept keys.
// ("HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", Abstract;
// rit.work HHR blog post, sections "Почему расстояние Хэмминга пропускает
// важные ключи" and "Два уровня маршрутизации решают разные ошибки";
// top-k selection as in Appendix Table 4 of the thelatestinai.com page.)
#include "hhr_internal.h"

namespace hhr {
namespace {

// ============================================================== query prep
// One lane per row of [R_h; W_h]; the G query vectors of the KV head are
// staged in LDS (fp32) and read as broadcasts.  Rotation rows write qrot and
// its sign split (max(q,0), min(q,0)) in fp64 for the page-bound kernel;
// hash waves ballot their 64 sign bits into one code word.
template <int D, int NB, bool BF16>
__global__ __launch_bounds__(D + NB) void qprep_kernel(const void* __restrict__ Q, const float* __restrict__ R,
                                                       const float* __restrict__ W, float* __restrict__ q_rot,
                                                       uint64_t* __restrict__ code_q, double* __restrict__ q_split,
                                                       uint32_t* __restrict__ counters, int n_counters, int Hq,
                                                       int Hkv, int G) {
    constexpr int NW = NB / 64;
    __shared__ float qs[8 * D];
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, row = tid;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;  // first query head of the group

    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = tid; i < n_counters; i += blockDim.x) counters[i] = 0u;

    for (int i = tid; i < G * D; i += blockDim.x)
        qs[i] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(Q)[q0 * D + i]) : static_cast<const float*>(Q)[q0 * D + i];

    const float* src = row < D ? R + ((int64_t)h * D + row) * D : W + ((int64_t)h * NB + (row - D)) * D;
    float m[D];
#pragma unroll
    for (int i = 0; i < D; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + i);
        m[i] = v.x; m[i + 1] = v.y; m[i + 2] = v.z; m[i + 3] = v.w;
    }
    __syncthreads();

    for (int i = 0; i < G; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
            const float4 x = *reinterpret_cast<const float4*>(qs + i * D + c);
            acc = __builtin_fmaf(m[c], x.x, acc);
            acc = __builtin_fmaf(m[c + 1], x.y, acc);
            acc = __builtin_fmaf(m[c + 2], x.z, acc);
            acc = __builtin_fmaf(m[c + 3], x.w, acc);
        }
        if (row < D) {
            q_rot[(q0 + i) * D + row] = acc;
            double* qsp = q_split + ((bh * D + row) * G + i) * 2;
            qsp[0] = acc >= 0.f ? (double)acc : 0.0;
            qsp[1] = acc < 0.f ? (double)acc : 0.0;
        } else {
            const uint64_t word = __ballot(acc > 0.f);
            if (lane == 0) code_q[(q0 + i) * NW + (row - D) / 64] = word;
        }
    }
}

// ============================================================== page bounds
// One lane per page; a wave covers one 64-page block of meta, so each
// float4 load of a dimension pair is one contiguous 1 KiB span per wave.  The
// lane sums in fp64, dimensions ascending, exactly the definition's order:
// per dimension fma(max(q,0), kmax, acc) then fma(min(q,0), kmin, acc) -- one
// of the two products is zero, the other is the larger of q*kmax and q*kmin,
// and every such product is exact in fp64.  q_split is uniform across the
// block (scalar loads).
template <int D, int G, int UNROLL>
__global__ __launch_bounds__(256) void page_bound_kernel(const float* __restrict__ meta,
                                                         const double* __restrict__ q_split,
                                                         const int32_t* __restrict__ seq_len,
                                                         double* __restrict__ score, int Hkv, int T, int P,
                                                         int64_t NPB, int64_t NPmax) {
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int64_t NP = n_pages_of(L, P);
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if ((int64_t)blockIdx.x * 256 >= NP) return;
    if (p >= NP) return;

    const float4* mp = reinterpret_cast<const float4*>(meta) + (bh * NPB + p / 64) * (D / 2) * 64 + (p & 63);
    const double* qs = q_split + bh * D * G * 2;
    double acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) acc[i] = 0.0;

    for (int j0 = 0; j0 < D / 2; j0 += UNROLL) {
        float4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = mp[(int64_t)(j0 + u) * 64];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int d = 2 * (j0 + u);
            const double a0 = v[u].x, c0 = v[u].y, a1 = v[u].z, c1 = v[u].w;
#pragma unroll
            for (int i = 0; i < G; ++i) {
                acc[i] = __builtin_fma(qs[(d * G + i) * 2], a0, acc[i]);
                acc[i] = __builtin_fma(qs[(d * G + i) * 2 + 1], c0, acc[i]);
                acc[i] = __builtin_fma(qs[((d + 1) * G + i) * 2], a1, acc[i]);
                acc[i] = __builtin_fma(qs[((d + 1) * G + i) * 2 + 1], c1, acc[i]);
            }
        }
    }
    double S = acc[0];
#pragma unroll
    for (int i = 1; i < G; ++i) S = acc[i] > S ? acc[i] : S;
    if (S == 0.0) S = 0.0;
    score[bh * NPmax + p] = S;
}

// ============================================================== page select
// Per (b, h): the `keep` pages with the largest score, ties to the lower page
// index, listed ascending.  Scores map to order-preserving 64-bit keys; an
// MSB-first radix select (8-bit digits, LDS histogram) finds the boundary
// bucket, then one ordered pass compacts the winners with block scans.
__device__ __forceinline__ uint64_t order_key(double s) {
    const uint64_t u = (uint64_t)__double_as_longlong(s);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kSelThreads = 1024;

// Finds, scanning digits from 255 down, the bucket where the running count
// reaches `need`.  Run by all threads; wave 0 does the work.
__device__ void find_digit_desc(const int* hist, int need, int* out /* [digit, above, eq] */) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int cnt[4], tot = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            cnt[k] = hist[255 - (lane * 4 + k)];
            tot += cnt[k];
        }
        int x = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int n = __shfl_up(x, off, 64);
            if (lane >= off) x += n;
        }
        int c = x - tot;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (c < need && c + cnt[k] >= need) {
                out[0] = 255 - (lane * 4 + k);
                out[1] = c;
                out[2] = cnt[k];
            }
            c += cnt[k];
        }
    }
}

__global__ __launch_bounds__(kSelThreads) void select_pages_kernel(
    const double* __restrict__ score, const int32_t* __restrict__ seq_len, const int32_t* __restrict__ keep_pages,
    int32_t* __restrict__ pages, int32_t* __restrict__ n_pages, int Hkv, int T, int P, int64_t NPmax,
    int max_keep) {
    __shared__ int hist[256];
    __shared__ int found[3];
    __shared__ int scan_lds[32];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int NP = (int)n_pages_of(L, P);
    int keep = keep_pages[b];
    keep = keep < 1 ? 1 : keep;
    keep = keep > NP ? NP : keep;
    keep = keep > max_keep ? max_keep : keep;
    const double* sc = score + bh * NPmax;
    int32_t* out = pages + bh * max_keep;

    uint64_t prefix = 0, mask = 0;
    int need = keep;
    bool all_in = (keep == NP);  // every page is kept: no selection needed
    for (int shift = 56; shift >= 0 && !all_in && keep > 0; shift -= 8) {
        for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (int p = tid; p < NP; p += blockDim.x) {
            const uint64_t k = order_key(sc[p]);
            if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
        }
        __syncthreads();
        find_digit_desc(hist, need, found);
        __syncthreads();
        const int dig = found[0], above = found[1], eq = found[2];
        need -= above;
        prefix |= (uint64_t)dig << shift;
        mask |= (uint64_t)255 << shift;
        if (eq == need) all_in = true;  // the whole boundary bucket is kept
        __syncthreads();
    }
    // Keep p iff its masked key beats the boundary bucket, or it is in the
    // bucket and (the bucket is kept whole, or it is among the first `need`).
    int base = 0, eq_base = 0;
    for (int p0 = 0; p0 < NP; p0 += blockDim.x) {
        const int p = p0 + tid;
        int gt = 0, eqf = 0;
        if (p < NP) {
            const uint64_t k = order_key(sc[p]) & mask;
            gt = k > prefix;
            eqf = k == prefix;
        }
        int eq_tot;
        const int eq_rank = eq_base + block_excl_scan(eqf, scan_lds, eq_tot);
        const int in = p < NP && (all_in ? (gt | eqf) : (gt | (eqf && eq_rank < need)));
        int tot;
        const int pos = base + block_excl_scan(in, scan_lds, tot);
        if (in && pos < max_keep) out[pos] = p;
        base += tot;
        eq_base += eq_tot;
    }
    for (int j = keep + tid; j < max_keep; j += blockDim.x) out[j] = -1;
    if (tid == 0) n_pages[bh] = keep;
}

// ============================================================== Hamming + key top-k
// Per (b, h): candidates are the keys t < L of the kept pages, in slot order
// j*P + r (ascending t).  H(t) = sum over the group's query heads and code
// words of popcount(code_q ^ code_t).  An LDS histogram of H gives the
// threshold h* with count(H < h*) < k_eff <= count(H <= h*); one ordered pass
// keeps H < h* and the first k_eff - count(H < h*) candidates with H == h*.
template <int NW>
__global__ __launch_bounds__(kSelThreads) void select_keys_kernel(
    const uint64_t* __restrict__ codes, const uint64_t* __restrict__ code_q, const int32_t* __restrict__ pages,
    const int32_t* __restrict__ n_pages, const int32_t* __restrict__ seq_len, uint16_t* __restrict__ ham,
    int32_t* __restrict__ sel, int32_t* __restrict__ k_eff_out, int Hq, int Hkv, int G, int T, int P,
    int max_keep, int top_k) {
    constexpr int NB = NW * 64;
    __shared__ int hist[8 * NB + 1];
    __shared__ int thr[3];
    __shared__ int scan_lds[32];
    __shared__ uint64_t cq[8 * NW];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int nbins = G * NB + 1;
    int np = n_pages[bh];
    np = np < 0 ? 0 : (np > max_keep ? max_keep : np);  // memory safety for a hand-filled workspace
    const int nslots = np * P;
    const int32_t* pl = pages + bh * max_keep;
    uint16_t* hm = ham + bh * (int64_t)max_keep * P;
    const uint64_t* ck = codes + bh * (int64_t)T * NW;

    for (int i = tid; i < nbins; i += blockDim.x) hist[i] = 0;
    for (int i = tid; i < G * NW; i += blockDim.x) cq[i] = code_q[((int64_t)b * Hq + (int64_t)h * G) * NW + i];
    __syncthreads();

    for (int c = tid; c < max_keep * P; c += blockDim.x) {
        uint16_t H = 0xFFFF;
        if (c < nslots) {
            const int t = pl[c / P] * P + c % P;
            if (t >= 0 && t < L) {
                uint64_t k[NW];
#pragma unroll
                for (int w = 0; w < NW; ++w) k[w] = ck[(int64_t)t * NW + w];
                int s = 0;
                for (int i = 0; i < G; ++i)
#pragma unroll
                    for (int w = 0; w < NW; ++w) s += __popcll(cq[i * NW + w] ^ k[w]);
                H = (uint16_t)s;
                atomicAdd(&hist[s], 1);
            }
        }
        hm[c] = H;
    }
    __syncthreads();

    // Threshold h*: ascending cumulative count reaches k_eff.  Thread i owns
    // bins [2i, 2i+2); a block scan gives each thread the count below them.
    {
        const int b0 = 2 * tid;
        const int c0 = b0 < nbins ? hist[b0] : 0, c1 = b0 + 1 < nbins ? hist[b0 + 1] : 0;
        int nvalid;
        const int below0 = block_excl_scan(c0 + c1, scan_lds, nvalid);
        const int keff = nvalid < top_k ? nvalid : top_k;
        if (tid == 0) {
            thr[0] = nbins;
            thr[1] = 0;
            thr[2] = keff;
        }
        __syncthreads();
        if (keff > 0) {
            if (below0 < keff && below0 + c0 >= keff) {
                thr[0] = b0;
                thr[1] = keff - below0;
            } else if (below0 + c0 < keff && below0 + c0 + c1 >= keff) {
                thr[0] = b0 + 1;
                thr[1] = keff - below0 - c0;
            }
        }
    }
    __syncthreads();
    const int hs = thr[0], need = thr[1], keff = thr[2];

    int32_t* so = sel + bh * top_k;
    int base = 0, eq_base = 0;
    for (int c0 = 0; c0 < nslots; c0 += blockDim.x) {
        const int c = c0 + tid;
        int lt = 0, eqf = 0, t = 0;
        if (c < nslots) {
            const int H = hm[c];
            if (H != 0xFFFF) {
                lt = H < hs;
                eqf = H == hs;
                t = pl[c / P] * P + c % P;
            }
        }
        int eq_tot;
        const int eq_rank = eq_base + block_excl_scan(eqf, scan_lds, eq_tot);
        const int in = lt | (eqf && eq_rank < need);
        int tot;
        const int pos = base + block_excl_scan(in, scan_lds, tot);
        if (in && pos < top_k) so[pos] = t;
        base += tot;
        eq_base += eq_tot;
    }
    for (int j = keff + tid; j < top_k; j += blockDim.x) so[j] = -1;
    if (tid == 0) k_eff_out[bh] = keff;
}

// ============================================================== gather attention
// Grid (splits, Hkv, B); a block takes kAttnChunk consecutive entries of the
// KV head's selected list.  Phase A: wave w forms the partial logits of its
// quarter of the head dimension for all 64 keys and all G query heads
// (lane = key); the quarters meet in LDS.  Softmax per head over the chunk
// in fp32.  Phase B: lane = dimension slice, each wave sums p * v over its
// quarter of the keys; waves meet in LDS.  The block writes (m, l, o) per
// query head; the last block of the KV head (device-scope counter) merges
// all splits with a log-sum-exp and writes out.
template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void attend_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                     const void* __restrict__ V, const int32_t* __restrict__ sel,
                                                     const int32_t* __restrict__ k_eff, float* __restrict__ partial,
                                                     uint32_t* __restrict__ counters, float* __restrict__ out,
                                                     int Hq, int Hkv, int T, int top_k, int n_splits, float scale) {
    constexpr int CH = kAttnChunk;   // keys per block
    constexpr int DQ = D / 4;        // dims per wave in phase A
    constexpr int DPL = D / 64;      // dims per lane in phase B
    constexpr int PSTR = D + 2;      // partial record: o[D], m, l
    __shared__ float qs[G * D];
    __shared__ float part[4][G][CH + 1];
    __shared__ float pw[G][CH];
    __shared__ float ored[4][G][D];
    __shared__ int idx[CH];
    __shared__ float hm[G][2];
    __shared__ int last_flag;

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t q0 = (int64_t)b * Hq + (int64_t)h * G;
    int keff = k_eff[bh];
    keff = keff < 0 ? 0 : (keff > top_k ? top_k : keff);
    const int c0 = split * CH;
    const int n = keff - c0 < 0 ? 0 : (keff - c0 > CH ? CH : keff - c0);

    if (n > 0) {
        for (int i = tid; i < G * D; i += blockDim.x)
            qs[i] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(Q)[q0 * D + i])
                         : static_cast<const float*>(Q)[q0 * D + i];
        if (tid < CH) {
            int t = tid < n ? sel[bh * top_k + c0 + tid] : 0;
            idx[tid] = (t < 0 || t >= T) ? 0 : t;
        }
        __syncthreads();

        // Phase A: partial logits over dims [wv*DQ, wv*DQ + DQ) for key `lane`.
        {
            const int t = idx[lane];
            float kk[DQ];
            if (BF16) {
                const uint16_t* kr = static_cast<const uint16_t*>(K) + (bh * T + t) * D + wv * DQ;
#pragma unroll
                for (int i = 0; i < DQ; i += 8) {
                    const uint4 u = *reinterpret_cast<const uint4*>(kr + i);
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        kk[i + 2 * k] = __uint_as_float(w4[k] << 16);
                        kk[i + 2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
                    }
                }
            } else {
                const float* kr = static_cast<const float*>(K) + (bh * T + t) * D + wv * DQ;
#pragma unroll
                for (int i = 0; i < DQ; i += 4) {
                    const float4 f = *reinterpret_cast<const float4*>(kr + i);
                    kk[i] = f.x; kk[i + 1] = f.y; kk[i + 2] = f.z; kk[i + 3] = f.w;
                }
            }
#pragma unroll
            for (int i = 0; i < G; ++i) {
                float s = 0.f;
#pragma unroll
                for (int d = 0; d < DQ; ++d) s = __builtin_fmaf(qs[i * D + wv * DQ + d], kk[d], s);
                part[wv][i][lane] = s;
            }
        }
        __syncthreads();

        // Logits and per-head softmax over the chunk (wave w handles heads w, w+4).
        for (int i = wv; i < G; i += 4) {
            float s = -__builtin_inff();
            if (lane < n) s = (part[0][i][lane] + part[1][i][lane] + part[2][i][lane] + part[3][i][lane]) * scale;
            float mx = s;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            const float p = lane < n ? __expf(s - mx) : 0.f;
            float l = p;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off, 64);
            pw[i][lane] = p;
            if (lane == 0) {
                hm[i][0] = mx;
                hm[i][1] = l;
            }
        }
        __syncthreads();

        // Phase B: o[i][d] = sum_t p[i][t] * v[t][d]; wave wv takes keys wv, wv+4, ...
        {
            float o[G][DPL];
#pragma unroll
            for (int i = 0; i < G; ++i)
#pragma unroll
                for (int k = 0; k < DPL; ++k) o[i][k] = 0.f;
            for (int j = wv; j < n; j += 4) {
                const int t = idx[j];
                float v[DPL];
                if (BF16) {
                    const uint16_t* vr = static_cast<const uint16_t*>(V) + (bh * T + t) * D + lane * DPL;
                    if (DPL == 2) {
                        const uint32_t u = *reinterpret_cast<const uint32_t*>(vr);
                        v[0] = __uint_as_float(u << 16);
                        v[DPL - 1] = __uint_as_float(u & 0xffff0000u);
                    } else {
                        v[0] = bf16_to_f32(vr[0]);
                    }
                } else {
                    const float* vr = static_cast<const float*>(V) + (bh * T + t) * D + lane * DPL;
#pragma unroll
                    for (int k = 0; k < DPL; ++k) v[k] = vr[k];
                }
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float p = pw[i][j];
#pragma unroll
                    for (int k = 0; k < DPL; ++k) o[i][k] = __builtin_fmaf(p, v[k], o[i][k]);
                }
            }
#pragma unroll
            for (int i = 0; i < G; ++i)
#pragma unroll
                for (int k = 0; k < DPL; ++k) ored[wv][i][lane * DPL + k] = o[i][k];
        }
        __syncthreads();
        float* rec = partial + ((q0 * n_splits) + split) * PSTR;  // head i at + i * n_splits * PSTR
        for (int x = tid; x < G * D; x += blockDim.x) {
            const int i = x / D, d = x % D;
            rec[(int64_t)i * n_splits * PSTR + d] = ored[0][i][d] + ored[1][i][d] + ored[2][i][d] + ored[3][i][d];
        }
        if (tid < G) {
            rec[(int64_t)tid * n_splits * PSTR + D] = hm[tid][0];
            rec[(int64_t)tid * n_splits * PSTR + D + 1] = hm[tid][1];
        }
    }

    // Last block of this KV head merges the splits.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&counters[bh], 1u);
        last_flag = prev == (uint32_t)(n_splits - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    const int used = (keff + CH - 1) / CH;
    for (int x = tid; x < G * D; x += blockDim.x) {
        const int i = x / D, d = x % D;
        const float* r0 = partial + (q0 + i) * (int64_t)n_splits * PSTR;
        float M = -__builtin_inff();
        for (int s = 0; s < used; ++s) M = fmaxf(M, r0[s * PSTR + D]);
        float Ls = 0.f, O = 0.f;
        for (int s = 0; s < used; ++s) {
            const float* r = r0 + s * PSTR;
            const float w = __expf(r[D] - M);
            Ls = __builtin_fmaf(r[D + 1], w, Ls);
            O = __builtin_fmaf(r[d], w, O);
        }
        out[(q0 + i) * D + d] = used > 0 ? O / Ls : 0.f;
    }
    if (tid == 0) counters[bh] = 0u;  // ready for the next call
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// ------------------------------------------------------------------ dispatch helpers
template <int D, int G>
hipError_t bounds_g(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    const dim3 grid((unsigned)((s.NPmax + 255) / 256), s.Hkv, s.B);
    hipLaunchKernelGGL((page_bound_kernel<D, G, 8>), grid, dim3(256), 0, st, a.meta,
                       reinterpret_cast<const double*>(a.ws + a.lay.q_split), a.seq_len,
                       reinterpret_cast<double*>(a.ws + a.lay.score), s.Hkv, s.T, s.P, s.NPB, s.NPmax);
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

template <int D, bool BF16, int G>
hipError_t attend_g(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    const dim3 grid(a.lay.n_splits, s.Hkv, s.B);
    hipLaunchKernelGGL((attend_kernel<D, BF16, G>), grid, dim3(256), 0, st, a.Q, a.K, a.V, a.sel,
                       reinterpret_cast<const int32_t*>(a.ws + a.lay.k_eff),
                       reinterpret_cast<float*>(a.ws + a.lay.partial),
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

template <int D, int NB, bool BF16>
hipError_t qprep_t(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    hipLaunchKernelGGL((qprep_kernel<D, NB, BF16>), dim3(s.Hkv, s.B), dim3(D + NB), 0, st, a.Q, a.R, a.W,
                       reinterpret_cast<float*>(a.ws + a.lay.q_rot), reinterpret_cast<uint64_t*>(a.ws + a.lay.code_q),
                       reinterpret_cast<double*>(a.ws + a.lay.q_split),
                       reinterpret_cast<uint32_t*>(a.ws + a.lay.counters), s.B * s.Hkv, s.Hq, s.Hkv, s.G);
    return hipGetLastError();
}

template <int D, int NB>
hipError_t qprep_dnb(const DecodeArgs& a, hipStream_t st) {
    return a.s.bf16 ? qprep_t<D, NB, true>(a, st) : qprep_t<D, NB, false>(a, st);
}

}  // namespace

hipError_t launch_qprep(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    if (s.D == 64 && s.NB == 64) return qprep_dnb<64, 64>(a, st);
    if (s.D == 64 && s.NB == 128) return qprep_dnb<64, 128>(a, st);
    if (s.D == 128 && s.NB == 64) return qprep_dnb<128, 64>(a, st);
    return qprep_dnb<128, 128>(a, st);
}

hipError_t launch_page_bounds(const DecodeArgs& a, hipStream_t st) {
    return a.s.D == 64 ? bounds_d<64>(a, st) : bounds_d<128>(a, st);
}

hipError_t launch_select_pages(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    hipLaunchKernelGGL(select_pages_kernel, dim3(s.Hkv, s.B), dim3(kSelThreads), 0, st,
                       reinterpret_cast<const double*>(a.ws + a.lay.score), a.seq_len, a.keep_pages,
                       reinterpret_cast<int32_t*>(a.ws + a.lay.pages), reinterpret_cast<int32_t*>(a.ws + a.lay.n_pages),
                       s.Hkv, s.T, s.P, s.NPmax, a.max_keep);
    return hipGetLastError();
}

hipError_t launch_select_keys(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    auto k = s.NW == 1 ? select_keys_kernel<1> : select_keys_kernel<2>;
    hipLaunchKernelGGL(k, dim3(s.Hkv, s.B), dim3(kSelThreads), 0, st, a.codes,
                       reinterpret_cast<const uint64_t*>(a.ws + a.lay.code_q),
                       reinterpret_cast<const int32_t*>(a.ws + a.lay.pages),
                       reinterpret_cast<const int32_t*>(a.ws + a.lay.n_pages), a.seq_len,
                       reinterpret_cast<uint16_t*>(a.ws + a.lay.ham), a.sel,
                       reinterpret_cast<int32_t*>(a.ws + a.lay.k_eff), s.Hq, s.Hkv, s.G, s.T, s.P, a.max_keep,
                       a.top_k);
    return hipGetLastError();
}

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
