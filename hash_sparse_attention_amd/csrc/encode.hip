// Cache encode: GKR page metadata (per-page per-dimension max/min of R_h k)
// and LHP key codes (sign bits of W_h k).  "HHR: Hierarchical Hash Retrieval
// for Efficient LLM Generation", Abstract; rit.work HHR blog post, section
// "Два уровня маршрутизации решают разные ошибки" (pages of adjacent keys,
// stored page bounds).
//
// Every projection is the canonical fp32 chain acc = fma(M[r][c], k[c], acc),
// c ascending from acc = +0, so any IEEE implementation of it -- on either
// mapping below -- produces the same bits.
//
// This file holds the bulk mapping on gfx950 (wave64), used for many keys:
// one lane per key.  The key row sits in VGPRs as fp32; the rows of
// [R_h; W_h] are wave-uniform, so they come in through scalar loads, one
// chunk ahead, and feed v_fma as SGPR operands.  A page is P adjacent lanes: its max/min is a
// butterfly over P lanes.  Each lane packs its own code words and stores
// them contiguously.  Appends of a few keys (the token just generated) use
// the row-per-lane projection kernel instead.
#include "hhr_internal.h"

namespace hhr {
namespace {

struct EncRange {
    int s, e;  // keys [s, e) of this sequence, clamped
};

__device__ __forceinline__ EncRange enc_range(const int32_t* start, const int32_t* count, int b, int max_count,
                                              int T) {
    int s = start[b];
    s = s < 0 ? 0 : (s > T ? T : s);
    int c = count[b];
    c = c < 0 ? 0 : c;
    c = c > max_count ? max_count : c;
    c = c > T - s ? T - s : c;
    return {s, s + c};
}

// ------------------------------------------------------------------ bulk
template <int D, int NB, bool BF16, bool M16, bool MS>
__global__ __launch_bounds__(256) void encode_bulk_kernel(const void* __restrict__ K, const float* __restrict__ R,
                                                          const float* __restrict__ W,
                                                          const int32_t* __restrict__ start,
                                                          const int32_t* __restrict__ count, int max_count,
                                                          float* __restrict__ meta, uint64_t* __restrict__ codes,
                                                          int Hkv, int T, int P, int64_t NPB) {
    constexpr int NW = NB / 64;
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * Hkv + h;
    const EncRange rg = enc_range(start, count, b, max_count, T);
    if (rg.e <= rg.s) return;
    const int base = (rg.s / P) * P + blockIdx.x * 256;  // a page boundary
    if (base + (int)(threadIdx.x & ~63) >= rg.e) return;  // whole wave past the range (no barriers below)
    const int t = base + threadIdx.x;
    const bool valid = t < rg.e;

    float k[D];
    if (valid) {
        if (BF16) {
            const uint4* kr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(K) + (bh * T + t) * D);
#pragma unroll
            for (int i = 0; i < D / 8; ++i) {
                const uint4 u = kr[i];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    k[8 * i + 2 * q] = __uint_as_float(w4[q] << 16);
                    k[8 * i + 2 * q + 1] = __uint_as_float(w4[q] & 0xffff0000u);
                }
            }
        } else {
            const float4* kr = reinterpret_cast<const float4*>(static_cast<const float*>(K) + (bh * T + t) * D);
#pragma unroll
            for (int i = 0; i < D / 4; ++i) {
                const float4 f = kr[i];
                k[4 * i] = f.x; k[4 * i + 1] = f.y; k[4 * i + 2] = f.z; k[4 * i + 3] = f.w;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < D; ++i) k[i] = 0.f;
    }

    // Rows of [R_h; W_h] stream in as wave-uniform chunks of CH columns:
    // scalar loads into SGPRs, which feed v_fma as operands.  Scalar loads
    // can return out of order, so a wait can only be for all of them; one
    // chunk is kept in flight: wait for the current chunk, issue the next
    // one, then run the CH FMAs of the current one, which cover its latency
    // (across row boundaries too).  Each chain is the canonical one: acc = +0,
    // c ascending.
    constexpr int CH = 32;       // columns per chunk
    constexpr int NCH = D / CH;  // chunks per row: even, so buffer A holds a row's first chunk on entry
    static_assert(NCH % 2 == 0, "chunks per row");
    const float* Rh = R + (int64_t)h * D * D;
    const float* Wh = W + (int64_t)h * NB * D;
    float A[CH], Bc[CH];
    auto load = [&](float (&c)[CH], const float* p) {
#pragma unroll
        for (int i = 0; i < CH; ++i) c[i] = p[i];
    };
    // The chain of the row at p_row; leaves the first chunk of the row at p_next in A.
    auto row_chain = [&](const float* p_row, const float* p_next) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            float(&cur)[CH] = (q & 1) ? Bc : A;
            float(&nxt)[CH] = (q & 1) ? A : Bc;
            // Wait for chunk q (then the only scalar load in flight), then issue
            // chunk q + 1, so the wait never covers the chunk just issued.
            // 0xc07f: lgkmcnt(0), vmcnt and expcnt left at their maximum.
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_sched_barrier(0);
            load(nxt, q + 1 < NCH ? p_row + (q + 1) * CH : p_next);
            __builtin_amdgcn_sched_barrier(0);  // the loads (and their address math) stay ahead of the FMAs
#pragma unroll
            for (int i = 0; i < CH; ++i) acc = __builtin_fmaf(cur[i], k[q * CH + i], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        return acc;
    };
    load(A, Rh);

    // Rotation rows, two at a time so a page leader stores one float4 per pair.
    const int p = t / P;
    const bool leader = (t - base) % P == 0 && valid;
    float4* mrow = reinterpret_cast<float4*>(meta) + (bh * NPB + p / 64) * (D / 2) * 64 + (p & 63);
    // bf16 meta: dimension quad r/4 of page p is one 16-byte slot; a pair is its (r % 4) / 2 half.
    uint2* mrow16 = reinterpret_cast<uint2*>(meta) + ((bh * NPB + p / 64) * (D / 4) * 64 + (p & 63)) * 2;
#pragma unroll 1
    for (int r = 0; r < D; r += 2) {
        float mx[2], mn[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float* row = Rh + (int64_t)(r + q) * D;
            const float acc = row_chain(row, r + q + 1 < D ? row + D : Wh);  // then hash row 0
            const float v = acc == 0.f ? 0.f : acc;
            mx[q] = valid ? v : -__builtin_inff();
            mn[q] = valid ? v : __builtin_inff();
            for (int o = 1; o < P; o <<= 1) {
                mx[q] = fmaxf(mx[q], __shfl_xor(mx[q], o, 64));
                mn[q] = fminf(mn[q], __shfl_xor(mn[q], o, 64));
            }
        }
        if (leader) {
            // The outputs are read by later steps, not by this launch or the
            // next: stored with the nontemporal hint (measured 2-3% faster).
            if (MS) {  // sign-split layout: dimension d's max run, then its min run, 64 pages each
                const int64_t e0 = ((bh * NPB + p / 64) * D + r) * 128 + (p & 63);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    if (M16) {
                        uint16_t* m = reinterpret_cast<uint16_t*>(meta) + e0 + q * 128;
                        __builtin_nontemporal_store((uint16_t)bf16_up(mx[q]), m);
                        __builtin_nontemporal_store((uint16_t)bf16_down(mn[q]), m + 64);
                    } else {
                        float* m = meta + e0 + q * 128;
                        __builtin_nontemporal_store(mx[q], m);
                        __builtin_nontemporal_store(mn[q], m + 64);
                    }
                }
            } else if (M16) {
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                const u2v m2 = {bf16_pair_out(mx[0], mn[0]), bf16_pair_out(mx[1], mn[1])};
                __builtin_nontemporal_store(m2, reinterpret_cast<u2v*>(mrow16 + (r / 4) * 64 * 2 + (r % 4) / 2));
            } else {
                typedef float f4v __attribute__((ext_vector_type(4)));
                const f4v m4 = {mx[0], mn[0], mx[1], mn[1]};
                __builtin_nontemporal_store(m4, reinterpret_cast<f4v*>(mrow + (r / 2) * 64));
            }
        }
    }

    // Hash rows: this lane's own code words.
    uint64_t code[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) code[w] = 0;
#pragma unroll 1
    for (int j = 0; j < NB; ++j) {
        const float* row = Wh + (int64_t)j * D;
        const float acc = row_chain(row, j + 1 < NB ? row + D : row);  // the last row reloads itself (in bounds)
        if (acc > 0.f) code[j >> 6] |= 1ull << (j & 63);
    }
    if (valid && t >= rg.s) {
        uint64_t* cp = codes + (bh * T + t) * NW;
#pragma unroll
        for (int w = 0; w < NW; ++w) __builtin_nontemporal_store(code[w], cp + w);
    }
}

template <int D, int NB, bool BF16, bool M16>
hipError_t launch_dnb(const Shape& s, const void* K, const float* R, const float* W, const int32_t* start,
                      const int32_t* count, int max_count, float* meta, uint64_t* codes, hipStream_t st) {
    const int tiles = (max_count + s.P - 1 + 255) / 256;  // keys [floor(s/P)P, e) in 256-key tiles
    auto kern = s.msplit ? encode_bulk_kernel<D, NB, BF16, M16, true> : encode_bulk_kernel<D, NB, BF16, M16, false>;
    hipLaunchKernelGGL(kern, dim3(tiles, s.Hkv, s.B), dim3(256), 0, st, K, R, W, start, count, max_count, meta, codes,
                       s.Hkv, s.T, s.P, s.NPB);
    return hipGetLastError();
}

template <int D, int NB>
hipError_t launch_dt(const Shape& s, const void* K, const float* R, const float* W, const int32_t* start,
                     const int32_t* count, int max_count, float* meta, uint64_t* codes, hipStream_t st) {
    if (s.meta16)
        return s.bf16 ? launch_dnb<D, NB, true, true>(s, K, R, W, start, count, max_count, meta, codes, st)
                      : launch_dnb<D, NB, false, true>(s, K, R, W, start, count, max_count, meta, codes, st);
    return s.bf16 ? launch_dnb<D, NB, true, false>(s, K, R, W, start, count, max_count, meta, codes, st)
                  : launch_dnb<D, NB, false, false>(s, K, R, W, start, count, max_count, meta, codes, st);
}

}  // namespace

hipError_t launch_encode(const Shape& s, const void* K, const float* R, const float* W, const int32_t* start,
                         const int32_t* count, int max_count, float* meta, uint64_t* codes, hipStream_t st) {
    if (s.D == 64 && s.NB == 64) return launch_dt<64, 64>(s, K, R, W, start, count, max_count, meta, codes, st);
    if (s.D == 64 && s.NB == 128) return launch_dt<64, 128>(s, K, R, W, start, count, max_count, meta, codes, st);
    if (s.D == 128 && s.NB == 64) return launch_dt<128, 64>(s, K, R, W, start, count, max_count, meta, codes, st);
    return launch_dt<128, 128>(s, K, R, W, start, count, max_count, meta, codes, st);
}

}  // namespace hhr
