// Cache encode: GKR page metadata (per-page per-dimension max/min of R_h k)
// and LHP key codes (sign bits of W_h k).  "HHR: Hierarchical Hash Retrieval
// for Efficient LLM Generation", Abstract; rit.work HHR blog post, section
// "Два уровня маршрутизации решают разные ошибки" (pages of adjacent keys,
// stored page bounds).
//
// Every projection is the canonical fp32 chain acc = fma(M[r][c], k[c], acc),
// c ascending from acc = +0, so any IEEE implementation of it -- the tiled
// mapping below or the row-per-lane projection kernel -- produces the same
// bits.
//
// This file holds the bulk mapping on gfx950 (wave64), used for many keys: a
// register-tiled product of [R_h; W_h] with a 64-key tile, both operands
// staged in LDS (below).  Appends of a few keys (the token just generated)
// use the row-per-lane projection kernel instead.
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
// A block owns a tile of 64 consecutive keys (a page boundary first, so every
// page of the tile is whole: P divides 64) and all D + NB rows of [R_h; W_h],
// one wave per 64 rows.  Columns arrive in chunks of kEncCols: the keys (widened
// to fp32) and the rows are staged in LDS with coalesced 16-byte loads, then
// each thread runs an 8 x 8 register tile -- keys kg + 8j, rows rg + 8i of its
// wave's 64, lane = kg + 8 rg -- reading 4 columns of a key or row per
// 16-byte LDS read, so 16 reads feed 256 FMAs.  Every accumulator is one
// canonical chain (columns ascending from +0).  Padding each LDS row by 4
// floats (a stride of kEncStride = 20) puts the 8 keys (or rows) a read
// touches in 8 distinct 4-bank groups.
//
// Epilogue: a rotation wave reduces each dimension's values over a page --
// within the thread over the keys of its register tile, then across the kg
// lanes -- pairs dimensions r, r + 1 (lanes 8 apart) and stores the page's
// metadata; a hash wave sets bit rg + 8i of its code word per key and ORs the
// word over the 8 rg lanes, and lane (kg, rg) stores key kg + 8 rg's word.
constexpr int kEncKeys = 64;            // keys per tile
constexpr int kEncCols = 16;            // columns per staged chunk
constexpr int kEncStride = kEncCols + 4;  // LDS row stride in floats (16-byte aligned, conflict-free reads)

template <int D, int NB, bool BF16, bool M16, bool MS>
__global__ __launch_bounds__(D + NB) __attribute__((amdgpu_waves_per_eu(3))) void encode_tile_kernel(
    const void* __restrict__ K, const float* __restrict__ R, const float* __restrict__ W,
    const int32_t* __restrict__ start, const int32_t* __restrict__ count, int max_count, float* __restrict__ meta,
    uint64_t* __restrict__ codes, int Hkv, int T, int P, int64_t NPB) {
    constexpr int MR = D + NB, NT = MR, NCH = D / kEncCols;
    static_assert(MR % 64 == 0 && D % kEncCols == 0 && kEncCols % 8 == 0, "tile shape");
    static_assert(kEncStride % 4 == 0 && kEncStride >= kEncCols, "16-byte aligned LDS rows");
    __shared__ float ks[kEncKeys * kEncStride];  // [key][column] of the chunk
    __shared__ float ms[MR * kEncStride];        // [row][column] of the chunk
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t bh = (int64_t)b * Hkv + h;
    const EncRange rng = enc_range(start, count, b, max_count, T);
    if (rng.e <= rng.s) return;
    const int tb = (rng.s / P) * P + blockIdx.x * kEncKeys;  // a page boundary
    if (tb >= rng.e) return;                                  // block-uniform
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = lane & 7, rg = lane >> 3;
    const float* Rh = R + (int64_t)h * D * D;
    const float* Wh = W + (int64_t)h * NB * D;

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    for (int c = 0; c < NCH; ++c) {
        if (c) __syncthreads();  // the previous chunk has been read
        // Keys: 64 x kEncCols columns in 16-byte pieces; keys past the range are zero.
        if constexpr (BF16) {
            constexpr int PK = kEncCols / 8;  // pieces per key
            for (int x = tid; x < kEncKeys * PK; x += NT) {
                const int kk = x / PK, q = x % PK, t = tb + kk;
                u32x4 u = {0u, 0u, 0u, 0u};
                if (t < rng.e)
                    u = load_stream16(static_cast<const uint16_t*>(K) + (bh * T + t) * D + c * kEncCols + q * 8);
                float* dst = ks + kk * kEncStride + q * 8;
                *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                                              __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
                *reinterpret_cast<float4*>(dst + 4) = make_float4(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u),
                                                                  __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u));
            }
        } else {
            constexpr int PK = kEncCols / 4;
            for (int x = tid; x < kEncKeys * PK; x += NT) {
                const int kk = x / PK, q = x % PK, t = tb + kk;
                u32x4 u = {0u, 0u, 0u, 0u};
                if (t < rng.e) u = load_stream16(static_cast<const float*>(K) + (bh * T + t) * D + c * kEncCols + q * 4);
                *reinterpret_cast<float4*>(ks + kk * kEncStride + q * 4) =
                    make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
            }
        }
        // Rows: MR x kEncCols columns, PR pieces of 4 a row, PR a thread.
        constexpr int PR = kEncCols / 4;
#pragma unroll
        for (int u = 0; u < PR; ++u) {
            const int x = tid + u * NT, r = x / PR, q = x % PR;
            const float* src = (r < D ? Rh + (int64_t)r * D : Wh + (int64_t)(r - D) * D) + c * kEncCols + q * 4;
            *reinterpret_cast<float4*>(ms + r * kEncStride + q * 4) = *reinterpret_cast<const float4*>(src);
        }
        __syncthreads();
        const float* kp = ks + kg * kEncStride;
        const float* rp = ms + (wave * 64 + rg) * kEncStride;
#pragma unroll
        for (int c4 = 0; c4 < kEncCols; c4 += 4) {
            float4 kv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) kv[j] = *reinterpret_cast<const float4*>(kp + 8 * j * kEncStride + c4);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 rv = *reinterpret_cast<const float4*>(rp + 8 * i * kEncStride + c4);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    acc[i][j] = __builtin_fmaf(rv.x, kv[j].x, acc[i][j]);
                    acc[i][j] = __builtin_fmaf(rv.y, kv[j].y, acc[i][j]);
                    acc[i][j] = __builtin_fmaf(rv.z, kv[j].z, acc[i][j]);
                    acc[i][j] = __builtin_fmaf(rv.w, kv[j].w, acc[i][j]);
                }
            }
        }
    }

    if (wave * 64 < D) {  // rotation rows: page max / min (wave-uniform branch)
        // With P >= 8 the 64 / P pages of the tile start at keys 8j, j a
        // multiple of P / 8, and lane kg = page stores; with P < 8 a page is
        // P adjacent kg lanes of one j, and its first lane stores.
        bool ok[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ok[j] = tb + kg + 8 * j < rng.e;
        const int pj = P >= 8 ? P / 8 : 1;  // register-tile keys per page
        const int pl = P >= 8 ? 8 : P;      // lanes per page
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wave * 64 + rg + 8 * i;  // dimension
            float mx[8], mn[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = acc[i][j] == 0.f ? 0.f : acc[i][j];
                mx[j] = ok[j] ? v : -__builtin_inff();
                mn[j] = ok[j] ? v : __builtin_inff();
            }
#pragma unroll
            for (int sj = 1; sj < 8; sj <<= 1) {
                if (sj < pj) {  // uniform
#pragma unroll
                    for (int j = 0; j < 8; j += 2 * sj) {
                        mx[j] = fmaxf(mx[j], mx[j + sj]);
                        mn[j] = fminf(mn[j], mn[j + sj]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j % pj) continue;  // uniform
                for (int o = 1; o < pl; o <<= 1) {
                    mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], o, 64));
                    mn[j] = fminf(mn[j], __shfl_xor(mn[j], o, 64));
                }
                // Dimension r + 1 sits 8 lanes up (rg + 1).
                const float mx1 = __shfl_xor(mx[j], 8, 64), mn1 = __shfl_xor(mn[j], 8, 64);
                const int kk0 = P >= 8 ? 8 * j : ((kg + 8 * j) & ~(P - 1));  // the page's first key in the tile
                const bool store = (rg & 1) == 0 && (P >= 8 ? kg == j / pj : (kg & (P - 1)) == 0) && tb + kk0 < rng.e;
                if (!store) continue;
                const int64_t p = (tb + kk0) / P;
                // The outputs are read by later steps, not by this launch or the
                // next: stored with the nontemporal hint.
                if (MS) {  // sign-split layout: dimension d's max run, then its min run, 64 pages each
                    const int64_t e0 = ((bh * NPB + p / 64) * D + r) * 128 + (p & 63);
                    if (M16) {
                        uint16_t* m = reinterpret_cast<uint16_t*>(meta) + e0;
                        __builtin_nontemporal_store((uint16_t)bf16_up(mx[j]), m);
                        __builtin_nontemporal_store((uint16_t)bf16_down(mn[j]), m + 64);
                        __builtin_nontemporal_store((uint16_t)bf16_up(mx1), m + 128);
                        __builtin_nontemporal_store((uint16_t)bf16_down(mn1), m + 192);
                    } else {
                        float* m = meta + e0;
                        __builtin_nontemporal_store(mx[j], m);
                        __builtin_nontemporal_store(mn[j], m + 64);
                        __builtin_nontemporal_store(mx1, m + 128);
                        __builtin_nontemporal_store(mn1, m + 192);
                    }
                } else if (M16) {  // dimension quad r / 4 is one 16-byte slot; the pair is its (r % 4) / 2 half
                    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                    const u2v m2 = {bf16_pair_out(mx[j], mn[j]), bf16_pair_out(mx1, mn1)};
                    uint2* m = reinterpret_cast<uint2*>(meta) + ((bh * NPB + p / 64) * (D / 4) * 64 + (p & 63)) * 2 +
                               (r / 4) * 64 * 2 + (r % 4) / 2;
                    __builtin_nontemporal_store(m2, reinterpret_cast<u2v*>(m));
                } else {  // dimension pair r / 2 is one 16-byte slot
                    typedef float f4v __attribute__((ext_vector_type(4)));
                    const f4v m4 = {mx[j], mn[j], mx1, mn1};
                    float4* m = reinterpret_cast<float4*>(meta) + (bh * NPB + p / 64) * (D / 2) * 64 + (r / 2) * 64 + (p & 63);
                    __builtin_nontemporal_store(m4, reinterpret_cast<f4v*>(m));
                }
            }
        }
    } else {  // hash rows: code word wave - D / 64, bit rg + 8i
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo[j] = 0u;
            hi[j] = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lo[j] |= (acc[i][j] > 0.f ? 1u : 0u) << (rg + 8 * i);
                hi[j] |= (acc[i + 4][j] > 0.f ? 1u : 0u) << (rg + 8 * i);
            }
#pragma unroll
            for (int o = 8; o < 64; o <<= 1) {
                lo[j] |= __shfl_xor(lo[j], o, 64);
                hi[j] |= __shfl_xor(hi[j], o, 64);
            }
        }
        uint32_t wl = lo[0], wh = hi[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            wl = rg == j ? lo[j] : wl;
            wh = rg == j ? hi[j] : wh;
        }
        const int t = tb + kg + 8 * rg;
        if (t >= rng.s && t < rng.e)
            __builtin_nontemporal_store(((uint64_t)wh << 32) | wl, codes + (bh * T + t) * (NB / 64) + (wave - D / 64));
    }
}

template <int D, int NB, bool BF16, bool M16>
hipError_t launch_dnb(const Shape& s, const void* K, const float* R, const float* W, const int32_t* start,
                      const int32_t* count, int max_count, float* meta, uint64_t* codes, hipStream_t st) {
    const int tiles = (max_count + s.P - 1 + kEncKeys - 1) / kEncKeys;  // keys [floor(s/P)P, e) in 64-key tiles
    auto kern = s.msplit ? encode_tile_kernel<D, NB, BF16, M16, true> : encode_tile_kernel<D, NB, BF16, M16, false>;
    hipLaunchKernelGGL(kern, dim3(tiles, s.Hkv, s.B), dim3(D + NB), 0, st, K, R, W, start, count, max_count, meta, codes,
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
