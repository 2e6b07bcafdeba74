// Selections of the HHR decode step, one 1024-thread block per (sequence,
// KV head):
//  - page select: the `keep` pages with the largest GKR bound, ties to the
//    lower page index ("HHR: Hierarchical Hash Retrieval for Efficient LLM
//    Generation", Abstract; rit.work HHR blog post, section "Два уровня
//    маршрутизации решают разные ошибки": low-bound pages are dropped whole);
//  - key select: LHP Hamming distances of the kept pages' keys and the top-k
//    smallest (distance, index) (same blog post, section "Почему расстояние
//    Хэмминга пропускает важные ключи"; Top-k of Appendix Table 4 on the
//    thelatestinai.com page).
// The decode step runs both in one launch, so the kept-page list goes from
// the first half to the second through LDS; the stage entry points run each
// half on its own.
//
// Latency matters more than bandwidth here (batch 1 gives 8 blocks).  Each
// thread takes up to 16 items of a chunk of 16K, lane-strided (item
// k * 1024 + tid) so every global load and store of a wave is contiguous, and
// all of them are issued up front.  Page scores are fp64 turned into
// order-preserving 64-bit keys; a block OR of (key ^ key of page 0) finds the
// bits they all share, so the MSB-first radix select starts below them, 11
// bits (2048 LDS bins) per pass.  Hamming distances are small integers: one
// LDS histogram and one scan find the threshold.  The ordered compaction
// reads per-item flags (pages) or distances (keys) back from LDS as a
// contiguous run per thread, so a single block scan of packed (before,
// at-threshold) counts gives every thread its first output position and the
// output lists come out ascending without a sort.  Inputs of more than one
// chunk loop over the chunks and re-read them.
#include "hhr_internal.h"

namespace hhr {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kRun = 16;                    // items per thread per chunk
constexpr int kChunk = kSelThreads * kRun;  // items per chunk
constexpr int kBits = 11;                   // radix digit width of the page select (measured: 11 beats 10 and 12)
constexpr int kBins = 1 << kBits;
constexpr int kListLds = kSelListLds;       // kept-page ids staged in LDS
static_assert(kChunk == kSelChunk, "chunk size");
constexpr uint16_t kNoKey = 0xFFFF;         // distance of a slot past the sequence

// Order-preserving key of a score; -0 is taken as +0 first (the two are the
// same score, so they tie and the lower page wins).
__device__ __forceinline__ uint64_t order_key(double s) {
    const uint64_t u = (uint64_t)__double_as_longlong(s + 0.0);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kRefine = 64;                 // boundary-bucket size ranked exactly by one wave
constexpr int kMaxGroup = 8;                // query heads per KV head
// sh.hist also holds the Hamming histogram (G * b + 1 bins, at most 8 * 128 + 1),
// and the split scan gives each thread two bins.
static_assert(kBins >= kMaxGroup * 128 + 1 && 2 * kSelThreads >= kMaxGroup * 128 + 1, "Hamming bins");

struct SelShared {
    int hist[kBins];
    int scan[32];
    int found[3];
    alignas(16) uint32_t red[4][16];        // per-wave OR / AND halves of the page keys (read as uint4)
    int cnt[256];                           // (round, wave) kept counts, then their prefix
    int n_bucket;                           // boundary-bucket items gathered for the exact rank
    int bidx[kRefine + 8];                  // padded: the rank loop reads 8 entries per step
    uint64_t bkey[kRefine + 8];
    uint64_t thr_key;                       // the keep-th (key, page) in (key desc, page asc)
    int thr_idx;
    int plist[kListLds];
    union {
        uint8_t pflag[kChunk];   // page select: bit 0 kept outright, bit 1 in the boundary bucket
        uint16_t dist[kChunk];   // key select: Hamming distance per slot of the chunk
    } u;
};

// Kept pages of one (b, h) into `out` (ascending, -1 padded) and, if asked,
// into LDS.  Returns the number kept.  `pre` holds the keys of the first
// chunk when the caller loaded them (lane-strided, any value past NP).
//
// One 11-bit radix pass below the bits all keys share usually leaves a
// boundary bucket of a few pages.  If it has at most 64, one wave ranks them
// exactly by (key desc, page asc) and the keep-th of that order, (kt, it),
// decides every page: kept iff key > kt or (key == kt and page <= it).
// Otherwise further passes narrow the bucket and the compaction keeps the
// first `need` pages of the final bucket in page order.
__device__ __forceinline__ int select_pages_block(const double* __restrict__ sc, int NP, int keep, int max_keep,
                                                  int32_t* __restrict__ out, bool write_out, SelShared& sh,
                                                  bool to_lds, const uint64_t (&pre)[kRun], bool preloaded) {
    const int tid = threadIdx.x;
    if (write_out)
        for (int j = keep + tid; j < max_keep; j += kSelThreads) out[j] = -1;
    if (keep == NP) {  // every page is kept
        for (int j = tid; j < NP; j += kSelThreads) {
            if (write_out) out[j] = j;
            if (to_lds && j < kListLds) sh.plist[j] = j;
        }
        return keep;
    }
    const int nchunks = (NP + kChunk - 1) / kChunk;
    const int run = nchunks <= 1 ? (NP + kSelThreads - 1) / kSelThreads : kRun;
    uint64_t key[kRun];
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            const int i = c * kChunk + k * kSelThreads + tid;
            key[k] = order_key(sc[i < NP ? i : 0]);  // entries past NP are masked by valid()
        }
    };
    auto valid = [&](int c, int k) { return k < run && c * kChunk + k * kSelThreads + tid < NP; };

    // Bits every key shares: OR over all keys of (key ^ key of page 0).
    uint64_t diff = 0;
    const uint64_t ref = order_key(sc[0]);
    if (nchunks == 1 && preloaded) {
#pragma unroll
        for (int k = 0; k < kRun; ++k) key[k] = pre[k];
#pragma unroll
        for (int k = 0; k < kRun; ++k)
            if (valid(0, k)) diff |= key[k] ^ ref;
    } else {
        for (int c = 0; c < nchunks; ++c) {
            load_chunk(c);
#pragma unroll
            for (int k = 0; k < kRun; ++k)
                if (valid(c, k)) diff |= key[k] ^ ref;
        }
    }
    const uint32_t dh = wave_or((uint32_t)(diff >> 32)), dl = wave_or((uint32_t)diff);
    if ((tid & 63) == 0) {
        sh.red[0][tid >> 6] = dh;
        sh.red[1][tid >> 6] = dl;
    }
    if (tid == 0) sh.n_bucket = 0;
    __syncthreads();
    diff = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) diff |= ((uint64_t)sh.red[0][w] << 32) | sh.red[1][w];
    uint64_t prefix, mask;
    int shift;
    if (diff == 0) {
        mask = ~0ull;  // every score is equal: the first `keep` pages win
        prefix = ref;
        shift = 0;
    } else {
        const int top = 63 - __clzll(diff);  // highest bit where scores differ
        mask = top == 63 ? 0ull : ~0ull << (top + 1);
        prefix = ref & mask;
        shift = top + 1;
    }
    int need = keep;
    bool all_in = false;   // the boundary bucket is kept whole
    bool by_pair = false;  // the exact (kt, it) rule decides
    uint64_t kt = 0;
    int it = 0;

    // Radix passes below the shared bits.
    while (!all_in && !by_pair && shift > 0) {
        const int width = shift < kBits ? shift : kBits;
        shift -= width;
        const int nb = 1 << width;
        for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            if (nchunks > 1) load_chunk(c);
#pragma unroll
            for (int k = 0; k < kRun; ++k)
                if (valid(c, k) && (key[k] & mask) == prefix) atomicAdd(&sh.hist[(key[k] >> shift) & (nb - 1)], 1);
        }
        __syncthreads();
        // Descending digits: thread i owns digits nb-1-DPT*i-j, j < DPT.
        constexpr int DPT = kBins / kSelThreads;
        int cnt[DPT], sum = 0;
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int d = nb - 1 - DPT * tid - j;
            cnt[j] = d >= 0 ? sh.hist[d] : 0;
            sum += cnt[j];
        }
        int tot;
        int above = block_excl_scan<kSelThreads>(sum, sh.scan, tot);
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            if (above < need && above + cnt[j] >= need) {
                sh.found[0] = nb - 1 - DPT * tid - j; sh.found[1] = above; sh.found[2] = cnt[j];
            }
            above += cnt[j];
        }
        __syncthreads();
        const int dig = sh.found[0];
        need -= sh.found[1];
        const int eq = sh.found[2];
        prefix |= (uint64_t)dig << shift;
        mask |= (uint64_t)(nb - 1) << shift;
        if (eq == need) {
            all_in = true;
        } else if (nchunks == 1 && eq <= kRefine) {
            // Rank the bucket's pages exactly with one wave.
#pragma unroll
            for (int k = 0; k < kRun; ++k)
                if (valid(0, k) && (key[k] & mask) == prefix) {
                    const int slot = atomicAdd(&sh.n_bucket, 1);
                    sh.bkey[slot] = key[k];
                    sh.bidx[slot] = k * kSelThreads + tid;
                }
            __syncthreads();
            if (tid < 64) {
                const int n = sh.n_bucket;
                const uint64_t mk = tid < n ? sh.bkey[tid] : 0;
                const int mi = tid < n ? sh.bidx[tid] : 0;
                int rank = 0;
                for (int j0 = 0; j0 < n; j0 += 8) {  // 8 broadcast reads in flight per step
                    uint64_t kj[8];
                    int ij[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        kj[u] = sh.bkey[j0 + u];  // entries past n are unused slots of the array
                        ij[u] = sh.bidx[j0 + u];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        rank += j0 + u < n && (kj[u] > mk || (kj[u] == mk && ij[u] < mi));
                }
                if (tid < n && rank == need - 1) {
                    sh.thr_key = mk;
                    sh.thr_idx = mi;
                }
            }
            __syncthreads();
            kt = sh.thr_key;
            it = sh.thr_idx;
            by_pair = true;
        }
        __syncthreads();
    }

    // Page p is kept iff (by_pair) its (key, p) is at or before (kt, it) in
    // (key desc, page asc) order; else iff its masked key beats the boundary
    // bucket, or it is in the bucket and (the bucket is kept whole, or it is
    // among the first `need` of the bucket in page order).
    const int cap = all_in ? 0x7fffffff : need;
    int base = 0, eq_base = 0;
    for (int c = 0; c < nchunks; ++c) {
        if (nchunks > 1) load_chunk(c);
#pragma unroll
        for (int k = 0; k < kRun; ++k)
            if (k < run) {
                const int i = c * kChunk + k * kSelThreads + tid;
                uint8_t f = 0;
                if (valid(c, k)) {
                    if (by_pair) {
                        f = key[k] > kt || (key[k] == kt && i <= it);
                    } else {
                        const uint64_t mk = key[k] & mask;
                        f = (uint8_t)((mk > prefix) | ((mk == prefix) << 1));
                    }
                }
                sh.u.pflag[k * kSelThreads + tid] = f;
            }
        __syncthreads();
        // Thread tid now owns the contiguous items [tid * run, tid * run + run).
        uint8_t f[kRun];
        int n_gt = 0, n_eq = 0;
#pragma unroll
        for (int k = 0; k < kRun; ++k) f[k] = k < run ? sh.u.pflag[tid * run + k] : (uint8_t)0;
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            n_gt += f[k] & 1;
            n_eq += f[k] >> 1;
        }
        int tot;
        const int packed = block_excl_scan<kSelThreads>((n_gt << 16) | n_eq, sh.scan, tot);
        int eq_rank = eq_base + (packed & 0xffff);
        int pos = base + (packed >> 16) + (eq_rank < cap ? eq_rank : cap);
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            bool in = f[k] & 1;
            if (f[k] >> 1) {
                in = eq_rank < cap;
                ++eq_rank;
            }
            if (in) {
                const int p = c * kChunk + tid * run + k;
                if (pos < max_keep) {
                    if (write_out) out[pos] = p;
                    if (to_lds && pos < kListLds) sh.plist[pos] = p;
                }
                ++pos;
            }
        }
        base += tot >> 16;
        eq_base += tot & 0xffff;
        __syncthreads();  // pflag is rewritten by the next chunk
    }
    return keep;
}

// select_pages_block for at most RUN * 1024 pages, RUN known at compile time
// and the scores already loaded (lane-strided, any value past NP), with the
// per-page work cut to a few instructions:
//  - the radix passes run on 32-bit order keys of the scores rounded to fp32
//    (a monotone map), so only pages tied with the threshold at fp32 need
//    the fp64 scores: a bucket of at most kRefine of them is ranked exactly
//    by one wave (64-bit keys, then page), which leaves a keep flag per
//    bucket page in LDS.  A larger tied bucket (rare: over kRefine pages
//    whose scores round to one fp32 value) falls back to the 64-bit select
//    above, re-reading the scores.
//  - page i = k * 1024 + tid sits in round k, wave tid / 64, lane tid % 64,
//    so page order is (round, wave, lane) order: the ordered list comes from
//    wave ballots and one prefix over the RUN x 16 (round, wave) counts; it
//    is built in LDS and copied out with coalesced stores.
// Needs max_keep <= kListLds.
template <int RUN>
__device__ __forceinline__ int select_pages_fast(const double* __restrict__ sc, int NP, int keep, int max_keep,
                                                 int32_t* __restrict__ out, bool write_out, SelShared& sh,
                                                 const double (&raw)[RUN]) {
    constexpr int NWV = kSelThreads / 64;
    static_assert(RUN * NWV <= 256, "one (round, wave) count per slot of sh.cnt");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (keep == NP) {  // every page is kept
        for (int j = tid; j < max_keep; j += kSelThreads) {
            if (write_out) out[j] = j < NP ? j : -1;
            if (j < NP) sh.plist[j] = j;
        }
        return keep;
    }
    bool valid[RUN];
    uint32_t key[RUN];
    uint32_t kor = 0, kand = ~0u;
#pragma unroll
    for (int k = 0; k < RUN; ++k) {
        valid[k] = k * kSelThreads + tid < NP;
        const uint32_t u = __float_as_uint((float)(raw[k] + 0.0));  // -0 as +0, then round to fp32
        key[k] = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
        kor |= valid[k] ? key[k] : 0u;
        kand &= valid[k] ? key[k] : ~0u;
    }
    // Bits every key shares: where the OR and the AND agree.  The first
    // pass's histogram is cleared under the same barrier.
    {
        const uint32_t o = wave_or(kor), a = wave_and(kand);
        if (lane == 0) {
            sh.red[0][wave] = o;
            sh.red[1][wave] = a;
        }
    }
    for (int i = tid; i < kBins; i += kSelThreads) sh.hist[i] = 0;
    if (tid == 0) sh.n_bucket = 0;
    __syncthreads();
    kor = 0;
    kand = ~0u;
#pragma unroll
    for (int w = 0; w < NWV; w += 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sh.red[0][w]);
        const uint4 b = *reinterpret_cast<const uint4*>(&sh.red[1][w]);
        kor |= a.x | a.y | a.z | a.w;
        kand &= b.x & b.y & b.z & b.w;
    }
    const uint32_t diff = kor ^ kand;
    int shift = diff == 0 ? 0 : 32 - __clz(diff);
    uint32_t mask = shift == 32 ? 0u : ~0u << shift, prefix = kand & mask;
    int need = keep;
    int state = 0;  // 0: undecided, 1: every bucket page kept, 2: bucket decided by the flags
    for (int pass = 0; state == 0 && shift > 0; ++pass) {
        const int width = shift < kBits ? shift : kBits;
        shift -= width;
        const int nb = 1 << width;
        if (pass == 0) {  // every valid key is in the bucket
#pragma unroll
            for (int k = 0; k < RUN; ++k)
                if (valid[k]) atomicAdd(&sh.hist[(key[k] >> shift) & (nb - 1)], 1);
        } else {
            for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
            __syncthreads();
#pragma unroll
            for (int k = 0; k < RUN; ++k)
                if (valid[k] && (key[k] & mask) == prefix) atomicAdd(&sh.hist[(key[k] >> shift) & (nb - 1)], 1);
        }
        __syncthreads();
        constexpr int DPT = kBins / kSelThreads;
        int cnt[DPT], sum = 0;
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int d = nb - 1 - DPT * tid - j;
            cnt[j] = d >= 0 ? sh.hist[d] : 0;
            sum += cnt[j];
        }
        int tot;
        int above = block_excl_scan<kSelThreads, false>(sum, sh.scan, tot);
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            if (above < need && above + cnt[j] >= need) {
                sh.found[0] = nb - 1 - DPT * tid - j; sh.found[1] = above; sh.found[2] = cnt[j];
            }
            above += cnt[j];
        }
        __syncthreads();
        need -= sh.found[1];
        const int eq = sh.found[2];
        prefix |= (uint32_t)sh.found[0] << shift;
        mask |= (uint32_t)(nb - 1) << shift;
        if (eq == need) {
            state = 1;
        } else if (eq <= kRefine) {
            // Gather the bucket (one LDS atomic per wave, slots from ballots),
            // rank it exactly by (64-bit key desc, page asc) and flag the
            // `need` first in LDS.
            int base = 0, wn = 0;
#pragma unroll
            for (int k = 0; k < RUN; ++k) wn += __popcll(__ballot(valid[k] && (key[k] & mask) == prefix));
            if (lane == 0 && wn > 0) base = atomicAdd(&sh.n_bucket, wn);
            base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
            for (int k = 0; k < RUN; ++k) {
                const bool in = valid[k] && (key[k] & mask) == prefix;
                const uint64_t bm = __ballot(in);
                if (in) {
                    const int slot = base + lanes_below(bm);
                    sh.bkey[slot] = order_key(raw[k]);
                    sh.bidx[slot] = k * kSelThreads + tid;
                }
                base += __popcll(bm);
            }
            __syncthreads();
            if (tid < 64) {
                const int n = sh.n_bucket;
                const uint64_t mk = tid < n ? sh.bkey[tid] : 0;
                const int mi = tid < n ? sh.bidx[tid] : 0;
                int rank = 0;
                for (int j0 = 0; j0 < n; j0 += 8) {
                    uint64_t kj[8];
                    int ij[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        kj[u] = sh.bkey[j0 + u];
                        ij[u] = sh.bidx[j0 + u];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        rank += j0 + u < n && (kj[u] > mk || (kj[u] == mk && ij[u] < mi));
                }
                if (tid < n) sh.u.pflag[mi] = rank < need;
            }
            __syncthreads();
            state = 2;
        }
    }
    if (state == 0) {  // over kRefine pages tie at fp32 on the boundary
        const uint64_t unused[kRun] = {};
        return select_pages_block(sc, NP, keep, max_keep, out, write_out, sh, true, unused, false);
    }

    // Kept pages: above the bucket, or in it and (all kept or flagged).
    bool g[RUN];
#pragma unroll
    for (int k = 0; k < RUN; ++k) {
        const uint32_t mk = key[k] & mask;
        g[k] = valid[k] && (mk > prefix || (mk == prefix && (state == 1 || sh.u.pflag[k * kSelThreads + tid])));
        const uint64_t bm = __ballot(g[k]);
        if (lane == 0) sh.cnt[k * NWV + wave] = __popcll(bm);
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefix of the counts in (round, wave) order
        constexpr int E = RUN * NWV, EPL = (E + 63) / 64;
        int v[EPL], sum = 0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int idx = lane * EPL + e;
            v[e] = idx < E ? sh.cnt[idx] : 0;
            sum += v[e];
        }
        int run = wave_incl_scan(sum) - sum;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const int idx = lane * EPL + e;
            if (idx < E) sh.cnt[idx] = run;
            run += v[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < RUN; ++k) {
        const uint64_t bm = __ballot(g[k]);
        if (g[k]) sh.plist[sh.cnt[k * NWV + wave] + lanes_below(bm)] = k * kSelThreads + tid;
    }
    __syncthreads();
    if (write_out)
        for (int j = tid; j < max_keep; j += kSelThreads) out[j] = j < keep ? sh.plist[j] : -1;
    return keep;
}

template <int NW>
__device__ __forceinline__ void load_code(const uint64_t* __restrict__ ck, int t, uint64_t (&kc)[NW]) {
    if constexpr (NW == 2) {
        const u32x4 v = load_stream16(ck + (int64_t)t * 2);  // each candidate's code is read once
        kc[0] = ((uint64_t)v.y << 32) | v.x;
        kc[1] = ((uint64_t)v.w << 32) | v.z;
    } else {
        kc[0] = ck[t];
    }
}

// One split block's share of a head's key scan: the Hamming distances of
// slots [split * per, split * per + per) of the kept pages (page list in
// LDS), written to hm and counted in the LDS histogram `hist` (zeroed by the
// caller, before a barrier); then the block's inclusive cumulative histogram
// goes to cum and its counts into the head's (ghist).  The split count keeps
// per <= kCompactSlots, so a thread has at most kSplitRun slots.
constexpr int kSplitRun = kCompactSlots / kSelThreads;
static_assert(kSplitRun * kSelThreads == kCompactSlots, "a split's slots fit the run");
template <int NW>
__device__ __forceinline__ void split_scan(const uint64_t* __restrict__ ck, const uint64_t (&cq)[kMaxGroup * NW], int G,
                                           const int* plist, int nslots, int P, int s_end, int w_start, int max_keep,
                                           uint16_t* __restrict__ hm, int* hist, int* scan, int split, int S,
                                           uint32_t* __restrict__ cum, uint32_t* __restrict__ ghist) {
    const int NBINS = G * NW * 64 + 1;
    const int tid = threadIdx.x;
    const int lp = 31 - __clz(P);  // P is a power of two
    const int per = (nslots + S - 1) / S;
    const int lo = split * per < nslots ? split * per : nslots, hi = lo + per < nslots ? lo + per : nslots;
    int tk[kSplitRun];
    uint64_t kc[kSplitRun][NW];
#pragma unroll
    for (int k = 0; k < kSplitRun; ++k) {  // lookups, then every code load, before any use
        const int s = lo + k * kSelThreads + tid;
        const int ss = s < hi ? s : 0;
        const int t = plist[ss >> lp] * P + (ss & (P - 1));
        tk[k] = (s < hi && t >= s_end && t < w_start) ? t : -1;
    }
#pragma unroll
    for (int k = 0; k < kSplitRun; ++k) load_code<NW>(ck, tk[k] >= 0 ? tk[k] : 0, kc[k]);
#pragma unroll
    for (int k = 0; k < kSplitRun; ++k) {
        const int s = lo + k * kSelThreads + tid;
        int hsum = 0;
#pragma unroll
        for (int i = 0; i < kMaxGroup; ++i) {
            if (i >= G) break;  // uniform
#pragma unroll
            for (int w = 0; w < NW; ++w) hsum += __popcll(cq[i * NW + w] ^ kc[k][w]);
        }
        if (tk[k] >= 0) atomicAdd(&hist[hsum], 1);
        if (s < hi) hm[s] = tk[k] < 0 ? kNoKey : (uint16_t)hsum;
    }
    if (split == 0)
        for (int s = nslots + tid; s < max_keep * P; s += kSelThreads) hm[s] = kNoKey;
    __syncthreads();
    // Thread i owns bins 2i and 2i+1: inclusive cumulative counts, and the
    // head's histogram (device atomics on the bins this block hit).
    const int b0 = 2 * tid;
    const int c0 = b0 < NBINS ? hist[b0] : 0, c1 = b0 + 1 < NBINS ? hist[b0 + 1] : 0;
    int tot;
    const int before = block_excl_scan<kSelThreads, false>(c0 + c1, scan, tot);
    if (b0 < NBINS) {
        cum[split * NBINS + b0] = (uint32_t)(before + c0);
        if (c0) atomicAdd(&ghist[b0], (uint32_t)c0);
    }
    if (b0 + 1 < NBINS) {
        cum[split * NBINS + b0 + 1] = (uint32_t)(before + c0 + c1);
        if (c1) atomicAdd(&ghist[b0 + 1], (uint32_t)c1);
    }
}

// LDSLIST: the kept-page list is read from LDS (else from the workspace); a
// compile-time choice, so every read is a plain LDS or global load rather
// than a generic one that waits on both queues.
// S > 1 (the decode step; every candidate in one chunk, the page list in
// LDS): the S blocks of a (b, h) each scan 1/S of the candidate slots, write
// their distances, their cumulative histogram (cum) and add their histogram
// into the head's (ghist).  The threshold, the ordered compaction and the
// attention then run in the compact+attend kernel.
//
// Forced keys (nsink, window > 0, single-block path only): the keys
// [0, s_end) and [w_start, L) take no part in the ranking (distance 0xFFFF)
// and are listed around the ranked ones: so = sinks, ranked, window.
template <int NW, bool LDSLIST>
__device__ __forceinline__ void select_keys_block(const uint64_t* __restrict__ ck, const uint64_t* __restrict__ cqg,
                                                  int G, const int32_t* __restrict__ pl, int np, int L,
                                                  int P, int max_keep, int top_k, uint16_t* __restrict__ hm,
                                                  int32_t* __restrict__ so, int32_t* __restrict__ keff_out,
                                                  SelShared& sh, int split, int S, uint32_t* __restrict__ cum,
                                                  uint32_t* __restrict__ ghist, int nsink = 0, int window = 0) {
    constexpr int NB = NW * 64;
    const int NBINS = G * NB + 1;
    const int tid = threadIdx.x;
    const int s_end = nsink < L ? nsink : L;
    const int w_start = L - window > s_end ? L - window : s_end;  // ranked keys: [s_end, w_start)
    const int sel_cap = top_k + nsink + window;
    const int nslots = np * P;
    const int lp = 31 - __clz(P);  // P is a power of two
    uint64_t cq[kMaxGroup * NW];
#pragma unroll
    for (int i = 0; i < kMaxGroup * NW; ++i) cq[i] = cqg[i < G * NW ? i : 0];
    for (int i = tid; i < NBINS; i += kSelThreads) sh.hist[i] = 0;

    const int nchunks = (nslots + kChunk - 1) / kChunk;
    const int run = nchunks <= 1 ? (nslots + kSelThreads - 1) / kSelThreads : kRun;
    int Hreg[kRun];
    auto page_of = [&](int s) { return LDSLIST ? sh.plist[s >> lp] : pl[s >> lp]; };
    // Distances of the chunk's slots c * kChunk + k * 1024 + tid (-1: no key).
    auto distances = [&](int c) {
        uint64_t kc[kRun][NW];
        // Every page lookup, then every code load, before any use; the item
        // guard is uniform (a scalar branch), the lane guard only clamps.
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            Hreg[k] = -1;
            if (k < run) {
                const int s = c * kChunk + k * kSelThreads + tid;
                const int ss = s < nslots ? s : 0;
                const int t = page_of(ss) * P + (ss & (P - 1));
                Hreg[k] = (s < nslots && t >= s_end && t < w_start) ? t : -1;
            }
        }
#pragma unroll
        for (int k = 0; k < kRun; ++k)
            if (k < run) load_code<NW>(ck, Hreg[k] >= 0 ? Hreg[k] : 0, kc[k]);
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            int hsum = 0;
#pragma unroll
            for (int i = 0; i < kMaxGroup; ++i) {
                if (i >= G) break;  // uniform
#pragma unroll
                for (int w = 0; w < NW; ++w) hsum += __popcll(cq[i * NW + w] ^ kc[k][w]);
            }
            Hreg[k] = Hreg[k] >= 0 ? hsum : -1;
        }
    };
    auto stage = [&]() {  // the chunk's distances into LDS, lane-strided
#pragma unroll
        for (int k = 0; k < kRun; ++k)
            if (k < run) sh.u.dist[k * kSelThreads + tid] = Hreg[k] < 0 ? kNoKey : (uint16_t)Hreg[k];
    };
    __syncthreads();

    if (LDSLIST && S > 1) {
        split_scan<NW>(ck, cq, G, sh.plist, nslots, P, s_end, w_start, max_keep, hm, sh.hist, sh.scan, split, S, cum,
                       ghist);
        return;
    } else {
        for (int c = 0; c < nchunks; ++c) {
            distances(c);
#pragma unroll
            for (int k = 0; k < kRun; ++k) {
                const int s = c * kChunk + k * kSelThreads + tid;
                if (k < run && s < nslots) hm[s] = Hreg[k] < 0 ? kNoKey : (uint16_t)Hreg[k];
                if (Hreg[k] >= 0) atomicAdd(&sh.hist[Hreg[k]], 1);
            }
            if (nchunks == 1) stage();
        }
        for (int s = nslots + tid; s < max_keep * P; s += kSelThreads) hm[s] = kNoKey;
        __syncthreads();
    }

    // Threshold h*: the ascending cumulative count reaches k_eff.
    int hs, need, keff;
    {
        const int b0 = 2 * tid;
        const int c0 = b0 < NBINS ? sh.hist[b0] : 0, c1 = b0 + 1 < NBINS ? sh.hist[b0 + 1] : 0;
        int nvalid;
        const int below0 = block_excl_scan<kSelThreads>(c0 + c1, sh.scan, nvalid);
        keff = nvalid < top_k ? nvalid : top_k;
        if (tid == 0) {
            sh.found[0] = NBINS;
            sh.found[1] = 0;
        }
        __syncthreads();
        if (keff > 0) {
            if (below0 < keff && below0 + c0 >= keff) {
                sh.found[0] = b0; sh.found[1] = keff - below0;
            } else if (below0 + c0 < keff && below0 + c0 + c1 >= keff) {
                sh.found[0] = b0 + 1; sh.found[1] = keff - below0 - c0;
            }
        }
        __syncthreads();
        hs = sh.found[0];
        need = sh.found[1];
    }

    // Keep H < h*, and the first `need` candidates with H == h* in slot order.
    int base = 0, eq_base = 0;
    for (int c = 0; c < nchunks; ++c) {
        if (nchunks > 1) {
            distances(c);
            stage();
            __syncthreads();
        }
        // Thread tid owns the contiguous slots [tid * run, tid * run + run) of the chunk.
        uint16_t hv[kRun];
        int pg[kRun];
        int n_lt = 0, n_eq = 0;
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            hv[k] = kNoKey;
            pg[k] = 0;
            if (k < run) {
                hv[k] = sh.u.dist[tid * run + k];
                const int s = c * kChunk + tid * run + k;
                pg[k] = page_of(s < nslots ? s : 0);
            }
        }
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            if (k >= run) hv[k] = kNoKey;
            n_lt += hv[k] < hs;
            n_eq += hv[k] == hs;
        }
        int tot;
        const int packed = block_excl_scan<kSelThreads>((n_lt << 16) | n_eq, sh.scan, tot);
        int eq_rank = eq_base + (packed & 0xffff);
        int pos = base + (packed >> 16) + (eq_rank < need ? eq_rank : need);
#pragma unroll
        for (int k = 0; k < kRun; ++k) {
            bool in = hv[k] < hs;
            if (hv[k] == hs) {
                in = eq_rank < need;
                ++eq_rank;
            }
            if (in) {
                const int s = c * kChunk + tid * run + k;
                if (pos < top_k) so[s_end + pos] = pg[k] * P + (s & (P - 1));
                ++pos;
            }
        }
        base += tot >> 16;
        eq_base += tot & 0xffff;
        __syncthreads();  // dist is rewritten by the next chunk
    }
    for (int j = tid; j < s_end; j += kSelThreads) so[j] = j;
    for (int j = tid; j < L - w_start; j += kSelThreads) so[s_end + keff + j] = w_start + j;
    const int listed = s_end + keff + (L - w_start);
    for (int j = listed + tid; j < sel_cap; j += kSelThreads) so[j] = -1;
    if (tid == 0) *keff_out = listed;
}

// Key half of the select kernels, after the page list (LDS or workspace).
template <int NW, bool KEYS>
__device__ __forceinline__ void keys_half(SelShared& sh, const uint64_t* __restrict__ codes,
                                          const uint64_t* __restrict__ code_q, int32_t* __restrict__ pl, int np,
                                          bool list_in_lds, uint16_t* __restrict__ ham, int32_t* __restrict__ sel,
                                          int32_t* __restrict__ k_eff_out, uint32_t* __restrict__ cum,
                                          uint32_t* __restrict__ ghist, int split, int S, int b, int h, int64_t bh,
                                          int64_t bhd, int Gh, int T, int P, int L, int max_keep, int top_k,
                                          int nsink, int window) {
    if (!KEYS) return;
    const uint64_t* ck = codes + bhd * (int64_t)T * NW;  // the unit's data head
    const uint64_t* cq = code_q + bh * Gh * NW;  // the group's Gh query codes
    uint16_t* hm = ham + bh * (int64_t)max_keep * P;
    const int NBINS = Gh * NW * 64 + 1;
    uint32_t* cb = cum + bh * (int64_t)S * NBINS;
    uint32_t* gb = ghist + bh * (int64_t)NBINS;
    const int64_t cap = (int64_t)top_k + nsink + window;
    if (list_in_lds)
        select_keys_block<NW, true>(ck, cq, Gh, pl, np, L, P, max_keep, top_k, hm, sel + bh * cap, k_eff_out + bh,
                                    sh, split, S, cb, gb, nsink, window);
    else if (split == 0)  // the page list is not in LDS: one block does the whole key select
        select_keys_block<NW, false>(ck, cq, Gh, pl, np, L, P, max_keep, top_k, hm, sel + bh * cap,
                                     k_eff_out + bh, sh, 0, 1, cb, gb, nsink, window);
}

// With S > 1 the compact+attend kernel's merging block polls the split
// partials until none holds the sentinel: each select block sets its own
// split's (o, m, l) of the group's query heads to it, after its last load.
__device__ __forceinline__ void mark_partials(float* __restrict__ part_o, float* __restrict__ part_ml, int64_t q0,
                                              int G, int D, int split, int pstride) {
    const float sent = __uint_as_float(kPartSentinel);
    const int tid = threadIdx.x, n4 = D / 4;
    for (int x = tid; x < G * n4; x += kSelThreads)
        *reinterpret_cast<float4*>(part_o + ((q0 + x / n4) * pstride + split) * D + (x % n4) * 4) =
            make_float4(sent, sent, sent, sent);
    if (tid < 2 * G) part_ml[((q0 + tid / 2) * pstride + split) * 2 + (tid & 1)] = sent;
}

// General select kernel: any number of pages (chunks of 16K) and slots.
template <int NW, bool PAGES, bool KEYS>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const double* __restrict__ score, const int32_t* __restrict__ keep_pages, const uint64_t* __restrict__ codes,
    const uint64_t* __restrict__ code_q, const int32_t* __restrict__ seq_len, int32_t* __restrict__ pages,
    int32_t* __restrict__ n_pages, uint16_t* __restrict__ ham, int32_t* __restrict__ sel,
    int32_t* __restrict__ k_eff_out, uint32_t* __restrict__ cum, uint32_t* __restrict__ ghist, float* __restrict__ part_o,
    float* __restrict__ part_ml, int pstride, int D, int S, int G, int Gh, int Hq, int Hkv, int T, int P, int64_t NPmax,
    int max_keep, int top_k, int nsink, int window, int share) {
    __shared__ SelShared sh;
    const int b = blockIdx.y, split = blockIdx.z;
    // Per-query-head selection: a KV head's units on its XCD (as the select kernels).
    int h = blockIdx.x;
    if (share > 1) {  // block-uniform
        const unsigned Hd = (unsigned)(Hkv / share);
        h = (int)((blockIdx.x % Hd) * (unsigned)share + blockIdx.x / Hd);
    }
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t bhd = data_head(b, h, Hkv, share);  // the unit's data head
    uint64_t pre[kRun];  // unused here: the general page select loads its chunks itself
    const int L = clamp_len(seq_len[b], T);
    const int NP = (int)n_pages_of(L, P);
    int32_t* pl = pages + bh * max_keep;
    int np;
    bool list_in_lds = false;
    if (PAGES) {
        int keep = keep_pages[b];
        keep = keep < 1 ? 1 : keep;
        keep = keep > NP ? NP : keep;
        keep = keep > max_keep ? max_keep : keep;
        np = select_pages_block(score + bh * NPmax, NP, keep, max_keep, pl, split == 0, sh, KEYS, pre, false);
        if (threadIdx.x == 0 && split == 0) n_pages[bh] = np;
        list_in_lds = KEYS && np <= kListLds;
        __syncthreads();
    } else {
        np = n_pages[bh];
        np = np < 0 ? 0 : (np > max_keep ? max_keep : np);  // memory safety for a hand-filled workspace
        if (np <= kListLds) {
            for (int i = threadIdx.x; i < np; i += kSelThreads) sh.plist[i] = pl[i];
            list_in_lds = true;
        }
        __syncthreads();
    }
    keys_half<NW, KEYS>(sh, codes, code_q, pl, np, list_in_lds, ham, sel, k_eff_out, cum, ghist, split, S, b, h, bh,
                        bhd, Gh, T, P, L, max_keep, top_k, nsink, window);
    if (KEYS && S > 1) mark_partials(part_o, part_ml, (int64_t)b * Hq + (int64_t)h * G, G, D, split, pstride);
}

// Split key scan after a separate page-select launch (S > 1, kept-page list
// within kListLds): only the split block's share of the scan, so the kernel
// holds few registers and two 1024-thread blocks share a compute unit.
struct SplitShared {
    int hist[kMaxGroup * 128 + 1];
    int scan[32];
    int plist[kListLds];
};

template <int NW>
__global__ __launch_bounds__(kSelThreads) void select_split_kernel(
    const double* __restrict__ score, const int32_t* __restrict__ keep_pages, const uint64_t* __restrict__ codes,
    const uint64_t* __restrict__ code_q, const int32_t* __restrict__ seq_len, int32_t* __restrict__ pages,
    int32_t* __restrict__ n_pages, uint16_t* __restrict__ ham, int32_t* __restrict__ sel,
    int32_t* __restrict__ k_eff_out, uint32_t* __restrict__ cum, uint32_t* __restrict__ ghist, float* __restrict__ part_o,
    float* __restrict__ part_ml, int pstride, int D, int S, int G, int Gh, int Hq, int Hkv, int T, int P, int64_t NPmax,
    int max_keep, int top_k, int nsink, int window, int share) {
    __shared__ SplitShared sh;
    const int b = blockIdx.y, split = blockIdx.z, tid = threadIdx.x;
    // Per-query-head selection: a KV head's units on its XCD (as the select kernels).
    int h = blockIdx.x;
    if (share > 1) {  // block-uniform
        const unsigned Hd = (unsigned)(Hkv / share);
        h = (int)((blockIdx.x % Hd) * (unsigned)share + blockIdx.x / Hd);
    }
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t bhd = data_head(b, h, Hkv, share);  // the unit's data head
    const int NBINS = Gh * NW * 64 + 1;
    uint64_t cq[kMaxGroup * NW];
#pragma unroll
    for (int i = 0; i < kMaxGroup * NW; ++i) cq[i] = code_q[bh * Gh * NW + (i < Gh * NW ? i : 0)];
    const int L = clamp_len(seq_len[b], T);
    int np = n_pages[bh];
    np = np < 0 ? 0 : (np > max_keep ? max_keep : np);  // memory safety for a hand-filled workspace
    np = np > kListLds ? kListLds : np;                  // the launch guarantees max_keep <= kListLds
    const int32_t* pl = pages + bh * max_keep;
    for (int i = tid; i < np; i += kSelThreads) sh.plist[i] = pl[i];
    for (int i = tid; i < NBINS; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    const int s_end = nsink < L ? nsink : L;
    const int w_start = L - window > s_end ? L - window : s_end;
    split_scan<NW>(codes + bhd * (int64_t)T * NW, cq, Gh, sh.plist, np * P, P, s_end, w_start, max_keep,
                   ham + bh * (int64_t)max_keep * P, sh.hist, sh.scan, split, S, cum + bh * (int64_t)S * NBINS,
                   ghist + bh * (int64_t)NBINS);
    mark_partials(part_o, part_ml, (int64_t)b * Hq + (int64_t)h * G, G, D, split, pstride);
}

// Hamming stage alone: the distance of every candidate slot of the kept
// pages (pages, n_pages and the query codes from the workspace) to the
// group's query codes, summed over the Gh codes, or 0xFFFF for a slot past
// the kept pages, past the sequence, or on a sink or window key -- the
// values the key select writes to ham.  One thread per slot.
template <int NW>
__global__ __launch_bounds__(256) void hamming_kernel(const uint64_t* __restrict__ codes,
                                                      const uint64_t* __restrict__ code_q,
                                                      const int32_t* __restrict__ seq_len,
                                                      const int32_t* __restrict__ pages,
                                                      const int32_t* __restrict__ n_pages, uint16_t* __restrict__ ham,
                                                      int Gh, int Hkv, int T, int P, int max_keep, int nsink,
                                                      int window, int share) {
    const int h = blockIdx.y, b = blockIdx.z;
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nslot = (int64_t)max_keep * P;
    if (s >= nslot) return;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    int np = n_pages[bh];
    np = np < 0 ? 0 : (np > max_keep ? max_keep : np);
    const int s_end = nsink < L ? nsink : L;
    const int w_start = L - window > s_end ? L - window : s_end;  // ranked keys: [s_end, w_start)
    const int lp = 31 - __clz(P);
    uint16_t out = kNoKey;
    if (s < (int64_t)np * P) {
        const int64_t t = (int64_t)pages[bh * max_keep + (s >> lp)] * P + (s & (P - 1));
        if (t >= s_end && t < w_start) {
            const uint64_t* ck = codes + data_head(b, h, Hkv, share) * (int64_t)T * NW;
            uint64_t kc[NW];
            load_code<NW>(ck, (int)t, kc);
            const uint64_t* cq = code_q + bh * Gh * NW;
            int hsum = 0;
            for (int i = 0; i < Gh; ++i)
#pragma unroll
                for (int w = 0; w < NW; ++w) hsum += __popcll(cq[i * NW + w] ^ kc[w]);
            out = (uint16_t)hsum;
        }
    }
    ham[bh * nslot + s] = out;
}

// Fast select kernel: at most RUN * 1024 pages (one chunk, RUN items per
// thread known at compile time) and at most kListLds kept pages; scores are
// loaded before the length is known.
template <int NW, int RUN, bool KEYS>
__global__ __launch_bounds__(kSelThreads) void select_fast_kernel(
    const double* __restrict__ score, const int32_t* __restrict__ keep_pages, const uint64_t* __restrict__ codes,
    const uint64_t* __restrict__ code_q, const int32_t* __restrict__ seq_len, int32_t* __restrict__ pages,
    int32_t* __restrict__ n_pages, uint16_t* __restrict__ ham, int32_t* __restrict__ sel,
    int32_t* __restrict__ k_eff_out, uint32_t* __restrict__ cum, uint32_t* __restrict__ ghist, float* __restrict__ part_o,
    float* __restrict__ part_ml, int pstride, int D, int S, int G, int Gh, int Hq, int Hkv, int T, int P, int64_t NPmax,
    int max_keep, int top_k, int nsink, int window, int share) {
    __shared__ SelShared sh;
    const int b = blockIdx.y, split = blockIdx.z;
    // Per-query-head selection: the units of one data head take the grid
    // slots of that head's XCD (workgroups go to the XCDs in turn), where its
    // page-bound pass left their scores.
    int h = blockIdx.x;
    if (share > 1) {  // block-uniform
        const unsigned Hd = (unsigned)(Hkv / share);
        h = (int)((blockIdx.x % Hd) * (unsigned)share + blockIdx.x / Hd);
    }
    const int64_t bh = (int64_t)b * Hkv + h;
    const int64_t bhd = data_head(b, h, Hkv, share);  // the unit's data head
    const double* scp = score + bh * NPmax;
    double raw[RUN];
#pragma unroll
    for (int k = 0; k < RUN; ++k) {  // every load issued, unconditionally (clamped), before any use
        const int64_t i = (int64_t)k * kSelThreads + threadIdx.x;
        raw[k] = __builtin_nontemporal_load(scp + (i < NPmax ? i : NPmax - 1));  // measured faster hinted
    }
    const int L = clamp_len(seq_len[b], T);
    const int NP = (int)n_pages_of(L, P);
    int keep = keep_pages[b];
    keep = keep < 1 ? 1 : keep;
    keep = keep > NP ? NP : keep;
    keep = keep > max_keep ? max_keep : keep;
    int32_t* pl = pages + bh * max_keep;
    const int np = select_pages_fast<RUN>(scp, NP, keep, max_keep, pl, split == 0, sh, raw);
    if (threadIdx.x == 0 && split == 0) n_pages[bh] = np;
    __syncthreads();
    if (KEYS) {  // max_keep <= kListLds here, so the page list is in LDS
        const int NBINS = Gh * NW * 64 + 1;
        select_keys_block<NW, true>(codes + bhd * (int64_t)T * NW, code_q + bh * Gh * NW, Gh,
                                    pl, np, L, P, max_keep, top_k, ham + bh * (int64_t)max_keep * P,
                                    sel + bh * ((int64_t)top_k + nsink + window), k_eff_out + bh, sh, split, S,
                                    cum + bh * (int64_t)S * NBINS, ghist + bh * (int64_t)NBINS, nsink, window);
        if (S > 1) mark_partials(part_o, part_ml, (int64_t)b * Hq + (int64_t)h * G, G, D, split, pstride);
    }
}

template <typename Kernel>
hipError_t select_launch(Kernel kernel, const DecodeArgs& a, int S, hipStream_t st) {
    const Shape& s = a.s;
    float* po = reinterpret_cast<float*>(a.ws + a.lay.partial);
    const size_t n_po = (size_t)s.B * s.Hq * a.lay.part_splits * s.D;
    hipLaunchKernelGGL(kernel, dim3(s.Hkv, s.B, S), dim3(kSelThreads), 0, st,
                       reinterpret_cast<const double*>(a.ws + a.lay.score), a.keep_pages, a.codes,
                       reinterpret_cast<const uint64_t*>(a.ws + (s.ham_mean ? a.lay.code_qm : a.lay.code_q)), a.seq_len,
                       reinterpret_cast<int32_t*>(a.ws + a.lay.pages), reinterpret_cast<int32_t*>(a.ws + a.lay.n_pages),
                       reinterpret_cast<uint16_t*>(a.ws + a.lay.ham), a.sel,
                       reinterpret_cast<int32_t*>(a.ws + a.lay.k_eff), reinterpret_cast<uint32_t*>(a.ws + a.lay.kcum),
                       reinterpret_cast<uint32_t*>(a.ws + a.lay.counters) + a.lay.ghist_off, po, po + n_po,
                       a.lay.part_splits, s.D, S, s.G, s.Gh, s.Hq, s.Hkv, s.T, s.P, s.NPmax, a.max_keep, a.top_k,
                       s.nsink, s.window, s.share);
    return hipGetLastError();
}

// Page select (+ keys): the fast kernel when every page fits one chunk.
template <int NW, bool KEYS>
hipError_t select_pages_nw(const DecodeArgs& a, int S, hipStream_t st) {
    const int64_t np = a.s.NPmax;
    if (a.max_keep > kListLds) return select_launch(select_kernel<NW, true, KEYS>, a, S, st);
    if (np <= 4 * kSelThreads) return select_launch(select_fast_kernel<NW, 4, KEYS>, a, S, st);
    if (np <= 8 * kSelThreads) return select_launch(select_fast_kernel<NW, 8, KEYS>, a, S, st);
    if (np <= kChunk) return select_launch(select_fast_kernel<NW, 16, KEYS>, a, S, st);
    return select_launch(select_kernel<NW, true, KEYS>, a, S, st);
}

// ============================================================== TopK (Oracle) key select
// The keys of one (b, h) with the largest exact logit z (fp64, from the
// logit kernel), equal z to the lower key, listed ascending.  The logit
// kernel leaves a histogram of topk_bin(z), a monotone 12-bit digit of z, so:
//  - collect (many blocks per (b, h)): finds the boundary digit d1 whose bin
//    holds the k_eff-th largest z, counts each block's keys above it and
//    appends the bin's keys (64-bit order key, index) to a bucket;
//  - threshold (one block per (b, h)): ranks the bucket exactly -- a radix
//    select on the order keys, then, among keys tied at the boundary value,
//    on the index -- and turns each block's count into its output offset;
//  - write (many blocks): every block compacts its selected keys in order.
// A bucket over kTopkCap keys (heavy ties) falls back to the block select
// above on all the scores.

// Boundary digit of the `need` largest: found[0] = d1, found[1] = keys in
// higher bins, found[2] = keys in bin d1.  `need` >= 1 and <= the total.
template <int NT>
__device__ __forceinline__ void topk_boundary(const uint32_t* __restrict__ gh, int need, int* scan, int* found) {
    constexpr int BPT = kTopkBins / NT;
    const int tid = threadIdx.x;
    int c[BPT], sum = 0;
#pragma unroll
    for (int m = 0; m < BPT; ++m) {
        c[m] = (int)gh[kTopkBins - 1 - BPT * tid - m];
        sum += c[m];
    }
    int tot;
    int above = block_excl_scan<NT>(sum, scan, tot);
#pragma unroll
    for (int m = 0; m < BPT; ++m) {
        if (above < need && above + c[m] >= need) {
            found[0] = kTopkBins - 1 - BPT * tid - m;
            found[1] = above;
            found[2] = c[m];
        }
        above += c[m];
    }
    __syncthreads();
}

// MSB-first radix select (descending) over the block's N-per-thread values
// v (valid where ok; `count` valid in all, 1 <= need): on return the values
// with (v & mask) > prefix rank above the boundary bucket {(v & mask) ==
// prefix}, `need` of which are taken, and all_in says that is all of it.
// Bits every valid value shares are skipped first.
template <int N>
__device__ __forceinline__ void radix_desc(const uint64_t (&v)[N], const bool (&ok)[N], int count, int& need,
                                           uint64_t& prefix, uint64_t& mask, bool& all_in, SelShared& sh) {
    const int tid = threadIdx.x;
    if (need >= count) {  // block-uniform
        prefix = 0;
        mask = 0;
        all_in = true;
        return;
    }
    uint64_t o = 0, a = ~0ull;
#pragma unroll
    for (int k = 0; k < N; ++k)
        if (ok[k]) {
            o |= v[k];
            a &= v[k];
        }
    const uint32_t oh = wave_or((uint32_t)(o >> 32)), ol = wave_or((uint32_t)o);
    const uint32_t ah = wave_and((uint32_t)(a >> 32)), al = wave_and((uint32_t)a);
    if ((tid & 63) == 0) {
        sh.red[0][tid >> 6] = oh;
        sh.red[1][tid >> 6] = ol;
        sh.red[2][tid >> 6] = ah;
        sh.red[3][tid >> 6] = al;
    }
    __syncthreads();
    o = 0;
    a = ~0ull;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) {
        o |= ((uint64_t)sh.red[0][w] << 32) | sh.red[1][w];
        a &= ((uint64_t)sh.red[2][w] << 32) | sh.red[3][w];
    }
    __syncthreads();
    const uint64_t diff = o ^ a;
    all_in = false;
    if (diff == 0) {  // every valid value is equal
        prefix = a;
        mask = ~0ull;
        return;
    }
    const int top = 63 - __clzll(diff);
    mask = top == 63 ? 0ull : ~0ull << (top + 1);
    prefix = a & mask;
    int shift = top + 1;
    while (!all_in && shift > 0) {
        const int width = shift < kBits ? shift : kBits;
        shift -= width;
        const int nb = 1 << width;
        for (int i = tid; i < nb; i += kSelThreads) sh.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < N; ++k)
            if (ok[k] && (v[k] & mask) == prefix) atomicAdd(&sh.hist[(v[k] >> shift) & (nb - 1)], 1);
        __syncthreads();
        constexpr int DPT = kBins / kSelThreads;
        int cnt[DPT], sum = 0;
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int d = nb - 1 - DPT * tid - j;
            cnt[j] = d >= 0 ? sh.hist[d] : 0;
            sum += cnt[j];
        }
        int tot;
        int above = block_excl_scan<kSelThreads>(sum, sh.scan, tot);
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            if (above < need && above + cnt[j] >= need) {
                sh.found[0] = nb - 1 - DPT * tid - j;
                sh.found[1] = above;
                sh.found[2] = cnt[j];
            }
            above += cnt[j];
        }
        __syncthreads();
        need -= sh.found[1];
        prefix |= (uint64_t)sh.found[0] << shift;
        mask |= (uint64_t)(nb - 1) << shift;
        all_in = sh.found[2] == need;
        __syncthreads();
    }
}

// Selection rule of a boundary-bin key with order key v and index t.
__device__ __forceinline__ bool topk_in_bucket(uint64_t v, int t, uint64_t p1, uint64_t m1, uint64_t p2,
                                               uint64_t m2) {
    const uint64_t w = (uint64_t)(0xffffffffu - (uint32_t)t);
    return (v & m1) > p1 || ((v & m1) == p1 && (w & m2) >= p2);
}

constexpr int kTopkRun = kTopkBlk / 256;  // keys per thread of a collect / write block

__global__ __launch_bounds__(256) void topk_collect_kernel(const double* __restrict__ score,
                                                           const uint32_t* __restrict__ hist,
                                                           const int32_t* __restrict__ seq_len,
                                                           uint32_t* __restrict__ bfill, uint64_t* __restrict__ bkey,
                                                           int32_t* __restrict__ bidx, int32_t* __restrict__ ocnt,
                                                           int Hkv, int T, int top_k, int nblk_max) {
    __shared__ int scan[32];
    __shared__ int found[3];
    __shared__ uint32_t bbase;
    const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int base = j * kTopkBlk;
    if (base >= L) return;  // block-uniform
    const int keff = top_k < L ? top_k : L;
    const double* sc = score + bh * T;
    double s[kTopkRun];
#pragma unroll
    for (int k = 0; k < kTopkRun; ++k) {
        const int i = base + k * 256 + tid;
        s[k] = sc[i < L ? i : L - 1];
    }
    topk_boundary<256>(hist + bh * kTopkBins, keff, scan, found);
    const uint32_t d1 = (uint32_t)found[0];
    const int e1 = found[2];
    int n_out = 0, n_b = 0;
    bool isb[kTopkRun];
#pragma unroll
    for (int k = 0; k < kTopkRun; ++k) {
        const bool valid = base + k * 256 + tid < L;
        const uint32_t bin = topk_bin(s[k]);
        n_out += valid && bin > d1;
        isb[k] = valid && bin == d1;
        n_b += isb[k];
    }
    int tot;
    block_excl_scan<256>(n_out, scan, tot);
    if (tid == 0) ocnt[bh * nblk_max + j] = tot;
    if (e1 > kTopkCap) return;  // the threshold kernel falls back to the full select
    int totb;
    int pos = block_excl_scan<256>(n_b, scan, totb);
    if (tid == 0 && totb > 0) bbase = atomicAdd(&bfill[bh], (uint32_t)totb);
    __syncthreads();
    if (n_b == 0) return;
    pos += (int)bbase;
#pragma unroll
    for (int k = 0; k < kTopkRun; ++k)
        if (isb[k]) {
            if (pos < kTopkCap) {
                bkey[bh * kTopkCap + pos] = order_key(s[k]);
                bidx[bh * kTopkCap + pos] = base + k * 256 + tid;
            }
            ++pos;
        }
}

// info per (b, h), 16 words: [0] 0 = rule below, 1 = list already written;
// [1] d1; [2..3] p1; [4..5] m1; [6..7] p2; [8..9] m2 (low word first).
constexpr int kTopkBucketRun = kTopkCap / kSelThreads;

__global__ __launch_bounds__(kSelThreads) void topk_threshold_kernel(
    const double* __restrict__ score, const uint32_t* __restrict__ hist, const uint64_t* __restrict__ bkey,
    const int32_t* __restrict__ bidx, const int32_t* __restrict__ ocnt, int32_t* __restrict__ off,
    uint32_t* __restrict__ info, int32_t* __restrict__ sel, int32_t* __restrict__ k_eff,
    const int32_t* __restrict__ seq_len, int Hkv, int T, int top_k, int nblk_max) {
    __shared__ SelShared sh;
    __shared__ int cntb[kTopkMaxBlk];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int keff = top_k < L ? top_k : L;
    int32_t* so = sel + bh * top_k;
    uint32_t* inf = info + bh * 16;
    for (int x = keff + tid; x < top_k; x += kSelThreads) so[x] = -1;
    if (tid == 0) k_eff[bh] = keff;
    if (keff == 0) {  // block-uniform
        if (tid == 0) inf[0] = 1u;
        return;
    }
    topk_boundary<kSelThreads>(hist + bh * kTopkBins, keff, sh.scan, sh.found);
    const uint32_t d1 = (uint32_t)sh.found[0];
    const int c_above = sh.found[1], e1 = sh.found[2];
    __syncthreads();
    if (e1 > kTopkCap) {  // block-uniform: heavy ties; select on every score
        uint64_t pre[kRun];
        select_pages_block(score + bh * T, L, keff, top_k, so, true, sh, false, pre, false);
        if (tid == 0) inf[0] = 1u;
        return;
    }
    uint64_t v[kTopkBucketRun];
    int32_t ix[kTopkBucketRun];
    bool ok[kTopkBucketRun];
#pragma unroll
    for (int k = 0; k < kTopkBucketRun; ++k) {
        const int slot = k * kSelThreads + tid;
        ok[k] = slot < e1;
        v[k] = ok[k] ? bkey[bh * kTopkCap + slot] : 0ull;
        ix[k] = ok[k] ? bidx[bh * kTopkCap + slot] : 0;
    }
    int need = keff - c_above;
    uint64_t p1, m1, p2 = 0, m2 = 0;
    bool all1;
    radix_desc<kTopkBucketRun>(v, ok, e1, need, p1, m1, all1, sh);
    if (!all1) {  // `need` of the keys whose order key is exactly p1: the lowest indices
        uint64_t w[kTopkBucketRun];
        bool okt[kTopkBucketRun];
        int nt = 0;
#pragma unroll
        for (int k = 0; k < kTopkBucketRun; ++k) {
            okt[k] = ok[k] && v[k] == p1;
            w[k] = (uint64_t)(0xffffffffu - (uint32_t)ix[k]);
            nt += okt[k];
        }
        int ntie;
        block_excl_scan<kSelThreads>(nt, sh.scan, ntie);
        bool all2;
        radix_desc<kTopkBucketRun>(w, okt, ntie, need, p2, m2, all2, sh);
    }
    if (tid == 0) {
        inf[0] = 0u;
        inf[1] = d1;
        inf[2] = (uint32_t)p1;
        inf[3] = (uint32_t)(p1 >> 32);
        inf[4] = (uint32_t)m1;
        inf[5] = (uint32_t)(m1 >> 32);
        inf[6] = (uint32_t)p2;
        inf[7] = (uint32_t)(p2 >> 32);
        inf[8] = (uint32_t)m2;
        inf[9] = (uint32_t)(m2 >> 32);
    }
    // Each collect block's output offset: its keys above d1 plus its taken
    // bucket keys, summed over the blocks before it.
    const int nblk = (L + kTopkBlk - 1) / kTopkBlk;
    for (int x = tid; x < nblk; x += kSelThreads) cntb[x] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTopkBucketRun; ++k)
        if (ok[k] && (uint32_t)ix[k] < (uint32_t)L && topk_in_bucket(v[k], ix[k], p1, m1, p2, m2))
            atomicAdd(&cntb[ix[k] / kTopkBlk], 1);
    __syncthreads();
    int run = 0;
    for (int x0 = 0; x0 < nblk; x0 += kSelThreads) {
        const int x = x0 + tid;
        const int c = x < nblk ? ocnt[bh * nblk_max + x] + cntb[x] : 0;
        int tot;
        const int pre = block_excl_scan<kSelThreads>(c, sh.scan, tot);
        if (x < nblk) off[bh * nblk_max + x] = run + pre;
        run += tot;
    }
}

__global__ __launch_bounds__(256) void topk_write_kernel(const double* __restrict__ score,
                                                         const uint32_t* __restrict__ info,
                                                         const int32_t* __restrict__ off,
                                                         const int32_t* __restrict__ seq_len,
                                                         int32_t* __restrict__ sel, int Hkv, int T, int top_k,
                                                         int nblk_max) {
    __shared__ int scan[32];
    const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int64_t bh = (int64_t)b * Hkv + h;
    const int L = clamp_len(seq_len[b], T);
    const int base = j * kTopkBlk;
    if (base >= L) return;  // block-uniform
    const uint32_t* inf = info + bh * 16;
    if (inf[0] != 0u) return;
    const uint32_t d1 = inf[1];
    const uint64_t p1 = ((uint64_t)inf[3] << 32) | inf[2], m1 = ((uint64_t)inf[5] << 32) | inf[4];
    const uint64_t p2 = ((uint64_t)inf[7] << 32) | inf[6], m2 = ((uint64_t)inf[9] << 32) | inf[8];
    const int t0 = base + tid * kTopkRun;  // this thread's contiguous keys
    const double* sc = score + bh * T;
    double s[kTopkRun];
#pragma unroll
    for (int m = 0; m < kTopkRun; ++m) s[m] = t0 + m < L ? sc[t0 + m] : 0.0;
    bool in[kTopkRun];
    int n = 0;
#pragma unroll
    for (int m = 0; m < kTopkRun; ++m) {
        const uint32_t bin = topk_bin(s[m]);
        in[m] = t0 + m < L &&
                (bin > d1 || (bin == d1 && topk_in_bucket(order_key(s[m]), t0 + m, p1, m1, p2, m2)));
        n += in[m];
    }
    int tot;
    int pos = off[bh * nblk_max + j] + block_excl_scan<256>(n, scan, tot);
    int32_t* so = sel + bh * top_k;
#pragma unroll
    for (int m = 0; m < kTopkRun; ++m)
        if (in[m]) {
            if (pos < top_k) so[pos] = t0 + m;
            ++pos;
        }
}

}  // namespace

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t st) {
    const Shape& s = a.d.s;
    const TopkLayout& t = a.tl;
    char* ws = a.d.ws;
    const dim3 grid((unsigned)t.nblk, s.Hkv, s.B);
    uint32_t* bfill = reinterpret_cast<uint32_t*>(ws + a.d.lay.counters) + (size_t)s.B * s.Hkv;
    hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(256), 0, st, reinterpret_cast<const double*>(ws + t.score),
                       reinterpret_cast<const uint32_t*>(ws + t.hist), a.d.seq_len, bfill,
                       reinterpret_cast<uint64_t*>(ws + t.bkey), reinterpret_cast<int32_t*>(ws + t.bidx),
                       reinterpret_cast<int32_t*>(ws + t.ocnt), s.Hkv, s.T, a.d.top_k, t.nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_threshold_kernel, dim3(s.Hkv, s.B), dim3(kSelThreads), 0, st,
                       reinterpret_cast<const double*>(ws + t.score), reinterpret_cast<const uint32_t*>(ws + t.hist),
                       reinterpret_cast<const uint64_t*>(ws + t.bkey), reinterpret_cast<const int32_t*>(ws + t.bidx),
                       reinterpret_cast<const int32_t*>(ws + t.ocnt), reinterpret_cast<int32_t*>(ws + t.off),
                       reinterpret_cast<uint32_t*>(ws + t.info), a.d.sel,
                       reinterpret_cast<int32_t*>(ws + a.d.lay.k_eff), a.d.seq_len, s.Hkv, s.T, a.d.top_k, t.nblk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_write_kernel, grid, dim3(256), 0, st, reinterpret_cast<const double*>(ws + t.score),
                       reinterpret_cast<const uint32_t*>(ws + t.info), reinterpret_cast<const int32_t*>(ws + t.off),
                       a.d.seq_len, a.d.sel, s.Hkv, s.T, a.d.top_k, t.nblk);
    return hipGetLastError();
}

hipError_t launch_select(const DecodeArgs& a, hipStream_t st) {
    const int S = a.lay.sel_splits;
    if (a.lay.sel_pages_apart) {  // the page list once per head, then S key-scan blocks per head read it
        const hipError_t e = select_pages_nw<1, false>(a, 1, st);
        if (e != hipSuccess) return e;
        if (a.max_keep > kListLds) return hipErrorInvalidValue;  // the split count is chosen so
        return a.s.NW == 1 ? select_launch(select_split_kernel<1>, a, S, st)
                           : select_launch(select_split_kernel<2>, a, S, st);
    }
    return a.s.NW == 1 ? select_pages_nw<1, true>(a, S, st) : select_pages_nw<2, true>(a, S, st);
}
hipError_t launch_select_pages(const DecodeArgs& a, hipStream_t st) {
    return select_pages_nw<1, false>(a, 1, st);  // the page half does not depend on the code width
}
hipError_t launch_hamming(const DecodeArgs& a, hipStream_t st) {
    const Shape& s = a.s;
    const int64_t nslot = (int64_t)a.max_keep * s.P;
    if (nslot <= 0) return hipSuccess;
    const dim3 grid((unsigned)((nslot + 255) / 256), s.Hkv, s.B);
    const uint64_t* cq = reinterpret_cast<const uint64_t*>(a.ws + (s.ham_mean ? a.lay.code_qm : a.lay.code_q));
    const int32_t* pg = reinterpret_cast<const int32_t*>(a.ws + a.lay.pages);
    const int32_t* npg = reinterpret_cast<const int32_t*>(a.ws + a.lay.n_pages);
    uint16_t* hm = reinterpret_cast<uint16_t*>(a.ws + a.lay.ham);
    if (s.NW == 1)
        hipLaunchKernelGGL(hamming_kernel<1>, grid, dim3(256), 0, st, a.codes, cq, a.seq_len, pg, npg, hm, s.Gh, s.Hkv,
                           s.T, s.P, a.max_keep, s.nsink, s.window, s.share);
    else
        hipLaunchKernelGGL(hamming_kernel<2>, grid, dim3(256), 0, st, a.codes, cq, a.seq_len, pg, npg, hm, s.Gh, s.Hkv,
                           s.T, s.P, a.max_keep, s.nsink, s.window, s.share);
    return hipGetLastError();
}
hipError_t launch_select_keys(const DecodeArgs& a, hipStream_t st) {
    return a.s.NW == 1 ? select_launch(select_kernel<1, false, true>, a, 1, st)
                       : select_launch(select_kernel<2, false, true>, a, 1, st);
}

}  // namespace hhr
