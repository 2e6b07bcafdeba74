// Host side of libhhr: argument validation, workspace layout, and the
// extern "C" entry points declared in include/hhr.h.  Every check runs
// before anything is enqueued; kernels run on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "hhr_internal.h"

namespace hhr {
namespace {

thread_local std::string g_last_error;

hhr_status fail(hhr_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

hhr_status ok() {
    g_last_error.clear();
    return HHR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hhr_status make_shape(const hhr_dims* d, Shape& s) {
    if (!d) return fail(HHR_E_NULL, "dims is NULL");
    if (d->batch < 1) return fail(HHR_E_SHAPE, "batch must be >= 1 (got %d)", d->batch);
    if (d->n_kv_heads < 1) return fail(HHR_E_SHAPE, "n_kv_heads must be >= 1 (got %d)", d->n_kv_heads);
    if (d->n_q_heads < d->n_kv_heads || d->n_q_heads % d->n_kv_heads)
        return fail(HHR_E_SHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", d->n_q_heads,
                    d->n_kv_heads);
    const int G = d->n_q_heads / d->n_kv_heads;
    if (G > 8) return fail(HHR_E_UNSUPPORTED, "query heads per KV head must be <= 8 (got %d)", G);
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(HHR_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
    if (d->hash_bits != 64 && d->hash_bits != 128)
        return fail(HHR_E_UNSUPPORTED, "hash_bits must be 64 or 128 (got %d)", d->hash_bits);
    if (d->page_size < 1 || d->page_size > 64 || (d->page_size & (d->page_size - 1)))
        return fail(HHR_E_UNSUPPORTED, "page_size must be a power of two in 1..64 (got %d)", d->page_size);
    if (d->max_ctx < 1 || d->max_ctx > (1 << 26))
        return fail(HHR_E_SHAPE, "max_ctx must be in 1..2^26 (got %d)", d->max_ctx);
    if (d->kv_dtype != HHR_F32 && d->kv_dtype != HHR_BF16)
        return fail(HHR_E_DTYPE, "kv_dtype must be HHR_F32 or HHR_BF16 (got %d)", d->kv_dtype);
    if (d->meta_dtype != HHR_F32 && d->meta_dtype != HHR_BF16)
        return fail(HHR_E_DTYPE, "meta_dtype must be HHR_F32 or HHR_BF16 (got %d)", d->meta_dtype);
    if (d->meta_layout != HHR_META_INTERLEAVED && d->meta_layout != HHR_META_SIGN_SPLIT)
        return fail(HHR_E_RANGE, "meta_layout must be HHR_META_INTERLEAVED or HHR_META_SIGN_SPLIT (got %d)",
                    d->meta_layout);
    if (d->per_head != 0 && d->per_head != 1)
        return fail(HHR_E_RANGE, "per_head must be 0 or 1 (got %d)", d->per_head);
    if ((d->page_group != 0 && d->page_group != 1) || (d->hamming_group != 0 && d->hamming_group != 1))
        return fail(HHR_E_RANGE, "page_group (%d) and hamming_group (%d) must be 0 or 1", d->page_group,
                    d->hamming_group);
    if (d->sink_tokens < 0 || d->sink_tokens > d->max_ctx || d->local_window < 0 || d->local_window > d->max_ctx)
        return fail(HHR_E_RANGE, "sink_tokens (%d) and local_window (%d) must be in 0..max_ctx", d->sink_tokens,
                    d->local_window);
    s.B = d->batch;
    s.Hq = d->n_q_heads;
    s.Hkv = d->n_kv_heads;
    s.G = G;
    s.D = d->head_dim;
    s.P = d->page_size;
    s.NB = d->hash_bits;
    s.NW = d->hash_bits / 64;
    s.T = d->max_ctx;
    s.NPmax = ((int64_t)s.T + s.P - 1) / s.P;
    s.NPB = (s.NPmax + 63) / 64;
    s.bf16 = d->kv_dtype == HHR_BF16;
    s.meta16 = d->meta_dtype == HHR_BF16;
    s.msplit = d->meta_layout == HHR_META_SIGN_SPLIT;
    s.nsink = d->sink_tokens;
    s.window = d->local_window;
    s.pg_min = d->page_group == 1;
    s.ham_mean = d->hamming_group == 1;
    s.Gh = s.ham_mean ? 1 : s.G;
    s.share = 1;
    s.per_head = d->per_head == 1;
    return HHR_OK;
}

hhr_status check_ptr(const void* p, const char* name, size_t align = 16) {
    if (!p) return fail(HHR_E_NULL, "%s is NULL", name);
    if (!aligned(p, align)) return fail(HHR_E_ALIGN, "%s is not %zu-byte aligned", name, align);
    return HHR_OK;
}

hhr_status check_sel(const Shape& s, int max_keep, int top_k) {
    if (max_keep < 1 || max_keep > s.NPmax)
        return fail(HHR_E_RANGE, "max_keep_pages must be in 1..%lld (got %d)", (long long)s.NPmax, max_keep);
    if ((int64_t)max_keep * s.P > (1 << 26)) return fail(HHR_E_RANGE, "max_keep_pages * page_size too large");
    if (top_k < 1 || top_k > (1 << 24)) return fail(HHR_E_RANGE, "top_k must be in 1..2^24 (got %d)", top_k);
    return HHR_OK;
}

#define HHR_TRY(expr)                       \
    do {                                    \
        const hhr_status st_ = (expr);      \
        if (st_ != HHR_OK) return st_;      \
    } while (0)

hhr_status hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(HHR_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return HHR_OK;
}

// Test and debug switches, read once per process from the environment.
//  HHR_TEST_FAIL=<text>: every launch whose name contains <text> ("*" for
//    all) fails with HHR_E_HIP before anything is enqueued, so callers' error
//    paths can be tested without a GPU.
//  HHR_DEBUG_SYNC=1: after every launch, synchronize the stream and check
//    for errors, so an asynchronous fault is reported by the call that
//    launched it (not allowed under stream capture).
const char* test_fail_target() {
    static const char* v = [] {
        const char* e = std::getenv("HHR_TEST_FAIL");
        return (e && *e) ? e : nullptr;
    }();
    return v;
}
bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("HHR_DEBUG_SYNC");
        return e && *e && std::strcmp(e, "0") != 0;
    }();
    return on;
}
hhr_status before_launch(const char* what) {
    const char* t = test_fail_target();
    if (t && (std::strcmp(t, "*") == 0 || std::strstr(what, t)))
        return fail(HHR_E_HIP, "%s: failed on purpose (HHR_TEST_FAIL=%s)", what, t);
    return HHR_OK;
}
hhr_status after_launch(hipStream_t st, const char* what) {
    if (!debug_sync()) return HHR_OK;
    const hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(HHR_E_HIP, "%s (HHR_DEBUG_SYNC): %s", what, hipGetErrorString(e));
    return hip_check(hipGetLastError(), what);
}

// Every kernel launch of the library: the test switch, the launch, then the debug check.
#define HHR_LAUNCH(expr, what, stream)               \
    do {                                              \
        HHR_TRY(before_launch(what));                 \
        HHR_TRY(hip_check((expr), what));             \
        HHR_TRY(after_launch((stream), what));        \
    } while (0)

// Common front half of the decode step and its stages.
hhr_status prepare(const hhr_dims* dims, int max_keep, int top_k, void* workspace, size_t ws_bytes,
                   DecodeArgs& a) {
    HHR_TRY(make_shape(dims, a.sd));
    a.s = selection_shape(a.sd);
    HHR_TRY(check_sel(a.s, max_keep, top_k));
    HHR_TRY(check_ptr(workspace, "workspace", 256));
    a.max_keep = max_keep;
    a.top_k = top_k;
    a.sel_cap = top_k + a.s.nsink + a.s.window;
    a.lay = ws_layout(a.s, max_keep, top_k);
    if (ws_bytes < a.lay.total)
        return fail(HHR_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, a.lay.total);
    a.ws = static_cast<char*>(workspace);
    a.sel = reinterpret_cast<int32_t*>(a.ws + a.lay.sel);
    a.scale = 0.f;
    a.Q = a.K = a.V = nullptr;
    a.R = a.W = a.meta = nullptr;
    a.codes = nullptr;
    a.seq_len = a.keep_pages = nullptr;
    a.out = nullptr;
    return HHR_OK;
}

float resolve_scale(float scale, int D) { return scale > 0.f ? scale : 1.0f / std::sqrt((float)D); }

// Selections and attention of the decode step, after the page bounds.
hhr_status launch_tail(const DecodeArgs& a, hipStream_t st) {
    HHR_LAUNCH(launch_select(a, st), "select launch", st);
    if (a.lay.sel_splits > 1)
        HHR_LAUNCH(launch_compact_attend(a, st), "compaction and attention launch", st);
    else
        HHR_LAUNCH(launch_attend(a, false, st), "attention launch", st);
    return HHR_OK;
}

}  // namespace

WsLayout ws_layout(const Shape& s, int max_keep, int top_k) {
    WsLayout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t BH = (size_t)s.B * s.Hkv, BQ = (size_t)s.B * s.Hq;
    const size_t forced = (size_t)s.nsink + s.window;  // sink / window keys block 0 of a split also attends
    const int sel_cap = top_k + s.nsink + s.window;
    l.n_splits = (sel_cap + kAttnChunk - 1) / kAttnChunk;
    l.q_rot = take(BQ * s.D * sizeof(float));
    l.code_q = take(BQ * s.NW * sizeof(uint64_t));
    l.code_qm = take(s.ham_mean ? BH * s.NW * sizeof(uint64_t) : 0);
    l.q_split = take(BH * s.D * s.G * 2 * sizeof(double));
    l.score = take(BH * (size_t)s.NPmax * sizeof(double));
    l.pages = take(BH * (size_t)max_keep * sizeof(int32_t));
    l.n_pages = take(BH * sizeof(int32_t));
    l.ham = take(BH * (size_t)max_keep * s.P * sizeof(uint16_t));
    l.sel = take(BH * (size_t)sel_cap * sizeof(int32_t));
    l.k_eff = take(BH * sizeof(int32_t));
    // Split key select.  A split block's latency grows with its share of the
    // candidate slots (the Hamming scan, the compaction and the gathers),
    // the head's merge with the number of splits.  Measured with 8 KV heads,
    // the layer is fastest near S = sqrt(slots / 32): 10 splits at 32K
    // context (3,280 slots) and 20 at 128K (13,120), against the 7 and 26 of
    // 512 slots per block, 2.3 and 0.9 us faster.  Below 2,048 slots the
    // blocks' fixed costs dominate and 512 slots per block stays faster.  No
    // more blocks than the GPU holds at once (each one repeats the page
    // select), unless more are needed for the compaction's kCompactSlots per
    // block; at most 64 blocks per head (then they run in rounds: the merge
    // never waits for a block that has not started).
    const size_t slots = (size_t)max_keep * s.P;
    const size_t BHs = BH > 0 ? BH : 1;
    int S = 1;
    if (max_keep <= kSelListLds && forced < (size_t)kCompactSlots) {
        size_t want = slots >= 2048 ? (size_t)std::lround(std::sqrt((double)slots / 32.0)) : (slots + 511) / 512;
        const size_t cap = 256 / BHs;
        want = want < cap ? want : cap;
        const size_t room = kCompactSlots - forced;  // candidate slots a block can take
        const size_t need = (slots + room - 1) / room;
        want = want < need ? need : want;
        want = want > 64 ? 64 : want;
        if (want >= 2 && (slots + want - 1) / want <= room) S = (int)want;
    }
    l.sel_splits = S;
    // Each of a head's S split blocks repeats the head's page select.  Once
    // the split blocks of all heads need more than about one and a half
    // rounds of the GPU's 256 CUs, the repeats cost more than a launch gap:
    // the page select then runs once per head, and the split blocks only scan.
    l.sel_pages_apart = S > 1 && BH * (size_t)S > 384;
    l.nbins = s.Gh * s.NB + 1;
    l.part_splits = l.n_splits > S ? l.n_splits : S;
    l.partial = take(BQ * (size_t)l.part_splits * (s.D + 2) * sizeof(float));
    l.ghist_off = BH;
    l.n_clear = (int)(BH + (S > 1 ? BH * l.nbins : 0));
    l.counters = take((size_t)l.n_clear * sizeof(uint32_t));
    l.kcum = take(S > 1 ? BH * S * (size_t)l.nbins * sizeof(uint32_t) : 0);
    l.total = off;
    return l;
}

void topk_layout(const Shape& s, int top_k, WsLayout& l, TopkLayout& t) {
    l = WsLayout{};
    t = TopkLayout{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    const size_t BH = (size_t)s.B * s.Hkv, BQ = (size_t)s.B * s.Hq;
    t.nblk = (s.T + kTopkBlk - 1) / kTopkBlk;
    t.score = take(BH * (size_t)s.T * sizeof(double));
    l.sel = take(BH * (size_t)top_k * sizeof(int32_t));
    l.k_eff = take(BH * sizeof(int32_t));
    t.q64 = take(BH * s.D * s.G * sizeof(double));
    t.hist = take(BH * kTopkBins * sizeof(uint32_t));
    t.info = take(BH * 16 * sizeof(uint32_t));
    t.bkey = take(BH * kTopkCap * sizeof(uint64_t));
    t.bidx = take(BH * kTopkCap * sizeof(int32_t));
    t.ocnt = take(BH * (size_t)t.nblk * sizeof(int32_t));
    t.off = take(BH * (size_t)t.nblk * sizeof(int32_t));
    l.n_splits = (top_k + kAttnChunk - 1) / kAttnChunk;
    l.part_splits = l.n_splits;
    l.sel_splits = 1;
    l.partial = take(BQ * (size_t)l.part_splits * (s.D + 2) * sizeof(float));
    l.counters = take(2 * BH * sizeof(uint32_t));
    l.total = off;
}

}  // namespace hhr

// Scratch of hhr_decode_step_append_noalloc: one copy per GPU, alive until the
// process ends.  Host code never passes `scratch` itself to a kernel (in host
// code the name is only a stand-in for the symbol); it passes the device
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[HHR_NOALLOC_SCRATCH_BYTES];

namespace hhr {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
hhr_status noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(HHR_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(HHR_E_UNSUPPORTED, "device index %d is beyond the %d devices the scratch table holds", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail(HHR_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        if (!p) return fail(HHR_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return HHR_OK;
}

}  // namespace
}  // namespace hhr

using namespace hhr;

extern "C" {

size_t hhr_meta_bytes(const hhr_dims* dims) {
    Shape s;
    if (make_shape(dims, s) != HHR_OK) return 0;
    return (size_t)s.B * s.Hkv * (size_t)s.NPB * 64 * s.D * 2 * (s.meta16 ? sizeof(uint16_t) : sizeof(float));
}

size_t hhr_codes_bytes(const hhr_dims* dims) {
    Shape s;
    if (make_shape(dims, s) != HHR_OK) return 0;
    return (size_t)s.B * s.Hkv * (size_t)s.T * s.NW * sizeof(uint64_t);
}

hhr_status hhr_encode_cache(const hhr_dims* dims, const void* K, const float* R, const float* W,
                            const int32_t* start, const int32_t* count, int32_t max_count, float* meta,
                            uint64_t* codes, void* stream) {
    Shape s;
    HHR_TRY(make_shape(dims, s));
    HHR_TRY(check_ptr(K, "K"));
    HHR_TRY(check_ptr(R, "R"));
    HHR_TRY(check_ptr(W, "W"));
    HHR_TRY(check_ptr(start, "start", 4));
    HHR_TRY(check_ptr(count, "count", 4));
    HHR_TRY(check_ptr(meta, "meta"));
    HHR_TRY(check_ptr(codes, "codes"));
    if (max_count < 0 || max_count > s.T)
        return fail(HHR_E_RANGE, "max_count must be in 0..max_ctx (got %d)", max_count);
    if (max_count == 0) return ok();
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (max_count <= kAppendMax) {
        ProjectArgs p{};
        p.keys = true;
        p.K = K;
        p.R = R;
        p.W = W;
        p.start = start;
        p.count = count;
        p.max_count = max_count;
        p.meta = meta;
        p.codes = codes;
        HHR_LAUNCH(launch_project(s, p, st), "append launch", st);
    } else {
        HHR_LAUNCH(launch_encode(s, K, R, W, start, count, max_count, meta, codes, st), "encode launch", st);
    }
    return ok();
}

size_t hhr_decode_workspace_bytes(const hhr_dims* dims, int32_t max_keep_pages, int32_t top_k) {
    Shape d;
    if (make_shape(dims, d) != HHR_OK) return 0;
    const Shape s = selection_shape(d);
    if (check_sel(s, max_keep_pages, top_k) != HHR_OK) return 0;
    return ws_layout(s, max_keep_pages, top_k).total;
}

hhr_status hhr_decode_workspace_layout(const hhr_dims* dims, int32_t max_keep_pages, int32_t top_k,
                                       hhr_workspace_layout* layout) {
    Shape d;
    HHR_TRY(make_shape(dims, d));
    const Shape s = selection_shape(d);
    HHR_TRY(check_sel(s, max_keep_pages, top_k));
    if (!layout) return fail(HHR_E_NULL, "layout is NULL");
    const WsLayout l = ws_layout(s, max_keep_pages, top_k);
    layout->q_rot = l.q_rot;
    layout->code_q = l.code_q;
    layout->q_split = l.q_split;
    layout->score = l.score;
    layout->pages = l.pages;
    layout->n_pages = l.n_pages;
    layout->ham = l.ham;
    layout->sel = l.sel;
    layout->k_eff = l.k_eff;
    layout->partial = l.partial;
    layout->counters = l.counters;
    layout->total = l.total;
    layout->n_splits = l.n_splits;
    return ok();
}

hhr_status hhr_decode_step(const hhr_dims* dims, const void* Q, const void* K, const void* V, const float* R,
                           const float* W, const float* meta, const uint64_t* codes, const int32_t* seq_len,
                           const int32_t* keep_pages, int32_t max_keep_pages, int32_t top_k, float softmax_scale,
                           float* out, int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(Q, "Q"));
    HHR_TRY(check_ptr(K, "K"));
    HHR_TRY(check_ptr(V, "V"));
    HHR_TRY(check_ptr(R, "R"));
    HHR_TRY(check_ptr(W, "W"));
    HHR_TRY(check_ptr(meta, "meta"));
    HHR_TRY(check_ptr(codes, "codes"));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    HHR_TRY(check_ptr(keep_pages, "keep_pages", 4));
    HHR_TRY(check_ptr(out, "out"));
    if (sel_idx) HHR_TRY(check_ptr(sel_idx, "sel_idx", 4));
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.R = R;
    a.W = W;
    a.meta = meta;
    a.codes = codes;
    a.seq_len = seq_len;
    a.keep_pages = keep_pages;
    a.out = out;
    a.scale = resolve_scale(softmax_scale, a.s.D);
    if (sel_idx) a.sel = sel_idx;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_qprep(a, st), "qprep launch", st);
    HHR_LAUNCH(launch_page_bounds(a, st), "page-bound launch", st);
    HHR_TRY(launch_tail(a, st));
    return ok();
}

hhr_status hhr_decode_step_append(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                                  const float* R, const float* W, float* meta, uint64_t* codes,
                                  const int32_t* append_start, const int32_t* append_count, int32_t max_append,
                                  const int32_t* seq_len, const int32_t* keep_pages, int32_t max_keep_pages,
                                  int32_t top_k, float softmax_scale, float* out, int32_t* sel_idx, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(Q, "Q"));
    HHR_TRY(check_ptr(K, "K"));
    HHR_TRY(check_ptr(V, "V"));
    HHR_TRY(check_ptr(R, "R"));
    HHR_TRY(check_ptr(W, "W"));
    HHR_TRY(check_ptr(meta, "meta"));
    HHR_TRY(check_ptr(codes, "codes"));
    HHR_TRY(check_ptr(append_start, "append_start", 4));
    HHR_TRY(check_ptr(append_count, "append_count", 4));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    HHR_TRY(check_ptr(keep_pages, "keep_pages", 4));
    HHR_TRY(check_ptr(out, "out"));
    if (sel_idx) HHR_TRY(check_ptr(sel_idx, "sel_idx", 4));
    if (max_append < 0 || max_append > a.s.T)
        return fail(HHR_E_RANGE, "max_append must be in 0..max_ctx (got %d)", max_append);
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.R = R;
    a.W = W;
    a.meta = meta;
    a.codes = codes;
    a.seq_len = seq_len;
    a.keep_pages = keep_pages;
    a.out = out;
    a.scale = resolve_scale(softmax_scale, a.s.D);
    if (sel_idx) a.sel = sel_idx;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (max_append > 0 && max_append <= kAppendMax) {
        // One launch projects the appended keys and the queries.
        ProjectArgs p{};
        p.keys = true;
        p.queries = true;
        p.Q = Q;
        p.K = K;
        p.R = R;
        p.W = W;
        p.start = append_start;
        p.count = append_count;
        p.max_count = max_append;
        p.meta = meta;
        p.codes = codes;
        p.q_rot = reinterpret_cast<float*>(a.ws + a.lay.q_rot);
        p.code_q = reinterpret_cast<uint64_t*>(a.ws + a.lay.code_q);
        p.code_qm = reinterpret_cast<uint64_t*>(a.ws + a.lay.code_qm);
        p.q_split = reinterpret_cast<double*>(a.ws + a.lay.q_split);
        p.counters = reinterpret_cast<uint32_t*>(a.ws + a.lay.counters);
        p.n_counters = a.lay.n_clear;
        p.qmean = a.s.ham_mean;
        HHR_LAUNCH(launch_project(a.sd, p, st), "append + qprep launch", st);
    } else {
        if (max_append > 0)
            HHR_LAUNCH(launch_encode(a.sd, K, R, W, append_start, append_count, max_append, meta, codes, st),
                       "encode launch", st);
        HHR_LAUNCH(launch_qprep(a, st), "qprep launch", st);
    }
    HHR_LAUNCH(launch_page_bounds(a, st), "page-bound launch", st);
    HHR_TRY(launch_tail(a, st));
    return ok();
}

size_t hhr_noalloc_scratch_bytes(void) { return HHR_NOALLOC_SCRATCH_BYTES; }

hhr_status hhr_decode_step_append_noalloc(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                                          const float* R, const float* W, float* meta, uint64_t* codes,
                                          const int32_t* append_start, const int32_t* append_count,
                                          int32_t max_append, const int32_t* seq_len, const int32_t* keep_pages,
                                          int32_t max_keep_pages, int32_t top_k, float softmax_scale, float* out,
                                          int32_t* sel_idx, void* stream) {
    Shape d;
    HHR_TRY(make_shape(dims, d));
    const Shape s = selection_shape(d);
    HHR_TRY(check_sel(s, max_keep_pages, top_k));
    const size_t need = ws_layout(s, max_keep_pages, top_k).total;
    if (need > (size_t)HHR_NOALLOC_SCRATCH_BYTES)
        return fail(HHR_E_WORKSPACE, "these arguments need %zu bytes of scratch; the static scratch holds %zu",
                    need, (size_t)HHR_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    HHR_TRY(noalloc_scratch(&ws));
    return hhr_decode_step_append(dims, Q, K, V, R, W, meta, codes, append_start, append_count, max_append, seq_len,
                                  keep_pages, max_keep_pages, top_k, softmax_scale, out, sel_idx, ws,
                                  (size_t)HHR_NOALLOC_SCRATCH_BYTES, stream);
}

hhr_status hhr_stage_qprep(const hhr_dims* dims, const void* Q, const float* R, const float* W,
                           int32_t max_keep_pages, int32_t top_k, void* workspace, size_t workspace_bytes,
                           void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(Q, "Q"));
    HHR_TRY(check_ptr(R, "R"));
    HHR_TRY(check_ptr(W, "W"));
    a.Q = Q;
    a.R = R;
    a.W = W;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_qprep(a, st), "qprep launch", st);
    return ok();
}

hhr_status hhr_stage_page_bounds(const hhr_dims* dims, const float* meta, const int32_t* seq_len,
                                 int32_t max_keep_pages, int32_t top_k, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(meta, "meta"));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    a.meta = meta;
    a.seq_len = seq_len;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_page_bounds(a, st), "page-bound launch", st);
    return ok();
}

hhr_status hhr_stage_select_pages(const hhr_dims* dims, const int32_t* seq_len, const int32_t* keep_pages,
                                  int32_t max_keep_pages, int32_t top_k, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    HHR_TRY(check_ptr(keep_pages, "keep_pages", 4));
    a.seq_len = seq_len;
    a.keep_pages = keep_pages;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_select_pages(a, st), "page-select launch", st);
    return ok();
}

hhr_status hhr_stage_hamming(const hhr_dims* dims, const uint64_t* codes, const int32_t* seq_len,
                             int32_t max_keep_pages, int32_t top_k, void* workspace, size_t workspace_bytes,
                             void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(codes, "codes"));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    a.codes = codes;
    a.seq_len = seq_len;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_hamming(a, st), "Hamming launch", st);
    return ok();
}

hhr_status hhr_stage_select_keys(const hhr_dims* dims, const uint64_t* codes, const int32_t* seq_len,
                                 int32_t max_keep_pages, int32_t top_k, int32_t* sel_idx, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(codes, "codes"));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    if (sel_idx) HHR_TRY(check_ptr(sel_idx, "sel_idx", 4));
    a.codes = codes;
    a.seq_len = seq_len;
    if (sel_idx) a.sel = sel_idx;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_select_keys(a, st), "key-select launch", st);
    return ok();
}

hhr_status hhr_stage_attend(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                            const int32_t* seq_len, int32_t max_keep_pages, int32_t top_k, float softmax_scale,
                            const int32_t* sel_idx, float* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
    DecodeArgs a;
    HHR_TRY(prepare(dims, max_keep_pages, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(Q, "Q"));
    HHR_TRY(check_ptr(K, "K"));
    HHR_TRY(check_ptr(V, "V"));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    HHR_TRY(check_ptr(out, "out"));
    if (sel_idx) HHR_TRY(check_ptr(sel_idx, "sel_idx", 4));
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.seq_len = seq_len;
    a.out = out;
    a.scale = resolve_scale(softmax_scale, a.s.D);
    if (sel_idx) a.sel = const_cast<int32_t*>(sel_idx);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_attend(a, true, st), "attention launch", st);
    return ok();
}

hhr_status hhr_topk_workspace_layout(const hhr_dims* dims, int32_t top_k, hhr_topk_layout* layout) {
    Shape s;
    HHR_TRY(make_shape(dims, s));
    if (top_k < 1 || top_k > (1 << 24)) return fail(HHR_E_RANGE, "top_k must be in 1..2^24 (got %d)", top_k);
    if (!layout) return fail(HHR_E_NULL, "layout is NULL");
    WsLayout l;
    TopkLayout t;
    topk_layout(s, top_k, l, t);
    layout->score = t.score;
    layout->sel = l.sel;
    layout->k_eff = l.k_eff;
    layout->total = l.total;
    return ok();
}

size_t hhr_topk_workspace_bytes(const hhr_dims* dims, int32_t top_k) {
    hhr_topk_layout l;
    if (hhr_topk_workspace_layout(dims, top_k, &l) != HHR_OK) return 0;
    return l.total;
}

namespace {
// Common front of the TopK (Oracle) entry points.
hhr_status topk_prepare(const hhr_dims* dims, int top_k, void* workspace, size_t workspace_bytes, TopkArgs& a) {
    HHR_TRY(make_shape(dims, a.d.s));
    a.d.s.per_head = false;  // the TopK step always shares one selection per KV head
    a.d.sd = a.d.s;
    if (top_k < 1 || top_k > (1 << 24)) return fail(HHR_E_RANGE, "top_k must be in 1..2^24 (got %d)", top_k);
    HHR_TRY(check_ptr(workspace, "workspace", 256));
    topk_layout(a.d.s, top_k, a.d.lay, a.tl);
    if (workspace_bytes < a.d.lay.total)
        return fail(HHR_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, a.d.lay.total);
    a.d.ws = static_cast<char*>(workspace);
    a.d.top_k = top_k;
    a.d.sel_cap = top_k;  // no forced keys on this path
    a.d.max_keep = 1;
    a.d.sel = reinterpret_cast<int32_t*>(a.d.ws + a.d.lay.sel);
    return HHR_OK;
}
}  // namespace

hhr_status hhr_stage_topk_logits(const hhr_dims* dims, const void* K, const int32_t* seq_len, int32_t top_k,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    TopkArgs a{};
    HHR_TRY(topk_prepare(dims, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(K, "K"));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    a.d.K = K;
    a.d.seq_len = seq_len;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_topk_logits(a, st), "logit launch", st);
    return ok();
}

hhr_status hhr_topk_decode_step(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                                const int32_t* seq_len, int32_t top_k, float softmax_scale, float* out,
                                int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream) {
    TopkArgs a{};
    HHR_TRY(topk_prepare(dims, top_k, workspace, workspace_bytes, a));
    HHR_TRY(check_ptr(Q, "Q"));
    HHR_TRY(check_ptr(K, "K"));
    HHR_TRY(check_ptr(V, "V"));
    HHR_TRY(check_ptr(seq_len, "seq_len", 4));
    HHR_TRY(check_ptr(out, "out"));
    if (sel_idx) HHR_TRY(check_ptr(sel_idx, "sel_idx", 4));
    a.d.Q = Q;
    a.d.K = K;
    a.d.V = V;
    a.d.seq_len = seq_len;
    a.d.out = out;
    a.d.scale = resolve_scale(softmax_scale, a.d.s.D);
    if (sel_idx) a.d.sel = sel_idx;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    HHR_LAUNCH(launch_topk_prep(a, st), "top-k prep launch", st);
    HHR_LAUNCH(launch_topk_logits(a, st), "logit launch", st);
    HHR_LAUNCH(launch_topk_select(a, st), "top-k select launch", st);
    HHR_LAUNCH(launch_attend(a.d, false, st), "attention launch", st);
    return ok();
}

const char* hhr_status_str(hhr_status st) {
    switch (st) {
        case HHR_OK: return "HHR_OK";
        case HHR_E_NULL: return "HHR_E_NULL";
        case HHR_E_SHAPE: return "HHR_E_SHAPE";
        case HHR_E_DTYPE: return "HHR_E_DTYPE";
        case HHR_E_ALIGN: return "HHR_E_ALIGN";
        case HHR_E_WORKSPACE: return "HHR_E_WORKSPACE";
        case HHR_E_RANGE: return "HHR_E_RANGE";
        case HHR_E_UNSUPPORTED: return "HHR_E_UNSUPPORTED";
        case HHR_E_HIP: return "HHR_E_HIP";
    }
    return "HHR_E_UNKNOWN";
}

const char* hhr_last_error(void) { return g_last_error.c_str(); }

int32_t hhr_abi_version(void) { return HHR_ABI_VERSION; }

}  // extern "C"
