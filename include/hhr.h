/*
 * hhr.h -- C ABI of the MI355X (gfx950) HHR decode-path library, libhhr.so.
 *
 * HHR (Hierarchical Hash Retrieval) selects, for each decode step, the keys a
 * query attends to in two stages and then runs exact attention on them
 * ("HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", Abstract;
 * rit.work HHR blog post, section "Два уровня маршрутизации решают разные
 * ошибки"):
 *   coarse  -- Geometry-Aware Key Routing (GKR): keys are rotated by a
 *              per-KV-head orthogonal R_h, adjacent keys are grouped into
 *              pages, each page stores per-dimension max/min of its rotated
 *              keys, and a page whose logit upper bound is low is dropped;
 *   fine    -- Learned Hash Projection (LHP): keys of the surviving pages are
 *              ranked by the Hamming distance between sign(W_h q) and
 *              sign(W_h k) bit codes and the top-k are kept;
 *   attend  -- softmax attention of the query over the kept keys.
 * R_h and W_h are inputs (learning them is outside this library).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array argument is a DEVICE pointer except `const hhr_dims*` and
 *    the layout struct, which are host pointers.  The caller owns every
 *    buffer; the library never allocates, frees or synchronizes, and it keeps
 *    no state between calls except a thread-local error message.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting.  Device faults surface at the
 *    caller's next synchronization.
 *  - All arguments are validated on the host before anything is enqueued.  On
 *    failure nothing is enqueued, nothing is written, a nonzero hhr_status is
 *    returned and hhr_last_error() describes it.  A failed launch returns
 *    HHR_E_HIP with the HIP error text.
 *  - Two environment switches, read once per process: HHR_TEST_FAIL=<text>
 *    makes every launch whose name contains <text> ("*": every launch) fail
 *    with HHR_E_HIP before anything is enqueued, for testing callers' error
 *    paths without a GPU; HHR_DEBUG_SYNC=1 synchronizes the stream and checks
 *    for errors after every launch, so an asynchronous fault is reported by
 *    the call that launched it (the one case where the library synchronizes;
 *    not for use under stream capture).
 *  - Per-sequence values held in device arrays (start, count, seq_len,
 *    keep_pages) are clamped inside the kernels so that no access leaves its
 *    buffer: seq_len to [0, max_ctx]; start to [0, max_ctx]; count to
 *    [0, min(max_count, max_ctx - start)].
 *  - Inputs must not alias outputs.  Every array must be 16-byte aligned and
 *    the workspace 256-byte aligned.  Non-finite inputs give undefined
 *    (memory-safe) results.
 *
 * Dimensions (v1 limits)
 * ----------------------
 *   B  = batch >= 1                 Hkv = n_kv_heads >= 1
 *   Hq = n_q_heads, G = Hq/Hkv in 1..8 (query head i uses KV head i/G)
 *   D  = head_dim in {64, 128}      b   = hash_bits in {64, 128}, NW = b/64
 *   P  = page_size, a power of two in 1..64;   T = max_ctx in 1..2^26 (row capacity)
 *   NP(L) = ceil(L/P) pages of a sequence of length L; NPmax = NP(T);
 *   NPB = ceil(NPmax/64) page blocks.
 *
 * Layouts (row-major, contiguous)
 * -------------------------------
 *   Q     [B][Hq][D]          kv_dtype (fp32, or bf16 bit patterns)
 *   K, V  [B][Hkv][T][D]      kv_dtype
 *   R     [Hkv][D][D]  fp32   rotated_r = sum_c R[h][r][c] * x_c
 *   W     [Hkv][b][D]  fp32   bit j of a code = [ sum_c W[h][j][c] * x_c > 0 ]
 *   codes [B][Hkv][T][NW] uint64; bit j of a code is bit j%64 of word j/64
 *   meta  meta_dtype HHR_F32: [B][Hkv][NPB][D/2][64][4] fp32, page-block
 *         interleaved: for page p = 64*blk + lane and dimension pair
 *         (2e, 2e+1) the four floats are (max_2e, min_2e, max_2e+1, min_2e+1)
 *         of the rotated keys of page p.  A wave of 64 lanes, one page each,
 *         reads one dimension pair of 64 pages as one contiguous 1 KiB span.
 *         meta_dtype HHR_BF16: [B][Hkv][NPB][D/4][64][8] bf16 bit patterns,
 *         the same interleave over dimension quads (max_4e, min_4e, ...,
 *         max_4e+3, min_4e+3); each max is rounded up and each min down to
 *         bf16 (outward), so the page bound below, computed from them, still
 *         bounds every key of the page.  The pointer type stays float* in
 *         the calls; the buffer holds hhr_meta_bytes(dims) bytes either way.
 *         meta_layout HHR_META_SIGN_SPLIT (either dtype): [B][Hkv][NPB][D][2][64],
 *         dimension-major: for page block blk, dimension d and side s (0 =
 *         max, 1 = min) the 64 pages' values are one contiguous run (256 B
 *         fp32, 128 B bf16).  With one query head per KV head (G = 1)
 *         the bound pass then reads, per dimension, only the side the sign
 *         of the rotated query coordinate picks -- half the metadata bytes
 *         -- with the same bound bit for bit (the side not read contributes
 *         an exact zero).  Grouped heads, per_head = 1 included (one pass
 *         per KV head serves its G query heads), read both sides.  Same
 *         byte count as the interleaved layout.
 *   out   [B][Hq][D] fp32
 *   sel_idx [B][U][top_k + sink_tokens + local_window] int32, U = Hkv (or Hq
 *         with per_head = 1): the selected key positions, ascending, padded
 *         with -1.  A row holds top_k entries when both forced-key variants
 *         are off.
 *
 * Arithmetic (what makes codes and selections reproducible bit for bit)
 * ---------------------------------------------------------------------
 *   - A projection (rotation row or hash row) is the canonical chain
 *     acc = +0.0f; for c = 0..D-1: acc = fmaf(M[r][c], x_c, acc)  (fp32, IEEE
 *     round-to-nearest-even, denormals kept).  bf16 inputs widen exactly.
 *   - A rotated key coordinate equal to -0 is stored as +0 before max/min.
 *   - The page bound of query head i is (kmax, kmin as stored in meta)
 *       U_i(p) = sum over r ascending of max(qrot_i,r * kmax_r, qrot_i,r * kmin_r)
 *     evaluated in fp64 (each product of two fp32 values is exact in fp64);
 *     the score of the KV head's group is S(p) = max_i U_i(p), with -0 read
 *     as +0.  The functional form is this library's reading of GKR's
 *     page-level logit upper bound (the pages state none): it bounds
 *     qrot_i . krot_t from above for every key t of the page, and an
 *     orthogonal R_h keeps that equal to q_i . k_t up to rounding.
 *   - The Hamming distance of key t is the sum over the group's query heads
 *     and the code words of popcount(code_q XOR code_t).
 *   - Attention accumulates in fp32 (online softmax over split chunks).
 */
#ifndef HHR_H
#define HHR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HHR_ABI_VERSION 8

typedef enum {
    HHR_OK = 0,
    HHR_E_NULL = 1,        /* a required pointer is NULL                    */
    HHR_E_SHAPE = 2,       /* a dimension is out of range or inconsistent   */
    HHR_E_DTYPE = 3,       /* unknown kv_dtype                              */
    HHR_E_ALIGN = 4,       /* a pointer is not aligned as required          */
    HHR_E_WORKSPACE = 5,   /* workspace smaller than required               */
    HHR_E_RANGE = 6,       /* a scalar argument is out of range             */
    HHR_E_UNSUPPORTED = 7, /* valid but not supported by this library      */
    HHR_E_HIP = 8          /* a HIP launch failed                           */
} hhr_status;

typedef enum { HHR_F32 = 0, HHR_BF16 = 1 } hhr_dtype;

/* Storage order of the page metadata (see "meta" under Layouts). */
typedef enum { HHR_META_INTERLEAVED = 0, HHR_META_SIGN_SPLIT = 1 } hhr_meta_layout;

typedef struct {
    int32_t batch;      /* B                                              */
    int32_t n_q_heads;  /* Hq                                             */
    int32_t n_kv_heads; /* Hkv                                            */
    int32_t head_dim;   /* D                                              */
    int32_t page_size;  /* P                                              */
    int32_t hash_bits;  /* b                                              */
    int32_t max_ctx;    /* T: row capacity of K, V and codes              */
    int32_t kv_dtype;   /* hhr_dtype of Q, K and V                        */
    int32_t meta_dtype; /* hhr_dtype of the page metadata: HHR_F32 (0, the
                           default) or HHR_BF16 (outward-rounded, half the
                           bytes; see "meta" under Layouts)               */
    int32_t sink_tokens;  /* decode variant, 0..max_ctx (0 = off): the first
                             sink_tokens keys are always attended          */
    int32_t local_window; /* decode variant, 0..max_ctx (0 = off): the last
                             local_window keys are always attended         */
    int32_t page_group;    /* decode variant: page score over the GQA group,
                              0 = max of the heads' bounds (default), 1 = min */
    int32_t hamming_group; /* decode variant: 0 = distance summed over the
                              group's query codes (default), 1 = distance to
                              the code of the group's mean query           */
    int32_t per_head;      /* decode variant: 0 = one selection per KV head,
                              shared by its G query heads (default); 1 = one
                              selection per query head: every per-(b, h)
                              workspace row and sel_idx row is then per
                              query head ([B][Hq]...), as if each KV head
                              were repeated for its G query heads (q_split
                              aside: see the workspace layout)             */
    int32_t meta_layout;   /* hhr_meta_layout of the page metadata: HHR_META_INTERLEAVED
                              (0, the default) or HHR_META_SIGN_SPLIT (1):
                              with G = 1 the bound pass reads half the
                              metadata bytes; encode and decode must agree */
} hhr_dims;

/* Bytes of the meta and codes buffers for these dims (0 if the dims are invalid). */
size_t hhr_meta_bytes(const hhr_dims* dims);
size_t hhr_codes_bytes(const hhr_dims* dims);

/*
 * hhr_encode_cache -- GKR page metadata and LHP key codes
 * ("HHR: Hierarchical Hash Retrieval for Efficient LLM Generation",
 * Abstract; rit.work HHR blog post, sections "Два уровня маршрутизации
 * решают разные ошибки" and "Когда HHR меняет планы запуска модели": the
 * deployment stores page bounds).
 *
 * For every sequence b it encodes keys [s, e) with s = start[b] and
 * e = s + count[b] (clamped as above; count[b] must not exceed max_count):
 *   codes[b][h][t]  for t in [s, e): the LHP code of K[b][h][t];
 *   meta of every page p with pP < e and (p+1)P > s: max/min over the keys
 *   [pP, min((p+1)P, e)) of R_h K[b][h][t], recomputed from K, so a page
 *   that straddles s includes the keys before s that K already holds.
 * Encoding [0,m) and then [m,n) gives the same bits as encoding [0,n).
 * Other parts of meta and codes are not touched.
 *   K     device, read   R, W   device, read   start, count  device int32 [B]
 *   max_count            host, >= 0 (0 enqueues nothing)
 *   meta, codes          device, written (layouts above)
 */
hhr_status hhr_encode_cache(const hhr_dims* dims, const void* K, const float* R, const float* W,
                            const int32_t* start, const int32_t* count, int32_t max_count,
                            float* meta, uint64_t* codes, void* stream);

/* Scratch the decode step needs for these arguments (0 if they are invalid). */
size_t hhr_decode_workspace_bytes(const hhr_dims* dims, int32_t max_keep_pages, int32_t top_k);

/*
 * Byte offsets, inside the decode workspace, of the intermediate results the
 * decode step leaves there (each region 256-byte aligned).  They stay valid
 * until the next call that uses the same workspace, so a caller can inspect
 * every stage of the last step:
 *   q_rot   fp32   [B][Hq][D]      R_h q_i (canonical chain)
 *   code_q  uint64 [B][Hq][NW]     LHP code of q_i
 *   q_split fp64   [B][Hkv][D][G][2]  (max(q,0), min(q,0)) of q_rot, per dim and head;
 *                  with per_head = 1 this region keeps the KV-head layout
 *                  (one pass over a KV head's metadata serves its G selections)
 *   score   fp64   [B][Hkv][NPmax] page score S(p); entries p >= NP(L) unspecified
 *   pages   int32  [B][Hkv][max_keep]  kept pages ascending, -1 padded
 *   n_pages int32  [B][Hkv]
 *   ham     uint16 [B][Hkv][max_keep*P] Hamming distance of candidate slot
 *                  j*P + r, i.e. key pages[j]*P + r; 0xFFFF if that key is
 *                  past the sequence or the slot is unused
 *   sel     int32  [B][Hkv][top_k + sink_tokens + local_window] selected
 *                  keys (when sel_idx is NULL)
 *   k_eff   int32  [B][Hkv] number of selected keys
 *   partial, counters: internal (private scratch may follow; total covers it)
 */
typedef struct {
    size_t q_rot, code_q, q_split, score, pages, n_pages, ham, sel, k_eff, partial, counters;
    size_t total;
    int32_t n_splits; /* attention splits per KV head */
} hhr_workspace_layout;

hhr_status hhr_decode_workspace_layout(const hhr_dims* dims, int32_t max_keep_pages, int32_t top_k,
                                       hhr_workspace_layout* layout);

/*
 * hhr_decode_step -- one HHR decode step of one layer
 * ("HHR: Hierarchical Hash Retrieval for Efficient LLM Generation",
 * Abstract; rit.work HHR blog post, section "Два уровня маршрутизации решают
 * разные ошибки"; top-k selection as in Appendix Table 4 of the
 * thelatestinai.com page on arXiv 2610.01230).
 *
 * For every sequence b (length L = seq_len[b]) and KV head h, with the G
 * query heads of h sharing one selection:
 *   1. qrot_i = R_h q_i and code_q,i (canonical chains);
 *   2. S(p) for p < NP(L) (fp64, see above); with page_group = 1 the min
 *      over the group's heads instead of the max;
 *   3. keep = clamp(keep_pages[b], 1, min(NP(L), max_keep_pages)) pages with
 *      the largest S, equal S going to the lower page index;
 *   4. candidates: keys t < L of the kept pages;
 *   5. H(t) = group Hamming distance; with hamming_group = 1, H(t) =
 *      popcount(code(qm) XOR code_t) for the group's mean query qm, qm_d =
 *      (sum_i q_i,d) / G in fp32 (heads ascending, one division), coded by
 *      the same canonical chain;
 *   6. the min(top_k, #candidates) candidates with the smallest (H(t), t),
 *      written ascending to sel_idx (or the workspace), -1 padded;
 *      with sink_tokens s or local_window w nonzero (the baselines' sink
 *      tokens and local window, Appendix Table 4 of the thelatestinai.com
 *      page), the keys t < min(s, L) and t >= max(min(s, L), L - w) are
 *      always selected and take no part in steps 4-6, and the list is the
 *      sink keys, then the step-6 keys, then the window keys (ascending);
 *      k_eff = the number listed, sel_idx rows hold top_k + s + w entries;
 *   7. out_i = sum_t softmax_t(scale * q_i . k_t) v_t over the selected t,
 *      scale = softmax_scale if > 0, else 1/sqrt(D).
 * L = 0 gives out = 0, no pages and no keys.
 *   Q, K, V, R, W, meta, codes      device, read (meta/codes from hhr_encode_cache)
 *   seq_len, keep_pages             device int32 [B], read
 *   max_keep_pages >= 1, top_k >= 1 host; they size the workspace
 *   out                             device fp32 [B][Hq][D], written
 *   sel_idx                         device int32 [B][Hkv][top_k + s + w], written, or NULL
 *   workspace, workspace_bytes      device scratch >= hhr_decode_workspace_bytes
 */
hhr_status hhr_decode_step(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                           const float* R, const float* W, const float* meta, const uint64_t* codes,
                           const int32_t* seq_len, const int32_t* keep_pages, int32_t max_keep_pages,
                           int32_t top_k, float softmax_scale, float* out, int32_t* sel_idx,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * hhr_decode_step_append -- append the token(s) just generated, then decode.
 * Same result as hhr_encode_cache(dims, K, R, W, append_start, append_count,
 * max_append, meta, codes, stream) followed by hhr_decode_step(...) with the
 * same arguments, but with max_append <= 64 the key append and the query
 * projection share one launch (the per-token path of a decode loop).  meta
 * and codes are read and written; every other argument means what it means
 * for those two calls.
 */
hhr_status hhr_decode_step_append(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                                  const float* R, const float* W, float* meta, uint64_t* codes,
                                  const int32_t* append_start, const int32_t* append_count, int32_t max_append,
                                  const int32_t* seq_len, const int32_t* keep_pages, int32_t max_keep_pages,
                                  int32_t top_k, float softmax_scale, float* out, int32_t* sel_idx, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * hhr_decode_step_append_noalloc -- hhr_decode_step_append without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It calls no hipMalloc, hipFree or other allocating routine:
 * its scratch is a static device array of HHR_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The call
 * runs on the current device (the one `stream` belongs to); the first call
 * on a device looks up that device's array once.
 *   - Arguments, results and errors are those of hhr_decode_step_append;
 *     out and sel_idx (or NULL) are the caller's.
 *   - Arguments whose hhr_decode_workspace_bytes exceeds the scratch size
 *     return HHR_E_WORKSPACE before anything is enqueued.
 *   - Every call on a GPU shares that GPU's array and leaves its intermediate
 *     results there (in the hhr_decode_workspace_layout of its arguments)
 *     until the next call.  Calls that overlap on one GPU (other streams,
 *     other threads) race on it: serialise them.  Everything a step needs
 *     cleared is cleared by the step's own kernels.
 */
#define HHR_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t hhr_noalloc_scratch_bytes(void);
hhr_status hhr_decode_step_append_noalloc(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                                          const float* R, const float* W, float* meta, uint64_t* codes,
                                          const int32_t* append_start, const int32_t* append_count,
                                          int32_t max_append, const int32_t* seq_len, const int32_t* keep_pages,
                                          int32_t max_keep_pages, int32_t top_k, float softmax_scale, float* out,
                                          int32_t* sel_idx, void* stream);

/*
 * hhr_topk_decode_step -- the TopK (Oracle) comparison step: keys chosen by
 * their exact attention logit, with no page bounds and no codes (the
 * "TopK (Oracle)" rows of Table 1 and Table 2 and "TopK-1.5%" in Appendix
 * Table 4 on the thelatestinai.com page for arXiv 2610.01230; rit.work HHR
 * blog post, section "Когда HHR меняет планы запуска модели").
 *
 * For every sequence b (length L = seq_len[b]) and KV head h, with the G
 * query heads of h sharing one selection as in hhr_decode_step:
 *   1. z(t) = max over the G heads of sum_d q_i,d * k_t,d for t < L, in fp64
 *      with d ascending from +0 (each product of two fp32 values is exact in
 *      fp64, so z is reproducible bit for bit); -0 is read as +0;
 *   2. the k_eff = min(top_k, L) keys with the largest z, equal z going to
 *      the lower t, written ascending to sel_idx (or the workspace), -1
 *      padded;
 *   3. out_i = sum_t softmax_t(scale * q_i . k_t) v_t over them, as step 7
 *      of hhr_decode_step.
 * Only batch, n_q_heads, n_kv_heads, head_dim, max_ctx and kv_dtype matter;
 * the other dims fields must still hold valid values.  The step reads all of
 * K (it is the exact reference, not a fast path).  A boundary bin of more
 * than 16384 keys tied within fp32 rounding (e.g. a constant query) takes a
 * slower single-block select; the result is the same.
 *   Q, K, V         device, read (layouts as for hhr_decode_step)
 *   seq_len         device int32 [B], read
 *   top_k >= 1      host
 *   out             device fp32 [B][Hq][D], written
 *   sel_idx         device int32 [B][Hkv][top_k], written, or NULL
 *   workspace       device scratch >= hhr_topk_workspace_bytes; afterwards
 *                   it holds z (fp64 [B][Hkv][max_ctx] at `score`; entries
 *                   t >= L unspecified), the selection (at `sel` when sel_idx
 *                   is NULL) and k_eff (int32 [B][Hkv] at `k_eff`)
 * Errors as for hhr_decode_step; nothing is enqueued on failure.
 */
typedef struct {
    size_t score, sel, k_eff, total;
} hhr_topk_layout;

hhr_status hhr_topk_workspace_layout(const hhr_dims* dims, int32_t top_k, hhr_topk_layout* layout);
size_t hhr_topk_workspace_bytes(const hhr_dims* dims, int32_t top_k);  /* 0 on invalid arguments */
hhr_status hhr_topk_decode_step(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                                const int32_t* seq_len, int32_t top_k, float softmax_scale, float* out,
                                int32_t* sel_idx, void* workspace, size_t workspace_bytes, void* stream);
/* Stage entry point for timing and tests: step 1's logit kernel alone, on a
 * workspace a full hhr_topk_decode_step with the same dims, Q and top_k has
 * used (it reads the widened queries that step left).  Rewrites z at `score`
 * and adds to a histogram that only the full step uses and clears. */
hhr_status hhr_stage_topk_logits(const hhr_dims* dims, const void* K, const int32_t* seq_len, int32_t top_k,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage entry points: each runs one stage of hhr_decode_step on the same
 * workspace (layout above), reading the previous stage's results from it and
 * writing its own there, so a test can drive one stage from known inputs.
 * Arguments mean what they mean for hhr_decode_step.
 *   qprep         Q, R, W              -> q_rot, code_q, q_split
 *   page_bounds   meta, seq_len        -> score            (reads q_split)
 *   select_pages  seq_len, keep_pages  -> pages, n_pages   (reads score)
 *   hamming       codes, seq_len       -> ham              (reads pages, n_pages, code_q)
 *   select_keys   codes, seq_len       -> ham, sel/sel_idx, k_eff (reads pages, n_pages, code_q)
 *   attend        Q, K, V, seq_len     -> out              (reads sel/sel_idx, k_eff)
 */
hhr_status hhr_stage_qprep(const hhr_dims* dims, const void* Q, const float* R, const float* W,
                           int32_t max_keep_pages, int32_t top_k, void* workspace,
                           size_t workspace_bytes, void* stream);
hhr_status hhr_stage_page_bounds(const hhr_dims* dims, const float* meta, const int32_t* seq_len,
                                 int32_t max_keep_pages, int32_t top_k, void* workspace,
                                 size_t workspace_bytes, void* stream);
hhr_status hhr_stage_select_pages(const hhr_dims* dims, const int32_t* seq_len, const int32_t* keep_pages,
                                  int32_t max_keep_pages, int32_t top_k, void* workspace,
                                  size_t workspace_bytes, void* stream);
/* Hamming stage alone (LHP; rit.work HHR blog post, section "Почему
 * расстояние Хэмминга пропускает важные ключи"): for every candidate slot of
 * the kept pages, the Hamming distance between the slot key's code and the
 * group's query codes (summed over the group's Gh codes, or to the mean
 * query's code with hamming_group = 1), as uint16 in the workspace's ham
 * region, [B][units][max_keep_pages * page_size]; 0xFFFF for a slot past the
 * kept pages or the sequence, or on a sink or window key.  These are the
 * values hhr_stage_select_keys also writes there.  Same argument checks and
 * error codes as the other stage entry points. */
hhr_status hhr_stage_hamming(const hhr_dims* dims, const uint64_t* codes, const int32_t* seq_len,
                             int32_t max_keep_pages, int32_t top_k, void* workspace,
                             size_t workspace_bytes, void* stream);
hhr_status hhr_stage_select_keys(const hhr_dims* dims, const uint64_t* codes, const int32_t* seq_len,
                                 int32_t max_keep_pages, int32_t top_k, int32_t* sel_idx,
                                 void* workspace, size_t workspace_bytes, void* stream);
hhr_status hhr_stage_attend(const hhr_dims* dims, const void* Q, const void* K, const void* V,
                            const int32_t* seq_len, int32_t max_keep_pages, int32_t top_k,
                            float softmax_scale, const int32_t* sel_idx, float* out,
                            void* workspace, size_t workspace_bytes, void* stream);

const char* hhr_status_str(hhr_status status);
/* Message of the last failed call on this thread ("" if none). */
const char* hhr_last_error(void);
int32_t hhr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HHR_H */
