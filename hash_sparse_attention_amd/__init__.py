"""Python binding of libhhr, the MI355X (gfx950) HHR decode-path library.

Argument marshalling only: every function forwards torch tensors' device
pointers and the current HIP stream to the C ABI declared in include/hhr.h
and raises HHRError on a nonzero status.  All computation happens in the HIP
kernels of libhhr.so; there is no CPU fallback -- importing the binding
without a built libhhr.so raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhhr.so")

HHR_F32, HHR_BF16 = 0, 1
HHR_META_INTERLEAVED, HHR_META_SIGN_SPLIT = 0, 1
STATUS = {0: "HHR_OK", 1: "HHR_E_NULL", 2: "HHR_E_SHAPE", 3: "HHR_E_DTYPE", 4: "HHR_E_ALIGN",
          5: "HHR_E_WORKSPACE", 6: "HHR_E_RANGE", 7: "HHR_E_UNSUPPORTED", 8: "HHR_E_HIP"}


class HHRError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "page_size", "hash_bits", "max_ctx", "kv_dtype",
        "meta_dtype", "sink_tokens", "local_window", "page_group", "hamming_group", "per_head", "meta_layout")]

    def __repr__(self):
        return "Dims(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "q_rot", "code_q", "q_split", "score", "pages", "n_pages", "ham", "sel", "k_eff", "partial",
        "counters", "total")] + [("n_splits", ctypes.c_int32)]


class TopkLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("score", "sel", "k_eff", "total")]


_lib = None


def lib():
    """The loaded libhhr.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with hash_sparse_attention_amd.build.build()")
        # torch first: it ships a HIP runtime with the same soname as ROCm's, and whichever loads first is
        # the one the process uses.  libhhr then runs on torch's runtime, the one that owns the tensors and
        # streams it is given (loaded the other way round, its launches found no device).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        p, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        D = ctypes.POINTER(Dims)
        sig = {
            "hhr_meta_bytes": (sz, [D]),
            "hhr_codes_bytes": (sz, [D]),
            "hhr_encode_cache": (ctypes.c_int, [D, p, p, p, p, p, i32, p, p, p]),
            "hhr_decode_workspace_bytes": (sz, [D, i32, i32]),
            "hhr_decode_workspace_layout": (ctypes.c_int, [D, i32, i32, ctypes.POINTER(WorkspaceLayout)]),
            "hhr_decode_step": (ctypes.c_int, [D, p, p, p, p, p, p, p, p, p, i32, i32, f32, p, p, p, sz, p]),
            "hhr_decode_step_append": (ctypes.c_int, [D, p, p, p, p, p, p, p, p, p, i32, p, p, i32, i32, f32, p, p,
                                                      p, sz, p]),
            "hhr_noalloc_scratch_bytes": (sz, []),
            "hhr_decode_step_append_noalloc": (ctypes.c_int, [D, p, p, p, p, p, p, p, p, p, i32, p, p, i32, i32, f32,
                                                              p, p, p]),
            "hhr_topk_workspace_layout": (ctypes.c_int, [D, i32, ctypes.POINTER(TopkLayout)]),
            "hhr_topk_workspace_bytes": (sz, [D, i32]),
            "hhr_topk_decode_step": (ctypes.c_int, [D, p, p, p, p, i32, f32, p, p, p, sz, p]),
            "hhr_stage_topk_logits": (ctypes.c_int, [D, p, p, i32, p, sz, p]),
            "hhr_stage_qprep": (ctypes.c_int, [D, p, p, p, i32, i32, p, sz, p]),
            "hhr_stage_page_bounds": (ctypes.c_int, [D, p, p, i32, i32, p, sz, p]),
            "hhr_stage_select_pages": (ctypes.c_int, [D, p, p, i32, i32, p, sz, p]),
            "hhr_stage_hamming": (ctypes.c_int, [D, p, p, i32, i32, p, sz, p]),
            "hhr_stage_select_keys": (ctypes.c_int, [D, p, p, i32, i32, p, p, sz, p]),
            "hhr_stage_attend": (ctypes.c_int, [D, p, p, p, p, i32, i32, f32, p, p, p, sz, p]),
            "hhr_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "hhr_last_error": (ctypes.c_char_p, []),
            "hhr_abi_version": (i32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


EXPORTED = ("hhr_meta_bytes", "hhr_codes_bytes", "hhr_encode_cache", "hhr_decode_workspace_bytes",
            "hhr_decode_workspace_layout", "hhr_decode_step", "hhr_decode_step_append", "hhr_noalloc_scratch_bytes",
            "hhr_decode_step_append_noalloc", "hhr_topk_workspace_layout",
            "hhr_topk_workspace_bytes", "hhr_topk_decode_step", "hhr_stage_topk_logits", "hhr_stage_qprep",
            "hhr_stage_page_bounds",
            "hhr_stage_select_pages", "hhr_stage_hamming", "hhr_stage_select_keys", "hhr_stage_attend",
            "hhr_status_str",
            "hhr_last_error", "hhr_abi_version")


def _check(st: int):
    if st != 0:
        raise HHRError(st, lib().hhr_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, n: int, what: str):
    """Raise before any launch if tensor t (when given) holds fewer than n elements."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements, the call writes {n}")


def _check_outputs(dims: "Dims", top_k: int, out, sel_idx):
    _need(out, dims.batch * dims.n_q_heads * dims.head_dim, "out")
    _need(sel_idx, dims.batch * sel_units(dims) * sel_cap(dims, top_k), "sel_idx")


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_dims(batch, n_q_heads, n_kv_heads, head_dim, page_size, hash_bits, max_ctx, bf16: bool,
              meta_bf16: bool = False, sink_tokens: int = 0, local_window: int = 0, page_group: int = 0,
              hamming_group: int = 0, per_head: bool = False, meta_split: bool = False) -> Dims:
    """meta_bf16: store page metadata as outward-rounded bf16 (half the bytes of the page-bound stream).
    sink_tokens, local_window: keys always attended by the decode step (the first and the last ones); its
    selection rows then hold top_k + sink_tokens + local_window entries (`sel_cap`).
    page_group = 1 scores a page by the min over the GQA group (default 0: max); hamming_group = 1 ranks keys
    by the distance to the code of the group's mean query (default 0: summed over the group's codes).
    per_head: one selection per query head instead of one per KV head (per-(b, h) rows become per query head).
    meta_split: store page metadata dimension-major with the max and min sides apart, so a selection of one
    query head reads only the side its query's sign picks (half the bytes of the page-bound stream)."""
    return Dims(batch, n_q_heads, n_kv_heads, head_dim, page_size, hash_bits, max_ctx,
                HHR_BF16 if bf16 else HHR_F32, HHR_BF16 if meta_bf16 else HHR_F32, int(sink_tokens),
                int(local_window), int(page_group), int(hamming_group), int(bool(per_head)),
                HHR_META_SIGN_SPLIT if meta_split else HHR_META_INTERLEAVED)


def sel_units(dims: Dims) -> int:
    """Selection rows per sequence: query heads with per-query-head selection, else KV heads."""
    return dims.n_q_heads if dims.per_head else dims.n_kv_heads


def sel_cap(dims: Dims, top_k: int) -> int:
    """Entries per (sequence, KV head) row of the decode step's selection."""
    return int(top_k) + dims.sink_tokens + dims.local_window


def dims_from(K, Q, W, page_size: int) -> Dims:
    """Dims from tensor shapes: K [B][Hkv][T][D], Q [B][Hq][D], W [Hkv][b][D]."""
    import torch
    B, Hkv, T, D = K.shape
    if K.dtype not in (torch.bfloat16, torch.float32) or Q.dtype != K.dtype:
        raise TypeError("Q and K must both be bfloat16 or both float32")
    return make_dims(B, Q.shape[1], Hkv, D, page_size, W.shape[1], T, K.dtype == torch.bfloat16)


def meta_bytes(dims: Dims) -> int:
    return int(lib().hhr_meta_bytes(ctypes.byref(dims)))


def codes_bytes(dims: Dims) -> int:
    return int(lib().hhr_codes_bytes(ctypes.byref(dims)))


def alloc_cache(dims: Dims, device="cuda"):
    """Device buffers for (meta, codes), sized by the library."""
    import torch
    meta = torch.empty(meta_bytes(dims) // 4, dtype=torch.float32, device=device)
    codes = torch.empty(codes_bytes(dims) // 8, dtype=torch.int64, device=device)
    return meta, codes


def encode_cache(dims: Dims, K, R, W, start, count, max_count: int, meta, codes, stream=None):
    _check(lib().hhr_encode_cache(ctypes.byref(dims), _ptr(K), _ptr(R), _ptr(W), _ptr(start), _ptr(count),
                                  int(max_count), _ptr(meta), _ptr(codes), _stream(stream)))


def workspace_bytes(dims: Dims, max_keep: int, top_k: int) -> int:
    return int(lib().hhr_decode_workspace_bytes(ctypes.byref(dims), int(max_keep), int(top_k)))


def workspace_layout(dims: Dims, max_keep: int, top_k: int) -> WorkspaceLayout:
    lay = WorkspaceLayout()
    _check(lib().hhr_decode_workspace_layout(ctypes.byref(dims), int(max_keep), int(top_k), ctypes.byref(lay)))
    return lay


def alloc_workspace(dims: Dims, max_keep: int, top_k: int, device="cuda"):
    import torch
    return torch.empty(workspace_bytes(dims, max_keep, top_k), dtype=torch.uint8, device=device)


def decode_step(dims: Dims, Q, K, V, R, W, meta, codes, seq_len, keep_pages, max_keep: int, top_k: int,
                out, workspace, sel_idx=None, scale: float = 0.0, stream=None):
    _check_outputs(dims, top_k, out, sel_idx)
    _check(lib().hhr_decode_step(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(R), _ptr(W), _ptr(meta),
                                 _ptr(codes), _ptr(seq_len), _ptr(keep_pages), int(max_keep), int(top_k),
                                 float(scale), _ptr(out), _ptr(sel_idx), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))


def decode_step_append(dims: Dims, Q, K, V, R, W, meta, codes, append_start, append_count, max_append: int,
                       seq_len, keep_pages, max_keep: int, top_k: int, out, workspace, sel_idx=None,
                       scale: float = 0.0, stream=None):
    _check_outputs(dims, top_k, out, sel_idx)
    _check(lib().hhr_decode_step_append(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(R), _ptr(W), _ptr(meta),
                                        _ptr(codes), _ptr(append_start), _ptr(append_count), int(max_append),
                                        _ptr(seq_len), _ptr(keep_pages), int(max_keep), int(top_k), float(scale),
                                        _ptr(out), _ptr(sel_idx), _ptr(workspace), workspace.numel(),
                                        _stream(stream)))


def noalloc_scratch_bytes() -> int:
    """Size of the library's static per-GPU scratch (the limit of decode_step_append_noalloc)."""
    return int(lib().hhr_noalloc_scratch_bytes())


def decode_step_append_noalloc(dims: Dims, Q, K, V, R, W, meta, codes, append_start, append_count,
                               max_append: int, seq_len, keep_pages, max_keep: int, top_k: int, out, sel_idx=None,
                               scale: float = 0.0, stream=None):
    """decode_step_append on the library's static per-GPU scratch instead of a caller workspace (nothing is
    allocated; calls that overlap on one GPU race on that scratch)."""
    _check_outputs(dims, top_k, out, sel_idx)
    _check(lib().hhr_decode_step_append_noalloc(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(R), _ptr(W),
                                                _ptr(meta), _ptr(codes), _ptr(append_start), _ptr(append_count),
                                                int(max_append), _ptr(seq_len), _ptr(keep_pages), int(max_keep),
                                                int(top_k), float(scale), _ptr(out), _ptr(sel_idx),
                                                _stream(stream)))


def topk_workspace_layout(dims: Dims, top_k: int) -> TopkLayout:
    lay = TopkLayout()
    _check(lib().hhr_topk_workspace_layout(ctypes.byref(dims), int(top_k), ctypes.byref(lay)))
    return lay


def alloc_topk_workspace(dims: Dims, top_k: int, device="cuda"):
    import torch
    return torch.empty(topk_workspace_layout(dims, top_k).total, dtype=torch.uint8, device=device)


def topk_decode_step(dims: Dims, Q, K, V, seq_len, top_k: int, out, workspace, sel_idx=None, scale: float = 0.0,
                     stream=None):
    """TopK (Oracle) step: keys by exact logit (fp64), then the same gather attention."""
    _need(out, dims.batch * dims.n_q_heads * dims.head_dim, "out")
    _need(sel_idx, dims.batch * dims.n_kv_heads * int(top_k), "sel_idx")
    _check(lib().hhr_topk_decode_step(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(seq_len), int(top_k),
                                      float(scale), _ptr(out), _ptr(sel_idx), _ptr(workspace), workspace.numel(),
                                      _stream(stream)))


def stage_topk_logits(dims: Dims, K, seq_len, top_k: int, workspace, stream=None):
    """The logit kernel of the TopK (Oracle) step alone (after one full step on the same workspace)."""
    _check(lib().hhr_stage_topk_logits(ctypes.byref(dims), _ptr(K), _ptr(seq_len), int(top_k), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))


def topk_workspace_view(dims: Dims, top_k: int, workspace):
    """(score fp64 [B][Hkv][max_ctx], sel int32 [B][Hkv][top_k], k_eff int32 [B][Hkv]) views of a TopK workspace."""
    import torch
    lay = topk_workspace_layout(dims, top_k)
    B, Hkv, T = dims.batch, dims.n_kv_heads, dims.max_ctx

    def region(off, dtype, shape, esize):
        n = esize
        for x in shape:
            n *= x
        return workspace[off:off + n].view(dtype).view(*shape)

    return (region(lay.score, torch.float64, (B, Hkv, T), 8), region(lay.sel, torch.int32, (B, Hkv, top_k), 4),
            region(lay.k_eff, torch.int32, (B, Hkv), 4))


def stage_qprep(dims, Q, R, W, max_keep, top_k, workspace, stream=None):
    _check(lib().hhr_stage_qprep(ctypes.byref(dims), _ptr(Q), _ptr(R), _ptr(W), int(max_keep), int(top_k),
                                 _ptr(workspace), workspace.numel(), _stream(stream)))


def stage_page_bounds(dims, meta, seq_len, max_keep, top_k, workspace, stream=None):
    _check(lib().hhr_stage_page_bounds(ctypes.byref(dims), _ptr(meta), _ptr(seq_len), int(max_keep), int(top_k),
                                       _ptr(workspace), workspace.numel(), _stream(stream)))


def stage_select_pages(dims, seq_len, keep_pages, max_keep, top_k, workspace, stream=None):
    _check(lib().hhr_stage_select_pages(ctypes.byref(dims), _ptr(seq_len), _ptr(keep_pages), int(max_keep),
                                        int(top_k), _ptr(workspace), workspace.numel(), _stream(stream)))


def stage_hamming(dims, codes, seq_len, max_keep, top_k, workspace, stream=None):
    _check(lib().hhr_stage_hamming(ctypes.byref(dims), _ptr(codes), _ptr(seq_len), int(max_keep), int(top_k),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))


def stage_select_keys(dims, codes, seq_len, max_keep, top_k, workspace, sel_idx=None, stream=None):
    _need(sel_idx, dims.batch * sel_units(dims) * sel_cap(dims, top_k), "sel_idx")
    _check(lib().hhr_stage_select_keys(ctypes.byref(dims), _ptr(codes), _ptr(seq_len), int(max_keep), int(top_k),
                                       _ptr(sel_idx), _ptr(workspace), workspace.numel(), _stream(stream)))


def stage_attend(dims, Q, K, V, seq_len, max_keep, top_k, out, workspace, sel_idx=None, scale=0.0, stream=None):
    _check_outputs(dims, top_k, out, sel_idx)
    _check(lib().hhr_stage_attend(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(seq_len), int(max_keep),
                                  int(top_k), float(scale), _ptr(sel_idx), _ptr(out), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))


@dataclass
class WorkspaceView:
    """Typed views of the intermediate results a decode step leaves in its workspace."""
    q_rot: object
    code_q: object
    q_split: object
    score: object
    pages: object
    n_pages: object
    ham: object
    sel: object
    k_eff: object


def workspace_view(dims: Dims, max_keep: int, top_k: int, workspace) -> WorkspaceView:
    import torch
    lay = workspace_layout(dims, max_keep, top_k)
    B, Hq, D, P = dims.batch, dims.n_q_heads, dims.head_dim, dims.page_size
    Hkv = sel_units(dims)  # per-(b, h) rows: query heads with per-query-head selection
    G, NW = Hq // Hkv, dims.hash_bits // 64
    NP = -(-dims.max_ctx // P)
    # The bound terms keep the per-KV-head layout, per-query-head selection included (one pass over a KV
    # head's metadata serves all its query heads).
    Hd = dims.n_kv_heads
    qs_shape = (B, Hd, D, Hq // Hd, 2)

    def region(off, dtype, shape):
        n = 1
        for s in shape:
            n *= s
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        return workspace[off:off + nbytes].view(dtype).view(*shape)

    return WorkspaceView(
        q_rot=region(lay.q_rot, torch.float32, (B, Hq, D)),
        code_q=region(lay.code_q, torch.int64, (B, Hq, NW)),
        q_split=region(lay.q_split, torch.float64, qs_shape),
        score=region(lay.score, torch.float64, (B, Hkv, NP)),
        pages=region(lay.pages, torch.int32, (B, Hkv, max_keep)),
        n_pages=region(lay.n_pages, torch.int32, (B, Hkv)),
        ham=region(lay.ham, torch.int16, (B, Hkv, max_keep * P)),
        sel=region(lay.sel, torch.int32, (B, Hkv, sel_cap(dims, top_k))),
        k_eff=region(lay.k_eff, torch.int32, (B, Hkv)),
    )


def meta_to_pages(meta_flat, dims: Dims):
    """Reshape the meta buffer (page-block interleaved, or sign-split) to [B][Hkv][NPmax][D][2] (max, min) fp32
    (bf16 metadata widened exactly); a host-side view helper."""
    import torch
    B, Hkv, D = dims.batch, dims.n_kv_heads, dims.head_dim
    NP = -(-dims.max_ctx // dims.page_size)
    NPB = -(-NP // 64)
    if dims.meta_layout == HHR_META_SIGN_SPLIT:
        m = meta_flat.view(torch.bfloat16) if dims.meta_dtype == HHR_BF16 else meta_flat
        m = m.reshape(B, Hkv, NPB, D, 2, 64)  # [..][blk][dim][max/min][lane]
        m = m.permute(0, 1, 2, 5, 3, 4).reshape(B, Hkv, NPB * 64, D, 2).float()
    elif dims.meta_dtype == HHR_BF16:
        m = meta_flat.view(torch.bfloat16).reshape(B, Hkv, NPB, D // 4, 64, 4, 2)  # [..][blk][quad][lane][dim][max/min]
        m = m.permute(0, 1, 2, 4, 3, 5, 6).reshape(B, Hkv, NPB * 64, D, 2).float()
    else:
        m = meta_flat.reshape(B, Hkv, NPB, D // 2, 64, 2, 2)  # [..][blk][pair][lane][dim-in-pair][max/min]
        m = m.permute(0, 1, 2, 4, 3, 5, 6).reshape(B, Hkv, NPB * 64, D, 2)
    return m[:, :, :NP]
