"""HHR decode-path oracle -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``hhr_oracle.c``, the plain CPU statement of what the
HHR decode path computes (canonical fp32 projections, fp64 page bounds, exact
sorts, fp64 attention).  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package; the GPU library
never does, and the two share no code.

Every function follows the passage cited in ``hhr_oracle.c``:
"HHR: Hierarchical Hash Retrieval for Efficient LLM Generation", Abstract;
the rit.work blog post on HHR, section "Два уровня маршрутизации решают
разные ошибки"; thelatestinai.com figure captions (Figures 2-4) and Appendix
Table 4.

Parity status: every stage is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute force, closed forms, invariants and
special cases that reduce to textbook routines).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hhr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# The mutation tests point this at a deliberately broken build of the same source.
_LIB_OVERRIDE = os.environ.get("HHR_ORACLE_LIB")
_lib = None


def compile_source(src: str, out: str, extra=()) -> str:
    """gcc build of an oracle source file (IEEE fp32/fp64, no contraction, no fast-math); `extra` adds
    flags (the sanitizer test builds with -fsanitize=address,undefined)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-mfma",
           "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter", *extra, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "page_size", "hash_bits", "max_ctx", "kv_bf16",
        "meta_bf16", "sink_tokens", "local_window", "page_group", "hamming_group")]


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        lib.oracle_project.argtypes = [ctypes.c_int32, ctypes.c_int32, p, p, p, ctypes.c_int64, p, p]
        lib.oracle_encode.argtypes = [ctypes.POINTER(_Dims), p, p, p, p, p, p, p]
        lib.oracle_decode.argtypes = [ctypes.POINTER(_Dims), p, p, p, p, p, p, p, p, p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_float] + [p] * 9
        lib.oracle_select_pages.argtypes = [ctypes.POINTER(_Dims), p, p, p, ctypes.c_int32, p, p]
        lib.oracle_topk.argtypes = [ctypes.POINTER(_Dims), p, p, p, p, ctypes.c_int32, ctypes.c_float] + [p] * 4
        lib.oracle_max_threads.argtypes = []
        for f in (lib.oracle_project, lib.oracle_encode, lib.oracle_decode, lib.oracle_select_pages,
                  lib.oracle_topk, lib.oracle_max_threads):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


@dataclass(frozen=True)
class Dims:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    hash_bits: int
    max_ctx: int
    kv_bf16: bool
    meta_bf16: bool = False  # page max/min rounded outward to bf16 values
    sink_tokens: int = 0     # decode: the first sink_tokens keys are always attended
    local_window: int = 0    # decode: the last local_window keys are always attended
    page_group: int = 0      # decode: page score over the group, 0 = max, 1 = min
    hamming_group: int = 0   # decode: 0 = H summed over the group's codes, 1 = H to the mean query's code
    per_head: bool = False   # decode: one selection per query head instead of one per KV head

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def words(self) -> int:
        return self.hash_bits // 64

    @property
    def max_pages(self) -> int:
        return -(-self.max_ctx // self.page_size)

    def c(self) -> _Dims:
        return _Dims(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.page_size,
                     self.hash_bits, self.max_ctx, int(self.kv_bf16), int(self.meta_bf16), int(self.sink_tokens),
                     int(self.local_window), int(self.page_group), int(self.hamming_group))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _kv(a, dims: Dims):
    return _c(a, np.uint16 if dims.kv_bf16 else np.float32)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def project(R, W, X):
    """Canonical-chain projection of the rows of X (n x D fp32) by one head's R (D x D) and W (b x D).

    Returns (Xrot [n][D] fp32, codes [n][b/64] uint64).
    """
    R = _c(R, np.float32); W = _c(W, np.float32); X = _c(X, np.float32)
    n, D = X.shape
    nb = W.shape[0]
    xr = np.zeros((n, D), np.float32)
    cd = np.zeros((n, nb // 64), np.uint64)
    st = _load().oracle_project(D, nb, _ptr(R), _ptr(W), _ptr(X), n, _ptr(xr), _ptr(cd))
    if st:
        raise ValueError(f"oracle_project failed ({st})")
    return xr, cd


def alloc_cache(dims: Dims):
    """Zeroed meta [B][Hkv][NPmax][D][2] fp32 and codes [B][Hkv][Tmax][b/64] uint64."""
    meta = np.zeros((dims.batch, dims.n_kv_heads, dims.max_pages, dims.head_dim, 2), np.float32)
    codes = np.zeros((dims.batch, dims.n_kv_heads, dims.max_ctx, dims.words), np.uint64)
    return meta, codes


def encode(dims: Dims, K, R, W, start, count, meta=None, codes=None):
    """Encode keys [start[b], start[b]+count[b]) into (meta, codes); returns them (updated in place)."""
    if meta is None or codes is None:
        meta, codes = alloc_cache(dims)
    K = _kv(K, dims); R = _c(R, np.float32); W = _c(W, np.float32)
    start = _c(np.asarray(start, np.int32), np.int32); count = _c(np.asarray(count, np.int32), np.int32)
    assert meta.flags.c_contiguous and codes.flags.c_contiguous
    st = _load().oracle_encode(ctypes.byref(dims.c()), _ptr(K), _ptr(R), _ptr(W), _ptr(start), _ptr(count),
                               _ptr(meta), _ptr(codes))
    if st:
        raise ValueError(f"oracle_encode failed ({st})")
    return meta, codes


def decode(dims: Dims, Q, K, V, R, W, meta, codes, seq_len, keep_pages, max_keep, top_k, scale=0.0):
    """One decode step; returns a dict of every intermediate and the fp64 output (sel holds
    top_k + sink_tokens + local_window entries per head).

    per_head: every query head selects for itself.  By definition that is the shared-selection step on the
    same inputs with each KV head's data (K, V, R_h, W_h, metadata, codes) repeated for its G query heads,
    which is what is run: the per-(b, h) outputs then hold one row per query head."""
    if dims.per_head and dims.group > 1:
        from dataclasses import replace
        G = dims.group
        rep = lambda a, axis: np.ascontiguousarray(np.repeat(np.asarray(a), G, axis=axis))
        de = replace(dims, n_kv_heads=dims.n_q_heads, per_head=False)
        return decode(de, Q, rep(K, 1), rep(V, 1), rep(R, 0), rep(W, 0), rep(meta, 1), rep(codes, 1), seq_len,
                      keep_pages, max_keep, top_k, scale)
    B, Hq, Hkv, D, P = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.page_size
    Q = _kv(Q, dims); K = _kv(K, dims); V = _kv(V, dims)
    R = _c(R, np.float32); W = _c(W, np.float32)
    meta = _c(meta, np.float32); codes = _c(codes, np.uint64)
    seq_len = _c(np.asarray(seq_len, np.int32), np.int32)
    keep_pages = _c(np.asarray(keep_pages, np.int32), np.int32)
    r = dict(
        q_rot=np.zeros((B, Hq, D), np.float32),
        code_q=np.zeros((B, Hq, dims.words), np.uint64),
        score=np.zeros((B, Hkv, dims.max_pages), np.float64),
        pages=np.zeros((B, Hkv, max_keep), np.int32),
        n_pages=np.zeros((B, Hkv), np.int32),
        ham=np.zeros((B, Hkv, max_keep * P), np.uint16),
        sel=np.zeros((B, Hkv, top_k + dims.sink_tokens + dims.local_window), np.int32),
        k_eff=np.zeros((B, Hkv), np.int32),
        out=np.zeros((B, Hq, D), np.float64),
    )
    st = _load().oracle_decode(
        ctypes.byref(dims.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(R), _ptr(W), _ptr(meta), _ptr(codes),
        _ptr(seq_len), _ptr(keep_pages), int(max_keep), int(top_k), float(scale),
        *(_ptr(r[k]) for k in ("q_rot", "code_q", "score", "pages", "n_pages", "ham", "sel", "k_eff", "out")))
    if st:
        raise ValueError(f"oracle_decode failed ({st})")
    return r


def select_pages(dims: Dims, score, seq_len, keep_pages, max_keep):
    """The page select of `decode` alone, on given scores [B][Hkv][NPmax] fp64: returns (pages, n_pages)."""
    score = _c(score, np.float64)
    assert score.shape == (dims.batch, dims.n_kv_heads, dims.max_pages)
    seq_len = _c(np.asarray(seq_len, np.int32), np.int32)
    keep_pages = _c(np.asarray(keep_pages, np.int32), np.int32)
    pages = np.zeros((dims.batch, dims.n_kv_heads, max_keep), np.int32)
    n_pages = np.zeros((dims.batch, dims.n_kv_heads), np.int32)
    st = _load().oracle_select_pages(ctypes.byref(dims.c()), _ptr(score), _ptr(seq_len), _ptr(keep_pages),
                                     int(max_keep), _ptr(pages), _ptr(n_pages))
    if st:
        raise ValueError(f"oracle_select_pages failed ({st})")
    return pages, n_pages


def topk(dims: Dims, Q, K, V, seq_len, top_k, scale=0.0):
    """TopK (Oracle) step: keys by exact logit, then attention; returns dict(score, sel, k_eff, out).

    score [B][Hkv][Tmax] fp64 is the group-max logit z(t) (0 for t >= L); only batch, heads,
    head_dim, max_ctx and the kv dtype of `dims` matter.
    """
    B, Hq, Hkv, D = dims.batch, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    Q = _kv(Q, dims); K = _kv(K, dims); V = _kv(V, dims)
    seq_len = _c(np.asarray(seq_len, np.int32), np.int32)
    r = dict(score=np.zeros((B, Hkv, dims.max_ctx), np.float64), sel=np.zeros((B, Hkv, top_k), np.int32),
             k_eff=np.zeros((B, Hkv), np.int32), out=np.zeros((B, Hq, D), np.float64))
    st = _load().oracle_topk(ctypes.byref(dims.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(seq_len), int(top_k),
                             float(scale), *(_ptr(r[k]) for k in ("score", "sel", "k_eff", "out")))
    if st:
        raise ValueError(f"oracle_topk failed ({st})")
    return r
