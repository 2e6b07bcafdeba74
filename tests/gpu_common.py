"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare them to the parity bar (bit-exact codes,
page metadata, query codes/rotations, page scores, page lists, Hamming
distances and key selections; attention within 2e-3 absolute)."""
from __future__ import annotations

import numpy as np

from synth import Workload

ATOL = 2e-3


def banner(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def to_dev(a, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def gpu_dims(wl: Workload):
    import hash_sparse_attention_amd as hsa
    return hsa.make_dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.page_size, wl.hash_bits, wl.ctx,
                         wl.dtype == "bf16", meta_bf16=wl.meta_bf16, sink_tokens=wl.sink_tokens,
                         local_window=wl.local_window, page_group=wl.page_group, hamming_group=wl.hamming_group,
                         per_head=wl.per_head, meta_split=wl.meta_split)


def oracle_dims(wl: Workload):
    import oracle
    return oracle.Dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.page_size, wl.hash_bits, wl.ctx,
                       wl.dtype == "bf16", wl.meta_bf16, wl.sink_tokens, wl.local_window, wl.page_group,
                       wl.hamming_group, wl.per_head)


def run_gpu(wl: Workload, d: dict, dev, keep=None, max_keep=None, top_k=None, seq=None, chunks=None,
            scale=0.0, use_sel_out=True):
    """Encode (one call, or the given (start, count, max_count) chunks) and one decode step on the GPU."""
    import torch

    import hash_sparse_attention_amd as hsa
    dims = gpu_dims(wl)
    seq = np.asarray(d["seq_len"] if seq is None else seq, np.int32)
    keep = np.asarray(d["keep"] if keep is None else keep, np.int32)
    max_keep = wl.max_keep if max_keep is None else max_keep
    top_k = wl.top_k if top_k is None else top_k
    t = {k: to_dev(d[k], dev) for k in ("Q", "K", "V", "R", "W")}
    seq_t, keep_t = to_dev(seq, dev), to_dev(keep, dev)
    meta, codes = hsa.alloc_cache(dims, dev)
    meta.fill_(float("nan"))
    codes.fill_(0x5A5A5A5A5A5A5A5A)
    if chunks is None:
        chunks = [(np.zeros(wl.batch, np.int32), seq, wl.ctx)]
    for st, cnt, mc in chunks:
        hsa.encode_cache(dims, t["K"], t["R"], t["W"], to_dev(np.asarray(st, np.int32), dev),
                         to_dev(np.asarray(cnt, np.int32), dev), mc, meta, codes)
    ws = hsa.alloc_workspace(dims, max_keep, top_k, dev)
    ws.fill_(0xA5)
    out = torch.full((wl.batch, wl.n_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device=dev)
    cap = hsa.sel_cap(dims, top_k)
    sel = torch.full((wl.batch, hsa.sel_units(dims), cap), -7, dtype=torch.int32, device=dev) if use_sel_out else None
    hsa.decode_step(dims, t["Q"], t["K"], t["V"], t["R"], t["W"], meta, codes, seq_t, keep_t, max_keep, top_k, out,
                    ws, sel_idx=sel, scale=scale)
    torch.cuda.synchronize()
    v = hsa.workspace_view(dims, max_keep, top_k, ws)
    r = dict(
        meta=hsa.meta_to_pages(meta, dims).cpu().numpy(),
        codes=codes.cpu().numpy().view(np.uint64).reshape(wl.batch, wl.n_kv_heads, wl.ctx, wl.hash_bits // 64),
        q_rot=v.q_rot.cpu().numpy(), code_q=v.code_q.cpu().numpy().view(np.uint64), score=v.score.cpu().numpy(),
        pages=v.pages.cpu().numpy(), n_pages=v.n_pages.cpu().numpy(), ham=v.ham.cpu().numpy().view(np.uint16),
        sel=(sel if use_sel_out else v.sel).cpu().numpy(), k_eff=v.k_eff.cpu().numpy(), out=out.cpu().numpy(),
    )
    r["_dev"] = dict(dims=dims, t=t, seq=seq_t, keep=keep_t, meta=meta, codes=codes, ws=ws, out=out, sel=sel,
                     max_keep=max_keep, top_k=top_k)
    return r


def run_oracle(wl: Workload, d: dict, keep=None, max_keep=None, top_k=None, seq=None, scale=0.0):
    import oracle
    od = oracle_dims(wl)
    seq = np.asarray(d["seq_len"] if seq is None else seq, np.int32)
    keep = np.asarray(d["keep"] if keep is None else keep, np.int32)
    max_keep = wl.max_keep if max_keep is None else max_keep
    top_k = wl.top_k if top_k is None else top_k
    meta, codes = oracle.encode(od, d["K"], d["R"], d["W"], np.zeros(wl.batch, np.int32), seq)
    r = oracle.decode(od, d["Q"], d["K"], d["V"], d["R"], d["W"], meta, codes, seq, keep, max_keep, top_k, scale)
    r["meta"], r["codes"] = meta, codes
    return r


def compare(wl: Workload, seq, g: dict, o: dict, batches=None, label=""):
    """Assert the parity bar for the listed sequences (default: all)."""
    P = wl.page_size
    batches = range(wl.batch) if batches is None else batches
    for gi, b in enumerate(batches):
        ob = gi if o["codes"].shape[0] != wl.batch else b  # the oracle may have run on a slice
        L = int(seq[b])
        NP = -(-L // P)
        for h in range(wl.n_kv_heads):
            tag = f"{label} b={b} h={h}"
            assert np.array_equal(g["codes"][b, h, :L], o["codes"][ob, h, :L]), f"codes {tag}"
            assert np.array_equal(g["meta"][b, h, :NP].view(np.uint32), o["meta"][ob, h, :NP].view(np.uint32)), \
                f"meta {tag}"
        for h in range(wl.n_q_heads if wl.per_head else wl.n_kv_heads):  # selection rows
            tag = f"{label} b={b} unit={h}"
            assert np.array_equal(g["score"][b, h, :NP].view(np.uint64), o["score"][ob, h, :NP].view(np.uint64)), \
                f"page scores {tag}"
            assert np.array_equal(g["pages"][b, h], o["pages"][ob, h]), f"pages {tag}"
            assert g["n_pages"][b, h] == o["n_pages"][ob, h], f"n_pages {tag}"
            assert np.array_equal(g["ham"][b, h], o["ham"][ob, h]), f"hamming {tag}"
            assert np.array_equal(g["sel"][b, h], o["sel"][ob, h]), f"selected keys {tag}"
            assert g["k_eff"][b, h] == o["k_eff"][ob, h], f"k_eff {tag}"
        for i in range(wl.n_q_heads):
            tag = f"{label} b={b} qhead={i}"
            assert np.array_equal(g["q_rot"][b, i].view(np.uint32), o["q_rot"][ob, i].view(np.uint32)), f"q_rot {tag}"
            assert np.array_equal(g["code_q"][b, i], o["code_q"][ob, i]), f"code_q {tag}"
            err = np.abs(g["out"][b, i].astype(np.float64) - o["out"][ob, i]).max()
            assert err <= ATOL, f"attention {tag}: max |diff| {err}"
