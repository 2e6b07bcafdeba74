"""Workload shapes and the seeded input recipe.

Shapes follow the models the HHR pages evaluate (thelatestinai.com page on
arXiv 2610.01230, Appendix Table 3: Llama-3.1-8B-Instruct has 32 layers, 32
attention heads, 8 KV heads, hidden size 4096 so head_dim 128, and a maximum
context of 131072; Mistral-7B-Instruct has 32 layers) and the 128-bit codes of
Appendix Table 4.  Values imitate the outlier-channel key geometry the GKR
rotation is meant to spread (Figure 3 caption): per-channel lognormal scales,
a few 20x outlier key channels, and queries correlated with 8 planted keys
along the query direction whose logits sit 8 standard deviations above the
random keys' mean (the largest of 128K random logits is about 4.5 of them
above it, so the planted keys lead every exact ranking).

Random numbers:
  numpy path: Generator(PCG64(SeedSequence([seed, workload_id, layer]))) with
  child streams spawned in a fixed order.  The torch path draws K, V and Q on
  the device with a seeded torch.Generator (different values, same recipe)
  and is used where host generation of multi-GB caches would be too slow.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int             # stable id mixed into the seed
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx: int             # Tmax: row capacity of the cache
    page_size: int
    hash_bits: int
    keep_percent: int    # pages kept, percent of each sequence's pages (rounded up, at least 1)
    top_k: int
    dtype: str           # "fp32" or "bf16" for Q, K, V
    layers: int = 1
    outliers: int = 0    # key channels scaled by 20
    ragged: tuple | None = None  # (lo, hi): per-sequence lengths uniform in [lo, hi]
    append_tokens: int = 0       # size of the encode-append chunk timed for this workload
    planted: int = 8
    meta_bf16: bool = False      # page metadata stored as outward-rounded bf16
    sink_tokens: int = 0         # decode variant: first keys always attended
    local_window: int = 0        # decode variant: last keys always attended
    page_group: int = 0          # decode variant: page score over the group, 0 = max, 1 = min
    hamming_group: int = 0       # decode variant: 0 = H summed over the group, 1 = H to the mean query's code
    per_head: bool = False       # decode variant: one selection per query head
    meta_split: bool = False     # page metadata stored sign-split (dimension-major, max and min sides apart)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def max_pages(self) -> int:
        return -(-self.ctx // self.page_size)

    @property
    def max_keep(self) -> int:
        return keep_for(self.ctx, self.page_size, self.keep_percent)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 8, 2, 64, 4096, 16, 64, 25, 256, "fp32"),
    "llama8b_32k": Workload("llama8b_32k", 1, 1, 32, 8, 128, 32768, 16, 128, 10, 2048, "bf16", outliers=2),
    "llama8b_128k": Workload("llama8b_128k", 2, 1, 32, 8, 128, 131072, 16, 128, 10, 4096, "bf16",
                             layers=32, outliers=2),
    "mistral7b_b8": Workload("mistral7b_b8", 3, 8, 32, 8, 128, 65536, 32, 64, 5, 2048, "bf16",
                             outliers=2, ragged=(32768, 65536)),
    "qwen7b_b16": Workload("qwen7b_b16", 4, 16, 28, 4, 128, 131072, 16, 128, 10, 4096, "bf16",
                           outliers=2, append_tokens=4096),
    # One query head per KV head (G = 1) at the Llama-3.1-8B KV-head shapes: the selection shape of the
    # sign-split metadata read.
    "mha_128k": Workload("mha_128k", 5, 1, 8, 8, 128, 131072, 16, 128, 10, 4096, "bf16", layers=32, outliers=2),
}


def keep_for(length: int, page: int, percent: int) -> int:
    """Pages kept for a sequence: ceil(percent * pages / 100), at least 1 (integer arithmetic)."""
    pages = -(-int(length) // page)
    return max(1, (percent * pages + 99) // 100)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _haar_orthogonal(rng: np.random.Generator, d: int) -> np.ndarray:
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


def _heads_params(wl: Workload, rngs):
    """Per-KV-head R, W, key/value channel scales (host, numpy)."""
    H, D, nb = wl.n_kv_heads, wl.head_dim, wl.hash_bits
    r_rng, w_rng, ks_rng, vs_rng, out_rng = rngs
    R = np.stack([_haar_orthogonal(r_rng, D) for _ in range(H)])
    W = w_rng.standard_normal((H, nb, D), dtype=np.float32)
    sK = ks_rng.lognormal(0.0, 1.0, (H, D))
    sV = vs_rng.lognormal(0.0, 1.0, (H, D))
    for h in range(H):
        if wl.outliers:
            ch = out_rng.choice(D, size=wl.outliers, replace=False)
            sK[h, ch] *= 20.0
    return R, W, sK, sV


def _lengths(wl: Workload, rng) -> np.ndarray:
    if wl.ragged is None:
        return np.full(wl.batch, wl.ctx, np.int32)
    lo, hi = wl.ragged
    return rng.integers(lo, hi + 1, size=wl.batch).astype(np.int32)


def _plant(u: np.ndarray, sK_h: np.ndarray) -> np.ndarray:
    """Key along u with u.k = 8 * std(u.k over the head's random keys)."""
    u = u.astype(np.float64)
    sigma = np.sqrt(np.sum(u ** 2 * sK_h ** 2))
    return (8.0 * sigma / np.sum(u ** 2)) * u


def make_layer(wl: Workload, layer: int = 0, seed: int = 0, lengths=None) -> dict:
    """Host (numpy) inputs of one layer.

    Returns Q [B][Hq][D], K/V [B][Hkv][T][D] (uint16 bf16 bit patterns, or fp32),
    R [Hkv][D][D] fp32, W [Hkv][b][D] fp32, seq_len [B] int32, keep [B] int32,
    planted [B][Hkv][n] int32 (the planted key positions).
    """
    ss = np.random.SeedSequence([seed, wl.wid, layer])
    kids = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(11)]
    R, W, sK, sV = _heads_params(wl, kids[0:5])
    k_rng, v_rng, qb_rng, qn_rng, pl_rng, len_rng = kids[5:11]
    B, Hq, H, D, T, G = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ctx, wl.group
    seq = np.asarray(lengths, np.int32) if lengths is not None else _lengths(wl, len_rng)
    K = k_rng.standard_normal((B, H, T, D), dtype=np.float32)
    K *= sK.astype(np.float32)[None, :, None, :]
    V = v_rng.standard_normal((B, H, T, D), dtype=np.float32)
    V *= sV.astype(np.float32)[None, :, None, :]
    Q = np.zeros((B, Hq, D), np.float32)
    planted = np.full((B, H, wl.planted), -1, np.int32)
    for b in range(B):
        for h in range(H):
            u = qb_rng.standard_normal(D)
            eps = qn_rng.standard_normal((G, D))
            Q[b, h * G:(h + 1) * G] = (u[None, :] + 0.5 * eps).astype(np.float32)
            n = min(wl.planted, int(seq[b]))
            if n:
                pos = np.sort(pl_rng.choice(int(seq[b]), size=n, replace=False))
                planted[b, h, :n] = pos
                K[b, h, pos] = _plant(u, sK[h]).astype(np.float32)[None, :]
    if wl.dtype == "bf16":
        Q, K, V = f32_to_bf16_bits(Q), f32_to_bf16_bits(K), f32_to_bf16_bits(V)
    keep = np.array([keep_for(int(L), wl.page_size, wl.keep_percent) for L in seq], np.int32)
    return dict(Q=Q, K=K, V=V, R=R, W=W, seq_len=seq, keep=keep, planted=planted)


def make_layer_torch(wl: Workload, layer: int, device, seed: int = 0, lengths=None) -> dict:
    """Device-resident inputs of one layer drawn with torch's generator (same recipe).

    Q/K/V are torch.bfloat16 (or float32) device tensors; R, W come from the
    numpy path (small), lengths and keep as int32 device tensors.
    """
    import torch

    ss = np.random.SeedSequence([seed, wl.wid, layer])
    kids = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(11)]
    R, W, sK, sV = _heads_params(wl, kids[0:5])
    qb_rng, qn_rng, pl_rng, len_rng = kids[7], kids[8], kids[9], kids[10]
    B, Hq, H, D, T, G = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.ctx, wl.group
    seq = np.asarray(lengths, np.int32) if lengths is not None else _lengths(wl, len_rng)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(ss.generate_state(1)[0]))
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    sKt = torch.from_numpy(sK.astype(np.float32)).to(device)
    sVt = torch.from_numpy(sV.astype(np.float32)).to(device)
    K = torch.empty((B, H, T, D), dtype=dt, device=device)
    V = torch.empty((B, H, T, D), dtype=dt, device=device)
    for b in range(B):
        for h in range(H):
            K[b, h] = (torch.randn((T, D), generator=gen, device=device) * sKt[h]).to(dt)
            V[b, h] = (torch.randn((T, D), generator=gen, device=device) * sVt[h]).to(dt)
    Q = np.zeros((B, Hq, D), np.float32)
    planted = np.full((B, H, wl.planted), -1, np.int32)
    for b in range(B):
        for h in range(H):
            u = qb_rng.standard_normal(D)
            eps = qn_rng.standard_normal((G, D))
            Q[b, h * G:(h + 1) * G] = (u[None, :] + 0.5 * eps).astype(np.float32)
            n = min(wl.planted, int(seq[b]))
            if n:
                pos = np.sort(pl_rng.choice(int(seq[b]), size=n, replace=False))
                planted[b, h, :n] = pos
                row = torch.from_numpy(_plant(u, sK[h]).astype(np.float32)).to(device).to(dt)
                K[b, h, torch.from_numpy(pos.astype(np.int64)).to(device)] = row
    keep = np.array([keep_for(int(L), wl.page_size, wl.keep_percent) for L in seq], np.int32)
    return dict(
        Q=torch.from_numpy(Q).to(device).to(dt), K=K, V=V,
        R=torch.from_numpy(R).to(device), W=torch.from_numpy(W).to(device),
        seq_len=torch.from_numpy(seq).to(device), keep=torch.from_numpy(keep).to(device),
        seq_len_host=seq, keep_host=keep, planted=planted)
