"""Retrieval fidelity of the HHR selection on seeded synthetic inputs.

The pages evaluate HHR's two-stage retrieval by how much of the exact attention
it keeps: recall of the keys exact attention ranks highest, and the effect
of the candidate budget and the code length ("HHR: Hierarchical Hash
Retrieval for Efficient LLM Generation", Abstract; thelatestinai.com page,
Figure 4 and Figures 9-10 captions).  Without the pages' datasets and
trained R_h / W_h, this module measures the same quantities on the seeded
synthetic workloads, for the selections the library makes.

Per (sequence, KV head), with z_i,t = scale * q_i . k_t in fp64 for the G
query heads i of the group and the keys t < L:
  - key recall: the share of the exact top-k keys (by max_i z_i,t, ties to
    the lower index, k = the number of keys the library selected) that the
    library selected;
  - page coverage: the share of those exact top-k keys whose page the
    library kept (what the page stage lets through to the Hamming stage);
  - attention mass: sum over the selected keys of the full softmax of z_i,
    averaged over the group's query heads;
  - output error: max |out - out_full| against full fp64 attention;
  - planted recall: the share of the planted keys that were selected.
Reported per setting as the mean over (sequence, KV head), the output error
as the max.

The Hamming-versus-logit view (thelatestinai.com page, Figure 2 caption:
Hamming distances of a random orthogonal projection followed by sign, set
against the query-key logits): for every query head i and key t < L of one
KV head, H_i(t) = popcount(code(q_i) XOR code(k_t)) from the library's own
codes against z_i(t) = q_i . k_t, tabulated by distance bin, with the rank
correlation between -H and z and the share of the exact top 1% keys that
the Hamming order also puts in its top 1%.

The exact references are plain fp64 numpy on the host: this is a
measurement tool beside the bench, not a path of the library, which is why
it sits outside the binding package.  `python fidelity.py --workload
llama8b_32k` runs a sweep of keep percentages and code lengths on the GPU
and prints one table; `--scatter` prints the Hamming-versus-logit table
instead.
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np


def _f32(x, bf16: bool) -> np.ndarray:
    if bf16:
        return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, np.float32)


def metrics(wl, d: dict, sel: np.ndarray, out: np.ndarray, pages: np.ndarray, n_pages: np.ndarray,
            scale: float = 0.0) -> dict:
    """Fidelity of one layer's selection.  sel [B][Hkv][top_k] (ascending, -1 padded), out [B][Hq][D],
    pages [B][Hkv][max_keep] (-1 padded), n_pages [B][Hkv]; d is the synthetic layer (synth.make_layer)."""
    bf16 = wl.dtype == "bf16"
    Q, K, V = _f32(d["Q"], bf16), _f32(d["K"], bf16), _f32(d["V"], bf16)
    G, P, D = wl.group, wl.page_size, wl.head_dim
    sc = scale if scale > 0 else 1.0 / np.sqrt(D)
    rec, cov, mass, plant = [], [], [], []
    err = 0.0
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for h in range(wl.n_kv_heads):
            chosen = sel[b, h][sel[b, h] >= 0].astype(np.int64)
            if L == 0 or len(chosen) == 0:
                continue
            q = Q[b, h * G:(h + 1) * G].astype(np.float64)
            z = sc * (q @ K[b, h, :L].astype(np.float64).T)  # [G][L]
            s = z.max(axis=0)
            k = len(chosen)
            exact = np.lexsort((np.arange(L), -s))[:k]
            rec.append(np.isin(exact, chosen).mean())
            kept = pages[b, h, :int(n_pages[b, h])]
            cov.append(np.isin(exact // P, kept).mean())
            zm = z - z.max(axis=1, keepdims=True)
            pr = np.exp(zm)
            pr /= pr.sum(axis=1, keepdims=True)
            mass.append(pr[:, chosen].sum(axis=1).mean())
            full = pr @ V[b, h, :L].astype(np.float64)  # [G][D]
            err = max(err, float(np.abs(out[b, h * G:(h + 1) * G].astype(np.float64) - full).max()))
            pl = d["planted"][b, h]
            pl = pl[pl >= 0]
            if len(pl):
                plant.append(np.isin(pl, chosen).mean())
    mean = lambda v: float(np.mean(v)) if v else float("nan")
    return dict(key_recall=mean(rec), page_coverage=mean(cov), attention_mass=mean(mass), out_max_err=err,
                planted_recall=mean(plant), units=len(rec))


def popcount64(x: np.ndarray) -> np.ndarray:
    """Bits set in each uint64 (SWAR, on the host)."""
    x = np.asarray(x, np.uint64)
    m1, m2, m4 = np.uint64(0x5555555555555555), np.uint64(0x3333333333333333), np.uint64(0x0F0F0F0F0F0F0F0F)
    x = x - ((x >> np.uint64(1)) & m1)
    x = (x & m2) + ((x >> np.uint64(2)) & m2)
    x = (x + (x >> np.uint64(4))) & m4
    return ((x * np.uint64(0x0101010101010101)) >> np.uint64(56)).astype(np.int64)


def _ranks(a: np.ndarray) -> np.ndarray:
    """Ranks 1..n with ties given their mean rank."""
    order = np.argsort(a, kind="stable")
    r = np.empty(len(a), np.float64)
    r[order] = np.arange(1, len(a) + 1)
    uniq, inv, cnt = np.unique(a, return_inverse=True, return_counts=True)
    sums = np.bincount(inv, weights=r)
    return (sums / cnt)[inv]


def hamming_logit(wl, d: dict, codes: np.ndarray, code_q: np.ndarray, b: int = 0, h: int = 0,
                  n_bins: int = 16) -> dict:
    """Hamming distance against logit on KV head h of sequence b, over every query head of its group.

    codes [B][Hkv][T][W] and code_q [B][Hq][W] (uint64) are the library's codes of the keys and queries.
    Returns rows (lo, hi, keys, mean z, p10 z, p90 z, max z) per distance bin [lo, hi], the Spearman
    correlation of -H with z (per query head, averaged), and the top-1% overlap (averaged).
    """
    bf16 = wl.dtype == "bf16"
    G, nb = wl.group, wl.hash_bits
    L = int(d["seq_len"][b])
    Q, K = _f32(d["Q"], bf16), _f32(d["K"], bf16)
    ck = np.asarray(codes[b, h, :L]).view(np.uint64)
    Hs, Zs, rho, top = [], [], [], []
    for i in range(h * G, (h + 1) * G):
        cq = np.asarray(code_q[b, i]).view(np.uint64)
        H = popcount64(ck ^ cq[None, :]).sum(axis=1)
        z = K[b, h, :L].astype(np.float64) @ Q[b, i].astype(np.float64)
        Hs.append(H)
        Zs.append(z)
        rz, rh = _ranks(z), _ranks(-H.astype(np.float64))
        rho.append(float(np.corrcoef(rz, rh)[0, 1]))
        k = max(1, L // 100)
        exact = np.lexsort((np.arange(L), -z))[:k]
        by_h = np.lexsort((np.arange(L), H))[:k]
        top.append(float(np.isin(exact, by_h).mean()))
    H, z = np.concatenate(Hs), np.concatenate(Zs)
    edges = np.linspace(0, nb, n_bins + 1)
    rows = []
    for j in range(n_bins):
        lo, hi = int(np.ceil(edges[j])), int(np.ceil(edges[j + 1])) - (1 if j + 1 < n_bins else 0)
        m = (H >= lo) & (H <= hi)
        if m.any():
            zz = z[m]
            rows.append((lo, hi, int(m.sum()), float(zz.mean()), float(np.percentile(zz, 10)),
                         float(np.percentile(zz, 90)), float(zz.max())))
        else:
            rows.append((lo, hi, 0, float("nan"), float("nan"), float("nan"), float("nan")))
    return dict(rows=rows, spearman=float(np.mean(rho)), top1_overlap=float(np.mean(top)), keys=int(len(z)))


def hamming_table(res: dict) -> str:
    lines = ["| H from | H to | keys | mean logit | p10 | p90 | max |", "|---|---|---|---|---|---|---|"]
    for lo, hi, n, mu, p10, p90, mx in res["rows"]:
        if n:
            lines.append(f"| {lo} | {hi} | {n} | {mu:.2f} | {p10:.2f} | {p90:.2f} | {mx:.2f} |")
    lines.append("")
    lines.append(f"Spearman(-H, logit) = {res['spearman']:.3f}; exact top-1% keys also in the Hamming top 1%: "
                 f"{res['top1_overlap']:.3f} ({res['keys']} (query head, key) pairs)")
    return "\n".join(lines)


def run_library(wl, d: dict, dev, scale: float = 0.0, want_codes: bool = False):
    """Encode and one decode step of the layer through the library; returns (out, sel, pages, n_pages), plus
    (codes, code_q) as host arrays when want_codes."""
    import torch

    import hash_sparse_attention_amd as hsa

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    dims = hsa.make_dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.page_size, wl.hash_bits, wl.ctx,
                         wl.dtype == "bf16", meta_bf16=wl.meta_bf16)
    t = {k: to_dev(d[k]) for k in ("Q", "K", "V", "R", "W")}
    seq, keep = to_dev(d["seq_len"]), to_dev(d["keep"])
    meta, codes = hsa.alloc_cache(dims, dev)
    hsa.encode_cache(dims, t["K"], t["R"], t["W"], to_dev(np.zeros(wl.batch, np.int32)), seq, wl.ctx, meta, codes)
    ws = hsa.alloc_workspace(dims, wl.max_keep, wl.top_k, dev)
    out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    sel = torch.empty((wl.batch, wl.n_kv_heads, wl.top_k), dtype=torch.int32, device=dev)
    hsa.decode_step(dims, t["Q"], t["K"], t["V"], t["R"], t["W"], meta, codes, seq, keep, wl.max_keep, wl.top_k,
                    out, ws, sel_idx=sel, scale=scale)
    torch.cuda.synchronize()
    v = hsa.workspace_view(dims, wl.max_keep, wl.top_k, ws)
    res = (out.cpu().numpy(), sel.cpu().numpy(), v.pages.cpu().numpy(), v.n_pages.cpu().numpy())
    if want_codes:
        nw = wl.hash_bits // 64
        cd = codes.view(wl.batch, wl.n_kv_heads, wl.ctx, nw).cpu().numpy().view(np.uint64)
        res = res + (cd, v.code_q.cpu().numpy().view(np.uint64))
    return res


def sweep(workload: str, keeps, bits, layer: int = 0, dev=None, meta_bf16: bool = False) -> list:
    import torch

    from synth import WORKLOADS, make_layer
    dev = dev or torch.device("cuda:0")
    rows = []
    for nb in bits:
        for kp in keeps:
            wl = WORKLOADS[workload].with_(hash_bits=nb, keep_percent=kp, meta_bf16=meta_bf16)
            d = make_layer(wl, layer=layer)
            out, sel, pages, n_pages = run_library(wl, d, dev)
            m = metrics(wl, d, sel, out, pages, n_pages)
            m.update(workload=workload, layer=layer, hash_bits=nb, keep_percent=kp, top_k=wl.top_k,
                     meta="bf16" if meta_bf16 else "fp32")
            rows.append(m)
            print(f"[fidelity] bits {nb} keep {kp}%: recall {m['key_recall']:.3f} coverage {m['page_coverage']:.3f} "
                  f"mass {m['attention_mass']:.3f} err {m['out_max_err']:.2e} planted {m['planted_recall']:.3f}",
                  file=sys.stderr, flush=True)
    return rows


def table(rows: list) -> str:
    lines = ["| code bits | keep % | top-k | key recall | page coverage | attention mass | max out err | planted recall |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['hash_bits']} | {r['keep_percent']} | {r['top_k']} | {r['key_recall']:.3f} | "
                     f"{r['page_coverage']:.3f} | {r['attention_mass']:.3f} | {r['out_max_err']:.2e} | "
                     f"{r['planted_recall']:.3f} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--keep", default="5,10,20,40", help="keep percentages of pages")
    ap.add_argument("--bits", default="64,128", help="code lengths")
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--meta", choices=("fp32", "bf16"), default="fp32")
    ap.add_argument("--json", default="", help="also write the rows to this file")
    ap.add_argument("--scatter", action="store_true", help="Hamming-versus-logit table instead of the sweep")
    ap.add_argument("--orthogonal-w", action="store_true",
                    help="with --scatter: codes from W_h = R_h (a random orthogonal projection, b = D)")
    ap.add_argument("--head", type=int, default=0)
    a = ap.parse_args(argv)
    if a.scatter:
        import torch

        from synth import WORKLOADS, make_layer
        nb = [int(x) for x in a.bits.split(",")][0]
        wl = WORKLOADS[a.workload].with_(hash_bits=nb, meta_bf16=a.meta == "bf16")
        d = make_layer(wl, layer=a.layer)
        if a.orthogonal_w:
            if nb != wl.head_dim:
                raise SystemExit("--orthogonal-w needs --bits equal to the head size")
            d["W"] = d["R"].copy()
        *_, cd, cq = run_library(wl, d, torch.device("cuda:0"), want_codes=True)
        res = hamming_logit(wl, d, cd, cq, h=a.head)
        print(hamming_table(res))
        if a.json:
            json.dump(res, open(a.json, "w"), indent=1)
        return
    rows = sweep(a.workload, [int(x) for x in a.keep.split(",")], [int(x) for x in a.bits.split(",")], a.layer,
                 meta_bf16=a.meta == "bf16")
    print(table(rows))
    if a.json:
        json.dump(rows, open(a.json, "w"), indent=1)


if __name__ == "__main__":
    main()
