"""GPU parity of the TopK (Oracle) step (keys by exact logit) with the CPU
oracle, through the C ABI.

Bit-exact: the fp64 group-max logits z(t), the selected keys and k_eff.
Attention output within 2e-3 absolute of the oracle's fp64 result.  The cases
cover several tiles and a ragged tail, every group size the kernels are
built for, both element types and head sizes, empty and short sequences,
top_k >= L, heavy exact ties (integer-valued inputs, a zero query) on both
sides of the bucket-size limit, and the full 128K Llama-shaped layer.
"""
import numpy as np
import pytest

from gpu_common import ATOL, banner, gpu_dims, oracle_dims, to_dev
from synth import WORKLOADS, Workload, f32_to_bf16_bits, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import hash_sparse_attention_amd as hsa
    hsa.lib()  # fails loudly if libhhr.so is missing
    return torch.device("cuda:0")


def run_topk_gpu(wl: Workload, d: dict, dev, top_k: int, seq=None, scale=0.0, use_sel_out=True):
    import torch

    import hash_sparse_attention_amd as hsa
    dims = gpu_dims(wl)
    t = {k: to_dev(d[k], dev) for k in ("Q", "K", "V")}
    seq = d["seq_len"] if seq is None else np.asarray(seq, np.int32)
    seq_t = to_dev(np.asarray(seq, np.int32), dev)
    ws = hsa.alloc_topk_workspace(dims, top_k, dev)
    ws.fill_(0xA5)  # stale workspace contents must not matter
    out = torch.full((wl.batch, wl.n_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device=dev)
    sel = torch.full((wl.batch, wl.n_kv_heads, top_k), -7, dtype=torch.int32, device=dev) if use_sel_out else None
    hsa.topk_decode_step(dims, t["Q"], t["K"], t["V"], seq_t, top_k, out, ws, sel_idx=sel, scale=scale)
    torch.cuda.synchronize()
    score, wsel, keff = hsa.topk_workspace_view(dims, top_k, ws)
    return dict(out=out.cpu().numpy(), sel=(sel if use_sel_out else wsel).cpu().numpy(),
                score=score.cpu().numpy(), k_eff=keff.cpu().numpy())


def run_topk_oracle(wl: Workload, d: dict, top_k: int, seq=None, scale=0.0):
    import oracle
    seq = d["seq_len"] if seq is None else np.asarray(seq, np.int32)
    return oracle.topk(oracle_dims(wl), d["Q"], d["K"], d["V"], seq, top_k, scale)


def compare_topk(wl, seq, g, o, label=""):
    for b in range(wl.batch):
        L = int(seq[b])
        for h in range(wl.n_kv_heads):
            tag = f"{label} b={b} h={h}"
            assert np.array_equal(g["score"][b, h, :L].view(np.uint64), o["score"][b, h, :L].view(np.uint64)), \
                f"logits {tag}"
            assert np.array_equal(g["sel"][b, h], o["sel"][b, h]), f"selected keys {tag}"
            assert g["k_eff"][b, h] == o["k_eff"][b, h], f"k_eff {tag}"
        for i in range(wl.n_q_heads):
            err = np.abs(g["out"][b, i].astype(np.float64) - o["out"][b, i]).max()
            assert err <= ATOL, f"attention {label} b={b} qhead={i}: max |diff| {err}"


CASES = [
    # name, workload, top_k
    ("tiny_fp32_d64_g4", WORKLOADS["tiny"], 256),
    ("bf16_d128_g4_ragged_b3", Workload("tk_b3", 130, 3, 32, 8, 128, 5000, 16, 128, 10, 300, "bf16", outliers=2,
                                        ragged=(1, 5000)), 300),
    ("bf16_d64_g1", Workload("tk_g1", 131, 2, 2, 2, 64, 2500, 16, 64, 10, 100, "bf16", ragged=(900, 2500)), 100),
    ("fp32_d128_g7", Workload("tk_g7", 132, 1, 14, 2, 128, 3001, 16, 128, 10, 500, "fp32", outliers=2), 500),
    ("bf16_d64_g8", Workload("tk_g8", 133, 2, 16, 2, 64, 1100, 16, 64, 10, 64, "bf16"), 64),
    ("fp32_d64_g3_short", Workload("tk_g3", 134, 2, 6, 2, 64, 700, 16, 64, 10, 900, "fp32", ragged=(30, 700)), 900),
    ("bf16_d128_g2_t1", Workload("tk_t1", 135, 1, 4, 2, 128, 1500, 16, 128, 10, 1, "bf16"), 1),
    ("bf16_d128_g5_g6", Workload("tk_g5", 136, 1, 10, 2, 128, 9000, 16, 128, 10, 1200, "bf16", outliers=2), 1200),
    ("bf16_d128_g6", Workload("tk_g6", 137, 1, 12, 2, 128, 4100, 16, 128, 10, 700, "bf16"), 700),
]


@pytest.mark.parametrize("name,wl,top_k", CASES, ids=[c[0] for c in CASES])
def test_topk_parity_shapes(dev, name, wl, top_k):
    banner(f"topk {name}")
    d = make_layer(wl)
    g = run_topk_gpu(wl, d, dev, top_k)
    o = run_topk_oracle(wl, d, top_k)
    compare_topk(wl, d["seq_len"], g, o, label=name)


def test_topk_empty_and_all_keys(dev):
    """L = 0 (no keys, zero output), L < top_k and top_k >= every length (exact full attention)."""
    wl = Workload("tk_edge", 138, 4, 8, 2, 64, 3000, 16, 64, 10, 4000, "bf16", outliers=2)
    banner("topk empty / all keys")
    d = make_layer(wl)
    seq = np.array([0, 1, 2999, 3000], np.int32)
    g = run_topk_gpu(wl, d, dev, 4000, seq=seq, use_sel_out=False)
    o = run_topk_oracle(wl, d, 4000, seq=seq)
    compare_topk(wl, seq, g, o, label="edge")
    assert (g["out"][0] == 0).all() and (g["sel"][0] == -1).all()


def _integer_layer(wl, seed, lo=-2, hi=2):
    """Integer-valued Q and K (exact logits, many ties between distinct keys)."""
    rng = np.random.default_rng(seed)
    d = make_layer(wl)
    Q = rng.integers(lo, hi + 1, d["Q"].shape).astype(np.float32)
    K = rng.integers(lo, hi + 1, (wl.batch, wl.n_kv_heads, wl.ctx, wl.head_dim)).astype(np.float32)
    if wl.dtype == "bf16":
        Q, K = f32_to_bf16_bits(Q), f32_to_bf16_bits(K)
    d["Q"], d["K"] = Q, K
    return d


@pytest.mark.parametrize("T,top_k,zero_q", [(6000, 1000, False), (20000, 3000, False), (12000, 5000, True),
                                            (20000, 3000, True)],
                         ids=["ties_bucket", "ties_large", "zero_query_bucket", "zero_query_fallback"])
def test_topk_exact_ties(dev, T, top_k, zero_q):
    """Equal logits go to the lower key: small-integer inputs tie thousands of keys at the boundary
    value; a zero query ties every key (over 16384 of them forces the single-block fallback)."""
    wl = Workload(f"tk_tie{T}", 139, 2, 8, 2, 64, T, 16, 64, 10, top_k, "bf16")
    banner(f"topk ties T={T} top_k={top_k} zero_q={zero_q}")
    d = _integer_layer(wl, 7 + T)
    if zero_q:
        d["Q"][:] = 0
    g = run_topk_gpu(wl, d, dev, top_k)
    o = run_topk_oracle(wl, d, top_k)
    compare_topk(wl, d["seq_len"], g, o, label="ties")


def test_topk_repeated_and_stale_workspace(dev):
    """Two steps on one workspace, the second with shorter sequences: bitwise equal to fresh runs."""
    import torch

    import hash_sparse_attention_amd as hsa
    wl = Workload("tk_rep", 140, 2, 8, 2, 128, 6000, 16, 128, 10, 400, "bf16", outliers=2)
    banner("topk repeated steps")
    d = make_layer(wl)
    dims = gpu_dims(wl)
    t = {k: to_dev(d[k], dev) for k in ("Q", "K", "V")}
    ws = hsa.alloc_topk_workspace(dims, 400, dev)
    outs = []
    for seq in ([6000, 5000], [3000, 17]):
        s_t = to_dev(np.array(seq, np.int32), dev)
        out = torch.empty((wl.batch, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
        sel = torch.empty((wl.batch, wl.n_kv_heads, 400), dtype=torch.int32, device=dev)
        hsa.topk_decode_step(dims, t["Q"], t["K"], t["V"], s_t, 400, out, ws, sel_idx=sel)
        torch.cuda.synchronize()
        outs.append((np.array(seq, np.int32), out.cpu().numpy(), sel.cpu().numpy()))
    for seq, out, sel in outs:
        o = run_topk_oracle(wl, d, 400, seq=seq)
        assert np.array_equal(sel, o["sel"])
        assert np.abs(out.astype(np.float64) - o["out"]).max() <= ATOL


def test_topk_llama8b_128k_one_layer_full(dev):
    """The 128K Llama-3.1-8B-shaped layer (8 KV heads x 131072 keys, top_k 4096): every logit, every
    selected key and every output against the oracle."""
    wl = WORKLOADS["llama8b_128k"]
    banner("topk llama8b_128k layer 0 full")
    d = make_layer(wl, layer=0)
    g = run_topk_gpu(wl, d, dev, wl.top_k)
    o = run_topk_oracle(wl, d, wl.top_k)
    compare_topk(wl, d["seq_len"], g, o, label="llama8b_128k topk")


@pytest.mark.parametrize("name", ["llama8b_32k", "mistral7b_b8"])
def test_topk_selection_is_exact_top_k_at_scale(dev, name):
    """The defining property, checked on the device's own logits at full size (no oracle): every
    unselected key has a smaller logit than every selected key, or an equal one and a higher index."""
    wl = WORKLOADS[name]
    banner(f"topk exact-top-k property {name}")
    d = make_layer(wl)
    g = run_topk_gpu(wl, d, dev, wl.top_k)
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for h in range(wl.n_kv_heads):
            keff = int(g["k_eff"][b, h])
            assert keff == min(wl.top_k, L)
            sel = g["sel"][b, h, :keff]
            assert (np.diff(sel) > 0).all() and (g["sel"][b, h, keff:] == -1).all()
            z = g["score"][b, h, :L]
            mask = np.zeros(L, bool)
            mask[sel] = True
            zmin = z[mask].min()
            assert (z[~mask] <= zmin).all(), f"{name} b={b} h={h}"
            tied_out = np.nonzero(~mask & (z == zmin))[0]
            tied_in = sel[z[sel] == zmin]
            assert len(tied_out) == 0 or tied_out.min() > tied_in.max()


def test_topk_graph_replay_matches_eager(dev):
    """A captured HIP graph of the TopK step replays to the eager result every time, with eager work and
    synchronizations between replays (the step clears its own counters with a kernel, not a memset)."""
    import torch

    import hash_sparse_attention_amd as hsa
    wl = WORKLOADS["llama8b_32k"]
    banner("topk graph capture and replay")
    d = make_layer(wl)
    dims = gpu_dims(wl)
    t = {k: to_dev(d[k], dev) for k in ("Q", "K", "V")}
    seq = to_dev(d["seq_len"], dev)
    ws = hsa.alloc_topk_workspace(dims, wl.top_k, dev)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev)
    sel = torch.empty((1, 8, wl.top_k), dtype=torch.int32, device=dev)

    def step():
        hsa.topk_decode_step(dims, t["Q"], t["K"], t["V"], seq, wl.top_k, out, ws, sel_idx=sel)

    step()
    torch.cuda.synchronize()
    ref_out, ref_sel = out.clone(), sel.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.fill_(float("nan"))
        sel.fill_(-9)
        _ = (t["K"][0, 0, :8].float() * 2).sum().item()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(sel, ref_sel), f"replay {rep}"
