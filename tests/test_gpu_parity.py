"""GPU parity of the HIP decode path with the CPU oracle, through the C ABI.

Bit-exact: key codes, page metadata, query rotations and codes, fp64 page
scores, kept-page lists, Hamming distances, selected keys.  Attention output
within 2e-3 absolute of the oracle's fp64 result.
"""
import numpy as np
import pytest

from gpu_common import banner, compare, run_gpu, run_oracle
from synth import WORKLOADS, Workload, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import hash_sparse_attention_amd as hsa
    hsa.lib()  # fails loudly if libhhr.so is missing
    return torch.device("cuda:0")


SHAPES = [
    # name, B, Hq, Hkv, D, T, P, b, keep%, top_k, dtype, ragged
    ("tiny", None),
    ("d64_b128_g1_p1", Workload("p1", 101, 2, 2, 2, 64, 300, 1, 128, 20, 17, "bf16", ragged=(1, 300))),
    ("d128_b64_g2_p4", Workload("p4", 102, 2, 4, 2, 128, 1000, 4, 64, 15, 100, "fp32", ragged=(500, 1000))),
    ("d128_b128_g7_p16", Workload("g7", 103, 3, 14, 2, 128, 2000, 16, 128, 10, 150, "bf16", outliers=2,
                                  ragged=(1, 2000))),
    ("d64_b64_g8_p64", Workload("g8", 104, 1, 16, 2, 64, 3000, 64, 64, 30, 400, "bf16")),
    ("d128_b128_g3_p32", Workload("g3", 105, 2, 6, 2, 128, 777, 32, 128, 40, 64, "fp32", ragged=(700, 777))),
    ("d128_b128_g4_p8_b3", Workload("b3", 106, 3, 8, 2, 128, 5000, 8, 128, 10, 333, "bf16", outliers=2,
                                    ragged=(4000, 5000))),
    ("d64_b128_g5_p2", Workload("g5", 107, 1, 5, 1, 64, 1500, 2, 128, 5, 70, "fp32")),
    ("d128_b64_g6_p16", Workload("g6", 108, 2, 12, 2, 128, 2500, 16, 64, 20, 120, "fp32", outliers=2,
                                 ragged=(900, 2500))),
]


@pytest.mark.parametrize("name,wl", SHAPES, ids=[s[0] for s in SHAPES])
def test_decode_parity_shapes(dev, name, wl):
    wl = WORKLOADS["tiny"] if wl is None else wl
    banner(f"decode parity {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


@pytest.mark.parametrize("name", ["tiny", "d64_b128_g1_p1", "d128_b128_g7_p16", "d64_b64_g8_p64", "llama8b_32k",
                                  "llama8b_128k"])
def test_bf16_meta_parity(dev, name):
    """Outward-rounded bf16 page metadata: meta (widened), scores, pages, distances, selections bit for bit and
    attention within the bar, against the oracle run with the same metadata rule."""
    wl = WORKLOADS[name] if name in WORKLOADS else dict(SHAPES)[name]
    wl = (WORKLOADS["tiny"] if wl is None else wl).with_(meta_bf16=True)
    banner(f"bf16 meta parity {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=f"{name} bf16 meta")


def test_empty_and_tiny_sequences(dev):
    wl = Workload("edge", 110, 4, 8, 2, 128, 600, 16, 128, 25, 40, "bf16")
    banner("empty and tiny sequences")
    d = make_layer(wl, lengths=[0, 1, 15, 600])
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label="edge")
    assert (g["out"][0] == 0).all() and (g["sel"][0] == -1).all()


@pytest.mark.parametrize("keep,top_k", [(0, 1), (10**6, 50), (3, 10**4), (2, 1)])
def test_keep_and_topk_edges(dev, keep, top_k):
    wl = WORKLOADS["tiny"]
    banner(f"keep={keep} top_k={top_k}")
    d = make_layer(wl)
    mk = min(wl.max_pages, 300)
    g = run_gpu(wl, d, dev, keep=[keep], max_keep=mk, top_k=top_k)
    o = run_oracle(wl, d, keep=[keep], max_keep=mk, top_k=top_k)
    compare(wl, d["seq_len"], g, o, label=f"keep={keep},k={top_k}")


def test_full_selection_is_full_attention(dev):
    wl = Workload("full", 111, 2, 8, 2, 128, 512, 16, 128, 100, 512, "bf16", outliers=2, ragged=(100, 512))
    banner("all pages kept, top_k >= length")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev, keep=[wl.max_pages] * 2, max_keep=wl.max_pages, top_k=512)
    o = run_oracle(wl, d, keep=[wl.max_pages] * 2, max_keep=wl.max_pages, top_k=512)
    compare(wl, d["seq_len"], g, o, label="full")


def test_ties_zero_projection_and_duplicate_pages(dev):
    wl = Workload("ties", 112, 1, 4, 2, 64, 1024, 16, 64, 10, 37, "fp32")
    banner("ties: W = 0 and duplicated pages")
    d = make_layer(wl)
    d["W"][:] = 0.0
    K = d["K"]
    for h in range(2):
        for p in range(1, 64, 3):
            K[0, h, p * 16:(p + 1) * 16] = K[0, h, 0:16]
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label="ties")


def test_split_select_empty_ties_and_duplicates(dev):
    """Enough candidate slots per KV head that the decode step splits the Hamming scan over several blocks:
    empty, one-key and one-page sequences beside a full one, every distance tied (W = 0, so the first
    k_eff candidates in key order win across block boundaries) and duplicated pages (tied page bounds)."""
    import hash_sparse_attention_amd as hsa
    from gpu_common import gpu_dims
    wl = Workload("split_ties", 115, 4, 8, 2, 128, 4096, 16, 128, 50, 700, "bf16", outliers=2)
    lay = hsa.workspace_layout(gpu_dims(wl), wl.max_keep, wl.top_k)
    banner(f"split select: {lay.total} workspace bytes")
    d = make_layer(wl, lengths=[0, 1, 16, 4096])
    d["W"][:] = 0.0
    K = d["K"]
    for h in range(2):
        for p in range(2, 256, 5):
            K[3, h, p * 16:(p + 1) * 16] = K[3, h, 16:32]
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label="split ties")
    assert (g["out"][0] == 0).all() and (g["sel"][0] == -1).all()


def test_explicit_scale_and_workspace_sel(dev):
    wl = WORKLOADS["tiny"]
    banner("explicit softmax scale, selection left in the workspace")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev, scale=0.05, use_sel_out=False)
    o = run_oracle(wl, d, scale=0.05)
    compare(wl, d["seq_len"], g, o, label="scale")


def test_encode_in_chunks_matches_single_shot(dev):
    """Bulk encode of a prefix, then 1-token appends (row-per-lane kernel), then a 100-key chunk
    (key-per-lane kernel) starting mid-page: bit-identical to the oracle's single-shot encode."""
    wl = Workload("chunks", 113, 2, 8, 2, 128, 1200, 16, 128, 20, 64, "bf16", outliers=2)
    banner("encode in chunks")
    d = make_layer(wl, lengths=[1100, 1037])
    B = 2
    chunks = [(np.zeros(B, np.int32), np.array([900, 837], np.int32), 900)]
    pos = np.array([900, 837], np.int32)
    for _ in range(5):
        chunks.append((pos.copy(), np.ones(B, np.int32), 1))
        pos += 1
    chunks.append((pos.copy(), np.array([30, 60], np.int32), 60))    # append kernel, counts differ
    pos += np.array([30, 60], np.int32)
    chunks.append((pos.copy(), np.array([100, 100], np.int32), 100))  # bulk kernel
    pos += 100
    chunks.append((pos.copy(), np.array([65, 35], np.int32), 100))    # bulk kernel, ragged counts
    pos += np.array([65, 35], np.int32)
    assert list(pos) == [1100, 1037]
    g = run_gpu(wl, d, dev, chunks=chunks)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label="chunks")


def test_llama8b_32k_full(dev):
    wl = WORKLOADS["llama8b_32k"]
    banner("llama8b_32k full layer")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label="llama8b_32k")


def test_llama8b_128k_one_layer_full(dev):
    wl = WORKLOADS["llama8b_128k"]
    banner("llama8b_128k layer 0 full")
    d = make_layer(wl, layer=0)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label="llama8b_128k L0")


def _sampled(wl, d, g, batches, label, keep=None):
    sl = {k: d[k][batches] for k in ("Q", "K", "V", "seq_len", "keep")}
    sl["R"], sl["W"] = d["R"], d["W"]
    wls = wl.with_(batch=len(batches))
    o = run_oracle(wls, sl)
    compare(wl, d["seq_len"], g, o, batches=batches, label=label)


def test_mistral7b_b8_ragged_sampled(dev):
    wl = WORKLOADS["mistral7b_b8"]
    banner("mistral7b_b8 ragged batch, oracle on sequences 0 and 5")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    _sampled(wl, d, g, [0, 5], "mistral7b_b8")


def test_qwen7b_b16_append_4096_sampled(dev):
    """Qwen2.5-7B attention shape (28 query / 4 KV heads, G = 7), batch 16 at 128K, inputs drawn on the device:
    encode all but the last 4096 tokens of each sequence, append those 4096 with hhr_encode_cache (the bulk
    path), decode; the oracle (single-shot encode + decode) runs on sequences 0 and 11."""
    import torch

    import hash_sparse_attention_amd as hsa
    from gpu_common import gpu_dims, to_dev
    from synth import make_layer_torch
    wl = WORKLOADS["qwen7b_b16"]
    banner("qwen7b_b16: 4096-token append, oracle on sequences 0 and 11")
    d = make_layer_torch(wl, 0, dev)
    dims = gpu_dims(wl)
    seq = d["seq_len_host"]
    new = np.full(wl.batch, wl.append_tokens, np.int32)
    pre = seq - new
    meta, codes = hsa.alloc_cache(dims, dev)
    meta.fill_(float("nan"))
    codes.fill_(0x5A5A5A5A5A5A5A5A)
    zero = to_dev(np.zeros(wl.batch, np.int32), dev)
    hsa.encode_cache(dims, d["K"], d["R"], d["W"], zero, to_dev(pre, dev), wl.ctx, meta, codes)
    hsa.encode_cache(dims, d["K"], d["R"], d["W"], to_dev(pre, dev), to_dev(new, dev), int(new.max()), meta, codes)
    ws = hsa.alloc_workspace(dims, wl.max_keep, wl.top_k, dev)
    ws.fill_(0xA5)
    out = torch.full((wl.batch, wl.n_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device=dev)
    sel = torch.full((wl.batch, wl.n_kv_heads, wl.top_k), -7, dtype=torch.int32, device=dev)
    hsa.decode_step(dims, d["Q"], d["K"], d["V"], d["R"], d["W"], meta, codes, d["seq_len"], d["keep"],
                    wl.max_keep, wl.top_k, out, ws, sel_idx=sel)
    torch.cuda.synchronize()
    v = hsa.workspace_view(dims, wl.max_keep, wl.top_k, ws)
    g = dict(meta=hsa.meta_to_pages(meta, dims).cpu().numpy(),
             codes=codes.cpu().numpy().view(np.uint64).reshape(wl.batch, wl.n_kv_heads, wl.ctx, 2),
             q_rot=v.q_rot.cpu().numpy(), code_q=v.code_q.cpu().numpy().view(np.uint64),
             score=v.score.cpu().numpy(), pages=v.pages.cpu().numpy(), n_pages=v.n_pages.cpu().numpy(),
             ham=v.ham.cpu().numpy().view(np.uint16), sel=sel.cpu().numpy(), k_eff=v.k_eff.cpu().numpy(),
             out=out.cpu().numpy())
    batches = [0, 11]

    def bits(x):
        return x[batches].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    sl = dict(Q=bits(d["Q"]), K=bits(d["K"]), V=bits(d["V"]), R=d["R"].cpu().numpy(), W=d["W"].cpu().numpy(),
              seq_len=seq[batches], keep=d["keep_host"][batches])
    o = run_oracle(wl.with_(batch=len(batches)), sl)
    compare(wl, seq, g, o, batches=batches, label="qwen7b_b16")


@pytest.mark.parametrize("meta_bf16,variant", [(False, {}), (True, {}),
                                               (False, dict(sink_tokens=3, local_window=40, hamming_group=1)),
                                               (True, dict(page_group=1)), (False, dict(per_head=True)),
                                               (False, dict(per_head=True, meta_split=True)),
                                               (True, dict(meta_split=True))],
                         ids=["fp32_meta", "bf16_meta", "sinks_window_mean_code", "bf16_meta_min_page", "per_head",
                              "per_head_sign_split", "bf16_meta_sign_split"])
def test_decode_step_append_matches_oracle(dev, meta_bf16, variant):
    """hhr_decode_step_append (fused append + query projection) equals the oracle's single-shot encode +
    decode, for a 1-token append, a ragged multi-token append, and an append larger than the fused limit."""
    import torch

    import hash_sparse_attention_amd as hsa
    from gpu_common import gpu_dims, to_dev
    wl = Workload("fused", 114, 3, 12, 3, 128, 700, 16, 128, 20, 48, "bf16", outliers=2, meta_bf16=meta_bf16,
                  **variant)
    d = make_layer(wl, lengths=[700, 650, 333])
    o = run_oracle(wl, d)
    for new in ([1, 1, 1], [5, 17, 1], [70, 3, 100]):
        banner(f"decode_step_append new={new}")
        new = np.array(new, np.int32)
        seq = d["seq_len"]
        pre = seq - new
        dims = gpu_dims(wl)
        t = {k: to_dev(d[k], dev) for k in ("Q", "K", "V", "R", "W")}
        meta, codes = hsa.alloc_cache(dims, dev)
        hsa.encode_cache(dims, t["K"], t["R"], t["W"], to_dev(np.zeros(3, np.int32), dev), to_dev(pre, dev),
                         int(pre.max()), meta, codes)
        ws = hsa.alloc_workspace(dims, wl.max_keep, wl.top_k, dev)
        out = torch.empty((3, 12, 128), dtype=torch.float32, device=dev)
        sel = torch.empty((3, hsa.sel_units(dims), hsa.sel_cap(dims, wl.top_k)), dtype=torch.int32, device=dev)
        hsa.decode_step_append(dims, t["Q"], t["K"], t["V"], t["R"], t["W"], meta, codes, to_dev(pre, dev),
                               to_dev(new, dev), int(new.max()), to_dev(seq, dev), to_dev(d["keep"], dev),
                               wl.max_keep, wl.top_k, out, ws, sel_idx=sel)
        torch.cuda.synchronize()
        v = hsa.workspace_view(dims, wl.max_keep, wl.top_k, ws)
        g = dict(meta=hsa.meta_to_pages(meta, dims).cpu().numpy(),
                 codes=codes.cpu().numpy().view(np.uint64).reshape(3, 3, wl.ctx, 2),
                 q_rot=v.q_rot.cpu().numpy(), code_q=v.code_q.cpu().numpy().view(np.uint64),
                 score=v.score.cpu().numpy(), pages=v.pages.cpu().numpy(), n_pages=v.n_pages.cpu().numpy(),
                 ham=v.ham.cpu().numpy().view(np.uint16), sel=sel.cpu().numpy(), k_eff=v.k_eff.cpu().numpy(),
                 out=out.cpu().numpy())
        compare(wl, seq, g, o, label=f"fused new={list(new)}")


def test_repeated_steps_are_bitwise_deterministic(dev):
    import torch

    import hash_sparse_attention_amd as hsa
    wl = WORKLOADS["llama8b_32k"].with_(batch=2, ragged=(20000, 32768))
    banner("determinism: three decode steps, bitwise equal")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    x = g["_dev"]
    outs = []
    for _ in range(3):
        x["out"].fill_(float("nan"))
        hsa.decode_step(x["dims"], x["t"]["Q"], x["t"]["K"], x["t"]["V"], x["t"]["R"], x["t"]["W"], x["meta"],
                        x["codes"], x["seq"], x["keep"], x["max_keep"], x["top_k"], x["out"], x["ws"],
                        sel_idx=x["sel"])
        torch.cuda.synchronize()
        outs.append((x["out"].clone(), x["sel"].clone()))
    for o_, s_ in outs[1:]:
        assert torch.equal(o_, outs[0][0]) and torch.equal(s_, outs[0][1])
    assert np.array_equal(outs[0][0].cpu().numpy(), g["out"])


def test_graph_replay_matches_eager(dev):
    """A captured HIP graph of append + decode replays to the eager result every time, with eager work and
    synchronizations between replays."""
    import torch

    import hash_sparse_attention_amd as hsa
    from gpu_common import gpu_dims, to_dev
    wl = WORKLOADS["llama8b_32k"]
    banner("graph capture and replay")
    d = make_layer(wl)
    dims = gpu_dims(wl)
    t = {k: to_dev(d[k], dev) for k in ("Q", "K", "V", "R", "W")}
    seq, keep = to_dev(d["seq_len"], dev), to_dev(d["keep"], dev)
    meta, codes = hsa.alloc_cache(dims, dev)
    hsa.encode_cache(dims, t["K"], t["R"], t["W"], to_dev(np.zeros(1, np.int32), dev), seq, wl.ctx, meta, codes)
    ws = hsa.alloc_workspace(dims, wl.max_keep, wl.top_k, dev)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device=dev)
    sel = torch.empty((1, 8, wl.top_k), dtype=torch.int32, device=dev)
    a_start, a_count = (seq - 1).contiguous(), torch.ones(1, dtype=torch.int32, device=dev)

    def step():
        hsa.decode_step_append(dims, t["Q"], t["K"], t["V"], t["R"], t["W"], meta, codes, a_start, a_count, 1,
                               seq, keep, wl.max_keep, wl.top_k, out, ws, sel_idx=sel)

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


def test_stages_from_oracle_intermediates(dev):
    """Each stage entry point, fed the oracle's result of the previous stage, reproduces the oracle's next
    result (isolates a stage from the ones before it)."""
    import torch

    import hash_sparse_attention_amd as hsa
    from gpu_common import gpu_dims, to_dev
    wl = WORKLOADS["tiny"].with_(batch=2, ragged=(3000, 4096))
    banner("stage isolation")
    d = make_layer(wl)
    o = run_oracle(wl, d)
    dims = gpu_dims(wl)
    mk, tk = wl.max_keep, wl.top_k
    ws = hsa.alloc_workspace(dims, mk, tk, dev)
    v = hsa.workspace_view(dims, mk, tk, ws)
    seq, keep = to_dev(d["seq_len"], dev), to_dev(d["keep"], dev)
    t = {k: to_dev(d[k], dev) for k in ("Q", "K", "V", "R", "W")}
    # meta/codes from the oracle, converted to the library's layouts on the host
    meta_gpu, codes_gpu = hsa.alloc_cache(dims, dev)
    NPB = -(-wl.max_pages // 64)
    om = np.zeros((2, wl.n_kv_heads, NPB * 64, wl.head_dim, 2), np.float32)
    om[:, :, :wl.max_pages] = o["meta"]
    om = om.reshape(2, wl.n_kv_heads, NPB, 64, wl.head_dim // 2, 2, 2).transpose(0, 1, 2, 4, 3, 5, 6)
    meta_gpu.copy_(torch.from_numpy(np.ascontiguousarray(om).reshape(-1)).to(dev))
    codes_gpu.copy_(torch.from_numpy(o["codes"].view(np.int64).reshape(-1)).to(dev))
    # stage 1 (qprep) -> compare
    hsa.stage_qprep(dims, t["Q"], t["R"], t["W"], mk, tk, ws)
    torch.cuda.synchronize()
    assert np.array_equal(v.q_rot.cpu().numpy().view(np.uint32), o["q_rot"].view(np.uint32))
    assert np.array_equal(v.code_q.cpu().numpy().view(np.uint64), o["code_q"])
    # stage 2 (bounds) on the oracle's meta
    hsa.stage_page_bounds(dims, meta_gpu, seq, mk, tk, ws)
    torch.cuda.synchronize()
    sc = v.score.cpu().numpy()
    for b in range(2):
        NP = -(-int(d["seq_len"][b]) // wl.page_size)
        assert np.array_equal(sc[b, :, :NP].view(np.uint64), o["score"][b, :, :NP].view(np.uint64))
    # stage 3 (page select) from the oracle's scores
    v.score.copy_(torch.from_numpy(o["score"]).to(dev))
    hsa.stage_select_pages(dims, seq, keep, mk, tk, ws)
    torch.cuda.synchronize()
    assert np.array_equal(v.pages.cpu().numpy(), o["pages"]) and np.array_equal(v.n_pages.cpu().numpy(), o["n_pages"])
    # stage 4 (key select) from the oracle's page lists and query codes
    v.pages.copy_(torch.from_numpy(o["pages"]).to(dev))
    v.n_pages.copy_(torch.from_numpy(o["n_pages"]).to(dev))
    v.code_q.copy_(torch.from_numpy(o["code_q"].view(np.int64)).to(dev))
    v.ham.fill_(0x1234)
    hsa.stage_hamming(dims, codes_gpu, seq, mk, tk, ws)
    torch.cuda.synchronize()
    assert np.array_equal(v.ham.cpu().numpy().view(np.uint16), o["ham"])
    v.ham.fill_(0x1234)
    sel = torch.empty((2, wl.n_kv_heads, tk), dtype=torch.int32, device=dev)
    hsa.stage_select_keys(dims, codes_gpu, seq, mk, tk, ws, sel_idx=sel)
    torch.cuda.synchronize()
    assert np.array_equal(v.ham.cpu().numpy().view(np.uint16), o["ham"])
    assert np.array_equal(sel.cpu().numpy(), o["sel"]) and np.array_equal(v.k_eff.cpu().numpy(), o["k_eff"])
    # stage 5 (attention) from the oracle's selection
    osel = torch.from_numpy(o["sel"]).to(dev)
    v.k_eff.copy_(torch.from_numpy(o["k_eff"]).to(dev))
    out = torch.empty((2, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    hsa.stage_attend(dims, t["Q"], t["K"], t["V"], seq, mk, tk, out, ws, sel_idx=osel)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy().astype(np.float64) - o["out"]).max() <= 2e-3


# The Hamming stage alone, after a full step on the same workspace: the distances of every candidate slot
# equal the oracle's, forced (sink and window) slots and slots past the kept pages or the sequence included.
HAM_SHAPES = [
    ("tiny_ragged", WORKLOADS["tiny"].with_(batch=2, ragged=(1000, 4096))),
    ("sinks_window_b64", Workload("hs1", 210, 2, 8, 2, 128, 3000, 16, 64, 20, 200, "bf16", ragged=(100, 3000),
                                  sink_tokens=4, local_window=40)),
    ("mean_code_g7", Workload("hs2", 211, 1, 14, 2, 128, 2000, 16, 128, 10, 150, "bf16", hamming_group=1)),
    ("p32_b64_fp32", Workload("hs3", 212, 2, 8, 2, 64, 4096, 32, 64, 15, 256, "fp32", ragged=(2000, 4096))),
]


@pytest.mark.parametrize("name,wl", HAM_SHAPES, ids=[s[0] for s in HAM_SHAPES])
def test_hamming_stage_alone(dev, name, wl):
    import torch

    import hash_sparse_attention_amd as hsa
    banner(f"Hamming stage {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    x = g["_dev"]
    v = hsa.workspace_view(x["dims"], x["max_keep"], x["top_k"], x["ws"])
    assert np.array_equal(g["ham"], o["ham"])
    v.ham.fill_(0x1234)
    hsa.stage_hamming(x["dims"], x["codes"], x["seq"], x["max_keep"], x["top_k"], x["ws"])
    torch.cuda.synchronize()
    assert np.array_equal(v.ham.cpu().numpy().view(np.uint16), o["ham"])


@pytest.mark.parametrize("npages,seq,keep,max_keep", [
    (8192, (8192 * 16, 3001 * 16 - 7, 0), (700, 250, 5), 1024),       # fast select, 8 pages a thread
    (4096, (4096 * 16, 2900 * 16, 17 * 16), (900, 300, 40), 1024),    # fast select, 4 pages a thread
    (20000, (20000 * 16, 9000 * 16, 100), (700, 2500, 3), 4096),      # general select (chunked)
    (12000, (12000 * 16, 11000 * 16, 1), (8500, 4000, 1), 9000),      # general select (list past LDS)
])
def test_page_select_stage_on_tied_scores(dev, npages, seq, keep, max_keep):
    """The page-select stage on given fp64 scores with hard ties straddling the keep boundary (clusters
    that tie only after rounding to fp32, more and fewer than 64 of them; exact duplicates; signed zeros
    and denormals; all scores equal) equals the oracle's page-select step bit for bit."""
    import torch

    import hash_sparse_attention_amd as hsa
    import oracle
    from gpu_common import gpu_dims, oracle_dims, to_dev
    from synth import tie_scores
    wl = Workload("ties", 95, 3, 8, 2, 64, npages * 16, 16, 64, 25, 256, "fp32")
    banner(f"page select on tied scores: {npages} pages, keep {keep}, max_keep {max_keep}")
    seq = np.asarray(seq, np.int32)
    keep = np.asarray(keep, np.int32)
    NP = [-(-int(L) // 16) for L in seq]
    S = tie_scores(int(npages) + int(max_keep), 3, 2, wl.max_pages, NP, keep)
    dims = gpu_dims(wl)
    ws = hsa.alloc_workspace(dims, max_keep, wl.top_k, dev)
    ws.fill_(0x5C)
    v = hsa.workspace_view(dims, max_keep, wl.top_k, ws)
    v.score.copy_(torch.from_numpy(S).to(dev))
    hsa.stage_select_pages(dims, to_dev(seq, dev), to_dev(keep, dev), max_keep, wl.top_k, ws)
    torch.cuda.synchronize()
    want_pages, want_n = oracle.select_pages(oracle_dims(wl), S, seq, keep, max_keep)
    assert np.array_equal(v.n_pages.cpu().numpy(), want_n)
    assert np.array_equal(v.pages.cpu().numpy(), want_pages)


def test_fidelity_harness_matches_oracle_selection(dev):
    """The retrieval-fidelity harness, run through the library, reports the same key recall, page coverage,
    attention mass and planted recall as on the oracle's selections (the selections are equal)."""
    from fidelity import metrics, run_library
    wl = WORKLOADS["tiny"].with_(batch=2, ragged=(2000, 4096))
    banner("fidelity harness")
    d = make_layer(wl)
    out, sel, pages, n_pages = run_library(wl, d, dev)
    g = metrics(wl, d, sel, out, pages, n_pages)
    o = run_oracle(wl, d)
    m = metrics(wl, d, o["sel"], o["out"], o["pages"], o["n_pages"])
    for k in ("key_recall", "page_coverage", "attention_mass", "planted_recall"):
        assert g[k] == m[k], k
    assert abs(g["out_max_err"] - m["out_max_err"]) <= 2e-3


def test_hamming_logit_table_matches_oracle_codes(dev):
    """The Hamming-versus-logit table from the library's key and query codes equals the one from the
    oracle's codes (the codes are bit-exact), with W_h = R_h as in the pages' random-orthogonal setup."""
    from fidelity import hamming_logit, run_library
    wl = WORKLOADS["tiny"].with_(hash_bits=64)
    banner("hamming vs logit table")
    d = make_layer(wl)
    d["W"] = d["R"].copy()
    *_, cd, cq = run_library(wl, d, dev, want_codes=True)
    o = run_oracle(wl, d)
    for h in range(wl.n_kv_heads):
        g = hamming_logit(wl, d, cd, cq, h=h)
        m = hamming_logit(wl, d, o["codes"], o["code_q"], h=h)
        assert np.array_equal(np.array(g["rows"], float), np.array(m["rows"], float), equal_nan=True)  # empty bins: NaN
        assert g["spearman"] == m["spearman"] and g["top1_overlap"] == m["top1_overlap"]


FORCED = [
    # sink tokens / local window (keys always attended; the rest ranked by the Hamming stage)
    ("tiny_s4_w64", WORKLOADS["tiny"].with_(sink_tokens=4, local_window=64)),
    ("bf16_b3_ragged_s1", Workload("fk1", 150, 3, 8, 2, 128, 5000, 16, 128, 10, 300, "bf16", outliers=2,
                                   ragged=(1, 5000), sink_tokens=1)),
    ("g7_w17", Workload("fk2", 151, 2, 14, 2, 128, 2000, 16, 128, 10, 150, "bf16", outliers=2, ragged=(1, 2000),
                        local_window=17)),
    ("p1_s7_w300", Workload("fk3", 152, 2, 2, 2, 64, 700, 1, 128, 20, 17, "fp32", ragged=(50, 700),
                            sink_tokens=7, local_window=300)),
    ("window_covers_all", Workload("fk4", 153, 2, 8, 2, 64, 1024, 16, 64, 25, 3, "fp32", ragged=(10, 1024),
                                   sink_tokens=5, local_window=1024)),
    ("llama8b_32k_s4_w64", WORKLOADS["llama8b_32k"].with_(sink_tokens=4, local_window=64)),
]


@pytest.mark.parametrize("name,wl", FORCED, ids=[f[0] for f in FORCED])
def test_sinks_and_local_window_parity(dev, name, wl):
    banner(f"forced keys {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


GROUPED = [
    # group aggregation variants: min page score over the GQA group, Hamming to the mean query's code
    ("tiny_min", WORKLOADS["tiny"].with_(page_group=1)),
    ("tiny_mean", WORKLOADS["tiny"].with_(hamming_group=1)),
    ("g7_min_mean_ragged", Workload("gv1", 160, 3, 14, 2, 128, 2000, 16, 128, 10, 150, "bf16", outliers=2,
                                    ragged=(1, 2000), page_group=1, hamming_group=1)),
    ("g8_mean_d64_p64", Workload("gv2", 161, 1, 16, 2, 64, 3000, 64, 64, 30, 400, "bf16", hamming_group=1)),
    ("g3_mean_fp32_sinks", Workload("gv3", 162, 2, 6, 2, 128, 777, 32, 128, 40, 64, "fp32", ragged=(700, 777),
                                    hamming_group=1, sink_tokens=4, local_window=16)),
    ("llama8b_32k_mean", WORKLOADS["llama8b_32k"].with_(hamming_group=1)),
]


@pytest.mark.parametrize("name,wl", GROUPED, ids=[g[0] for g in GROUPED])
def test_group_aggregation_variants_parity(dev, name, wl):
    banner(f"group variant {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)



@pytest.mark.parametrize("name,wl", [
    ("lhp_only_40k", Workload("lhp1", 170, 1, 8, 2, 128, 40000, 16, 128, 100, 2048, "bf16", outliers=2)),
    ("lhp_only_ragged_b2", Workload("lhp2", 171, 2, 8, 2, 64, 70000, 16, 64, 100, 900, "bf16",
                                    ragged=(30000, 70000))),
], ids=["lhp_only_40k", "lhp_only_ragged_b2"])
def test_lhp_only_many_candidates(dev, name, wl):
    """LHP-only (every page kept, so the Hamming stage ranks every key): more candidate slots than one
    select chunk, spread over up to 64 split blocks per head."""
    banner(f"LHP-only {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


PER_HEAD = [
    # one selection per query head (the group does not share)
    ("tiny_per_head", WORKLOADS["tiny"].with_(per_head=True)),
    ("g7_per_head_ragged", Workload("ph1", 180, 3, 14, 2, 128, 2000, 16, 128, 10, 150, "bf16", outliers=2,
                                    ragged=(1, 2000), per_head=True)),
    ("g8_per_head_bf16meta_sinks", Workload("ph2", 181, 2, 16, 2, 64, 3000, 64, 64, 30, 400, "bf16",
                                            meta_bf16=True, sink_tokens=2, local_window=33, per_head=True)),
    ("g4_per_head_mean_min_fp32", Workload("ph3", 182, 2, 8, 2, 64, 1500, 8, 128, 15, 90, "fp32",
                                           ragged=(700, 1500), per_head=True, page_group=1, hamming_group=1)),
    ("llama8b_32k_per_head", WORKLOADS["llama8b_32k"].with_(per_head=True)),
    # one bound pass per KV head writes its query heads' bounds: more group sizes of that pass
    ("g2_per_head_p4_ragged", Workload("ph4", 183, 2, 4, 2, 128, 1200, 4, 128, 20, 80, "bf16", ragged=(600, 1200),
                                       per_head=True)),
    ("g3_per_head_d64_fp32", Workload("ph5", 184, 1, 6, 2, 64, 2000, 16, 64, 10, 100, "fp32", per_head=True)),
]


@pytest.mark.parametrize("name,wl", PER_HEAD, ids=[p[0] for p in PER_HEAD])
def test_per_query_head_selection_parity(dev, name, wl):
    banner(f"per-head selection {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


# Paths the shapes above do not reach (each is named by the kernel path it takes at these sizes).
PATH_SHAPES = [
    # D = 128 with G = 8: the largest attention tiles (8 query heads x 128 dims per row) on the split select.
    ("d128_g8_split_64q8kv", Workload("g8s", 180, 1, 64, 8, 128, 8192, 16, 128, 25, 512, "bf16", outliers=2)),
    ("d128_g8_split_16q2kv", Workload("g8t", 181, 1, 16, 2, 128, 8192, 16, 128, 25, 1024, "bf16", outliers=2)),
    ("d128_g8_lhp_only", Workload("g8l", 182, 1, 16, 2, 128, 8192, 16, 128, 100, 700, "fp32", outliers=2)),
    # More than 16384 pages per sequence (page size 4 at 80K): the general page select, split key select.
    ("p4_80k_20000_pages", Workload("p4l", 183, 1, 8, 2, 128, 80000, 4, 128, 5, 2048, "bf16", outliers=2)),
    # More than 8192 kept pages: the page list stays in the workspace, one key-select block per head.
    # Sequence 0 keeps 7500 pages (its list fits in LDS), sequence 1 all 9216 (it does not).
    ("keep_9216_pages", Workload("k9k", 184, 2, 8, 2, 64, 36864, 4, 64, 100, 3000, "bf16")),
    # Many heads with split key selects: 16 x 8 heads keep up to 512 pages (8192 slots), so each head needs 4
    # compaction blocks and the 512 split blocks exceed one and a half rounds of the CUs: the page select runs
    # once per head in its own launch and the split blocks read its list.
    ("many_heads_pages_apart", Workload("mhp", 185, 16, 32, 8, 64, 16384, 16, 64, 50, 1024, "bf16", outliers=2,
                                        ragged=(12000, 16384))),
]
PATH_LENGTHS = {"keep_9216_pages": [30000, 36864]}

# bf16 K/V on the split path scores on the matrix cores: the query rows of the score tile are the group's
# heads, so the group sizes the shapes above leave out are covered here (one head per selection with Hq = Hkv;
# a second row of four heads that is partly empty at G = 5, 6, 7), with ragged lengths, and with sink tokens
# and a local window listed after the ranked keys of the first split.
MFMA_SHAPES = [
    ("bf16_split_d128_g1_mha", Workload("mf1", 200, 1, 4, 4, 128, 8192, 16, 128, 25, 512, "bf16", outliers=2)),
    ("bf16_split_d128_g2_ragged", Workload("mf2", 201, 2, 4, 2, 128, 6000, 16, 128, 20, 400, "bf16",
                                          ragged=(3000, 6000))),
    ("bf16_split_d64_g3", Workload("mf3", 202, 1, 6, 2, 64, 8192, 16, 64, 25, 600, "bf16")),
    ("bf16_split_d128_g5", Workload("mf5", 203, 1, 10, 2, 128, 8192, 16, 128, 25, 700, "bf16", outliers=2)),
    ("bf16_split_d64_g6_ragged", Workload("mf6", 204, 2, 12, 2, 64, 4096, 8, 64, 30, 300, "bf16",
                                         ragged=(1000, 4096))),
    ("bf16_split_d128_g6", Workload("mf7", 205, 1, 12, 2, 128, 8192, 16, 128, 25, 512, "bf16")),
    ("bf16_split_d64_g7", Workload("mf8", 206, 1, 14, 2, 64, 8192, 32, 64, 25, 800, "bf16", outliers=2)),
    ("bf16_split_d128_g2_sinks_window", Workload("mf9", 207, 2, 4, 2, 128, 8192, 16, 128, 25, 500, "bf16",
                                                ragged=(5000, 8192), sink_tokens=4, local_window=64)),
]


@pytest.mark.parametrize("name,wl", MFMA_SHAPES, ids=[s[0] for s in MFMA_SHAPES])
def test_bf16_split_group_sizes(dev, name, wl):
    banner(f"decode parity {name}: G {wl.n_q_heads // wl.n_kv_heads}, max_keep {wl.max_keep}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


@pytest.mark.parametrize("name,wl", PATH_SHAPES, ids=[s[0] for s in PATH_SHAPES])
def test_decode_parity_paths(dev, name, wl):
    import hash_sparse_attention_amd as hsa
    from gpu_common import gpu_dims
    lay = hsa.workspace_layout(gpu_dims(wl), wl.max_keep, wl.top_k)
    banner(f"decode parity {name}: max_keep {wl.max_keep}, {lay.total} workspace bytes")
    d = make_layer(wl, lengths=PATH_LENGTHS.get(name))
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


# Sign-split page metadata: encode and append write it, the bound kernel reads one side per dimension when a
# KV head has one query head (G = 1), and both sides for grouped heads, per-query-head selection included
# (one pass per KV head).
SPLIT_SHAPES = [
    ("mha_g1_bf16", Workload("ms1", 190, 2, 4, 4, 128, 3000, 16, 128, 10, 200, "bf16", outliers=2,
                             ragged=(1000, 3000), meta_split=True)),
    ("mha_g1_d64_bf16meta_fp32", Workload("ms2", 191, 1, 2, 2, 64, 5000, 8, 64, 15, 300, "fp32", meta_split=True,
                                          meta_bf16=True)),
    ("per_head_g4", Workload("ms3", 192, 1, 16, 4, 128, 4096, 16, 128, 10, 256, "bf16", outliers=2, per_head=True,
                             meta_split=True)),
    ("shared_g4_both_sides", Workload("ms4", 193, 1, 8, 2, 128, 4096, 16, 128, 25, 512, "bf16", outliers=2,
                                      meta_split=True)),
    ("shared_g7_bf16meta_min_page", Workload("ms5", 194, 1, 14, 2, 128, 2000, 16, 128, 10, 150, "bf16",
                                             meta_split=True, meta_bf16=True, page_group=1)),
    ("mha_g1_p1_sinks", Workload("ms6", 195, 2, 3, 3, 64, 700, 1, 64, 20, 50, "bf16", ragged=(1, 700),
                                 meta_split=True, sink_tokens=2, local_window=9)),
    ("per_head_g8_d64_bf16meta", Workload("ms7", 197, 2, 16, 2, 64, 2500, 32, 64, 20, 120, "fp32",
                                          ragged=(900, 2500), per_head=True, meta_split=True, meta_bf16=True)),
    ("per_head_g2_ragged", Workload("ms8", 198, 3, 4, 2, 128, 1800, 8, 128, 15, 100, "bf16", ragged=(1, 1800),
                                    per_head=True, meta_split=True)),
]


@pytest.mark.parametrize("name,wl", SPLIT_SHAPES, ids=[s[0] for s in SPLIT_SHAPES])
def test_sign_split_metadata_parity(dev, name, wl):
    banner(f"sign-split metadata {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


def test_sign_split_encode_in_chunks(dev):
    """Bulk encode, 1-token appends and a mid-page chunk into the sign-split layout: bit-identical to the oracle's
    single-shot encode, and the decode on it equal to the oracle's."""
    wl = Workload("ms_chunks", 196, 2, 8, 8, 128, 1200, 16, 128, 20, 64, "bf16", outliers=2, meta_split=True)
    banner("sign-split encode in chunks")
    d = make_layer(wl, lengths=[1100, 1037])
    chunks = [(np.zeros(2, np.int32), np.array([900, 837], np.int32), 900)]
    pos = np.array([900, 837], np.int32)
    for _ in range(3):
        chunks.append((pos.copy(), np.ones(2, np.int32), 1))
        pos += 1
    chunks.append((pos.copy(), np.array([197, 197], np.int32), 197))
    pos += 197
    assert list(pos) == [1100, 1037]
    g = run_gpu(wl, d, dev, chunks=chunks)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label="sign-split chunks")


BULK_CHUNK_SHAPES = [
    # name, workload (B=2, G=2); every page-size branch of the tiled encode's page reduction
    ("p1_d64_b128_bf16", Workload("bc1", 201, 2, 4, 2, 64, 1000, 1, 128, 20, 64, "bf16")),
    ("p2_d128_b64_fp32_m16", Workload("bc2", 202, 2, 4, 2, 128, 1000, 2, 64, 20, 64, "fp32", meta_bf16=True)),
    ("p4_d128_b128_fp32_split", Workload("bc4", 203, 2, 4, 2, 128, 1000, 4, 128, 20, 64, "fp32", meta_split=True)),
    ("p8_d64_b64_bf16", Workload("bc8", 204, 2, 4, 2, 64, 1000, 8, 64, 20, 64, "bf16", outliers=2)),
    ("p32_d128_b64_bf16_m16_split", Workload("bc32", 205, 2, 4, 2, 128, 1000, 32, 64, 20, 64, "bf16",
                                             meta_bf16=True, meta_split=True)),
    ("p64_d64_b128_fp32", Workload("bc64", 206, 2, 4, 2, 64, 1000, 64, 128, 30, 64, "fp32")),
]


@pytest.mark.parametrize("name,wl", BULK_CHUNK_SHAPES, ids=[s[0] for s in BULK_CHUNK_SHAPES])
def test_bulk_encode_mid_page_chunks(dev, name, wl):
    """Bulk encodes (more than 64 keys, the tiled kernel) that start mid-page and mid-tile, with ragged and zero
    counts and max_count above every count: codes and page bounds bit-identical to the oracle's single-shot encode,
    and the decode on them equal to the oracle's."""
    banner(f"bulk encode mid-page chunks {name}")
    d = make_layer(wl, lengths=[977, 941])
    chunks = [(np.zeros(2, np.int32), np.array([301, 299], np.int32), 301),      # ends mid-page, mid-tile
              (np.array([301, 299], np.int32), np.array([130, 0], np.int32), 200),  # sequence 1 appends nothing
              (np.array([431, 299], np.int32), np.array([67, 197], np.int32), 250),
              (np.array([498, 496], np.int32), np.array([479, 445], np.int32), 479)]
    assert [int(s + c) for s, c in zip(chunks[-1][0], chunks[-1][1])] == [977, 941]
    g = run_gpu(wl, d, dev, chunks=chunks)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)
