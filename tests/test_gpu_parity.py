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
]


@pytest.mark.parametrize("name,wl", SHAPES, ids=[s[0] for s in SHAPES])
def test_decode_parity_shapes(dev, name, wl):
    wl = WORKLOADS["tiny"] if wl is None else wl
    banner(f"decode parity {name}")
    d = make_layer(wl)
    g = run_gpu(wl, d, dev)
    o = run_oracle(wl, d)
    compare(wl, d["seq_len"], g, o, label=name)


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
