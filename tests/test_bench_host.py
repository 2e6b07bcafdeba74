"""Host-side logic of bench.py, on the CPU: the byte model behind the roofline
figures, the rule that counter-derived traffic is reported only for the kernel
source it was measured on, the committed counter summaries against that model,
and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports no GPU code at module level)
from synth.workloads import WORKLOADS  # noqa: E402


def test_page_bound_bytes_per_launch():
    """One page costs its 2*D stored bounds (4 or 2 bytes each) plus its fp64 score."""
    wl = WORKLOADS["llama8b_128k"]
    seq = [wl.ctx] * wl.batch
    b, pages = bench.page_bound_bytes_per_launch(wl, seq)
    assert pages == 8 * (131072 // 16)
    assert b == pages * (2 * 128 * 4 + 8) == 67_633_152
    b16, pages16 = bench.page_bound_bytes_per_launch(wl.with_(meta_bf16=True), seq)
    assert pages16 == pages and b16 == pages * (2 * 128 * 2 + 8)
    # One selection per query head streams its KV head's metadata once per query head.
    bph, pph = bench.page_bound_bytes_per_launch(wl.with_(per_head=True), seq)
    assert pph == 4 * pages and bph == 4 * b


def test_page_count_rounds_partial_pages_up():
    wl = WORKLOADS["mistral7b_b8"]  # page 32, 8 KV heads
    _, pages = bench.page_bound_bytes_per_launch(wl, [1, 32, 33, 64])
    assert pages == 8 * (1 + 1 + 2 + 2)


def test_bf16_metadata_saves_exactly_half_the_bound_reads():
    wl = WORKLOADS["llama8b_128k"]
    seq, keep = [wl.ctx], [wl.max_keep]
    full = bench.algorithmic_bytes_per_layer(wl, seq, keep, 4096 * 8)
    half = bench.algorithmic_bytes_per_layer(wl.with_(meta_bf16=True), seq, keep, 4096 * 8)
    n_pages = wl.ctx // wl.page_size
    # The whole stream's bounds (8 heads) plus the appended page's bounds.
    assert full - half == 8 * n_pages * 2 * 128 * 2 + 8 * 2 * 128 * 2


def test_counter_traffic_only_for_the_profiled_source(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel, first version\n")
    rec = tmp_path / "pmc.json"
    rec.write_text(json.dumps({"source_sha256_16": bench.source_digest(str(src)), "bytes_per_launch": 1234.5}))
    assert bench.pmc_traffic(str(rec), str(src)) == 1234.5
    src.write_text("// kernel, edited\n")
    assert bench.pmc_traffic(str(rec), str(src)) is None
    assert bench.pmc_traffic(str(tmp_path / "absent.json"), str(src)) is None
    rec.write_text("not json")
    assert bench.pmc_traffic(str(rec), str(src)) is None


@pytest.mark.parametrize("path", [bench.PMC_FILE, bench.TOPK_PMC_FILE])
def test_committed_counter_summaries_against_the_byte_model(path):
    """Each committed summary states the algorithmic bytes of the launch it
    measured (the same model bench.py uses) and HBM traffic within 15% above it."""
    rec = json.load(open(path))
    wl = WORKLOADS["llama8b_128k"]
    if "page_bound" in rec["kernel"]:
        alg, _ = bench.page_bound_bytes_per_launch(wl, [wl.ctx])
    else:  # one fp64 logit written per key of K (bf16 keys)
        keys = wl.n_kv_heads * wl.ctx
        alg = keys * (wl.head_dim * 2 + 8)
    assert rec["algorithmic_bytes_per_launch"] == alg
    assert rec["fetch_bytes"] + rec["write_bytes"] == pytest.approx(rec["bytes_per_launch"])
    assert 1.0 <= rec["bytes_per_launch"] / alg < 1.15
    assert len(rec["source_sha256_16"]) == 16 and rec["command"]


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120, env={**os.environ, **env})
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_encode_append_work_model():
    """The 4096-token append to 16 sequences x 4 KV heads at 128K (head_dim 128, 128-bit codes, page 16, bf16 K,
    fp32 bounds): 262,144 keys, each (128 + 128) chains of 128 FMAs; K read, 16-byte codes and the 16,384 touched
    pages' bounds written, R_h and W_h read once."""
    import numpy as np
    wl = WORKLOADS["qwen7b_b16"]
    seq = np.full(wl.batch, wl.ctx)
    m = bench.encode_model(wl, seq - wl.append_tokens, seq)
    assert m["keys"] == 16 * 4 * 4096 == 262_144
    assert m["flops"] == 262_144 * 256 * 128 * 2 == 17_179_869_184
    assert m["pages"] == 16 * 4 * (4096 // 16)
    assert m["k_read"] == 262_144 * 128 * 2 and m["codes_written"] == 262_144 * 16
    assert m["meta_written"] == 16_384 * 2 * 128 * 4
    assert m["hbm_bytes"] == 67_108_864 + 4_194_304 + 16_777_216 + 4 * 256 * 128 * 4


def test_encode_model_counts_partial_pages_once():
    """A chunk that starts and ends inside pages touches every page it overlaps once; an empty chunk nothing."""
    wl = WORKLOADS["tiny"]  # page 16, 2 KV heads
    m = bench.encode_model(wl, [5, 7], [40, 7])
    assert m["keys"] == 35 * 2
    assert m["pages"] == 3 * 2  # pages 0, 1, 2 of the first sequence


def test_sign_split_halves_the_bound_bytes_of_one_query_head_selections():
    """With sign-split metadata a selection of one query head reads one stored side per dimension."""
    seq = [131072]
    mha = WORKLOADS["mha_128k"]
    full, pages = bench.page_bound_bytes_per_launch(mha, seq)
    half, pages2 = bench.page_bound_bytes_per_launch(mha.with_(meta_split=True), seq)
    assert pages == pages2 == 8 * 8192
    assert full == pages * (2 * 128 * 4 + 8) and half == pages * (128 * 4 + 8)
    # Grouped selections read both sides whatever the layout; per-query-head ones read one.
    llama = WORKLOADS["llama8b_128k"]
    assert bench.meta_sides(llama.with_(meta_split=True)) == 2
    assert bench.meta_sides(llama.with_(meta_split=True, per_head=True)) == 1
    assert bench.meta_sides(llama.with_(per_head=True)) == 2


def test_step_spread_and_description():
    med, p10, p90 = bench.spread([5.0, 1.0, 3.0, 2.0, 4.0])
    assert med == 3.0 and abs(p10 - 1.4) < 1e-12 and abs(p90 - 4.6) < 1e-12
    d = bench.describe(WORKLOADS["qwen7b_b16"].with_(meta_split=True))
    assert d.startswith("qwen7b_b16: Qwen2.5-7B-shaped") and "sign-split" in d


def test_counter_traffic_only_for_the_profiled_workload():
    """The committed bound-kernel counters describe llama8b_128k with fp32 interleaved metadata and shared
    selections, measured on the current decode.hip; any other workload reports no traffic."""
    wl = WORKLOADS["llama8b_128k"]
    rec = json.load(open(bench.PMC_FILE))
    assert rec["source_sha256_16"] == bench.source_digest(), "page-bound counters predate the current decode.hip"
    assert bench.traffic_from_profile(wl) == rec["bytes_per_launch"]
    assert 1.0 <= rec["bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] < 1.05
    for other in (wl.with_(meta_bf16=True), wl.with_(meta_split=True), wl.with_(per_head=True),
                  WORKLOADS["qwen7b_b16"]):
        assert bench.traffic_from_profile(other) is None


def _line():
    return {"metric": "m", "value": 2.0e10, "unit": "keys/s", "n_gpus": 1, "steps": 100, "warmup": 10,
            "ms_per_step": 1.6, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", "config": {"workload": "w"},
            "roofline": {"bound": "hbm", "achieved": 5000.0, "peak": 8000.0, "unit": "GB/s", "frac": 0.625,
                         "traffic": None},
            "cpu_baseline": {"value": 1.4e8, "unit": "keys/s", "cores": 8, "kind": "oracle", "sample": "s"}}


def test_result_line_contract_is_checked():
    """Every mode checks its line before printing: a complete line passes; a missing field, an incomplete
    roofline or CPU baseline, a non-finite value or an inconsistent fraction is refused."""
    bench.check_line(_line())
    bench.check_line(dict(_line(), cpu_baseline=None))
    for bad in (
        {k: v for k, v in _line().items() if k != "roofline"},
        dict(_line(), config={"model": "x"}),
        dict(_line(), roofline={k: v for k, v in _line()["roofline"].items() if k != "traffic"}),
        dict(_line(), roofline=dict(_line()["roofline"], bound="dram")),
        dict(_line(), roofline=dict(_line()["roofline"], frac=0.5)),
        dict(_line(), cpu_baseline={"value": 1.0, "unit": "keys/s"}),
        dict(_line(), value=float("nan")),
    ):
        with pytest.raises(ValueError):
            bench.check_line(bad)
