"""Shape fuzzing of the oracle's invariants (CPU only).

Hypothesis draws small decode shapes -- group size, head dim, page size,
code width, context, ragged lengths, keep fraction, top_k, K/V precision --
and every drawn shape must satisfy what the pages and the mathematics fix,
each checked against an independent statement rather than the oracle's own
code:
  - the page score bounds every rotated logit of the page's keys for every
    head of the group (the GKR bound is an upper bound: "HHR: Hierarchical
    Hash Retrieval for Efficient LLM Generation", Abstract);
  - the kept pages are the first `keep` of numpy's lexsort by (-score, page);
  - each candidate's distance is a brute-force popcount of the code XORs,
    summed over the group (rit.work HHR blog post, section "Почему
    расстояние Хэмминга пропускает важные ключи");
  - the selected keys are the first top_k of numpy's lexsort by (H, t);
  - the output is textbook fp64 softmax attention over the selected keys.
The draws are derandomized, so the suite is reproducible.
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from synth import Workload, make_layer  # noqa: E402
from test_oracle_pins import _softmax_attention, dims_for, f32  # noqa: E402


@st.composite
def shapes(draw):
    G = draw(st.sampled_from([1, 2, 3, 4, 7, 8]))
    H = draw(st.sampled_from([1, 2]))
    D = draw(st.sampled_from([16, 32, 64, 128]))
    P = draw(st.sampled_from([1, 2, 4, 8, 16, 32]))
    nb = draw(st.sampled_from([64, 128]))
    T = draw(st.integers(1, 300))
    B = draw(st.integers(1, 2))
    lo = draw(st.integers(0, T))
    keep = draw(st.integers(1, 100))
    top_k = draw(st.integers(1, 200))
    dtype = draw(st.sampled_from(["fp32", "bf16"]))
    seed = draw(st.integers(0, 10_000))
    return Workload("fuzz", 300 + seed, B, G * H, H, D, T, P, nb, keep, top_k, dtype, ragged=(lo, T))


def _popcount(x):
    return np.array([bin(int(v)).count("1") for v in np.asarray(x, np.uint64).ravel()]).reshape(np.shape(x))


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])
@given(wl=shapes())
def test_oracle_invariants_on_random_shapes(oracle_mod, wl):
    o = oracle_mod
    d = make_layer(wl)
    dims = dims_for(o, wl)
    seq = d["seq_len"]
    meta, codes = o.encode(dims, d["K"], d["R"], d["W"], np.zeros(wl.batch, np.int32), seq)
    r = o.decode(dims, d["Q"], d["K"], d["V"], d["R"], d["W"], meta, codes, seq, d["keep"], wl.max_keep, wl.top_k)
    G, P, NW = wl.group, wl.page_size, wl.hash_bits // 64
    Qf, Kf, Vf = f32(d["Q"], wl), f32(d["K"], wl), f32(d["V"], wl)
    for b in range(wl.batch):
        L = int(seq[b])
        NP = -(-L // P)
        for h in range(wl.n_kv_heads):
            # page bound >= every rotated logit of the page (exact up to fp64 rounding of the bound's sum)
            if L:
                kr, _ = o.project(d["R"][h], d["W"][h], Kf[b, h, :L])
                qr = r["q_rot"][b, h * G:(h + 1) * G].astype(np.float64)
                lt = qr @ kr.astype(np.float64).T
                mag = np.abs(qr) @ np.abs(kr.astype(np.float64)).T
                for p in range(NP):
                    sl = slice(p * P, min((p + 1) * P, L))
                    assert r["score"][b, h, p] >= lt[:, sl].max() - 1e-12 * mag[:, sl].max()
            # kept pages = lexsort by (-score, page)
            keep = int(min(max(int(d["keep"][b]), 1), NP, wl.max_keep)) if NP else 0
            S = r["score"][b, h, :NP]
            want_pages = np.sort(np.lexsort((np.arange(NP), -S))[:keep])
            n = int(r["n_pages"][b, h])
            assert n == keep
            assert np.array_equal(r["pages"][b, h, :n], want_pages)
            assert (r["pages"][b, h, n:] == -1).all()
            # distances = brute-force popcounts over the group's query codes
            t = (want_pages[:, None] * P + np.arange(P)[None, :]).ravel()
            ok = t < L
            cq = r["code_q"][b * wl.n_q_heads + h * G: b * wl.n_q_heads + (h + 1) * G].reshape(G, NW) \
                if r["code_q"].ndim == 2 else r["code_q"][b, h * G:(h + 1) * G].reshape(G, NW)
            kc = codes[b, h, t[ok]].reshape(-1, NW) if ok.any() else np.zeros((0, NW), np.uint64)
            Hw = sum(_popcount(np.bitwise_xor(kc, cq[i][None, :])).sum(1) for i in range(G)) if ok.any() else []
            ham = r["ham"][b, h, :n * P]
            assert np.array_equal(ham[ok].astype(np.int64), np.asarray(Hw, np.int64))
            assert (ham[~ok] == 0xFFFF).all()
            # selection = first top_k of lexsort by (H, t), ascending, -1 padded
            tc, Hc = t[ok], np.asarray(Hw, np.int64)
            keff = min(wl.top_k, len(tc))
            want_sel = np.sort(tc[np.lexsort((tc, Hc))[:keff]]) if keff else np.zeros(0, np.int64)
            assert int(r["k_eff"][b, h]) == keff
            assert np.array_equal(r["sel"][b, h, :keff], want_sel)
            assert (r["sel"][b, h, keff:] == -1).all()
            # attention = textbook softmax attention over the selection
            for i in range(h * G, (h + 1) * G):
                if keff:
                    ref = _softmax_attention(Qf[b, i].astype(np.float64), Kf[b, h, want_sel].astype(np.float64),
                                             Vf[b, h, want_sel].astype(np.float64), 1 / np.sqrt(wl.head_dim))
                    assert np.abs(r["out"][b, i] - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max())
