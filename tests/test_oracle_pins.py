"""Pins of the CPU oracle against what the HHR pages and the mathematics fix.

None of these checks retypes the oracle's code: each compares it with an
independent statement -- a hand-worked example (tests/golden), a closed form,
an invariant the pages state, a brute-force count, or a special case that
reduces to a textbook routine (numpy lexsort, numpy softmax attention).
Sources: "HHR: Hierarchical Hash Retrieval for Efficient LLM Generation",
Abstract; rit.work HHR blog post, sections "Почему расстояние Хэмминга
пропускает важные ключи" and "Два уровня маршрутизации решают разные
ошибки"; thelatestinai.com page, Figure 3 caption and Appendix Table 4.
"""
import json
import os

import numpy as np
import pytest

from synth import WORKLOADS, Workload, bf16_bits_to_f32, f32_to_bf16_bits, make_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U24 = 2.0 ** -24


def gamma(n):
    return n * U24 / (1 - n * U24)


def bits_of(codes):
    """[..., W] uint64 -> [..., 64W] bool, bit j = bit j%64 of word j//64."""
    c = np.asarray(codes, np.uint64)
    j = np.arange(64, dtype=np.uint64)
    b = ((c[..., None] >> j) & np.uint64(1)).astype(bool)
    return b.reshape(*c.shape[:-1], c.shape[-1] * 64)


def dims_for(o, wl: Workload):
    return o.Dims(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.page_size, wl.hash_bits,
                  wl.ctx, wl.dtype == "bf16", wl.meta_bf16, wl.sink_tokens, wl.local_window, wl.page_group,
                  wl.hamming_group, wl.per_head)


def f32(x, wl):
    return bf16_bits_to_f32(x) if wl.dtype == "bf16" else np.asarray(x, np.float32)


def run(o, wl, data, max_keep=None, top_k=None, keep=None, seq=None, scale=0.0):
    dims = dims_for(o, wl)
    seq = data["seq_len"] if seq is None else np.asarray(seq, np.int32)
    meta, codes = o.encode(dims, data["K"], data["R"], data["W"], np.zeros(wl.batch, np.int32), seq)
    mk = wl.max_keep if max_keep is None else max_keep
    r = o.decode(dims, data["Q"], data["K"], data["V"], data["R"], data["W"], meta, codes, seq,
                 data["keep"] if keep is None else keep, mk, wl.top_k if top_k is None else top_k, scale)
    return dims, meta, codes, r


SMALL = Workload("pin_small", 90, 2, 4, 2, 16, 96, 4, 64, 25, 16, "fp32")


# ----------------------------------------------------------------------------- codes

@pytest.mark.parametrize("D,nb", [(8, 64), (16, 128), (64, 64), (128, 128)])
def test_codes_match_fp64_sign_within_rounding(oracle_mod, D, nb):
    """sign(W x) with the canonical fp32 chain vs exact fp64: every disagreement is explained by
    the fp32 rounding bound gamma_D * sum|W_jd x_d|."""
    rng = np.random.default_rng(D * 1000 + nb)
    R = np.eye(D, dtype=np.float32)
    W = rng.standard_normal((nb, D)).astype(np.float32)
    X = (rng.standard_normal((500, D)) * rng.lognormal(0, 1, D)).astype(np.float32)
    _, codes = oracle_mod.project(R, W, X)
    y64 = X.astype(np.float64) @ W.astype(np.float64).T
    bound = gamma(D) * (np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T)
    got = bits_of(codes)
    want = y64 > 0
    bad = (got != want) & (np.abs(y64) > bound)
    assert not bad.any()
    assert (got != want).mean() < 1e-3


def test_code_bit_order_lsb_first(oracle_mod):
    """W = diag(s), x = 1: bit j is set iff s_j > 0, in word j//64 at position j%64."""
    D = 128
    rng = np.random.default_rng(1)
    s = np.where(rng.random(D) < 0.5, -1.0, 1.0).astype(np.float32)
    W = np.diag(s).astype(np.float32)
    _, codes = oracle_mod.project(np.eye(D, dtype=np.float32), W, np.ones((1, D), np.float32))
    want0 = sum(1 << j for j in range(64) if s[j] > 0)
    want1 = sum(1 << (j - 64) for j in range(64, 128) if s[j] > 0)
    assert int(codes[0, 0]) == want0 and int(codes[0, 1]) == want1


def test_code_identity_projection_is_sign_of_input(oracle_mod):
    """W = I: bit j = [x_j > 0] exactly; zeros of either sign give 0."""
    D = 64
    rng = np.random.default_rng(2)
    X = rng.standard_normal((50, D)).astype(np.float32)
    X[0, :8] = 0.0
    X[1, :8] = -0.0
    _, codes = oracle_mod.project(np.eye(D, dtype=np.float32), np.eye(D, dtype=np.float32), X)
    assert np.array_equal(bits_of(codes), X > 0)


# ----------------------------------------------------------------------------- rotation

def test_rotation_orientation_with_permutation(oracle_mod):
    """R = permutation with R[r][perm[r]] = 1 gives xrot_r = x_perm[r] (catches a transposed R)."""
    D = 16
    perm = np.roll(np.arange(D), 3)  # not an involution
    R = np.zeros((D, D), np.float32)
    R[np.arange(D), perm] = 1.0
    X = np.random.default_rng(3).standard_normal((10, D)).astype(np.float32)
    xr, _ = oracle_mod.project(R, np.eye(64, D, dtype=np.float32), X)
    assert np.array_equal(xr, X[:, perm])


@pytest.mark.parametrize("D", [16, 64, 128])
def test_rotation_preserves_logits(oracle_mod, D):
    """Orthogonal R keeps q.k: |Rq.Rk - q.k| <= 1e-5 |q||k| (fp64 over the fp32 values)."""
    rng = np.random.default_rng(D)
    A = rng.standard_normal((D, D))
    Qm, Rr = np.linalg.qr(A)
    R = (Qm * np.sign(np.diag(Rr))).astype(np.float32)
    X = (rng.standard_normal((200, D)) * rng.lognormal(0, 1, D)).astype(np.float32)
    xr, _ = oracle_mod.project(R, np.eye(64, D, dtype=np.float32), X)
    q, k = X[:100].astype(np.float64), X[100:].astype(np.float64)
    qr, kr = xr[:100].astype(np.float64), xr[100:].astype(np.float64)
    lhs = qr @ kr.T
    rhs = q @ k.T
    tol = 1e-5 * np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(k, axis=1)[None, :]
    assert (np.abs(lhs - rhs) <= tol).all()


def test_rotation_accuracy_against_fp64(oracle_mod):
    """Each rotated coordinate is within gamma_D * sum|R x| of the exact fp64 product (no dropped term)."""
    D = 128
    rng = np.random.default_rng(5)
    R = rng.standard_normal((D, D)).astype(np.float32)
    X = rng.standard_normal((64, D)).astype(np.float32)
    xr, _ = oracle_mod.project(R, np.eye(64, D, dtype=np.float32), X)
    exact = X.astype(np.float64) @ R.astype(np.float64).T
    bound = gamma(D) * (np.abs(X.astype(np.float64)) @ np.abs(R.astype(np.float64)).T)
    assert (np.abs(xr - exact) <= bound).all()


# ----------------------------------------------------------------------------- page metadata

def test_meta_identity_rotation_is_raw_page_min_max(oracle_mod):
    """R = I: meta is the textbook per-page per-channel max/min of the raw keys, partial page included."""
    wl = SMALL.with_(batch=1, n_kv_heads=1, n_q_heads=2, ctx=90)
    d = make_layer(wl)
    d["R"] = np.broadcast_to(np.eye(wl.head_dim, dtype=np.float32), d["R"].shape).copy()
    dims = dims_for(oracle_mod, wl)
    L = 90
    meta, _ = oracle_mod.encode(dims, d["K"], d["R"], d["W"], [0], [L])
    K = f32(d["K"], wl)[0, 0]
    for p in range(-(-L // wl.page_size)):
        blk = K[p * wl.page_size:min((p + 1) * wl.page_size, L)]
        assert np.array_equal(meta[0, 0, p, :, 0], blk.max(0))
        assert np.array_equal(meta[0, 0, p, :, 1], blk.min(0))


def test_meta_permutation_rotation(oracle_mod):
    wl = SMALL.with_(batch=1, n_kv_heads=1, n_q_heads=1, ctx=32)
    d = make_layer(wl)
    D = wl.head_dim
    perm = np.roll(np.arange(D), 5)
    R = np.zeros((1, D, D), np.float32)
    R[0, np.arange(D), perm] = 1.0
    meta, _ = oracle_mod.encode(dims_for(oracle_mod, wl), d["K"], R, d["W"], [0], [32])
    K = f32(d["K"], wl)[0, 0][:, perm]
    for p in range(32 // wl.page_size):
        blk = K[p * wl.page_size:(p + 1) * wl.page_size]
        assert np.array_equal(meta[0, 0, p, :, 0], blk.max(0))
        assert np.array_equal(meta[0, 0, p, :, 1], blk.min(0))


@pytest.mark.parametrize("m", [1, 5, 37, 64])
def test_encode_append_equals_single_shot(oracle_mod, m):
    """Encoding [0,m) then [m,n) is bit-identical to encoding [0,n) (meta and codes)."""
    wl = SMALL.with_(dtype="bf16")
    d = make_layer(wl)
    dims = dims_for(oracle_mod, wl)
    n = 90
    B = wl.batch
    one_meta, one_codes = oracle_mod.encode(dims, d["K"], d["R"], d["W"], [0] * B, [n] * B)
    meta, codes = oracle_mod.encode(dims, d["K"], d["R"], d["W"], [0] * B, [m] * B)
    meta, codes = oracle_mod.encode(dims, d["K"], d["R"], d["W"], [m] * B, [n - m] * B, meta, codes)
    npg = -(-n // wl.page_size)
    assert np.array_equal(meta[:, :, :npg].view(np.uint32), one_meta[:, :, :npg].view(np.uint32))
    assert np.array_equal(codes[:, :, :n], one_codes[:, :, :n])


# ----------------------------------------------------------------------------- page bounds

def _hand_case(o, case, keep=None):
    D, P = case["head_dim"], case["page_size"]
    Qv = np.array(case["queries"], np.float32)
    Kv = np.array(case["keys"], np.float32)
    G = Qv.shape[0]
    T = Kv.shape[0]
    L = case.get("length", T)
    dims = o.Dims(1, G, 1, D, P, 64, T, False)
    R = np.eye(D, dtype=np.float32)[None]
    W = np.random.default_rng(0).standard_normal((1, 64, D)).astype(np.float32)
    K = Kv[None, None]
    V = np.ones_like(K)
    meta, codes = o.encode(dims, K, R, W, [0], [L])
    npg = -(-L // P)
    kp = keep if keep is not None else case.get("keep", npg)
    r = o.decode(dims, Qv[None], K, V, R, W, meta, codes, [L], [kp], npg, 4)
    return meta, r


def test_page_bound_hand_worked_examples(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "page_bound_hand.json")))
    for case in g["cases"]:
        meta, r = _hand_case(oracle_mod, case)
        npg = len(case["scores"])
        assert np.array_equal(meta[0, 0, :npg, :, 0], np.array(case["kmax"], np.float32)), case["name"]
        assert np.array_equal(meta[0, 0, :npg, :, 1], np.array(case["kmin"], np.float32)), case["name"]
        assert np.array_equal(r["score"][0, 0, :npg], np.array(case["scores"])), case["name"]
        if "pages" in case:
            assert list(r["pages"][0, 0, :len(case["pages"])]) == case["pages"], case["name"]


@pytest.mark.parametrize("G,P", [(1, 1), (4, 4), (7, 16), (2, 3)])
def test_page_bound_is_upper_bound_of_every_logit(oracle_mod, G, P):
    """S(p) >= max over the page's keys and the group's heads of qrot.krot (exact up to fp64 rounding),
    and >= the raw logit q.k minus the rotation tolerance; with P = 1 it is equal to the max logit."""
    wl = Workload("pin_ub", 91, 2, 2 * G, 2, 32, 200, P, 64, 30, 32, "bf16", outliers=2, ragged=(150, 200))
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d, max_keep=-(-200 // P))
    Qf, Kf = f32(d["Q"], wl), f32(d["K"], wl)
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for h in range(wl.n_kv_heads):
            kr, _ = oracle_mod.project(d["R"][h], d["W"][h], Kf[b, h, :L])
            qr = r["q_rot"][b, h * G:(h + 1) * G].astype(np.float64)
            lt = qr @ kr.astype(np.float64).T                          # [G][L] rotated logits
            raw = Qf[b, h * G:(h + 1) * G].astype(np.float64) @ Kf[b, h, :L].astype(np.float64).T
            qn = np.linalg.norm(Qf[b, h * G:(h + 1) * G].astype(np.float64), axis=1)[:, None]
            kn = np.linalg.norm(Kf[b, h, :L].astype(np.float64), axis=1)[None, :]
            for p in range(-(-L // P)):
                sl = slice(p * P, min((p + 1) * P, L))
                S = r["score"][b, h, p]
                mag = np.abs(qr) @ np.abs(kr[sl].astype(np.float64)).T
                assert S >= lt[:, sl].max() - 1e-12 * mag.max()
                assert S >= (raw[:, sl] - 1e-5 * qn * kn[:, sl]).max()
                if P == 1:
                    assert abs(S - lt[:, sl].max()) <= 1e-12 * mag.max()


def _bf16_step(v, down: bool):
    """The bf16 value adjacent to the bf16 value v (fp32 array, low 16 bits zero), toward -inf (down) or +inf;
    from the IEEE bit layout, independent of the oracle's code."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.int64)
    neg = (u >> 31) == 1
    mag_up = (neg & down) | (~neg & ~down)  # moving away from zero
    zero = (u & 0x7FFFFFFF) == 0
    out = np.where(mag_up, u + 0x10000, u - 0x10000)
    out = np.where(zero, np.where(down, 0x80010000, 0x00010000), out)
    return out.astype(np.uint32).view(np.float32)


def test_bf16_meta_is_outward_rounding_of_fp32_meta(oracle_mod):
    """With bf16 metadata every stored max is the smallest bf16 value >= the page's true max and every min the
    largest bf16 value <= its true min (the true values: the fp32-metadata encode of the same keys)."""
    wl = WORKLOADS["tiny"].with_(batch=2, ragged=(1000, 4096))
    d = make_layer(wl)
    seq = d["seq_len"]
    dm32 = dims_for(oracle_mod, wl)
    dm16 = dims_for(oracle_mod, wl.with_(meta_bf16=True))
    m32, _ = oracle_mod.encode(dm32, d["K"], d["R"], d["W"], np.zeros(wl.batch, np.int32), seq)
    m16, _ = oracle_mod.encode(dm16, d["K"], d["R"], d["W"], np.zeros(wl.batch, np.int32), seq)
    for b in range(wl.batch):
        NP = -(-int(seq[b]) // wl.page_size)
        mx32, mn32 = m32[b, :, :NP, :, 0], m32[b, :, :NP, :, 1]
        mx16, mn16 = m16[b, :, :NP, :, 0], m16[b, :, :NP, :, 1]
        assert (mx16.view(np.uint32) & 0xFFFF == 0).all() and (mn16.view(np.uint32) & 0xFFFF == 0).all()
        assert (mx16 >= mx32).all() and (mn16 <= mn32).all()
        assert (_bf16_step(mx16, down=True) < mx32).all()     # nothing bf16 in [true max, stored max)
        assert (_bf16_step(mn16, down=False) > mn32).all()    # nothing bf16 in (stored min, true min]
        assert (mx16 > mx32).any()  # the rounding is not vacuous on these keys


def test_bf16_meta_rounding_special_values(oracle_mod):
    """Hand cases through a one-key page: values already bf16 stay; positive and negative values round
    outward; +0 stays +0 (the rotation is the identity, so the page max/min are the key itself)."""
    D = 32
    vals = np.zeros(D, np.float32)
    vals[:8] = [1.0, -1.0, 1.0 + 2.0 ** -10, -(1.0 + 2.0 ** -10), 3.0e-39, -3.0e-39, 0.0, 65504.0]
    K = vals[None, None, None, :]
    R = np.eye(D, dtype=np.float32)[None]
    W = np.eye(64, D, dtype=np.float32)[None]
    dm = oracle_mod.Dims(1, 1, 1, D, 1, 64, 1, False, True)
    m, _ = oracle_mod.encode(dm, K, R, W, np.array([0], np.int32), np.array([1], np.int32))
    mx, mn = m[0, 0, 0, :8, 0], m[0, 0, 0, :8, 1]
    up = [1.0, -1.0, 1.0 + 2.0 ** -7, -1.0, None, None, 0.0, 65536.0]
    dn = [1.0, -1.0, 1.0, -(1.0 + 2.0 ** -7), None, None, 0.0, 65504.0 - 224.0]
    for i in (0, 1, 2, 3, 6):
        assert mx[i] == np.float32(up[i]) and mn[i] == np.float32(dn[i]), i
    # 3e-39 (an fp32 denormal): the max rounds up to a bf16 denormal above it, the min down to below it
    assert mx[4] >= vals[4] and mn[4] <= vals[4] and mx[5] >= vals[5] and mn[5] <= vals[5]
    assert mx[7] == np.float32(65536.0) and mn[7] == np.float32(65280.0)


@pytest.mark.parametrize("G,P", [(4, 4), (2, 16)])
def test_bf16_meta_bound_still_bounds_every_logit(oracle_mod, G, P):
    """The page bound from bf16 metadata is >= the bound from fp32 metadata of the same keys, hence >= every
    rotated logit of the page."""
    wl = Workload("pin_ub16", 92, 2, 2 * G, 2, 32, 200, P, 64, 30, 32, "bf16", outliers=2, ragged=(150, 200))
    d = make_layer(wl)
    _, _, _, r32 = run(oracle_mod, wl, d, max_keep=-(-200 // P))
    _, _, _, r16 = run(oracle_mod, wl.with_(meta_bf16=True), d, max_keep=-(-200 // P))
    Kf = f32(d["K"], wl)
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        NP = -(-L // P)
        assert (r16["score"][b, :, :NP] >= r32["score"][b, :, :NP]).all()
        for h in range(wl.n_kv_heads):
            kr, _ = oracle_mod.project(d["R"][h], d["W"][h], Kf[b, h, :L])
            lt = r16["q_rot"][b, h * G:(h + 1) * G].astype(np.float64) @ kr.astype(np.float64).T
            for p in range(NP):
                assert r16["score"][b, h, p] >= lt[:, p * P:min((p + 1) * P, L)].max() - 1e-9


def test_page_select_is_lexsort_of_scores(oracle_mod):
    """Kept pages = textbook lexsort by (-S, p), first keep, ascending."""
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    for h in range(wl.n_kv_heads):
        S = r["score"][0, h, :wl.max_pages]
        order = np.lexsort((np.arange(len(S)), -S))
        want = np.sort(order[:d["keep"][0]])
        assert np.array_equal(r["pages"][0, h, :len(want)], want)
        assert (r["pages"][0, h, len(want):] == -1).all()
        assert r["n_pages"][0, h] == len(want)


def test_page_select_ties_go_to_lower_index(oracle_mod):
    """Duplicate pages have equal bounds; the lower index wins the last slot."""
    wl = SMALL.with_(batch=1, n_kv_heads=1, n_q_heads=2, ctx=64, page_size=4, dtype="fp32")
    d = make_layer(wl)
    K = d["K"]
    dup = [3, 9, 12]
    for p in dup[1:]:
        K[0, 0, p * 4:(p + 1) * 4] = K[0, 0, dup[0] * 4:(dup[0] + 1) * 4]
    K[0, 0, dup[0] * 4:(dup[0] + 1) * 4] *= 50.0
    for p in dup[1:]:
        K[0, 0, p * 4:(p + 1) * 4] = K[0, 0, dup[0] * 4:(dup[0] + 1) * 4]
    d["Q"][0] = K[0, 0, dup[0] * 4][None, :]  # make those pages the top three
    dims, meta, codes, r = run(oracle_mod, wl, d, keep=[2], max_keep=4)
    S = r["score"][0, 0]
    assert S[3] == S[9] == S[12] and S[3] == S.max()
    assert list(r["pages"][0, 0, :2]) == [3, 9]


def test_page_select_step_is_brute_force_on_given_scores(oracle_mod):
    """The page-select step alone, on scores with hard ties (fp32-tied clusters, exact duplicates, signed
    zeros, denormals, all equal) and ragged lengths: the first keep of the pages sorted by (-S, p) in plain
    Python (values compared as numbers, so -0 == +0), listed ascending and -1 padded; keep clamped."""
    from synth import tie_scores
    B, H, P, T = 3, 2, 16, 4096 * 16
    NPmax = -(-T // P)
    seq = np.array([T, 3001 * P - 7, 0], np.int32)
    NP = [-(-int(L) // P) for L in seq]
    keep = np.array([700, 250, 5], np.int32)
    mk = 1024
    S = tie_scores(11, B, H, NPmax, NP, keep)
    dims = oracle_mod.Dims(B, 4 * H, H, 64, P, 64, T, False)
    pages, n_pages = oracle_mod.select_pages(dims, S, seq, keep, mk)
    for b in range(B):
        for h in range(H):
            kp = max(1, min(int(keep[b]), NP[b], mk))
            if NP[b] == 0:
                kp = 0
            order = sorted(range(NP[b]), key=lambda p: (-float(S[b, h, p]), p))
            want = sorted(order[:kp])
            assert list(pages[b, h, :kp]) == want, (b, h)
            assert (pages[b, h, kp:] == -1).all()
            assert n_pages[b, h] == kp


def test_page_select_step_matches_decode(oracle_mod):
    """The page-select step on the decode step's own scores gives the decode step's page lists."""
    wl = WORKLOADS["tiny"].with_(batch=2, ragged=(1000, 4096))
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    pages, n_pages = oracle_mod.select_pages(dims, r["score"], d["seq_len"], d["keep"], wl.max_keep)
    assert np.array_equal(pages, r["pages"]) and np.array_equal(n_pages, r["n_pages"])


def test_keep_is_clamped(oracle_mod):
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    npg = wl.max_pages
    for keep, mk, want in [(0, 8, 1), (-5, 8, 1), (10**6, npg + 5, npg), (500, 8, 8)]:
        _, _, _, r = run(oracle_mod, wl, d, keep=[keep], max_keep=mk)
        assert (r["n_pages"] == want).all()


# ----------------------------------------------------------------------------- Hamming + top-k

def _vec_from_code(code: int, D: int):
    return np.array([1.0 if (code >> j) & 1 else -1.0 for j in range(D)], np.float32)


def test_hamming_and_topk_hand_worked(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "hamming_hand.json")))
    D, P = g["head_dim"], g["page_size"]
    qs = np.stack([_vec_from_code(int(c, 16), D) for c in g["query_codes"]])
    ks = np.stack([_vec_from_code(int(c, 16), D) for c in g["key_codes"]])
    G, T = len(qs), len(ks)
    dims = oracle_mod.Dims(1, G, 1, D, P, 64, T, False)
    eye = np.eye(D, dtype=np.float32)[None]
    meta, codes = oracle_mod.encode(dims, ks[None, None], eye, eye, [0], [T])
    assert [hex(int(c)) for c in codes[0, 0, :, 0]] == [hex(int(c, 16)) for c in g["key_codes"]]
    for k, want in g["top_k"].items():
        r = oracle_mod.decode(dims, qs[None], ks[None, None], ks[None, None], eye, eye, meta, codes,
                              [T], [T // P], T // P, int(k))
        assert list(r["ham"][0, 0, :T]) == g["distances"]
        assert list(r["sel"][0, 0, :len(want)]) == want
        assert r["k_eff"][0, 0] == len(want)


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_hamming_is_brute_force_popcount(oracle_mod, name):
    """H of each candidate = sum over heads and words of Python int.bit_count(code_q ^ code_t)."""
    wl = WORKLOADS["tiny"] if name == "tiny" else Workload("pin_rag", 92, 3, 6, 2, 32, 300, 8, 128, 20, 40,
                                                          "bf16", ragged=(100, 300))
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    G, P, Wd = wl.group, wl.page_size, wl.hash_bits // 64
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for h in range(wl.n_kv_heads):
            cq = [[int(r["code_q"][b, h * G + i, w]) for w in range(Wd)] for i in range(G)]
            for j in range(r["n_pages"][b, h]):
                p = r["pages"][b, h, j]
                for rr in range(P):
                    t = p * P + rr
                    slot = r["ham"][b, h, j * P + rr]
                    if t >= L:
                        assert slot == 0xFFFF
                        continue
                    want = sum((cq[i][w] ^ int(codes[b, h, t, w])).bit_count() for i in range(G) for w in range(Wd))
                    assert slot == want


def test_key_select_is_lexsort(oracle_mod):
    """Selected keys = textbook lexsort of candidates by (H, t), first k_eff, ascending."""
    wl = Workload("pin_ks", 93, 2, 8, 2, 32, 512, 8, 64, 25, 60, "fp32", ragged=(300, 512))
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    P = wl.page_size
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for h in range(wl.n_kv_heads):
            n = r["n_pages"][b, h]
            t = (r["pages"][b, h, :n, None] * P + np.arange(P)[None, :]).ravel()
            H = r["ham"][b, h, :n * P].astype(np.int64)
            ok = t < L
            t, H = t[ok], H[ok]
            order = np.lexsort((t, H))
            keff = min(wl.top_k, len(t))
            want = np.sort(t[order[:keff]])
            assert r["k_eff"][b, h] == keff
            assert np.array_equal(r["sel"][b, h, :keff], want)
            assert (r["sel"][b, h, keff:] == -1).all()


def test_zero_hash_projection_selects_first_candidates(oracle_mod):
    """W = 0: every code is 0, every H is 0, so the first k_eff candidates (ascending) win."""
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    d["W"] = np.zeros_like(d["W"])
    dims, meta, codes, r = run(oracle_mod, wl, d)
    assert not codes.any() and not r["code_q"].any()
    P = wl.page_size
    for h in range(wl.n_kv_heads):
        t = (r["pages"][0, h, :r["n_pages"][0, h], None] * P + np.arange(P)[None, :]).ravel()
        assert np.array_equal(r["sel"][0, h], t[:wl.top_k])


def test_topk_larger_than_candidates_pads(oracle_mod):
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d, keep=[3], max_keep=3, top_k=100)
    assert (r["k_eff"] == 48).all()
    assert (r["sel"][..., 48:] == -1).all() and (r["sel"][..., :48] >= 0).all()


# ----------------------------------------------------------------------------- attention

def test_attention_hand_worked(oracle_mod):
    g = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))
    q = np.array([g["query"]], np.float32)
    K = np.array(g["keys"], np.float32)[None, None]
    V = np.array(g["values"], np.float32)[None, None]
    dims = oracle_mod.Dims(1, 1, 1, 2, 1, 64, 2, False)
    R = np.eye(2, dtype=np.float32)[None]
    W = np.ones((1, 64, 2), np.float32)
    meta, codes = oracle_mod.encode(dims, K, R, W, [0], [2])
    r = oracle_mod.decode(dims, q[None], K, V, R, W, meta, codes, [2], [2], 2, 2, g["scale"])
    assert np.abs(r["out"][0, 0] - np.array(g["out"])).max() <= g["tol"]


def _softmax_attention(q, K, V, scale):
    s = (K @ q) * scale
    w = np.exp(s - s.max())
    return (w[:, None] * V).sum(0) / w.sum()


@pytest.mark.parametrize("name", ["tiny", "bf16_ragged"])
def test_full_selection_equals_full_attention(oracle_mod, name):
    """keep every page and top_k >= L: the method is exact softmax attention over all keys."""
    wl = WORKLOADS["tiny"].with_(ctx=1024) if name == "tiny" else \
        Workload("pin_full", 94, 2, 6, 3, 32, 300, 16, 64, 100, 300, "bf16", outliers=2, ragged=(1, 300))
    d = make_layer(wl)
    npg = wl.max_pages
    dims, meta, codes, r = run(oracle_mod, wl, d, keep=[npg] * wl.batch, max_keep=npg, top_k=wl.ctx)
    Qf, Kf, Vf = (f32(d[k], wl).astype(np.float64) for k in ("Q", "K", "V"))
    G = wl.group
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for i in range(wl.n_q_heads):
            h = i // G
            ref = _softmax_attention(Qf[b, i], Kf[b, h, :L], Vf[b, h, :L], 1 / np.sqrt(wl.head_dim))
            assert np.abs(r["out"][b, i] - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max())
        assert (r["k_eff"][b] == L).all()


def test_sparse_attention_uses_selected_keys(oracle_mod):
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    Qf, Kf, Vf = (np.asarray(d[k], np.float64) for k in ("Q", "K", "V"))
    for i in range(wl.n_q_heads):
        h = i // wl.group
        s = r["sel"][0, h, :r["k_eff"][0, h]]
        ref = _softmax_attention(Qf[0, i], Kf[0, h, s], Vf[0, h, s], 1 / np.sqrt(wl.head_dim))
        assert np.abs(r["out"][0, i] - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max())


def test_empty_sequence(oracle_mod):
    wl = WORKLOADS["tiny"].with_(batch=2)
    d = make_layer(wl, lengths=[0, 100])
    dims, meta, codes, r = run(oracle_mod, wl, d)
    assert (r["out"][0] == 0).all() and (r["k_eff"][0] == 0).all() and (r["sel"][0] == -1).all()
    assert (r["n_pages"][0] == 0).all() and (r["pages"][0] == -1).all()
    for h in range(wl.n_kv_heads):
        pg = r["pages"][1, h, :r["n_pages"][1, h]]
        assert r["k_eff"][1, h] == sum(min(wl.page_size, 100 - p * wl.page_size) for p in pg) > 0


def test_rows_past_length_are_ignored(oracle_mod):
    wl = Workload("pin_poison", 95, 2, 4, 2, 32, 256, 16, 64, 50, 40, "bf16", ragged=(100, 200))
    d = make_layer(wl)
    _, m0, c0, r0 = run(oracle_mod, wl, d)
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        d["K"][b, :, L:] = f32_to_bf16_bits(np.full((wl.n_kv_heads, wl.ctx - L, wl.head_dim), 1e4, np.float32))
        d["V"][b, :, L:] = d["K"][b, :, L:]
    _, m1, c1, r1 = run(oracle_mod, wl, d)
    for k in ("score", "pages", "ham", "sel", "out"):
        assert np.array_equal(r0[k], r1[k]), k


def _planted_hits(wl, d, r):
    """(planted keys, planted keys whose page was kept, planted keys selected) over all (sequence, KV head)."""
    tot = kept_n = sel_n = 0
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            kept, sel = set(r["pages"][b, h].tolist()), set(r["sel"][b, h].tolist())
            for t in d["planted"][b, h]:
                if t >= 0:
                    tot += 1
                    kept_n += int(t // wl.page_size in kept)
                    sel_n += int(t in sel)
    return tot, kept_n, sel_n


def test_planted_keys_in_kept_pages_are_selected(oracle_mod):
    """End-to-end expectation 1 (sanity, not parity): on the tiny workload every planted key whose page survives
    the coarse stage is kept by the Hamming stage."""
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    hits = 0
    for h in range(wl.n_kv_heads):
        kept = set(r["pages"][0, h])
        surv = {t for t in d["planted"][0, h] if t // wl.page_size in kept}
        assert surv <= set(r["sel"][0, h])
        hits += len(surv)
    assert hits > 0


@pytest.mark.parametrize("name", ["tiny", "llama8b_32k"])
def test_hamming_stage_selects_every_planted_key(oracle_mod, name):
    """End-to-end expectation 2: with every page kept, the Hamming stage alone selects all 8 planted keys of
    every KV head (each sits about 27 degrees from its queries, so its code differs from theirs in far fewer
    bits than a random key's)."""
    wl = WORKLOADS[name]
    d = make_layer(wl)
    NPg = wl.max_pages
    _, _, _, r = run(oracle_mod, wl, d, keep=np.full(wl.batch, NPg, np.int32), max_keep=NPg)
    tot, kept_n, sel_n = _planted_hits(wl, d, r)
    assert tot == 8 * wl.batch * wl.n_kv_heads and kept_n == tot and sel_n == tot


def test_page_stage_keeps_planted_pages_above_chance(oracle_mod):
    """End-to-end expectation 3: at 32K with 10% of pages kept, the coarse stage keeps planted pages at well
    over the keep fraction (at least twice it), and each planted key whose page is kept is selected.  With a
    random rotation the box bound of a random 16-key page sits far above any one key's logit, so a planted
    page is not kept every time (the seeded layer keeps 19 of 64); all 8 planted keys per head reach the
    selection only when the page stage passes them."""
    wl = WORKLOADS["llama8b_32k"]
    d = make_layer(wl)
    _, _, _, r = run(oracle_mod, wl, d)
    tot, kept_n, sel_n = _planted_hits(wl, d, r)
    frac = float(d["keep"][0]) / wl.max_pages
    assert tot == 64 and kept_n / tot >= 2.0 * frac
    assert sel_n == kept_n


# ----------------------------------------------------------------------------- fidelity harness metrics

def test_fidelity_metrics_on_oracle_selections(oracle_mod):
    """The harness's metrics on known selections: selecting every key of every page (keep all, top_k >= L)
    gives recall, coverage, mass and planted recall 1 and full attention's output; the oracle's sparse
    selection gives values in [0, 1] and selects the planted keys of kept pages."""
    from fidelity import metrics
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    NPg = wl.max_pages
    dims, meta, codes, r = run(oracle_mod, wl, d, keep=[NPg], max_keep=NPg, top_k=wl.ctx)
    m = metrics(wl, d, r["sel"], r["out"], r["pages"], r["n_pages"])
    assert m["key_recall"] == 1.0 and m["page_coverage"] == 1.0 and m["planted_recall"] == 1.0
    assert abs(m["attention_mass"] - 1.0) < 1e-12 and m["out_max_err"] < 1e-9
    dims, meta, codes, r = run(oracle_mod, wl, d)
    m = metrics(wl, d, r["sel"], r["out"], r["pages"], r["n_pages"])
    for k in ("key_recall", "page_coverage", "attention_mass", "planted_recall"):
        assert 0.0 <= m[k] <= 1.0, k
    assert m["key_recall"] <= m["page_coverage"] + 1e-12  # a key the page stage dropped cannot be selected


def test_fidelity_recall_counts_the_exact_top_k(oracle_mod):
    """Hand-built selections: the exact top-k itself has recall 1; its first half padded with keys outside
    it has recall 1/2 (recall is measured at the selection's own size)."""
    from fidelity import metrics
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    G, L = wl.group, int(d["seq_len"][0])
    sel = np.full_like(r["sel"], -1)
    half = np.full_like(r["sel"], -1)
    for h in range(wl.n_kv_heads):
        q = f32(d["Q"], wl)[0, h * G:(h + 1) * G].astype(np.float64)
        s = (q @ f32(d["K"], wl)[0, h, :L].astype(np.float64).T).max(axis=0)
        order = np.lexsort((np.arange(L), -s))
        k = 64
        sel[0, h, :k] = np.sort(order[:k])
        half[0, h, :k] = np.sort(np.concatenate([order[:k // 2], order[L - k // 2:]]))
    assert metrics(wl, d, sel, r["out"], r["pages"], r["n_pages"])["key_recall"] == 1.0
    assert metrics(wl, d, half, r["out"], r["pages"], r["n_pages"])["key_recall"] == 0.5


# ----------------------------------------------------------------------------- TopK (Oracle) selection

def _int_layer(seed, B, Hq, Hkv, D, T, lo=-3, hi=3, bf16=False):
    """Integer-valued Q, K, V: every logit is an exact integer whatever the summation order."""
    rng = np.random.default_rng(seed)
    Q = rng.integers(lo, hi + 1, (B, Hq, D)).astype(np.float32)
    K = rng.integers(lo, hi + 1, (B, Hkv, T, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    if bf16:
        return f32_to_bf16_bits(Q), f32_to_bf16_bits(K), f32_to_bf16_bits(V)
    return Q, K, V


@pytest.mark.parametrize("G,D,bf16", [(1, 16, False), (4, 16, True), (3, 64, False), (8, 8, True)])
def test_topk_select_is_lexsort_of_integer_logits(oracle_mod, G, D, bf16):
    """TopK (Oracle) keeps the keys of largest exact group-max logit, ties to the lower key: with
    integer-valued inputs the logits are exact integers, so numpy's int64 products and lexsort
    state the expected selection exactly (and the small range makes ties common)."""
    B, Hkv, T, top_k = 2, 2, 203, 37
    Q, K, V = _int_layer(11 + G + D, B, G * Hkv, Hkv, D, T, bf16=bf16)
    seq = np.array([203, 29], np.int32)  # the second is shorter than top_k
    dims = oracle_mod.Dims(B, G * Hkv, Hkv, D, 16, 64, T, bf16)
    r = oracle_mod.topk(dims, Q, K, V, seq, top_k)
    Qi = (bf16_bits_to_f32(Q) if bf16 else Q).astype(np.int64)
    Ki = (bf16_bits_to_f32(K) if bf16 else K).astype(np.int64)
    for b in range(B):
        L = int(seq[b])
        for h in range(Hkv):
            z = (Qi[b, h * G:(h + 1) * G] @ Ki[b, h, :L].T).max(axis=0)
            keff = min(top_k, L)
            want = np.sort(np.lexsort((np.arange(L), -z))[:keff])
            assert r["k_eff"][b, h] == keff
            assert (r["sel"][b, h, :keff] == want).all()
            assert (r["sel"][b, h, keff:] == -1).all()
            assert (r["score"][b, h, :L] == z.astype(np.float64)).all()
            assert (r["score"][b, h, L:] == 0).all()


def test_topk_ties_go_to_lower_key(oracle_mod):
    """All logits equal (zero query): the first top_k keys are kept."""
    B, Hkv, G, D, T = 1, 1, 2, 8, 100
    Q, K, V = _int_layer(5, B, G * Hkv, Hkv, D, T)
    Q[:] = 0
    dims = oracle_mod.Dims(B, G * Hkv, Hkv, D, 16, 64, T, False)
    r = oracle_mod.topk(dims, Q, K, V, [T], 10)
    assert (r["sel"][0, 0] == np.arange(10)).all()


@pytest.mark.parametrize("name", ["tiny", "bf16_ragged"])
def test_topk_all_keys_is_full_attention(oracle_mod, name):
    """top_k >= L keeps every key: the output is exact softmax attention (numpy fp64)."""
    wl = WORKLOADS["tiny"].with_(ctx=1024) if name == "tiny" else \
        Workload("pin_topk_full", 95, 2, 6, 3, 32, 300, 16, 64, 100, 300, "bf16", outliers=2, ragged=(1, 300))
    d = make_layer(wl)
    r = oracle_mod.topk(dims_for(oracle_mod, wl), d["Q"], d["K"], d["V"], d["seq_len"], wl.ctx)
    Qf, Kf, Vf = (f32(d[k], wl).astype(np.float64) for k in ("Q", "K", "V"))
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        assert (r["sel"][b, :, :L] == np.arange(L)).all() and (r["k_eff"][b] == L).all()
        for i in range(wl.n_q_heads):
            h = i // wl.group
            ref = _softmax_attention(Qf[b, i], Kf[b, h, :L], Vf[b, h, :L], 1 / np.sqrt(wl.head_dim))
            assert np.abs(r["out"][b, i] - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max())


def test_topk_logits_near_fp64_dot(oracle_mod):
    """The group-max logit of random fp32 data is the fp64 dot product up to fp64 rounding."""
    wl = WORKLOADS["tiny"].with_(ctx=512)
    d = make_layer(wl)
    r = oracle_mod.topk(dims_for(oracle_mod, wl), d["Q"], d["K"], d["V"], d["seq_len"], 64)
    Q, K = np.asarray(d["Q"], np.float64), np.asarray(d["K"], np.float64)
    G = wl.group
    for h in range(wl.n_kv_heads):
        z = (Q[0, h * G:(h + 1) * G] @ K[0, h].T).max(axis=0)
        bound = wl.head_dim * 2.0 ** -52 * (np.abs(Q[0, h * G:(h + 1) * G]) @ np.abs(K[0, h]).T).max(axis=0)
        assert (np.abs(r["score"][0, h] - z) <= bound).all()


def test_topk_equals_hhr_path_at_page_size_one_without_rotation(oracle_mod):
    """With one key per page, R_h = I and every candidate kept by the Hamming stage, the page bound
    of a page is its key's exact logit, so the HHR step selects what TopK (Oracle) selects."""
    wl = Workload("pin_topk_p1", 96, 2, 8, 2, 32, 160, 1, 64, 25, 24, "bf16", outliers=2, ragged=(50, 160))
    d = make_layer(wl)
    d["R"] = np.stack([np.eye(wl.head_dim, dtype=np.float32)] * wl.n_kv_heads)
    top_k = 24
    t = oracle_mod.topk(dims_for(oracle_mod, wl), d["Q"], d["K"], d["V"], d["seq_len"], top_k)
    dims, meta, codes, r = run(oracle_mod, wl, d, keep=[top_k] * wl.batch, max_keep=top_k, top_k=top_k)
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        assert (r["score"][b, :, :L] == t["score"][b, :, :L]).all()
    assert (r["pages"] == t["sel"]).all() and (r["sel"] == t["sel"]).all()
    assert np.abs(r["out"] - t["out"]).max() == 0.0


def test_topk_recalls_planted_keys(oracle_mod):
    """The planted keys sit well above the random keys' logits: a top-k of 16 holds all 8."""
    wl = WORKLOADS["tiny"]
    d = make_layer(wl)
    r = oracle_mod.topk(dims_for(oracle_mod, wl), d["Q"], d["K"], d["V"], d["seq_len"], 16)
    for h in range(wl.n_kv_heads):
        assert np.isin(d["planted"][0, h], r["sel"][0, h]).all()


def test_hamming_logit_table_on_known_codes():
    """Four keys whose Hamming distances to the query are 0, 10, 20, 64 and whose logits fall 3, 2, 1, 0:
    each lands in its distance bin, the rank correlation of -H with the logit is 1 (and -1 reversed), and
    the exact top key is the Hamming top key."""
    from fidelity import hamming_logit, popcount64
    wl = Workload("ham_pin", 97, 1, 1, 1, 2, 4, 1, 64, 100, 4, "fp32")
    K = np.zeros((1, 1, 4, 2), np.float32)
    K[0, 0, :, 0] = [3, 2, 1, 0]
    d = dict(Q=np.array([[[1.0, 0.0]]], np.float32), K=K, seq_len=np.array([4], np.int32))
    cq = np.zeros((1, 1, 1), np.uint64)
    ck = np.array([0, (1 << 10) - 1, (1 << 20) - 1, 2 ** 64 - 1], np.uint64).reshape(1, 1, 4, 1)
    assert list(popcount64(ck.ravel())) == [0, 10, 20, 64]
    r = hamming_logit(wl, d, ck, cq)
    got = {(lo, hi): (n, mu) for lo, hi, n, mu, *_ in r["rows"] if n}
    assert got == {(0, 3): (1, 3.0), (8, 11): (1, 2.0), (20, 23): (1, 1.0), (60, 64): (1, 0.0)}
    assert r["spearman"] == pytest.approx(1.0) and r["top1_overlap"] == 1.0 and r["keys"] == 4
    d["K"] = K[:, :, ::-1].copy()
    r = hamming_logit(wl, d, ck, cq)
    assert r["spearman"] == pytest.approx(-1.0) and r["top1_overlap"] == 0.0


# ----------------------------------------------------------------------------- sink tokens and a local window

def _popcount(x):
    return bin(int(x)).count("1")


@pytest.mark.parametrize("sinks,window,ragged", [(4, 64, None), (1, 0, (100, 4096)), (0, 17, (1, 4096)),
                                                  (7, 300, (50, 400))])
def test_forced_keys_plus_hamming_top_k_of_the_rest(oracle_mod, sinks, window, ragged):
    """With sinks s and window w: the page list is the plain step's; the selection is [0, s), then the
    top_k of the kept pages' other keys by (H, t) (brute-force popcount, numpy lexsort), then the last w keys."""
    wl = WORKLOADS["tiny"].with_(batch=3 if ragged else 1, ragged=ragged, sink_tokens=sinks, local_window=window)
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    plain = run(oracle_mod, wl.with_(sink_tokens=0, local_window=0), d)[3]
    assert (r["pages"] == plain["pages"]).all() and (r["n_pages"] == plain["n_pages"]).all()
    G, P, cap = wl.group, wl.page_size, wl.top_k + sinks + window
    assert r["sel"].shape[-1] == cap
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        s_end = min(sinks, L)
        w_start = max(s_end, L - window)
        for h in range(wl.n_kv_heads):
            cand = [p * P + j for p in r["pages"][b, h, :r["n_pages"][b, h]] for j in range(P)]
            cand = np.array([t for t in cand if t < L and s_end <= t < w_start], np.int64)
            H = np.array([sum(_popcount(r["code_q"][b, i, w] ^ codes[b, h, t, w]) for i in range(h * G, (h + 1) * G)
                               for w in range(wl.hash_bits // 64)) for t in cand], np.int64)
            pick = np.sort(cand[np.lexsort((cand, H))[:wl.top_k]]) if len(cand) else np.zeros(0, np.int64)
            want = np.concatenate([np.arange(s_end), pick, np.arange(w_start, L)])
            assert r["k_eff"][b, h] == len(want)
            assert (r["sel"][b, h, :len(want)] == want).all() and (r["sel"][b, h, len(want):] == -1).all()
            ham = r["ham"][b, h]
            for j, p in enumerate(r["pages"][b, h, :r["n_pages"][b, h]]):
                for q in range(P):
                    t = p * P + q
                    if t < L and (t < s_end or t >= w_start):
                        assert ham[j * P + q] == 0xFFFF


def test_window_covering_the_sequence_is_full_attention(oracle_mod):
    """A local window at least as long as the sequence forces every key: exact softmax attention (numpy
    fp64) whatever keep and top_k are, with no key listed twice."""
    wl = WORKLOADS["tiny"].with_(batch=2, ctx=1024, ragged=(10, 1024), sink_tokens=5, local_window=1024, top_k=3)
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl, d)
    Qf, Kf, Vf = (np.asarray(d[k], np.float64) for k in ("Q", "K", "V"))
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        assert (r["k_eff"][b] == L).all() and (r["sel"][b, :, :L] == np.arange(L)).all()
        for i in range(wl.n_q_heads):
            ref = _softmax_attention(Qf[b, i], Kf[b, i // wl.group, :L], Vf[b, i // wl.group, :L],
                                     1 / np.sqrt(wl.head_dim))
            assert np.abs(r["out"][b, i] - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max())


# ----------------------------------------------------------------------------- group aggregation variants

@pytest.mark.parametrize("name", ["tiny", "bf16_g7"])
def test_page_group_min_is_min_of_single_head_scores(oracle_mod, name):
    """page_group = 1: S(p) is the min over the group of U_i(p); each U_i(p) is the score of a run with
    one query head per KV head (G = 1), so the min of those runs' scores must equal it exactly."""
    wl = WORKLOADS["tiny"] if name == "tiny" else \
        Workload("pin_g7", 98, 2, 14, 2, 64, 600, 8, 64, 20, 40, "bf16", outliers=2, ragged=(100, 600))
    d = make_layer(wl)
    r = run(oracle_mod, wl.with_(page_group=1), d)[3]
    G = wl.group
    per = []
    for j in range(G):
        d1 = dict(d)
        d1["Q"] = np.ascontiguousarray(d["Q"][:, j::G])
        per.append(run(oracle_mod, wl.with_(n_q_heads=wl.n_kv_heads), d1)[3]["score"])
    want = np.minimum.reduce(per)
    for b in range(wl.batch):
        NP = -(-int(d["seq_len"][b]) // wl.page_size)
        assert (r["score"][b, :, :NP] == want[b, :, :NP]).all()


def _f32_mean(q):
    """fp32 mean over axis 0: sequential fp32 sum (rows ascending), then one fp32 division."""
    acc = np.zeros(q.shape[1], np.float32)
    for row in q:
        acc = (acc + row.astype(np.float32)).astype(np.float32)
    return (acc / np.float32(q.shape[0])).astype(np.float32)


@pytest.mark.parametrize("name", ["tiny", "bf16_g7"])
def test_hamming_group_mean_uses_the_mean_query_code(oracle_mod, name):
    """hamming_group = 1: every candidate's H is the popcount of code(mean query) XOR its code, the mean
    query's code coming from the pinned projection of a numpy fp32 mean."""
    wl = WORKLOADS["tiny"] if name == "tiny" else \
        Workload("pin_g7m", 99, 2, 14, 2, 64, 600, 8, 128, 20, 40, "bf16", outliers=2, ragged=(100, 600))
    d = make_layer(wl)
    dims, meta, codes, r = run(oracle_mod, wl.with_(hamming_group=1), d)
    G, P, NW = wl.group, wl.page_size, wl.hash_bits // 64
    Qf = f32(d["Q"], wl)
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for h in range(wl.n_kv_heads):
            qm = _f32_mean(Qf[b, h * G:(h + 1) * G])
            _, cm = oracle_mod.project(d["R"][h], d["W"][h], qm[None, :])
            for j, p in enumerate(r["pages"][b, h, :r["n_pages"][b, h]]):
                for q in range(P):
                    t = int(p) * P + q
                    want = sum(_popcount(cm[0, w] ^ codes[b, h, t, w]) for w in range(NW)) if t < L else 0xFFFF
                    assert r["ham"][b, h, j * P + q] == want


def test_hamming_group_mean_code_on_exact_means(oracle_mod):
    """Independent of the oracle's mean and projection: with W_h = I (code bit d = [x_d > 0]) and group
    queries q_i = m + delta_i whose deltas sum to zero in small dyadic values, the fp32 sum and the division
    by G = 4 are exact, so the mean is m by construction.  Every kept candidate's distance must then be
    popcount([m > 0] XOR [k_t > 0]) over the 64 dimensions; the shared (sum over heads) distances must
    differ somewhere, so the check is not vacuous."""
    wl = WORKLOADS["tiny"].with_(batch=2, keep_percent=100)
    d = make_layer(wl)
    G, D, P = wl.group, wl.head_dim, wl.page_size
    rng = np.random.default_rng(7)
    Q = np.zeros((wl.batch, wl.n_q_heads, D), np.float32)
    means = np.zeros((wl.batch, wl.n_kv_heads, D), np.float32)
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            m = rng.choice([-1, 1], D) * rng.integers(2, 9, D) * 0.5   # +-1 .. +-4 in halves, never 0
            delta = rng.integers(-12, 13, (G - 1, D)) * 0.25            # up to +-3 in quarters
            delta = np.vstack([delta, -delta.sum(axis=0)])              # columns sum to exactly 0
            Q[b, h * G:(h + 1) * G] = (m[None, :] + delta).astype(np.float32)
            means[b, h] = m
    d["Q"] = Q
    d["W"] = np.ascontiguousarray(np.broadcast_to(np.eye(D, dtype=np.float32), (wl.n_kv_heads, D, D)))
    keep = np.full(wl.batch, wl.max_pages, np.int32)
    _, _, _, rm = run(oracle_mod, wl.with_(hamming_group=1), d, keep=keep, max_keep=wl.max_pages)
    _, _, _, rs = run(oracle_mod, wl, d, keep=keep, max_keep=wl.max_pages)
    K = f32(d["K"], wl)
    differs = False
    for b in range(wl.batch):
        L = int(d["seq_len"][b])
        for h in range(wl.n_kv_heads):
            want = ((K[b, h, :L] > 0) != (means[b, h] > 0)[None, :]).sum(axis=1)
            got = rm["ham"][b, h, :L]  # every page kept: slot j * P + r is key j * P + r
            assert (rm["pages"][b, h, :-(-L // P)] == np.arange(-(-L // P))).all()
            assert np.array_equal(got.astype(np.int64), want)
            differs |= bool((rs["ham"][b, h, :L] != got).any())
    assert differs


def test_hamming_group_mean_with_one_head_is_the_plain_step(oracle_mod):
    """With G = 1 the mean query is the query: both aggregations give the same distances and keys."""
    wl = WORKLOADS["tiny"].with_(n_q_heads=2)
    d = make_layer(wl)
    d["Q"] = np.ascontiguousarray(d["Q"][:, :2])
    a = run(oracle_mod, wl, d)[3]
    m = run(oracle_mod, wl.with_(hamming_group=1, page_group=1), d)[3]
    for k in ("score", "pages", "ham", "sel", "k_eff"):
        assert (a[k] == m[k]).all(), k


# ----------------------------------------------------------------------------- per-query-head selection

PH = Workload("pin_ph", 100, 2, 8, 2, 64, 700, 8, 128, 100, 5000, "bf16", outliers=2, ragged=(200, 700))


def test_per_head_scores_max_to_the_shared_score(oracle_mod):
    """The shared page score is the max over the group of the bounds, so it equals the max of the per-head
    scores exactly, page by page."""
    wl = WORKLOADS["tiny"].with_(batch=2, ragged=(1000, 4096))
    d = make_layer(wl)
    shared = run(oracle_mod, wl, d)[3]
    ph = run(oracle_mod, wl.with_(per_head=True), d)[3]
    G = wl.group
    assert ph["score"].shape[1] == wl.n_q_heads and ph["sel"].shape[1] == wl.n_q_heads
    for b in range(wl.batch):
        NP = -(-int(d["seq_len"][b]) // wl.page_size)
        for h in range(wl.n_kv_heads):
            assert (ph["score"][b, h * G:(h + 1) * G, :NP].max(axis=0) == shared["score"][b, h, :NP]).all()


def test_per_head_distances_sum_to_the_shared_distance(oracle_mod):
    """With every page kept the candidate slots line up, and the shared Hamming distance is the sum of the
    group's per-head distances; with top_k >= L both are full attention, head by head."""
    wl = PH
    d = make_layer(wl)
    npg = wl.max_pages
    kw = dict(keep=[npg] * wl.batch, max_keep=npg, top_k=wl.ctx)
    shared = run(oracle_mod, wl, d, **kw)[3]
    ph = run(oracle_mod, wl.with_(per_head=True), d, **kw)[3]
    G = wl.group
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            grp = ph["ham"][b, h * G:(h + 1) * G].astype(np.int64)
            valid = shared["ham"][b, h] != 0xFFFF
            assert ((grp == 0xFFFF).all(axis=0) == ~valid).all()
            assert (grp[:, valid].sum(axis=0) == shared["ham"][b, h, valid]).all()
    assert np.abs(ph["out"] - shared["out"]).max() <= 1e-12


def test_per_head_with_one_head_per_group_is_the_plain_step(oracle_mod):
    wl = WORKLOADS["tiny"].with_(n_q_heads=2)
    d = make_layer(wl)
    d["Q"] = np.ascontiguousarray(d["Q"][:, :2])
    a = run(oracle_mod, wl, d)[3]
    m = run(oracle_mod, wl.with_(per_head=True), d)[3]
    for k in ("score", "pages", "ham", "sel", "k_eff", "out"):
        assert (a[k] == m[k]).all(), k
