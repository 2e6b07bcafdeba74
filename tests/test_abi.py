"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes buffers, and rejects bad arguments on the host before
anything is enqueued (all pointers below are fake; no call here reaches a
kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hhr.h")


@pytest.fixture(scope="module")
def hsa():
    import hash_sparse_attention_amd as h
    if not os.path.exists(h.LIB_PATH):
        pytest.fail("libhhr.so is not built: run __graft_entry__.build()")
    return h


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hhr_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(hsa):
    names = declared_functions()
    assert len(names) >= 14
    L = ctypes.CDLL(hsa.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(hsa.EXPORTED)


def test_version_and_status_strings(hsa):
    L = hsa.lib()
    assert L.hhr_abi_version() == 8
    for code, name in hsa.STATUS.items():
        assert L.hhr_status_str(code).decode() == name


def dims(**kw):
    import hash_sparse_attention_amd as h
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, page_size=16, hash_bits=128,
                max_ctx=131072, bf16=True)
    base.update(kw)
    return h.make_dims(**base)


FAKE = ctypes.c_void_p(0x10000)           # 64 KiB aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10004)


def call_decode(h, d, max_keep=820, top_k=4096, ws_bytes=None, ws=FAKE, q=FAKE, sel=None):
    L = h.lib()
    nbytes = L.hhr_decode_workspace_bytes(ctypes.byref(d), max_keep, top_k) if ws_bytes is None else ws_bytes
    return L.hhr_decode_step(ctypes.byref(d), q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, max_keep, top_k,
                             0.0, FAKE, sel, ws, nbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 7), (dict(head_dim=256), 7), (dict(hash_bits=192), 7), (dict(hash_bits=32), 7),
    (dict(page_size=0), 7), (dict(page_size=128), 7), (dict(page_size=24), 7), (dict(n_q_heads=36), 2), (dict(n_q_heads=4), 2),
    (dict(n_q_heads=72), 7), (dict(batch=0), 2), (dict(max_ctx=0), 2), (dict(max_ctx=(1 << 26) + 1), 2),
])
def test_bad_dims_rejected(hsa, kw, status):
    d = dims(**kw)
    assert call_decode(hsa, d, ws_bytes=1 << 30) == status
    assert hsa.lib().hhr_last_error().decode()
    assert hsa.lib().hhr_meta_bytes(ctypes.byref(d)) == 0


def test_bad_dtype(hsa):
    d = dims()
    d.kv_dtype = 7
    assert call_decode(hsa, d, ws_bytes=1 << 30) == 3


def test_bad_meta_dtype_and_meta_bytes(hsa):
    L = hsa.lib()
    d = dims()
    d.meta_dtype = 5
    assert call_decode(hsa, d, ws_bytes=1 << 30) == 3
    assert L.hhr_meta_bytes(ctypes.byref(d)) == 0
    f32, b16 = dims(), dims(meta_bf16=True)
    # fp32 meta: B * Hkv * NPB * 64 pages * D * (max, min) * 4 bytes; bf16 meta is half of it
    assert L.hhr_meta_bytes(ctypes.byref(f32)) == 1 * 8 * 128 * 64 * 128 * 2 * 4
    assert L.hhr_meta_bytes(ctypes.byref(b16)) * 2 == L.hhr_meta_bytes(ctypes.byref(f32))


def test_meta_layout_checked_and_sized_like_interleaved(hsa):
    L = hsa.lib()
    d = dims()
    d.meta_layout = 2
    assert call_decode(hsa, d, ws_bytes=1 << 30) == 6  # HHR_E_RANGE
    assert "meta_layout" in L.hhr_last_error().decode()
    assert L.hhr_meta_bytes(ctypes.byref(d)) == 0
    for bf in (False, True):
        a, b = dims(meta_bf16=bf), dims(meta_bf16=bf, meta_split=True)
        assert b.meta_layout == hsa.HHR_META_SIGN_SPLIT
        assert L.hhr_meta_bytes(ctypes.byref(a)) == L.hhr_meta_bytes(ctypes.byref(b)) > 0


def test_null_and_alignment(hsa):
    L = hsa.lib()
    d = dims()
    assert L.hhr_decode_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 820, 4096, 0.0, FAKE,
                             None, FAKE, 1 << 30, None) == 1
    assert call_decode(hsa, d, q=None) == 1
    assert "Q" in L.hhr_last_error().decode()
    assert call_decode(hsa, d, q=FAKE_ODD) == 4
    assert call_decode(hsa, d, ws=ctypes.c_void_p(0x10010)) == 4  # workspace needs 256-byte alignment
    assert call_decode(hsa, d, sel=ctypes.c_void_p(0x10002)) == 4


@pytest.mark.parametrize("max_keep,top_k", [(0, 10), (8193, 10), (10, 0), (10, -3)])
def test_selection_sizes_rejected(hsa, max_keep, top_k):
    d = dims()
    assert call_decode(hsa, d, max_keep=max_keep, top_k=top_k, ws_bytes=1 << 30) == 6
    assert hsa.lib().hhr_decode_workspace_bytes(ctypes.byref(d), max_keep, top_k) == 0


def test_workspace_too_small(hsa):
    d = dims()
    need = hsa.lib().hhr_decode_workspace_bytes(ctypes.byref(d), 820, 4096)
    assert call_decode(hsa, d, ws_bytes=need - 1) == 5
    assert str(need) in hsa.lib().hhr_last_error().decode()


def test_encode_validation(hsa):
    L = hsa.lib()
    d = dims()
    assert L.hhr_encode_cache(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, None) == 6
    assert L.hhr_encode_cache(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 131073, FAKE, FAKE, None) == 6
    assert L.hhr_encode_cache(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE, None) == 1
    assert L.hhr_encode_cache(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE_ODD, FAKE, None) == 4
    # max_count = 0 is a valid no-op that enqueues nothing
    assert L.hhr_encode_cache(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None) == 0
    assert L.hhr_last_error().decode() == ""


def test_stage_validation(hsa):
    L = hsa.lib()
    d = dims()
    n = L.hhr_decode_workspace_bytes(ctypes.byref(d), 820, 4096)
    assert L.hhr_stage_qprep(ctypes.byref(d), None, FAKE, FAKE, 820, 4096, FAKE, n, None) == 1
    assert L.hhr_stage_page_bounds(ctypes.byref(d), FAKE, FAKE, 820, 4096, FAKE, n - 1, None) == 5
    assert L.hhr_stage_select_pages(ctypes.byref(d), FAKE, None, 820, 4096, FAKE, n, None) == 1
    assert L.hhr_stage_select_keys(ctypes.byref(d), FAKE, FAKE, 0, 4096, None, FAKE, n, None) == 6
    assert L.hhr_stage_attend(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 820, 4096, 0.0, None, None, FAKE, n,
                              None) == 1


def test_buffer_sizes(hsa):
    L = hsa.lib()
    d = dims()
    # meta: B * Hkv * ceil(ceil(T/P)/64) * 64 pages * D * (max, min) fp32
    assert L.hhr_meta_bytes(ctypes.byref(d)) == 8 * 8192 * 128 * 2 * 4
    assert L.hhr_codes_bytes(ctypes.byref(d)) == 8 * 131072 * 2 * 8
    d2 = dims(max_ctx=1000, page_size=16, batch=3, n_kv_heads=2, n_q_heads=4, head_dim=64, hash_bits=64)
    assert L.hhr_meta_bytes(ctypes.byref(d2)) == 3 * 2 * 64 * 64 * 2 * 4   # 63 pages round up to one block
    assert L.hhr_codes_bytes(ctypes.byref(d2)) == 3 * 2 * 1000 * 8


def test_workspace_layout_regions(hsa):
    d = dims(batch=3, max_ctx=5000, page_size=32, hash_bits=64)
    lay = hsa.workspace_layout(d, 17, 300)
    B, Hq, Hkv, D, P, G = 3, 32, 8, 128, 32, 4
    sizes = {"q_rot": B * Hq * D * 4, "code_q": B * Hq * 8, "q_split": B * Hkv * D * G * 16,
             "score": B * Hkv * 157 * 8, "pages": B * Hkv * 17 * 4, "n_pages": B * Hkv * 4,
             "ham": B * Hkv * 17 * P * 2, "sel": B * Hkv * 300 * 4, "k_eff": B * Hkv * 4,
             "partial": B * Hq * lay.n_splits * (D + 2) * 4, "counters": B * Hkv * 4}
    spans = sorted((getattr(lay, k), getattr(lay, k) + v) for k, v in sizes.items())
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert all(s % 256 == 0 for s, _ in spans)
    assert spans[-1][1] <= lay.total
    assert 1 <= lay.n_splits <= 300
    assert hsa.workspace_bytes(d, 17, 300) == lay.total


def test_topk_entry_validates_before_launch(hsa):
    """hhr_topk_decode_step rejects bad arguments on the host; the layout covers every region."""
    L = hsa.lib()
    d = dims()
    lay = hsa.TopkLayout()
    assert L.hhr_topk_workspace_layout(ctypes.byref(d), 4096, ctypes.byref(lay)) == 0
    B, Hkv, T = 1, 8, 131072
    assert lay.score % 256 == 0 and lay.sel % 256 == 0 and lay.k_eff % 256 == 0
    assert lay.total >= lay.score + B * Hkv * T * 8 and lay.total >= lay.sel + B * Hkv * 4096 * 4
    assert L.hhr_topk_workspace_bytes(ctypes.byref(d), 4096) == lay.total
    assert L.hhr_topk_workspace_bytes(ctypes.byref(d), 0) == 0

    def call(top_k=4096, ws_bytes=None, q=FAKE, ws=FAKE, sel=None):
        n = lay.total if ws_bytes is None else ws_bytes
        return L.hhr_topk_decode_step(ctypes.byref(d), q, FAKE, FAKE, FAKE, top_k, 0.0, FAKE, sel, ws, n, None)

    assert call(top_k=0) == 6
    assert call(q=None) == 1
    assert call(ws_bytes=lay.total - 1) == 5
    assert "workspace" in L.hhr_last_error().decode()
    assert call(ws=FAKE_ODD) == 4
    assert call(sel=ctypes.c_void_p(0x10002)) == 4
    bad = dims(head_dim=96)
    assert L.hhr_topk_decode_step(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 16, 0.0, FAKE, None, FAKE, 1 << 40,
                                  None) == 7


def test_forced_key_fields_are_validated_and_size_the_selection(hsa):
    """sink_tokens and local_window must lie in 0..max_ctx; they widen the workspace's selection rows."""
    L = hsa.lib()
    base = dims()
    wide = dims(sink_tokens=4, local_window=64)
    lay0, lay1 = hsa.WorkspaceLayout(), hsa.WorkspaceLayout()
    assert L.hhr_decode_workspace_layout(ctypes.byref(base), 820, 4096, ctypes.byref(lay0)) == 0
    assert L.hhr_decode_workspace_layout(ctypes.byref(wide), 820, 4096, ctypes.byref(lay1)) == 0
    assert lay1.k_eff - lay1.sel >= 8 * (4096 + 68) * 4 and lay1.n_splits == -(-(4096 + 68) // 128)
    assert hsa.sel_cap(wide, 4096) == 4096 + 68
    for bad in (dict(sink_tokens=-1), dict(local_window=-3), dict(local_window=131073)):
        d = dims(**bad)
        assert L.hhr_decode_workspace_bytes(ctypes.byref(d), 820, 4096) == 0
        assert call_decode(hsa, d, ws_bytes=1 << 40) == 6
        assert "sink_tokens" in L.hhr_last_error().decode()


def test_group_variant_fields_are_validated(hsa):
    """page_group and hamming_group accept 0 or 1 only, checked before anything is enqueued."""
    L = hsa.lib()
    for ok in (dict(page_group=1), dict(hamming_group=1), dict(page_group=1, hamming_group=1)):
        assert L.hhr_decode_workspace_bytes(ctypes.byref(dims(**ok)), 820, 4096) > 0
    for bad in (dict(page_group=2), dict(hamming_group=-1)):
        d = dims(**bad)
        assert L.hhr_decode_workspace_bytes(ctypes.byref(d), 820, 4096) == 0
        assert call_decode(hsa, d, ws_bytes=1 << 40) == 6
        assert "page_group" in L.hhr_last_error().decode()
