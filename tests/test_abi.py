"""The C-ABI library loads, exports every declared entry point, and rejects
bad configurations on the host (no GPU needed: nothing here reaches HIP)."""

import ctypes
import os
import re

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd.build import LIB_PATH, ROOT

HEADER = os.path.join(ROOT, "include", "segkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from long_context_serving_amd.build import build
        build()
    return S.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(segkv_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(S.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {LIB_PATH}").read()
    exported = set(re.findall(r" T (segkv_\w+)", out))
    assert exported == set(declared_functions())


def _cfg(**kw):
    base = dict(num_layers=1, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64, max_seqs=4,
                num_pages=100)
    base.update(kw)
    if "head_window" not in base:  # one global head, the rest local, in every layer
        n = max(base["num_layers"], 1) * max(base["num_kv_heads"], 1)
        base["head_window"] = [0 if i % base["num_kv_heads"] == 0 else 64 for i in range(n)]
    return base


@pytest.mark.parametrize("kw,msg", [
    (dict(num_q_heads=6, num_kv_heads=4), "multiple"),
    (dict(head_dim=96), "head_dim"),
    (dict(page_size=48), "page_size"),
    (dict(max_seqs=0), "max_seqs"),
    (dict(num_pages=0), "num_pages"),
    (dict(num_pages=2 ** 31), "num_pages"),
    (dict(head_window=[0, -1]), "head_window"),
    (dict(num_layers=0), "num_layers"),
    (dict(softmax_scale=-1.0), "softmax_scale"),
    (dict(rope_theta=-1.0), "rope_theta"),
    (dict(rope_theta=1.0), "rope_theta"),
    (dict(rope_style=2), "rope_style"),
    (dict(rope_dims=8), "rope_dims"),
    (dict(rope_dims=136), "rope_dims"),
    (dict(head_dim=64, rope_dims=80), "rope_dims"),
])
def test_create_rejects_bad_config(lib, kw, msg):
    with pytest.raises(S.SegKVError) as e:
        S.SegKV(planning=True, **_cfg(**kw))
    assert e.value.code == S.SEGKV_E_INVAL
    assert msg in str(e.value)


def test_create_rejects_half_set_pools(lib):
    cfg = S._Config()
    cfg.num_layers, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim = 1, 2, 2, 64
    cfg.page_size, cfg.max_seqs, cfg.num_pages = 16, 1, 4
    win = (ctypes.c_int32 * 2)(0, 0)
    cfg.head_window = ctypes.cast(win, ctypes.POINTER(ctypes.c_int32))
    cfg.k_pool = 0x1000  # never dereferenced: rejected before any use
    h = ctypes.c_void_p()
    assert lib.segkv_create(ctypes.byref(cfg), ctypes.byref(h)) == S.SEGKV_E_INVAL
    assert h.value is None
    assert b"both" in lib.segkv_last_error(None)


def test_planning_context_refuses_device_calls(lib):
    kv = S.SegKV(planning=True, **_cfg())
    ids = (ctypes.c_int32 * 1)(0)
    cu = (ctypes.c_int32 * 2)(0, 1)
    assert lib.segkv_prefill(kv._h, 0, 1, ids, cu, None, None, None) == S.SEGKV_E_STATE
    assert lib.segkv_decode(kv._h, 0, 1, ids, None, None, None) == S.SEGKV_E_STATE
    assert lib.segkv_set_timing(kv._h, 1) == S.SEGKV_E_STATE
    # an append carrying device pointers is refused too, before any state change
    nq = (ctypes.c_int32 * 1)(0)
    assert lib.segkv_append_pages(kv._h, 0, 1, ids, cu, nq, 0x1000, 0x1000) == S.SEGKV_E_STATE
    assert kv.page_table(0, 0, 0)[1] == 0


def test_binding_checks_the_window_table_size(lib):
    with pytest.raises(ValueError):
        S.SegKV(planning=True, **_cfg(num_layers=2, head_window=[0, 64]))


def test_null_context_is_rejected(lib):
    assert lib.segkv_release(None, 0) == S.SEGKV_E_INVAL
    assert lib.segkv_free_pages(None) == S.SEGKV_E_INVAL
    lib.segkv_destroy(None)


def test_tuning_knobs(lib):
    kv = S.SegKV(planning=True, **_cfg())
    kv.set_tuning(S.TUNE_DECODE_MIN_PAGES, 8)
    kv.set_tuning(S.TUNE_PREFILL_SPLIT_TILES, 0)
    for v in (0, 1, 2, 3, 4, 5):
        kv.set_tuning(S.TUNE_PREFILL_KERNEL, v)
    with pytest.raises(S.SegKVError):
        kv.set_tuning(S.TUNE_PREFILL_KERNEL, 6)
    with pytest.raises(S.SegKVError):
        kv.set_tuning(7, 1)


def test_relocation_offsets_on_a_planning_context(lib):
    kv = S.SegKV(planning=True, **_cfg(num_layers=2, head_window=[0, 64, 0, 64], rope_style=1, rope_dims=64))
    kv.set_relocation(1, [[5, 0], [0, -9]])
    kv.set_relocation(1, None)
    kv.set_relocation(3, np.zeros((2, 2)))
    with pytest.raises(S.SegKVError) as e:
        kv.set_relocation(4, None)
    assert e.value.code == S.SEGKV_E_RANGE
    with pytest.raises(ValueError):
        kv.set_relocation(0, [1, 2, 3])
    with pytest.raises(ValueError):
        kv.set_relocation(0, [[2 ** 31, 0], [0, 0]])
    assert kv.release(1) == S.SEGKV_OK


def test_merge_refused_in_planning_context(lib):
    kv = S.SegKV(planning=True, **_cfg())
    assert lib.segkv_merge(kv._h, 4, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None) == S.SEGKV_E_STATE
    assert lib.segkv_merge(None, 4, None, None, None, None, None, None, None) == S.SEGKV_E_INVAL


def test_scores_and_topk_refused_in_planning_context(lib):
    kv = S.SegKV(planning=True, **_cfg())
    ids = (ctypes.c_int32 * 1)(0)
    cu = (ctypes.c_int32 * 2)(0, 1)
    k = (ctypes.c_int32 * 1)(1)
    assert lib.segkv_token_scores(kv._h, 0, 1, ids, cu, None, None, None) == S.SEGKV_E_STATE
    assert lib.segkv_topk(kv._h, 1, cu, None, k, None) == S.SEGKV_E_STATE


def _ws(lib, q_tokens, **kw):
    c = _cfg(**kw)
    return S.SegKV.workspace_bytes_for(c["num_layers"], c["num_q_heads"], c["num_kv_heads"], c["head_dim"],
                                       c["page_size"], c["max_seqs"], c["num_pages"], c["head_window"], q_tokens)


def test_workspace_bytes_bound(lib):
    n0 = _ws(lib, 0)
    n1 = _ws(lib, 4096)
    n2 = _ws(lib, 65536)
    assert 0 < n0 <= n1 <= n2
    # more sequences, pages or a wider head dim never need less
    assert _ws(lib, 4096, max_seqs=64) >= n1
    assert _ws(lib, 4096, num_pages=100_000) >= n1 + 4 * (100_000 - 100) - 16
    assert _ws(lib, 4096, head_dim=64) <= n1
    # a global head's token-score partial rows grow with the square of the chunk
    g = _ws(lib, 65536, head_window=[0, 0])
    loc = _ws(lib, 65536, head_window=[64, 64])
    assert g > loc
    # the prefill's split partials alone: two per resident workgroup of >= 1 CU, 256 rows x (D + 1) fp32
    assert n0 >= 2 * 256 * 129 * 4


@pytest.mark.parametrize("kw", [dict(num_q_heads=6, num_kv_heads=4), dict(head_dim=96), dict(max_seqs=0),
                                dict(num_pages=0), dict(num_layers=0)])
def test_workspace_bytes_of_invalid_config_is_zero(lib, kw):
    assert _ws(lib, 16, **kw) == 0


def test_workspace_bytes_of_negative_tokens_is_zero(lib):
    assert _ws(lib, -1) == 0


def test_create_rejects_bad_workspace(lib):
    import ctypes as ct
    c = _cfg()
    win, win_p = S._i32(c["head_window"])
    cfg = S._Config()
    cfg.num_layers, cfg.num_q_heads, cfg.num_kv_heads = c["num_layers"], c["num_q_heads"], c["num_kv_heads"]
    cfg.head_dim, cfg.page_size, cfg.max_seqs, cfg.num_pages = c["head_dim"], c["page_size"], c["max_seqs"], c["num_pages"]
    cfg.head_window = win_p
    h = ct.c_void_p()
    cfg.max_batch_q_tokens = -5
    assert lib.segkv_create(ct.byref(cfg), ct.byref(h)) == S.SEGKV_E_INVAL
    assert b"max_batch_q_tokens" in lib.segkv_last_error(None)
    cfg.max_batch_q_tokens = 0
    # a workspace given with a bad alignment or no size (checked before any device use)
    cfg.workspace, cfg.workspace_bytes = 0x1001, 4096
    cfg.k_pool = cfg.v_pool = 0x10000
    assert lib.segkv_create(ct.byref(cfg), ct.byref(h)) == S.SEGKV_E_INVAL
    assert b"aligned" in lib.segkv_last_error(None)
    cfg.workspace, cfg.workspace_bytes = 0x1000, 0
    assert lib.segkv_create(ct.byref(cfg), ct.byref(h)) == S.SEGKV_E_INVAL
    assert b"0 bytes" in lib.segkv_last_error(None)
