"""The C ABI on the host (no GPU needed): symbols, problem checks, workspace sizing, host planner, metadata checks."""
import ctypes

import numpy as np
import pytest

import latent_kv_cache_absorbed_amd as lkd

OK, NULLP, SHAPE, DTYPE, MISAL, UNSUP, WS, META, HIP, STRUCT = range(10)


def mla(**kw):
    base = dict(variant="mla", batch=4, heads=128, groups=1, d_latent=512, d_rope=64, page_size=64, num_pages=100,
                max_pages_per_seq=20, q_dtype="bf16", kv_dtype="bf16", out_dtype="bf16", scale=0.07, num_splits=0)
    base.update(kw)
    return lkd.make_problem(**base)


def test_library_exports_every_declared_function():
    L = lkd.lib()
    names = lkd.header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert L.ld_abi_version() == 2


def test_status_strings():
    for s in range(10):
        assert lkd.status_string(s)
    assert "unknown" in lkd.status_string(1234)


@pytest.mark.parametrize("kw", [
    dict(variant="mla"), dict(variant="gla", groups=2, d_latent=256), dict(variant="mlra", groups=4, d_latent=128),
    dict(variant="gqa", heads=64, groups=8, d_latent=128, d_rope=0), dict(variant="mqa", heads=64, d_latent=128, d_rope=0),
    dict(variant="gta", heads=64, groups=8, d_latent=128, d_rope=0), dict(kv_dtype="fp8_e4m3"),
    dict(variant="gla", groups=2, d_latent=256, kv_dtype="fp8_e4m3"),
    dict(heads=16, d_latent=64, d_rope=16, q_dtype="f32", kv_dtype="f32", out_dtype="f32"),
    dict(out_dtype="f32"), dict(batch=0), dict(num_splits=7), dict(q_len=2), dict(q_len=16),
    dict(variant="mqa", heads=64, d_latent=512, d_rope=0, q_len=3), dict(q_len=2, kv_dtype="fp8_e4m3"),
    dict(variant="gla", groups=2, d_latent=256, q_len=2), dict(variant="gqa", heads=64, groups=8, d_latent=128,
                                                               d_rope=0, q_len=3),
    dict(variant="mlra", groups=4, d_latent=128, q_len=2)])
def test_supported_problems_check_ok(kw):
    p = mla(**kw)
    assert lkd.check_problem(p) == OK
    assert lkd.workspace_size(p) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), SHAPE), (dict(heads=0), SHAPE), (dict(variant="mla", groups=2), SHAPE),
    (dict(variant="gla", groups=3, d_latent=256), SHAPE), (dict(variant="gqa", heads=64, groups=8, d_latent=128), SHAPE),
    (dict(d_rope=0), SHAPE), (dict(page_size=0), SHAPE), (dict(num_pages=0), SHAPE), (dict(num_splits=-2), SHAPE),
    (dict(scale=float("nan")), SHAPE), (dict(scale=0.0), SHAPE), (dict(scale=-0.1), SHAPE), (dict(max_pages_per_seq=1 << 20, page_size=1 << 12), SHAPE),
    (dict(q_dtype="f32"), DTYPE), (dict(kv_dtype="f32"), DTYPE), (dict(out_dtype="fp8_e4m3"), DTYPE),
    (dict(variant="gqa", heads=64, groups=8, d_latent=128, d_rope=0, kv_dtype="fp8_e4m3"), DTYPE),
    (dict(d_latent=384), UNSUP), (dict(d_rope=32), UNSUP), (dict(heads=256), UNSUP),
    (dict(q_dtype="f32", kv_dtype="f32", out_dtype="f32"), UNSUP),
    (dict(q_len=0), SHAPE), (dict(q_len=17), SHAPE),
])
def test_bad_problems_rejected(kw, status):
    assert lkd.check_problem(mla(**kw)) == status


def test_workspace_grows_with_query_tokens():
    # partial blocks and combine pieces per unit scale with the query tokens (one work group each)
    assert lkd.workspace_size(mla(q_len=4)) > lkd.workspace_size(mla(q_len=1))


def test_struct_size_guard():
    p = mla()
    p.struct_size = 4
    assert lkd.check_problem(p) == STRUCT


def test_decode_rejects_before_touching_memory():
    """Host-checkable errors return before anything is queued (fake pointers are never dereferenced)."""
    L = lkd.lib()
    p = mla()
    cache = lkd.KVCache(0x10000, None, None, None)
    good = ctypes.c_void_p(0x20000)
    ws = lkd.workspace_size(p)
    args = lambda q=good, qr=good, bt=good, out=good, w=good, wsz=ws: (  # noqa: E731
        ctypes.byref(p), q, qr, ctypes.byref(cache), bt, good, out, good, w, wsz, None)
    assert L.ld_latent_decode(*args(q=None)) == NULLP
    assert L.ld_latent_decode(*args(qr=None)) == NULLP
    assert L.ld_latent_decode(*args(q=ctypes.c_void_p(0x20008))) == MISAL
    assert L.ld_latent_decode(*args(w=ctypes.c_void_p(0x20010))) == MISAL
    assert L.ld_latent_decode(*args(wsz=ws - 1)) == WS
    bad = mla(d_latent=384)
    assert L.ld_latent_decode(ctypes.byref(bad), good, good, ctypes.byref(cache), good, good, good, good, good, ws,
                              None) == UNSUP
    fp8 = mla(kv_dtype="fp8_e4m3")
    assert L.ld_latent_decode(ctypes.byref(fp8), good, good, ctypes.byref(cache), good, good, good, good, good, ws,
                              None) == NULLP          # rope / scale pools missing
    gqa = mla(variant="gqa", heads=64, groups=8, d_latent=128, d_rope=0)
    assert L.ld_latent_decode(ctypes.byref(gqa), good, None, ctypes.byref(cache), good, good, good, good, good, ws,
                              None) == NULLP          # V pool missing
    empty = mla(batch=0)
    assert L.ld_latent_decode(ctypes.byref(empty), None, None, None, None, None, None, None, None, 0, None) == OK


def test_combine_rejects_bad_arguments():
    L = lkd.lib()
    g = ctypes.c_void_p(0x10000)
    assert L.ld_split_kv_combine(4, 6, 2, g, g, g, 0, g, g, None) == SHAPE          # d_v not a multiple of 4
    assert L.ld_split_kv_combine(4, 8, 0, g, g, g, 0, g, g, None) == SHAPE
    assert L.ld_split_kv_combine(4, 8, 2, g, g, g, 2, g, g, None) == DTYPE
    assert L.ld_split_kv_combine(4, 8, 2, None, g, g, 0, g, g, None) == NULLP
    assert L.ld_split_kv_combine(4, 8, 2, ctypes.c_void_p(0x10004), g, g, 0, g, g, None) == MISAL
    assert L.ld_split_kv_combine(0, 8, 2, None, None, None, 0, None, None, None) == OK


def test_append_rejects_before_touching_memory():
    L = lkd.lib()
    g = ctypes.c_void_p(0x10000)
    cache = lkd.KVCache(0x20000, None, None, None)
    call = lambda p, c=g, kr=g, bt=g, sl=g, cch=cache, base=10000.0: L.ld_cache_append(  # noqa: E731
        ctypes.byref(p), c, kr, bt, sl, ctypes.byref(cch), base, None)
    assert call(mla(), c=None) == NULLP
    assert call(mla(), kr=None) == NULLP
    assert call(mla(), c=ctypes.c_void_p(0x10008)) == MISAL
    assert call(mla(), base=0.0) == SHAPE
    assert call(mla(), base=float("nan")) == SHAPE
    assert call(mla(d_rope=63)) == SHAPE
    assert call(mla(q_dtype="fp8_e4m3")) == DTYPE
    assert call(mla(variant="gqa", heads=64, groups=8, d_latent=128, d_rope=0)) == UNSUP
    assert call(mla(kv_dtype="fp8_e4m3")) == NULLP                 # rope / scale pools missing
    p = mla()
    p.struct_size = 4
    assert call(p) == STRUCT
    assert call(mla(batch=0), c=None, kr=None, bt=None, sl=None) == OK


def test_projection_rejects_bad_arguments():
    L = lkd.lib()
    g = ctypes.c_void_p(0x10000)
    assert L.ld_head_projection(4, 2, 48, 32, g, g, g, 1, None) == SHAPE       # n not a multiple of 32
    assert L.ld_head_projection(4, 2, 64, 40, g, g, g, 1, None) == SHAPE       # k not a multiple of 16
    assert L.ld_head_projection(4, 0, 64, 32, g, g, g, 1, None) == SHAPE
    assert L.ld_head_projection(4, 2, 64, 32, g, g, g, 2, None) == DTYPE       # fp8 output
    assert L.ld_head_projection(4, 2, 64, 32, None, g, g, 1, None) == NULLP
    assert L.ld_head_projection(4, 2, 64, 32, g, ctypes.c_void_p(0x10008), g, 1, None) == MISAL
    assert L.ld_head_projection(0, 2, 64, 32, None, None, None, 1, None) == OK


def test_workspace_grows_with_forced_splits():
    assert lkd.workspace_size(mla(num_splits=16)) > lkd.workspace_size(mla(num_splits=1))


# ---------------------------------------------------------------------------------------------
# host planner invariants
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("lens,splits,cus", [
    ([4096] * 64, 0, 256), ([131072], 0, 256), ([1048576], 0, 256), ([0, 1, 63, 64, 65, 5000], 0, 256),
    ([0, 0, 0], 0, 256), ([1000, 7], 3, 256), ([1, 2, 3], 8, 4), (list(range(0, 70000, 997)), 0, 80),
])
def test_planner_covers_every_token_once(lens, splits, cus):
    B = len(lens)
    p = mla(batch=B, num_splits=splits, max_pages_per_seq=max(1, (max(lens) + 63) // 64), num_pages=10 ** 6)
    chunk, units, ns, first = lkd.plan_host(p, np.array(lens, np.int32), cus)
    assert units == int(ns.sum())
    assert list(first) == list(np.concatenate([[0], np.cumsum(ns)[:-1]])) if B else True
    for b, L in enumerate(lens):
        if L == 0:
            assert ns[b] == 0
            continue
        ck = chunk if splits == 0 else max(64, -(-(-(-L // splits)) // 64) * 64)
        assert ck % 64 == 0 and ck >= 64
        bounds = [(s * ck, min(L, (s + 1) * ck)) for s in range(ns[b])]
        assert bounds[0][0] == 0 and bounds[-1][1] == L
        assert all(a < e for a, e in bounds)                       # no empty unit
        assert all(bounds[i][1] == bounds[i + 1][0] for i in range(len(bounds) - 1))
        if splits:
            assert ns[b] <= splits
    if splits == 0:
        # bound the workspace is sized for: units <= target + B, with target <= cus
        assert units <= cus + B


def test_planner_balances_one_long_sequence():
    p = mla(batch=1, max_pages_per_seq=16384, num_pages=16385)
    chunk, units, ns, _ = lkd.plan_host(p, np.array([1048576], np.int32), 256)
    assert units == 256 and chunk == 4096


def test_planner_fills_the_chip_in_one_round_for_ragged_lengths():
    # ragged lengths: the chunk is the smallest page multiple giving at most one unit per CU
    lens = np.random.default_rng(7).integers(1024, 65537, size=64).astype(np.int32)
    p = mla(batch=64, max_pages_per_seq=1024, num_pages=64 * 1024 + 1)
    chunk, units, ns, _ = lkd.plan_host(p, lens, 256)
    assert units <= 256 and chunk % 64 == 0
    smaller = chunk - 64
    assert smaller < 64 or int(np.sum(-(-lens.astype(np.int64) // smaller))) > 256


def test_planner_splits_batch_decode_across_the_chip():
    p = mla(batch=64, max_pages_per_seq=64, num_pages=4097)
    chunk, units, ns, _ = lkd.plan_host(p, np.full(64, 4096, np.int32), 256)
    assert chunk == 1024 and units == 256 and set(ns) == {4}


# ---------------------------------------------------------------------------------------------
# metadata validation
# ---------------------------------------------------------------------------------------------
def test_validate_metadata():
    p = mla(batch=2, num_pages=10, max_pages_per_seq=3)
    bt = np.array([[0, 1, 2], [3, 4, 99]], np.int32)      # 99 is unused by a 128-token sequence
    assert lkd.validate_metadata(p, bt, np.array([192, 128], np.int32)) == OK
    assert lkd.validate_metadata(p, bt, np.array([192, 129], np.int32)) == META    # now page 99 is used
    assert lkd.validate_metadata(p, bt, np.array([193, 0], np.int32)) == META      # longer than capacity
    assert lkd.validate_metadata(p, bt, np.array([-1, 0], np.int32)) == META
    bt[0, 0] = -3
    assert lkd.validate_metadata(p, bt, np.array([5, 0], np.int32)) == META


def test_noalloc_rejects_oversized_problems_before_touching_the_device():
    """ld_latent_decode_noalloc checks the problem's workspace against its fixed array first: a problem
    that needs more returns LD_ERR_WORKSPACE_TOO_SMALL with no device call (so this runs without a GPU)."""
    import ctypes

    import numpy as np

    import latent_kv_cache_absorbed_amd as lkd
    p = lkd.make_problem("mla", 64, 128, 1, 512, 64, 64, 4097, 64, "bf16", "bf16", "bf16", 0.07, q_len=4)
    assert lkd.workspace_size(p) > lkd.NOALLOC_SCRATCH_BYTES
    buf = np.zeros(1024, np.uint8)
    base = buf.ctypes.data + (-buf.ctypes.data) % 256
    ptr = ctypes.c_void_p(base)
    cache = lkd.KVCache(base, None, None, None)
    st = lkd.lib().ld_latent_decode_noalloc(ctypes.byref(p), ptr, ptr, ctypes.byref(cache), ptr, ptr, ptr, ptr, None)
    assert st == 6
    bad = lkd.make_problem("mla", 1, 128, 2, 512, 64, 64, 4, 4, "bf16", "bf16", "bf16", 0.07)   # MLA with 2 groups
    assert lkd.lib().ld_latent_decode_noalloc(ctypes.byref(bad), ptr, ptr, ctypes.byref(cache), ptr, ptr, ptr, ptr,
                                              None) == 2
