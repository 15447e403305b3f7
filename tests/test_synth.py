"""The seeded input generator: determinism, paging layout, poison placement, fp8 storage."""
import numpy as np
import torch

import oracle
import synth


def test_draws_are_reproducible_from_two_integers():
    a = synth.normal_tensor(synth.generator(7, 1), (3, 5), "bf16")
    b = synth.normal_tensor(synth.generator(7, 1), (3, 5), "bf16")
    c = synth.normal_tensor(synth.generator(7, 2), (3, 5), "bf16")
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_layout_covers_every_logical_page_once():
    lens = [0, 1, 64, 65, 300]
    lay = synth.plan_pages(synth.generator(1, 0), lens, 64, shuffle=True, spare_pages=2)
    used = []
    for b, L in enumerate(lens):
        n = (L + 63) // 64
        used += list(lay.block_table[b, :n])
        assert np.all(lay.block_table[b, n:] == lay.spare_pages[0])
    assert sorted(used + list(lay.spare_pages)) == list(range(lay.num_pages))
    assert lay.block_table.dtype == np.int32 and lay.seq_lens.dtype == np.int32


def test_content_does_not_depend_on_the_shuffle():
    lens = [100, 7]
    a = synth.make_inputs("mla", 2, 2, 1, 8, 4, lens, seed=3, shuffle=True, kv_dtype="f32", q_dtype="f32")
    b = synth.make_inputs("mla", 2, 2, 1, 8, 4, lens, seed=3, shuffle=False, kv_dtype="f32", q_dtype="f32")
    for s in range(2):
        ra = oracle.logical_rows(a.k_pool.numpy(), a.layout.block_table[s], lens[s], 64)
        rb = oracle.logical_rows(b.k_pool.numpy(), b.layout.block_table[s], lens[s], 64)
        np.testing.assert_array_equal(ra, rb)


def test_poison_is_exactly_the_unused_slots():
    lens = [70, 64, 3]
    inp = synth.make_inputs("mla", 3, 2, 1, 8, 4, lens, seed=4, kv_dtype="bf16")
    pool = inp.k_pool.float().numpy()
    nan_rows = np.isnan(pool).all(axis=-1)
    expect = np.zeros_like(nan_rows)
    for b, L in enumerate(lens):
        for j in range(((L + 63) // 64) * 64):
            if j >= L:
                expect[inp.layout.block_table[b, j // 64], j % 64] = True
    expect[inp.layout.spare_pages] = True
    np.testing.assert_array_equal(nan_rows, expect)
    assert not np.isnan(pool[~nan_rows]).any()


def test_fp8_storage_round_trip_and_poison():
    inp = synth.make_inputs("mla", 2, 2, 1, 512, 64, [130, 64], seed=5, kv_dtype="fp8_e4m3")
    codes = inp.k_pool.numpy()
    scales = inp.scale_pool.numpy()
    lay = inp.layout
    for b, L in enumerate([130, 64]):
        c = oracle.logical_rows(codes, lay.block_table[b], L, 64)
        s = oracle.logical_rows(scales, lay.block_table[b], L, 64)
        vals = oracle.e4m3_decode(c)
        assert np.all(np.isfinite(vals)) and np.all(np.isfinite(s)) and np.all(s > 0)
        # per-token scale puts the largest magnitude at (or next to) 448
        assert np.all(np.abs(vals).max(axis=1) >= 416.0)
    assert (codes[lay.spare_pages[0]] == 0x7F).all() and np.isnan(scales[lay.spare_pages[0]]).all()
    last = lay.block_table[0, 2]
    assert (codes[last, 2:] == 0x7F).all() and not (codes[last, :2] == 0x7F).any()


def test_fp8_quantiser_relative_error_within_half_ulp():
    # regenerate the draw the pool was built from and compare element-wise
    lay = synth.plan_pages(synth.generator(6, 0), [64], 64, shuffle=False, spare_pages=0)
    codes, scales = synth.fill_pool_e4m3(synth.generator(6, 3), lay, 512, poison=False)
    x = synth.generator(6, 3).standard_normal(64 * 512, dtype=np.float32).reshape(64, 512).astype(np.float64)
    deq = oracle.e4m3_decode(codes[0].numpy()) * scales[0].numpy().astype(np.float64)[:, None]
    y = x / scales[0].numpy().astype(np.float64)[:, None]
    normal = np.abs(y) >= 2.0 ** -6
    rel = np.abs(deq - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
