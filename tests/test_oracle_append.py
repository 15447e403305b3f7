"""Pins for the oracle's cache append: the E4M3 encoder, the per-token quantiser and the slot rule.

Each pin reaches the expected result by another route: torch's float8_e4m3fn
conversion (an independent round-to-nearest-even implementation), the decoder
round trip over every code, the format's error bound, brute force over the
code table, and the decode oracle's own addressing.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def test_encode_inverts_decode_on_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_encode_matches_torch_round_to_nearest_even():
    # every finite value, every midpoint between neighbours (the ties), and a dense random sweep
    vals = np.sort(np.unique(oracle.e4m3_decode(np.arange(0x7F))))
    mids = (vals[1:] + vals[:-1]) / 2
    r = _rng(1)
    sweep = np.concatenate([vals, mids, -vals, -mids, r.uniform(-448, 448, 20000), r.normal(0, 0.01, 5000)])
    sweep = sweep.astype(np.float32)           # the kernel's quotients are fp32 values
    ref = torch.from_numpy(sweep).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(sweep), ref)


def test_ties_go_to_the_even_code():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39); 1.1875 between 0x39 and 1.25 (0x3A)
    assert oracle.e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert oracle.e4m3_encode(np.array([1.1875]))[0] == 0x3A
    # halfway between 0 and the smallest subnormal 2^-9 goes to 0; 1.5 * 2^-9 to 2 * 2^-9
    assert oracle.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00
    assert oracle.e4m3_encode(np.array([1.5 * 2.0 ** -9]))[0] == 0x02


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([float("nan")]))


@pytest.mark.parametrize("seed,d", [(2, 512), (3, 256), (4, 64), (5, 1)])
def test_quantised_row_is_within_the_format_error_bound(seed, d):
    c = _rng(seed).normal(0, 3.0, d).astype(np.float32)
    codes, scale = oracle.quantize_row_e4m3(c)
    assert scale.dtype == np.float32 and scale == np.float32(np.abs(c).max() / np.float32(448))
    deq = oracle.e4m3_decode(codes) * np.float64(scale)
    # 3 mantissa bits: half a quantum is 2^-4 of the value for normals, 2^-10 * scale below 2^-6 * scale
    bound = np.maximum(np.abs(c) * 2.0 ** -4, 2.0 ** -10 * float(scale)) * (1 + 1e-6)
    assert np.all(np.abs(deq - c) <= bound)
    # the largest magnitude maps to +-448 (code 0x7E / 0xFE)
    k = int(np.argmax(np.abs(c)))
    assert codes[k] & 0x7F == 0x7E


def test_zero_row_has_unit_scale_and_zero_codes():
    codes, scale = oracle.quantize_row_e4m3(np.zeros(16, np.float32))
    assert scale == 1.0 and not codes.any()


def test_quantiser_against_brute_force_nearest():
    c = _rng(6).normal(0, 1, 300).astype(np.float32)
    codes, scale = oracle.quantize_row_e4m3(c)
    y = np.clip(c / scale, -448, 448).astype(np.float64)
    table = oracle.e4m3_decode(np.arange(0x7F))
    for yi, ci in zip(y, codes):
        dist = np.abs(table - abs(yi))
        best = np.flatnonzero(dist == dist.min())
        pick = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert (ci & 0x7F) == pick and bool(ci & 0x80) == (math.copysign(1, yi) < 0)


def test_appended_token_is_the_last_row_the_decode_reads():
    r = _rng(7)
    page, B, D, dr = 16, 3, 8, 4
    lens = np.array([1, 17, 40])
    table = r.permutation(12).reshape(B, 4)
    c = r.normal(size=(B, D))
    kr = r.normal(size=(B, dr))
    pool = np.full((12, page, D + dr), np.nan)
    for w in oracle.cache_append(c, kr, table, lens, page_size=page, fp8=False):
        pool[w["page"], w["slot"]] = np.concatenate([w["latent"], w["rope"]])
    for b in range(B):
        last = oracle.logical_rows(pool, table[b], lens[b], page)[-1]
        np.testing.assert_array_equal(last[:D], c[b])
        np.testing.assert_allclose(last[D:], oracle.rope(kr[b], lens[b] - 1), rtol=0, atol=0)
    # a zero-length sequence writes nothing
    assert len(oracle.cache_append(c, kr, table, np.array([0, 5, 0]), page_size=page, fp8=False)) == 1


def test_append_writes_only_where_the_metadata_points():
    """Lengths above the block table's capacity and page entries outside the pool get no write."""
    c = np.ones((4, 8))
    kr = np.zeros((4, 2))
    table = np.array([[0, 1], [2, -1], [3, 4], [5, 7]], np.int32)
    lens = np.array([5, 12, 17, 9], np.int32)        # page 4: b1 -> entry -1, b2 -> 17 > 2 * 8, b3 -> 7 >= 6
    w = oracle.cache_append(c, kr, table, lens, page_size=8, fp8=False, num_pages=6)
    assert [x["b"] for x in w] == [0]
    assert (w[0]["page"], w[0]["slot"]) == (0, 4)
    # without a pool size only the capacity rule applies
    w = oracle.cache_append(c, kr, table, lens, page_size=8, fp8=False)
    assert [x["b"] for x in w] == [0, 1, 3]
