"""Pins for the CPU oracle: closed forms, identities the pages state, brute force and library routines.

None of these re-type the oracle's own formulas: each compares the oracle with
something that reaches the same number by another route.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------------------------
# closed forms of softmax attention
# ------------------------------------------------------------------------------------------------
def test_single_token_returns_its_value_and_score():
    r = _rng(1)
    q, k, v = r.normal(size=8), r.normal(size=(1, 8)), r.normal(size=(1, 5))
    o, lse = oracle.attend(q, k, v, 0.3)
    np.testing.assert_allclose(o, v[0], rtol=0, atol=1e-15)
    assert lse == pytest.approx(0.3 * float(q @ k[0]), rel=1e-15, abs=1e-15)


def test_two_tokens_weight_is_logistic_of_score_gap():
    r = _rng(2)
    q, K, V = r.normal(size=6), r.normal(size=(2, 6)), r.normal(size=(2, 3))
    scale = 0.7
    s0, s1 = scale * (K[0] @ q), scale * (K[1] @ q)
    p0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    o, lse = oracle.attend(q, K, V, scale)
    np.testing.assert_allclose(o, p0 * V[0] + (1 - p0) * V[1], rtol=1e-14, atol=1e-14)
    assert lse == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), rel=1e-14)


def test_identical_keys_average_values():
    r = _rng(3)
    L = 37
    q, k, V = r.normal(size=10), r.normal(size=10), r.normal(size=(L, 4))
    K = np.tile(k, (L, 1))
    o, lse = oracle.attend(q, K, V, 0.25)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-13, atol=1e-14)
    assert lse == pytest.approx(0.25 * float(q @ k) + math.log(L), rel=1e-14)


def test_zero_query_averages_values_with_lse_log_length():
    r = _rng(4)
    L = 50
    o, lse = oracle.attend(np.zeros(7), r.normal(size=(L, 7)), r.normal(size=(L, 3)) + 2.0, 1.0)
    assert lse == pytest.approx(math.log(L), rel=1e-15)


def test_empty_sequence():
    o, lse = oracle.attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 6)), 1.0)
    assert np.all(o == 0) and o.shape == (6,) and lse == -np.inf
    O, L = oracle.attend_heads(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 6)), 1.0)
    assert np.all(O == 0) and np.all(L == -np.inf)


def test_weights_are_a_probability_vector():
    r = _rng(5)
    L = 23
    q, K = r.normal(size=9) * 3, r.normal(size=(L, 9))
    p, _ = oracle.attend(q, K, np.eye(L), 0.5)      # V = identity exposes the weights
    assert np.all(p >= 0)
    assert abs(p.sum() - 1.0) <= 1e-12
    # weights are ordered like the scores
    s = K @ q
    assert np.all(np.diff(p[np.argsort(s)]) >= -1e-15)


def test_golden_two_token_example():
    with open(os.path.join(GOLDEN, "two_token_closed_form.json")) as f:
        g = json.load(f)
    K = np.array([[math.log(3.0) if x == "ln3" else x for x in row] for row in g["K"]], np.float64)
    o, lse = oracle.attend(np.array(g["q"]), K, np.array(g["V"]), g["scale"])
    np.testing.assert_allclose(o, g["expected_out"], rtol=1e-14)
    assert lse == pytest.approx(math.log(4.0), rel=1e-15)


def test_large_scores_do_not_overflow():
    q = np.array([1000.0, 0.0])
    K = np.array([[1.0, 0.0], [0.999, 0.0], [-5.0, 0.0]])
    o, lse = oracle.attend(q, K, np.eye(3), 1.0)
    assert np.all(np.isfinite(o)) and np.isfinite(lse)
    assert o[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-12)


# ------------------------------------------------------------------------------------------------
# brute force in 40-digit decimal arithmetic (correctly rounded exp / ln)
# ------------------------------------------------------------------------------------------------
def _decimal_attention(q, K, V, scale):
    getcontext().prec = 40
    qd = [Decimal(float(x)) for x in q]
    sc = Decimal(float(scale))
    scores = [sc * sum((Decimal(float(a)) * b for a, b in zip(row, qd)), Decimal(0)) for row in K]
    weights = [s.exp() for s in scores]
    total = sum(weights, Decimal(0))
    out = []
    for c in range(len(V[0])):
        out.append(sum((w * Decimal(float(V[j][c])) for j, w in enumerate(weights)), Decimal(0)) / total)
    return [float(x) for x in out], float(total.ln())


@pytest.mark.parametrize("seed,L,d,dv", [(10, 1, 2, 1), (11, 3, 4, 2), (12, 8, 4, 4), (13, 5, 3, 3), (14, 8, 1, 2)])
def test_decimal_brute_force(seed, L, d, dv):
    r = _rng(seed)
    q, K, V = r.normal(size=d) * 2, r.normal(size=(L, d)), r.normal(size=(L, dv))
    o, lse = oracle.attend(q, K, V, 0.6)
    od, lsed = _decimal_attention(q, K, V, 0.6)
    np.testing.assert_allclose(o, od, rtol=1e-13, atol=1e-14)
    assert lse == pytest.approx(lsed, rel=1e-13, abs=1e-14)
    O, LS = oracle.attend_heads(q[None], K, V, 0.6)
    np.testing.assert_allclose(O[0], od, rtol=1e-13, atol=1e-14)
    assert LS[0] == pytest.approx(lsed, rel=1e-13, abs=1e-14)


# ------------------------------------------------------------------------------------------------
# library routine: torch CPU fp64 scaled_dot_product_attention on the materialised q/k/v
# ------------------------------------------------------------------------------------------------
def _mla_model_inputs(seed, H=4, dn=8, dr=4, dc=16, dv=8, L=29):
    r = _rng(seed)
    return dict(q_nope=r.normal(size=(H, dn)), q_rope=r.normal(size=(H, dr)),
                W_UK=r.normal(size=(H, dn, dc)) / math.sqrt(dn), W_UV=r.normal(size=(H, dv, dc)) / math.sqrt(dc),
                C=r.normal(size=(L, dc)), KR=r.normal(size=(L, dr)))


def test_materialised_mla_matches_torch_sdpa():
    m = _mla_model_inputs(20)
    scale = 1.0 / math.sqrt(12.0)
    o, lse = oracle.mla_materialised(m["q_nope"], m["q_rope"], m["W_UK"], m["W_UV"], m["C"], m["KR"], scale)
    H = m["q_nope"].shape[0]
    qs, ks, vs = [], [], []
    for h in range(H):
        qs.append(np.concatenate([m["q_nope"][h], m["q_rope"][h]]))
        ks.append(np.concatenate([np.einsum("nc,lc->ln", m["W_UK"][h], m["C"]), m["KR"]], axis=1))
        vs.append(np.einsum("vc,lc->lv", m["W_UV"][h], m["C"]))
    q = torch.tensor(np.array(qs))[:, None, :]
    k = torch.tensor(np.array(ks))
    v = torch.tensor(np.array(vs))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[:, 0, :].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    # lse by torch's logsumexp of the same scores
    s = torch.einsum("hd,hld->hl", q[:, 0, :], k) * scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=1e-13)


# ------------------------------------------------------------------------------------------------
# identities the pages state
# ------------------------------------------------------------------------------------------------
def test_absorbed_mla_equals_materialised():
    """W_UK folded into the query gives the same attention; the latent output maps back by W_UV."""
    m = _mla_model_inputs(21, H=6, dn=8, dr=4, dc=24, dv=10, L=41)
    scale = 1.0 / math.sqrt(12.0)
    o_mat, lse_mat = oracle.mla_materialised(m["q_nope"], m["q_rope"], m["W_UK"], m["W_UV"], m["C"], m["KR"], scale)
    q_lat = oracle.absorb_query(m["q_nope"], m["W_UK"])
    # absorbed MLA = one MQA whose shared key row is [c ; kr] and whose value is c
    pool = np.concatenate([m["C"], m["KR"]], axis=1)[None]           # one page holding all 41 rows
    o_lat, lse_lat = oracle.decode_paged("mla", q_lat[None], m["q_rope"][None], pool, np.zeros((1, 1), np.int32),
                                         np.array([41]), groups=1, scale=scale, page_size=41, d_rope=4)
    o_back = np.einsum("hvc,hc->hv", m["W_UV"], o_lat[0])
    np.testing.assert_allclose(o_back, o_mat, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_lat[0], lse_mat, rtol=1e-13)


def test_absorb_query_against_explicit_sum():
    r = _rng(22)
    qn, W = r.normal(size=(3, 5)), r.normal(size=(3, 5, 7))
    got = oracle.absorb_query(qn, W)
    for h in range(3):
        for c in range(7):
            assert got[h, c] == pytest.approx(sum(qn[h, n] * W[h, n, c] for n in range(5)), rel=1e-13, abs=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    r = _rng(23)
    H, nkv, L, d = 8, 2, 19, 6
    Q, K, V = r.normal(size=(H, d)), r.normal(size=(L, nkv, d)), r.normal(size=(L, nkv, d))
    o, lse = oracle.shared_kv_attention(Q, K, V, 0.4)
    Kr = np.repeat(K, H // nkv, axis=1)          # kv head g serves query heads g*per .. g*per+per-1
    Vr = np.repeat(V, H // nkv, axis=1)
    o2, lse2 = oracle.shared_kv_attention(Q, Kr, Vr, 0.4)    # n_kv = H: plain MHA
    np.testing.assert_allclose(o, o2, rtol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14)
    for h in range(H):                            # and MHA per head is one attention each
        oh, lh = oracle.attend(Q[h], Kr[:, h], Vr[:, h], 0.4)
        np.testing.assert_allclose(o[h], oh, rtol=1e-14)


def test_mqa_equals_mha_with_identical_kv_heads():
    r = _rng(24)
    H, L, d = 5, 17, 4
    Q, K, V = r.normal(size=(H, d)), r.normal(size=(L, 1, d)), r.normal(size=(L, 1, d))
    o, lse = oracle.shared_kv_attention(Q, K, V, 0.5)
    o2, lse2 = oracle.shared_kv_attention(Q, np.tile(K, (1, H, 1)), np.tile(V, (1, H, 1)), 0.5)
    np.testing.assert_allclose(o, o2, rtol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-14)


def test_gta_is_gqa_with_value_tied_to_key():
    inp = synth.make_inputs("gta", 2, 8, 2, 16, 0, [70, 3], seed=30, kv_dtype="f32", q_dtype="f32")
    kw = dict(groups=2, scale=0.25, page_size=64)
    bt, sl = inp.layout.block_table, inp.layout.seq_lens
    kp = inp.k_pool.double().numpy()
    o1, l1 = oracle.decode_paged("gta", inp.q_lat.double().numpy(), None, kp, bt, sl, **kw)
    o2, l2 = oracle.decode_paged("gqa", inp.q_lat.double().numpy(), None, kp, bt, sl, v_pool=kp.copy(), **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def _latent_problem(variant, groups, d_lat, H=8, lens=(70, 5), seed=31, d_rope=8):
    inp = synth.make_inputs(variant, len(lens), H, groups, d_lat, d_rope, list(lens), seed=seed,
                            kv_dtype="f32", q_dtype="f32")
    return inp


def _run(inp, variant=None, groups=None, **extra):
    return oracle.decode_paged(variant or inp.variant, inp.q_lat.double().numpy(),
                               None if inp.q_rope is None else inp.q_rope.double().numpy(),
                               inp.k_pool.double().numpy(), inp.layout.block_table, inp.layout.seq_lens,
                               groups=groups or inp.groups, scale=inp.scale, page_size=inp.layout.page_size,
                               d_rope=inp.d_rope, **extra)


def test_gla_one_group_is_mla():
    inp = _latent_problem("gla", 1, 32)
    o1, l1 = _run(inp, "gla", 1)
    o2, l2 = _run(inp, "mla", 1)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_gla_two_groups_are_two_mla_problems():
    """GLA-2 = two MLA problems: heads of group g attend [c_g ; kr] with value c_g."""
    inp = _latent_problem("gla", 2, 16, H=8)
    o, l = _run(inp)
    kp = inp.k_pool.double().numpy()
    for g in range(2):
        sub = np.concatenate([kp[..., g * 16:(g + 1) * 16], kp[..., 32:]], axis=-1)
        hs = slice(4 * g, 4 * g + 4)
        og, lg = oracle.decode_paged("mla", inp.q_lat.double().numpy()[:, hs], inp.q_rope.double().numpy()[:, hs],
                                     sub, inp.layout.block_table, inp.layout.seq_lens, groups=1, scale=inp.scale,
                                     page_size=64, d_rope=8)
        np.testing.assert_array_equal(o[:, hs], og)
        np.testing.assert_array_equal(l[:, hs], lg)


def test_mlra_one_branch_is_mla():
    inp = _latent_problem("mlra", 1, 16)
    o1, l1 = _run(inp, "mlra", 1)
    o2, l2 = oracle.decode_paged("mla", inp.q_lat.double().numpy()[:, :, 0], inp.q_rope.double().numpy()[:, :, 0],
                                 inp.k_pool.double().numpy(), inp.layout.block_table, inp.layout.seq_lens, groups=1,
                                 scale=inp.scale, page_size=64, d_rope=8)
    np.testing.assert_array_equal(o1[:, :, 0], o2)
    np.testing.assert_array_equal(l1[:, :, 0], l2)


def test_mlra_absorbed_equals_materialised_branch_sum():
    """MLRA: attend per branch, then sum the branch outputs; absorbed per branch = materialised per branch."""
    r = _rng(32)
    H, G, dn, dr, dg, dv, L = 3, 4, 6, 4, 8, 5, 23
    qn, qr = r.normal(size=(H, G, dn)), r.normal(size=(H, G, dr))
    WUK = r.normal(size=(H, G, dn, dg)) / math.sqrt(dn)
    WUV = r.normal(size=(H, G, dv, dg)) / math.sqrt(dg)
    Cb, KR = r.normal(size=(G, L, dg)), r.normal(size=(L, dr))
    scale = 1.0 / math.sqrt(dn + dr)
    o_mat, lse_mat = oracle.mlra_materialised(qn, qr, WUK, WUV, Cb, KR, scale)
    # the branch sum is the sum of independent MLA attentions, one per branch
    acc = np.zeros((H, dv))
    for b in range(G):
        ob, lb = oracle.mla_materialised(qn[:, b], qr[:, b], WUK[:, b], WUV[:, b], Cb[b], KR, scale)
        acc += ob
        np.testing.assert_allclose(lse_mat[:, b], lb, rtol=1e-14)
    np.testing.assert_allclose(o_mat, acc, rtol=1e-13, atol=1e-14)
    # absorbed, paged form
    q_lat = oracle.absorb_query(qn, WUK)                                 # [H, G, dg]
    row = np.concatenate([Cb.transpose(1, 0, 2).reshape(L, G * dg), KR], axis=1)
    o_lat, lse_lat = oracle.decode_paged("mlra", q_lat[None], qr[None], row[None], np.zeros((1, 1), np.int32),
                                         np.array([L]), groups=G, scale=scale, page_size=L, d_rope=dr)
    o_back = np.einsum("hbvc,hbc->hv", WUV, o_lat[0])
    np.testing.assert_allclose(o_back, o_mat, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_lat[0], lse_mat, rtol=1e-13)
    # and the sum must differ from attending the summed latent (the pages contrast the two orders)
    o_mla_order, _ = oracle.mla_materialised(qn.sum(1), qr.sum(1), WUK.sum(1), WUV.sum(1), Cb.sum(0), KR, scale)
    assert np.max(np.abs(o_mla_order - o_mat)) > 1e-3


def test_gla_absorbed_equals_materialised():
    r = _rng(33)
    H, G, dn, dr, dg, dv, L = 4, 2, 6, 4, 8, 5, 31
    qn, qr = r.normal(size=(H, dn)), r.normal(size=(H, dr))
    WUK, WUV = r.normal(size=(H, dn, dg)), r.normal(size=(H, dv, dg))
    Cg, KR = r.normal(size=(G, L, dg)), r.normal(size=(L, dr))
    o_mat, lse_mat = oracle.gla_materialised(qn, qr, WUK, WUV, Cg, KR, 0.3)
    q_lat = oracle.absorb_query(qn, WUK)
    row = np.concatenate([Cg.transpose(1, 0, 2).reshape(L, G * dg), KR], axis=1)
    o_lat, lse_lat = oracle.decode_paged("gla", q_lat[None], qr[None], row[None], np.zeros((1, 1), np.int32),
                                         np.array([L]), groups=G, scale=0.3, page_size=L, d_rope=dr)
    np.testing.assert_allclose(np.einsum("hvc,hc->hv", WUV, o_lat[0]), o_mat, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_lat[0], lse_mat, rtol=1e-13)
    # heads 0,1 use group 0 only: changing group 1's latent leaves them unchanged
    Cg2 = Cg.copy()
    Cg2[1] += 1.0
    o2, _ = oracle.gla_materialised(qn, qr, WUK, WUV, Cg2, KR, 0.3)
    np.testing.assert_array_equal(o2[:2], o_mat[:2])
    assert np.max(np.abs(o2[2:] - o_mat[2:])) > 1e-6


# ------------------------------------------------------------------------------------------------
# split-KV: any partition merged by the lse rule equals the single pass
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("bounds", [[(0, 10), (10, 64)], [(0, 1), (1, 2), (2, 64)], [(0, 32), (32, 32), (32, 64)],
                                    [(0, 64)], [(0, 5), (5, 17), (17, 40), (40, 64)]])
def test_split_then_combine_equals_single_pass(bounds):
    r = _rng(40)
    q, K, V = r.normal(size=12) * 2, r.normal(size=(64, 12)), r.normal(size=(64, 7))
    o, lse = oracle.attend(q, K, V, 0.4)
    parts = oracle.attend_split(q, K, V, 0.4, bounds)
    oc, lc = oracle.combine_partials([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(oc, o, rtol=1e-13, atol=1e-14)
    assert lc == pytest.approx(lse, rel=1e-14)


def test_two_identical_halves_add_log_two():
    r = _rng(41)
    q, K, V = r.normal(size=5), r.normal(size=(9, 5)), r.normal(size=(9, 3))
    o, lse = oracle.attend(q, K, V, 1.0)
    oc, lc = oracle.combine_partials([o, o], [lse, lse])
    np.testing.assert_allclose(oc, o, rtol=1e-15)
    assert lc == pytest.approx(lse + math.log(2.0), rel=1e-15)
    oe, le = oracle.combine_partials([o, np.zeros(3)], [lse, -np.inf])     # an empty part changes nothing
    np.testing.assert_allclose(oe, o, rtol=1e-15)
    assert le == lse
    o0, l0 = oracle.combine_partials([np.zeros(3)], [-np.inf])
    assert np.all(o0 == 0) and l0 == -np.inf
    # no parts at all is the attention of an empty sequence
    oz, lz = oracle.combine_partials(np.zeros((0, 3)), np.zeros(0))
    oa, la = oracle.attend(q, K[:0], V[:0], 1.0)
    np.testing.assert_array_equal(oz, oa)
    assert lz == la == -np.inf


# ------------------------------------------------------------------------------------------------
# paging: the oracle reads logically, so the physical placement does not matter
# ------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("variant,groups,d,dr", [("mla", 1, 32, 8), ("gqa", 2, 16, 0)])
def test_shuffled_and_identity_tables_agree(variant, groups, d, dr):
    lens = [130, 64, 1, 0, 200]
    a = synth.make_inputs(variant, 5, 4, groups, d, dr, lens, seed=50, shuffle=True, kv_dtype="f32", q_dtype="f32")
    b = synth.make_inputs(variant, 5, 4, groups, d, dr, lens, seed=50, shuffle=False, kv_dtype="f32", q_dtype="f32")
    assert not np.array_equal(a.layout.block_table, b.layout.block_table)
    oa, la = _run(a, v_pool=None if a.v_pool is None else a.v_pool.double().numpy())
    ob, lb = _run(b, v_pool=None if b.v_pool is None else b.v_pool.double().numpy())
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)
    assert np.all(np.isfinite(oa)) and np.all(oa[3] == 0) and np.all(la[3] == -np.inf)


def test_poisoned_slots_are_never_read():
    inp = synth.make_inputs("mla", 3, 4, 1, 16, 8, [65, 1, 127], seed=51, kv_dtype="f32", q_dtype="f32")
    assert np.isnan(inp.k_pool.numpy()).any()
    o, l = _run(inp)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def test_logical_rows_follow_the_block_table():
    pool = np.arange(4 * 3).reshape(4, 3)       # 4 pages of 3 slots; value = 3*page + slot
    rows = oracle.logical_rows(pool, np.array([2, 0, 3]), 7, 3)
    assert list(rows) == [6, 7, 8, 0, 1, 2, 9]


# ------------------------------------------------------------------------------------------------
# RoPE invariants (flavour is a reading; these hold for any rotation-pair RoPE)
# ------------------------------------------------------------------------------------------------
def test_rope_invariants():
    r = _rng(60)
    x, y = r.normal(size=64), r.normal(size=64)
    np.testing.assert_allclose(oracle.rope(x, 0), x, rtol=0, atol=0)
    assert np.linalg.norm(oracle.rope(x, 1234)) == pytest.approx(np.linalg.norm(x), rel=1e-14)
    for m, n in [(5, 2), (100, 37), (4096, 4095)]:
        assert oracle.rope(x, m) @ oracle.rope(y, n) == pytest.approx(oracle.rope(x, m - n) @ y, rel=1e-9, abs=1e-9)
    # pair 0 turns by exactly pos radians
    e = np.zeros(64)
    e[0] = 1.0
    np.testing.assert_allclose(oracle.rope(e, 1.0)[:2], [math.cos(1.0), math.sin(1.0)], rtol=1e-15)


# ------------------------------------------------------------------------------------------------
# fp8 E4M3
# ------------------------------------------------------------------------------------------------
def test_e4m3_all_codes_match_torch_decoder():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3_spec_values():
    assert oracle.e4m3_value(0x7E) == 448.0           # largest finite
    assert oracle.e4m3_value(0x01) == 2.0 ** -9       # smallest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6       # smallest normal
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0xB8) == -1.0
    assert oracle.e4m3_value(0x80) == 0.0 and math.copysign(1, oracle.e4m3_value(0x80)) == -1


def test_fp8_cache_decodes_to_code_value_times_scale():
    inp = synth.make_inputs("gla", 2, 4, 2, 16, 8, [90, 40], seed=70, kv_dtype="fp8_e4m3")
    codes = inp.k_pool
    deq = codes.view(torch.float8_e4m3fn).to(torch.float64) * inp.scale_pool.to(torch.float64)[..., None]
    row = torch.cat([deq, inp.rope_pool.to(torch.float64)], dim=-1).numpy()
    kw = dict(groups=2, scale=inp.scale, page_size=64, d_rope=8)
    o1, l1 = oracle.decode_paged("gla", inp.q_lat.double().numpy(), inp.q_rope.double().numpy(), codes.numpy(),
                                 inp.layout.block_table, inp.layout.seq_lens, rope_pool=inp.rope_pool.double().numpy(),
                                 scale_pool=inp.scale_pool.double().numpy(), **kw)
    o2, l2 = oracle.decode_paged("gla", inp.q_lat.double().numpy(), inp.q_rope.double().numpy(), row,
                                 inp.layout.block_table, inp.layout.seq_lens, **kw)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ------------------------------------------------------------------------------------------------
# algorithmic bytes per token (the benchmark's byte counts)
# ------------------------------------------------------------------------------------------------
def test_bytes_per_token_fixed_by_the_pages():
    with open(os.path.join(GOLDEN, "bytes_per_token.json")) as f:
        items = {it["name"]: it for it in json.load(f)["items"]}
    mla = synth.kv_bytes_per_token("mla", 1, 512, 64, "bf16")
    assert mla == 2 * items["absorbed MLA row dims"]["value"] == 2 * sum(items["absorbed MLA row dims"]["parts"])
    share = synth.kv_bytes_per_token("mla", 1, 128, 64, "bf16")     # one MLRA branch + the RoPE key
    assert share == 2 * 128 * items["MLRA-4 per-device read under 4-way TP, in units of d_h = 128"]["value"]
    assert 3 * share == mla
    gqa = synth.kv_bytes_per_token("gqa", 8, 128, 0, "bf16")
    gta = synth.kv_bytes_per_token("gta", 8, 128, 0, "bf16")
    assert gta == items["GTA cache relative to GQA"]["value"] * gqa
    assert synth.kv_bytes_per_token("gla", 2, 256, 64, "fp8_e4m3") == 512 + 128 + 4


# ------------------------------------------------------------------------------------------------
# several query tokens per sequence (multi-token decode): causal attention over the last positions
# ------------------------------------------------------------------------------------------------
def _tokens_inputs(variant, lens, q_len, seed):
    G, d, dr = (1, 24, 8) if variant == "mla" else (1, 16, 0)
    return synth.make_inputs(variant, len(lens), 3, G, d, dr, lens, scale=0.3, seed=seed, q_dtype="f32",
                             kv_dtype="f32", out_dtype="f32", page_size=8, q_len=q_len)


def _tokens_oracle(inp):
    f64 = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    return oracle.decode_paged_tokens(inp.variant, f64(inp.q_lat), f64(inp.q_rope), f64(inp.k_pool),
                                      inp.layout.block_table, inp.layout.seq_lens, q_len=inp.q_len, groups=1,
                                      scale=inp.scale, page_size=inp.layout.page_size, v_pool=f64(inp.v_pool),
                                      d_rope=inp.d_rope)


@pytest.mark.parametrize("variant", ["mla", "mqa"])
def test_tokens_match_causal_sdpa(variant):
    """Every (token, head) row against torch's attention over the whole sequence with a causal mask
    whose last q_len query positions are the tokens."""
    Q, lens = 3, [9, 20, 3]
    inp = _tokens_inputs(variant, lens, Q, 41)
    out, lse = _tokens_oracle(inp)
    H, d = inp.heads, inp.d_lat
    for b, L in enumerate(lens):
        rows = oracle.logical_rows(inp.k_pool.double().numpy(), inp.layout.block_table[b], L, inp.layout.page_size)
        if variant == "mla":
            K, V = rows, rows[:, :d]
            q = np.concatenate([inp.q_lat[b].double().numpy(), inp.q_rope[b].double().numpy()], axis=1)
        else:
            K = rows[:, 0, :]
            V = oracle.logical_rows(inp.v_pool.double().numpy(), inp.layout.block_table[b], L,
                                    inp.layout.page_size)[:, 0, :]
            q = inp.q_lat[b].double().numpy()
        pos = np.repeat(np.arange(L - Q, L), H)           # row i*H + h sits at position L - Q + i
        mask = np.arange(L)[None, :] <= pos[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None], torch.tensor(K)[None], torch.tensor(V)[None],
            attn_mask=torch.tensor(mask)[None], scale=inp.scale)[0].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)
        s = np.where(mask, (q @ K.T) * inp.scale, -np.inf)
        np.testing.assert_allclose(lse[b], torch.logsumexp(torch.tensor(s), dim=1).numpy(), rtol=1e-13)


def test_tokens_one_is_the_single_token_decode():
    inp = _tokens_inputs("mla", [7, 30], 1, 42)
    f64 = lambda t: t.double().numpy()  # noqa: E731
    o1, l1 = _tokens_oracle(inp)
    o2, l2 = oracle.decode_paged("mla", f64(inp.q_lat), f64(inp.q_rope), f64(inp.k_pool), inp.layout.block_table,
                                 inp.layout.seq_lens, groups=1, scale=inp.scale, page_size=inp.layout.page_size,
                                 d_rope=inp.d_rope)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_tokens_before_the_first_row_see_nothing():
    """A sequence shorter than q_len: its first tokens have no visible row (out 0, lse -inf); the
    first token that sees one row returns that row's value."""
    Q = 4
    inp = _tokens_inputs("mla", [2, 12], Q, 43)
    out, lse = _tokens_oracle(inp)
    H, d = inp.heads, inp.d_lat
    assert np.all(out[0, : 2 * H] == 0) and np.all(lse[0, : 2 * H] == -np.inf)
    row0 = oracle.logical_rows(inp.k_pool.double().numpy(), inp.layout.block_table[0], 1, inp.layout.page_size)[0]
    np.testing.assert_allclose(out[0, 2 * H: 3 * H], np.broadcast_to(row0[:d], (H, d)), rtol=1e-14)
    assert np.all(np.isfinite(lse[1]))
