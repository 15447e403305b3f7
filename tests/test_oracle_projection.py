"""Pins for the oracle's head projections: explicit sums, the query absorption, the materialised MLA
output and MLRA's branch sum (each reached by another route than the oracle's own product)."""
import math

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def test_projection_against_explicit_sum():
    r = _rng(1)
    A, W = r.normal(size=(3, 2, 5)), r.normal(size=(2, 4, 5))
    got = oracle.head_projection(A, W)
    for m in range(3):
        for h in range(2):
            for n in range(4):
                assert got[m, h, n] == pytest.approx(sum(W[h, n, k] * A[m, h, k] for k in range(5)), rel=1e-13)


def test_query_absorption_is_the_projection_by_the_transposed_key_up_projection():
    r = _rng(2)
    qn, W_UK = r.normal(size=(4, 3, 6)), r.normal(size=(3, 6, 10))     # [B, H, dn], [H, dn, dc]
    got = oracle.head_projection(qn, np.transpose(W_UK, (0, 2, 1)))
    ref = np.stack([oracle.absorb_query(qn[b], W_UK) for b in range(4)])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_up_projection_of_the_absorbed_output_is_the_materialised_mla_output():
    r = _rng(3)
    H, dn, dr, dc, dv, L = 4, 6, 4, 12, 5, 23
    q_nope, q_rope = r.normal(size=(H, dn)), r.normal(size=(H, dr))
    W_UK, W_UV = r.normal(size=(H, dn, dc)) / 3, r.normal(size=(H, dv, dc)) / 3
    C, KR = r.normal(size=(L, dc)), r.normal(size=(L, dr))
    scale = 1 / math.sqrt(dn + dr)
    o_mat, _ = oracle.mla_materialised(q_nope, q_rope, W_UK, W_UV, C, KR, scale)
    q_lat = oracle.head_projection(q_nope[None], np.transpose(W_UK, (0, 2, 1)))[0]
    pool = np.concatenate([C, KR], axis=1)[None]
    o_lat, _ = oracle.decode_paged("mla", q_lat[None], q_rope[None], pool, np.zeros((1, 1), np.int32), np.array([L]),
                                   groups=1, scale=scale, page_size=L, d_rope=dr)
    o = oracle.head_projection(o_lat, W_UV)[0]
    np.testing.assert_allclose(o, o_mat, rtol=1e-11, atol=1e-12)


def test_stacked_branch_projection_is_the_sum_of_branch_projections():
    r = _rng(4)
    G, B, H, dc, dv = 4, 3, 2, 5, 7
    W = r.normal(size=(G, H, dv, dc))
    O = r.normal(size=(B, H, G, dc))                        # per-branch latent outputs
    got = oracle.head_projection(O.reshape(B, H, G * dc), oracle.stack_branch_weights(W))
    ref = sum(oracle.head_projection(O[:, :, g, :], W[g]) for g in range(G))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
