"""Helpers for the GPU tests: upload seeded inputs, run the library, run the oracle, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import latent_kv_cache_absorbed_amd as lkd


def to_dev(t):
    return None if t is None else t.contiguous().cuda()


def run_gpu(inp: synth.DecodeInputs, num_splits: int = 0, block_table=None, seq_lens=None, out_dtype=None):
    """Run ld_latent_decode on the problem; returns (out, lse) as CPU float64 numpy arrays."""
    bt = torch.from_numpy(inp.layout.block_table if block_table is None else block_table).cuda()
    sl = torch.from_numpy(inp.layout.seq_lens if seq_lens is None else seq_lens).cuda()
    k = to_dev(inp.k_pool)
    out, lse = lkd.latent_decode(to_dev(inp.q_lat), to_dev(inp.q_rope), k, bt, sl, variant=inp.variant,
                                 scale=inp.scale, groups=inp.groups, v=to_dev(inp.v_pool), rope=to_dev(inp.rope_pool),
                                 kscale=to_dev(inp.scale_pool), num_splits=num_splits,
                                 out_dtype=out_dtype or inp.out_dtype, q_len=inp.q_len)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy()


def run_oracle(inp: synth.DecodeInputs, batches=None, heads=None):
    f64 = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    k = inp.k_pool.numpy() if inp.kv_dtype == "fp8_e4m3" else f64(inp.k_pool)
    if inp.q_len > 1:
        return oracle.decode_paged_tokens(inp.variant, f64(inp.q_lat), f64(inp.q_rope), k, inp.layout.block_table,
                                          inp.layout.seq_lens, q_len=inp.q_len, groups=inp.groups, scale=inp.scale,
                                          page_size=inp.layout.page_size, v_pool=f64(inp.v_pool),
                                          rope_pool=f64(inp.rope_pool), scale_pool=f64(inp.scale_pool),
                                          d_rope=inp.d_rope, batches=batches, heads=heads)
    return oracle.decode_paged(inp.variant, f64(inp.q_lat), f64(inp.q_rope), k, inp.layout.block_table,
                               inp.layout.seq_lens, groups=inp.groups, scale=inp.scale,
                               page_size=inp.layout.page_size, v_pool=f64(inp.v_pool), rope_pool=f64(inp.rope_pool),
                               scale_pool=f64(inp.scale_pool), d_rope=inp.d_rope, batches=batches, heads=heads)


def row_rel_err(got, ref, mask=None):
    """max over rows of max_k |got - ref| / max_k |ref| (rows = all but the last axis)."""
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    if mask is not None:
        m = mask.reshape(-1)
        g, r = g[m], r[m]
    if g.size == 0:
        return 0.0
    den = np.max(np.abs(r), axis=1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.max(np.abs(g - r), axis=1) / den))


def lse_err(got, ref, mask=None):
    g, r = got.reshape(-1), ref.reshape(-1)
    if mask is not None:
        g, r = g[mask.reshape(-1)], r[mask.reshape(-1)]
    fin = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), fin), "lse finiteness differs"
    assert np.array_equal(g[~fin], r[~fin])
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(g[fin] - r[fin]) / np.maximum(1.0, np.abs(r[fin]))))


def tolerance(inp) -> float:
    """Acceptance bound: 1e-5 for an all-fp32 problem, 1e-2 for bf16 inputs or an fp8 cache."""
    return 1e-5 if (inp.kv_dtype == "f32" and inp.q_dtype == "f32" and inp.out_dtype == "f32") else 1e-2


# ---------------------------------------------------------------------------------------------------
# the comparison in the materialised space: per-head up-projections W_UK / W_UV for the sampled rows
# ---------------------------------------------------------------------------------------------------
def absorb_sampled_queries(inp: synth.DecodeInputs, batches, heads, d_nope: int = 128, d_v: int = 128,
                           seed: int = 0):
    """Draw per-head W_UK ~ N(0, 1/d_nope), W_UV ~ N(0, 1/d_g) and q^C ~ N(0, 1) for the sampled heads (for
    MLRA one set per branch), and replace the sampled rows of ``inp.q_lat`` by the absorbed queries
    W_UK^T q^C in fp64, rounded to the query dtype (the other rows keep their N(0, 1) draw).

    Returns (W_UK [nh, nb, dn, dg], W_UV [nh, nb, dv, dg], q_nope [len(batches), nh, nb, dn]).
    """
    nb = inp.groups if inp.variant == "mlra" else 1
    dg = inp.d_lat
    nh = len(heads)
    rng = synth.generator(900 + seed, 0)
    W_UK = rng.standard_normal((nh, nb, d_nope, dg)) / np.sqrt(d_nope)
    W_UV = rng.standard_normal((nh, nb, d_v, dg)) / np.sqrt(dg)
    q_nope = rng.standard_normal((len(batches), nh, nb, d_nope))
    for i, b in enumerate(batches):
        for j, h in enumerate(heads):
            for br in range(nb):
                q = torch.from_numpy(oracle.absorb_query(q_nope[i, j, br], W_UK[j, br])).to(inp.q_lat.dtype)
                if inp.variant == "mlra":
                    inp.q_lat[b, h, br] = q
                else:
                    inp.q_lat[b, h] = q
    return W_UK, W_UV, q_nope


def materialised_errors(inp: synth.DecodeInputs, got_o, got_l, batches, heads, weights):
    """Map the GPU's latent rows through W_UV in fp64 (MLRA: the branch sum of the mapped branch outputs)
    and compare with the oracle's materialised per-head attention (k = [W_UK c ; k_r], v = W_UV c).

    Returns (max row-relative out error, max lse error) over the sampled rows.
    """
    W_UK, W_UV, q_nope = weights
    heads = list(heads)
    eo, el = 0.0, 0.0
    f64 = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    qr_all = f64(inp.q_rope)
    for i, b in enumerate(batches):
        L = int(inp.layout.seq_lens[b])
        bt, ps = inp.layout.block_table[b], inp.layout.page_size
        if inp.kv_dtype == "fp8_e4m3":
            lat = oracle.e4m3_decode(oracle.logical_rows(inp.k_pool.numpy(), bt, L, ps)) * \
                oracle.logical_rows(f64(inp.scale_pool), bt, L, ps)[:, None]
            kr = oracle.logical_rows(f64(inp.rope_pool), bt, L, ps)
        else:
            rows = oracle.logical_rows(f64(inp.k_pool), bt, L, ps)
            lat, kr = rows[:, :rows.shape[1] - inp.d_rope], rows[:, rows.shape[1] - inp.d_rope:]
        dg = inp.d_lat
        g_o = got_o[b][heads]
        if inp.variant == "mla":
            ref_o, ref_l = oracle.mla_materialised(q_nope[i, :, 0], qr_all[b][heads], W_UK[:, 0], W_UV[:, 0], lat, kr,
                                                   inp.scale)
            mapped = np.einsum("hvc,hc->hv", W_UV[:, 0], g_o)
        elif inp.variant == "gla":
            # gla_materialised maps head h of its H rows to group h // (H / G): the sampled heads are passed
            # group by group, the same number from each group
            per = inp.heads // inp.groups
            order = sorted(range(len(heads)), key=lambda j: heads[j] // per)
            counts = np.bincount([heads[j] // per for j in order], minlength=inp.groups)
            assert np.all(counts == counts[0]), "sample the same number of heads from every group"
            groups_c = [lat[:, g * dg:(g + 1) * dg] for g in range(inp.groups)]
            ro, rl = oracle.gla_materialised(q_nope[i, order, 0], qr_all[b][[heads[j] for j in order]],
                                             W_UK[order, 0], W_UV[order, 0], groups_c, kr, inp.scale)
            ref_o, ref_l = np.empty_like(ro), np.empty_like(rl)
            ref_o[order], ref_l[order] = ro, rl
            mapped = np.einsum("hvc,hc->hv", W_UV[:, 0], g_o)
        elif inp.variant == "mlra":
            branches = [lat[:, g * dg:(g + 1) * dg] for g in range(inp.groups)]
            ref_o, ref_l = oracle.mlra_materialised(q_nope[i], qr_all[b][heads], W_UK, W_UV, branches, kr, inp.scale)
            mapped = np.einsum("hgvc,hgc->hv", W_UV, g_o)
        else:
            raise ValueError("the materialised form belongs to the latent variants")
        eo = max(eo, row_rel_err(mapped, ref_o))
        el = max(el, lse_err(got_l[b][heads], ref_l))
    return eo, el
