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
