"""GPU parity at the benchmark workloads' full sizes, in the benchmark's launch configuration
(automatic split-KV plan, shuffled pages): the whole problem runs on the GPU, the fp64 oracle
recomputes a sample of (sequence, head) rows one by one.

Latent variants are checked twice on the same run: the latent output against the absorbed oracle
(``decode_paged``), and in the materialised space, where the sampled heads get per-head
up-projections (W_UK ~ N(0, 1/128), W_UV ~ N(0, 1/d_g), q^C ~ N(0, 1)), the GPU consumes the absorbed
queries W_UK^T q^C rounded to bf16, and its latent rows mapped through W_UV in fp64 (MLRA: summed over
the branches) are compared with the oracle's materialised per-head attention.  Shared-KV variants have
no up-projections: their oracle is ``shared_kv_attention`` itself."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import (absorb_sampled_queries, lse_err, materialised_errors, row_rel_err, run_gpu, run_oracle,
                      tolerance)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latent_kv_cache_absorbed_amd as lkd
    lkd.lib()


@pytest.mark.parametrize("name,batches,heads", [
    ("mla_b64_l4k", [0, 31, 63], [0, 1, 64, 127]),
    ("mla_b1_l128k", [0], [0, 77, 127]),
    ("mla_b1_l512k", [0], [5, 126]),
    ("mla_b1_l1m", [0], [0, 127]),
    ("mlra4_b1_l128k", [0], [0, 100]),
    ("mlra4_b1_l512k", [0], [3, 64]),
    ("mlra4_b1_l1m", [0], [1, 127]),
    ("gla2_fp8_b64_mixed", [0, 17, 63], [0, 63, 64, 127]),
    ("gqa_b32_l32k", [0, 13, 31], [0, 7, 8, 63]),
    ("mqa_b32_l32k", [0, 31], [0, 63]),
    ("gta_b32_l32k", [5], [0, 9, 63]),
    ("mlra4_tp4_share_b1_l1m", [0], [0, 101]),
    ("gla2_tp2_share_fp8_b64_mixed", [1, 40], [0, 33, 63]),
])
def test_full_size_sampled(name, batches, heads):
    inp = synth.make_workload_inputs(synth.WORKLOADS[name])
    print(f"case {name} batches={batches} heads={heads}", flush=True)
    latent = inp.variant in ("mla", "gla", "mlra")
    weights = absorb_sampled_queries(inp, batches, heads, seed=len(name)) if latent else None
    got_o, got_l = run_gpu(inp)
    ref_o, ref_l = run_oracle(inp, batches=batches, heads=heads)
    mask = ~np.isnan(ref_l)
    assert mask.sum() > 0
    tol = tolerance(inp)
    eo = row_rel_err(got_o, ref_o, mask)
    el = lse_err(got_l, ref_l, mask)
    print(f"   absorbed:     out err {eo:.3e}  lse err {el:.3e}  tol {tol:g}", flush=True)
    assert eo <= tol and el <= tol
    if latent:
        mo, ml = materialised_errors(inp, got_o, got_l, batches, heads, weights)
        print(f"   materialised: out err {mo:.3e}  lse err {ml:.3e}  tol {tol:g}", flush=True)
        assert mo <= tol and ml <= tol
    # rows the oracle skipped are still finite
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
