"""ld_latent_decode_noalloc (the decode step whose workspace is the library's fixed device array) against
ld_latent_decode with a caller workspace, through the C ABI, on consecutive calls of decreasing size
(needs an MI355X).  Both run the same kernels over the same plan, so the results must be the same bits;
each is also held to the oracle's bound."""
import ctypes
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import lse_err, row_rel_err, run_oracle, to_dev, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latent_kv_cache_absorbed_amd as lkd
    lkd.lib()


def _decoder(inp):
    import latent_kv_cache_absorbed_amd as lkd
    return lkd.Decoder(to_dev(inp.q_lat), to_dev(inp.q_rope), to_dev(inp.k_pool),
                       torch.from_numpy(inp.layout.block_table).cuda(), torch.from_numpy(inp.layout.seq_lens).cuda(),
                       variant=inp.variant, scale=inp.scale, groups=inp.groups, v=to_dev(inp.v_pool),
                       rope=to_dev(inp.rope_pool), kscale=to_dev(inp.scale_pool))


_S = 1 / math.sqrt(192)
_CASES = [
    # a batch above the one-launch combine limit with a sequence merged in several chunks (combine
    # arrival counters in the array), then smaller problems, then the first again
    ("mla", 128, 1, 512, 64, [40000] + [300 + 97 * i for i in range(9)], "bf16"),
    ("mla", 128, 1, 512, 64, [1500, 77], "bf16"),
    ("gla", 128, 2, 256, 64, [3000, 1, 650], "fp8_e4m3"),
    ("mla", 128, 1, 512, 64, [64], "bf16"),
    ("mla", 128, 1, 512, 64, [40000] + [300 + 97 * i for i in range(9)], "bf16"),
]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    for i, (variant, H, G, d, dr, lens, kv) in enumerate(_CASES):
        inp = synth.make_inputs(variant, len(lens), H, G, d, dr, lens, scale=_S, seed=60 + i, kv_dtype=kv)
        print(f"case noalloc call {i}: {variant} kv={kv} lens={lens[:4]}", flush=True)
        ref, got = _decoder(inp), _decoder(inp)
        for t in (got.out, got.lse):
            t.fill_(float("nan"))
        ref.run()
        got.run_noalloc()
        torch.cuda.synchronize()
        assert torch.equal(got.out, ref.out) and torch.equal(got.lse, ref.lse), f"call {i} differs"
        o, l = got.out.double().cpu().numpy(), got.lse.double().cpu().numpy()
        ro, rl = run_oracle(inp, batches=[0, len(lens) - 1], heads=[0, 77, 127])
        m = ~np.isnan(rl)
        eo, el = row_rel_err(o, ro, m), lse_err(l, rl, m)
        print(f"   out err {eo:.3e}  lse err {el:.3e}", flush=True)
        assert eo <= tolerance(inp) and el <= tolerance(inp)


def test_noalloc_rejects_problems_above_the_array():
    import latent_kv_cache_absorbed_amd as lkd
    # 4 query tokens x 128 heads x batch 64 needs more workspace than the array holds
    p = lkd.make_problem("mla", 64, 128, 1, 512, 64, 64, 4097, 64, "bf16", "bf16", "bf16", _S, q_len=4)
    assert lkd.workspace_size(p) > lkd.NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    ptr = ctypes.c_void_p(buf.data_ptr())
    cache = lkd.KVCache(buf.data_ptr(), None, None, None)
    st = lkd.lib().ld_latent_decode_noalloc(ctypes.byref(p), ptr, ptr, ctypes.byref(cache), ptr, ptr, ptr, ptr, None)
    assert st == 6          # LD_ERR_WORKSPACE_TOO_SMALL, before anything is queued
    torch.cuda.synchronize()
