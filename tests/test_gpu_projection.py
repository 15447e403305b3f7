"""GPU parity of ld_head_projection against the CPU fp64 oracle (needs an MI355X).

bf16 operands are exact in fp32 and so are their products, so the only error is the fp32
accumulation over k terms and, for a bf16 result, its final rounding.  Each output is checked
against the standard bound for that: |c - ref| <= (k + 2) 2^-24 sum_t |w a| (+ 2^-8 |ref| for bf16).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latent_kv_cache_absorbed_amd as lkd
    lkd.lib()


def _check(A, W, out_dtype, got=None):
    import latent_kv_cache_absorbed_amd as lkd
    m, H, k = A.shape
    print(f"case projection m={m} H={H} n={W.shape[1]} k={k} out={out_dtype}", flush=True)
    if got is None:
        got = lkd.head_projection(A.cuda(), W.cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = got.double().cpu().numpy()
    a64, w64 = A.double().numpy(), W.double().numpy()
    ref = oracle.head_projection(a64, w64)
    mag = oracle.head_projection(np.abs(a64), np.abs(w64))
    bound = (k + 2) * 2.0 ** -24 * mag + (2.0 ** -8 * np.abs(ref) if out_dtype == "bf16" else 0.0) + 1e-30
    err = np.abs(got - ref)
    worst = float(np.max(err / bound))
    print(f"   worst error / bound {worst:.3f}", flush=True)
    assert worst <= 1.0
    return got, ref


def _bf16(r, *shape, std=1.0):
    return torch.from_numpy(r.normal(0, std, shape).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("m,H,n,k", [(64, 128, 512, 128), (64, 128, 128, 512), (1, 128, 512, 128),
                                     (130, 4, 192, 256), (70, 3, 64, 64),
                                     (100, 3, 64, 48), (33, 5, 32, 16), (65, 2, 96, 400)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_projection(m, H, n, k, out_dtype):
    r = np.random.default_rng(m * 7 + n + k)
    _check(_bf16(r, m, H, k), _bf16(r, H, n, k, std=k ** -0.5), out_dtype)


def test_query_absorption_then_decode_matches_the_materialised_model():
    """q_lat = W_UK^T q^C on the GPU, fed to the GPU decode, mapped back by W_UV on the GPU: the result
    is the oracle's materialised per-head MLA attention (to the bf16 bound of the decode)."""
    import math

    import latent_kv_cache_absorbed_amd as lkd
    import synth
    r = np.random.default_rng(5)
    B, H, dn, dr, dc, dv, L = 2, 128, 128, 64, 512, 128, 700
    q_nope, q_rope = _bf16(r, B, H, dn), _bf16(r, B, H, dr)
    W_UK, W_UV = _bf16(r, H, dn, dc, std=dn ** -0.5), _bf16(r, H, dv, dc, std=dc ** -0.5)
    inp = synth.make_inputs("mla", B, H, 1, dc, dr, [L, 300], scale=1 / math.sqrt(dn + dr), seed=6)
    dev = torch.device("cuda")
    q_lat = lkd.head_projection(q_nope.to(dev), W_UK.transpose(1, 2).contiguous().to(dev), out_dtype="bf16")
    bt = torch.from_numpy(inp.layout.block_table).to(dev)
    sl = torch.from_numpy(inp.layout.seq_lens).to(dev)
    o_lat, _ = lkd.latent_decode(q_lat, q_rope.to(dev), inp.k_pool.to(dev), bt, sl, variant="mla", scale=inp.scale)
    o = lkd.head_projection(o_lat, W_UV.to(dev), out_dtype="f32")
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    pool = inp.k_pool.double().numpy()
    for b in range(B):
        rows = oracle.logical_rows(pool, inp.layout.block_table[b], inp.layout.seq_lens[b], inp.layout.page_size)
        ref, _ = oracle.mla_materialised(q_nope[b].double().numpy(), q_rope[b].double().numpy(),
                                         W_UK.double().numpy(), W_UV.double().numpy(), rows[:, :dc], rows[:, dc:],
                                         inp.scale)
        rel = np.max(np.abs(o[b] - ref), axis=1) / np.max(np.abs(ref), axis=1)
        print(f"   sequence {b}: max row error {rel.max():.3e}", flush=True)
        assert rel.max() <= 1e-2     # bf16 roundings on the way: q_lat, P, o_lat (the up-projection is f32)


def test_mlra_branch_sum_as_one_stacked_projection():
    r = np.random.default_rng(7)
    G, B, H, dc, dv = 4, 3, 128, 128, 128
    Wb = _bf16(r, G, H, dv, dc, std=(G * dc) ** -0.5)
    O = _bf16(r, B, H, G, dc)
    Ws = torch.from_numpy(oracle.stack_branch_weights(Wb.float().numpy()).astype(np.float32)).to(torch.bfloat16)
    got, _ = _check(O.reshape(B, H, G * dc).contiguous(), Ws.contiguous(), "f32")
    ref = sum(oracle.head_projection(O[:, :, g, :].double().numpy(), Wb[g].double().numpy()) for g in range(G))
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-4)
