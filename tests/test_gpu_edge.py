"""GPU edge cases: workspace bounds when forced splits are exceeded, every E4M3 code through the decode's
conversion, and NaN inputs reaching only the rows that attend them (needs an MI355X)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import lse_err, row_rel_err, run_gpu, run_oracle, to_dev, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latent_kv_cache_absorbed_amd as lkd
    lkd.lib()


def test_forced_splits_capped_by_unit_pages_in_a_large_batch():
    """num_splits = 2 with sequences of 8,438 pages: no split may span more than 512 pages, so every sequence
    gets 17 splits (two combine chunks each) in a batch of 9 (the per-task combine).  The workspace must
    hold all 153 units and 18 combine tasks; the result must still match the oracle at the fp32 bound."""
    import latent_kv_cache_absorbed_amd as lkd
    lens = [270000] * 8 + [265000]
    inp = synth.make_inputs("mla", 9, 16, 1, 64, 16, lens, page_size=32, kv_dtype="f32", q_dtype="f32",
                            out_dtype="f32", scale=1 / math.sqrt(48), seed=51)
    chunk, units, ns, first = lkd.plan_host(lkd.make_problem("mla", 9, 16, 1, 64, 16, 32, inp.layout.num_pages,
                                                             inp.layout.max_pages_per_seq, "f32", "f32", "f32",
                                                             inp.scale, num_splits=2), inp.layout.seq_lens, 256)
    assert list(ns) == [17] * 9
    print(f"case forced 2 splits, 9 x 270K tokens, page 32: {units} units", flush=True)
    got_o, got_l = run_gpu(inp, num_splits=2)
    ref_o, ref_l = run_oracle(inp)
    eo, el = row_rel_err(got_o, ref_o), lse_err(got_l, ref_l)
    print(f"   out err {eo:.3e}  lse err {el:.3e}", flush=True)
    assert eo <= 1e-5 and el <= 1e-5


def _all_codes_row(rng, width):
    """A row of `width` E4M3 codes holding every finite code (254 of them) at least once, shuffled."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    reps = -(-width // len(finite))
    row = np.tile(finite, reps)[:width] if width >= len(finite) else None
    assert row is not None and set(row.tolist()) == set(finite.tolist())
    return rng.permutation(row)


@pytest.mark.parametrize("variant,H,d", [("gla", 64, 256), ("mla", 128, 512)])
def test_e4m3_every_code_through_the_decode(variant, H, d):
    """Single-row sequences whose latent holds every finite E4M3 code, per-token scales powers of two: the
    softmax weight is exactly 1, so the f32 output must equal code_value x scale bit for bit (the decode's
    fp8 -> bf16 conversion and the scale folded into P are exact for every code)."""
    import latent_kv_cache_absorbed_amd as lkd
    rng = np.random.default_rng(77)
    scales = [1.0, 2.0 ** -3, 2.0 ** 4, 2.0 ** -9]
    B = len(scales)
    inp = synth.make_inputs(variant, B, H, 1, d, 64, [1] * B, kv_dtype="fp8_e4m3", scale=1 / math.sqrt(192),
                            seed=52)
    codes = inp.k_pool.clone()
    sc = inp.scale_pool.clone()
    rows = []
    for b in range(B):
        page = int(inp.layout.block_table[b, 0])
        row = _all_codes_row(rng, d)
        codes[page, 0] = torch.from_numpy(row)
        sc[page, 0] = scales[b]
        rows.append(row)
    # a zero query: every score is 0, so the weight of the one row is exactly 1 and lse is exactly 0
    q_lat = torch.zeros_like(inp.q_lat)
    q_rope = torch.zeros_like(inp.q_rope)
    print(f"case every E4M3 code through the {variant} d={d} decode, scales {scales}", flush=True)
    bt = torch.from_numpy(inp.layout.block_table).cuda()
    sl = torch.from_numpy(inp.layout.seq_lens).cuda()
    out, lse = lkd.latent_decode(q_lat.cuda(), q_rope.cuda(), codes.cuda(), bt, sl, variant=variant,
                                 scale=inp.scale, groups=1, rope=to_dev(inp.rope_pool), kscale=sc.cuda(),
                                 out_dtype="f32")
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    for b in range(B):
        want = oracle.e4m3_decode(rows[b]) * scales[b]
        assert np.array_equal(out[b], np.broadcast_to(want, out[b].shape)), f"sequence {b}"
    assert np.all(lse.cpu().numpy() == 0.0)


@pytest.mark.parametrize("variant,G,d,dr,lens,splits", [
    ("mla", 1, 512, 64, [300, 5000, 70], 0),        # the middle sequence is split (combine over splits)
    ("mla", 1, 512, 64, [40000] + [300] * 9, 0),    # the per-task combine with a multi-chunk sequence
    ("gqa", 8, 128, 0, [900, 3000], 3),
])
def test_nan_query_reaches_only_its_row(variant, G, d, dr, lens, splits):
    """A NaN in one head's query (latent or RoPE part) makes that row's out and lse NaN, as the oracle's
    arithmetic does, and leaves every other row bit for bit as it was without the NaN."""
    H = 128 if variant == "mla" else 64
    inp = synth.make_inputs(variant, len(lens), H, G, d, dr, lens, scale=1 / math.sqrt(d + dr), seed=53)
    print(f"case NaN query {variant} lens={lens[:4]} splits={splits}", flush=True)
    o0, l0 = run_gpu(inp, num_splits=splits)
    bad = [(0, 3), (1, 100)]
    inp.q_lat[0, 3, 17] = float("nan")
    if variant == "mla":
        inp.q_rope[1, 100, 5] = float("nan")
    else:
        inp.q_lat[1, 100 % H, 5] = float("nan")
    o1, l1 = run_gpu(inp, num_splits=splits)
    mask = np.zeros(l0.shape, bool)
    for b, h in bad:
        mask[b, h % H] = True
    assert np.all(np.isnan(o1[mask])) and np.all(np.isnan(l1[mask]))
    assert np.array_equal(o1[~mask], o0[~mask]) and np.array_equal(l1[~mask], l0[~mask])
    # the oracle agrees: NaN exactly in the poisoned rows, the GPU's other rows within tolerance
    heads = [3, 4, 100 % H]
    ref_o, ref_l = run_oracle(inp, batches=[0, 1], heads=heads)
    ok = np.zeros(l0.shape, bool)
    for b in (0, 1):
        for h in heads:
            if mask[b, h]:
                assert np.isnan(ref_l[b, h]) and np.all(np.isnan(ref_o[b, h]))
            else:
                ok[b, h] = True
    assert ok.sum() == 4
    assert row_rel_err(o1, ref_o, ok) <= tolerance(inp) and lse_err(l1, ref_l, ok) <= tolerance(inp)


def test_split_combine_standalone_nan_lse():
    """ld_split_kv_combine: a NaN among a row's split lse makes the row NaN (the oracle's combine does the
    same); -inf splits keep zero weight; other rows are unaffected."""
    import latent_kv_cache_absorbed_amd as lkd
    r = np.random.default_rng(8)
    rows, S, dv = 6, 5, 32
    po = r.normal(size=(rows, S, dv)).astype(np.float32)
    pl = r.normal(size=(rows, S)).astype(np.float32)
    ns = np.full(rows, S, np.int32)
    pl[1, 2] = np.nan
    pl[2, :] = np.nan
    pl[3, 0] = -np.inf
    o, l = lkd.split_kv_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), torch.from_numpy(ns).cuda())
    o, l = o.double().cpu().numpy(), l.double().cpu().numpy()
    for i in range(rows):
        eo, el = oracle.combine_partials(po[i].astype(np.float64), pl[i].astype(np.float64))
        if np.isnan(el):
            assert np.isnan(l[i]) and np.all(np.isnan(o[i]))
        else:
            assert np.max(np.abs(o[i] - eo)) <= 1e-5 * max(1.0, np.max(np.abs(eo)))
            assert abs(l[i] - el) <= 1e-5 * max(1.0, abs(el))


@pytest.mark.parametrize("splits,spikes", [(0, [64 * 5 + 40, 2999]), (1, [2000]), (3, [1100, 1101])])
def test_score_far_above_the_first_rows(splits, spikes):
    """Keys whose scores exceed every other row's by a factor above 2^400 in the softmax (a unit's later rows dominating
    its first): the result is the oracle's, i.e. the weight concentrates on those keys, whatever reference
    the kernel's softmax starts from (the absorbed-MLA kernel runs such a unit again with its exact max)."""
    lens = [3000, 700]
    inp = synth.make_inputs("mla", 2, 128, 1, 512, 64, lens, scale=1 / math.sqrt(192), seed=54)
    q = inp.q_lat[0].float()                                  # [H, 512]
    for t in spikes:
        page, slot = int(inp.layout.block_table[0, t // 64]), t % 64
        inp.k_pool[page, slot, :512] = (8.0 * q[0]).to(inp.k_pool.dtype)   # head 0 scores ~300 there
    print(f"case score spikes at {spikes} splits={splits}", flush=True)
    got_o, got_l = run_gpu(inp, num_splits=splits)
    ref_o, ref_l = run_oracle(inp)
    eo, el = row_rel_err(got_o, ref_o), lse_err(got_l, ref_l)
    print(f"   out err {eo:.3e}  lse err {el:.3e}  head-0 lse {ref_l[0, 0]:.1f}", flush=True)
    assert ref_l[0, 0] > 200                                   # the spike dominates head 0 by far
    assert eo <= tolerance(inp) and el <= tolerance(inp)
