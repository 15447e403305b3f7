"""GPU parity: the HIP path against the CPU fp64 oracle on seeded inputs (needs an MI355X)."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import lse_err, row_rel_err, run_gpu, run_oracle, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latent_kv_cache_absorbed_amd as lkd
    lkd.lib()          # fails loudly when the library is missing


def _check(inp, num_splits=0, tol=None, **kw):
    print(f"case variant={inp.variant} kv={inp.kv_dtype} H={inp.heads} G={inp.groups} d={inp.d_lat}+{inp.d_rope} "
          f"lens={list(inp.layout.seq_lens)[:8]} splits={num_splits}", flush=True)
    got_o, got_l = run_gpu(inp, num_splits=num_splits)
    ref_o, ref_l = run_oracle(inp, **kw)
    mask = ~np.isnan(ref_l)
    tol = tolerance(inp) if tol is None else tol
    eo = row_rel_err(got_o, ref_o, mask)
    el = lse_err(got_l, ref_l, mask)
    print(f"   out err {eo:.3e}  lse err {el:.3e}  tol {tol:g}", flush=True)
    assert eo <= tol and el <= tol
    return got_o, got_l


# --- the tiny fp32 absorbed-MLA workload, exactly as specified (1e-5)
def test_mla_tiny_f32_contiguous():
    w = synth.WORKLOADS["mla_tiny_f32"]
    _check(synth.make_workload_inputs(w))


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_mla_tiny_f32_splits(splits):
    w = synth.WORKLOADS["mla_tiny_f32"]
    _check(synth.make_workload_inputs(w, seq_lens=[256, 77], shuffle=True), num_splits=splits)


# --- MLA bf16, 128 heads, 576-dim shared rows: ragged lengths, shuffled pages, NaN-poisoned tails
@pytest.mark.parametrize("lens", [[1, 63, 64, 65], [300, 1000, 4097], [31, 32, 33, 129]])
def test_mla_bf16_ragged(lens):
    inp = synth.make_inputs("mla", len(lens), 128, 1, 512, 64, lens, scale=1 / math.sqrt(192), seed=11)
    _check(inp)


@pytest.mark.parametrize("splits", [1, 2, 5])
def test_mla_bf16_forced_splits(splits):
    inp = synth.make_inputs("mla", 2, 128, 1, 512, 64, [1500, 700], scale=1 / math.sqrt(192), seed=12)
    _check(inp, num_splits=splits)


def test_mla_bf16_small_heads():
    inp = synth.make_inputs("mla", 3, 16, 1, 64, 16, [100, 1, 257], scale=0.25, seed=13)
    _check(inp)


@pytest.mark.parametrize("groups,heads", [(4, 112), (1, 100)])
def test_mlra_bf16_partial_head_block(groups, heads):
    # MLRA branches on the pipelined kernel with a partly filled last 32-head block: absent heads' query
    # rows are neither read past the tensor nor written
    inp = synth.make_inputs("mlra", 2, heads, groups, 128, 64, [300, 2100], scale=1 / math.sqrt(192), seed=18)
    _check(inp)


def test_mla_bf16_partial_head_block():
    # 112 heads: the 128-head work group holds 16 absent heads, whose query rows it must neither read
    # past the last sequence's rows nor let into the result
    inp = synth.make_inputs("mla", 3, 112, 1, 512, 64, [300, 4097, 33], scale=1 / math.sqrt(192), seed=17)
    _check(inp)


# --- GLA-2 (bf16 and fp8) and MLRA-4
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_gla2(kv):
    inp = synth.make_inputs("gla", 3, 128, 2, 256, 64, [1, 500, 1111], scale=1 / math.sqrt(192), seed=14,
                            kv_dtype=kv)
    _check(inp)


# --- one GPU's tensor-parallel share: one MLRA-4 branch (128 heads, 128 + 64 dims) and one GLA-2
# group (64 heads, 256 + 64 dims)
def test_mlra4_one_branch():
    inp = synth.make_inputs("mlra", 2, 128, 1, 128, 64, [900, 65], scale=1 / math.sqrt(192), seed=21)
    _check(inp)


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_gla2_one_group(kv):
    inp = synth.make_inputs("gla", 3, 64, 1, 256, 64, [1, 700, 1300], scale=1 / math.sqrt(192), seed=22,
                            kv_dtype=kv)
    _check(inp)


# fp8 caches over the other kernel shapes, with units of none, one, two and many stages and forced
# splits: MLRA-4 (two branches per work group), one 256-dim latent shared by 128 heads (four head
# blocks), GLA-4 (four groups per work group) and MLA
@pytest.mark.parametrize("variant,G,d,lens", [
    ("mlra", 4, 128, [1, 32, 33, 64, 65, 3000]),
    ("gla", 1, 256, [1, 31, 96, 2049]),
    ("gla", 4, 256, [2, 160, 1025]),
    ("mla", 1, 512, [0, 33, 130, 3001]),
])
def test_fp8_shapes(variant, G, d, lens):
    inp = synth.make_inputs(variant, len(lens), 128, G, d, 64, lens, scale=1 / math.sqrt(192), seed=23,
                            kv_dtype="fp8_e4m3")
    _check(inp)
    _check(inp, num_splits=5)


def test_mla_fp8():
    inp = synth.make_inputs("mla", 2, 128, 1, 512, 64, [600, 65], scale=1 / math.sqrt(192), seed=15,
                            kv_dtype="fp8_e4m3")
    _check(inp)


def test_mlra4():
    inp = synth.make_inputs("mlra", 2, 128, 4, 128, 64, [700, 33], scale=1 / math.sqrt(192), seed=16)
    _check(inp)


# --- shared-KV baselines
@pytest.mark.parametrize("variant,groups", [("gqa", 8), ("mqa", 1), ("gta", 8)])
def test_shared_kv(variant, groups):
    inp = synth.make_inputs(variant, 3, 64, groups, 128, 0, [5, 300, 1025], scale=1 / math.sqrt(128), seed=17)
    _check(inp)


# a single kv head of large head dim (MFA-style MQA) and GQA over 256-dim heads
@pytest.mark.parametrize("variant,H,G,d,lens", [
    ("mqa", 64, 1, 256, [5, 300, 1025]),
    ("mqa", 32, 1, 256, [64, 777]),
    ("mqa", 64, 1, 512, [1, 130, 2049]),
    ("mqa", 32, 1, 512, [33, 900]),
    ("gqa", 32, 4, 256, [250, 3000]),
])
def test_shared_kv_large_head_dim(variant, H, G, d, lens):
    inp = synth.make_inputs(variant, len(lens), H, G, d, 0, lens, scale=1 / math.sqrt(d), seed=24)
    _check(inp)
    _check(inp, num_splits=3)


def test_shared_kv_f32():
    inp = synth.make_inputs("gqa", 2, 16, 4, 64, 0, [90, 200], scale=0.125, seed=18, kv_dtype="f32", q_dtype="f32",
                            out_dtype="f32")
    _check(inp)


# --- edge cases
def test_empty_sequences():
    inp = synth.make_inputs("mla", 3, 128, 1, 512, 64, [0, 70, 0], scale=1 / math.sqrt(192), seed=19)
    o, l = _check(inp)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(l[0] == -np.inf) and np.all(l[2] == -np.inf)


def test_shuffled_and_identity_tables_bitwise_equal():
    a = synth.make_inputs("mla", 2, 128, 1, 512, 64, [333, 129], scale=0.07, seed=20, shuffle=True)
    b = synth.make_inputs("mla", 2, 128, 1, 512, 64, [333, 129], scale=0.07, seed=20, shuffle=False)
    oa, la = run_gpu(a)
    ob, lb = run_gpu(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_run_to_run_bitwise_deterministic():
    inp = synth.make_inputs("gla", 2, 128, 2, 256, 64, [2000, 10], scale=0.07, seed=21, kv_dtype="fp8_e4m3")
    o1, l1 = run_gpu(inp)
    o2, l2 = run_gpu(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_split_combine_standalone():
    import latent_kv_cache_absorbed_amd as lkd
    import oracle
    r = np.random.default_rng(5)
    rows, S, dv = 37, 6, 64
    po = r.normal(size=(rows, S, dv)).astype(np.float32)
    pl = (r.normal(size=(rows, S)) * 3).astype(np.float32)
    ns = r.integers(0, S + 1, size=rows).astype(np.int32)
    pl[3, :2] = -np.inf
    o, l = lkd.split_kv_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(),
                                torch.from_numpy(ns).cuda())
    o, l = o.double().cpu().numpy(), l.double().cpu().numpy()
    for i in range(rows):
        eo, el = oracle.combine_partials(po[i, :ns[i]].astype(np.float64).reshape(ns[i], dv),
                                         pl[i, :ns[i]].astype(np.float64))
        if ns[i] == 0 or el == -np.inf:
            assert np.all(o[i] == 0) and l[i] == -np.inf
            continue
        assert np.max(np.abs(o[i] - eo)) <= 1e-5 * max(1.0, np.max(np.abs(eo)))
        assert abs(l[i] - el) <= 1e-5 * max(1.0, abs(el))


# --- one long sequence split many ways (planner units written cooperatively, multi-wave combine)
def test_mla_bf16_one_long_sequence_many_splits():
    inp = synth.make_inputs("mla", 1, 128, 1, 512, 64, [40000], scale=1 / math.sqrt(192), seed=22)
    _check(inp)


# a batch above the one-launch combine limit in which one sequence is merged in several chunks
# (its last chunk task to finish merges the chunk results)
def test_mla_bf16_multi_chunk_sequence_in_a_large_batch():
    lens = [40000] + [300 + 97 * i for i in range(9)]
    inp = synth.make_inputs("mla", len(lens), 128, 1, 512, 64, lens, scale=1 / math.sqrt(192), seed=24)
    _check(inp)


@pytest.mark.parametrize("splits", [9, 40])
def test_mla_bf16_forced_many_splits(splits):
    inp = synth.make_inputs("mla", 3, 128, 1, 512, 64, [5000, 64, 2600], scale=1 / math.sqrt(192), seed=23)
    _check(inp, num_splits=splits)


# --- ld_latent_decode derives the split plan inside the decode kernel (and leaves the plan arrays
# for the combine); ld_plan + ld_decode_planned + ld_combine_planned read it from the workspace.
# Same planner rule, same kernels: the two give the same bits.  Cases cover empty sequences, an
# all-empty batch, forced splits, a batch above the one-launch combine limit with a sequence merged
# in several chunks, and two work groups per unit (MLRA-4: two branches per work group).
_S = 1 / math.sqrt(192)


@pytest.mark.parametrize("variant,H,G,d,dr,lens,splits,kv", [
    ("mla", 128, 1, 512, 64, [0, 70, 0, 4097, 1], 0, "bf16"),
    ("mla", 128, 1, 512, 64, [0, 0], 0, "bf16"),
    ("mla", 128, 1, 512, 64, [5000, 64, 2600], 9, "bf16"),
    ("mla", 128, 1, 512, 64, [1500, 700], 1, "bf16"),
    ("mla", 128, 1, 512, 64, [40000] + [300 + 97 * i for i in range(9)], 0, "bf16"),
    ("mlra", 128, 4, 128, 64, [700, 33, 2500], 0, "bf16"),
    ("gla", 128, 2, 256, 64, [1, 500, 1111], 0, "fp8_e4m3"),
])
def test_fused_plan_matches_staged_plan(variant, H, G, d, dr, lens, splits, kv):
    import latent_kv_cache_absorbed_amd as lkd
    from gpu_util import to_dev
    inp = synth.make_inputs(variant, len(lens), H, G, d, dr, lens, scale=_S, seed=31, kv_dtype=kv)
    print(f"case fused vs staged plan {variant} lens={lens} splits={splits} kv={kv}", flush=True)
    bt = torch.from_numpy(inp.layout.block_table).cuda()
    sl = torch.from_numpy(inp.layout.seq_lens).cuda()
    mk = lambda: lkd.Decoder(to_dev(inp.q_lat), to_dev(inp.q_rope), to_dev(inp.k_pool), bt, sl,  # noqa: E731
                             variant=variant, scale=inp.scale, groups=G, rope=to_dev(inp.rope_pool),
                             kscale=to_dev(inp.scale_pool), num_splits=splits)
    fused, staged = mk(), mk()
    for d_ in (fused, staged):
        d_.out.fill_(float("nan"))
        d_.lse.fill_(float("nan"))
        d_.workspace.fill_(0xFF)
    fused.run()
    staged.plan()
    staged.decode()
    staged.combine()
    torch.cuda.synchronize()
    assert torch.equal(fused.out, staged.out) and torch.equal(fused.lse, staged.lse)
    assert not torch.isnan(fused.out).any()


# --- several query tokens per sequence (multi-token / speculative decode, MLA and MQA): sequences
# shorter than q_len (their first tokens see no row), one-, two- and many-stage units, forced
# splits, 64 heads, an fp8 cache, large MQA head dims; the staged path gives the fused path's bits
@pytest.mark.parametrize("variant,H,d,dr,lens,Q,splits,kv", [
    ("mla", 128, 512, 64, [1, 2, 3, 700, 2049], 2, 0, "bf16"),
    ("mla", 128, 512, 64, [4, 130, 5000], 4, 0, "bf16"),
    ("mla", 128, 512, 64, [300, 3000], 3, 5, "bf16"),
    ("mla", 64, 512, 64, [97, 1500], 2, 0, "bf16"),
    ("mla", 128, 512, 64, [2, 900], 2, 0, "fp8_e4m3"),
    ("mqa", 64, 128, 0, [5, 1025], 3, 0, "bf16"),
    ("mqa", 64, 512, 0, [64, 777], 2, 0, "bf16"),
])
def test_multi_token_decode(variant, H, d, dr, lens, Q, splits, kv):
    _multi_token_case(variant, H, 1, d, dr, lens, Q, splits, kv)


# the grouped variants: each token's rows span all groups (row i*H + h, group h / (H/G))
@pytest.mark.parametrize("variant,H,G,d,dr,lens,Q,splits,kv", [
    ("gla", 128, 2, 256, 64, [1, 300, 2049], 2, 0, "bf16"),
    ("gla", 128, 2, 256, 64, [3, 1111], 3, 4, "fp8_e4m3"),
    ("gla", 128, 4, 256, 64, [70, 900], 2, 0, "bf16"),
    ("gqa", 64, 8, 128, 0, [2, 500, 1025], 3, 0, "bf16"),
    ("gta", 64, 8, 128, 0, [40, 700], 2, 0, "bf16"),
    ("mlra", 128, 4, 128, 64, [1, 600, 2000], 2, 0, "bf16"),
    ("mlra", 128, 1, 128, 64, [5, 1500], 3, 3, "bf16"),
])
def test_multi_token_decode_grouped(variant, H, G, d, dr, lens, Q, splits, kv):
    _multi_token_case(variant, H, G, d, dr, lens, Q, splits, kv)


def _multi_token_case(variant, H, G, d, dr, lens, Q, splits, kv):
    import latent_kv_cache_absorbed_amd as lkd
    from gpu_util import to_dev
    inp = synth.make_inputs(variant, len(lens), H, G, d, dr, lens, scale=1 / math.sqrt(d + dr), seed=25,
                            kv_dtype=kv, q_len=Q)
    _check(inp, num_splits=splits)
    bt = torch.from_numpy(inp.layout.block_table).cuda()
    sl = torch.from_numpy(inp.layout.seq_lens).cuda()
    mk = lambda: lkd.Decoder(to_dev(inp.q_lat), to_dev(inp.q_rope), to_dev(inp.k_pool), bt, sl,  # noqa: E731
                             variant=variant, scale=inp.scale, groups=G, v=to_dev(inp.v_pool),
                             rope=to_dev(inp.rope_pool), kscale=to_dev(inp.scale_pool), num_splits=splits, q_len=Q)
    fused, staged = mk(), mk()
    fused.run()
    staged.plan()
    staged.decode()
    staged.combine()
    torch.cuda.synchronize()
    assert torch.equal(fused.out, staged.out) and torch.equal(fused.lse, staged.lse)


# --- the device planner (ld_plan's kernel and the decode kernel's fused prologue) against the host
# planner ld_plan_host: unit count and chunk (header words 0 and 1, at the start of the workspace)
# and every unit record (from byte 256), for batches within one wave of lengths, above it (the
# lengths are cached 64 per register) and above the 1,024 cached lengths
@pytest.mark.parametrize("lens_kind,splits", [("one_long", 0), ("b64", 0), ("b300", 0), ("b1500", 0), ("b300", 3)])
def test_device_plan_matches_host_plan(lens_kind, splits):
    import latent_kv_cache_absorbed_amd as lkd
    from gpu_util import to_dev
    r = np.random.default_rng(41)
    lens = {"one_long": [40000], "b64": list(r.integers(1, 5000, 64)),
            "b300": list(r.integers(0, 700, 300)), "b1500": list(r.integers(0, 300, 1500))}[lens_kind]
    inp = synth.make_inputs("mla", len(lens), 128, 1, 512, 64, lens, scale=_S, seed=42)
    print(f"case device plan {lens_kind} splits={splits} B={len(lens)}", flush=True)
    bt = torch.from_numpy(inp.layout.block_table).cuda()
    sl = torch.from_numpy(inp.layout.seq_lens).cuda()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for fused in (False, True):
        d = lkd.Decoder(to_dev(inp.q_lat), to_dev(inp.q_rope), to_dev(inp.k_pool), bt, sl, variant="mla",
                        scale=inp.scale, num_splits=splits)
        d.workspace.fill_(0xFF)
        if fused:
            d.run()
        else:
            d.plan()
        torch.cuda.synchronize()
        chunk, units, ns, first = lkd.plan_host(d.problem, inp.layout.seq_lens, cus)
        ws = d.workspace.cpu().numpy()
        header = ws[:16].view(np.int32)
        assert header[0] == units and (splits > 0 or header[1] == chunk), (header[:2], units, chunk)
        rec = ws[256:256 + 16 * units].view(np.int32).reshape(units, 4)
        for b in range(len(lens)):
            if ns[b] == 0:
                continue
            ck = chunk if splits == 0 else max(64, -(-(-(-int(lens[b]) // splits)) // 64) * 64)
            for s_ in range(ns[b]):
                u = first[b] + s_
                assert list(rec[u]) == [b, s_ * ck, min(int(lens[b]), (s_ + 1) * ck), s_], (fused, b, s_, rec[u])


# --- the whole step (plan + decode + one- and two-level combine) captured in a HIP graph: every
# replay, with eager work on the same buffers in between, reproduces the eager result bit for bit
@pytest.mark.parametrize("lens", [[1500, 77, 3000], [40000]])
def test_graph_replay_matches_eager(lens):
    import latent_kv_cache_absorbed_amd as lkd
    from gpu_util import to_dev
    inp = synth.make_inputs("mla", len(lens), 128, 1, 512, 64, lens, scale=1 / math.sqrt(192), seed=23)
    print(f"case graph replay lens={lens}", flush=True)
    bt = torch.from_numpy(inp.layout.block_table).cuda()
    sl = torch.from_numpy(inp.layout.seq_lens).cuda()
    d = lkd.Decoder(to_dev(inp.q_lat), to_dev(inp.q_rope), to_dev(inp.k_pool), bt, sl, variant="mla",
                    scale=inp.scale)
    out0, lse0 = (t.clone() for t in d.run())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        d.run()
    torch.cuda.synchronize()
    for r in range(4):
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        d.workspace.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out, out0) and torch.equal(d.lse, lse0), f"replay {r} differs from the eager run"


def test_plan_decode_then_combine_is_the_step():
    """ld_plan_decode followed by ld_combine_planned gives ld_latent_decode's bits (the benchmark times the
    decode kernel inside the step this way)."""
    import latent_kv_cache_absorbed_amd as lkd
    from gpu_util import to_dev
    for lens in ([40000] + [300 + 97 * i for i in range(9)], [5000, 64, 2600]):
        inp = synth.make_inputs("mla", len(lens), 128, 1, 512, 64, lens, scale=_S, seed=33)
        bt = torch.from_numpy(inp.layout.block_table).cuda()
        sl = torch.from_numpy(inp.layout.seq_lens).cuda()
        mk = lambda: lkd.Decoder(to_dev(inp.q_lat), to_dev(inp.q_rope), to_dev(inp.k_pool), bt, sl,  # noqa: E731
                                 variant="mla", scale=inp.scale)
        one, two = mk(), mk()
        two.out.fill_(float("nan"))
        two.workspace.fill_(0xFF)
        one.run()
        two.plan_decode()
        two.combine()
        torch.cuda.synchronize()
        assert torch.equal(one.out, two.out) and torch.equal(one.lse, two.lse)
