"""GPU parity of ld_cache_append against the CPU oracle (needs an MI355X).

Bytes the method fixes exactly are compared bit for bit: the latent copy, the E4M3 codes and the fp32
scale of an fp8 cache (both sides decide them in fp32), and every cache slot the append must not
touch.  The rotated RoPE key is compared with the oracle's fp64 rotation to one unit in the last
place of the cache dtype (bf16: 2^-7 relative; f32: 2^-22 relative), since both round an fp64 value.
"""
import math

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


_TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _case(variant, groups, d_lat, d_rope, lens, *, kv="bf16", inp="bf16", page=64, num_pages=40, max_pages=None,
          seed=0, base=10000.0):
    import latent_kv_cache_absorbed_amd as lkd
    r = np.random.default_rng(seed)
    B = len(lens)
    lens = np.asarray(lens, np.int32)
    if max_pages is None:
        max_pages = max(1, int(math.ceil(max(lens.max(), 1) / page)))
    # any page may serve any sequence here (only one slot per sequence is written); distinct slots
    table = r.integers(0, num_pages, size=(B, max_pages)).astype(np.int32)
    for b in range(B):                                    # make the B target slots distinct
        if lens[b] >= 1:
            table[b, (lens[b] - 1) // page] = b % num_pages
    D = groups * d_lat
    c = torch.from_numpy(r.normal(0, 2.0, (B, D)).astype(np.float32)).to(_TDT[inp])
    kr = torch.from_numpy(r.normal(0, 1.0, (B, d_rope)).astype(np.float32)).to(_TDT[inp])
    dev = torch.device("cuda")
    if kv == "fp8_e4m3":
        k0 = torch.from_numpy(r.integers(0, 0x7F, size=(num_pages, page, D)).astype(np.uint8))
        rope0 = torch.from_numpy(r.normal(size=(num_pages, page, d_rope)).astype(np.float32)).to(torch.bfloat16)
        sc0 = torch.from_numpy(r.uniform(0.5, 2, size=(num_pages, page)).astype(np.float32))
    else:
        k0 = torch.from_numpy(r.normal(size=(num_pages, page, D + d_rope)).astype(np.float32)).to(_TDT[kv])
        rope0 = sc0 = None
    k = k0.to(dev)
    rope = None if rope0 is None else rope0.to(dev)
    sc = None if sc0 is None else sc0.to(dev)
    print(f"case append {variant} G={groups} d={d_lat}+{d_rope} kv={kv} in={inp} lens={list(lens)[:6]}", flush=True)
    lkd.cache_append(c.to(dev), kr.to(dev), k, torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev),
                     variant=variant, groups=groups, rope_base=base, rope=rope, kscale=sc)
    torch.cuda.synchronize()
    writes = oracle.cache_append(c.float().numpy(), kr.double().numpy(), table, lens, page_size=page,
                                 fp8=(kv == "fp8_e4m3"), base=base)
    return writes, (k0, rope0, sc0), (k.cpu(), None if rope is None else rope.cpu(), None if sc is None else sc.cpu())


def _ulp_close(got, ref, rel):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.abs(got - ref) <= rel * np.maximum(np.abs(ref), 1e-30) + 1e-300), (got, ref)


def _check(writes, before, after, kv, d_lat_total, d_rope, inp_dtype):
    k0, rope0, sc0 = before
    k1, rope1, sc1 = after
    touched = np.zeros(k0.shape[:2], bool)
    rel = 2.0 ** -22 if kv == "f32" else 2.0 ** -7
    for w in writes:
        p, s = w["page"], w["slot"]
        touched[p, s] = True
        if kv == "fp8_e4m3":
            np.testing.assert_array_equal(k1[p, s].numpy(), w["codes"])
            assert sc1[p, s].item() == float(w["scale"])
            _ulp_close(rope1[p, s].double().numpy(), w["rope"], rel)
        else:
            lat = torch.from_numpy(w["latent"]).to(_TDT[inp_dtype]).to(_TDT[kv])   # the input, in the cache dtype
            np.testing.assert_array_equal(k1[p, s, :d_lat_total].double().numpy(), lat.double().numpy())
            _ulp_close(k1[p, s, d_lat_total:].double().numpy(), w["rope"], rel)
    # nothing else changed
    np.testing.assert_array_equal(k1[~touched].view(torch.uint8).numpy(), k0[~touched].view(torch.uint8).numpy())
    if rope0 is not None:
        np.testing.assert_array_equal(rope1[~touched].view(torch.int16).numpy(), rope0[~touched].view(torch.int16).numpy())
        np.testing.assert_array_equal(sc1[~touched].numpy(), sc0[~touched].numpy())


@pytest.mark.parametrize("lens", [[1, 64, 65, 300], [4096] * 3, [0, 17, 0, 2]])
def test_append_mla_bf16(lens):
    writes, before, after = _case("mla", 1, 512, 64, lens, seed=1)
    assert len(writes) == sum(1 for L in lens if L >= 1)
    _check(writes, before, after, "bf16", 512, 64, "bf16")


def test_append_mla_fp8():
    writes, before, after = _case("mla", 1, 512, 64, [1, 700, 64, 1300], kv="fp8_e4m3", seed=2)
    _check(writes, before, after, "fp8_e4m3", 512, 64, "bf16")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_append_gla2(kv):
    writes, before, after = _case("gla", 2, 256, 64, [5, 900, 4097], kv=kv, seed=3)
    _check(writes, before, after, kv, 512, 64, "bf16")


def test_append_mlra4():
    writes, before, after = _case("mlra", 4, 128, 64, [33, 1], seed=4)
    _check(writes, before, after, "bf16", 512, 64, "bf16")


def test_append_f32_cache_and_f32_input_to_bf16_cache():
    writes, before, after = _case("mla", 1, 64, 16, [3, 250], kv="f32", inp="f32", page=16, seed=5)
    _check(writes, before, after, "f32", 64, 16, "f32")
    writes, before, after = _case("mla", 1, 64, 16, [3, 250], kv="bf16", inp="f32", page=16, seed=6)
    _check(writes, before, after, "bf16", 64, 16, "f32")


def test_append_at_a_million_tokens():
    # positions near 2^20: the rotation angles reach 10^6 radians
    writes, before, after = _case("mla", 1, 512, 64, [1048576, 1000003], max_pages=16384, num_pages=8, seed=7)
    _check(writes, before, after, "bf16", 512, 64, "bf16")


def test_append_zero_rows_and_huge_values_fp8():
    import latent_kv_cache_absorbed_amd as lkd
    dev = torch.device("cuda")
    c = torch.zeros((3, 512), dtype=torch.bfloat16)
    c[1, 7] = 3.0e38
    c[1, 8] = -1.0e-30
    c[2] = torch.linspace(-1e-3, 1e-3, 512).to(torch.bfloat16)
    kr = torch.zeros((3, 64), dtype=torch.bfloat16)
    k = torch.zeros((4, 64, 512), dtype=torch.uint8, device=dev)
    rope = torch.zeros((4, 64, 64), dtype=torch.bfloat16, device=dev)
    sc = torch.zeros((4, 64), dtype=torch.float32, device=dev)
    table = torch.tensor([[0], [1], [2]], dtype=torch.int32)
    lens = torch.tensor([1, 2, 3], dtype=torch.int32)
    lkd.cache_append(c.to(dev), kr.to(dev), k, table.to(dev), lens.to(dev), rope=rope, kscale=sc)
    torch.cuda.synchronize()
    for w in oracle.cache_append(c.float().numpy(), kr.double().numpy(), table.numpy(), lens.numpy(), page_size=64,
                                 fp8=True):
        np.testing.assert_array_equal(k[w["page"], w["slot"]].cpu().numpy(), w["codes"])
        assert sc[w["page"], w["slot"]].item() == float(w["scale"])


def test_append_skips_invalid_metadata():
    """A block-table entry outside the pool (-1, num_pages) or a length above the table's capacity writes
    nothing: every byte of every pool is unchanged, while the valid sequences in the same call are written."""
    import latent_kv_cache_absorbed_amd as lkd
    r = np.random.default_rng(9)
    page, num_pages, max_pages = 64, 6, 2
    lens = np.array([10, 70, 129, 128, 1], np.int32)    # 129 > capacity 128
    table = np.array([[-1, 0], [1, 6], [2, 3], [4, 5], [0, 1]], np.int32)   # b0: page -1, b1: page 6
    dev = torch.device("cuda")
    for kv in ("bf16", "fp8_e4m3"):
        c = torch.from_numpy(r.normal(size=(5, 512)).astype(np.float32)).to(torch.bfloat16)
        kr = torch.from_numpy(r.normal(size=(5, 64)).astype(np.float32)).to(torch.bfloat16)
        if kv == "fp8_e4m3":
            k0 = torch.from_numpy(r.integers(0, 0x7F, size=(num_pages, page, 512)).astype(np.uint8))
            rope0 = torch.from_numpy(r.normal(size=(num_pages, page, 64)).astype(np.float32)).to(torch.bfloat16)
            sc0 = torch.from_numpy(r.uniform(0.5, 2, size=(num_pages, page)).astype(np.float32))
        else:
            k0 = torch.from_numpy(r.normal(size=(num_pages, page, 576)).astype(np.float32)).to(torch.bfloat16)
            rope0 = sc0 = None
        k = k0.to(dev)
        rope = None if rope0 is None else rope0.to(dev)
        sc = None if sc0 is None else sc0.to(dev)
        print(f"case append invalid metadata kv={kv} lens={list(lens)}", flush=True)
        lkd.cache_append(c.to(dev), kr.to(dev), k, torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev),
                         rope=rope, kscale=sc)
        torch.cuda.synchronize()
        writes = oracle.cache_append(c.float().numpy(), kr.double().numpy(), table, lens, page_size=page,
                                     fp8=(kv == "fp8_e4m3"), num_pages=num_pages)
        assert sorted(w["b"] for w in writes) == [3, 4]       # b0, b1 (bad page) and b2 (too long) skipped
        after = (k.cpu(), None if rope is None else rope.cpu(), None if sc is None else sc.cpu())
        _check(writes, (k0, rope0, sc0), after, kv, 512, 64, "bf16")
