"""Host tests of the Python binding's shape checks (no GPU): every buffer the library reads on the device
must agree with the shape derived from q_latent, or the binding raises before anything is queued."""
import pytest
import torch

from latent_kv_cache_absorbed_amd.binding import decode_shapes


def _mla(B=3, H=128, P=10, page=64, dr=64, d=512, mp=4, fp8=False):
    t = dict(q_latent=torch.empty(B, H, d, dtype=torch.bfloat16), q_rope=torch.empty(B, H, dr, dtype=torch.bfloat16),
             block_table=torch.empty(B, mp, dtype=torch.int32), seq_lens=torch.empty(B, dtype=torch.int32))
    if fp8:
        t.update(k=torch.empty(P, page, d, dtype=torch.uint8), rope=torch.empty(P, page, dr, dtype=torch.bfloat16),
                 kscale=torch.empty(P, page, dtype=torch.float32))
    else:
        t.update(k=torch.empty(P, page, d + dr, dtype=torch.bfloat16))
    return t


def _call(t, variant="mla", **kw):
    t = dict(t)
    args = [t.pop(n) for n in ("q_latent", "q_rope", "k", "block_table", "seq_lens")]
    return decode_shapes(*args, variant=variant, **t, **kw)


def test_valid_shapes_pass():
    assert _call(_mla()) == (3, 128, 1, 512, 64)
    assert _call(_mla(fp8=True)) == (3, 128, 1, 512, 64)
    g = _mla(d=256)
    g["k"] = torch.empty(10, 64, 2 * 256 + 64, dtype=torch.bfloat16)
    assert _call(g, "gla", groups=2) == (3, 128, 2, 256, 64)
    assert _call(g, "gla") == (3, 128, 2, 256, 64)
    m = dict(q_latent=torch.empty(1, 128, 4, 128, dtype=torch.bfloat16),
             q_rope=torch.empty(1, 128, 4, 64, dtype=torch.bfloat16), k=torch.empty(5, 64, 576, dtype=torch.bfloat16),
             block_table=torch.empty(1, 5, dtype=torch.int32), seq_lens=torch.empty(1, dtype=torch.int32))
    assert _call(m, "mlra") == (1, 128, 4, 128, 64)
    s = dict(q_latent=torch.empty(2, 64, 128, dtype=torch.bfloat16), q_rope=None,
             k=torch.empty(7, 64, 8, 128, dtype=torch.bfloat16), block_table=torch.empty(2, 3, dtype=torch.int32),
             seq_lens=torch.empty(2, dtype=torch.int32), v=torch.empty(7, 64, 8, 128, dtype=torch.bfloat16))
    assert _call(s, "gqa") == (2, 64, 8, 128, 0)
    s.pop("v")
    assert _call(s, "gta") == (2, 64, 8, 128, 0)
    assert _call(_mla(H=256), q_len=2) == (3, 128, 1, 512, 64)


@pytest.mark.parametrize("what", ["short_seq_lens", "long_seq_lens", "2d_seq_lens", "few_table_rows", "1d_table",
                                  "q_rope_heads", "q_rope_batch", "k_row", "k_dims"])
def test_mla_mismatch_raises(what):
    t = _mla()
    if what == "short_seq_lens":
        t["seq_lens"] = torch.empty(2, dtype=torch.int32)
    elif what == "long_seq_lens":
        t["seq_lens"] = torch.empty(4, dtype=torch.int32)
    elif what == "2d_seq_lens":
        t["seq_lens"] = torch.empty(3, 1, dtype=torch.int32)
    elif what == "few_table_rows":
        t["block_table"] = torch.empty(2, 4, dtype=torch.int32)
    elif what == "1d_table":
        t["block_table"] = torch.empty(12, dtype=torch.int32)
    elif what == "q_rope_heads":
        t["q_rope"] = torch.empty(3, 64, 64, dtype=torch.bfloat16)
    elif what == "q_rope_batch":
        t["q_rope"] = torch.empty(2, 128, 64, dtype=torch.bfloat16)
    elif what == "k_row":
        t["k"] = torch.empty(10, 64, 512, dtype=torch.bfloat16)
    elif what == "k_dims":
        t["k"] = torch.empty(10, 64, 1, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _call(t)


@pytest.mark.parametrize("what", ["rope_pages", "rope_dims", "scale_pages", "scale_missing"])
def test_fp8_pool_mismatch_raises(what):
    t = _mla(fp8=True)
    if what == "rope_pages":
        t["rope"] = torch.empty(9, 64, 64, dtype=torch.bfloat16)
    elif what == "rope_dims":
        t["rope"] = torch.empty(10, 64, 32, dtype=torch.bfloat16)
    elif what == "scale_pages":
        t["kscale"] = torch.empty(10, 32, dtype=torch.float32)
    else:
        t["kscale"] = None
    with pytest.raises(ValueError):
        _call(t)


def test_shared_kv_mismatch_raises():
    base = dict(q_latent=torch.empty(2, 64, 128, dtype=torch.bfloat16), q_rope=None,
                k=torch.empty(7, 64, 8, 128, dtype=torch.bfloat16), block_table=torch.empty(2, 3, dtype=torch.int32),
                seq_lens=torch.empty(2, dtype=torch.int32))
    with pytest.raises(ValueError):                       # GQA without V
        _call(base, "gqa")
    with pytest.raises(ValueError):                       # V of another shape
        _call(dict(base, v=torch.empty(6, 64, 8, 128, dtype=torch.bfloat16)), "gqa")
    with pytest.raises(ValueError):                       # head dim of K differs from the query's
        _call(dict(base, k=torch.empty(7, 64, 8, 64, dtype=torch.bfloat16)), "gta")
    with pytest.raises(ValueError):                       # groups argument contradicts K
        _call(base, "gta", groups=4)


def test_bad_variant_and_q_len():
    with pytest.raises(ValueError):
        _call(_mla(), "mha")
    with pytest.raises(ValueError):
        _call(_mla(H=128), q_len=3)                       # 128 rows not a multiple of 3
    with pytest.raises(ValueError):                       # mlra needs [B, H, G, d] queries
        _call(_mla(), "mlra")
