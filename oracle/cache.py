"""Plain statement of appending one decode step's token to the paged latent cache.

TEST INFRASTRUCTURE: used by tests, the smoke check and the benchmark's CPU
baseline only.  The GPU library never imports it and shares no code with it.

What is appended (sources cited by page title and section):

* [MLA-RoPE]  the MLA explainer on mlqm.cn (news 371735), section 2.2: the key
  has a semantic part (the compressed latent c^KV) and a separate position part
  k^R that carries RoPE; section 2.4: what the cache keeps per token.
* [MLRA]  "超越MLA！新架构MLRA百万token，解码最高2.8倍速 | ICLR'26" (aitntnews), the
  MLA paragraph: only the latent and the decoupled RoPE key are cached, one
  shared 576-dim row per token.
* [GTA-GLA]  the GTA/GLA page (jsbsmhs.com): the large model is served in FP8.

Readings where the pages are silent: the new token sits
at logical position L - 1 of a sequence whose length L already counts it; its
RoPE key is rotated by that position before it is stored (the [MLRA] reading;
[MLA-RoPE] section 2.4's "recompute k^R every step" is the other one); RoPE
rotates consecutive pairs by pos * base^(-2i/d) (``attention.rope``); an fp8
cache stores OCP E4M3 codes of latent / scale with one fp32 scale per token,
scale = amax / 448 computed in fp32 (1 for an all-zero row), the quotient
latent / scale rounded in fp32 and clamped to +-448, then rounded to the
nearest code with ties to the even code; the RoPE key of an fp8 cache is kept
in bf16 in its own pool.
"""
from __future__ import annotations

import numpy as np

from .attention import _E4M3_TABLE, rope

__all__ = ["E4M3_MAX", "e4m3_encode", "quantize_row_e4m3", "append_slot", "cache_append"]

E4M3_MAX = 448.0

# non-negative finite codes 0x00 .. 0x7E in increasing value order (code order is value order)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _E4M3_TABLE[:0x7F]


def e4m3_encode(y):
    """Nearest OCP E4M3 code of each (float) value in [-448, 448], ties to the even code.

    The sign bit is the value's sign bit (so -0.0 gives 0x80).  Written from the
    format's definition: the candidate codes are all finite non-negative codes,
    and the nearest by absolute difference wins.
    """
    y = np.asarray(y, np.float64)
    if np.any(np.abs(y) > E4M3_MAX) or np.any(np.isnan(y)):
        raise ValueError("e4m3_encode takes finite values in [-448, 448]")
    a = np.abs(y)
    # index of the first table value >= a, and the one below it
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], code)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_row_e4m3(c):
    """E4M3 codes and fp32 scale of one token's latent row (all its groups share the scale)."""
    c32 = np.asarray(c, np.float32)
    amax = np.float32(np.max(np.abs(c32))) if c32.size else np.float32(0)
    scale = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    y = np.clip(c32 / scale, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))   # fp32 division
    return e4m3_encode(y), scale


def append_slot(block_table_row, L: int, page_size: int):
    """(physical page, slot) of logical position L - 1 of a sequence of length L."""
    pos = int(L) - 1
    return int(np.asarray(block_table_row)[pos // page_size]), pos % page_size


def cache_append(c_new, kr_new, block_table, seq_lens, *, page_size: int, fp8: bool, base: float = 10000.0,
                 num_pages: int | None = None):
    """What one append writes, per sequence b with 1 <= L_b <= capacity.

    c_new [B, D] (the new token's latent, all groups), kr_new [B, dr] (its
    un-rotated RoPE key).  Returns a list of dicts with b, page, slot, pos and
    either ``latent`` (fp64 values) or ``codes`` / ``scale`` (fp8), plus
    ``rope`` (the rotated key, fp64).

    Reading (the pages do not treat bad metadata): the token is written only to
    the slot the metadata names.  A sequence whose length exceeds the block
    table's capacity (columns x page_size), or whose page entry lies outside
    the pool [0, num_pages) when ``num_pages`` is given, gets no write.
    """
    c_new = np.asarray(c_new)
    kr_new = np.asarray(kr_new, np.float64)
    block_table = np.asarray(block_table)
    capacity = block_table.shape[1] * page_size
    writes = []
    for b in range(c_new.shape[0]):
        L = int(seq_lens[b])
        if L < 1 or L > capacity:
            continue
        page, slot = append_slot(block_table[b], L, page_size)
        if num_pages is not None and not 0 <= page < num_pages:
            continue
        w = {"b": b, "page": page, "slot": slot, "pos": L - 1,
             "rope": rope(kr_new[b], L - 1, base) if kr_new.shape[-1] else np.zeros(0)}
        if fp8:
            w["codes"], w["scale"] = quantize_row_e4m3(c_new[b])
        else:
            w["latent"] = np.asarray(c_new[b], np.float64)
        writes.append(w)
    return writes
