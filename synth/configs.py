"""Workload shapes and the seeded problem builder used by tests and the benchmark.

A problem is one decode step: every sequence has one query token per head at
position L_b - 1, and its cache holds L_b rows (the current token included).

Variants and what one cache row holds:

* ``mla``   one shared row per token: latent c (d_lat) followed by the already
            rotated RoPE key (d_rope); every head scores against the whole row
            and averages the latent part.
* ``gla``   ``groups`` latent slices of d_lat each, then one shared RoPE key;
            head h belongs to group h // (H / groups) and uses its group's slice.
* ``mlra``  ``groups`` latent branches of d_lat each, then one shared RoPE key;
            every head attends every branch separately (one softmax per branch).
* ``gqa`` / ``mqa`` / ``gta``  per-kv-head K (and V) rows of d_lat dims, no RoPE
            segment; ``gta`` has one tied state that serves as both K and V.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from .inputs import PagedLayout, fill_pool, fill_pool_e4m3, generator, normal_tensor, plan_pages

__all__ = ["Workload", "WORKLOADS", "DecodeInputs", "make_inputs", "uniform_lengths", "kv_bytes_per_token",
           "LATENT_VARIANTS", "SHARED_VARIANTS"]

LATENT_VARIANTS = ("mla", "gla", "mlra")
SHARED_VARIANTS = ("gqa", "mqa", "gta")


@dataclass(frozen=True)
class Workload:
    name: str
    variant: str
    batch: int
    heads: int
    groups: int
    d_lat: int
    d_rope: int
    seq_len: int | tuple          # one length for all sequences, or ("uniform", lo, hi)
    page_size: int = 64
    kv_dtype: str = "bf16"
    q_dtype: str = "bf16"
    out_dtype: str = "bf16"
    scale: float = 1.0
    shuffle: bool = True
    seed: int = 0
    q_len: int = 1

    def lengths(self) -> np.ndarray:
        if isinstance(self.seq_len, tuple):
            _, lo, hi = self.seq_len
            return uniform_lengths(self.seed, self.batch, lo, hi)
        return np.full(self.batch, int(self.seq_len), np.int32)


def uniform_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths drawn uniformly from the integers in [lo, hi]."""
    return generator(seed, 6).integers(lo, hi + 1, size=batch).astype(np.int32)


_S192 = 1.0 / math.sqrt(192.0)
_S128 = 1.0 / math.sqrt(128.0)

WORKLOADS = {
    # tiny fp32 absorbed MLA, contiguous (identity block table)
    "mla_tiny_f32": Workload("mla_tiny_f32", "mla", 2, 16, 1, 64, 16, 256, kv_dtype="f32", q_dtype="f32",
                             out_dtype="f32", scale=1.0 / math.sqrt(48.0), shuffle=False, seed=1),
    # DeepSeek-V3-shaped batch decode
    "mla_b64_l4k": Workload("mla_b64_l4k", "mla", 64, 128, 1, 512, 64, 4096, scale=_S192, seed=2),
    # long single-sequence decode
    "mla_b1_l128k": Workload("mla_b1_l128k", "mla", 1, 128, 1, 512, 64, 131072, scale=_S192, seed=3),
    "mla_b1_l512k": Workload("mla_b1_l512k", "mla", 1, 128, 1, 512, 64, 524288, scale=_S192, seed=3),
    "mla_b1_l1m": Workload("mla_b1_l1m", "mla", 1, 128, 1, 512, 64, 1048576, scale=_S192, seed=3),
    "mlra4_b1_l128k": Workload("mlra4_b1_l128k", "mlra", 1, 128, 4, 128, 64, 131072, scale=_S192, seed=3),
    "mlra4_b1_l512k": Workload("mlra4_b1_l512k", "mlra", 1, 128, 4, 128, 64, 524288, scale=_S192, seed=3),
    "mlra4_b1_l1m": Workload("mlra4_b1_l1m", "mlra", 1, 128, 4, 128, 64, 1048576, scale=_S192, seed=3),
    # shared-KV baselines
    "gqa_b32_l32k": Workload("gqa_b32_l32k", "gqa", 32, 64, 8, 128, 0, 32768, scale=_S128, seed=4),
    "mqa_b32_l32k": Workload("mqa_b32_l32k", "mqa", 32, 64, 1, 128, 0, 32768, scale=_S128, seed=4),
    "gta_b32_l32k": Workload("gta_b32_l32k", "gta", 32, 64, 8, 128, 0, 32768, scale=_S128, seed=4),
    # speculative decode over the DeepSeek-V3-shaped batch: two and four query tokens per sequence
    "mla_q2_b64_l4k": Workload("mla_q2_b64_l4k", "mla", 64, 128, 1, 512, 64, 4096, scale=_S192, seed=2, q_len=2),
    "mla_q4_b64_l4k": Workload("mla_q4_b64_l4k", "mla", 64, 128, 1, 512, 64, 4096, scale=_S192, seed=2, q_len=4),
    # one kv head of a large head dim (the MFA-style cache: MQA with d >> 128)
    "mqa_d512_b32_l32k": Workload("mqa_d512_b32_l32k", "mqa", 32, 64, 1, 512, 0, 32768,
                                  scale=1.0 / math.sqrt(512.0), seed=4),
    # GLA-2 over an fp8 latent cache with imbalanced lengths
    "gla2_fp8_b64_mixed": Workload("gla2_fp8_b64_mixed", "gla", 64, 128, 2, 256, 64, ("uniform", 1024, 65536),
                                   kv_dtype="fp8_e4m3", scale=_S192, seed=5),
    # one GPU's share under the tensor-parallel layouts the pages describe: one MLRA-4 branch (all
    # 128 heads, a 128-dim latent block + the shared rope key) under TP-4, and one GLA-2 latent group
    # (its 64 heads, a 256-dim latent + rope) under TP-2
    "mlra4_tp4_share_b1_l128k": Workload("mlra4_tp4_share_b1_l128k", "mlra", 1, 128, 1, 128, 64, 131072,
                                         scale=_S192, seed=3),
    "mlra4_tp4_share_b1_l1m": Workload("mlra4_tp4_share_b1_l1m", "mlra", 1, 128, 1, 128, 64, 1048576,
                                       scale=_S192, seed=3),
    "gla2_tp2_share_fp8_b64_mixed": Workload("gla2_tp2_share_fp8_b64_mixed", "gla", 64, 64, 1, 256, 64,
                                             ("uniform", 1024, 65536), kv_dtype="fp8_e4m3", scale=_S192, seed=5),
}


def kv_bytes_per_token(variant: str, groups: int, d_lat: int, d_rope: int, kv_dtype: str) -> int:
    """Algorithmic cache bytes one token contributes (each stored byte read once)."""
    if variant in LATENT_VARIANTS:
        if kv_dtype == "fp8_e4m3":
            return groups * d_lat + 2 * d_rope + 4
        el = 4 if kv_dtype == "f32" else 2
        return el * (groups * d_lat + d_rope)
    el = 4 if kv_dtype == "f32" else 2
    per = groups * d_lat * el
    return per if variant == "gta" else 2 * per


@dataclass
class DecodeInputs:
    """Host (CPU) tensors of one decode problem, in the library's layouts."""

    variant: str
    heads: int
    groups: int
    d_lat: int
    d_rope: int
    scale: float
    layout: PagedLayout
    kv_dtype: str
    q_dtype: str
    out_dtype: str
    q_lat: torch.Tensor                 # [B,H,d] | [B,H,G,d] (mlra)
    q_rope: torch.Tensor | None         # [B,H,dr] | [B,H,G,dr] (mlra) | None
    k_pool: torch.Tensor                # latent: [P,page,G*d+dr] (or fp8 codes [P,page,G*d]); shared: [P,page,G,d]
    rope_pool: torch.Tensor | None      # fp8 only: bf16 [P,page,dr]
    scale_pool: torch.Tensor | None     # fp8 only: f32 [P,page]
    v_pool: torch.Tensor | None         # gqa/mqa: [P,page,G,d]
    q_len: int = 1                      # query tokens per sequence; q_lat/q_rope then hold q_len*H rows

    @property
    def batch(self) -> int:
        return self.layout.batch

    @property
    def d_v(self) -> int:
        return self.d_lat

    @property
    def rows_per_seq(self) -> int:
        return self.heads * self.q_len * (self.groups if self.variant == "mlra" else 1)

    def kv_bytes(self) -> int:
        per = kv_bytes_per_token(self.variant, self.groups, self.d_lat, self.d_rope, self.kv_dtype)
        return per * int(self.layout.seq_lens.astype(np.int64).sum())


def make_inputs(variant: str, batch: int, heads: int, groups: int, d_lat: int, d_rope: int, seq_lens,
                *, page_size: int = 64, kv_dtype: str = "bf16", q_dtype: str = "bf16", out_dtype: str = "bf16",
                scale: float = 1.0, shuffle: bool = True, seed: int = 0, poison: bool = True,
                max_pages_per_seq: int | None = None, spare_pages: int = 1, q_len: int = 1) -> DecodeInputs:
    """Draw one seeded decode problem.  All values are N(0,1) in their storage type.  With q_len > 1
    (mla, mqa) every sequence has q_len query tokens: q_lat / q_rope hold q_len*H rows, row i*H + h."""
    if variant not in LATENT_VARIANTS + SHARED_VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    seq_lens = np.broadcast_to(np.asarray(seq_lens, np.int64), (batch,)).copy()
    layout = plan_pages(generator(seed, 0), seq_lens, page_size, shuffle=shuffle,
                        max_pages_per_seq=max_pages_per_seq, spare_pages=spare_pages)
    rope_pool = scale_pool = v_pool = q_rope = None
    if variant in LATENT_VARIANTS:
        if variant == "mlra":
            q_lat = normal_tensor(generator(seed, 1), (batch, q_len * heads, groups, d_lat), q_dtype)
            q_rope = normal_tensor(generator(seed, 2), (batch, q_len * heads, groups, d_rope), q_dtype)
        else:
            q_lat = normal_tensor(generator(seed, 1), (batch, q_len * heads, d_lat), q_dtype)
            q_rope = normal_tensor(generator(seed, 2), (batch, q_len * heads, d_rope), q_dtype)
        if kv_dtype == "fp8_e4m3":
            k_pool, scale_pool = fill_pool_e4m3(generator(seed, 3), layout, groups * d_lat, poison=poison)
            rope_pool = fill_pool(generator(seed, 4), layout, (d_rope,), "bf16", poison=poison)
        else:
            k_pool = fill_pool(generator(seed, 3), layout, (groups * d_lat + d_rope,), kv_dtype, poison=poison)
    else:
        if d_rope != 0:
            raise ValueError("shared-KV variants carry no RoPE segment")
        if kv_dtype == "fp8_e4m3":
            raise ValueError("the fp8 cache path covers the latent variants")
        q_lat = normal_tensor(generator(seed, 1), (batch, q_len * heads, d_lat), q_dtype)
        k_pool = fill_pool(generator(seed, 3), layout, (groups, d_lat), kv_dtype, poison=poison)
        if variant != "gta":
            v_pool = fill_pool(generator(seed, 5), layout, (groups, d_lat), kv_dtype, poison=poison)
    return DecodeInputs(variant=variant, heads=heads, groups=groups, d_lat=d_lat, d_rope=d_rope, scale=float(scale),
                        layout=layout, kv_dtype=kv_dtype, q_dtype=q_dtype, out_dtype=out_dtype, q_lat=q_lat,
                        q_rope=q_rope, k_pool=k_pool, rope_pool=rope_pool, scale_pool=scale_pool, v_pool=v_pool,
                        q_len=q_len)


def make_workload_inputs(w: Workload, **overrides) -> DecodeInputs:
    kw = dict(page_size=w.page_size, kv_dtype=w.kv_dtype, q_dtype=w.q_dtype, out_dtype=w.out_dtype,
              scale=w.scale, shuffle=w.shuffle, seed=w.seed, q_len=w.q_len)
    kw.update(overrides)
    lens = kw.pop("seq_lens", None)
    batch = kw.pop("batch", w.batch)
    if lens is None:
        lens = w.lengths()[:batch] if batch <= w.batch else np.resize(w.lengths(), batch)
    return make_inputs(w.variant, batch, w.heads, w.groups, w.d_lat, w.d_rope, lens, **kw)


__all__.append("make_workload_inputs")
