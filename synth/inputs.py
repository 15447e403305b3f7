"""Seeded synthetic tensors and paged-cache layouts.

Every draw comes from numpy's PCG64 seeded by ``SeedSequence([config_id,
tensor_id])`` so a tensor is reproducible from two integers.  Values are drawn
in float32 and then stored in the cache's storage type (fp32, bf16 or OCP
e4m3 with a per-token fp32 scale); the stored values are the inputs, and both
the oracle and the GPU library read exactly those stored values.

Paged cache: the logical rows of sequence ``b`` occupy ``ceil(L_b / page)``
logical pages.  Logical pages are drawn in logical order and then placed at
physical page ``perm[k]`` of one shared pool, where ``perm`` is a seeded random
permutation (or the identity).  ``block_table[b, i]`` names the physical page
that holds logical page ``i`` of sequence ``b``.  Unused table entries point at
a spare page.  Slots past ``L_b`` in a sequence's last page and every spare
page are filled with NaN (bf16/fp32 NaN, e4m3 code 0x7F, NaN scale) so that a
reader that touches a row it must not attend produces NaN.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "generator",
    "normal_tensor",
    "PagedLayout",
    "plan_pages",
    "fill_pool",
    "fill_pool_e4m3",
    "E4M3_MAX",
    "torch_dtype",
]

E4M3_MAX = 448.0          # largest finite OCP E4M3 magnitude
E4M3_NAN_CODE = 0x7F      # S.1111.111 with S = 0


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.float8_e4m3fn}[name]


def generator(config_id: int, tensor_id: int) -> np.random.Generator:
    """PCG64 stream for tensor ``tensor_id`` of configuration ``config_id``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(config_id), int(tensor_id)])))


def _normal_f32(rng: np.random.Generator, n: int, std: float) -> np.ndarray:
    x = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_tensor(rng: np.random.Generator, shape, dtype: str = "bf16", std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) draws stored in ``dtype`` (a CPU torch tensor)."""
    n = int(np.prod(shape)) if len(shape) else 1
    x = torch.from_numpy(_normal_f32(rng, n, std)).reshape(tuple(shape))
    return x.to(torch_dtype(dtype))


@dataclass
class PagedLayout:
    """Where every logical page of every sequence lives in the physical pool."""

    page_size: int
    seq_lens: np.ndarray            # int32 [B]
    block_table: np.ndarray         # int32 [B, max_pages_per_seq]
    num_pages: int                  # physical pages in the pool (incl. spare pages)
    perm: np.ndarray                # logical page index -> physical page index
    first_logical: np.ndarray       # int64 [B]: index of sequence b's first logical page
    spare_pages: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def logical_pages(self) -> int:
        return int(self.perm.shape[0])


def plan_pages(rng: np.random.Generator | None, seq_lens, page_size: int = 64, *,
               max_pages_per_seq: int | None = None, shuffle: bool = True,
               spare_pages: int = 1) -> PagedLayout:
    """Assign physical pages to the logical pages of every sequence."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if np.any(seq_lens < 0):
        raise ValueError("negative sequence length")
    pages_per_seq = (seq_lens + page_size - 1) // page_size
    if max_pages_per_seq is None:
        max_pages_per_seq = max(1, int(pages_per_seq.max(initial=0)))
    if np.any(pages_per_seq > max_pages_per_seq):
        raise ValueError("a sequence needs more pages than max_pages_per_seq")
    n_logical = int(pages_per_seq.sum())
    num_pages = n_logical + spare_pages
    if shuffle:
        if rng is None:
            raise ValueError("shuffle needs a generator")
        order = rng.permutation(num_pages)
    else:
        order = np.arange(num_pages)
    perm = order[:n_logical].astype(np.int64)
    spare = order[n_logical:].astype(np.int64)
    first = np.zeros(len(seq_lens), np.int64)
    if len(seq_lens) > 1:
        first[1:] = np.cumsum(pages_per_seq)[:-1]
    fill = int(spare[0]) if spare_pages > 0 else 0
    table = np.full((len(seq_lens), max_pages_per_seq), fill, dtype=np.int64)
    for b in range(len(seq_lens)):
        n = int(pages_per_seq[b])
        table[b, :n] = perm[first[b]:first[b] + n]
    return PagedLayout(page_size=page_size, seq_lens=seq_lens.astype(np.int32),
                       block_table=table.astype(np.int32), num_pages=num_pages, perm=perm,
                       first_logical=first, spare_pages=spare)


def _poison_slots(layout: PagedLayout):
    """(physical page, first poisoned slot) for every page with slots past its sequence's end."""
    out = []
    for b in range(layout.batch):
        L = int(layout.seq_lens[b])
        if L % layout.page_size:
            last = int(layout.block_table[b, L // layout.page_size])
            out.append((last, L % layout.page_size))
    for p in layout.spare_pages:
        out.append((int(p), 0))
    return out


def fill_pool(rng: np.random.Generator, layout: PagedLayout, row_shape, dtype: str = "bf16",
              std: float = 1.0, poison: bool = True, chunk_pages: int = 2048) -> torch.Tensor:
    """Physical pool [num_pages, page, *row_shape] holding N(0, std^2) logical rows.

    Logical page ``k`` is drawn k-th (so the content of a sequence does not
    depend on the shuffle) and stored at physical page ``perm[k]``.
    """
    row_shape = tuple(int(s) for s in row_shape)
    page = layout.page_size
    per_page = page * int(np.prod(row_shape))
    pool = torch.empty((layout.num_pages, page) + row_shape, dtype=torch_dtype(dtype))
    perm_t = torch.from_numpy(layout.perm)
    for k0 in range(0, layout.logical_pages, chunk_pages):
        k1 = min(layout.logical_pages, k0 + chunk_pages)
        x = torch.from_numpy(_normal_f32(rng, (k1 - k0) * per_page, std))
        pool[perm_t[k0:k1]] = x.reshape((k1 - k0, page) + row_shape).to(pool.dtype)
    if poison:
        for p, s in _poison_slots(layout):
            pool[p, s:] = float("nan")
    else:
        for p, s in _poison_slots(layout):
            pool[p, s:] = 0
    return pool


def fill_pool_e4m3(rng: np.random.Generator, layout: PagedLayout, d_lat: int, *, std: float = 1.0,
                   poison: bool = True, chunk_pages: int = 1024):
    """fp8 latent pool: codes uint8 [P, page, d_lat] (OCP E4M3) and fp32 scale [P, page].

    Each token's latent row is drawn N(0, std^2) in float32, its scale is
    amax/448 (1 for an all-zero row), and the stored code is torch's
    round-to-nearest-even float8_e4m3fn conversion of row/scale (clamped to
    +-448 first, so nothing saturates to NaN).  The cache stores the codes and
    the scale; the value a reader must use is code_value * scale.
    """
    page = layout.page_size
    codes = torch.empty((layout.num_pages, page, d_lat), dtype=torch.uint8)
    scales = torch.empty((layout.num_pages, page), dtype=torch.float32)
    perm_t = torch.from_numpy(layout.perm)
    for k0 in range(0, layout.logical_pages, chunk_pages):
        k1 = min(layout.logical_pages, k0 + chunk_pages)
        x = torch.from_numpy(_normal_f32(rng, (k1 - k0) * page * d_lat, std)).reshape(k1 - k0, page, d_lat)
        amax = x.abs().amax(dim=-1)
        s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        y = (x / s[..., None]).clamp_(-E4M3_MAX, E4M3_MAX)
        codes[perm_t[k0:k1]] = y.to(torch.float8_e4m3fn).view(torch.uint8)
        scales[perm_t[k0:k1]] = s
    for p, s in _poison_slots(layout):
        if poison:
            codes[p, s:] = E4M3_NAN_CODE
            scales[p, s:] = float("nan")
        else:
            codes[p, s:] = 0
            scales[p, s:] = 1.0
    return codes, scales
