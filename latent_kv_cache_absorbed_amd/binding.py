"""Python binding of the C ABI in include/latent_decode.h (ctypes; argument marshalling only).

Every step of the decode runs in the gfx950 kernels of ``liblatent_decode.so``.
This module only checks that tensors are contiguous device tensors of the
right dtype, derives the ``ld_problem`` shape from them, allocates outputs and
the workspace with torch when the caller does not pass them, and calls the
library on torch's current stream.  There is no CPU fallback: if the library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "LatentDecodeError", "Decoder", "lib", "library_path", "Problem", "KVCache", "VARIANTS", "DTYPES",
    "make_problem", "workspace_size", "latent_decode", "decode_shapes", "split_kv_combine", "validate_metadata", "plan_host",
    "cache_append", "head_projection", "NOALLOC_SCRATCH_BYTES",
    "check_problem", "status_string", "header_functions",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "liblatent_decode.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "latent_decode.h")

VARIANTS = {"mla": 0, "gla": 1, "mlra": 2, "gqa": 3, "mqa": 4, "gta": 5}
DTYPES = {"f32": 0, "bf16": 1, "fp8_e4m3": 2}
_TORCH_DTYPE = {torch.float32: "f32", torch.bfloat16: "bf16", torch.uint8: "fp8_e4m3",
                torch.float8_e4m3fn: "fp8_e4m3"}


class LatentDecodeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("variant", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_groups", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("num_splits", ctypes.c_int32),
                ("q_len", ctypes.c_int32)]


class KVCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("rope", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("scale", ctypes.c_void_p)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with `python -m latent_kv_cache_absorbed_amd.build`")
        L = ctypes.CDLL(library_path)
        i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER(Problem)
        ip = ctypes.POINTER(ctypes.c_int32)
        L.ld_abi_version.restype = i32
        L.ld_abi_version.argtypes = []
        L.ld_status_string.restype = ctypes.c_char_p
        L.ld_status_string.argtypes = [i32]
        L.ld_check_problem.restype = i32
        L.ld_check_problem.argtypes = [P]
        L.ld_workspace_size.restype = i32
        L.ld_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
        L.ld_latent_decode.restype = i32
        L.ld_latent_decode.argtypes = [P, vp, vp, ctypes.POINTER(KVCache), vp, vp, vp, vp, vp, sz, vp]
        L.ld_plan_decode.restype = i32
        L.ld_plan_decode.argtypes = [P, vp, vp, ctypes.POINTER(KVCache), vp, vp, vp, vp, vp, sz, vp]
        L.ld_latent_decode_noalloc.restype = i32
        L.ld_latent_decode_noalloc.argtypes = [P, vp, vp, ctypes.POINTER(KVCache), vp, vp, vp, vp, vp]
        L.ld_plan.restype = i32
        L.ld_plan.argtypes = [P, vp, vp, sz, vp]
        L.ld_decode_planned.restype = i32
        L.ld_decode_planned.argtypes = [P, vp, vp, ctypes.POINTER(KVCache), vp, vp, vp, vp, vp, sz, vp]
        L.ld_combine_planned.restype = i32
        L.ld_combine_planned.argtypes = [P, vp, vp, vp, sz, vp]
        L.ld_cache_append.restype = i32
        L.ld_cache_append.argtypes = [P, vp, vp, vp, vp, ctypes.POINTER(KVCache), ctypes.c_float, vp]
        L.ld_head_projection.restype = i32
        L.ld_head_projection.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp]
        L.ld_split_kv_combine.restype = i32
        L.ld_split_kv_combine.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp, vp, vp]
        L.ld_validate_metadata.restype = i32
        L.ld_validate_metadata.argtypes = [P, ip, ip]
        L.ld_plan_host.restype = i32
        L.ld_plan_host.argtypes = [P, ip, i32, ip, ip, ip, ip]
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions include/latent_decode.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ld_\w+)\s*\(", text, re.M)))


def status_string(status: int) -> str:
    try:
        return lib().ld_status_string(int(status)).decode()
    except RuntimeError:
        return f"status {status}"


def make_problem(variant: str, batch: int, heads: int, groups: int, d_latent: int, d_rope: int, page_size: int,
                 num_pages: int, max_pages_per_seq: int, q_dtype: str, kv_dtype: str, out_dtype: str, scale: float,
                 num_splits: int = 0, q_len: int = 1) -> Problem:
    return Problem(ctypes.sizeof(Problem), VARIANTS[variant], batch, heads, groups, d_latent, d_rope, page_size,
                   num_pages, max_pages_per_seq, DTYPES[q_dtype], DTYPES[kv_dtype], DTYPES[out_dtype], float(scale),
                   num_splits, q_len)


def check_problem(p: Problem) -> int:
    return lib().ld_check_problem(ctypes.byref(p))


def workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    st = lib().ld_workspace_size(ctypes.byref(p), ctypes.byref(n))
    if st:
        raise LatentDecodeError(st, "ld_workspace_size")
    return n.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def decode_shapes(q_latent, q_rope, k, block_table, seq_lens, *, variant: str, groups: int | None = None, v=None,
                  rope=None, kscale=None, q_len: int = 1):
    """Check the tensors' shapes against one another (any device) and return (B, H, G, d, d_rope).

    The library reads these buffers on the device with the sizes derived here, so a mismatch (a short
    seq_lens, a block table with too few rows, a query or pool of the wrong shape) raises ValueError
    instead of becoming an out-of-bounds read.
    """
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    if q_len < 1:
        raise ValueError("q_len must be >= 1")
    kv_dtype = _TORCH_DTYPE.get(k.dtype)
    if kv_dtype is None:
        raise ValueError(f"k has dtype {k.dtype}")
    latent = variant in ("mla", "gla", "mlra")
    want_qdim = 4 if variant == "mlra" else 3
    if q_latent.dim() != want_qdim:
        raise ValueError(f"q_latent must have {want_qdim} dims for {variant}, has shape {tuple(q_latent.shape)}")
    B, rows, d = q_latent.shape[0], q_latent.shape[1], q_latent.shape[-1]
    if rows % q_len:
        raise ValueError(f"q_latent has {rows} rows per sequence, not a multiple of q_len={q_len}")
    H = rows // q_len
    if seq_lens.dim() != 1 or seq_lens.numel() != B:
        raise ValueError(f"seq_lens has shape {tuple(seq_lens.shape)}, expected [{B}]")
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.shape[1] < 1:
        raise ValueError(f"block_table has shape {tuple(block_table.shape)}, expected [{B}, max_pages_per_seq]")
    if k.dim() < 3:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected [num_pages, page_size, ...]")
    P, page = k.shape[0], k.shape[1]
    if latent:
        if q_rope is None or q_rope.dim() != want_qdim:
            raise ValueError(f"q_rope must have {want_qdim} dims for {variant}")
        dr = q_rope.shape[-1]
        if variant == "mlra":
            G = q_latent.shape[2]
        elif variant == "mla":
            G = 1
        else:
            lat_cols = k.shape[-1] if kv_dtype == "fp8_e4m3" else k.shape[-1] - dr
            G = groups if groups is not None else lat_cols // d
        if tuple(q_rope.shape[:-1]) != tuple(q_latent.shape[:-1]):
            raise ValueError(f"q_rope has shape {tuple(q_rope.shape)}, q_latent {tuple(q_latent.shape)}")
        row = G * d if kv_dtype == "fp8_e4m3" else G * d + dr
        if k.dim() != 3 or k.shape[2] != row:
            raise ValueError(f"k has shape {tuple(k.shape)}, expected [num_pages, page_size, {row}]")
        if kv_dtype == "fp8_e4m3":
            if rope is None or tuple(rope.shape) != (P, page, dr):
                raise ValueError(f"rope must have shape [{P}, {page}, {dr}]")
            if kscale is None or tuple(kscale.shape) != (P, page):
                raise ValueError(f"kscale must have shape [{P}, {page}]")
    else:
        dr = 0
        if k.dim() != 4 or k.shape[3] != d:
            raise ValueError(f"k has shape {tuple(k.shape)}, expected [num_pages, page_size, kv_heads, {d}]")
        G = k.shape[2]
        if variant != "gta" and (v is None or tuple(v.shape) != tuple(k.shape)):
            raise ValueError(f"v must have k's shape {tuple(k.shape)}")
    if groups is not None and groups != G:
        raise ValueError(f"groups={groups} does not match the tensors ({G})")
    return B, H, G, d, dr


class Decoder:
    """A decode problem bound to its device tensors: ``run()`` is one ld_latent_decode call.

    ``plan()``, ``decode()`` and ``combine()`` call the three stages separately
    (same stream, same workspace), e.g. to plan once for several layers.
    Layouts as in include/latent_decode.h; ``k`` holds the cache rows (for an
    fp8 latent cache: the E4M3 codes as uint8 or float8_e4m3fn, with ``rope``
    and ``kscale`` beside it).  ``q_len`` > 1 (mla, mqa): q_latent / q_rope, out
    and lse hold q_len*H rows per sequence, row i*H + h for query token i.
    """

    def __init__(self, q_latent, q_rope, k, block_table, seq_lens, *, variant: str, scale: float,
                 groups: int | None = None, v=None, rope=None, kscale=None, out=None, lse=None,
                 out_dtype: str | None = None, num_splits: int = 0, q_len: int = 1, workspace=None):
        if variant not in VARIANTS:
            raise ValueError(f"unknown variant {variant!r}")
        _need(q_latent, "q_latent", (torch.float32, torch.bfloat16))
        _need(k, "k", tuple(_TORCH_DTYPE))
        _need(block_table, "block_table", (torch.int32,))
        _need(seq_lens, "seq_lens", (torch.int32,))
        kv_dtype = _TORCH_DTYPE[k.dtype]
        q_dtype = _TORCH_DTYPE[q_latent.dtype]
        latent = variant in ("mla", "gla", "mlra")
        if latent:
            _need(q_rope, "q_rope", (q_latent.dtype,))
            if kv_dtype == "fp8_e4m3":
                _need(rope, "rope", (torch.bfloat16,))
                _need(kscale, "kscale", (torch.float32,))
        elif variant != "gta":
            _need(v, "v", (k.dtype,))
        B, H, G, d, dr = decode_shapes(q_latent, q_rope, k, block_table, seq_lens, variant=variant, groups=groups,
                                       v=v, rope=rope, kscale=kscale, q_len=q_len)
        out_dtype = out_dtype or ("f32" if q_dtype == "f32" else "bf16")
        self.problem = make_problem(variant, B, H, G, d, dr, k.shape[1], k.shape[0], block_table.shape[1], q_dtype,
                                    kv_dtype, out_dtype, scale, num_splits, q_len)
        rows = (H * G if variant == "mlra" else H) * max(q_len, 1)
        Hq = H * max(q_len, 1)
        odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        dev = q_latent.device
        if out is None:
            out = torch.empty((B, Hq, G, d) if variant == "mlra" else (B, rows, d), dtype=odt, device=dev)
        if lse is None:
            lse = torch.empty((B, Hq, G) if variant == "mlra" else (B, rows), dtype=torch.float32, device=dev)
        _need(out, "out", (odt,))
        _need(lse, "lse", (torch.float32,))
        if out.numel() != B * rows * d or lse.numel() != B * rows:
            raise ValueError("out/lse have the wrong size")
        ws_bytes = workspace_size(self.problem)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        _need(workspace, "workspace")
        self.cache = KVCache(k.data_ptr(), None if rope is None else rope.data_ptr(),
                             None if v is None else v.data_ptr(), None if kscale is None else kscale.data_ptr())
        # keep every tensor alive for as long as the pointers are used
        self.tensors = (q_latent, q_rope, k, v, rope, kscale, block_table, seq_lens)
        self.q_latent, self.q_rope, self.block_table, self.seq_lens = q_latent, q_rope, block_table, seq_lens
        self.out, self.lse, self.workspace = out, lse, workspace
        self.ws_bytes = workspace.numel() * workspace.element_size()
        self.device = dev

    def _stream(self, stream):
        return ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream)

    def plan(self, stream=None):
        st = lib().ld_plan(ctypes.byref(self.problem), _ptr(self.seq_lens), _ptr(self.workspace), self.ws_bytes,
                           self._stream(stream))
        if st:
            raise LatentDecodeError(st, "ld_plan")

    def decode(self, stream=None):
        st = lib().ld_decode_planned(ctypes.byref(self.problem), _ptr(self.q_latent), _ptr(self.q_rope),
                                     ctypes.byref(self.cache), _ptr(self.block_table), _ptr(self.seq_lens),
                                     _ptr(self.out), _ptr(self.lse), _ptr(self.workspace), self.ws_bytes,
                                     self._stream(stream))
        if st:
            raise LatentDecodeError(st, "ld_decode_planned")

    def combine(self, stream=None):
        st = lib().ld_combine_planned(ctypes.byref(self.problem), _ptr(self.out), _ptr(self.lse),
                                      _ptr(self.workspace), self.ws_bytes, self._stream(stream))
        if st:
            raise LatentDecodeError(st, "ld_combine_planned")

    def plan_decode(self, stream=None):
        """ld_plan_decode: the first launch of run() (the decode kernel planning for itself); combine()
        completes the step."""
        st = lib().ld_plan_decode(ctypes.byref(self.problem), _ptr(self.q_latent), _ptr(self.q_rope),
                                  ctypes.byref(self.cache), _ptr(self.block_table), _ptr(self.seq_lens),
                                  _ptr(self.out), _ptr(self.lse), _ptr(self.workspace), self.ws_bytes,
                                  self._stream(stream))
        if st:
            raise LatentDecodeError(st, "ld_plan_decode")

    def run(self, stream=None):
        st = lib().ld_latent_decode(ctypes.byref(self.problem), _ptr(self.q_latent), _ptr(self.q_rope),
                                    ctypes.byref(self.cache), _ptr(self.block_table), _ptr(self.seq_lens),
                                    _ptr(self.out), _ptr(self.lse), _ptr(self.workspace), self.ws_bytes,
                                    self._stream(stream))
        if st:
            raise LatentDecodeError(st, "ld_latent_decode")
        return self.out, self.lse

    def run_noalloc(self, stream=None):
        """ld_latent_decode_noalloc: the same step with the library's fixed device array as workspace
        (this object's own workspace tensor is not used)."""
        st = lib().ld_latent_decode_noalloc(ctypes.byref(self.problem), _ptr(self.q_latent), _ptr(self.q_rope),
                                            ctypes.byref(self.cache), _ptr(self.block_table), _ptr(self.seq_lens),
                                            _ptr(self.out), _ptr(self.lse), self._stream(stream))
        if st:
            raise LatentDecodeError(st, "ld_latent_decode_noalloc")
        return self.out, self.lse


NOALLOC_SCRATCH_BYTES = 64 << 20     # LD_NOALLOC_SCRATCH_BYTES


def latent_decode(q_latent, q_rope, k, block_table, seq_lens, *, variant: str, scale: float, groups: int | None = None,
                  v=None, rope=None, kscale=None, out=None, lse=None, out_dtype: str | None = None,
                  num_splits: int = 0, q_len: int = 1, workspace=None, stream=None):
    """One decode step; returns (out, lse).  See ``Decoder`` for the arguments."""
    d = Decoder(q_latent, q_rope, k, block_table, seq_lens, variant=variant, scale=scale, groups=groups, v=v,
                rope=rope, kscale=kscale, out=out, lse=lse, out_dtype=out_dtype, num_splits=num_splits,
                q_len=q_len, workspace=workspace)
    return d.run(stream)


def cache_append(c_new, kr_new, k, block_table, seq_lens, *, variant: str = "mla", groups: int = 1,
                 rope_base: float = 10000.0, rope=None, kscale=None, stream=None):
    """ld_cache_append: write each sequence's new token (at position seq_lens[b] - 1) into the paged cache.

    c_new [B, groups * d_latent] and kr_new [B, d_rope] (un-rotated) in f32 or bf16; ``k`` is the
    cache (f32/bf16 rows [P, page, G*d_latent + d_rope], or fp8 codes [P, page, G*d_latent] with the
    bf16 ``rope`` pool and the f32 ``kscale`` pool beside it), updated in place.
    """
    if variant not in ("mla", "gla", "mlra"):
        raise ValueError("cache_append covers the latent variants (mla, gla, mlra)")
    _need(c_new, "c_new", (torch.float32, torch.bfloat16))
    _need(kr_new, "kr_new", (c_new.dtype,))
    _need(k, "k", tuple(_TORCH_DTYPE))
    _need(block_table, "block_table", (torch.int32,))
    _need(seq_lens, "seq_lens", (torch.int32,))
    kv_dtype = _TORCH_DTYPE[k.dtype]
    if kv_dtype == "fp8_e4m3":
        _need(rope, "rope", (torch.bfloat16,))
        _need(kscale, "kscale", (torch.float32,))
    B, D = c_new.shape
    dr = kr_new.shape[-1]
    if D % groups:
        raise ValueError("c_new's width is not groups * d_latent")
    p = make_problem(variant, B, groups, groups, D // groups, dr, k.shape[1], k.shape[0], block_table.shape[1],
                     _TORCH_DTYPE[c_new.dtype], kv_dtype, "f32", 1.0)
    cache = KVCache(k.data_ptr(), None if rope is None else rope.data_ptr(), None,
                    None if kscale is None else kscale.data_ptr())
    if stream is None:
        stream = torch.cuda.current_stream(c_new.device).cuda_stream
    st = lib().ld_cache_append(ctypes.byref(p), _ptr(c_new), _ptr(kr_new), _ptr(block_table), _ptr(seq_lens),
                               ctypes.byref(cache), float(rope_base), ctypes.c_void_p(stream))
    if st:
        raise LatentDecodeError(st, "ld_cache_append")


def head_projection(a, w, *, out_dtype: str = "bf16", out=None, stream=None):
    """ld_head_projection: c[i, h, j] = sum_t w[h, j, t] a[i, h, t]; a bf16 [m, H, k], w bf16 [H, n, k]."""
    _need(a, "a", (torch.bfloat16,))
    _need(w, "w", (torch.bfloat16,))
    m, H, k = a.shape
    if w.shape[0] != H or w.shape[2] != k:
        raise ValueError(f"w has shape {tuple(w.shape)}, expected [{H}, n, {k}]")
    n = w.shape[1]
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if out is None:
        out = torch.empty((m, H, n), dtype=odt, device=a.device)
    _need(out, "out", (odt,))
    if stream is None:
        stream = torch.cuda.current_stream(a.device).cuda_stream
    st = lib().ld_head_projection(m, H, n, k, _ptr(a), _ptr(w), _ptr(out), DTYPES[out_dtype], ctypes.c_void_p(stream))
    if st:
        raise LatentDecodeError(st, "ld_head_projection")
    return out


def split_kv_combine(partial_out, partial_lse, row_num_splits, *, out_dtype: str = "f32", out=None, lse=None,
                     stream=None):
    """Merge split partials: partial_out [rows, S, d_v] f32, partial_lse [rows, S] f32, row_num_splits [rows] i32."""
    _need(partial_out, "partial_out", (torch.float32,))
    _need(partial_lse, "partial_lse", (torch.float32,))
    _need(row_num_splits, "row_num_splits", (torch.int32,))
    rows, S, dv = partial_out.shape
    odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    if out is None:
        out = torch.empty((rows, dv), dtype=odt, device=partial_out.device)
    if lse is None:
        lse = torch.empty((rows,), dtype=torch.float32, device=partial_out.device)
    if stream is None:
        stream = torch.cuda.current_stream(partial_out.device).cuda_stream
    st = lib().ld_split_kv_combine(rows, dv, S, _ptr(partial_out), _ptr(partial_lse), _ptr(row_num_splits),
                                   DTYPES[out_dtype], _ptr(out), _ptr(lse), ctypes.c_void_p(stream))
    if st:
        raise LatentDecodeError(st, "ld_split_kv_combine")
    return out, lse


def validate_metadata(p: Problem, block_table_host, seq_lens_host) -> int:
    bt = torch.as_tensor(block_table_host, dtype=torch.int32).contiguous()
    sl = torch.as_tensor(seq_lens_host, dtype=torch.int32).contiguous()
    ip = ctypes.POINTER(ctypes.c_int32)
    return lib().ld_validate_metadata(ctypes.byref(p), ctypes.cast(bt.data_ptr(), ip), ctypes.cast(sl.data_ptr(), ip))


def plan_host(p: Problem, seq_lens_host, num_cus: int):
    """Host planner: returns (chunk, num_units, splits[B], first_unit[B])."""
    sl = torch.as_tensor(seq_lens_host, dtype=torch.int32).contiguous()
    B = p.batch
    splits = torch.zeros(max(B, 1), dtype=torch.int32)
    first = torch.zeros(max(B, 1), dtype=torch.int32)
    chunk, units = ctypes.c_int32(0), ctypes.c_int32(0)
    ip = ctypes.POINTER(ctypes.c_int32)
    st = lib().ld_plan_host(ctypes.byref(p), ctypes.cast(sl.data_ptr(), ip), num_cus, ctypes.byref(chunk),
                            ctypes.byref(units), ctypes.cast(splits.data_ptr(), ip), ctypes.cast(first.data_ptr(), ip))
    if st:
        raise LatentDecodeError(st, "ld_plan_host")
    return chunk.value, units.value, splits[:B].numpy().copy(), first[:B].numpy().copy()
