#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one decode step of the whole hot path (split-KV plan, decode kernel,
log-sum-exp combine) over one batch of seeded synthetic inputs that are
already resident in HBM.  The default workload is absorbed MLA at the
DeepSeek-V3 shape: batch 64, 128 heads, 576-dim shared cache rows (512 latent +
64 RoPE), 4096 tokens per sequence, bf16, paged (64-token pages, shuffled
block table).  Consecutive steps read different copies of the cache (4 copies,
about 1.2 GB) so the 256 MB Infinity Cache cannot serve a repeat.

Prints one JSON line.  ``value`` is algorithmic KV-cache bytes per second of a
whole step; ``roofline`` describes the decode kernel alone (timed with HIP
events on the stream it is launched on); ``cpu_baseline`` is the CPU fp64
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s + tokens/s vs 1-GPU HBM/MFMA roofline, MLA 128h@4K–1M"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3
DECODE_SRC = os.path.join(ROOT, "latent_kv_cache_absorbed_amd", "csrc", "decode.hip")


def flops_per_token_head(w) -> int:
    """2 * (score dims + value dims) per (query row, token) of the absorbed / shared form."""
    if w.variant in ("mla", "gla"):
        return 2 * (w.d_lat + w.d_rope + w.d_lat)
    if w.variant == "mlra":
        return 2 * (w.d_lat + w.d_rope + w.d_lat) * w.groups
    return 2 * (w.d_lat + w.d_lat)


def source_sha() -> str:
    with open(DECODE_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter summaries, if they match this kernel."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_source_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float):
    """Time the oracle as it stands on a bounded sample of sequences (all heads each)."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    f64 = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    k = inp.k_pool.numpy() if inp.kv_dtype == "fp8_e4m3" else f64(inp.k_pool)
    args = (inp.variant, f64(inp.q_lat), f64(inp.q_rope), k, inp.layout.block_table, inp.layout.seq_lens)
    kw = dict(groups=inp.groups, scale=inp.scale, page_size=inp.layout.page_size, v_pool=f64(inp.v_pool),
              rope_pool=f64(inp.rope_pool), scale_pool=f64(inp.scale_pool), d_rope=inp.d_rope)
    B = inp.batch
    t0 = time.perf_counter()
    oracle.decode_paged(*args, batches=[0], **kw)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(B, budget_s / max(t1, 1e-3))))
    t0 = time.perf_counter()
    oracle.decode_paged(*args, batches=list(range(n)), **kw)
    dt = time.perf_counter() - t0
    per_tok = inp.kv_bytes() / max(1, int(inp.layout.seq_lens.astype(np.int64).sum()))
    toks = int(inp.layout.seq_lens[:n].astype(np.int64).sum())
    gbs = per_tok * toks / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} of {B} sequences x all {inp.heads} heads ({toks} cached tokens), fp64 numpy, "
                      f"{dt:.1f} s", "seconds": round(dt, 3), "tokens_per_s": round(n / dt, 3)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mla_b64_l4k")
    ap.add_argument("--copies", type=int, default=4, help="cache copies rotated across steps")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path is per-GPU and this build has no multi-GPU path.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import latent_kv_cache_absorbed_amd as lkd
    import synth

    lkd.lib()
    w = synth.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = synth.make_workload_inputs(w)
    dev = torch.device("cuda:0")
    up = lambda t: None if t is None else t.contiguous().to(dev)  # noqa: E731
    q_lat, q_rope = up(inp.q_lat), up(inp.q_rope)
    bt = torch.from_numpy(inp.layout.block_table).to(dev)
    sl = torch.from_numpy(inp.layout.seq_lens).to(dev)
    k0, v0, r0, s0 = up(inp.k_pool), up(inp.v_pool), up(inp.rope_pool), up(inp.scale_pool)
    copies = []
    for c in range(max(1, args.copies)):
        cl = (lambda t: None if t is None else (t if c == 0 else t.clone()))  # noqa: E731
        copies.append((cl(k0), cl(v0), cl(r0), cl(s0)))
    decs = []
    first = None
    for (k, v, r, s) in copies:
        d = lkd.Decoder(q_lat, q_rope, k, bt, sl, variant=w.variant, scale=w.scale, groups=w.groups, v=v, rope=r,
                        kscale=s, num_splits=args.num_splits,
                        out=None if first is None else first.out, lse=None if first is None else first.lse,
                        workspace=None if first is None else first.workspace)
        first = first or d
        decs.append(d)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        decs[i % len(decs)].run()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        d = decs[i % len(decs)]
        e = ev[i]
        e[0].record(stream)
        d.plan()
        e[1].record(stream)
        d.decode()
        e[2].record(stream)
        d.combine()
        e[3].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    plan_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    dec_all = np.array([e[1].elapsed_time(e[2]) for e in ev])
    comb_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    dec_ms = float(np.mean(dec_all))

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    ms = total_ms / K
    t = ms * 1e-3
    lens = inp.layout.seq_lens.astype(np.int64)
    kv_bytes = inp.kv_bytes()
    q_bytes = inp.q_lat.numel() * inp.q_lat.element_size() + (
        0 if inp.q_rope is None else inp.q_rope.numel() * inp.q_rope.element_size())
    out_el = 4 if inp.out_dtype == "f32" else 2
    out_bytes = inp.batch * inp.rows_per_seq * (inp.d_v * out_el + 4)
    flops = inp.heads * int(lens.sum()) * flops_per_token_head(w)
    dec_alg_bytes = kv_bytes + q_bytes              # what the decode kernel must read
    achieved = dec_alg_bytes / (dec_ms * 1e-3) / 1e9
    mfma_peak = MFMA_F32_PEAK_TFLOPS if inp.kv_dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    mfma_tflops = flops / (dec_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(args.workload)
    res = {
        "metric": METRIC,
        "value": round(kv_bytes / t / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.kv_dtype == "bf16" else ("fp8_e4m3+bf16" if inp.kv_dtype == "fp8_e4m3" else "f32"),
        "data": "synthetic",
        "config": {"workload": args.workload, "variant": w.variant, "batch": inp.batch, "heads": inp.heads,
                   "groups": inp.groups, "d_latent": inp.d_lat, "d_rope": inp.d_rope,
                   "seq_len": int(lens.max()) if lens.min() == lens.max() else [int(lens.min()), int(lens.max())],
                   "total_cached_tokens": int(lens.sum()), "page_size": inp.layout.page_size,
                   "kv_dtype": inp.kv_dtype, "cache_copies": len(decs), "num_splits": args.num_splits},
        "tokens_per_s": round(inp.batch / t, 1),
        "kv_tokens_per_s": round(float(lens.sum()) / t, 1),
        "hbm_frac_step": round((kv_bytes + q_bytes + out_bytes) / t / 1e9 / HBM_PEAK_GBS, 4),
        "stage_ms": {"plan": round(plan_ms, 5), "decode": round(dec_ms, 5), "combine": round(comb_ms, 5),
                     "decode_p10": round(float(np.percentile(dec_all, 10)), 5),
                     "decode_p90": round(float(np.percentile(dec_all, 90)), 5)},
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": int(dec_alg_bytes),
                     "mfma_tflops": round(mfma_tflops, 2), "mfma_frac": round(mfma_tflops / mfma_peak, 4),
                     "flops_per_launch": int(flops), "decode_source_sha": source_sha()},
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
