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
whole step; ``roofline`` describes the decode kernel alone (its average
duration over back-to-back launches, timed with HIP events on the stream it is
launched on); ``cpu_baseline`` is the CPU fp64 oracle timed on a bounded sample
of the same workload.

``--summarize-profile TRACE FETCH WRITE`` turns the csv output of three
rocprofv3 runs of this script (``--kernel-trace --stats``, ``--pmc FETCH_SIZE``
and ``--pmc WRITE_SIZE``, the last two with ``--calibrate-copy-mib``) into the
text summaries kept under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import functools
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s + tokens/s vs 1-GPU HBM/MFMA roofline, MLA 128h@4K–1M"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3
DECODE_SRC = [os.path.join(ROOT, "latent_kv_cache_absorbed_amd", "csrc", f) for f in ("decode.hip", "decode_common.h", "plan_common.h")]
PROFILES = os.path.join(ROOT, "profiles")


def flops_per_token_head(w) -> int:
    """2 * (score dims + value dims) per (query row, token) of the absorbed / shared form."""
    if w.variant in ("mla", "gla"):
        return 2 * (w.d_lat + w.d_rope + w.d_lat)
    if w.variant == "mlra":
        return 2 * (w.d_lat + w.d_rope + w.d_lat) * w.groups
    return 2 * (w.d_lat + w.d_lat)


def source_sha() -> str:
    """Hash of the decode kernel's sources (the kernel file and the device headers it includes)."""
    h = hashlib.sha256()
    for path in DECODE_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, f"decode_{workload}_traffic.json")


def traffic_from_profile(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter summaries, if they match this kernel."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_source_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float):
    """Time the oracle as it stands on a bounded sample: whole sequences (all heads), repeated until the
    budget is spent."""
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
    lens = inp.layout.seq_lens.astype(np.int64)
    run = oracle.decode_paged
    if inp.q_len > 1:
        run = functools.partial(oracle.decode_paged_tokens, q_len=inp.q_len)
    t0 = time.perf_counter()
    run(*args, batches=[0], **kw)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(B, budget_s / max(t1, 1e-3))))
    batches = list(range(n))
    reps, toks = 0, 0
    t0 = time.perf_counter()
    while True:
        run(*args, batches=batches, **kw)
        reps += 1
        toks += int(lens[:n].sum())
        dt = time.perf_counter() - t0
        if dt >= min(budget_s, 10.0) or dt * (reps + 1) / reps > 3 * budget_s:
            break
    per_tok = inp.kv_bytes() / max(1, int(lens.sum()))
    gbs = per_tok * toks / dt / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} of {B} sequences x all {inp.heads} heads, {reps} pass(es), {toks} cached tokens, "
                      f"fp64 numpy, {dt:.1f} s", "seconds": round(dt, 3), "tokens_per_s": round(n * reps / dt, 3)}


def _kernel_rows(trace_dir: str):
    with open(os.path.join(trace_dir, "run_kernel_stats.csv")) as f:
        return list(csv.DictReader(f))


def _last_calls_us(trace_dir: str, n: int):
    """Average duration (us) of each kernel's last n dispatches (the timed part of the run)."""
    with open(os.path.join(trace_dir, "run_kernel_trace.csv")) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    per = {}
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: sum(v[-n:]) / len(v[-n:]) for k, v in per.items()}


def _counter(dir_: str, name: str):
    rows = list(csv.DictReader(open(os.path.join(dir_, "run_counter_collection.csv"))))
    out = {}
    for r in rows:
        if r["Counter_Name"] == name:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize_profile(workload: str, trace_dir: str, fetch_dir: str, write_dir: str, copy_mib: int,
                      commands: list[str]) -> None:
    """Write profiles/decode_kernel_<workload>.md and profiles/decode_<workload>_traffic.json."""
    import numpy as np

    stats = _kernel_rows(trace_dir)
    fetch = _counter(fetch_dir, "FETCH_SIZE")
    write = _counter(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024
    dec = lambda d: [v for k, v in d.items() if "decode_kernel" in k][0]  # noqa: E731
    # calibration: the copy of exactly copy_mib MiB reads and writes copy_kib KiB
    fcopy = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs if abs(v - copy_kib) < 0.6 * copy_kib]
    wcopy = [v for k, vs in write.items() if "copyBuffer" in k for v in vs if abs(v - copy_kib) < 0.6 * copy_kib]
    fscale = copy_kib / fcopy[-1]
    wscale = copy_kib / wcopy[-1]
    f_kib = float(np.median(dec(fetch)))
    w_kib = float(np.median(dec(write)))
    hbm = (f_kib * fscale + w_kib * wscale) * 1024
    t = {"workload": workload, "decode_source_sha": source_sha(), "hbm_bytes_per_launch": int(hbm),
         "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "fetch_scale": round(fscale, 5),
         "write_scale": round(wscale, 5), "calibration": f"plain device copy of {copy_mib} MiB",
         "commands": commands[1:]}
    with open(traffic_path(workload), "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    last = _last_calls_us(trace_dir, 40)
    lines = [f"# decode_kernel, workload {workload}", "",
             "Kernel durations (rocprofv3 kernel trace; the average over the whole run includes the warm-up,",
             "whose first launches run at lower clocks; the last 40 calls are the timed part of the run):", "",
             f"    {commands[0]}", "",
             "| kernel | calls | average us | last 40 calls, average us | min us | max us |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{last.get(r['Name'], float('nan')):.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines += ["", "HBM traffic of one decode launch (TCC counters, one pass per counter):", ""]
    lines += [f"    {c}" for c in commands[1:]]
    lines += ["", f"- FETCH_SIZE {f_kib:.0f} KiB per dispatch; the {copy_mib} MiB copy reads {fcopy[-1]:.0f} KiB "
                  f"-> scale {fscale:.4f}",
              f"- WRITE_SIZE {w_kib:.0f} KiB per dispatch; the copy writes {wcopy[-1]:.0f} KiB -> scale {wscale:.4f}",
              f"- HBM bytes per launch: {hbm / 1e6:.1f} MB (read {f_kib * fscale * 1024 / 1e6:.1f} MB, "
              f"write {w_kib * wscale * 1024 / 1e6:.1f} MB)",
              f"- decode source sha256[:16] {source_sha()}", ""]
    with open(os.path.join(PROFILES, f"decode_kernel_{workload}.md"), "w") as f:
        f.write("\n".join(lines))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mla_b64_l4k")
    ap.add_argument("--copies", type=int, default=4, help="cache copies rotated across steps")
    ap.add_argument("--min-warmup-ms", type=float, default=50.0,
                    help="keep running untimed warmup steps until this much wall time has passed")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="time each step as the replay of a HIP graph holding its plan, decode and combine launches "
                         "(the eager time is reported too); default: eager launches")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--profile-commands", nargs=3, default=None, help="the three commands, for the summary")
    args = ap.parse_args()

    if args.summarize_profile:
        cmds = args.profile_commands or ["(not given)"] * 3
        summarize_profile(args.workload, *args.summarize_profile, args.calibrate_copy_mib or 512, cmds)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path runs on one GPU; there is no multi-GPU path.", file=sys.stderr)
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
                        kscale=s, num_splits=args.num_splits, q_len=w.q_len,
                        out=None if first is None else first.out, lse=None if first is None else first.lse,
                        workspace=None if first is None else first.workspace)
        first = first or d
        decs.append(d)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    stream = torch.cuda.current_stream(dev)
    # W warmup steps, continued (untimed) until the GPU has run steps for at least --min-warmup-ms:
    # its clocks take tens of milliseconds of load to settle (a step timed after 10 warmup steps
    # of ~0.12 ms each runs ~20% slower than after 200)
    t_wu = time.perf_counter()
    warmup_run = 0
    for i in range(args.warmup):
        decs[i % len(decs)].run()
        warmup_run += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t_wu) * 1e3 < args.min_warmup_ms:
        for i in range(10):
            decs[(warmup_run + i) % len(decs)].run()
        warmup_run += 10
        torch.cuda.synchronize()

    # ---- the timed steps: plan + decode + combine, K times back to back, launched eagerly; with
    # --graph each step is instead the replay of a HIP graph holding the step's launches (one graph per
    # cache copy), and the eager time is reported beside it
    K = args.steps

    def time_steps(step):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K):
            step(i)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop)

    eager_ms = time_steps(lambda i: decs[i % len(decs)].run())
    graphs = []
    if args.graph:
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            for d in decs:
                d.run()                       # one eager run on the capture stream first
        torch.cuda.synchronize()
        for d in decs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                d.run()
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        total_ms = time_steps(lambda i: graphs[i % len(graphs)].replay())
    else:
        total_ms = eager_ms

    # ---- per-stage kernel durations: each stage launched K times back to back (the plan only depends
    # on seq_lens, so one plan serves every decode and combine launch), per-launch average
    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(K):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    plan_ms = timed(lambda i: decs[i % len(decs)].plan())
    dec_ms = timed(lambda i: decs[i % len(decs)].decode())
    comb_ms = timed(lambda i: decs[i % len(decs)].combine())
    # the cache append of the step's new tokens (the step before the attention), timed on its own
    # (latent variants): K launches back to back into cache copy 0 (one slot per sequence rewritten)
    append_ms = None
    if w.variant in ("mla", "gla", "mlra"):
        gen = torch.Generator(device=dev).manual_seed(7)
        c_new = torch.randn((inp.batch, inp.groups * inp.d_lat), generator=gen, device=dev).to(q_lat.dtype)
        kr_new = torch.randn((inp.batch, inp.d_rope), generator=gen, device=dev).to(q_lat.dtype)
        k_c, _, r_c, s_c = copies[0]
        app = lambda i: lkd.cache_append(c_new, kr_new, k_c, bt, sl, variant=w.variant,  # noqa: E731
                                         groups=inp.groups, rope=r_c, kscale=s_c)
        app(0)
        append_ms = timed(app)
    # the projections around the step (absorbed MLA shapes: d_nope 128, d_v 128, per head): the query
    # absorption q_lat = W_UK^T q^C and the output up-projection W_UV o_lat, each timed on its own
    proj = {}
    if w.variant in ("mla", "gla", "mlra"):
        gen = torch.Generator(device=dev).manual_seed(8)
        dn = dv = 128
        dl = inp.d_lat * (inp.groups if w.variant == "mlra" else 1)     # MLRA: the branches side by side
        qn = torch.randn((inp.batch, inp.heads, dn), generator=gen, device=dev).to(torch.bfloat16)
        w_uk_t = (torch.randn((inp.heads, dl, dn), generator=gen, device=dev) * dn ** -0.5).to(torch.bfloat16)
        ol = torch.randn((inp.batch, inp.heads, dl), generator=gen, device=dev).to(torch.bfloat16)
        w_uv = (torch.randn((inp.heads, dv, dl), generator=gen, device=dev) * dl ** -0.5).to(torch.bfloat16)
        for name, (A, W) in {"q_absorb": (qn, w_uk_t), "up_proj": (ol, w_uv)}.items():
            out_t = torch.empty((A.shape[0], A.shape[1], W.shape[1]), dtype=torch.bfloat16, device=dev)
            run_p = lambda i, A=A, W=W, o=out_t: lkd.head_projection(A, W, out=o)  # noqa: E731
            run_p(0)
            t_ms = timed(run_p)
            nbytes = (A.numel() + W.numel() + out_t.numel()) * 2
            proj[name] = {"ms": round(t_ms, 5), "m": A.shape[0], "heads": A.shape[1], "n": W.shape[1], "k": W.shape[2],
                          "bytes": nbytes, "gbs": round(nbytes / (t_ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(nbytes / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # single-launch spread of the decode kernel
    one = []
    for i in range(min(K, 20)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        decs[i % len(decs)].decode()
        e1.record(stream)
        torch.cuda.synchronize()
        one.append(e0.elapsed_time(e1))

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
    # query token i of Q sees the first L - Q + 1 + i rows
    seen = sum(int(np.maximum(lens - inp.q_len + 1 + i, 0).sum()) for i in range(inp.q_len))
    flops = inp.heads * seen * flops_per_token_head(w)
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
        "warmup_steps_run": warmup_run,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.kv_dtype == "bf16" else ("fp8_e4m3+bf16" if inp.kv_dtype == "fp8_e4m3" else "f32"),
        "data": "synthetic",
        "config": {"workload": args.workload, "variant": w.variant, "batch": inp.batch, "heads": inp.heads,
                   "groups": inp.groups, "d_latent": inp.d_lat, "d_rope": inp.d_rope,
                   "seq_len": int(lens.max()) if lens.min() == lens.max() else [int(lens.min()), int(lens.max())],
                   "total_cached_tokens": int(lens.sum()), "page_size": inp.layout.page_size, "q_len": inp.q_len,
                   "kv_dtype": inp.kv_dtype, "cache_copies": len(decs), "num_splits": args.num_splits},
        "tokens_per_s": round(inp.batch * inp.q_len / t, 1),
        "kv_tokens_per_s": round(float(lens.sum()) / t, 1),
        "hbm_frac_step": round((kv_bytes + q_bytes + out_bytes) / t / 1e9 / HBM_PEAK_GBS, 4),
        "stage_ms": {"plan": round(plan_ms, 5), "decode": round(dec_ms, 5), "combine": round(comb_ms, 5),
                     "append": None if append_ms is None else round(append_ms, 5),
                     "decode_single_p10": round(float(np.percentile(one, 10)), 5),
                     "decode_single_p50": round(float(np.percentile(one, 50)), 5),
                     "decode_single_p90": round(float(np.percentile(one, 90)), 5)},
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": int(dec_alg_bytes),
                     "mfma_tflops": round(mfma_tflops, 2), "mfma_frac": round(mfma_tflops / mfma_peak, 4),
                     "flops_per_launch": int(flops), "decode_source_sha": source_sha()},
        "projections": proj or None,
        "launch": "hip_graph" if args.graph else "eager",
        "eager_ms_per_step": round(eager_ms / K, 5),
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
