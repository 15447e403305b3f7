#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one decode step of the whole hot path (split-KV plan, decode kernel,
log-sum-exp combine: ``ld_latent_decode``) over one batch of seeded synthetic
inputs that are already resident in HBM.  The default workload is absorbed MLA
at the DeepSeek-V3 shape: batch 64, 128 heads, 576-dim shared cache rows (512
latent + 64 RoPE), 4096 tokens per sequence, bf16, paged (64-token pages,
shuffled block table).  The long-context workloads (one sequence of 1M tokens
for MLA and MLRA-4, and the fp8 GLA-2 batch of imbalanced lengths) are timed
in the same run and reported as sub-objects.

Timing.  Before every timed step a 1 GiB scratch buffer is read (a reduction,
outside the timed events), which evicts the L2 caches and the 256 MB Infinity
Cache, so every step reads its cache from HBM.  A read rather than a write: a
1 GiB write flush leaves the Infinity Cache full of dirty lines, whose
write-back then lands in the next step (it added ~37 us to the batch-64 step).  Each step is bracketed by HIP events on
the stream the library launches on; the line reports the median and the
10th/90th percentiles over the steps.  The decode kernel is timed inside the
same step: ``ld_plan_decode`` (the step's first launch), an event, then
``ld_combine_planned`` (its second), which is ``ld_latent_decode`` launch for
launch.  ``roofline`` takes the decode kernel's mean in-step duration.

Prints one JSON line.  ``--summarize-profile`` turns rocprofv3 csv output of
this script into the summaries kept under profiles/.
"""
from __future__ import annotations

import argparse
import csv
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
DECODE_SRC = [os.path.join(ROOT, "latent_kv_cache_absorbed_amd", "csrc", f)
              for f in ("decode.hip", "decode_pipe.hip", "decode_pipe_fp8.hip", "decode_common.h", "plan_common.h")]
PROFILES = os.path.join(ROOT, "profiles")
DEFAULT_WORKLOAD = "mla_b64_l4k"
LONG_WORKLOADS = ("mla_b1_l1m", "mlra4_b1_l1m", "gla2_fp8_b64_mixed")
FLUSH_BYTES = 1 << 30         # scratch read before every timed step (4x the Infinity Cache)
XCDS = 8                        # MI355X: 8 XCDs of 32 CUs


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


def profile_record(workload: str):
    """The committed rocprofv3 counter record of this workload, if it was taken on this decode source."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_source_sha") != source_sha():
        return None
    return t


def host_threads() -> int:
    """Host cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS when that is set."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def oracle_args(inp):
    f64 = lambda t: None if t is None else t.double().numpy()  # noqa: E731
    k = inp.k_pool.numpy() if inp.kv_dtype == "fp8_e4m3" else f64(inp.k_pool)
    args = (inp.variant, f64(inp.q_lat), f64(inp.q_rope), k, inp.layout.block_table, inp.layout.seq_lens)
    kw = dict(groups=inp.groups, scale=inp.scale, page_size=inp.layout.page_size, v_pool=f64(inp.v_pool),
              rope_pool=f64(inp.rope_pool), scale_pool=f64(inp.scale_pool), d_rope=inp.d_rope)
    return args, kw


def run_oracle(inp, batches, heads=None):
    import oracle
    args, kw = oracle_args(inp)
    if inp.q_len > 1:
        return oracle.decode_paged_tokens(*args, q_len=inp.q_len, batches=batches, heads=heads, **kw)
    return oracle.decode_paged(*args, batches=batches, heads=heads, **kw)


def cpu_baseline(inp, budget_s: float):
    """Time the oracle as it stands on a bounded sample: whole sequences (all heads), repeated until the
    budget is spent, with the BLAS thread pool set to the cores this process may use."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    cores = host_threads()
    B = inp.batch
    lens = inp.layout.seq_lens.astype(np.int64)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        run_oracle(inp, [0])
        t1 = time.perf_counter() - t0
        n = int(max(1, min(B, budget_s / max(t1, 1e-3))))
        batches = list(range(n))
        reps, toks = 0, 0
        t0 = time.perf_counter()
        while True:
            run_oracle(inp, batches)
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


def parity_sample(inp, got_o, got_l):
    """Max errors of this run's output against the oracle on a sample of rows (first and last sequence,
    first and last head): row-normalised out error and lse error, as the parity tests measure them."""
    import numpy as np
    B, H = inp.batch, inp.heads * inp.q_len
    batches = sorted({0, B - 1})
    heads = sorted({0, H - 1})
    ref_o, ref_l = run_oracle(inp, batches, heads)
    mask = ~np.isnan(ref_l)
    g = got_o.reshape(-1, got_o.shape[-1])[mask.reshape(-1)]
    r = ref_o.reshape(-1, ref_o.shape[-1])[mask.reshape(-1)]
    den = np.max(np.abs(r), axis=1)
    eo = float(np.max(np.max(np.abs(g - r), axis=1) / np.where(den > 0, den, 1.0)))
    gl, rl = got_l[mask], ref_l[mask]
    fin = np.isfinite(rl)
    el = float(np.max(np.abs(gl[fin] - rl[fin]) / np.maximum(1.0, np.abs(rl[fin])))) if fin.any() else 0.0
    tol = 1e-5 if (inp.kv_dtype == "f32" and inp.q_dtype == "f32" and inp.out_dtype == "f32") else 1e-2
    return {"out_err": float(f"{eo:.4g}"), "lse_err": float(f"{el:.4g}"), "tol": tol, "rows": int(mask.sum()),
            "sample": f"sequences {batches} x query rows {heads} vs the fp64 oracle", "pass": bool(eo <= tol and el <= tol)}


def _pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs, np.float64), q))


def measure(name, steps, warmup, min_warmup_ms, dev, flush, num_splits=0, stages=False, keep=False):
    """Time one workload; returns (result dict, inputs, Decoder)."""
    import numpy as np
    import torch

    import latent_kv_cache_absorbed_amd as lkd
    import synth

    w = synth.WORKLOADS[name]
    t_gen = time.perf_counter()
    inp = synth.make_workload_inputs(w)
    up = lambda t: None if t is None else t.contiguous().to(dev)  # noqa: E731
    d = lkd.Decoder(up(inp.q_lat), up(inp.q_rope), up(inp.k_pool), torch.from_numpy(inp.layout.block_table).to(dev),
                    torch.from_numpy(inp.layout.seq_lens).to(dev), variant=w.variant, scale=w.scale, groups=w.groups,
                    v=up(inp.v_pool), rope=up(inp.rope_pool), kscale=up(inp.scale_pool), num_splits=num_splits,
                    q_len=w.q_len)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen
    stream = torch.cuda.current_stream(dev)

    def do_flush():
        torch.sum(flush, dtype=torch.int64)   # reads the whole buffer; leaves no dirty lines

    # warmup: W steps (each after a flush), continued until the GPU has been busy for min_warmup_ms
    # (its clocks take tens of milliseconds of load to settle)
    t_wu = time.perf_counter()
    warmup_run = 0
    while warmup_run < warmup or (time.perf_counter() - t_wu) * 1e3 < min_warmup_ms:
        for _ in range(5):
            do_flush()
            d.run()
            warmup_run += 1
        torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # (a) the step as one ld_latent_decode call: K steps, each bracketed by its own events
    e0, e1 = [ev() for _ in range(steps)], [ev() for _ in range(steps)]
    torch.cuda.synchronize()
    t_region = time.perf_counter()
    for i in range(steps):
        do_flush()
        e0[i].record(stream)
        d.run()
        e1[i].record(stream)
    torch.cuda.synchronize()
    region_s = time.perf_counter() - t_region
    step_ms = [a.elapsed_time(b) for a, b in zip(e0, e1)]
    # (b) the same step as its two launches with an event between: the decode kernel in the step
    f0, fm, f1 = [ev() for _ in range(steps)], [ev() for _ in range(steps)], [ev() for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        do_flush()
        f0[i].record(stream)
        d.plan_decode()
        fm[i].record(stream)
        d.combine()
        f1[i].record(stream)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in zip(f0, fm)]
    comb_ms = [a.elapsed_time(b) for a, b in zip(fm, f1)]

    lens = inp.layout.seq_lens.astype(np.int64)
    kv_bytes = inp.kv_bytes()
    q_bytes = inp.q_lat.numel() * inp.q_lat.element_size() + (
        0 if inp.q_rope is None else inp.q_rope.numel() * inp.q_rope.element_size())
    out_el = 4 if inp.out_dtype == "f32" else 2
    out_bytes = inp.batch * inp.rows_per_seq * (inp.d_v * out_el + 4)
    seen = sum(int(np.maximum(lens - inp.q_len + 1 + i, 0).sum()) for i in range(inp.q_len))
    flops = inp.heads * seen * flops_per_token_head(w)
    t_med = _pct(step_ms, 50) * 1e-3
    dec_mean = float(np.mean(dec_ms)) * 1e-3
    dec_alg_bytes = kv_bytes + q_bytes
    achieved = dec_alg_bytes / dec_mean / 1e9
    mfma_peak = MFMA_F32_PEAK_TFLOPS if inp.kv_dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    mfma_tflops = flops / dec_mean / 1e12
    prof = profile_record(name)
    res = {
        "workload": name,
        "value": round(kv_bytes / t_med / 1e9, 2),
        "unit": "GB/s",
        "ms_per_step": round(t_med * 1e3, 5),
        "step_us": {"median": round(t_med * 1e6, 2), "p10": round(_pct(step_ms, 10) * 1e3, 2),
                    "p90": round(_pct(step_ms, 90) * 1e3, 2), "mean": round(float(np.mean(step_ms)) * 1e3, 2),
                    "steps": steps},
        "in_step_us": {"decode_mean": round(dec_mean * 1e6, 2), "decode_median": round(_pct(dec_ms, 50) * 1e3, 2),
                       "decode_p10": round(_pct(dec_ms, 10) * 1e3, 2), "decode_p90": round(_pct(dec_ms, 90) * 1e3, 2),
                       "combine_median": round(_pct(comb_ms, 50) * 1e3, 2),
                       "two_launch_step_median": round(_pct([a + b for a, b in zip(dec_ms, comb_ms)], 50) * 1e3, 2)},
        "tokens_per_s": round(inp.batch * inp.q_len / t_med, 1),
        "kv_tokens_per_s": round(float(lens.sum()) / t_med, 1),
        "hbm_frac_step": round((kv_bytes + q_bytes + out_bytes) / t_med / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": decode_kernel_name(w, inp), "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if prof is None else prof.get("hbm_bytes_per_launch"),
                     "traffic_source": None if prof is None else os.path.relpath(traffic_path(name), ROOT),
                     "alg_bytes_per_launch": int(dec_alg_bytes), "duration": "mean in-step decode launch (HIP events)",
                     "mfma_tflops": round(mfma_tflops, 2), "mfma_frac": round(mfma_tflops / mfma_peak, 4),
                     "mfma_busy_counter": None if prof is None else prof.get("mfma_busy_frac"),
                     "flops_per_launch": int(flops), "decode_source_sha": source_sha()},
        "config": {"workload": name, "variant": w.variant, "batch": inp.batch, "heads": inp.heads,
                   "groups": inp.groups, "d_latent": inp.d_lat, "d_rope": inp.d_rope,
                   "seq_len": int(lens.max()) if lens.min() == lens.max() else [int(lens.min()), int(lens.max())],
                   "total_cached_tokens": int(lens.sum()), "page_size": inp.layout.page_size, "q_len": inp.q_len,
                   "kv_dtype": inp.kv_dtype, "num_splits": num_splits},
        "kv_bytes": int(kv_bytes),
        "warmup_steps_run": warmup_run,
        "timed_region_s": round(region_s, 4),
        "input_gen_s": round(gen_s, 2),
    }
    if stages:
        res["stages_back_to_back_ms"] = stage_times(d, steps, stream)
    if not keep:
        del d
        torch.cuda.empty_cache()
        return res, inp, None
    return res, inp, d


def stage_times(d, K, stream):
    """Per-launch averages of the staged path (ld_plan, ld_decode_planned, ld_combine_planned), each launched
    K times back to back (no flush: the same cache is re-read, so these can be served from the caches)."""
    import torch

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / K, 5)

    return {"plan": timed(d.plan), "decode_planned": timed(d.decode), "combine": timed(d.combine)}


def around_step(inp, w, dev, K, stream, k_cache, bt, sl, rope, kscale, flush):
    """The kernels around the step, timed like the step: K launches of each, every one after a 1 GiB read
    (outside its events: the caches are cold and the host has queued the launch before the GPU reaches
    it, so the events bracket the kernel, not the binding's argument marshalling); the median launch.
    The cache append of the step's new tokens and the projections (query absorption, output
    up-projection) at the workload's shapes."""
    import numpy as np
    import torch

    import latent_kv_cache_absorbed_amd as lkd

    def timed(fn):
        fn()
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            torch.sum(flush, dtype=torch.int64)
            e0[i].record(stream)
            fn()
            e1[i].record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in zip(e0, e1)]))

    out = {}
    gen = torch.Generator(device=dev).manual_seed(7)
    q_dt = torch.bfloat16 if inp.q_dtype == "bf16" else torch.float32
    c_new = torch.randn((inp.batch, inp.groups * inp.d_lat), generator=gen, device=dev).to(q_dt)
    kr_new = torch.randn((inp.batch, inp.d_rope), generator=gen, device=dev).to(q_dt)
    out["append_ms"] = round(timed(lambda: lkd.cache_append(c_new, kr_new, k_cache, bt, sl, variant=w.variant,
                                                          groups=inp.groups, rope=rope, kscale=kscale)), 5)
    dn = dv = 128
    dl = inp.d_lat * (inp.groups if w.variant == "mlra" else 1)
    qn = torch.randn((inp.batch, inp.heads, dn), generator=gen, device=dev).to(torch.bfloat16)
    w_uk_t = (torch.randn((inp.heads, dl, dn), generator=gen, device=dev) * dn ** -0.5).to(torch.bfloat16)
    ol = torch.randn((inp.batch, inp.heads, dl), generator=gen, device=dev).to(torch.bfloat16)
    w_uv = (torch.randn((inp.heads, dv, dl), generator=gen, device=dev) * dl ** -0.5).to(torch.bfloat16)
    for pname, (A, W) in {"q_absorb": (qn, w_uk_t), "up_proj": (ol, w_uv)}.items():
        o_t = torch.empty((A.shape[0], A.shape[1], W.shape[1]), dtype=torch.bfloat16, device=dev)
        t_ms = timed(lambda A=A, W=W, o=o_t: lkd.head_projection(A, W, out=o))
        nbytes = (A.numel() + W.numel() + o_t.numel()) * 2
        out[pname] = {"ms": round(t_ms, 5), "m": A.shape[0], "heads": A.shape[1], "n": W.shape[1], "k": W.shape[2],
                      "bytes": nbytes, "gbs": round(nbytes / (t_ms * 1e-3) / 1e9, 1),
                      "hbm_frac": round(nbytes / (t_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


# ----------------------------------------------------------------------------------------------
# rocprofv3 summaries
# ----------------------------------------------------------------------------------------------
def _csv(dir_: str, suffix: str):
    for root, _, files in os.walk(dir_):
        for f in files:
            if f.endswith(suffix):
                with open(os.path.join(root, f)) as fh:
                    return list(csv.DictReader(fh))
    raise FileNotFoundError(f"no *{suffix} under {dir_}")


def _counter(dir_: str, name: str):
    out = {}
    for r in _csv(dir_, "counter_collection.csv"):
        if r["Counter_Name"] == name:
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def is_decode(kernel_name: str) -> bool:
    """The decode kernels (decode_kernel of decode.hip, decode_pipe_kernel of decode_pipe.hip,
    decode_pipe8_kernel of decode_pipe_fp8.hip)."""
    return any(k in kernel_name for k in ("decode_kernel", "decode_pipe_kernel", "decode_pipe8_kernel"))


def decode_kernel_name(w, inp) -> str:
    """The kernel the library launches for a workload's decode (its dispatch rule, restated)."""
    if w.variant == "mla" and inp.kv_dtype == "bf16" and inp.heads == 128 and inp.d_lat == 512 and inp.d_rope == 64:
        return "decode_pipe_kernel"
    if (w.variant == "mlra" and inp.kv_dtype == "bf16" and inp.heads == 128 and inp.d_lat == 128 and inp.d_rope == 64
            and inp.groups in (1, 4)):
        return "decode_pipe_kernel"
    if (inp.kv_dtype == "fp8_e4m3" and w.variant in ("mla", "gla") and inp.d_lat == 256 and inp.d_rope == 64
            and inp.heads == 64 * inp.groups and inp.groups in (1, 2)):
        return "decode_pipe8_kernel"
    return "decode_kernel"


def summarize_profile(workload: str, trace_dir: str, fetch_dir: str, write_dir: str, mfma_dir: str, copy_mib: int,
                      steps: int, commands: list[str], num_cus: int = 256) -> None:
    """Write profiles/decode_kernel_<workload>.md and profiles/decode_<workload>_traffic.json.

    The decode kernel's in-step launches are its last 2 x steps dispatches (bench.py times the step twice,
    once as ld_latent_decode and once as its two launches with an event between them)."""
    import numpy as np

    rows = sorted(_csv(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    per = {}
    for r in rows:
        per.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    dec_name = [k for k in per if is_decode(k)][0]
    in_step = per[dec_name][-2 * steps:]
    comb = {k: v for k, v in per.items() if "combine" in k}
    fetch, write = _counter(fetch_dir, "FETCH_SIZE"), _counter(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024
    pick = lambda d: [v for k, vs in d.items() if is_decode(k) for v in vs]  # noqa: E731
    # calibration: the copy of exactly copy_mib MiB reads and writes copy_kib KiB
    fcopy = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs if abs(v - copy_kib) < 0.6 * copy_kib]
    wcopy = [v for k, vs in write.items() if "copyBuffer" in k for v in vs if abs(v - copy_kib) < 0.6 * copy_kib]
    fscale = copy_kib / fcopy[-1]
    wscale = copy_kib / wcopy[-1]
    f_kib = float(np.median(pick(fetch)[-2 * steps:]))
    w_kib = float(np.median(pick(write)[-2 * steps:]))
    hbm = (f_kib * fscale + w_kib * wscale) * 1024
    mf = {c: float(np.median(pick(_counter(mfma_dir, c))[-2 * steps:]))
          for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16")}
    # SQ_VALU_MFMA_BUSY_CYCLES sums the MFMA-busy cycles of every SIMD (4 per CU): each 32x32x16 MFMA adds
    # its 32 cycles, so it equals the MFMA count x 32.  GRBM_GUI_ACTIVE comes back summed over the
    # XCDs (one GRBM each), so the kernel's own busy cycles are GRBM_GUI_ACTIVE / XCDS.
    gpu_cycles = mf["GRBM_GUI_ACTIVE"] / XCDS
    mfma_busy = mf["SQ_VALU_MFMA_BUSY_CYCLES"] / (gpu_cycles * num_cus * 4)
    t = {"workload": workload, "decode_source_sha": source_sha(), "hbm_bytes_per_launch": int(hbm),
         "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "fetch_scale": round(fscale, 5),
         "write_scale": round(wscale, 5), "calibration": f"plain device copy of {copy_mib} MiB",
         "in_step_decode_us_mean": round(float(np.mean(in_step)), 2),
         "in_step_decode_us_median": round(float(np.median(in_step)), 2),
         "mfma_counters_per_dispatch": mf, "mfma_busy_frac": round(mfma_busy, 4),
         "commands": commands}
    with open(traffic_path(workload), "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    lines = [f"# decode_kernel, workload {workload}", "",
             "Kernel durations (rocprofv3 kernel trace).  The decode kernel's in-step launches are its last",
             f"{2 * steps} dispatches: bench.py times {steps} steps as ld_latent_decode and {steps} as its two",
             "launches with an event between; every step follows a 1 GiB read of a scratch buffer.", "",
             f"    {commands[0]}", "",
             "| kernel | calls | mean us (all calls) | in-step mean us | in-step median us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for k, v in per.items():
        tail = v[-2 * steps:] if (k == dec_name or k in comb) else v
        lines.append(f"| {k[:80]} | {len(v)} | {np.mean(v):.1f} | {np.mean(tail):.1f} | {np.median(tail):.1f} | "
                     f"{min(v):.1f} | {max(v):.1f} |")
    lines += ["", "HBM traffic of one in-step decode launch (TCC counters, one pass per counter, median over the",
              "in-step dispatches):", ""]
    lines += [f"    {c}" for c in commands[1:3]]
    lines += ["", f"- FETCH_SIZE {f_kib:.0f} KiB per dispatch; the {copy_mib} MiB copy reads {fcopy[-1]:.0f} KiB "
                  f"-> scale {fscale:.4f}",
              f"- WRITE_SIZE {w_kib:.0f} KiB per dispatch; the copy writes {wcopy[-1]:.0f} KiB -> scale {wscale:.4f}",
              f"- HBM bytes per launch: {hbm / 1e6:.1f} MB (read {f_kib * fscale * 1024 / 1e6:.1f} MB, "
              f"write {w_kib * wscale * 1024 / 1e6:.1f} MB)", "",
              "MFMA activity of one in-step decode launch (SQ/GRBM counters, median over the in-step dispatches):", "",
              f"    {commands[3]}", ""]
    lines += [f"- {c} {v:.4g}" for c, v in mf.items()]
    lines += [f"- MFMA bf16 flops counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512): "
              f"{mf['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.2f} GFLOP per launch"]
    lines += [f"- kernel busy cycles = GRBM_GUI_ACTIVE / {XCDS} XCDs = {gpu_cycles:.4g} "
              f"({gpu_cycles / (t['in_step_decode_us_mean'] * 1e-6) / 1e9:.2f} GHz over the traced in-step duration)",
              f"- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x {num_cus} CUs x 4 SIMDs) = {mfma_busy:.4f}",
              f"- decode source sha256[:16] {source_sha()}", ""]
    with open(os.path.join(PROFILES, f"decode_kernel_{workload}.md"), "w") as f:
        f.write("\n".join(lines))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--long-steps", type=int, default=50, help="timed steps of each long-context workload")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context sub-objects")
    ap.add_argument("--min-warmup-ms", type=float, default=50.0,
                    help="keep running untimed warmup steps until this much wall time has passed")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--stages", action="store_true", help="also time the staged path's launches back to back")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-around", action="store_true", help="skip the append / projection timings")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    ap.add_argument("--summarize-profile", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "MFMA_DIR"))
    ap.add_argument("--profile-commands", nargs=4, default=None, help="the four commands, for the summary")
    args = ap.parse_args()

    if args.summarize_profile:
        cmds = args.profile_commands or ["(not given)"] * 4
        summarize_profile(args.workload, *args.summarize_profile, args.calibrate_copy_mib or 512, args.steps, cmds)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path runs on one GPU; there is no multi-GPU path.", file=sys.stderr)
        return 2

    import torch

    import latent_kv_cache_absorbed_amd as lkd

    lkd.lib()
    dev = torch.device("cuda:0")
    flush = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    res, inp, d = measure(args.workload, args.steps, args.warmup, args.min_warmup_ms, dev, flush,
                          num_splits=args.num_splits, stages=args.stages, keep=True)
    stream = torch.cuda.current_stream(dev)
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if inp.kv_dtype == "bf16" else ("fp8_e4m3+bf16" if inp.kv_dtype == "fp8_e4m3" else "f32"),
        "data": "synthetic",
        "config": res["config"],
    }
    for k in ("step_us", "in_step_us", "tokens_per_s", "kv_tokens_per_s", "hbm_frac_step", "roofline",
              "warmup_steps_run", "timed_region_s", "input_gen_s", "stages_back_to_back_ms"):
        if k in res:
            line[k] = res[k]
    line["timing"] = ("per-step HIP events on the launch stream, a 1 GiB read (reduction) before each step outside "
                      "the events evicts L2 and the Infinity Cache; value and ms_per_step from the median step")
    if not args.no_parity:
        d.run()
        torch.cuda.synchronize()
        line["parity"] = parity_sample(inp, d.out.double().cpu().numpy(), d.lse.double().cpu().numpy())
    if not args.no_around and inp.variant in ("mla", "gla", "mlra"):
        import synth
        w = synth.WORKLOADS[args.workload]
        line["around_step"] = around_step(inp, w, dev, args.steps, stream, d.tensors[2], d.block_table, d.seq_lens,
                                          d.tensors[4], d.tensors[5], flush)
    del d
    torch.cuda.empty_cache()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if not args.no_long and args.workload == DEFAULT_WORKLOAD:
        longs = []
        for name in LONG_WORKLOADS:
            r, _, _ = measure(name, args.long_steps, args.warmup, args.min_warmup_ms, dev, flush)
            longs.append({k: r[k] for k in ("workload", "value", "unit", "step_us", "in_step_us", "tokens_per_s",
                                            "kv_tokens_per_s", "hbm_frac_step", "roofline", "config")})
            torch.cuda.empty_cache()
        line["long_context"] = longs
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
