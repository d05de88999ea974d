#!/usr/bin/env python3
"""Benchmark of the RoPE-4D joint-attention forward on one MI355X.

One step = one call of the attention library on one batch of the 2048x2048
text-to-image workload with CFG (cond + uncond batched): B=2, S=16,896
(512 text + 128x128 image tokens), H=24, D=128, bf16 in/out, inputs resident
in HBM before timing.  Throughput is attention TFLOP/s = 4*B*H*S^2*D / t.
The timed call is klein_rope4d_attn_fwd, the attention's own signature: the
key rotation pass, the pass that regroups the values into key-major tiles,
the attention kernel and its merge kernel (the split-KV schedule), in the
buffer the library creates on the first (warm-up) call.
The same schedule with a caller workspace (workspace_entry_ms), with the
static scratch of the entry point that allocates nothing (noalloc_entry_ms)
and the per-tile kernels that need no memory (per_tile_kernels_ms) are timed
beside it.

Prints ONE JSON line.  Fields beyond the common ones:
  roofline      -- the attention kernel against dense bf16 MFMA peak, with the
                   HBM traffic measured by rocprofv3 counters when the stored
                   measurement matches the current kernel sources;
  cpu_baseline  -- the fp64 CPU oracle timed on a bounded sample of the same
                   workload (a seeded subset of query rows), scaled to TFLOP/s;
  fp8           -- the FP8 E4M3 variant on the 2048x2048 edit workload
                   (S = 33,280), against dense fp8 MFMA peak;
  clock         -- the engine clock the attention kernels ran at, from a short
                   rocprofv3 counter run of this script right after the timing
                   (GRBM_GUI_ACTIVE per XCD over the dispatch duration), and
                   the fraction of the MFMA peak at that clock;
  next          -- the adjacent workloads: the attention backward at the
                   headline shape, the 1024x1024 workloads warm and cold, and
                   a 2048x2048 edit with two references.
"""

import argparse
import json
import os
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "joint-attention TFLOP/s + % MFMA peak at 2048² (16,896 tok, 24 heads×128)"
PEAK_BF16 = 2516.6      # dense bf16 MFMA, TFLOP/s (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP8 = 5033.2       # dense fp8 MFMA, TFLOP/s
def stored_traffic(name, call):
    """Memory bytes per call from a committed rocprofv3 counter summary
    (profiles/traffic_<name>.json), if it was taken on the current kernel
    sources; else None."""
    from joint_attention_rope_amd.profiling import CALLS, sources_hash
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("call") != call or rec.get("sources_hash") != sources_hash(CALLS[call]["sources"]):
        return None
    return rec.get("hbm_bytes_per_launch")


def traffic_source(name):
    """Where a stored traffic figure comes from: the summary file and the
    hash of the kernel sources it was taken on."""
    try:
        with open(os.path.join(ROOT, "profiles", f"traffic_{name}.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return f"profiles/traffic_{name}.json (rocprofv3 FETCH_SIZE + WRITE_SIZE passes, " \
           f"kernel sources hash {rec.get('sources_hash')})"


def to_device(inp, dev):
    """Seeded host inputs -> GPU tensors holding exactly the generator's bits."""
    import numpy as np
    import torch
    if inp.descale is None:
        conv = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        conv = lambda a: torch.from_numpy(a).to(dev)
    return conv(inp.q), conv(inp.k), conv(inp.v), torch.from_numpy(inp.pos).to(dev)


def time_gpu(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps          # ms per launch


def time_gpu_calls(fn, steps, warmup, torch):
    """Like time_gpu, with an event between every timed call: returns the mean
    ms per call over the whole timed region and the per-call durations."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, per


def workspace(kl, torch, cfg, dev):
    """The split-KV workspace of a workload's shape (None if it needs none)."""
    dt = kl.KLEIN_DTYPE_FP8_E4M3 if cfg.dtype == "fp8" else kl.KLEIN_DTYPE_BF16
    n = kl.klein_attn_workspace_size(cfg.B, cfg.S, cfg.H, cfg.D, dt)
    return torch.empty(n, dtype=torch.uint8, device=dev) if n else None


def cpu_baseline(inp, cfg, target_s=15.0):
    """Time the fp64 oracle on a seeded sample of query rows of batch entry 0,
    all heads; scale its rate to TFLOP/s with the same 4*S*D flops per row."""
    import numpy as np
    import oracle
    from workloads import Inputs
    visible = len(os.sched_getaffinity(0))
    # a shared host may give each GPU a share of its threads (16 on the
    # MI355X hosts measured), whatever the affinity mask shows;
    # OMP_NUM_THREADS states that share
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    workers = min(visible, share) if share > 0 else visible
    sub = Inputs(cfg, inp.q[:1], inp.k[:1], inp.v[:1], inp.pos, inp.descale)
    rng = np.random.default_rng(12345)
    # a discarded warm-up (thread pool, BLAS), then a calibration sample that
    # sizes the timed one to about target_s seconds
    oracle.attention_inputs_rows(sub, np.arange(8), workers=workers)
    rows = np.sort(rng.choice(cfg.S, size=128, replace=False))
    t0 = time.perf_counter()
    oracle.attention_inputs_rows(sub, rows, workers=workers)
    t_cal = time.perf_counter() - t0
    n = int(min(cfg.S, max(128, 128 * target_s / max(t_cal, 1e-3))))
    # larger samples run faster per row (bigger blocks, better balance), so
    # one short run is resized once
    for _ in range(2):
        rows = np.sort(rng.choice(cfg.S, size=n, replace=False))
        t0 = time.perf_counter()
        oracle.attention_inputs_rows(sub, rows, workers=workers)
        dt = time.perf_counter() - t0
        if dt >= 0.7 * target_s or n == cfg.S:
            break
        n = int(min(cfg.S, n * target_s / max(dt, 1e-3)))
    flops = 4.0 * n * cfg.S * cfg.D * cfg.H
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "cores_visible": visible,
        "kind": "oracle",
        "sample": f"{n} seeded query rows x {cfg.H} heads of batch entry 0 "
                  f"(all {cfg.S} keys each), float64 NumPy, {dt:.1f} s",
    }


def time_per_tile(kl, fn, steps, warmup, torch):
    """time_gpu of fn with the library's buffer limit at 0, so that the plain
    entry points run the per-tile kernels that need no memory."""
    kl.klein_set_buffer_limit(0)
    try:
        return time_gpu(fn, steps, warmup, torch)
    finally:
        kl.klein_set_buffer_limit(kl.KLEIN_DEFAULT_BUFFER_LIMIT)


def plain_call(kl, inp, q, k, v, pos, out):
    """The timed entry point for a workload: klein_rope4d_attn_fwd (bf16) or
    klein_rope4d_attn_fwd_fp8 (E4M3 codes with the workload's descales)."""
    if inp.descale is None:
        return lambda: kl.klein_rope4d_attn_fwd(q, k, v, pos, out)
    return lambda: kl.klein_rope4d_attn_fwd_fp8(q, k, v, pos, out, *inp.descale)


# kernels whose engine clock the counter run reports
CLOCK_KERNELS = {"bf16": "attn_fwd_bf16_kernel", "fp8": "attn_fwd_fp8_kernel"}


def clock_child(torch, kl, dev):
    """--clock-child: a few calls of the two timed entry points on their
    workloads, for the counter run that observed_clock() makes of this."""
    from workloads import get_config, make_inputs
    for cid in (4, 5):
        c = get_config(cid)
        print(f"[clock] {c.dtype} S={c.S}: generating inputs", file=sys.stderr, flush=True)
        xi = make_inputs(c)
        xq, xk, xv, xp = to_device(xi, dev)
        xo = torch.empty(xq.shape, dtype=torch.bfloat16, device=dev)
        call = plain_call(kl, xi, xq, xk, xv, xp, xo)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        print(f"[clock] {c.dtype}: 5 calls done", file=sys.stderr, flush=True)
        del xq, xk, xv, xo


def observed_clock():
    """Engine clock while the attention kernels run: one rocprofv3 counter
    pass (GRBM_GUI_ACTIVE, the busy cycles of each XCD) over a child run of
    this script (--clock-child), divided by each dispatch's duration; the mean
    over the last three dispatches of each kernel, in MHz.  The profiler runs
    as a child process (never in place of this one)."""
    import csv
    import shutil
    prof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    out = tempfile.mkdtemp(prefix="klein_clock_", dir="/tmp")
    cmd = [prof, "--log-level", "error", "--pmc", "GRBM_GUI_ACTIVE", "--output-format", "csv",
           "-d", out, "-o", "clk", "--", sys.executable, os.path.join(ROOT, "bench.py"),
           "--clock-child"]
    print("[clock] counter run: " + " ".join(cmd[:8]) + " ... -- bench.py --clock-child",
          file=sys.stderr, flush=True)
    res = {"method": "rocprofv3 --pmc GRBM_GUI_ACTIVE over a child run of bench.py --clock-child "
                     "right after the timed region: busy cycles per XCD / dispatch duration, "
                     "mean of the last 3 dispatches"}
    try:
        r = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"),
                           stdout=subprocess.DEVNULL, timeout=240)
        # the profiler can end with a signal after the program's results are
        # complete; the counters file decides
        found = [os.path.join(dp, f) for dp, _, fs in os.walk(out) for f in fs
                 if f.endswith("counter_collection.csv")]
        if not found:
            res["error"] = f"no counter output (exit status {r.returncode})"
            return res
        per = {}
        with open(found[0]) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != "GRBM_GUI_ACTIVE":
                    continue
                for key, name in CLOCK_KERNELS.items():
                    if name in row["Kernel_Name"]:
                        d = per.setdefault(key, {}).setdefault(
                            int(row["Dispatch_Id"]),
                            [0.0, int(row["End_Timestamp"]) - int(row["Start_Timestamp"])])
                        d[0] += float(row["Counter_Value"])
        for key, disp in per.items():
            last = [disp[k] for k in sorted(disp)][-3:]
            res[f"{key}_mhz"] = round(sum(c / 8 / ns * 1e3 for c, ns in last) / len(last), 1)
        return res
    except (OSError, subprocess.SubprocessError, ValueError, KeyError) as e:
        res["error"] = f"{type(e).__name__}: {e}"
        return res
    finally:
        shutil.rmtree(out, ignore_errors=True)


def qkv_rows(torch, kl, dev, pos):
    """The QKV projection with the RoPE-4D epilogue at the headline shape
    (hidden C = H D = 3072, an assumption: the pages give no width), bf16 and
    E4M3 operands, each against torch's GEMM (hipBLASLt) on the same operands
    without the rotation."""
    from workloads import get_config
    c = get_config(4)
    C = c.H * c.D
    print(f"[next] qkv projection M={c.B * c.S} N={3 * C} K={C}", file=sys.stderr, flush=True)
    g = torch.Generator(device=dev).manual_seed(404)
    xx = torch.randn(c.B, c.S, C, device=dev, generator=g).to(torch.bfloat16)
    ww = (torch.randn(3 * C, C, device=dev, generator=g) / C ** 0.5).to(torch.bfloat16)
    bb = (torch.randn(3 * C, device=dev, generator=g) * 0.1).to(torch.bfloat16)
    pp = torch.from_numpy(pos).to(dev)
    qo = torch.empty(c.B, c.S, c.H, c.D, dtype=torch.float16, device=dev)
    ko = torch.empty_like(qo)
    vo = torch.empty(c.B, c.S, c.H, c.D, dtype=torch.bfloat16, device=dev)
    pms = time_gpu(lambda: kl.klein_qkv_rope4d_proj(xx, ww, bb, pp, qo, ko, vo), 10, 3, torch)
    yy = torch.empty(c.B, c.S, 3 * C, dtype=torch.bfloat16, device=dev)
    xm = xx.view(-1, C)
    tms = time_gpu(lambda: torch.addmm(bb, xm, ww.t(), out=yy.view(-1, 3 * C)), 10, 3, torch)
    gf = 2.0 * c.B * c.S * 3 * C * C
    rows = [{
        "workload": f"QKV projection + RoPE-4D epilogue: x [{c.B}, {c.S}, {C}] bf16, "
                    f"W [{3 * C}, {C}] bf16, bias; q', k' fp16, v bf16",
        "ms_per_call": round(pms, 4), "tflops": round(gf / (pms * 1e-3) / 1e12, 2),
        "peak": PEAK_BF16, "frac": round(gf / (pms * 1e-3) / 1e12 / PEAK_BF16, 4),
        "torch_addmm_ms": round(tms, 4),
        "torch_addmm_tflops": round(gf / (tms * 1e-3) / 1e12, 2)}]
    del yy
    # the same projection on E4M3 operands (per-tensor amax/448 scales),
    # against torch's fp8 GEMM (torch._scaled_mm, hipBLASLt) on the codes
    sx = float(xx.float().abs().max()) / 448.0
    sw = float(ww.float().abs().max()) / 448.0
    x8 = (xx.float() / sx).to(torch.float8_e4m3fn)
    w8 = (ww.float() / sw).to(torch.float8_e4m3fn)
    xq, wq = x8.view(torch.uint8), w8.view(torch.uint8)
    fms = time_gpu(lambda: kl.klein_qkv_rope4d_proj(xq, wq, bb, pp, qo, ko, vo,
                                                    descales=(sx, sw)), 10, 3, torch)
    rec_fp8 = {
        "workload": f"QKV projection + RoPE-4D epilogue, FP8 operands: x [{c.B}, {c.S}, {C}] "
                    f"and W [{3 * C}, {C}] E4M3 with per-tensor scales, bf16 bias; "
                    f"q', k' fp16, v bf16",
        "ms_per_call": round(fms, 4), "tflops": round(gf / (fms * 1e-3) / 1e12, 2),
        "peak": PEAK_FP8, "frac": round(gf / (fms * 1e-3) / 1e12 / PEAK_FP8, 4)}
    try:
        one = torch.ones((), device=dev)
        sa_, sb_ = one * sx, one * sw
        x8m = x8.view(-1, C)
        yy8 = lambda: torch._scaled_mm(x8m, w8.t(), scale_a=sa_, scale_b=sb_,
                                       out_dtype=torch.bfloat16)
        sms = time_gpu(yy8, 10, 3, torch)
        rec_fp8["torch_scaled_mm_ms"] = round(sms, 4)
        rec_fp8["torch_scaled_mm_tflops"] = round(gf / (sms * 1e-3) / 1e12, 2)
    except Exception as e:     # the comparison only; the projection is timed above
        rec_fp8["torch_scaled_mm"] = f"unavailable: {e}"
    rows.append(rec_fp8)
    del xx, ww, bb, qo, ko, vo, x8, w8, xq, wq
    return rows


def next_rows(torch, kl, dev, inp4, steps):
    """The adjacent workloads, each against its MFMA peak: the attention
    backward at the headline shape (LoRA / DreamBooth-style training), the
    1024x1024 workloads warm and cold, a 2048x2048 edit with two references
    (tokens grow by one image grid per reference) and the QKV projection that
    feeds the attention."""
    from workloads import get_config, make_inputs
    rows = []
    # backward at the 2048x2048 CFG shape: forward with lse once, then the
    # timed backward call (prep, scale, dK/dV and dQ kernels); flops counted
    # as 2.5x the forward's (the five S^2-sized products)
    c = get_config(4)
    print(f"[next] backward S={c.S}", file=sys.stderr, flush=True)
    xq, xk, xv, xp = to_device(inp4, dev)
    xo = torch.empty(xq.shape, dtype=torch.bfloat16, device=dev)
    xl = torch.empty(c.B, c.H, c.S, dtype=torch.float32, device=dev)
    kl.klein_rope4d_attn_fwd_lse(xq, xk, xv, xp, xo, xl)
    g = torch.Generator(device=dev).manual_seed(505)
    xd = torch.randn(xq.shape, device=dev, generator=g).to(torch.bfloat16)
    gq, gk, gv = (torch.empty_like(xq) for _ in range(3))
    xw = torch.empty(kl.klein_attn_bwd_workspace_size(c.B, c.S, c.H, c.D), dtype=torch.uint8,
                     device=dev)
    bms = time_gpu(lambda: kl.klein_rope4d_attn_bwd(xq, xk, xv, xp, xo, xd, xl, gq, gk, gv, xw),
                   max(3, steps // 2), 2, torch)
    bf = 2.5 * c.flops
    rows.append({"workload": f"attention backward (dq, dk, dv through RoPE-4D), {c.name}: "
                             f"B={c.B}, S={c.S}, H={c.H}, D={c.D}, bf16",
                 "ms_per_call": round(bms, 4), "tflops": round(bf / (bms * 1e-3) / 1e12, 2),
                 "peak": PEAK_BF16, "frac": round(bf / (bms * 1e-3) / 1e12 / PEAK_BF16, 4)})
    del xq, xk, xv, xo, xl, xd, gq, gk, gv, xw
    # the 1024x1024 workloads, warm (back to back) and cold (a 1 GiB buffer
    # written before each call, so no input is left in L2 or the Infinity Cache)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    for cid in (2, 3):
        c = get_config(cid)
        print(f"[next] {c.name} warm and cold", file=sys.stderr, flush=True)
        xi = make_inputs(c)
        xq, xk, xv, xp = to_device(xi, dev)
        xo = torch.empty(xq.shape, dtype=torch.bfloat16, device=dev)
        call = plain_call(kl, xi, xq, xk, xv, xp, xo)
        _, wper = time_gpu_calls(call, 50, 100, torch)
        cold = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(30):
            flush.fill_(1.0)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        wt, ct = c.flops / (med(wper) * 1e-3) / 1e12, c.flops / (med(cold) * 1e-3) / 1e12
        rows.append({"workload": f"{c.name}: B={c.B}, S={c.S}, H={c.H}, D={c.D}, bf16 "
                                 f"(klein_rope4d_attn_fwd)",
                     "warm_ms_median": round(med(wper), 4), "cold_ms_median": round(med(cold), 4),
                     "warm_tflops": round(wt, 2), "cold_tflops": round(ct, 2),
                     "peak": PEAK_BF16, "warm_frac": round(wt / PEAK_BF16, 4),
                     "cold_frac": round(ct / PEAK_BF16, 4)})
        del xq, xk, xv, xo
    del flush
    # a 2048x2048 edit with two reference images (t = 1, 2), bf16
    c = get_config(3, grid=128, refs=2)
    print(f"[next] 2048x2048 edit, 2 references, S={c.S}", file=sys.stderr, flush=True)
    xi = make_inputs(c)
    xq, xk, xv, xp = to_device(xi, dev)
    xo = torch.empty(xq.shape, dtype=torch.bfloat16, device=dev)
    xms = time_gpu(plain_call(kl, xi, xq, xk, xv, xp, xo), 5, 2, torch)
    xt = c.flops / (xms * 1e-3) / 1e12
    rows.append({"workload": f"2048x2048 edit with 2 references: B={c.B}, S={c.S} ({c.text} "
                             f"text + 3 x 128x128), H={c.H}, D={c.D}, bf16 "
                             f"(klein_rope4d_attn_fwd)",
                 "ms_per_call": round(xms, 4), "tflops": round(xt, 2), "peak": PEAK_BF16,
                 "frac": round(xt / PEAK_BF16, 4)})
    del xq, xk, xv, xo
    rows.extend(qkv_rows(torch, kl, dev, inp4.pos))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--extra", action="store_true",
                    help="also time an fp8 2048x2048 edit with 3 references, one GPU's share "
                         "of sharded shapes, block-sparse attention and the QKV projection, "
                         "and report them under 'extra'")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the counter run that measures the engine clock")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the adjacent workloads (backward, 1024x1024, multi-reference)")
    ap.add_argument("--clock-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after timing, run an elementwise fp32 copy of MIB MiB three "
                         "times (a kernel of known HBM traffic for scaling counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention shards by batch entry and head with no exchange; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import joint_attention_rope_amd as kl
    from workloads import get_config, make_inputs

    dev = "cuda:0"
    if args.clock_child:
        clock_child(torch, kl, dev)
        return
    cfg = get_config(4)
    inp = make_inputs(cfg)
    q, k, v, pos = to_device(inp, dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    # the timed call: klein_rope4d_attn_fwd, the attention's own signature; its
    # buffer (keys rotated once, values in key-major tiles, split-KV partials)
    # is created by the first warm-up call, and the inputs are resident before
    # timing.  The same schedule with a caller workspace, with the static
    # scratch of the entry point that allocates nothing, and the per-tile
    # kernels (buffer limit 0) are timed after it for reference.
    ms, per_call = time_gpu_calls(lambda: kl.klein_rope4d_attn_fwd(q, k, v, pos, out),
                                  args.steps, args.warmup, torch)
    buf_mb = kl.klein_attn_workspace_size(cfg.B, cfg.S, cfg.H, cfg.D) / 1e6
    n_ref = max(3, args.steps // 4)
    ws = workspace(kl, torch, cfg, dev)
    ws_ms = time_gpu(lambda: kl.klein_rope4d_attn_fwd_ws(q, k, v, pos, out, ws), n_ref, 2, torch)
    del ws
    noalloc_ms = time_gpu(lambda: kl.klein_rope4d_attn_fwd_noalloc(q, k, v, pos, out),
                          n_ref, 2, torch)
    per_tile_ms = time_per_tile(kl, lambda: kl.klein_rope4d_attn_fwd(q, k, v, pos, out), n_ref, 2,
                                torch)
    tflops = cfg.flops / (ms * 1e-3) / 1e12
    traffic = stored_traffic("attn_fwd_bf16_2048px_t2i_cfg", "attn_fwd_bf16_splitkv")
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V; uncond text tokens zeroed)",
        "config": {"workload": "2048x2048 text-to-image with CFG: B=2, S=16896 "
                               "(512 text + 128x128 image), H=24, D=128, bf16",
                   "global_batch": cfg.B, "seq_len": cfg.S, "heads": cfg.H,
                   "head_dim": cfg.D, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16, 4),
                     "traffic": traffic,
                     "traffic_source": traffic_source("attn_fwd_bf16_2048px_t2i_cfg")
                     if traffic is not None else None},
        "entry_point": "klein_rope4d_attn_fwd (split-KV schedule in the library's buffer, "
                       f"{buf_mb:.1f} MB)",
        "workspace_entry_ms": round(ws_ms, 4),
        "noalloc_entry_ms": round(noalloc_ms, 4),
        "per_tile_kernels_ms": round(per_tile_ms, 4),
        "ms_per_call_median": round(sorted(per_call)[len(per_call) // 2], 4),
        "ms_per_call_min": round(min(per_call), 4),
    }
    del q, k, v, out
    if not args.no_fp8:
        try:
            cfg5 = get_config(5)
            inp5 = make_inputs(cfg5)
            q5, k5, v5, p5 = to_device(inp5, dev)
            o5 = torch.empty(q5.shape, dtype=torch.bfloat16, device=dev)
            ms5 = time_gpu(lambda: kl.klein_rope4d_attn_fwd_fp8(q5, k5, v5, p5, o5,
                                                                *inp5.descale),
                           max(3, args.steps // 2), max(1, args.warmup // 2), torch)
            ws5 = workspace(kl, torch, cfg5, dev)
            ws5_ms = time_gpu(lambda: kl.klein_rope4d_attn_fwd_ws(q5, k5, v5, p5, o5, ws5,
                                                                  descales=inp5.descale),
                              3, 1, torch)
            per_tile5 = time_per_tile(kl, lambda: kl.klein_rope4d_attn_fwd_fp8(
                q5, k5, v5, p5, o5, *inp5.descale), 3, 1, torch)
            t5 = cfg5.flops / (ms5 * 1e-3) / 1e12
            traffic5 = stored_traffic("attn_fwd_fp8_2048px_edit", "attn_fwd_fp8_splitkv")
            rec["fp8"] = {"workload": "2048x2048 edit: B=1, S=33280 (512 text + 2 x 128x128), "
                                      "H=24, D=128, e4m3 in, bf16 out",
                          "ms_per_call": round(ms5, 4), "tflops": round(t5, 2),
                          "peak": PEAK_FP8, "frac": round(t5 / PEAK_FP8, 4),
                          "traffic": traffic5,
                          "traffic_source": traffic_source("attn_fwd_fp8_2048px_edit")
                          if traffic5 is not None else None,
                          "entry_point": "klein_rope4d_attn_fwd_fp8 (split-KV schedule in "
                                         "the library's buffer)",
                          "workspace_entry_ms": round(ws5_ms, 4),
                          "per_tile_kernels_ms": round(per_tile5, 4)}
            del q5, k5, v5, o5, ws5
        except kl.KleinError as e:
            rec["fp8"] = {"error": str(e)}
    if not args.no_clock:
        clk = observed_clock()
        for key, t, peak in (("bf16", tflops, PEAK_BF16),
                             ("fp8", rec.get("fp8", {}).get("tflops"), PEAK_FP8)):
            mhz = clk.get(f"{key}_mhz")
            if mhz and t:
                # the same rate against the MFMA peak at the clock observed
                clk[f"{key}_frac_at_observed_clock"] = round(t / (peak * mhz / 2400.0), 4)
        rec["clock"] = clk
    if not args.no_next:
        rec["next"] = next_rows(torch, kl, dev, inp, args.steps)
    if args.extra:
        rec["extra"] = []
        # (the bf16 edit with 2 references is in "next")
        for cid, refs, peak in ((5, 3, PEAK_FP8),):
            c = get_config(cid, grid=128, refs=refs)
            print(f"[extra] generating {c.dtype} S={c.S} inputs", file=sys.stderr, flush=True)
            xi = make_inputs(c)
            print(f"[extra] timing {c.dtype} S={c.S}", file=sys.stderr, flush=True)
            xq, xk, xv, xp = to_device(xi, dev)
            xo = torch.empty(xq.shape, dtype=torch.bfloat16, device=dev)
            call = plain_call(kl, xi, xq, xk, xv, xp, xo)
            xms = time_gpu(call, 5, 2, torch)
            dms = time_per_tile(kl, call, 3, 1, torch)
            xt = c.flops / (xms * 1e-3) / 1e12
            rec["extra"].append({
                "workload": f"2048x2048 edit with {refs} references: B={c.B}, S={c.S} "
                            f"({c.text} text + {refs + 1} x 128x128), H={c.H}, D={c.D}, {c.dtype}",
                "ms_per_call": round(xms, 4), "tflops": round(xt, 2), "peak": peak,
                "frac": round(xt / peak, 4), "per_tile_kernels_ms": round(dms, 4)})
            del xq, xk, xv, xo
        # one GPU's share of the 2048x2048 workload under sequence parallelism
        # (heads split over GPUs after an all-to-all): 3 or 4 heads of one CFG
        # branch (8- or 6-way), 6 heads of one branch (4-way), both branches
        # with 3 heads; the workload's inputs and positions at that size
        for B, H in ((1, 3), (1, 4), (1, 6), (2, 3)):
            c = get_config(4, B=B, H=H, uncond_zero_text=B == 2)
            print(f"[extra] shard B={B} H={H} S={c.S}", file=sys.stderr, flush=True)
            xi = make_inputs(c)
            xq, xk, xv, xp = to_device(xi, dev)
            xo = torch.empty(xq.shape, dtype=torch.bfloat16, device=dev)
            call = plain_call(kl, xi, xq, xk, xv, xp, xo)
            # calls of ~0.5-1 ms: ~100 ms of warm-up first, so that the clock has
            # left the idle state of the input generation before timing
            xms = time_gpu(call, 50, 150, torch)
            dms = time_per_tile(kl, call, 50, 150, torch)
            xt = c.flops / (xms * 1e-3) / 1e12
            rec["extra"].append({
                "workload": f"one GPU's share of 2048x2048 t2i: B={B}, S={c.S}, H={H}, D={c.D}, "
                            f"bf16 ({B * H * ((c.S + 255) // 256)} query tiles)",
                "ms_per_call": round(xms, 4), "tflops": round(xt, 2), "peak": PEAK_BF16,
                "frac": round(xt / PEAK_BF16, 4), "per_tile_kernels_ms": round(dms, 4),
                "per_tile_kernels_tflops": round(c.flops / (dms * 1e-3) / 1e12, 2)})
            del xq, xk, xv, xo
        # block-sparse: the bench workloads with a seeded structured mask
        # (text blocks, a band around each query block, 30 % of the rest)
        from workloads import make_block_mask
        for cid, peak in ((4, PEAK_BF16), (5, PEAK_FP8)):
            c = get_config(cid)
            print(f"[extra] block-sparse {c.dtype} S={c.S}", file=sys.stderr, flush=True)
            xi = inp if cid == 4 else make_inputs(c)
            xq, xk, xv, xp = to_device(xi, dev)
            xo = torch.empty(xq.shape, dtype=torch.bfloat16, device=dev)
            mask = make_block_mask(c.B, c.H, c.S, c.text, 0.3, seed=cid)
            xm = torch.from_numpy(mask).to(dev)
            desc = xi.descale or (1.0, 1.0, 1.0)
            sms = time_gpu(lambda: kl.klein_rope4d_attn_fwd_blocksparse(
                xq, xk, xv, xp, xo, xm, descales=desc), 5, 2, torch)
            if xi.descale is None:
                dense = lambda: kl.klein_rope4d_attn_fwd(xq, xk, xv, xp, xo)
            else:
                dense = lambda: kl.klein_rope4d_attn_fwd_fp8(xq, xk, xv, xp, xo, *xi.descale)
            dms = time_gpu(dense, 5, 2, torch)
            qn = np.minimum(256, c.S - 256 * np.arange(mask.shape[2]))
            kn = np.minimum(64, c.S - 64 * np.arange(mask.shape[3]))
            pairs = float(np.einsum("bhij,i,j->", mask.astype(np.float64), qn, kn))
            eff = 4.0 * c.D * pairs / (sms * 1e-3) / 1e12
            # the same with the keys rotated once into a workspace
            dt = kl.KLEIN_DTYPE_BF16 if xi.descale is None else kl.KLEIN_DTYPE_FP8_E4M3
            xw = torch.empty(kl.klein_attn_workspace_size(c.B, c.S, c.H, c.D, dt),
                             dtype=torch.uint8, device=dev)
            wms = time_gpu(lambda: kl.klein_rope4d_attn_fwd_blocksparse(
                xq, xk, xv, xp, xo, xm, descales=desc, workspace=xw), 5, 2, torch)
            weff = 4.0 * c.D * pairs / (wms * 1e-3) / 1e12
            rec["extra"].append({
                "workload": f"block-sparse {c.name}: B={c.B}, S={c.S}, H={c.H}, D={c.D}, "
                            f"{c.dtype}; mask keeps {100 * mask.mean():.1f} % of 256x64 blocks",
                "ms_per_call": round(sms, 4), "dense_ms_per_call": round(dms, 4),
                "speedup_vs_dense": round(dms / sms, 3),
                "effective_tflops": round(eff, 2), "peak": peak, "frac": round(eff / peak, 4),
                "keys_rotated_once_ms": round(wms, 4),
                "keys_rotated_once_effective_tflops": round(weff, 2)})
            del xq, xk, xv, xo, xm, xw
    if args.extra:
        # the attention on the projection's pre-rotated output, against the
        # fused-rotation attention
        c = get_config(4)
        C = c.H * c.D
        print(f"[extra] attention on pre-rotated q', k' S={c.S}", file=sys.stderr, flush=True)
        g = torch.Generator(device=dev).manual_seed(404)
        xx = torch.randn(c.B, c.S, C, device=dev, generator=g).to(torch.bfloat16)
        ww = (torch.randn(3 * C, C, device=dev, generator=g) / C ** 0.5).to(torch.bfloat16)
        pp = torch.from_numpy(inp.pos).to(dev)
        qo = torch.empty(c.B, c.S, c.H, c.D, dtype=torch.float16, device=dev)
        ko = torch.empty_like(qo)
        vo = torch.empty(c.B, c.S, c.H, c.D, dtype=torch.bfloat16, device=dev)
        oo = torch.empty_like(vo)
        kl.klein_qkv_rope4d_proj(xx, ww, None, pp, qo, ko, vo)
        ams = time_gpu(lambda: kl.klein_attn_fwd_prerotated(qo, ko, vo, oo), 10, 3, torch)
        rec["extra"].append({
            "workload": f"attention on pre-rotated fp16 q', k' (bf16 v): {c.name}, B={c.B}, "
                        f"S={c.S}, H={c.H}, D={c.D}",
            "ms_per_call": round(ams, 4), "tflops": round(c.flops / (ams * 1e-3) / 1e12, 2),
            "peak": PEAK_BF16, "frac": round(c.flops / (ams * 1e-3) / 1e12 / PEAK_BF16, 4),
            "fused_rotation_ms": round(ms, 4)})
        del xx, ww, qo, ko, vo, oo
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)        # reads 4n bytes, writes 4n bytes
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = 4 * n
        del src, dst
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
