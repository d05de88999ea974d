"""Turn rocprofv3 CSV output into the committed profile summaries.

Three rocprofv3 runs of bench.py feed the trace/traffic summary (each with
--copy-calibration, which adds an elementwise fp32 copy of known size):

  rocprofv3 --kernel-trace --stats --output-format csv -d STATS -o run -- python3 bench.py ...
  rocprofv3 --pmc FETCH_SIZE      --output-format csv -d FETCH -o run -- python3 bench.py ...
  rocprofv3 --pmc WRITE_SIZE      --output-format csv -d WRITE -o run -- python3 bench.py ...

FETCH_SIZE / WRITE_SIZE (KiB per dispatch, L2-to-memory traffic) are scaled by
known_bytes / counter for the copy kernel, then reported per call (the
attention kernel plus, on the split-KV path, its merge kernel) next to the
call's algorithmic bytes.

  python -m joint_attention_rope_amd.profiling --call attn_fwd_bf16_splitkv \
      --name attn_fwd_bf16_2048px_t2i_cfg --workload 4 --stats STATS --fetch FETCH \
      --write WRITE --steps 5 --copy-mib 1024 --command "..."

Two more --pmc runs with the SQ counter sets below feed the instruction and
utilisation summary (--counters PASS1 PASS2 instead of --stats/--fetch/--write).
"""

import argparse
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL = "MulFunctor"

# A profiled call of an entry point: the elementwise passes dispatched before
# the attention kernel (the keys rotated once; for bf16 the values regrouped
# into key-major tiles), the attention kernel (matched on the demangled name,
# template arguments included) and, on the split-KV path, the merge kernel
# dispatched after it; and the sources the measurement depends on.
CALLS = {
    "attn_fwd_bf16_splitkv": {
        "before": ["rope4d_fp16_kernel<128>", "v_tiles_kernel<128>"],
        "kernel": "attn_fwd_bf16_kernel<128, false, 1, true, true>",
        "merge": "split_merge_kernel<128>",
        "sources": ["klein_device.hpp", "attn_fwd_bf16.hip", "split_schedule.hip",
                    "rope_apply.hip"]},
    "attn_fwd_fp8_splitkv": {
        "before": ["rope4d_fp8_kernel<128>"],
        "kernel": "attn_fwd_fp8_kernel<128, false, true, true>",
        "merge": "split_merge_kernel<128>",
        "sources": ["klein_device.hpp", "attn_fwd_fp8.hip", "split_schedule.hip"]},
    "attn_fwd_bf16_dense": {
        "before": [], "kernel": "attn_fwd_bf16_kernel<128, false, 0, false, false>",
        "merge": None, "sources": ["klein_device.hpp", "attn_fwd_bf16.hip"]},
    "attn_fwd_fp8_dense": {
        "before": [], "kernel": "attn_fwd_fp8_kernel<128, false, false, false>", "merge": None,
        "sources": ["klein_device.hpp", "attn_fwd_fp8.hip"]},
}


def sources_hash(names):
    """Short hash of the kernel sources a measurement was taken on."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(PKG, "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirname, suffix):
    for root, _, files in os.walk(dirname):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirname}")


def _pair(ids_kernel, ids_other, after=True):
    """For each attention dispatch id, the nearest dispatch id of the other
    kernel after it (before the next attention dispatch), or with after=False
    before it (after the previous attention dispatch); None if there is none."""
    ks = sorted(ids_kernel)
    os_ = sorted(ids_other)
    out = {}
    for i, k in enumerate(ks):
        if after:
            nxt = ks[i + 1] if i + 1 < len(ks) else float("inf")
            out[k] = next((m for m in os_ if k < m < nxt), None)
        else:
            prv = ks[i - 1] if i > 0 else -1
            cand = [m for m in os_ if prv < m < k]
            out[k] = cand[-1] if cand else None
    return out


def _ids(rows, name):
    return [int(r["Dispatch_Id"]) for r in rows if name and name in r["Kernel_Name"]]


def call_durations_ns(stats_dir, call):
    """Per call, in dispatch order: (passes before the kernel ns, attention
    kernel ns, merge kernel ns)."""
    c = CALLS[call]
    rows = _rows(_find(stats_dir, "kernel_trace.csv"))
    dur = {int(r["Dispatch_Id"]): int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows}
    ks = _ids(rows, c["kernel"])
    pm = _pair(ks, _ids(rows, c["merge"]))
    pbs = [_pair(ks, _ids(rows, b), after=False) for b in c["before"]]
    get = lambda d: dur[d] if d is not None else 0
    return [(sum(get(pb[k]) for pb in pbs), dur[k], get(pm[k])) for k in sorted(ks)]


def counter_per_dispatch(pmc_dir, kernel, counter):
    """Counter value per dispatch of a kernel (summed over reporting units)."""
    per = {}
    for r in _rows(_find(pmc_dir, "counter_collection.csv")):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            k = int(r["Dispatch_Id"])
            per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    return per


def call_counter(pmc_dir, call, counter):
    """Per call: the counter of the attention kernel plus those of the
    passes before it and of its merge."""
    c = CALLS[call]
    ks = counter_per_dispatch(pmc_dir, c["kernel"], counter)
    ms = counter_per_dispatch(pmc_dir, c["merge"], counter) if c["merge"] else {}
    pm = _pair(list(ks), list(ms))
    out = [ks[k] + (ms[pm[k]] if pm[k] is not None else 0.0) for k in sorted(ks)]
    for b in c["before"]:
        bs = counter_per_dispatch(pmc_dir, b, counter)
        pb = _pair(list(ks), list(bs), after=False)
        out = [o + (bs[pb[k]] if pb[k] is not None else 0.0) for o, k in zip(out, sorted(ks))]
    return out


# Counter passes (8 SQ counters and one GRBM counter per pass at most).
COUNTER_PASSES = [
    "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_TRANS_F32 SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_SALU "
    "SQ_INSTS_VMEM SQ_WAVES SQ_ACTIVE_INST_ANY",
]
SIMDS = 256 * 4


def counter_means(dirs, kernel):
    """Mean per dispatch of every counter collected for `kernel` in `dirs`
    (values of one dispatch summed over the units that report them)."""
    out = {}
    for d in dirs:
        per = {}
        for r in _rows(_find(d, "counter_collection.csv")):
            if kernel in r["Kernel_Name"]:
                key = (r["Dispatch_Id"], r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        by = {}
        for (_, c), v in per.items():
            by.setdefault(c, []).append(v)
        for c, vs in by.items():
            out[c] = sum(vs) / len(vs)
    return out


def mean_duration_ns(pmc_dir, kernel):
    """Mean dispatch duration of a kernel in a counter run."""
    per = {}
    for r in _rows(_find(pmc_dir, "counter_collection.csv")):
        if kernel in r["Kernel_Name"]:
            per[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return sum(per.values()) / len(per) if per else None


def counters_markdown(kernel, cfg, dirs, command, units=None, unit_name=None):
    """Instruction mix per wave-tile (one wave's 32 queries against one
    64-key tile; or per `units` of `unit_name` when given) and MFMA
    utilisation from the SQ counter passes."""
    c = counter_means(dirs, kernel)
    if units:
        tiles = units
        per = f"Units per dispatch: {units} ({unit_name})."
    else:
        nqt = (cfg.S + 255) // 256
        nkt = (cfg.S + 63) // 64
        tiles = cfg.B * cfg.H * nqt * 8 * nkt
        per = (f"Wave-tiles per dispatch: {tiles} (B x H x {nqt} query tiles x 8 waves x "
               f"{nkt} key tiles).")
    rows = [("SQ_INSTS_MFMA", "MFMA instructions"), ("SQ_INSTS_VALU", "VALU instructions (incl. MFMA)"),
            ("SQ_INSTS_VALU_TRANS_F32", "transcendental VALU (exp, sin, cos)"),
            ("SQ_INSTS_LDS", "LDS instructions"), ("SQ_LDS_BANK_CONFLICT", "LDS bank-conflict cycles"),
            ("SQ_INSTS_SALU", "SALU instructions"), ("SQ_INSTS_VMEM", "vector memory instructions"),
            ("SQ_VALU_MFMA_BUSY_CYCLES", "MFMA busy cycles"),
            ("SQ_WAIT_INST_LDS", "cycles waiting for LDS data (x4)"),
            ("SQ_WAIT_INST_ANY", "cycles waiting for any dependency (x4)"),
            ("SQ_WAVE_CYCLES", "wave cycles (x4)")]
    lines = [f"| counter | meaning | per dispatch | per {'unit' if units else 'wave-tile'} |",
             "|---|---|---|---|"]
    for k, m in rows:
        if k in c:
            lines.append(f"| {k} | {m} | {c[k]:.4e} | {c[k] / tiles:.2f} |")
    util = ""
    if "GRBM_GUI_ACTIVE" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        # GRBM_GUI_ACTIVE is reported once per XCD: the busy cycles of one
        # dispatch are its mean over the 8 XCDs
        busy = c["GRBM_GUI_ACTIVE"] / 8
        util = (f"\nMFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x {SIMDS} SIMDs) "
                f"= {c['SQ_VALU_MFMA_BUSY_CYCLES']:.4e} / ({busy:.4e} x {SIMDS}) = "
                f"**{100 * c['SQ_VALU_MFMA_BUSY_CYCLES'] / (busy * SIMDS):.1f} %** of the cycles the "
                f"GPU was busy with the dispatch.\n")
        dur = mean_duration_ns(dirs[0], kernel)
        if dur:
            util += (f"\nEffective engine clock = (GRBM_GUI_ACTIVE / 8 XCDs) / mean dispatch duration "
                     f"= {busy:.4e} / {dur:.4e} ns = **{busy / dur * 1e3:.0f} MHz** (peak 2400).\n")
    return (f"## Counters (rocprofv3 --pmc, two passes)\n\n{per}\n\n```\n{command}\n```\n\n"
            + "\n".join(lines) + "\n" + util)


def gemm_ceiling(sizes=(8192, 16384)):
    """Vendor GEMM throughput on this GPU (hipBLASLt through torch): the
    practical MFMA ceiling that a dense contraction reaches here, on random
    and on all-zero operands (the difference is data-dependent power)."""
    import torch
    dev = "cuda"

    def rate(fn, flops, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return flops / (e0.elapsed_time(e1) / n * 1e-3) / 1e12

    rows = []
    for m in sizes:
        a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
        b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
        z = torch.zeros_like(a)
        one = torch.tensor(1.0, device=dev)
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.to(torch.float8_e4m3fn).t().contiguous().t()
        rows.append((m, rate(lambda: a @ b, 2 * m ** 3), rate(lambda: z @ z, 2 * m ** 3),
                     rate(lambda: torch._scaled_mm(a8, b8, one, one, out_dtype=torch.bfloat16),
                          2 * m ** 3)))
        del a, b, z, a8, b8
    return rows


def algorithmic_bytes(workload):
    from workloads import get_config
    cfg = get_config(workload)
    n = cfg.B * cfg.S * cfg.H * cfg.D
    elem = 1 if cfg.dtype == "fp8" else 2
    return cfg, 3 * n * elem + 16 * cfg.S, 2 * n


BWD_SOURCES = ["klein_device.hpp", "attn_bwd.hip"]
BWD_KERNELS = (("prep", "attn_bwd_prep_kernel<128>"), ("scale", "attn_bwd_scale_kernel"),
               ("dK/dV", "attn_bwd_dkdv_kernel<128>"), ("dQ", "attn_bwd_dq_kernel<128>"))


def backward_markdown(stats_dir, workloads, command, last=None):
    """Per-kernel durations of the backward's kernels (their last `last`
    dispatches, or all), one table per workload; a workload's dispatches are
    told apart by their grids (prep: one work-item per 8 channels of B S H D,
    rounded up to 256; scale: B H workgroups of 256; dK/dV and dQ: B H
    ceil(S / 256) workgroups of 512)."""
    from workloads import get_config
    rows = _rows(_find(stats_dir, "kernel_trace.csv"))
    size = lambda r: int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
    md = [f"# attn_bwd kernels\n\nThe backward's kernels (prep, scale, dK/dV, dQ) at D = 128; sources "
          f"hash {sources_hash(BWD_SOURCES)} ({', '.join(BWD_SOURCES)}).\n\nCommand (run from "
          f"/tmp with TMPDIR=/tmp; R = repository root):\n\n```\n{command}\n```\n"]
    for w in workloads:
        cfg = get_config(w)
        grids = {"prep": -(-cfg.B * cfg.S * cfg.H * cfg.D // 8 // 256) * 256,
                 "scale": cfg.B * cfg.H * 256,
                 "dK/dV": cfg.B * cfg.H * -(-cfg.S // 256) * 512,
                 "dQ": cfg.B * cfg.H * -(-cfg.S // 256) * 512}
        durs = {label: [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in rows
                        if name in r["Kernel_Name"] and size(r) == grids[label]]
                for label, name in BWD_KERNELS}
        if last:
            durs = {k: v[-last:] for k, v in durs.items()}
        if not all(durs.values()):
            continue
        mean = {k: sum(v) / len(v) for k, v in durs.items()}
        unit = cfg.B * cfg.H * cfg.S * cfg.S * cfg.D
        total = sum(mean.values())
        md.append(f"\n## {cfg.name}: B={cfg.B}, S={cfg.S}, H={cfg.H}, D={cfg.D}\n\n"
                  f"| kernel | dispatches | mean ms | MFMA flops (x B H S^2 D) | TFLOP/s on them |\n"
                  f"|---|---|---|---|---|\n")
        for label, units in (("prep", 0), ("scale", 0), ("dK/dV", 8), ("dQ", 6)):
            rate = f"{units * unit / (mean[label] * 1e-3) / 1e12:.1f}" if units else "-"
            md.append(f"| {label} | {len(durs[label])} | {mean[label]:.4f} | {units or '-'} | "
                      f"{rate} |\n")
        md.append(f"| the backward (sum of the means) | | {total:.4f} | 10 (algorithmic) | "
                  f"{10 * unit / (total * 1e-3) / 1e12:.1f} |\n")
        # dQ runs beside dK/dV on a second stream, so a call's time is its
        # span: the i-th prep's start to the end of the i-th call's last kernel
        span = {label: [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
                        if name in r["Kernel_Name"] and size(r) == grids[label]]
                for label, name in BWD_KERNELS}
        if last:
            span = {k: v[-last:] for k, v in span.items()}
        n = min(len(v) for v in span.values())
        spans = [(max(span[k][i][1] for k in span) - min(span[k][i][0] for k in span)) / 1e6
                 for i in range(n)]
        if spans:
            ms = sum(spans) / len(spans)
            md.append(f"| the backward per call (first start to last end; dK/dV and dQ overlap) | "
                      f"{len(spans)} | {ms:.4f} | 10 (algorithmic) | "
                      f"{10 * unit / (ms * 1e-3) / 1e12:.1f} |\n")
    return "".join(md)


def drive(what, steps):
    """Calls to trace or count on their own (run under rocprofv3): 'qkv' =
    the QKV projection with its RoPE epilogue at the 2048x2048 CFG shape
    (x [2, 16896, 3072] -> q', k', v), bf16 then FP8 operands, each followed
    by the vendor GEMM on the same operands (torch.addmm, torch._scaled_mm);
    'sparse' = the block-sparse attention with keys rotated once, on the
    bench workloads with their seeded masks (bf16 workload 4, fp8 workload
    5); 'bwd' = the attention backward at the 2048x2048 CFG shape (the
    forward with lse once, then the backward calls).  `steps` calls of each
    after ten warm-up calls."""
    import sys
    import torch
    sys.path.insert(0, ROOT)
    import joint_attention_rope_amd as kl
    from workloads import get_config, make_block_mask, make_inputs
    dev = "cuda:0"

    def run(fn):
        # ten warm-up calls: the clock ramps up over the first calls after
        # the idle input preparation
        for _ in range(10 + steps):
            fn()
        torch.cuda.synchronize()

    if what == "qkv":
        c = get_config(4)
        C = c.H * c.D
        g = torch.Generator(device=dev).manual_seed(404)
        xx = torch.randn(c.B, c.S, C, device=dev, generator=g).to(torch.bfloat16)
        ww = (torch.randn(3 * C, C, device=dev, generator=g) / C ** 0.5).to(torch.bfloat16)
        bb = (torch.randn(3 * C, device=dev, generator=g) * 0.1).to(torch.bfloat16)
        pp = torch.from_numpy(make_inputs(get_config(4, B=1, H=1)).pos).to(dev)
        qo = torch.empty(c.B, c.S, c.H, c.D, dtype=torch.float16, device=dev)
        ko = torch.empty_like(qo)
        vo = torch.empty(c.B, c.S, c.H, c.D, dtype=torch.bfloat16, device=dev)
        yy = torch.empty(c.B * c.S, 3 * C, dtype=torch.bfloat16, device=dev)
        run(lambda: kl.klein_qkv_rope4d_proj(xx, ww, bb, pp, qo, ko, vo))
        run(lambda: torch.addmm(bb, xx.view(-1, C), ww.t(), out=yy))
        sx = float(xx.float().abs().max()) / 448.0
        sw = float(ww.float().abs().max()) / 448.0
        x8 = (xx.float() / sx).to(torch.float8_e4m3fn)
        w8 = (ww.float() / sw).to(torch.float8_e4m3fn)
        run(lambda: kl.klein_qkv_rope4d_proj(x8.view(torch.uint8), w8.view(torch.uint8), bb, pp,
                                             qo, ko, vo, descales=(sx, sw)))
        one = torch.ones((), device=dev)
        run(lambda: torch._scaled_mm(x8.view(-1, C), w8.t(), scale_a=one * sx, scale_b=one * sw,
                                     out_dtype=torch.bfloat16))
    elif what == "sparse":
        for cid in (4, 5):
            c = get_config(cid)
            xi = make_inputs(c)
            if xi.descale is None:
                conv = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
            else:
                conv = lambda a: torch.from_numpy(a).to(dev)
            q, k, v = conv(xi.q), conv(xi.k), conv(xi.v)
            p = torch.from_numpy(xi.pos).to(dev)
            o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
            m = torch.from_numpy(make_block_mask(c.B, c.H, c.S, c.text, 0.3, seed=cid)).to(dev)
            dt = kl.KLEIN_DTYPE_BF16 if xi.descale is None else kl.KLEIN_DTYPE_FP8_E4M3
            w = torch.empty(kl.klein_attn_workspace_size(c.B, c.S, c.H, c.D, dt),
                            dtype=torch.uint8, device=dev)
            run(lambda: kl.klein_rope4d_attn_fwd_blocksparse(
                q, k, v, p, o, m, descales=xi.descale or (1.0, 1.0, 1.0), workspace=w))
    elif what == "bwd":
        c = get_config(4)
        xi = make_inputs(c)
        q, k, v = (torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)
                   for a in (xi.q, xi.k, xi.v))
        p = torch.from_numpy(xi.pos).to(dev)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(c.B, c.H, c.S, dtype=torch.float32, device=dev)
        kl.klein_rope4d_attn_fwd_lse(q, k, v, p, o, lse)
        g = torch.Generator(device=dev).manual_seed(505)
        do = torch.randn(q.shape, device=dev, generator=g).to(torch.bfloat16)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        w = torch.empty(kl.klein_attn_bwd_workspace_size(c.B, c.S, c.H, c.D), dtype=torch.uint8,
                        device=dev)
        run(lambda: kl.klein_rope4d_attn_bwd(q, k, v, p, o, do, lse, dq, dk, dv, w))
    else:
        raise ValueError(what)


def kernels_markdown(name, stats_dir, kernels, command, note="", last=None):
    """Mean duration of each listed kernel (label=name-substring; its last
    `last` dispatches, or all) from a kernel trace, with TFLOP/s when a flop
    count is given as label=substring=flops."""
    rows = _rows(_find(stats_dir, "kernel_trace.csv"))
    md = [f"# {name}\n\n{note}\n\nCommand (run from /tmp with TMPDIR=/tmp; R = repository "
          f"root):\n\n```\n{command}\n```\n\n| kernel | dispatches | mean ms | min ms | "
          f"TFLOP/s at the mean |\n|---|---|---|---|---|\n"]
    for spec in kernels:
        parts = spec.split("=")
        label, pat = parts[0], parts[1]
        flops = float(parts[2]) if len(parts) > 2 else None
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in rows
             if pat in r["Kernel_Name"]]
        if last:
            d = d[-last:]
        if not d:
            md.append(f"| {label} | 0 | - | - | - |\n")
            continue
        mean = sum(d) / len(d)
        rate = f"{flops / (mean * 1e-3) / 1e12:.1f}" if flops else "-"
        md.append(f"| {label} (`{pat}`) | {len(d)} | {mean:.4f} | {min(d):.4f} | {rate} |\n")
    return "".join(md)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--call", choices=sorted(CALLS),
                    help="the profiled call (attention kernel + its merge, if any)")
    ap.add_argument("--name")
    ap.add_argument("--workload", type=int)
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--steps", type=int, help="timed calls (after the warm-up calls)")
    ap.add_argument("--warmup", type=int, default=0,
                    help="warm-up calls of the profiled entry point before the timed ones")
    ap.add_argument("--copy-mib", type=int)
    ap.add_argument("--command")
    ap.add_argument("--bench-ms", type=float, default=None,
                    help="ms per call that bench.py printed in the stats run")
    ap.add_argument("--counters", nargs=2, metavar=("PASS1", "PASS2"),
                    help="write profiles/<name>_counters.md from two --pmc runs instead")
    ap.add_argument("--backward", metavar="STATS",
                    help="write profiles/attn_bwd_kernels.md from a kernel trace of "
                         "--drive bwd (the backward at the 2048x2048 CFG shape; with --steps, "
                         "its last dispatches)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="measure vendor GEMM throughput on the GPU and print a markdown table")
    ap.add_argument("--drive", choices=["qkv", "sparse", "bwd"],
                    help="run the QKV projection, the block-sparse attention or the backward "
                         "--steps times after ten warm-up calls (for rocprofv3)")
    ap.add_argument("--kernels", nargs="+", metavar="LABEL=PATTERN[=FLOPS]",
                    help="write profiles/<name>.md: mean duration of each kernel in --stats")
    ap.add_argument("--note", default="")
    ap.add_argument("--kernel-pattern", help="with --counters: any kernel, by name substring")
    ap.add_argument("--sources", nargs="+", default=[], help="with --kernel-pattern: its sources")
    ap.add_argument("--units", type=int, help="with --kernel-pattern: work units per dispatch")
    ap.add_argument("--unit-name", default="")
    args = ap.parse_args()
    if args.drive:
        drive(args.drive, args.steps or 5)
        return
    if args.kernels:
        md = kernels_markdown(args.name, args.stats, args.kernels, args.command, args.note,
                              last=args.steps)
        with open(os.path.join(ROOT, "profiles", f"{args.name}.md"), "w") as f:
            f.write(md)
        print(md)
        return
    if args.backward:
        import sys
        sys.path.insert(0, ROOT)
        md = backward_markdown(args.backward, (4,), args.command, last=args.steps)
        with open(os.path.join(ROOT, "profiles", "attn_bwd_kernels.md"), "w") as f:
            f.write(md)
        print(md)
        return
    if args.gemm_ceiling:
        print("| M = N = K | bf16, random | bf16, zeros | fp8 e4m3 (scaled_mm), random |")
        print("|---|---|---|---|")
        for m, r, z, f in gemm_ceiling():
            print(f"| {m} | {r:.0f} TFLOP/s | {z:.0f} TFLOP/s | {f:.0f} TFLOP/s |", flush=True)
        return

    import sys
    sys.path.insert(0, ROOT)
    if args.counters and args.kernel_pattern:
        md = f"# {args.name} counters\n\nKernel `{args.kernel_pattern}`; sources hash " \
             f"{sources_hash(args.sources)} ({', '.join(args.sources)}).\n\n" + \
             counters_markdown(args.kernel_pattern, None, args.counters, args.command,
                               units=args.units, unit_name=args.unit_name)
        with open(os.path.join(ROOT, "profiles", f"{args.name}_counters.md"), "w") as f:
            f.write(md)
        print(md)
        return
    call = CALLS[args.call]
    srcs = call["sources"]
    shash = sources_hash(srcs)
    kinds = "".join(f"`{b}` + " for b in call["before"]) + f"`{call['kernel']}`" + \
        (f" + `{call['merge']}`" if call["merge"] else "")
    if args.counters:
        from workloads import get_config
        md = f"# {args.name} counters\n\nKernel {kinds} (counters of the attention kernel); " \
             f"sources hash {shash} ({', '.join(srcs)}).\n\n" + \
             counters_markdown(call["kernel"], get_config(args.workload), args.counters, args.command)
        with open(os.path.join(ROOT, "profiles", f"{args.name}_counters.md"), "w") as f:
            f.write(md)
        print(md)
        return
    cfg, algo_read, algo_write = algorithmic_bytes(args.workload)
    # the call's dispatches in order: warm-up calls, then the timed ones
    # (later calls of the same kernel, e.g. other workloads, are not counted)
    calls = call_durations_ns(args.stats, args.call)[:args.warmup + args.steps]
    durs = [sum(c) for c in calls]
    timed = calls[args.warmup:]
    avg_all = sum(durs) / len(durs) / 1e6
    avg_timed = sum(sum(c) for c in timed) / len(timed) / 1e6
    avg_rot = sum(c[0] for c in timed) / len(timed) / 1e6
    avg_attn = sum(c[1] for c in timed) / len(timed) / 1e6
    avg_merge = sum(c[2] for c in timed) / len(timed) / 1e6

    copy_bytes = args.copy_mib * (1 << 20)
    cf = list(counter_per_dispatch(args.fetch, COPY_KERNEL, "FETCH_SIZE").values())
    cw = list(counter_per_dispatch(args.write, COPY_KERNEL, "WRITE_SIZE").values())
    f_scale = copy_bytes / (sum(cf) / len(cf) * 1024.0)
    w_scale = copy_bytes / (sum(cw) / len(cw) * 1024.0)
    kf = call_counter(args.fetch, args.call, "FETCH_SIZE")
    kw = call_counter(args.write, args.call, "WRITE_SIZE")
    read_b = sum(kf) / len(kf) * 1024.0 * f_scale
    write_b = sum(kw) / len(kw) * 1024.0 * w_scale
    flops = cfg.flops
    tflops = flops / (avg_timed * 1e-3) / 1e12

    md = f"""# {args.name}

Call of {kinds} on the workload {cfg.name}: B={cfg.B}, S={cfg.S}, H={cfg.H}, D={cfg.D}, {cfg.dtype}.
Sources hash {shash} ({', '.join(srcs)}).

Commands (run from /tmp with TMPDIR=/tmp; R = repository root):

```
{args.command}
```

## Kernel trace (rocprofv3 --kernel-trace --stats)

| quantity | value |
|---|---|
| calls | {len(durs)} |
| average duration per call, all calls | {avg_all:.4f} ms |
| average duration per call, calls {args.warmup + 1}-{args.warmup + args.steps} (the timed calls) | {avg_timed:.4f} ms |
| of which the passes before the kernel ({', '.join(b.split('<')[0] for b in call['before']) or 'none'}) | {avg_rot:.4f} ms |
| of which the attention kernel | {avg_attn:.4f} ms |
| of which the merge kernel | {avg_merge:.4f} ms |
| min / max per call | {min(durs) / 1e6:.4f} / {max(durs) / 1e6:.4f} ms |
| bench.py ms per call, plain run in the same lease | {args.bench_ms if args.bench_ms is not None else 'n/a'} |
| attention flops per call (4 B H S^2 D) | {flops:.4e} |
| TFLOP/s at the timed average | {tflops:.1f} |

## Memory traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)

Calibration: an elementwise fp32 copy of {copy_bytes} bytes read and written.
FETCH_SIZE read {sum(cf) / len(cf):.0f} KiB for it (scale {f_scale:.4f}),
WRITE_SIZE {sum(cw) / len(cw):.0f} KiB (scale {w_scale:.4f}).

| per call | counter (KiB) | scaled bytes | algorithmic bytes | ratio |
|---|---|---|---|---|
| read  | {sum(kf) / len(kf):.0f} | {read_b:.4e} | {algo_read:.4e} | {read_b / algo_read:.2f} |
| write | {sum(kw) / len(kw):.0f} | {write_b:.4e} | {algo_write:.4e} | {write_b / algo_write:.2f} |
| total | | {read_b + write_b:.4e} | {algo_read + algo_write:.4e} | {(read_b + write_b) / (algo_read + algo_write):.2f} |
"""
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{args.name}.md"), "w") as f:
        f.write(md)
    with open(os.path.join(out_dir, f"traffic_{args.name}.json"), "w") as f:
        json.dump({"call": args.call, "sources_hash": shash,
                   "hbm_bytes_per_launch": round(read_b + write_b),
                   "read_bytes": round(read_b), "write_bytes": round(write_b),
                   "algorithmic_bytes": algo_read + algo_write,
                   "avg_ms_timed": round(avg_timed, 4)}, f, indent=1)
    print(md)


if __name__ == "__main__":
    main()
