"""Turn rocprofv3 CSV output into the committed profile summaries.

Three rocprofv3 runs of bench.py feed it (each with --copy-calibration, which
adds an elementwise fp32 copy of known size):

  rocprofv3 --kernel-trace --stats --output-format csv -d STATS -o run -- python3 bench.py ...
  rocprofv3 --pmc FETCH_SIZE      --output-format csv -d FETCH -o run -- python3 bench.py ...
  rocprofv3 --pmc WRITE_SIZE      --output-format csv -d WRITE -o run -- python3 bench.py ...

FETCH_SIZE / WRITE_SIZE (KiB per dispatch, L2-to-memory traffic) are scaled by
known_bytes / counter for the copy kernel, then reported per launch of the
attention kernel next to its algorithmic bytes.

  python -m joint_attention_rope_amd.profiling --kernel attn_fwd_bf16_kernel \
      --name attn_fwd_bf16_2048px_t2i_cfg --workload 4 --stats STATS --fetch FETCH \
      --write WRITE --steps 5 --copy-mib 1024 --command "..."
"""

import argparse
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL = "MulFunctor"

KERNEL_SOURCES = {
    "attn_fwd_bf16_kernel": ["klein_device.hpp", "attn_fwd_bf16.hip"],
    "attn_fwd_fp8_kernel": ["klein_device.hpp", "attn_fwd_fp8.hip"],
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


def kernel_durations_ns(stats_dir, kernel):
    rows = _rows(_find(stats_dir, "kernel_trace.csv"))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in rows if kernel in r["Kernel_Name"]]


def counter_per_dispatch(pmc_dir, kernel, counter):
    rows = _rows(_find(pmc_dir, "counter_collection.csv"))
    return [float(r["Counter_Value"]) for r in rows
            if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter]


def algorithmic_bytes(workload):
    from workloads import get_config
    cfg = get_config(workload)
    n = cfg.B * cfg.S * cfg.H * cfg.D
    elem = 1 if cfg.dtype == "fp8" else 2
    return cfg, 3 * n * elem + 16 * cfg.S, 2 * n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--name", required=True)
    ap.add_argument("--workload", type=int, required=True)
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--steps", type=int, required=True, help="timed calls (last N dispatches)")
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--bench-ms", type=float, default=None,
                    help="ms per call that bench.py printed in the stats run")
    args = ap.parse_args()

    import sys
    sys.path.insert(0, ROOT)
    cfg, algo_read, algo_write = algorithmic_bytes(args.workload)
    durs = kernel_durations_ns(args.stats, args.kernel)
    timed = durs[-args.steps:]
    avg_all = sum(durs) / len(durs) / 1e6
    avg_timed = sum(timed) / len(timed) / 1e6

    copy_bytes = args.copy_mib * (1 << 20)
    cf = counter_per_dispatch(args.fetch, COPY_KERNEL, "FETCH_SIZE")
    cw = counter_per_dispatch(args.write, COPY_KERNEL, "WRITE_SIZE")
    f_scale = copy_bytes / (sum(cf) / len(cf) * 1024.0)
    w_scale = copy_bytes / (sum(cw) / len(cw) * 1024.0)
    kf = counter_per_dispatch(args.fetch, args.kernel, "FETCH_SIZE")
    kw = counter_per_dispatch(args.write, args.kernel, "WRITE_SIZE")
    read_b = sum(kf) / len(kf) * 1024.0 * f_scale
    write_b = sum(kw) / len(kw) * 1024.0 * w_scale
    flops = cfg.flops
    tflops = flops / (avg_timed * 1e-3) / 1e12
    srcs = KERNEL_SOURCES[args.kernel]
    shash = sources_hash(srcs)

    md = f"""# {args.name}

Kernel `{args.kernel}` on the workload {cfg.name}: B={cfg.B}, S={cfg.S}, H={cfg.H}, D={cfg.D}, {cfg.dtype}.
Kernel sources hash {shash} ({', '.join(srcs)}).

Commands (run from /tmp with TMPDIR=/tmp; R = repository root):

```
{args.command}
```

## Kernel trace (rocprofv3 --kernel-trace --stats)

| quantity | value |
|---|---|
| dispatches of the kernel | {len(durs)} |
| average duration, all dispatches | {avg_all:.4f} ms |
| average duration, last {args.steps} (the timed calls) | {avg_timed:.4f} ms |
| min / max | {min(durs) / 1e6:.4f} / {max(durs) / 1e6:.4f} ms |
| bench.py ms per call in the same run | {args.bench_ms if args.bench_ms is not None else 'n/a'} |
| attention flops per launch (4 B H S^2 D) | {flops:.4e} |
| TFLOP/s at the timed average | {tflops:.1f} |

## Memory traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)

Calibration: an elementwise fp32 copy of {copy_bytes} bytes read and written.
FETCH_SIZE read {sum(cf) / len(cf):.0f} KiB for it (scale {f_scale:.4f}),
WRITE_SIZE {sum(cw) / len(cw):.0f} KiB (scale {w_scale:.4f}).

| per launch | counter (KiB) | scaled bytes | algorithmic bytes | ratio |
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
        json.dump({"kernel": args.kernel, "sources_hash": shash,
                   "hbm_bytes_per_launch": round(read_b + write_b),
                   "read_bytes": round(read_b), "write_bytes": round(write_b),
                   "algorithmic_bytes": algo_read + algo_write,
                   "avg_ms_timed": round(avg_timed, 4)}, f, indent=1)
    print(md)


if __name__ == "__main__":
    main()
