"""Build the gfx950 HIP library libklein_attn.so in-tree with hipcc; its race
check copy libklein_attn_sync.so (the attention kernels compiled with
KLEIN_SYNC_CHECK: a full wait and a workgroup barrier at every stage
boundary of their pipeline step, otherwise the same objects), which the GPU
tests compare with the library bit for bit; and the measurement harness
step_clock (the bf16 and fp8 attention kernels and the QKV projection with
per-part cycle counters, linked with the library's other objects; not part
of the library).

Usage: python -m joint_attention_rope_amd.build
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libklein_attn.so")
SYNC_LIB = os.path.join(PKG, "libklein_attn_sync.so")
STEP_CLOCK = os.path.join(PKG, "step_clock")
# the harness replaces these sources (it includes them with the cycle counters
# on; it is compiled with the attention kernels' flags, which leave the
# projection's instructions unchanged)
STEP_CLOCK_REPLACES = ("attn_fwd_bf16.hip", "attn_fwd_fp8.hip", "qkv_rope_proj.hip")
# sources compiled a second time, with KLEIN_SYNC_CHECK, for the race check copy
SYNC_CHECKED = ("attn_fwd_bf16.hip", "attn_fwd_fp8.hip")
SOURCES = ["api.cpp", "attn_fwd_bf16.hip", "attn_fwd_fp8.hip", "qkv_rope_proj.hip", "rope_apply.hip",
           "split_schedule.hip", "attn_bwd.hip", "noalloc.hip"]
# Device kernels never see NaN inputs on purpose (a NaN in q/k/v propagates to
# out either way), so min/max need no IEEE NaN canonicalisation.  The host
# argument checks (std::isfinite on descales) keep full NaN semantics.
KERNEL_FLAGS = {"attn_fwd_bf16.hip": ["-fno-honor-nans"], "attn_fwd_fp8.hip": ["-fno-honor-nans"],
                "attn_bwd.hip": ["-fno-honor-nans"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # never let the compiler form packed fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source (always) and link libklein_attn.so, its race
    check copy and the step_clock harness."""
    tag = "%d" % os.getpid()
    objs = {}
    try:
        cflags = [f for f in FLAGS if f != "-shared"]
        for src in SOURCES + ["step_clock.hip"]:
            obj = os.path.join(CSRC, src + ".o" + tag)
            flags = KERNEL_FLAGS.get(STEP_CLOCK_REPLACES[0] if src == "step_clock.hip" else src, [])
            _run([HIPCC, *cflags, *flags, "-c", "-o", obj, os.path.join(CSRC, src)], verbose)
            objs[src] = obj
        for src in SYNC_CHECKED:
            obj = os.path.join(CSRC, src + ".sync.o" + tag)
            _run([HIPCC, *cflags, *KERNEL_FLAGS.get(src, []), "-DKLEIN_SYNC_CHECK", "-c", "-o", obj,
                  os.path.join(CSRC, src)], verbose)
            objs[src + ".sync"] = obj
        lib_objs = [objs[s] for s in SOURCES]
        tmp = LIB + ".tmp" + tag
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *lib_objs], verbose)
        os.replace(tmp, LIB)
        sync_objs = [objs[s + ".sync"] if s in SYNC_CHECKED else objs[s] for s in SOURCES]
        tmp = SYNC_LIB + ".tmp" + tag
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *sync_objs], verbose)
        os.replace(tmp, SYNC_LIB)
        clock_objs = [objs[s] for s in SOURCES if s not in STEP_CLOCK_REPLACES] + [objs["step_clock.hip"]]
        tmp = STEP_CLOCK + ".tmp" + tag
        _run([HIPCC, "--offload-arch=gfx950", "-o", tmp, *clock_objs], verbose)
        os.replace(tmp, STEP_CLOCK)
    finally:
        for o in objs.values():
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
