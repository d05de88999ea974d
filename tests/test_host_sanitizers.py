"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

Every source of the library is rebuilt with the sanitizers on the host side
only (each -fsanitize= follows -Xarch_host; the GPU code is compiled as
usual) and linked into tests/abi_driver.cpp, which walks the argument checks
of every entry point, the split-KV planner over a sweep of shapes, the
workspace-size arithmetic and the status strings, and -- with no GPU
visible -- checks that every call that reaches the device reports
KLEIN_ERR_NO_DEVICE.  A sanitizer finding aborts the test program.  Skipped
when a GPU is visible: the program passes fake pointers, which only a machine
without a device may see past the argument checks.
"""

import os
import subprocess

import pytest
import torch

from joint_attention_rope_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; the driver's fake pointers are for machines without one")
    out = tmp_path_factory.mktemp("san")
    flags = [f for f in libbuild.FLAGS if f not in ("-shared", "-fPIC")]
    objs = []
    sources = [os.path.join(libbuild.CSRC, s) for s in libbuild.SOURCES]
    for path in sources + [os.path.join(HERE, "abi_driver.cpp")]:
        src = os.path.basename(path)
        obj = str(out / (src + ".o"))
        cmd = [libbuild.HIPCC, *flags, *libbuild.KERNEL_FLAGS.get(src, []), "-g", *SAN,
               "-c", "-o", obj, path]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(out / "abi_driver")
    r = subprocess.run([libbuild.HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_abi_paths_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "no device: device-reaching calls report NO_DEVICE" in r.stdout
    assert r.stdout.strip().endswith("ok (0 failed checks)")
