"""Sanitizer builds on the CPU: the fp64 oracle (oracle/*.c) and the host side
of the C ABI (argument validation and the host helpers) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (recovery off, so any finding
aborts), each driven by a small C program over its entry points
(tests/sanitize/).  No GPU: the ABI driver only reaches host code.  The
library's sanitized build is cached under tests/sanitize/_build by a hash of
its sources."""
import glob
import hashlib
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(SAN, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_C = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    srcs = [os.path.join(SAN, "oracle_driver.c")] + [os.path.join(ROOT, "oracle", f) for f in
                                                      ("fs_oracle.c", "fsb_oracle.c", "fsb_plain.c")]
    subprocess.check_call(["gcc", "-std=c99", *SAN_C, "-I", os.path.join(ROOT, "oracle"), *srcs,
                           "-lm", "-lpthread", "-o", exe])
    assert "oracle driver: done" in _run(exe)


def _abi_driver():
    srcs = sorted(glob.glob(os.path.join(ROOT, "long_context_fs_amd", "csrc", "*")))
    srcs += [os.path.join(SAN, "abi_driver.c"), os.path.join(ROOT, "include", "fs.h")]
    h = hashlib.sha256()
    for s in srcs:
        h.update(open(s, "rb").read())
    tag = h.hexdigest()[:16]
    exe = os.path.join(BUILD, f"abi_driver_{tag}")
    if os.path.exists(exe):
        return exe
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    procs = []
    for src in sorted(glob.glob(os.path.join(ROOT, "long_context_fs_amd", "csrc", "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src) + f".{tag}.o")
        # host code sanitized; the device code is built as usual
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-c", src, "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE))
        objs.append(obj)
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err.decode()[-3000:]
    drv = os.path.join(BUILD, f"abi_driver.{tag}.o")
    subprocess.check_call(["gcc", "-std=c99", *SAN_C, "-I", os.path.join(ROOT, "include"), "-c",
                           os.path.join(SAN, "abi_driver.c"), "-o", drv])
    tmp = exe + ".tmp"
    subprocess.check_call([HIPCC, "-fsanitize=address,undefined", "-fno-gpu-sanitize", *objs, drv,
                           "-o", tmp])
    os.replace(tmp, exe)
    for o in objs + [drv]:
        os.remove(o)
    for old in glob.glob(os.path.join(BUILD, "abi_driver_*")):   # builds of older sources
        if old != exe:
            os.remove(old)
    return exe


@pytest.mark.slow
def test_abi_host_side_under_asan_ubsan():
    assert "abi driver: done" in _run(_abi_driver())
