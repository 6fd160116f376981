"""CPU builds with AddressSanitizer and UndefinedBehaviorSanitizer:

* the oracle (gcc, the whole of oracle/dms_oracle.c in one unit with a driver
  that calls every entry point on small and edge-case inputs), and
* the host side of the C ABI (compact_decode_attention_amd/csrc/dms_api.cpp
  built with the sanitizers on the host only, linked with the normally built
  kernel objects, and a driver that walks the configuration checks, the
  argument checks and the error paths without a GPU).

Any out-of-bounds access, leak or undefined operation aborts the driver and
fails the test.  Nothing here touches a GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="4")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-O1", "-g", "-fopenmp", "-std=c11", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    assert "oracle driver ok" in run([exe], env=ENV).stdout


def test_host_abi_under_asan_and_ubsan(tmp_path):
    from compact_decode_attention_amd import build as B
    objs = []
    for src in ("dms_kernels.hip", "dms_prefill_mfma.hip"):  # the kernels as the library builds them
        obj = os.path.join(B.BUILD, src + ".o")
        if not os.path.exists(obj):
            os.makedirs(B.BUILD, exist_ok=True)
            obj = B._compile(src)
        objs.append(obj)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    api, drv, exe = str(tmp_path / "api.o"), str(tmp_path / "drv.o"), str(tmp_path / "abi_san")
    run([B.HIPCC] + flags + san + ["-c", os.path.join(B.CSRC, "dms_api.cpp"), "-o", api])
    run([B.HIPCC] + flags + san + ["-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    run([B.HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
         "-fsanitize=undefined", drv, api] + objs + ["-o", exe])
    assert "abi driver ok" in run([exe], env=ENV).stdout
