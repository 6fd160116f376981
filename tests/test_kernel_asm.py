"""The direct-to-LDS loads of the three-wave prefill kernel are inline
assembly that sets M0 (the LDS destination) without the compiler knowing.
That is sound only while the compiler itself uses M0 nowhere in that kernel.
This test compiles the kernel source to gfx950 assembly (with the library's
own flags) and checks that invariant, so a compiler or source change that
starts using M0 there fails here, on the CPU, not as wrong results."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from compact_decode_attention_amd import build

SRC = os.path.join(build.CSRC, "dms_prefill_mfma.hip")


def kernel_bodies(asm, name_part):
    """{symbol: [instruction lines]} of every function whose symbol contains name_part."""
    out, cur = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = m.group(1) if name_part in m.group(1) else None
            if cur:
                out[cur] = []
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
        if cur:
            t = line.split(";")[0].strip()
            if t and not t.startswith("."):
                out[cur].append(t)
    return out


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
def test_m0_is_only_the_lds_destination_of_the_direct_loads():
    d = tempfile.mkdtemp(prefix="dms_asm_")
    try:
        out = os.path.join(d, "prefill.s")
        flags = [f for f in build.FLAGS if f != "-fPIC"]
        r = subprocess.run([build.HIPCC] + flags + ["--cuda-device-only", "-S", SRC, "-o", out],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        bodies = kernel_bodies(open(out).read(), "prefill_attend3_kernel")
    finally:
        shutil.rmtree(d, ignore_errors=True)
    assert bodies, "no prefill_attend3_kernel in the assembly"
    for sym, ins in bodies.items():
        n_dma = 0
        for j, t in enumerate(ins):
            uses_m0 = re.search(r"\bm0\b", t) is not None
            if " lds" in t and t.startswith("buffer_load"):
                n_dma += 1
                assert ins[j - 1].startswith("s_mov_b32 m0,"), (sym, ins[j - 1], t)
            elif uses_m0:
                # the only other M0 instruction allowed: the write right before a direct load
                assert t.startswith("s_mov_b32 m0,") and j + 1 < len(ins) and " lds" in ins[j + 1], (sym, t)
        assert n_dma > 0, sym
