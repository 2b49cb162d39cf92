"""Register and scratch budget of the gfx950 kernels, read from the compiler's code-object metadata
(device-only assembly, the library's own flags).  Runs on the CPU: hipcc cross-compiles.

Every kernel must be free of scratch (no private segment, no spilled vector registers; scalar
registers spill to lanes of a vector register, not to memory) and of out-of-line calls (a call
makes the kernel's register count the callee's plus what is live across the call, and needs a
stack in scratch).  The streaming kernel is launched with 8 waves per SIMD in mind, so it must
stay within 64 VGPRs: above that the chip fits fewer of its workgroups and the row reads lose
the latency hiding they rely on.
"""

import os
import re
import shutil
import subprocess

import pytest

from draft_verification_04_amd import build as B

HIP_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]
DEVICE_FLAGS = [f for f in B.FLAGS if f not in ("-fPIC", "-shared")] + ["--cuda-device-only", "-S"]


def _kernels(asm):
    meta = asm[asm.index("amdhsa.kernels:"):]
    out = {}
    for block in re.split(r"\n  - ", meta):
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        out[name.group(1)] = {k: int(re.search(r"\." + k + r":\s+(\d+)", block).group(1))
                              for k in ("private_segment_fixed_size", "vgpr_count", "vgpr_spill_count",
                                        "sgpr_spill_count")}
    return out


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not found")
    d = tmp_path_factory.mktemp("asm")
    procs = {}
    for s in HIP_SOURCES:
        out = str(d / (s + ".s"))
        cmd = [B.HIPCC] + DEVICE_FLAGS + ["-I", B.INCLUDE, "-I", B.CSRC, os.path.join(B.CSRC, s), "-o", out]
        procs[s] = (subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True), out)
    asm = {}
    for s, (p, out) in procs.items():
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{s}: {err[-2000:]}"
        with open(out) as f:
            asm[s] = f.read()
    return asm


def test_no_scratch_and_no_calls(assembly):
    seen = 0
    for src, asm in assembly.items():
        assert "s_swappc_b64" not in asm, f"{src}: a device function was left out of line"
        for name, r in _kernels(asm).items():
            seen += 1
            assert r["private_segment_fixed_size"] == 0, (src, name, r)
            assert r["vgpr_spill_count"] == 0, (src, name, r)
    assert seen >= 20


def test_streaming_kernel_fits_eight_waves_per_simd(assembly):
    ks = {n: r for n, r in _kernels(assembly["verify.hip"]).items() if "stream_kernel" in n}
    assert len(ks) == 4            # bf16 and fp32 rows, calls with and without top-k
    for name, r in ks.items():
        assert r["vgpr_count"] <= 64, (name, r)
