"""The one-wave-per-SIMD GEMM (csrc/kernels_gemm_w4.hip) issues its MFMAs
as inline asm, so the compiler cannot insert the wait states between an
MFMA writing an accumulator register and another instruction touching it.
The kernel is written so that no such instruction exists between the first
MFMA and the fence of nops after the K loop; this test compiles the source
for gfx950 and checks that in the generated code: for every instantiation,
one K loop holding all 128 MFMAs (two K-steps of 64), no other
instruction naming an AGPR from the first MFMA to the fence, and the
accumulators' zeroing at least 16 instructions before the first MFMA."""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
CSRC = os.path.join(ROOT, "heterogeneous_embed_decode_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp()
    try:
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}",
               f"-I{CSRC}", "--cuda-device-only", "-S", os.path.join(CSRC, "kernels_gemm_w4.hip"),
               "-o", os.path.join(d, "w4.s")]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        return open(os.path.join(d, "w4.s")).read().split("\n")
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_no_accumulator_access_inside_the_mfma_region():
    src = _asm()
    names = [l.split(":")[0] for l in src if re.match(r"^_Z\S*gemm_w4_kernel\S*:", l)]
    assert len(names) == 2, names   # SwiGLU and plain bf16
    for name in names:
        s = next(i for i, l in enumerate(src) if l.startswith(name + ":"))
        e = next(i for i in range(s + 1, len(src)) if src[i].startswith(".Lfunc_end"))
        body = [l.strip() for l in src[s:e]]
        code = [l for l in body if l and not l.startswith((";", "."))]
        mfma = [i for i, l in enumerate(code) if l.startswith("v_mfma")]
        fence = next(i for i, l in enumerate(code) if l.startswith("s_nop 15"))
        assert len(mfma) == 128 and mfma[-1] < fence, name
        agpr = [l for i, l in enumerate(code) if mfma[0] <= i < fence and not l.startswith("v_mfma")
                and re.search(r"\ba\d|\ba\[", l)]
        assert not agpr, (name, agpr[:4])
        # the zeroing writes of the accumulators lie well before the first
        # MFMA reads them (the hardware needs a few wait states there)
        zero = [i for i, l in enumerate(code[:mfma[0]]) if re.search(r"\ba\d|\ba\[", l)]
        assert zero and mfma[0] - zero[-1] >= 16, (name, mfma[0] - zero[-1] if zero else None)
        heads = [i for i, l in enumerate(body) if "Loop Header" in l]
        assert len(heads) == 1, name
        end = next(i for i in range(heads[0], len(body)) if body[i].startswith("s_cbranch"))
        assert sum(1 for l in body[heads[0]:end] if l.startswith("v_mfma")) == 128, name
