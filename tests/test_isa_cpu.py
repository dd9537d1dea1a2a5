"""The hot loop of the 256x256 bf16 TN kernel, compiled for gfx950 here, must
keep every value in registers: no scratch (spill) access and no
`s_waitcnt vmcnt(0)` inside the MFMA loop. A scratch reload there is waited
for with vmcnt, which drains every global load in flight and stalls the
pipeline; the register allocation of this kernel sits close to the 256-VGPR
limit, so an unrelated change to the kernel can tip it over. The AMD assembly
of our own build is read (hipcc --save-temps), nothing else."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_gemm_epilogue_02_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

SRC = """#include "kernels.hpp"
namespace mg {
using TL = Tile<FAM_BF16, true, true, 256, 256, 2, 2, 128, 2, 7>;
template __global__ void gemm_persistent<TL>(KArgs);
}
"""


def mfma_loops(asm: str):
    """Basic blocks (by label) holding at least 32 MFMAs: the unrolled k-loop."""
    blocks, cur, lines = [], None, []
    for line in asm.split("\n"):
        if re.match(r"^\.LBB\d+_\d+:", line):
            if cur is not None:
                blocks.append((cur, lines))
            cur, lines = line.split(":")[0], []
        elif cur is not None:
            lines.append(line)
    if cur is not None:
        blocks.append((cur, lines))
    return [(lab, ls) for lab, ls in blocks if sum("v_mfma" in x for x in ls) >= 32]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_bf16_tn_256_mainloop_has_no_spills_or_drains():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "k.hip")
        with open(src, "w") as fh:
            fh.write(SRC)
        cmd = [HIPCC, "-x", "hip", "-c", src, "-o", os.path.join(d, "k.o"), "-O3", "-std=c++17",
               "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--save-temps"]
        r = subprocess.run(cmd, cwd=d, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        asm_files = [f for f in os.listdir(d) if f.endswith(".s") and "gfx950" in f]
        assert asm_files, os.listdir(d)
        with open(os.path.join(d, asm_files[0])) as fh:
            asm = fh.read()
    loops = mfma_loops(asm)
    assert loops, "no MFMA loop found"
    for lab, ls in loops:
        body = "\n".join(x for x in ls if not x.strip().startswith(";"))
        n_mfma = body.count("v_mfma_f32_32x32x16_bf16")
        assert n_mfma % 64 == 0, (lab, n_mfma)
        assert "scratch_" not in body, f"{lab}: scratch access in the MFMA loop"
        assert "vmcnt(0)" not in body, f"{lab}: vmcnt(0) drain in the MFMA loop"
        # one k-tile per 64 MFMAs: 16 global loads and 16 LDS writes per thread
        assert body.count("buffer_load_dwordx4") == 16 * (n_mfma // 64), lab
        assert body.count("ds_write_b128") == 16 * (n_mfma // 64), lab
