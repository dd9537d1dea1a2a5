"""The hot loop of the 256x256 and 128x128 bf16 kernels (every operand
layout), compiled for gfx950 here, must
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
using TL = Tile<FAM_BF16, %s, %s, %d, %d, 2, 2, 128, 2, 7>;
template __global__ void gemm_persistent<TL>(KArgs);
}
"""


def mfma_loops(asm: str, per_kt: int):
    """Basic blocks (by label) holding at least one k-tile of MFMAs: the
    unrolled k-loop."""
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
    return [(lab, ls) for lab, ls in blocks if sum("v_mfma" in x for x in ls) >= per_kt]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("a_kc,b_kc", [(True, True), (True, False), (False, True), (False, False)],
                         ids=["tn", "nn", "tt", "nt"])
@pytest.mark.parametrize("bm", [256, 128])
def test_bf16_mainloop_has_no_spills_or_drains(bm, a_kc, b_kc):
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "k.hip")
        with open(src, "w") as fh:
            fh.write(SRC % (str(a_kc).lower(), str(b_kc).lower(), bm, bm))
        cmd = [HIPCC, "-x", "hip", "-c", src, "-o", os.path.join(d, "k.o"), "-O3", "-std=c++17",
               "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--save-temps"]
        r = subprocess.run(cmd, cwd=d, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        asm_files = [f for f in os.listdir(d) if f.endswith(".s") and "gfx950" in f]
        assert asm_files, os.listdir(d)
        with open(os.path.join(d, asm_files[0])) as fh:
            asm = fh.read()
    # per wave and k-tile (64 k): (bm/64)^2 MFMAs per substep, 4 substeps;
    # each thread loads (and writes to LDS) bm/16 16-byte chunks
    f = bm // 64
    per_kt = 4 * f * f
    loops = mfma_loops(asm, per_kt)
    assert loops, "no MFMA loop found"
    for lab, ls in loops:
        body = "\n".join(x for x in ls if not x.strip().startswith(";"))
        n_mfma = body.count("v_mfma_f32_32x32x16_bf16")
        assert n_mfma % per_kt == 0, (lab, n_mfma)
        kts = n_mfma // per_kt
        assert "scratch_" not in body, f"{lab}: scratch access in the MFMA loop"
        assert "vmcnt(0)" not in body, f"{lab}: vmcnt(0) drain in the MFMA loop"
        assert body.count("buffer_load_dwordx4") == (bm // 16) * kts, lab
        assert body.count("ds_write_b128") == (bm // 16) * kts, lab
        # fragment reads: 16 bytes per K-contiguous fragment, two transposing
        # 8-byte reads per M/N-contiguous one (f + f fragments per substep)
        n_tr = (0 if a_kc else 2 * f) + (0 if b_kc else 2 * f)
        assert body.count("ds_read_b64_tr_b16") == n_tr * 4 * kts, lab
