"""Code-generation guard (CPU, no GPU): no instruction other than another
MFMA may write a register that an MFMA still reads as its accumulator input.

An MFMA whose accumulator input (srcC) is a different register block from its
destination keeps reading that block while it runs (a 32x32 f32 MFMA runs 16
passes). The compiler has produced, for a two-pass float32 forward, the first
P V product of a pass with srcC = a rescaled copy of the zeroed accumulator and
then overwritten that copy with an LDS load 0 issue slots later and with VALU
results 1-15 slots later, with no wait states in between; the output then had
wrong values in exactly the accumulator registers those writes hit. This test
compiles every kernel source for gfx950 with the library's own flags and scans
the assembly: after an MFMA with srcC != dst, no VALU, LDS or memory
instruction may write a srcC register within 20 issue slots of straight-line
code (s_nop n counts n + 1). MFMA-to-MFMA overlaps are ordered by the matrix
pipeline and allowed.
"""
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

from attention_fa2_fwd_02_amd import build as hip_build

STORES = ("ds_write", "buffer_store", "global_store", "flat_store", "scratch_store")
WINDOW = 20


def _regs(tok):
    tok = tok.strip()
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _written(op, args):
    """VGPRs an instruction writes (its first operand, except for stores,
    compares and scalar instructions, which write no VGPR)."""
    if not args or op.startswith(STORES) or op.startswith(("s_", "v_cmp")):
        return set()
    return _regs(args[0])


def srcc_war(lines):
    """(distance, mfma, writer) for every non-MFMA write into the srcC block of
    an earlier MFMA with srcC != dst, within WINDOW issue slots."""
    live, hits = [], []
    for raw in lines:
        line = raw.split(";")[0].strip()
        if not line or line.startswith("."):
            continue
        if line.endswith(":") or line.startswith(("s_cbranch", "s_branch", "s_setpc")):
            live = []
            continue
        op = line.split()[0]
        args = line[len(op):].split(",") if len(line) > len(op) else []
        slots = int(line.split()[1]) + 1 if op == "s_nop" else 1
        if op.startswith("v_mfma"):
            live = [(c, age + slots, txt) for c, age, txt in live]
            dst, srcc = _regs(args[0]), _regs(args[3]) if len(args) > 3 else set()
            if srcc and srcc != dst:
                live.append((srcc, 0, line))
            continue
        w = _written(op, args)
        for c, age, txt in live:
            if w & c:
                hits.append((age, txt, line))
        live = [(c, age + slots, txt) for c, age, txt in live if age + slots <= WINDOW]
    return hits


def test_scanner_finds_a_planted_hazard():
    """The scanner itself: a srcC != dst MFMA followed by an LDS load into its
    srcC block is reported; the in-place form and a distant write are not."""
    bad = ["v_mfma_f32_32x32x2_f32 v[18:33], v172, v66, v[34:49]", "ds_read_b128 v[40:43], v170 offset:16"]
    assert [h[0] for h in srcc_war(bad)] == [0]
    in_place = ["v_mfma_f32_32x32x2_f32 v[18:33], v172, v66, v[18:33]", "v_mov_b32_e32 v20, 0"]
    assert srcc_war(in_place) == []
    far = ["v_mfma_f32_32x32x2_f32 v[18:33], v172, v66, v[34:49]", "s_nop 7", "s_nop 7", "s_nop 7",
           "v_mov_b32_e32 v35, 0"]
    assert srcc_war(far) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not Path("/opt/rocm/bin/hipcc").exists(),
                    reason="needs hipcc")
def test_no_write_into_a_running_mfma_accumulator_input(tmp_path):
    hipcc = hip_build._hipcc()
    flags = [f for f in hip_build.HIPCC_FLAGS if f != "-fPIC"]
    sources = sorted(hip_build.CSRC.glob("*.hip"))

    def asm(src):
        out = tmp_path / (src.stem + ".s")
        r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", str(src), "-o", str(out)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return out

    with ThreadPoolExecutor(min(8, len(sources))) as ex:
        files = list(ex.map(asm, sources))
    kernels, bad = 0, []
    for f in files:
        lines = f.read_text().split("\n")
        starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\w+:", l)]
        for s in starts:
            e = next((i for i in range(s, len(lines)) if "s_endpgm" in lines[i]), None)
            if e is None:  # a symbol that is not a kernel body
                continue
            kernels += 1
            for hit in srcc_war(lines[s:e]):
                bad.append((f.name, lines[s].split(":")[0][:80], *hit))
    assert kernels > 100, kernels
    assert not bad, "\n".join(map(str, bad[:10]))
