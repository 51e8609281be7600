"""Build-time properties of the FP8-cache attention kernel that its speed
relies on, checked on the generated gfx950 assembly (hipcc, no GPU needed).

The stage loop issues the next tile's direct global->LDS loads early and only
waits for them at the next barrier.  Memory counters retire in order, so any
scratch (spill) reload inside the loop would wait for those loads too: the
loop must stay free of scratch accesses for every instantiation.  The
score blocks' inline asm names v222..v255 as clobbers and uses them as
fixed scratch; a compiler that cannot honour that fails to build, which the
compile here also catches.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_context_parallelism_amd", "csrc")


def _hipcc():
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def fp8_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from decode_context_parallelism_amd import build
    out = tmp_path_factory.mktemp("asm") / "attention_fp8.s"
    flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"]
    cmd = [hipcc, *flags, "-S", "--cuda-device-only", os.path.join(CSRC, "attention_fp8.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    return out.read_text()


def _kernels(asm):
    """(name, body) of each attention_fp8_kernel instantiation."""
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\S*attention_fp8_kernel\S*):", asm, re.M)]
    assert len(starts) == 8, [n for _, n in starts]   # PartLds x QF8 x P8
    out = []
    for pos, name in starts:
        end = asm.find(".Lfunc_end", pos)   # a kernel has several s_endpgm (early exits)
        out.append((name, asm[pos:end]))
    return out


def _loop_blocks(body, min_depth):
    """Instructions of the basic blocks at loop depth >= min_depth."""
    blocks, cur, depth = [], [], 0
    for line in body.splitlines():
        m = re.match(r"^(\.LBB\S+:|; %bb\.\d+:)(.*)$", line)
        if m:
            if depth >= min_depth:
                blocks.extend(cur)
            d = re.search(r"Depth=(\d+)", m.group(2))
            depth, cur = (int(d.group(1)) if d else 0), []
            continue
        cur.append(line)
    if depth >= min_depth:
        blocks.extend(cur)
    return blocks


def test_stage_loop_is_spill_free(fp8_asm):
    for name, body in _kernels(fp8_asm):
        loop = _loop_blocks(body, 2)
        assert any("v_mfma_scale_f32_32x32x64_f8f6f4" in l for l in loop), name   # the stage loop was found
        spills = [l.strip() for l in loop if re.search(r"\bscratch_(load|store)", l)]
        assert not spills, (name, spills[:4])


def test_loop_keeps_output_accumulator_in_agprs(fp8_asm):
    # the 16 output tiles stay in AGPRs across the loop: no wholesale copies out
    for name, body in _kernels(fp8_asm):
        loop = _loop_blocks(body, 2)
        reads = sum(1 for l in loop if "v_accvgpr_read_b32" in l)
        # only the rare rescale path reads them (256 reads, once)
        assert reads <= 256, (name, reads)


def test_score_blocks_match_their_generator():
    # the asm score blocks are written by gen_score_blocks.py; the source must
    # be what the generator writes
    import sys
    gen = os.path.join(CSRC, "gen_score_blocks.py")
    res = subprocess.run([sys.executable, gen, "--check"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr


def test_asm_blocks_assemble(tmp_path):
    # the -S output above is not run through the assembler's operand checks
    # (constant-bus limits, operand kinds); an object build is
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from decode_context_parallelism_amd import build
    flags = [f for f in build.HIPCC_FLAGS if f != "-fPIC"]
    cmd = [hipcc, *flags, "-c", "--cuda-device-only", os.path.join(CSRC, "attention_fp8.hip"),
           "-o", str(tmp_path / "attention_fp8.o")]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
