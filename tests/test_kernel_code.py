"""Generated code of the direct-to-LDS kernels (no GPU): their K loops must
hold no vector ALU instruction between the MFMAs.

On gfx950 one vector ALU instruction between two dependent
v_mfma_f32_32x32x2_f32 stalls the second for most of an MFMA's duration,
and these kernels read their LDS operands with inline-asm loads whose
results arrive later (waited for with explicit s_waitcnt): a register copy
the compiler might insert between such a load and its wait would read the
value too early.  Both show up as vector ALU instructions in the loop blocks
that carry the MFMAs, which this test compiles the source for gfx950 and
looks for."""
import os
import re
import shutil
import subprocess

import pytest

from fp32_sgemm_f32_amd import build

SRC = os.path.join(build.CSRC, "gemm_mfma_dl.hip")


def _hipcc_available():
    return os.path.exists(build.hipcc())


@pytest.fixture(scope="module")
def dl_asm(tmp_path_factory):
    if not _hipcc_available():
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("asm") / "dl.s")
    cmd = [build.hipcc(), *[f for f in build.COMMON if f not in ("-fPIC", "-fvisibility=hidden")],
           "-x", "hip", "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def kernels(asm):
    """name -> list of (block label, instructions) for each DL kernel."""
    lines = asm.split("\n")
    out = {}
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\w*sgemm_mfma_dl_kernel\w*):", lines[i])
        if not m:
            i += 1
            continue
        name = m.group(1)
        blocks, cur = [], ("entry", [])
        i += 1
        while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
            ln = lines[i]
            if re.match(r"^\.LBB\w+:", ln):
                blocks.append(cur)
                cur = (ln, [])
            elif ln.startswith("\t") and not ln.strip().startswith((";", ".")):
                cur[1].append(ln.strip())
            i += 1
        blocks.append(cur)
        out[name] = blocks
    return out


def test_every_configuration_is_compiled(dl_asm):
    ks = kernels(dl_asm)
    # 9 whole-tile configurations (A M x K, B K x N), the 4 configurations of
    # the automatic choice in the 3 other storage orders and with edge
    # masking in all 4, each with and without Stream-K.
    assert len(ks) == 2 * (9 + 4 * 3 + 4 * 4)


def is_edge(name):
    # MfmaDlCore<..., EDGE, TA, TB>: the three booleans close the argument list.
    m = re.search(r"ELb([01])ELb[01]ELb[01]EE", name)
    assert m, name
    return m.group(1) == "1"


def test_mfma_loops_hold_no_vector_alu(dl_asm):
    """Whole-tile kernels: no vector ALU instruction at all in a loop block
    that carries MFMAs.  Edge-masking kernels: only the once-per-tile switch
    to the K-tail source offsets (v_mov_b32 of offsets, in the block that
    issues the tail chunk's loads) and v_readfirstlane_b32 (scalar
    bookkeeping)."""
    bad = []
    checked = 0
    for name, blocks in kernels(dl_asm).items():
        allowed = ("v_mfma", "v_nop") + (("v_mov_b32", "v_readfirstlane_b32") if is_edge(name) else ())
        for label, ins in blocks:
            if "Loop" not in label or not any(x.startswith("v_mfma") for x in ins):
                continue
            checked += 1
            valu = [x for x in ins if x.startswith("v_") and not x.startswith(allowed)]
            if valu:
                bad.append((name[:90], label.split(":")[0], valu[:4]))
    assert checked > 100
    assert not bad, "vector ALU in MFMA loop blocks: " + repr(bad[:6])


def test_no_kernel_spills_to_scratch(dl_asm):
    """Every direct-to-LDS kernel, split (Stream-K) instances included, keeps
    its state in registers: a private segment would mean spills to scratch
    memory."""
    descriptors = re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", dl_asm, re.S)
    assert len(descriptors) == 2 * (9 + 4 * 3 + 4 * 4)
    for name, body in descriptors:
        m = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body)
        assert m and m.group(1) == "0", f"{name}: private segment {m and m.group(1)}"
