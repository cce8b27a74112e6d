"""Generated code of the direct-to-LDS kernels (no GPU), compiled here for
gfx950:

* correctness: these kernels read their LDS operands with inline-asm loads
  whose results arrive later and are waited for with explicit s_waitcnt; the
  compiler does not know they are in flight and could copy or reuse a
  destination before its wait.  A dataflow pass over every kernel's control
  flow graph (asm_hazards) finds any instruction that names the destination
  of an LDS read not yet covered by an `s_waitcnt lgkmcnt`;
* speed: their K loops hold no vector ALU instruction between the MFMAs (on
  gfx950 one between two dependent v_mfma_f32_32x32x2_f32 stalls the second
  for most of an MFMA's duration), and no kernel spills to scratch."""
import os
import re
import shutil
import subprocess

import pytest

import asm_hazards
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


# 9 whole-tile configurations (A M x K, B K x N), the 4 configurations of
# the automatic choice in the 3 other storage orders and with edge masking in
# all 4, each with and without Stream-K; plus the 4 kernels compiled for one
# product each (whole tiles only).
N_KERNELS = 2 * (9 + 4 * 3 + 4 * 4) + 4


def test_every_configuration_is_compiled(dl_asm):
    ks = kernels(dl_asm)
    assert len(ks) == N_KERNELS
    assert sum("FixedShape" in k for k in ks) == 4


def is_edge(name):
    # MfmaDlCore<..., EDGE, TA, TB>: the three booleans close the argument list.
    m = re.search(r"ELb([01])ELb[01]ELb[01]E(?:E|NS_1\d(?:Runtime|Fixed)Shape)", name)
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
    assert len(descriptors) == N_KERNELS
    for name, body in descriptors:
        m = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body)
        assert m and m.group(1) == "0", f"{name}: private segment {m and m.group(1)}"


def test_no_lds_read_used_before_its_wait(dl_asm):
    """No instruction of any direct-to-LDS kernel (any block, loop or not,
    split or whole-tile instance) reads or writes a register that an LDS
    read is still loading."""
    fs = asm_hazards.functions(dl_asm, r"_Z\w*sgemm_mfma_dl_kernel\w*")
    assert len(fs) == N_KERNELS
    bad = {name[:100]: found[:3] for name, blocks in fs.items() if (found := asm_hazards.hazards(blocks))}
    assert not bad, f"LDS read destinations used before their wait: {bad}"


PLANTED = {
    # name: (instructions, hazards expected)
    "copy_before_wait": (["ds_read_b128 v[0:3], v8", "v_mov_b32 v10, v2"], 1),
    "wait_then_copy": (["ds_read_b128 v[0:3], v8", "s_waitcnt lgkmcnt(0)", "v_mov_b32 v10, v2"], 0),
    # lgkmcnt(1) covers a read only once another LDS operation follows it.
    "partial_wait_too_early": (["ds_read_b32 v0, v8", "s_waitcnt lgkmcnt(1)", "v_add_f32 v1, v0, v0"], 1),
    "partial_wait_covered": (["ds_read_b32 v0, v8", "ds_read_b32 v1, v9", "s_waitcnt lgkmcnt(1)",
                              "v_add_f32 v2, v0, v0"], 0),
    "partial_wait_newest_pending": (["ds_read_b32 v0, v8", "ds_read_b32 v1, v9", "s_waitcnt lgkmcnt(1)",
                                     "v_add_f32 v2, v1, v1"], 1),
    # A scalar load completes out of order: it does not cover the LDS read.
    "scalar_load_does_not_count": (["ds_read_b32 v0, v8", "s_load_dword s0, s[2:3], 0x0",
                                    "s_waitcnt lgkmcnt(1)", "v_mov_b32 v1, v0"], 1),
    "mfma_operand_early": (["ds_read_b128 v[4:7], v8", "v_mfma_f32_32x32x2_f32 a[0:15], v4, v5, a[0:15]"], 1),
    "overwritten_in_flight": (["ds_read_b32 v0, v8", "v_mov_b32 v0, 0"], 1),
    "address_of_next_read": (["ds_read_b32 v0, v8", "ds_read_b32 v1, v0"], 1),
    "raw_immediate_wait": (["ds_read_b32 v0, v8", "s_waitcnt 0xc07f", "v_mov_b32 v1, v0"], 0),
}


@pytest.mark.parametrize("case", list(PLANTED))
def test_hazard_check_on_planted_snippets(case):
    ins, expected = PLANTED[case]
    assert len(asm_hazards.hazards([("entry", ins)])) == expected


def test_hazard_check_follows_branches_and_loops():
    # A read issued at the end of a loop body, used at the loop head before
    # any wait: only the back edge carries it.
    loop = [("entry", ["s_mov_b32 s0, 0"]),
            (".LBB0_1:", ["v_mov_b32 v5, v0", "s_waitcnt lgkmcnt(0)", "ds_read_b32 v0, v8",
                          "s_cmp_lt_i32 s0, 4", "s_cbranch_scc1 .LBB0_1"]),
            ("tail", ["s_endpgm"])]
    assert len(asm_hazards.hazards(loop)) == 1
    # A read pending only on the taken side of a branch.
    branch = [("entry", ["s_cmp_eq_u32 s0, 0", "s_cbranch_scc1 .LBB0_2"]),
              ("u1", ["ds_read_b32 v0, v8", "s_branch .LBB0_3"]),
              (".LBB0_2:", ["s_nop 0"]),
              (".LBB0_3:", ["v_mov_b32 v1, v0", "s_endpgm"])]
    assert len(asm_hazards.hazards(branch)) == 1


def test_hazard_check_catches_a_removed_wait(dl_asm):
    """Deleting one lgkmcnt wait ahead of an MFMA in a real kernel's K loop
    must be caught."""
    fs = asm_hazards.functions(dl_asm, r"_Z\w*sgemm_mfma_dl_kernel\w*")
    name = sorted(fs)[0]
    blocks = fs[name]
    for bi, (label, ins) in enumerate(blocks):
        for k in range(len(ins) - 1):
            if ins[k].startswith("s_waitcnt lgkmcnt") and ins[k + 1].startswith("v_mfma"):
                planted = list(blocks)
                planted[bi] = (label, ins[:k] + ins[k + 1:])
                assert asm_hazards.hazards(planted), (name, label, k)
                return
    pytest.fail("no lgkmcnt wait ahead of an MFMA found")


VALU_SRC = os.path.join(build.CSRC, "gemm_valu.hip")


@pytest.fixture(scope="module")
def valu_asm(tmp_path_factory):
    if not _hipcc_available():
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("asm") / "valu.s")
    cmd = [build.hipcc(), *[f for f in build.COMMON if f not in ("-fPIC", "-fvisibility=hidden")],
           "-x", "hip", "--cuda-device-only", "-S", VALU_SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def test_valu_multiply_adds_avoid_the_accumulator_bank(valu_asm):
    """The vector-ALU cores issue v_fmac_f32 with the row operand a as the
    second source: a multiply-add whose accumulator shares that source's VGPR
    bank (register number mod 4) runs 27% slower on gfx950, and with b there
    the compiler put almost every one in that case.  With a there, 2 of a
    row's 8 accumulators share its bank when the row is allocated
    contiguously (25%; measured 28-31%): fail above 40%."""
    fs = asm_hazards.functions(valu_asm, r"_Z\w*sgemm_valu_kernel\w*")
    assert len(fs) == 4   # two cores, each with and without the split part
    for name, blocks in fs.items():
        fmacs = [i for _, ins in blocks for i in ins if i.startswith("v_fmac_f32")]
        same = 0
        for ins in fmacs:
            dst, _src0, src1 = (x.strip() for x in ins.split(None, 1)[1].split(","))
            if dst.startswith("v") and src1.startswith("v") and int(dst[1:]) % 4 == int(src1[1:]) % 4:
                same += 1
        assert len(fmacs) >= 512, name
        assert same / len(fmacs) <= 0.40, f"{name}: {same}/{len(fmacs)} multiply-adds with src1 in the accumulator's bank"


def test_valu_loops_hold_no_lds_read_hazard(valu_asm):
    """The vector-ALU cores' LDS reads are the compiler's own; the dataflow
    check holds for them too."""
    fs = asm_hazards.functions(valu_asm, r"_Z\w*sgemm_valu_kernel\w*")
    bad = {n[:80]: h[:3] for n, b in fs.items() if (h := asm_hazards.hazards(b))}
    assert not bad, bad
