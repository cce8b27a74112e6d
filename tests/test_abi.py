"""The C-ABI library on the host: it loads, exports exactly what the header
declares, and rejects bad arguments before touching the GPU."""
import os
import re

import pytest

import fp32_sgemm_f32_amd as sg
import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sgemm_f32.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgemm_f32\w*)\s*\(", text)))


def exported_functions():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    return sorted({ln.split()[-1] for ln in out.splitlines() if " T " in ln})


def test_library_loads():
    assert sg.library() is not None


def test_exports_match_header():
    declared = header_functions()
    assert declared, "no declarations parsed"
    assert exported_functions() == declared
    lib = sg.library()
    for name in declared:
        assert hasattr(lib, name)


def test_plan_struct_matches_header():
    """The binding's plan structure has the header's fields, in order, with
    the same C types (int / long long / double), so the plan query fills it
    as the library writes it."""
    import ctypes
    text = open(HEADER).read()
    body = re.search(r"typedef struct sgemm_f32_plan_t \{(.*?)\} sgemm_f32_plan_t;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        m = re.match(r"(long long|int|double)\s+(.*)", decl)
        assert m, decl
        ctype = {"long long": ctypes.c_longlong, "int": ctypes.c_int, "double": ctypes.c_double}[m.group(1)]
        fields += [(name.strip(), ctype) for name in m.group(2).split(",")]
    assert [(n, t) for n, t in sg._Plan._fields_] == fields


def test_granule():
    # Any shape: ragged edges are masked.
    assert sg.granule() == (1, 1, 1)


def test_status_strings():
    texts = [sg.status_string(s) for s in range(0, 10)]
    assert all(texts) and len(set(texts)) == 10
    assert sg.status_string(12345) == "unknown status"


def test_no_hip_error_recorded():
    assert sg.last_hip_error() == 0


ALIGNED = 0x10000000       # never dereferenced: every case fails validation first


def call(M, N, K, A=ALIGNED, lda=None, B=ALIGNED + (1 << 30), ldb=None, C=ALIGNED + (2 << 30),
         ldc=None, config=sg.CFG_AUTO, sched=sg.SCHED_AUTO):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return sg.sgemm_raw(M, N, K, A, lda, B, ldb, C, ldc, 0, config, sched)


@pytest.mark.parametrize("shape", [(-128, 128, 32), (128, -128, 32), (128, 128, -32)])
def test_rejects_shape(shape):
    assert call(*shape) == sg.ERR_SHAPE


VALIDATION_ERRORS = (sg.ERR_SHAPE, sg.ERR_LD, sg.ERR_ALIGN, sg.ERR_NULL, sg.ERR_ALIAS, sg.ERR_CONFIG)


@pytest.mark.parametrize("shape", [(100, 128, 32), (128, 200, 32), (128, 128, 48), (1, 1, 1), (7, 13, 5)])
def test_accepts_any_shape(shape):
    # Ragged shapes pass argument validation (a device is needed beyond it).
    assert call(*shape) not in VALIDATION_ERRORS


def test_accepts_any_leading_dimension_and_float_alignment():
    assert call(128, 128, 64, lda=66) not in VALIDATION_ERRORS
    assert call(128, 128, 64, ldc=130) not in VALIDATION_ERRORS
    assert call(128, 128, 64, A=ALIGNED + 4) not in VALIDATION_ERRORS


def test_rejects_leading_dimension():
    assert call(128, 128, 64, lda=60) == sg.ERR_LD
    assert call(128, 128, 64, ldb=124) == sg.ERR_LD
    assert call(128, 128, 64, ldc=124) == sg.ERR_LD


def test_rejects_null():
    assert call(128, 128, 64, A=0) == sg.ERR_NULL
    assert call(128, 128, 64, B=0) == sg.ERR_NULL
    assert call(128, 128, 64, C=0) == sg.ERR_NULL


def test_rejects_alignment():
    # Pointers must at least be aligned to a float.
    assert call(128, 128, 64, A=ALIGNED + 2) == sg.ERR_ALIGN
    assert call(128, 128, 64, B=ALIGNED + (1 << 30) + 1) == sg.ERR_ALIGN
    assert call(128, 128, 64, C=ALIGNED + (2 << 30) + 6) == sg.ERR_ALIGN


def test_rejects_alias():
    # C starts inside A's extent, and B's.
    assert call(128, 128, 64, C=ALIGNED + 4096) == sg.ERR_ALIAS
    assert call(128, 128, 64, C=ALIGNED + (1 << 30) + 256) == sg.ERR_ALIAS
    # Adjacent, non-overlapping regions are fine up to the device checks; here
    # C sits right after A: that is not an alias (rejected later, on a GPU only).


def test_rejects_unknown_config_or_schedule():
    assert call(128, 128, 64, config=99) == sg.ERR_CONFIG
    assert call(128, 128, 64, config=-1) == sg.ERR_CONFIG
    assert call(128, 128, 64, sched=7) == sg.ERR_CONFIG


def test_k_zero_ignores_a_and_b_layout():
    # With K == 0 only C is checked: A/B strides and alignment do not matter,
    # but C's still do (and valid arguments would then need a device).
    assert call(128, 128, 0, lda=1, ldb=3, C=ALIGNED + (2 << 30) + 2) == sg.ERR_ALIGN
    assert call(128, 128, 0, A=ALIGNED + 1, lda=1, ldb=3) not in VALIDATION_ERRORS
    assert call(128, 128, 0, lda=1, ldb=3, ldc=100) == sg.ERR_LD
    assert call(128, 128, 0, A=0, B=0, C=0) == sg.ERR_NULL


def test_empty_output_is_a_no_op():
    # M == 0 or N == 0: nothing to compute, nothing touched, no device needed.
    assert call(0, 128, 64, A=0, B=0, C=0) == sg.OK
    assert call(128, 0, 64, A=0, B=0, C=0) == sg.OK


def test_tflops_accounting_matches_pages():
    """2 n^3 / t reproduces every TFLOP/s figure the pages print from their
    times, allowing for the rounding of both printed numbers."""
    path = os.path.join(os.path.dirname(__file__), "golden", "page_timings.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 24
    for tag, n, t, printed in rows:
        n = int(n)
        mant, _, exp = t.partition("e")
        half = 0.5 * 10.0 ** -len(mant.split(".")[1]) * 10.0 ** int(exp or 0)
        t = float(t)
        lo = workloads.tflops(n, n, n, t + half)
        hi = workloads.tflops(n, n, n, t - half)
        p_half = 0.5 * 10.0 ** -len(printed.split(".")[1])
        assert lo - p_half <= float(printed) <= hi + p_half, tag


def noalloc(M, N, K, A=ALIGNED, lda=None, B=ALIGNED + (1 << 30), ldb=None, C=ALIGNED + (2 << 30), ldc=None,
            ta=0, tb=0):
    lda = (M if ta else K) if lda is None else lda
    ldb = (K if tb else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return sg.gemm_noalloc_raw(ta, tb, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc, 0)


def test_noalloc_rejects_bad_arguments_before_the_device():
    """The no-allocation call checks its arguments as sgemm_f32_gemm does,
    before it looks up any device memory (no GPU needed for these)."""
    assert noalloc(-1, 64, 64) == sg.ERR_SHAPE
    assert noalloc(64, 64, 64, lda=60) == sg.ERR_LD
    assert noalloc(64, 64, 64, ldc=60) == sg.ERR_LD
    assert noalloc(64, 64, 64, A=0) == sg.ERR_NULL
    assert noalloc(64, 64, 64, C=ALIGNED + (2 << 30) + 2) == sg.ERR_ALIGN
    assert noalloc(64, 64, 64, C=ALIGNED + 1024) == sg.ERR_ALIAS
    assert noalloc(64, 64, 64, ta=2) == sg.ERR_CONFIG
    assert noalloc(0, 64, 64, A=0, B=0, C=0) == sg.OK
    assert noalloc(64, 0, 64, A=0, B=0, C=0) == sg.OK
