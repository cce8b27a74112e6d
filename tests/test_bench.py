"""bench.py's host-side pieces (no GPU): the --gpus contract and the digest
that ties the recorded HBM traffic to the kernel sources it was taken on."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_only_ignores_comments_and_layout():
    b = load_bench()
    a = "int f(int x) {  // one\n  return x + 1; /* two\n lines */ }\n"
    c = "int f(int x) { return x + 1; }"
    assert b.code_only(a) == b.code_only(c)
    assert b.code_only(a) != b.code_only(c.replace("+ 1", "+ 2"))


def test_digest_follows_the_code():
    b = load_bench()
    base = b.kernel_source_digest()
    texts = {f: open(os.path.join(ROOT, f), encoding="utf-8").read() for f in b.KERNEL_SOURCES}
    first = b.KERNEL_SOURCES[0]
    commented = dict(texts, **{first: texts[first] + "\n// a comment only\n"})
    assert b.kernel_source_digest(commented.get) == base
    changed = dict(texts, **{first: texts[first] + "\nstatic int extra_symbol;\n"})
    assert b.kernel_source_digest(changed.get) != base


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
