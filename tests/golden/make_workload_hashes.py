"""Write workload_sha256.txt: the SHA-256 of every seeded input matrix.

Calls only the input generator (workloads), never the GPU library.  Rerun
after a deliberate change of the generator recipe; the test
tests/test_workloads.py::test_hashes_match_golden checks the stored digests.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads  # noqa: E402


def main():
    lines = ["# name M N K dist seed sha256(A) sha256(B)"]
    for w in workloads.WORKLOADS.values():
        A, B = workloads.generate_workload(w)
        lines.append(f"{w.name} {w.M} {w.N} {w.K} {w.dist} {w.seed} "
                     f"{workloads.sha256(A)} {workloads.sha256(B)}")
    with open(os.path.join(HERE, "workload_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
