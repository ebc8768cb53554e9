#!/usr/bin/env python3
"""Writes tests/golden/full_output_sha256.txt: the SHA-256 of the CPU
oracle's WHOLE output C for every matmul workload, next to the SHA-256 of its
seeded operands.

Uses only ``oracle`` (the plain C triple loop of the fixed-order definition:
Verde and RepOps article, section 3.2, item 2) and the seeded input
generators; nothing from the GPU library.  The GPU tests and the benchmark
compare the digest of the GPU's full output with these, so every output of
every configuration is checked against the oracle, not only samples.

C is hashed as its M x N float32 values in row-major order, little-endian
(the bytes of a C-contiguous numpy array on this host).

Run:  python tests/golden/make_full_output_hashes.py [--threads T] [workload ...]
(the 4096 x 14336 x 4096 product takes about 5 minutes on 8 threads).
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

OUT = os.path.join(HERE, "full_output_sha256.txt")


def main():
    import oracle
    from bit_reproducible_fp32_amd import inputs

    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=None)
    ap.add_argument("workloads", nargs="*")
    args = ap.parse_args()
    names = args.workloads or list(inputs.WORKLOADS)
    rows = {}
    if os.path.exists(OUT):
        for line in open(OUT):
            if line.strip() and not line.startswith("#"):
                rows[line.split("|")[0].strip()] = line.rstrip("\n")
    for name in names:
        w = inputs.WORKLOADS[name]
        A, B = inputs.make_operands(name)
        t0 = time.perf_counter()
        C = oracle.matmul_f32(A, B, w.trans_a, w.trans_b, nthreads=args.threads)
        dt = time.perf_counter() - t0
        ha = hashlib.sha256(A.tobytes()).hexdigest()
        hb = hashlib.sha256(B.tobytes()).hexdigest()
        hc = hashlib.sha256(C.tobytes()).hexdigest()
        rows[name] = "%s | %d %d %d | %s | %s | %s" % (name, w.M, w.N, w.K, ha, hb, hc)
        print("%s: C %s (%.1f s)" % (name, hc, dt), flush=True)
        del A, B, C
    order = [n for n in inputs.WORKLOADS if n in rows]
    with open(OUT + ".tmp", "w") as f:
        f.write("# SHA-256 of the oracle's full output C (M x N float32, row-major, little-endian)\n"
                "# for each matmul workload, with the SHA-256 of its stored operands A and B.\n"
                "# Written by tests/golden/make_full_output_hashes.py, which calls only the CPU\n"
                "# oracle and the seeded input generators.\n"
                "# workload | M N K | sha256(A) | sha256(B) | sha256(C)\n")
        for n in order:
            f.write(rows[n] + "\n")
    os.replace(OUT + ".tmp", OUT)


if __name__ == "__main__":
    main()
