"""Write the stored N(0,1) k-means codebooks used as shared inputs by the tests.

Calls only ``oracle`` (fp64 k-means on the SplitMix64/Box-Muller stream).
Usage:  python tests/golden/make_codebooks.py [--samples N] [--iters I]
Output: tests/golden/codebook_g{4,8}.txt -- a header of key=value lines then K
rows of g fp16-exact values written with enough digits to round-trip exactly.
"""

import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

SEED = 20250524


def write(path, C, meta):
    with open(path, "w") as f:
        for k, v in meta.items():
            f.write(f"# {k}={v}\n")
        for row in C:
            f.write(" ".join(repr(float(x)) for x in row) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--samples", type=int, default=1 << 20)
    ap.add_argument("--iters", type=int, default=200)
    ap.add_argument("--g", type=int, nargs="*", default=[8, 4])
    a = ap.parse_args()
    for g in a.g:
        t = time.time()
        C, dist, it, conv = oracle.build_codebook(SEED, g, 256, a.samples, a.iters)
        meta = dict(seed=SEED, g=g, K=256, n_samples=a.samples, max_iters=a.iters, iterations=it,
                    converged=int(conv), distortion_per_dim=repr(dist),
                    generator="oracle.build_codebook (SplitMix64 -> Box-Muller -> Lloyd k-means, fp64, fp16 rounding)")
        write(os.path.join(HERE, f"codebook_g{g}.txt"), C, meta)
        print(f"g={g}: distortion/dim {dist:.6f} iterations {it} converged {conv} ({time.time() - t:.0f}s)", flush=True)


if __name__ == "__main__":
    main()
