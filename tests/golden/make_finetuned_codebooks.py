"""Write the cosine fine-tuned codebooks used as shared inputs by the tests.

Starts from the stored k-means codebooks (codebook_g{4,8}.txt) and calls only
``oracle.cosine_finetune`` (full-batch gradient descent on the mean cosine
distance of d = 128 N(0,1) vectors, fp64, fp16 rounding at the end).
Usage:  python tests/golden/make_finetuned_codebooks.py [--vectors N] [--iters I] [--lr LR]
Output: tests/golden/codebook_g{4,8}_ft.txt, same format as the k-means files.
"""

import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from golden_io import load_codebook  # noqa: E402
from make_codebooks import write  # noqa: E402

SEED = 20250525


def main():
    ap = argparse.ArgumentParser()
    # as many g-blocks as k-means saw samples (2^20): 2^20 g / 128 vectors
    ap.add_argument("--vectors", type=int, default=0)
    ap.add_argument("--iters", type=int, default=30)
    ap.add_argument("--lr", type=float, default=300.0)
    ap.add_argument("--g", type=int, nargs="*", default=[8, 4])
    a = ap.parse_args()
    for g in a.g:
        t = time.time()
        nv = a.vectors or (1 << 20) * g // 128
        C0, _ = load_codebook(g)
        _, C16, losses = oracle.cosine_finetune(C0, g, SEED, nv, a.iters, a.lr)
        W = oracle.normal_stream(SEED, 0, nv * 128).reshape(nv, 128)
        final = oracle.mean_cosine_distance(W, C16, g)
        meta = dict(seed=SEED, g=g, K=256, n_vectors=nv, d=128, iters=a.iters, lr=a.lr,
                    start=f"codebook_g{g}.txt", cos_dist_start=repr(float(losses[0])),
                    cos_dist_final_fp16=repr(final),
                    generator="oracle.cosine_finetune (full-batch gradient descent on the mean cosine distance, "
                              "fp64, fp16 rounding)")
        write(os.path.join(HERE, f"codebook_g{g}_ft.txt"), C16, meta)
        print(f"g={g}: mean cosine distance {losses[0]:.6f} -> {final:.6f} ({time.time() - t:.0f}s)", flush=True)


if __name__ == "__main__":
    main()
