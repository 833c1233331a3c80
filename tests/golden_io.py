"""Readers of the stored fixtures under tests/golden/."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_codebook(g, finetuned=False):
    """(centroids float64 [256, g], header dict) of tests/golden/codebook_g{g}.txt
    (codebook_g{g}_ft.txt: the cosine fine-tuned one)."""
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, f"codebook_g{g}{'_ft' if finetuned else ''}.txt")) as f:
        for line in f:
            if line.startswith("#"):
                k, _, v = line[1:].strip().partition("=")
                meta[k] = v
            elif line.strip():
                rows.append([float(t) for t in line.split()])
    return np.array(rows), meta


def have_codebook(g, finetuned=False):
    return os.path.exists(os.path.join(GOLDEN, f"codebook_g{g}{'_ft' if finetuned else ''}.txt"))
