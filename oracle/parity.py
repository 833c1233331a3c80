"""Comparison rules between the HIP path and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Indices: equal to the oracle's wherever the oracle does not flag a near tie
(second-best distance within tau of the best, tau from the fp32 decision
arithmetic) or a token at the degenerate-shift threshold; every other index
must still be a valid choice -- its exact fp64 distance within tau of the best.
Scales: |rel diff| <= 1e-3 on tokens whose indices all match (one fp16 ulp is
2^-10 < 1e-3).  o: ||do|| / ||o|| <= 1e-3 per tensor.  Attention: per row,
||dout|| <= 1e-3 ||out_ref|| and max|dout| <= 1e-3 max|out_ref|, with out_ref
computed by the oracle on the dequantized GPU-written cache.
"""

import numpy as np

from . import nsn as oracle

REL = 1e-3


def gpu_to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype.is_floating_point else t.cpu().numpy()


def check_encode_head(x, C, g, idx_gpu, s1_gpu, s2p_gpu, o_gpu, o_given=None, report=None):
    """Compare one (L, d) tensor's encode against the oracle.  o_given (exact)
    switches the oracle to a reused mean.  Returns a dict of counts."""
    ref = oracle.encode_head(x, C, g, o_given)
    L, m = ref["idx"].shape
    # o
    if o_given is None:
        do = np.linalg.norm(o_gpu - ref["o_exact"]) / max(np.linalg.norm(ref["o_exact"]), 1e-30)
        assert do <= REL, f"o rel err {do}"
    # indices
    mism = idx_gpu != ref["idx"]
    allowed = ref["tie"] | ref["edge"][:, None]
    bad = mism & ~allowed
    assert not bad.any(), (f"{int(bad.sum())} index mismatches outside near ties, e.g. token/sub-vector "
                           f"{np.argwhere(bad)[:5].tolist()}")
    if mism.any():  # flagged mismatches must still be near-optimal choices
        v = oracle.subvectors(ref["w"], g)
        tok, sv = np.nonzero(mism)
        dg = np.sum((v[tok, sv] - C[idx_gpu[tok, sv]]) ** 2, axis=1)
        excess = dg - ref["d1"][tok, sv]
        assert np.all(excess <= ref["tau"][tok, sv] + 1e-12), f"invalid near-tie choice, excess {excess.max()}"
    # scales on fully matching, non-edge tokens
    good = ~mism.any(axis=1) & ~ref["edge"]
    for name, gv, rv in (("s1", s1_gpu, ref["s1"]), ("s2p", s2p_gpu, ref["s2p"])):
        gv, rv = gv[good], rv[good]
        den = np.maximum(np.abs(rv), 1e-30)
        rel = np.where(rv == 0, np.abs(gv), np.abs(gv - rv) / den)
        assert rel.size == 0 or rel.max() <= REL, f"{name} rel err {rel.max()} at {np.argmax(rel)}"
    out = dict(total=int(mism.size), flagged=int(ref["tie"].sum()), mismatched=int(mism.sum()),
               tokens=L, degenerate=int(ref["degen"].sum()))
    if report is not None:
        for k, v in out.items():
            report[k] = report.get(k, 0) + v
    return out


def check_attention_rows(out_gpu, out_ref):
    """out_* (R, d).  Per-row relative L2 and max-abs criteria."""
    assert np.all(np.isfinite(out_gpu))
    for r in range(out_ref.shape[0]):
        nr = np.linalg.norm(out_ref[r])
        e = np.linalg.norm(out_gpu[r] - out_ref[r])
        assert e <= REL * nr, f"row {r}: rel L2 err {e / nr}"
        assert np.max(np.abs(out_gpu[r] - out_ref[r])) <= REL * np.max(np.abs(out_ref[r])), f"row {r}: max-abs err"


def attention_ref_group(q_np, kc, vc, C, g, b, hk, GQ, S):
    """Oracle attention for the GQ query heads of (b, KV head hk) over S tokens of
    host copies of the GPU-written cache: kc/vc = (idx, s1, s2p, o) numpy arrays."""
    K = oracle.dequantize_head(kc[0][b, hk, :S], kc[1][b, hk, :S], kc[2][b, hk, :S], kc[3][b, hk], C, g)
    V = oracle.dequantize_head(vc[0][b, hk, :S], vc[1][b, hk, :S], vc[2][b, hk, :S], vc[3][b, hk], C, g)
    return np.stack([oracle.attention_dense(q_np[b, hk * GQ + j], K, V) for j in range(GQ)])
