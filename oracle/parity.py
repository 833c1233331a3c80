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

import math

import numpy as np

from . import nsn as oracle

REL = 1e-3


def gpu_to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype.is_floating_point else t.cpu().numpy()


def check_encode_head(x, C, g, idx_gpu, s1_gpu, s2p_gpu, o_gpu, o_given=None, report=None, signs=None):
    """Compare one (L, d) tensor's encode against the oracle.  o_given (exact)
    switches the oracle to a reused mean; signs (+-1 per channel) to the
    randomized rotation.  Returns a dict of counts."""
    ref = oracle.encode_head(x, C, g, o_given, signs=signs)
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


def attention_ref_group(q_np, kc, vc, C, g, b, hk, GQ, S, signs=None):
    """Oracle attention for the GQ query heads of (b, KV head hk) over S tokens of
    host copies of the GPU-written cache: kc/vc = (idx, s1, s2p, o) numpy arrays."""
    K = oracle.dequantize_head(kc[0][b, hk, :S], kc[1][b, hk, :S], kc[2][b, hk, :S], kc[3][b, hk], C, g, signs)
    V = oracle.dequantize_head(vc[0][b, hk, :S], vc[1][b, hk, :S], vc[2][b, hk, :S], vc[3][b, hk], C, g, signs)
    return np.stack([oracle.attention_dense(q_np[b, hk * GQ + j], K, V) for j in range(GQ)])


def dq_head_from_bytes(rec):
    """Parameters of one nsn_dq_head record (80 bytes, as written by the library)."""
    rec = np.asarray(rec, dtype=np.uint8)
    nib = np.stack([rec[:64] & 15, rec[:64] >> 4], axis=1).reshape(128).astype(np.int64)
    scale = float(rec[64:68].view(np.float32)[0])
    base = int(rec[68:70].view(np.uint16)[0])
    stride = int(rec[70:72].view(np.uint16)[0])
    return dict(o_codes=nib - 8, o_scale=scale, s1_base=base, s1_stride=stride)


def s1_codes_from_bytes(s1c, L):
    """Codes of tokens 0 .. L-1 from the packed nibble bytes of one tensor."""
    s1c = np.asarray(s1c, dtype=np.uint8)
    nib = np.stack([s1c & 15, s1c >> 4], axis=1).reshape(-1).astype(np.int64)
    return nib[:L]


def check_dq_head(x, head_gpu):
    """The GPU-computed head record of a double-quantized tensor against the
    oracle's: o scale to fp32 rounding of the mean, o codes equal except where
    o / scale lies within 1e-4 of a rounding midpoint, the s1 grid from fp16
    patterns that may differ by one at a rounding boundary of s1."""
    x = np.asarray(x, dtype=np.float64)
    L, d = x.shape
    s1 = np.sqrt(np.sum(x * x, axis=1)) / math.sqrt(d)
    y = np.zeros_like(x)
    nz = s1 > 0
    y[nz] = x[nz] / s1[nz, None]
    o = y.mean(axis=0)
    codes, scale, _ = oracle.dq_o(o)
    assert abs(head_gpu["o_scale"] - scale) <= 1e-5 * max(scale, 1e-30), (head_gpu["o_scale"], scale)
    q = o / scale if scale > 0 else np.zeros_like(o)
    near_half = np.abs(np.abs(q - np.floor(q)) - 0.5) < 1e-4
    bad = (head_gpu["o_codes"] != codes) & ~near_half
    assert not bad.any(), f"o codes differ at channels {np.flatnonzero(bad)[:8]}"
    base, stride = oracle.dq_s1_params(s1)
    assert abs(head_gpu["s1_base"] - base) <= 1, (head_gpu["s1_base"], base)
    assert abs(head_gpu["s1_stride"] - stride) <= 1, (head_gpu["s1_stride"], stride)


def check_encode_head_dq(x, C, g, idx_gpu, s1c_gpu, s2p_gpu, head_gpu, report=None, signs=None):
    """One (L, d) tensor of a double-quantized encode against the oracle, which is
    given the GPU's parameters (as for a reused o): indices as check_encode_head,
    s1 codes equal except where s1 is within 2^-20 (relative) of an fp16 rounding
    midpoint or of a code boundary, s2' to 1e-3 on matching tokens."""
    ref = oracle.encode_head_dq(x, C, g, dq=head_gpu, signs=signs)
    L, m = ref["idx"].shape
    s1 = ref["s1_exact"]
    # s1 codes: the decision depends on the fp16 pattern of s1, taken in fp32 on the GPU
    b_lo = oracle.f16_bits(s1 * (1 - 2.0 ** -20))
    b_hi = oracle.f16_bits(s1 * (1 + 2.0 ** -20))
    c_lo = oracle.dq_s1_codes(s1 * (1 - 2.0 ** -20), head_gpu["s1_base"], head_gpu["s1_stride"])
    c_hi = oracle.dq_s1_codes(s1 * (1 + 2.0 ** -20), head_gpu["s1_base"], head_gpu["s1_stride"])
    s1_edge = (b_lo != b_hi) | (c_lo != c_hi)
    code_bad = (s1c_gpu != ref["s1c"]) & ~s1_edge
    assert not code_bad.any(), f"s1 codes differ at tokens {np.flatnonzero(code_bad)[:8]}"
    code_mism = s1c_gpu != ref["s1c"]
    mism = idx_gpu != ref["idx"]
    allowed = ref["tie"] | ref["edge"][:, None] | code_mism[:, None]
    bad = mism & ~allowed
    assert not bad.any(), (f"{int(bad.sum())} index mismatches outside near ties, e.g. "
                           f"{np.argwhere(bad)[:5].tolist()}")
    good = ~mism.any(axis=1) & ~ref["edge"] & ~code_mism
    gv, rv = s2p_gpu[good], ref["s2p"][good]
    rel = np.where(rv == 0, np.abs(gv), np.abs(gv - rv) / np.maximum(np.abs(rv), 1e-30))
    assert rel.size == 0 or rel.max() <= REL, f"s2p rel err {rel.max()}"
    out = dict(total=int(mism.size), flagged=int(ref["tie"].sum()), mismatched=int(mism.sum()),
               code_edges=int(s1_edge.sum()), tokens=L)
    if report is not None:
        for k, v in out.items():
            report[k] = report.get(k, 0) + v
    return out
