"""fp64 NumPy oracle of the NSNQuant encode / decode-attention path.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is
imported by the product library.

Citations name sections of the Technical Summary of the English gist.science
explainer "NSNQuant: A Double Normalization Approach for Calibration-Free
Low-Bit Vector Quantization of KV Cache" (gist.science/paper/2505.18231):

  [NSN]   "1. Normalize-Shift-Normalize (NSN)"
  [HAD]   "2. Hadamard Transform"
  [VQ]    "3. Vector Quantization and Codebook"
  [IMPL]  "4. Implementation Details"

Readings taken where the page is silent (each repeated at its function):

  * norms are Euclidean; s1 is defined so that x = s1 * y, s2 so that z = s2 * u;
  * the channel mean o runs over the L tokens of one (batch, head) tensor handed
    to one encode call; a single appended token reuses a stored o;
  * an all-zero token has s1 = 0 and y = 0 (it still counts in the mean);
  * a token whose shifted vector z is (numerically) zero, ||z|| <= EPS_Z*sqrt(d),
    has s2 = 0, u = 0 and alpha = 1, so it reconstructs to s1 * o;
  * the Hadamard matrix is Sylvester's, natural (not sequency) order, scaled by
    1/sqrt(d), with no random signs (the page says the naive transform is the
    one implemented); the randomized variant the page names for its guarantee is
    kept as an option: w = H D u with D = diag(signs), signs a given +-1 vector
    (the random draw is an input), undone by u = D H w;
  * sub-vectors are contiguous g-blocks of the rotated token;
  * assignment is to the nearest centroid in squared L2, lowest index on ties;
  * the scale adjustment keeps the component of the reconstruction parallel to
    the rotated token equal to it: alpha = ||w||^2 / <w, w_hat> (guard: alpha = 1
    when <w, w_hat> <= 0 or s2 = 0); it is folded into s2' = s2 * alpha;
  * s1 and s2' are stored as IEEE fp16 (round to nearest even), o as fp32;
  * decode attention: score scale 1/sqrt(d), query head h reads KV head
    h // (Hq/Hkv), no mask, no positional rotation, fp32 output.

The cosine fine-tune of the codebook ([VQ]) is taken as full-batch gradient
descent on the mean cosine distance between d-dim N(0,1) vectors and their
quantizations, with the nearest-centroid assignment recomputed each iteration
and held fixed for the gradient (see cosine_finetune).

Parity on alpha beyond this reading is unpinned.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "EPS_Z",
    "sylvester_hadamard",
    "hadamard_orthonormal",
    "nsn_forward",
    "nsn_inverse",
    "rotate",
    "unrotate",
    "signs_from_mask",
    "subvectors",
    "nearest_centroid_bruteforce",
    "nearest_centroid",
    "near_tie_tau",
    "scale_adjust",
    "to_f16",
    "to_f32",
    "encode_head",
    "encode",
    "dequantize_head",
    "dequantize",
    "attention_dense",
    "decode_attention",
    "decode_attention_lut",
    "decode_attention_residual",
    "decode_attention_blocks",
    "splitmix64",
    "normal_stream",
    "kmeans",
    "build_codebook",
    "codebook_distortion",
    "cosine_loss_grad",
    "mean_cosine_distance",
    "cosine_finetune",
    "f16_bits",
    "f16_from_bits",
    "dq_o",
    "dq_s1_params",
    "dq_s1_codes",
    "dq_s1_values",
    "dq_codebook",
    "encode_head_dq",
    "dequantize_head_dq",
    "decode_attention_dq",
    "rope",
    "decode_attention_rope",
]

# Relative threshold below which the shifted token z is treated as zero
# (reading: the page does not say what happens when a token equals the mean).
EPS_Z = 1e-4

_U64 = np.uint64
_MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# [HAD] Hadamard transform
# ---------------------------------------------------------------------------
def sylvester_hadamard(d: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix H_d (entries +-1), natural order.

    [HAD]: the naive (non-randomised) Hadamard transform is the one used.
    Built by the recursion H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]].
    """
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_orthonormal(d: int) -> np.ndarray:
    """H_d / sqrt(d): symmetric, orthonormal and its own inverse ([HAD])."""
    return sylvester_hadamard(d) / math.sqrt(d)


def rotate(u: np.ndarray, signs: np.ndarray | None = None) -> np.ndarray:
    """w = H u for each row of u (H symmetric, so u @ H == (H u^T)^T) ([HAD]).

    signs (d,) of +-1: the randomized transform w = H D u, D = diag(signs)."""
    if signs is not None:
        u = u * np.asarray(signs, np.float64)
    return u @ hadamard_orthonormal(u.shape[-1])


def unrotate(w: np.ndarray, signs: np.ndarray | None = None) -> np.ndarray:
    """The inverse of rotate: u = D H w (H and D are their own inverses)."""
    u = w @ hadamard_orthonormal(w.shape[-1])
    if signs is not None:
        u = u * np.asarray(signs, np.float64)
    return u


def signs_from_mask(mask: bytes | np.ndarray, d: int = 128) -> np.ndarray:
    """+-1 signs from a bit mask: bit c % 8 of byte c // 8 set <=> channel c negated."""
    b = np.frombuffer(bytes(mask), dtype=np.uint8) if not isinstance(mask, np.ndarray) else mask.astype(np.uint8)
    bits = (b[np.arange(d) // 8] >> (np.arange(d) % 8)) & 1
    return 1.0 - 2.0 * bits.astype(np.float64)


# ---------------------------------------------------------------------------
# [NSN] Normalize-Shift-Normalize
# ---------------------------------------------------------------------------
def nsn_forward(x: np.ndarray, o: np.ndarray | None = None, eps_z: float = EPS_Z) -> dict:
    """Normalize-Shift-Normalize of one (L, d) tensor ([NSN]).

    1. token-wise: s1_i = ||x_i|| / sqrt(d), y_i = x_i / s1_i   (||y_i|| = sqrt(d))
    2. channel-wise: o = mean_i y_i, z_i = y_i - o              (given o is reused)
    3. token-wise: s2_i = ||z_i|| / sqrt(d), u_i = z_i / s2_i   (||u_i|| = sqrt(d))

    Returns s1, y, o, z, s2, u and per-token flags:
      ``zero_x``   token was exactly zero (s1 = 0, y = 0);
      ``degen``    ||z|| <= eps_z*sqrt(d): s2 = 0, u = 0 (reading);
      ``edge``     ||z|| / sqrt(d) lies within 1e-6 of eps_z, where an fp32
                   implementation may legitimately decide the other way.
    """
    x = np.asarray(x, dtype=np.float64)
    L, d = x.shape
    rd = math.sqrt(d)
    nx = np.sqrt(np.sum(x * x, axis=1))
    s1 = nx / rd
    zero_x = nx == 0.0
    y = np.zeros_like(x)
    nz_rows = ~zero_x
    y[nz_rows] = x[nz_rows] / s1[nz_rows, None]
    if o is None:
        o = y.mean(axis=0) if L > 0 else np.zeros(d)
    else:
        o = np.asarray(o, dtype=np.float64)
    z = y - o[None, :]
    nzz = np.sqrt(np.sum(z * z, axis=1))
    rel = nzz / rd
    degen = rel <= eps_z
    edge = np.abs(rel - eps_z) <= 1e-6
    s2 = np.where(degen, 0.0, rel)
    u = np.zeros_like(z)
    keep = ~degen
    u[keep] = z[keep] / s2[keep, None]
    return dict(s1=s1, y=y, o=o, z=z, s2=s2, u=u, zero_x=zero_x, degen=degen, edge=edge)


def nsn_inverse(s1: np.ndarray, s2: np.ndarray, u: np.ndarray, o: np.ndarray) -> np.ndarray:
    """x = s1 * (s2 * u + o): reconstruction from the byproducts ([NSN])."""
    return s1[:, None] * (s2[:, None] * u + o[None, :])


# ---------------------------------------------------------------------------
# [VQ] nearest centroid against one global codebook
# ---------------------------------------------------------------------------
def subvectors(w: np.ndarray, g: int) -> np.ndarray:
    """Split rows of w (L, d) into contiguous g-blocks -> (L, d//g, g) (reading)."""
    L, d = w.shape
    if d % g:
        raise ValueError("g must divide d")
    return w.reshape(L, d // g, g)


def nearest_centroid_bruteforce(v: np.ndarray, C: np.ndarray):
    """Explicit loop form: for each row of v (N, g) the index of the nearest
    row of C (K, g) in squared L2, lowest index on ties ([VQ]; small inputs).
    Returns (idx, dist) with dist the (N, K) explicit distances."""
    v = np.asarray(v, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    N, K = v.shape[0], C.shape[0]
    dist = np.empty((N, K))
    idx = np.empty(N, dtype=np.int64)
    for n in range(N):
        best, bi = math.inf, -1
        for k in range(K):
            diff = v[n] - C[k]
            dk = float(np.dot(diff, diff))
            dist[n, k] = dk
            if dk < best:  # strict: the lowest index wins a tie
                best, bi = dk, k
        idx[n] = bi
    return idx, dist


def nearest_centroid(v: np.ndarray, C: np.ndarray, chunk: int = 32768):
    """Nearest centroid for many rows (expanded form, fp64 BLAS, chunked).

    D_k = ||v||^2 + ||C_k||^2 - 2 <v, C_k>; argmin with the lowest index on ties
    (np.argmin returns the first minimum).  Returns idx, d1 (best distance),
    d2 (second-best distance over the other indices) ([VQ])."""
    v = np.asarray(v, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    N = v.shape[0]
    cn = np.sum(C * C, axis=1)
    idx = np.empty(N, dtype=np.int64)
    d1 = np.empty(N)
    d2 = np.empty(N)
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        vv = v[s:e]
        D = (np.sum(vv * vv, axis=1)[:, None] + cn[None, :]) - 2.0 * (vv @ C.T)
        i = np.argmin(D, axis=1)
        r = np.arange(e - s)
        idx[s:e] = i
        d1[s:e] = D[r, i]
        D[r, i] = np.inf
        d2[s:e] = D.min(axis=1) if C.shape[0] > 1 else np.inf
    return idx, d1, d2


def near_tie_tau(d1, d2, vnorm2, cmax2):
    """Gap below which an fp32 implementation may pick a different (equally
    valid up to rounding) centroid.  Derived from the fp32 decision arithmetic:
    relative key precision 2^-15 on the two smallest distances, fp32
    accumulation over terms of size ||v||^2 + max ||C||^2, and the fp32 error of
    the rotated token itself; doubled for margin.  Not a property of the method."""
    d1 = np.asarray(d1, dtype=np.float64)
    d2 = np.asarray(d2, dtype=np.float64)
    return (2.0 ** -13) * (np.abs(d1) + np.abs(d2)) + (2.0 ** -18) * (vnorm2 + cmax2) + 2.0 ** -16


def scale_adjust(w: np.ndarray, w_hat: np.ndarray, mode: str = "par") -> np.ndarray:
    """Per-token scale of the quantized rotated token ([VQ], "Scale Adjustment").

    The page: the quantized vector is scaled to keep the components parallel to
    the original vector, so that the error is orthogonal.  Reading ("par"):
    alpha = ||w||^2 / <w, w_hat>, i.e. <w, alpha*w_hat> = ||w||^2.  Alternatives
    kept for study only: "ls" = <w, w_hat>/||w_hat||^2, "norm" = ||w||/||w_hat||.
    Guard: alpha = 1 when the denominator is <= 0 or w = 0."""
    w = np.asarray(w, dtype=np.float64)
    w_hat = np.asarray(w_hat, dtype=np.float64)
    ww = np.sum(w * w, axis=1)
    wh = np.sum(w * w_hat, axis=1)
    hh = np.sum(w_hat * w_hat, axis=1)
    if mode == "par":
        num, den = ww, wh
    elif mode == "ls":
        num, den = wh, hh
    elif mode == "norm":
        num, den = np.sqrt(ww), np.sqrt(hh)
    else:
        raise ValueError(mode)
    ok = (den > 0) & (ww > 0)
    alpha = np.ones_like(ww)
    alpha[ok] = num[ok] / den[ok]
    return alpha


def to_f16(a) -> np.ndarray:
    """IEEE binary16, round to nearest even, returned as float64 values."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def to_f32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def encode_head(x: np.ndarray, C: np.ndarray, g: int, o: np.ndarray | None = None,
                alpha_mode: str = "par", signs: np.ndarray | None = None) -> dict:
    """Encode one (L, d) K or V tensor ([NSN], [HAD], [VQ]).

    Returns idx (L, d/g) int, s1 and s2p as stored fp16 values, o as stored fp32
    (the o actually used for the shift is the unrounded one when computed here,
    the given one when reused), plus diagnostics: w, s2, alpha, d1, d2, tau,
    tie (per sub-vector near-tie flag) and the NSN flags."""
    C = np.asarray(C, dtype=np.float64)
    L, d = x.shape
    n = nsn_forward(x, o)
    w = rotate(n["u"], signs)
    v = subvectors(w, g).reshape(-1, g)
    idx, d1, d2 = nearest_centroid(v, C)
    cmax2 = float(np.max(np.sum(C * C, axis=1)))
    tau = near_tie_tau(d1, d2, np.sum(v * v, axis=1), cmax2)
    tie = (d2 - d1) <= tau
    idx = idx.reshape(L, d // g)
    w_hat = C[idx].reshape(L, d)
    alpha = scale_adjust(w, w_hat, alpha_mode)
    alpha = np.where(n["degen"], 1.0, alpha)
    s2p = n["s2"] * alpha
    return dict(idx=idx, s1=to_f16(n["s1"]), s2p=to_f16(s2p), o=to_f32(n["o"]),
                o_exact=n["o"], w=w, s2=n["s2"], alpha=alpha, s1_exact=n["s1"],
                s2p_exact=s2p, d1=d1.reshape(L, -1), d2=d2.reshape(L, -1),
                tau=tau.reshape(L, -1), tie=tie.reshape(L, -1),
                zero_x=n["zero_x"], degen=n["degen"], edge=n["edge"])


def encode(x: np.ndarray, C: np.ndarray, g: int, o: np.ndarray | None = None,
           signs: np.ndarray | None = None) -> dict:
    """Batched encode of x (B, H, L, d); o (B, H, d) given => reused."""
    B, H, L, d = x.shape
    out = {}
    for b in range(B):
        for h in range(H):
            r = encode_head(x[b, h], C, g, None if o is None else o[b, h], signs=signs)
            for k, val in r.items():
                out.setdefault(k, np.empty((B, H) + np.shape(val), dtype=np.asarray(val).dtype))
                out[k][b, h] = val
    return out


def dequantize_head(idx, s1, s2p, o, C, g, signs: np.ndarray | None = None) -> np.ndarray:
    """x_hat_i = s1_i * (s2'_i * H w_hat_i + o) from stored values ([NSN], [IMPL]);
    with signs, x_hat_i = s1_i * (s2'_i * D H w_hat_i + o)."""
    C = np.asarray(C, dtype=np.float64)
    idx = np.asarray(idx)
    L, m = idx.shape
    w_hat = C[idx].reshape(L, m * g)
    u_hat = unrotate(w_hat, signs)
    return nsn_inverse(np.asarray(s1, np.float64), np.asarray(s2p, np.float64), u_hat,
                       np.asarray(o, np.float64))


def dequantize(idx, s1, s2p, o, C, g, signs: np.ndarray | None = None) -> np.ndarray:
    """Batched dequantize: idx (B, H, L, m), s1/s2p (B, H, L), o (B, H, d)."""
    B, H, L, m = idx.shape
    out = np.empty((B, H, L, m * g))
    for b in range(B):
        for h in range(H):
            out[b, h] = dequantize_head(idx[b, h], s1[b, h], s2p[b, h], o[b, h], C, g, signs)
    return out


# ---------------------------------------------------------------------------
# [IMPL] attention over the quantized cache
# ---------------------------------------------------------------------------
def attention_dense(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Single-query softmax attention: softmax(K q / sqrt(d)) . V, fp64,
    max-subtracted (plain definition; reading for the 1/sqrt(d) scale)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    s = K @ q / math.sqrt(q.shape[0])
    s = s - s.max()
    p = np.exp(s)
    return (p @ V) / p.sum()


def decode_attention(q, k_idx, k_s1, k_s2p, k_o, v_idx, v_s1, v_s2p, v_o, C, g,
                     signs: np.ndarray | None = None) -> np.ndarray:
    """Decode attention of q (B, Hq, d) over the quantized cache (B, Hkv, S, m).

    Dense definition on the dequantized cache ([IMPL]: attention computed over
    the cache using the NSN byproducts).  Query head h reads KV head h // G."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_idx.shape[1]
    G = Hq // Hkv
    out = np.empty((B, Hq, d))
    for b in range(B):
        for hk in range(Hkv):
            Kh = dequantize_head(k_idx[b, hk], k_s1[b, hk], k_s2p[b, hk], k_o[b, hk], C, g, signs)
            Vh = dequantize_head(v_idx[b, hk], v_s1[b, hk], v_s2p[b, hk], v_o[b, hk], C, g, signs)
            for j in range(G):
                out[b, hk * G + j] = attention_dense(q[b, hk * G + j], Kh, Vh)
    return out


def decode_attention_residual(q, k_idx, k_s1, k_s2p, k_o, v_idx, v_s1, v_s2p, v_o, C, g, k_res, v_res,
                              signs: np.ndarray | None = None) -> np.ndarray:
    """Decode attention over a coded cache plus a window of the newest tokens
    kept as raw rows ([IMPL] "Residuals": when the window is full its tokens are
    coded and added to the end of the cache).

    q (B, Hq, d); the quantized arrays hold S tokens per (b, KV head), S >= 0;
    k_res, v_res (B, Hkv, R, d) are the residual tokens as stored (fp16 values,
    exact in fp64), R >= 0, S + R >= 1.  The plain definition: one softmax over
    the S dequantized tokens followed by the R residual tokens.  Query head h
    reads KV head h // G."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_res.shape[1]
    G = Hq // Hkv
    S = k_idx.shape[2]
    out = np.empty((B, Hq, d))
    for b in range(B):
        for hk in range(Hkv):
            Kr = np.asarray(k_res[b, hk], np.float64)
            Vr = np.asarray(v_res[b, hk], np.float64)
            if S > 0:
                Kh = dequantize_head(k_idx[b, hk], k_s1[b, hk], k_s2p[b, hk], k_o[b, hk], C, g, signs)
                Vh = dequantize_head(v_idx[b, hk], v_s1[b, hk], v_s2p[b, hk], v_o[b, hk], C, g, signs)
                Kr = np.concatenate([Kh, Kr])
                Vr = np.concatenate([Vh, Vr])
            for j in range(G):
                out[b, hk * G + j] = attention_dense(q[b, hk * G + j], Kr, Vr)
    return out


def decode_attention_blocks(q, k_idx, k_s1, k_s2p, k_o, k_ob, v_idx, v_s1, v_s2p, v_o, v_ob, C, g, S0, Rb,
                            k_res=None, v_res=None, signs: np.ndarray | None = None) -> np.ndarray:
    """Decode attention over a cache whose flushed residual blocks were each
    quantized as a tensor of their own ([IMPL] "Residuals": a full window is
    quantized and appended; [NSN]: the shift is the channel mean of the tensor being
    quantized), so each block keeps its own o.

    The quantized arrays hold S0 + nblk Rb tokens per (b, KV head): tokens [0, S0)
    use k_o / v_o (B, Hkv, d), block j (tokens S0 + j Rb .. S0 + (j+1) Rb - 1) uses
    k_ob[j] / v_ob[j] ((nblk, B, Hkv, d)); then the optional raw residual rows
    (B, Hkv, R, d).  The plain definition: every segment dequantized with its own o,
    one softmax over all of them in order.  Query head h reads KV head h // G."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_idx.shape[1]
    G = Hq // Hkv
    nblk = 0 if k_ob is None else len(k_ob)
    out = np.empty((B, Hq, d))
    for b in range(B):
        for hk in range(Hkv):
            Ks, Vs = [], []
            segs = [(0, S0, k_o[b, hk] if S0 > 0 else None, v_o[b, hk] if S0 > 0 else None)]
            segs += [(S0 + j * Rb, S0 + (j + 1) * Rb, k_ob[j][b, hk], v_ob[j][b, hk]) for j in range(nblk)]
            for t0, t1, ko, vo in segs:
                if t1 <= t0:
                    continue
                Ks.append(dequantize_head(k_idx[b, hk, t0:t1], k_s1[b, hk, t0:t1], k_s2p[b, hk, t0:t1], ko, C, g,
                                          signs))
                Vs.append(dequantize_head(v_idx[b, hk, t0:t1], v_s1[b, hk, t0:t1], v_s2p[b, hk, t0:t1], vo, C, g,
                                          signs))
            if k_res is not None and k_res.shape[2] > 0:
                Ks.append(np.asarray(k_res[b, hk], np.float64))
                Vs.append(np.asarray(v_res[b, hk], np.float64))
            K, V = np.concatenate(Ks), np.concatenate(Vs)
            for j in range(G):
                out[b, hk * G + j] = attention_dense(q[b, hk * G + j], K, V)
    return out


def decode_attention_lut(q, k_idx, k_s1, k_s2p, k_o, v_idx, v_s1, v_s2p, v_o, C, g) -> np.ndarray:
    """The same attention, reordered the way a quantized-cache kernel computes it
    (one head, fp64): with q~ = H q, score_i = s1_i (s2'_i sum_j <q~_j, C[idx_ij]> +
    <q, o_K>) / sqrt(d); the value sum is accumulated in the rotated domain and
    rotated back once: out = (H sum_i p_i s1_i s2'_i w_hat_i + (sum_i p_i s1_i) o_V)
    / sum_i p_i.  Used only to check that reordering against the dense form."""
    q = np.asarray(q, np.float64)
    C = np.asarray(C, np.float64)
    B, Hq, d = q.shape
    Hkv = k_idx.shape[1]
    G = Hq // Hkv
    m = d // g
    Hn = hadamard_orthonormal(d)
    out = np.empty((B, Hq, d))
    for b in range(B):
        for hk in range(Hkv):
            for j in range(G):
                h = hk * G + j
                qt = Hn @ q[b, h]
                lut = qt.reshape(m, g) @ C.T                       # (m, K)
                ki = k_idx[b, hk]
                dots = lut[np.arange(m)[None, :], ki].sum(axis=1)  # (S,)
                s = k_s1[b, hk] * (k_s2p[b, hk] * dots + q[b, h] @ k_o[b, hk]) / math.sqrt(d)
                p = np.exp(s - s.max())
                vh = C[v_idx[b, hk]].reshape(-1, d)
                acc = (p * v_s1[b, hk] * v_s2p[b, hk]) @ vh
                beta = np.sum(p * v_s1[b, hk])
                out[b, h] = (Hn @ acc + beta * v_o[b, hk]) / p.sum()
    return out


# ---------------------------------------------------------------------------
# [VQ] codebook: k-means on synthetic N(0, 1) samples
# ---------------------------------------------------------------------------
def splitmix64(seed: int, start: int, n: int) -> np.ndarray:
    """Outputs start..start+n-1 of SplitMix64 (Steele, Lea, Flood, OOPSLA 2014)
    seeded with ``seed``: output i = mix(seed + (i + 1) * 0x9E3779B97F4A7C15) with
    mix(z) = z ^ z>>30, * 0xBF58476D1CE4E5B9, ^ >>27, * 0x94D049BB133111EB, ^ >>31
    (all mod 2^64).  Counter-based, so any slice can be drawn independently."""
    i = np.arange(start + 1, start + n + 1, dtype=_U64)
    with np.errstate(over="ignore"):
        z = _U64(seed & _MASK64) + i * _U64(0x9E3779B97F4A7C15)
        z = (z ^ (z >> _U64(30))) * _U64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> _U64(27))) * _U64(0x94D049BB133111EB)
        z = z ^ (z >> _U64(31))
    return z


def normal_stream(seed: int, start: int, n: int) -> np.ndarray:
    """Standard normals start..start+n-1 of the stream: pair p uses SplitMix64
    outputs 2p, 2p+1 -> u1 = (top 53 bits + 1) * 2^-53 in (0, 1],
    u2 = top 53 bits * 2^-53 in [0, 1); Box-Muller (1958):
    normal 2p = sqrt(-2 ln u1) cos(2 pi u2), normal 2p+1 = sqrt(-2 ln u1) sin(2 pi u2)."""
    p0 = start // 2
    p1 = (start + n + 1) // 2
    bits = splitmix64(seed, 2 * p0, 2 * (p1 - p0))
    a = bits[0::2] >> _U64(11)
    b = bits[1::2] >> _U64(11)
    u1 = (a.astype(np.float64) + 1.0) * (2.0 ** -53)
    u2 = b.astype(np.float64) * (2.0 ** -53)
    r = np.sqrt(-2.0 * np.log(u1))
    t = 2.0 * math.pi * u2
    z = np.empty(2 * (p1 - p0))
    z[0::2] = r * np.cos(t)
    z[1::2] = r * np.sin(t)
    off = start - 2 * p0
    return z[off:off + n]


def kmeans(X: np.ndarray, K: int, max_iters: int, chunk: int = 65536):
    """Lloyd k-means ([VQ]: codebook initialised by k-means on N(0,1) data).

    Reading: initial centroids are the first K samples; each iteration assigns
    every sample to its nearest centroid (lowest index on ties) and stops if no
    assignment changed, otherwise moves each centroid to its cell mean.  An
    empty cell is re-seeded: empty cells in increasing index take the samples
    farthest from their assigned centroid (ties: lower sample index first).
    Returns (C, iterations_run, converged)."""
    X = np.asarray(X, dtype=np.float64)
    N, g = X.shape
    C = X[:K].copy()
    prev = None
    it = 0
    converged = False
    while it < max_iters:
        idx, d1, _ = nearest_centroid(X, C, chunk)
        it += 1
        if prev is not None and np.array_equal(idx, prev):
            converged = True
            break
        prev = idx
        cnt = np.bincount(idx, minlength=K)
        sums = np.zeros((K, g))
        _segment_sum(sums, idx, X)
        empty = np.flatnonzero(cnt == 0)
        nz = cnt > 0
        C[nz] = sums[nz] / cnt[nz, None]
        if empty.size:
            order = np.lexsort((np.arange(N), -d1))  # farthest first, lower index first
            C[empty] = X[order[: empty.size]]
    return C, it, converged


def _segment_sum(out: np.ndarray, idx: np.ndarray, X: np.ndarray) -> None:
    for t in range(X.shape[1]):
        out[:, t] = np.bincount(idx, weights=X[:, t], minlength=out.shape[0])


def codebook_distortion(X: np.ndarray, C: np.ndarray) -> float:
    """Mean over samples of min_k ||x - C_k||^2, divided by the dimension."""
    _, d1, _ = nearest_centroid(X, C)
    return float(np.mean(np.maximum(d1, 0.0)) / X.shape[1])


def cosine_loss_grad(W: np.ndarray, C: np.ndarray, g: int, idx: np.ndarray):
    """Mean cosine distance of the rows of W (N, d) to their quantization
    w_hat = concatenated centroids C[idx] (idx (N, d/g), held fixed), and its
    gradient with respect to C ([VQ]: fine-tune to minimise the cosine distance
    between original and quantized vectors).

    With c_i = <w_i, w_hat_i> / (|w_i| |w_hat_i|) and loss = mean_i (1 - c_i):
    d c_i / d w_hat_i = w_i / (|w_i| |w_hat_i|) - c_i w_hat_i / |w_hat_i|^2, and
    the gradient of centroid k is minus the mean over vectors of that vector
    restricted to the blocks assigned to k.  A vector whose quantization is zero
    counts as distance 1 and contributes no gradient.
    Returns (loss, grad (K, g))."""
    W = np.asarray(W, dtype=np.float64)
    N, d = W.shape
    m = d // g
    What = C[idx.reshape(-1)].reshape(N, d)
    nw = np.linalg.norm(W, axis=1)
    nh = np.linalg.norm(What, axis=1)
    ok = (nw > 0) & (nh > 0)
    c = np.zeros(N)
    c[ok] = np.sum(W[ok] * What[ok], axis=1) / (nw[ok] * nh[ok])
    dc = np.zeros_like(W)
    dc[ok] = W[ok] / (nw[ok] * nh[ok])[:, None] - (c[ok] / nh[ok] ** 2)[:, None] * What[ok]
    grad = np.zeros_like(C, dtype=np.float64)
    _segment_sum(grad, idx.reshape(-1), -dc.reshape(N * m, g) / N)
    return float(np.mean(1.0 - c)), grad


def mean_cosine_distance(W: np.ndarray, C: np.ndarray, g: int) -> float:
    """Mean over the rows of W of 1 - cos(w, w_hat), w_hat the nearest-centroid
    quantization of w's contiguous g-blocks (the quantity the fine-tune lowers;
    with the scale adjustment, 1 - cos^2 is the relative squared error)."""
    W = np.asarray(W, dtype=np.float64)
    idx = nearest_centroid(W.reshape(-1, g), C)[0].reshape(W.shape[0], -1)
    return cosine_loss_grad(W, C, g, idx)[0]


def cosine_finetune(C0: np.ndarray, g: int, seed: int, n_vectors: int, iters: int, lr: float,
                    d: int = 128):
    """Fine-tune a k-means codebook for cosine distance ([VQ], codebook
    construction: after k-means on N(0,1) data the codebook is tuned to minimise
    the cosine distance between original and quantized vectors, with no model in
    the loop).

    Readings (the page names neither data, optimiser nor schedule): the data are
    n_vectors d-dim N(0,1) vectors from the SplitMix64/Box-Muller stream of
    ``seed`` (vector i = normals i*d .. i*d+d-1); each of ``iters`` iterations
    assigns every g-block to its nearest centroid under the current codebook
    (squared L2, lowest index on ties), then takes one full-batch gradient step
    C <- C - lr * grad of the mean cosine distance with that assignment held
    fixed (the argmin itself has zero derivative almost everywhere).
    Returns (C fp64, C rounded to fp16, losses before each step)."""
    W = normal_stream(seed, 0, n_vectors * d).reshape(n_vectors, d)
    C = np.array(C0, dtype=np.float64)
    losses = []
    for _ in range(iters):
        idx = nearest_centroid(W.reshape(-1, g), C)[0].reshape(n_vectors, d // g)
        loss, grad = cosine_loss_grad(W, C, g, idx)
        losses.append(loss)
        C = C - lr * grad
    return C, to_f16(C), np.array(losses)


def build_codebook(seed: int, g: int, K: int = 256, n_samples: int = 1 << 20,
                   max_iters: int = 200):
    """Global codebook ([VQ]): k-means on ``n_samples`` g-dim N(0,1) vectors from
    the SplitMix64/Box-Muller stream of ``seed`` (vector i = normals
    i*g..i*g+g-1), then rounded to fp16 (reading: makes the entries exact matrix-
    core operands).  The cosine fine-tune is a separate step (cosine_finetune).
    Returns (C fp16-exact float64 (K, g), distortion per dim, iterations, converged)."""
    X = normal_stream(seed, 0, n_samples * g).reshape(n_samples, g)
    C, it, conv = kmeans(X, K, max_iters)
    C16 = to_f16(C)
    return C16, codebook_distortion(X, C16), it, conv


# ---------------------------------------------------------------------------
# [VQ] double quantization (DQ): o, s1 and the codebook entries in 4 bits
# ---------------------------------------------------------------------------
# The page quantizes the NSN parameters (the mean o and the scale s1) and the
# codebook entries to 4 bits.  Readings (the page gives no format):
#   * o: symmetric absmax per (batch, head) tensor, one fp32 scale
#     max|o| / 7, codes -7 .. 7 (round half to even), o_q = code * scale;
#   * s1: a 4-bit code per token on a uniform grid over the fp16 bit pattern of
#     s1 (piecewise logarithmic in s1): base = smallest pattern over the
#     tensor's non-zero tokens, stride = max(1, ceil((largest - base) / 14));
#     code 0 marks a zero token, codes 1 .. 15 the patterns base + (c-1) stride;
#   * the quantized parameters are used by the encoding itself (y = x / s1_q,
#     z = y - o_q), so that x = s1_q (s2 u + o_q) still holds exactly before
#     the vector quantization; o itself is the mean of x / s1 (unquantized);
#   * codebook: one step D = max|C| / 7.5 (fp32) for all entries, mid-rise
#     levels (k - 7.5) D, k = 0 .. 15, nearest level, then fp16.


def f16_bits(a) -> np.ndarray:
    """IEEE binary16 bit patterns (round to nearest even) as int64."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16).astype(np.int64)


def f16_from_bits(b) -> np.ndarray:
    return np.asarray(b, dtype=np.int64).astype(np.uint16).view(np.float16).astype(np.float64)


def dq_o(o: np.ndarray):
    """4-bit o of one tensor: (codes -7..7 int, scale, o_q values).  The scale
    max|o| / 7 is kept as fp32 (its storage format); each code is the nearest
    integer (ties to even) of o / scale, decided in fp64, and o_q = code * scale
    (exact in fp64)."""
    o = np.asarray(o, dtype=np.float64)
    scale = float(to_f32(np.max(np.abs(o)) / 7.0)) if o.size else 0.0
    if scale == 0.0:
        codes = np.zeros(o.shape, dtype=np.int64)
    else:
        codes = np.clip(np.rint(o / scale), -7, 7).astype(np.int64)
    return codes, scale, codes * scale


def dq_s1_params(s1: np.ndarray):
    """(base, stride) of the s1 grid from the tensor's s1 values (reading above).
    A tensor without non-zero tokens gets base = pattern of 1.0, stride 1."""
    b = f16_bits(s1)
    nz = np.asarray(s1) > 0
    if not np.any(nz):
        return 0x3C00, 1
    lo, hi = int(np.min(b[nz])), int(np.max(b[nz]))
    return lo, max(1, -((lo - hi) // 14))


def dq_s1_codes(s1: np.ndarray, base: int, stride: int) -> np.ndarray:
    """Nearest grid code (ties up) of each s1, clamped to 1 .. 15; 0 for s1 = 0."""
    b = f16_bits(s1)
    q = 1 + np.minimum(14, (np.maximum(b - base, 0) + stride // 2) // stride)
    return np.where(np.asarray(s1) > 0, q, 0).astype(np.int64)


def dq_s1_values(codes: np.ndarray, base: int, stride: int) -> np.ndarray:
    """s1_q of each code: the fp16 value with pattern base + (code-1) stride
    (capped at the largest finite fp16), 0 for code 0."""
    codes = np.asarray(codes, dtype=np.int64)
    pat = np.minimum(base + (codes - 1) * stride, 0x7BFF)
    return np.where(codes > 0, f16_from_bits(np.maximum(pat, 0)), 0.0)


def dq_codebook(C: np.ndarray):
    """4-bit codebook: (codes 0..15, step D (fp32), C_q fp16-exact values)."""
    C = np.asarray(C, dtype=np.float64)
    D = float(to_f32(np.max(np.abs(C)) / 7.5))
    if D == 0.0:
        return np.full(C.shape, 8, dtype=np.int64), 0.0, np.zeros_like(C)
    k = np.clip(np.floor(C / D + 8.0), 0, 15).astype(np.int64)
    return k, D, to_f16((k - 7.5) * D)


def encode_head_dq(x: np.ndarray, C: np.ndarray, g: int, dq: dict | None = None,
                   signs: np.ndarray | None = None) -> dict:
    """Encode one (L, d) tensor with double-quantized NSN parameters ([NSN],
    [HAD], [VQ] including DQ).  ``dq`` None computes the parameters from x
    (o_codes, o_scale, s1_base, s1_stride); a given ``dq`` is reused (append).
    Returns idx, s1 codes, s2p (fp16), the parameters, o_q, s1_q and the
    diagnostics of encode_head (w, d1, d2, tau, tie, degen, edge), plus the
    pre-quantization pieces (s2, u) that reconstruct x exactly."""
    C = np.asarray(C, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    L, d = x.shape
    rd = math.sqrt(d)
    s1 = np.sqrt(np.sum(x * x, axis=1)) / rd
    if dq is None:
        y = np.zeros_like(x)
        nz = s1 > 0
        y[nz] = x[nz] / s1[nz, None]
        o_codes, o_scale, o_q = dq_o(y.mean(axis=0) if L > 0 else np.zeros(d))
        base, stride = dq_s1_params(s1)
        dq = dict(o_codes=o_codes, o_scale=o_scale, s1_base=base, s1_stride=stride)
    else:
        o_q = np.asarray(dq["o_codes"]) * dq["o_scale"]
    codes = dq_s1_codes(s1, dq["s1_base"], dq["s1_stride"])
    s1q = dq_s1_values(codes, dq["s1_base"], dq["s1_stride"])
    y = np.zeros_like(x)
    nz = s1q > 0
    y[nz] = x[nz] / s1q[nz, None]
    z = y - o_q[None, :]
    rel = np.sqrt(np.sum(z * z, axis=1)) / rd
    degen = rel <= EPS_Z
    edge = np.abs(rel - EPS_Z) <= 1e-6
    s2 = np.where(degen, 0.0, rel)
    u = np.zeros_like(z)
    u[~degen] = z[~degen] / s2[~degen, None]
    w = rotate(u, signs)
    v = subvectors(w, g).reshape(-1, g)
    idx, d1, d2 = nearest_centroid(v, C)
    tau = near_tie_tau(d1, d2, np.sum(v * v, axis=1), float(np.max(np.sum(C * C, axis=1))))
    idx = idx.reshape(L, d // g)
    alpha = np.where(degen, 1.0, scale_adjust(w, C[idx].reshape(L, d)))
    s2p = s2 * alpha
    return dict(idx=idx, s1c=codes, s2p=to_f16(s2p), dq=dq, o_q=o_q, s1q=s1q, s1_exact=s1,
                s1_bits=f16_bits(s1), s2=s2, u=u, w=w, alpha=alpha, s2p_exact=s2p,
                d1=d1.reshape(L, -1), d2=d2.reshape(L, -1), tau=tau.reshape(L, -1),
                tie=((d2 - d1) <= tau).reshape(L, -1), degen=degen, edge=edge)


def dequantize_head_dq(idx, s1c, s2p, dq: dict, C, g, signs: np.ndarray | None = None) -> np.ndarray:
    """x_hat_i = s1_q(code_i) (s2'_i H w_hat_i + o_q) ([NSN] with the DQ parameters)."""
    s1q = dq_s1_values(s1c, dq["s1_base"], dq["s1_stride"])
    o_q = np.asarray(dq["o_codes"]) * dq["o_scale"]
    return dequantize_head(idx, s1q, s2p, o_q, C, g, signs)


def decode_attention_dq(q, k_idx, k_s1c, k_s2p, k_dq, v_idx, v_s1c, v_s2p, v_dq, C, g,
                        signs: np.ndarray | None = None) -> np.ndarray:
    """Decode attention over a double-quantized cache: the plain definition on
    the dequantized K and V.  k_dq / v_dq are [B][Hkv] nested lists of the
    per-tensor parameter dicts; the other arrays as in decode_attention."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_idx.shape[1]
    G = Hq // Hkv
    out = np.empty((B, Hq, d))
    for b in range(B):
        for hk in range(Hkv):
            K = dequantize_head_dq(k_idx[b, hk], k_s1c[b, hk], k_s2p[b, hk], k_dq[b][hk], C, g, signs)
            V = dequantize_head_dq(v_idx[b, hk], v_s1c[b, hk], v_s2p[b, hk], v_dq[b][hk], C, g, signs)
            for j in range(G):
                out[b, hk * G + j] = attention_dense(q[b, hk * G + j], K, V)
    return out


# ---------------------------------------------------------------------------
# [IMPL] keys quantized before the rotary position embedding
# ---------------------------------------------------------------------------
# The page applies NSN to keys before RoPE; the cache then holds pre-RoPE keys and
# the score rotates each dequantized key by its position.  Readings: the
# rotate-half convention of the LLaMA / Mistral code (channel j pairs with
# j + d/2, frequency theta_j = base^(-2j/d), j < d/2); the query is given already
# rotated to its own position; cached token i sits at position i.


def rope(x: np.ndarray, positions, base: float = 10000.0) -> np.ndarray:
    """Rotary embedding of the rows of x (n, d) at the given positions (fp64):
    out_j = x_j cos(p theta_j) - x_{j+d/2} sin(p theta_j),
    out_{j+d/2} = x_{j+d/2} cos(p theta_j) + x_j sin(p theta_j)."""
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    h = d // 2
    theta = base ** (-2.0 * np.arange(h) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s_ = np.cos(ang), np.sin(ang)
    lo, hi = x[:, :h], x[:, h:]
    return np.concatenate([lo * c - hi * s_, hi * c + lo * s_], axis=1)


def decode_attention_rope(q, k_idx, k_s1, k_s2p, k_o, v_idx, v_s1, v_s2p, v_o, C, g,
                          base: float = 10000.0, signs: np.ndarray | None = None) -> np.ndarray:
    """Decode attention over a cache of pre-RoPE quantized keys ([IMPL]): the
    plain definition, softmax over i of q . rope(k_hat_i, i) / sqrt(d), then the
    weighted sum of the (unrotated) dequantized values.  q (B, Hq, d) is the
    rotated query; query head h reads KV head h // G."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_idx.shape[1]
    S = k_idx.shape[2]
    G = Hq // Hkv
    out = np.empty((B, Hq, d))
    for b in range(B):
        for hk in range(Hkv):
            K = dequantize_head(k_idx[b, hk], k_s1[b, hk], k_s2p[b, hk], k_o[b, hk], C, g, signs)
            V = dequantize_head(v_idx[b, hk], v_s1[b, hk], v_s2p[b, hk], v_o[b, hk], C, g, signs)
            Kr = rope(K, np.arange(S), base)
            for j in range(G):
                out[b, hk * G + j] = attention_dense(q[b, hk * G + j], Kr, V)
    return out
