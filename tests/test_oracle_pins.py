"""Pins of the fp64 oracle against what the mathematics and the pages fix.

Each test checks the oracle against something other than itself: a hand-worked
example, a closed form, an invariant, a special case that reduces to a library
routine, or brute force on tiny inputs.  No GPU.
"""

import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import scipy.stats
from scipy.spatial.distance import cdist

import oracle
from golden_io import load_codebook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hand_example():
    vals = {}
    with open(os.path.join(GOLDEN, "nsn_hand_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            vals[k] = np.array([float(t) for t in v])
    return vals




# ---------------------------------------------------------------- Hadamard
def test_hadamard_small_explicit():
    assert np.array_equal(oracle.sylvester_hadamard(2), np.array([[1.0, 1.0], [1.0, -1.0]]))
    h4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=float)
    assert np.array_equal(oracle.sylvester_hadamard(4), h4)
    np.testing.assert_allclose(oracle.hadamard_orthonormal(2), np.array([[1, 1], [1, -1]]) / math.sqrt(2))


@pytest.mark.parametrize("d", [8, 32, 128])
def test_hadamard_matches_scipy_and_is_orthonormal_involution(d):
    H = oracle.hadamard_orthonormal(d)
    assert np.array_equal(oracle.sylvester_hadamard(d), scipy.linalg.hadamard(d).astype(float))
    np.testing.assert_allclose(H @ H.T, np.eye(d), atol=1e-14)
    np.testing.assert_allclose(H @ H, np.eye(d), atol=1e-14)
    assert np.array_equal(H, H.T)
    e0 = np.zeros(d)
    e0[0] = 1
    np.testing.assert_allclose(H @ e0, np.full(d, 1 / math.sqrt(d)), atol=1e-15)
    x = np.random.default_rng(1).standard_normal((5, d))
    np.testing.assert_allclose(np.linalg.norm(oracle.rotate(x), axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # rotate() applies H to each row (not H^T on the other side): compare per-row products
    np.testing.assert_allclose(oracle.rotate(x), (H @ x.T).T, atol=1e-13)


# ---------------------------------------------------------------- NSN
def test_nsn_hand_worked_example():
    v = _hand_example()
    x = np.stack([v["x0"], v["x1"]])
    n = oracle.nsn_forward(x)
    np.testing.assert_allclose(n["s1"], v["s1"], atol=1e-15)
    np.testing.assert_allclose(n["o"], v["o"], atol=1e-15)
    np.testing.assert_allclose(n["s2"], v["s2"], atol=1e-15)
    np.testing.assert_allclose(n["u"], np.stack([v["u0"], v["u1"]]), atol=1e-15)
    w = oracle.rotate(n["u"])
    np.testing.assert_allclose(w, np.stack([v["w0"], v["w1"]]), atol=1e-15)


def test_nsn_invariants_random():
    rng = np.random.default_rng(2)
    L, d = 300, 128
    x = rng.standard_normal((L, d)) * np.exp(0.5 * rng.standard_normal(d)) + 1.4 * rng.standard_normal(d)
    n = oracle.nsn_forward(x)
    rd = math.sqrt(d)
    np.testing.assert_allclose(np.linalg.norm(n["y"], axis=1), rd, rtol=1e-13)
    np.testing.assert_allclose(n["z"].sum(axis=0), 0.0, atol=1e-11)
    np.testing.assert_allclose(np.linalg.norm(n["u"], axis=1), rd, rtol=1e-13)
    np.testing.assert_allclose(oracle.nsn_inverse(n["s1"], n["s2"], n["u"], n["o"]), x, rtol=1e-12, atol=1e-12)
    # s1 is the token norm over sqrt(d) (not the norm itself), the mean is over tokens
    np.testing.assert_allclose(n["s1"] * rd, np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(n["o"], (x / np.linalg.norm(x, axis=1, keepdims=True)).mean(axis=0) * rd, rtol=1e-12)
    # after NSN + Hadamard the mean per-channel second moment is exactly 1 (sum ||w||^2 = L d)
    w = oracle.rotate(n["u"])
    assert abs(np.mean(w * w) - 1.0) < 1e-12


def test_nsn_degenerate_tokens():
    d = 16
    x = np.zeros((3, d))
    x[1] = np.arange(d) + 1.0
    x[2] = -np.arange(d) * 0.5
    n = oracle.nsn_forward(x)
    assert n["zero_x"].tolist() == [True, False, False]
    assert n["s1"][0] == 0.0 and not np.any(n["y"][0])
    np.testing.assert_allclose(oracle.nsn_inverse(n["s1"], n["s2"], n["u"], n["o"]), x, atol=1e-12)
    # one token: it equals the mean, so z = 0 -> s2 = 0, u = 0, reconstruction s1*o = x
    n1 = oracle.nsn_forward(x[1:2])
    assert n1["degen"][0] and n1["s2"][0] == 0.0 and not np.any(n1["u"])
    np.testing.assert_allclose(oracle.nsn_inverse(n1["s1"], n1["s2"], n1["u"], n1["o"]), x[1:2], rtol=1e-14)
    # all tokens equal up to scale: every z vanishes
    xs = np.stack([x[1], 2 * x[1], 0.25 * x[1]])
    ns = oracle.nsn_forward(xs)
    assert ns["degen"].all()
    np.testing.assert_allclose(oracle.nsn_inverse(ns["s1"], ns["s2"], ns["u"], ns["o"]), xs, rtol=1e-13)


def test_nsn_reuses_given_mean():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 32))
    o = rng.standard_normal(32)
    n = oracle.nsn_forward(x, o)
    assert np.array_equal(n["o"], o)
    np.testing.assert_allclose(n["z"], n["y"] - o, atol=0)


# ---------------------------------------------------------------- nearest centroid
def test_nearest_centroid_hand_example():
    C = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    idx, dist = oracle.nearest_centroid_bruteforce(np.array([[0.6, 0.1]]), C)
    np.testing.assert_allclose(dist[0], [0.37, 0.17, 1.17], atol=1e-15)
    assert idx[0] == 1
    i2, d1, d2 = oracle.nearest_centroid(np.array([[0.6, 0.1]]), C)
    assert i2[0] == 1 and abs(d1[0] - 0.17) < 1e-15 and abs(d2[0] - 0.37) < 1e-15


def test_nearest_centroid_forms_agree_and_match_scipy():
    rng = np.random.default_rng(4)
    C = rng.standard_normal((64, 4))
    v = rng.standard_normal((200, 4))
    ib, db = oracle.nearest_centroid_bruteforce(v, C)
    ie, d1, d2 = oracle.nearest_centroid(v, C)
    assert np.array_equal(ib, ie)
    np.testing.assert_allclose(d1, db.min(axis=1), atol=1e-12)
    ref = cdist(v, C, "sqeuclidean")
    assert np.array_equal(ie, ref.argmin(axis=1))
    np.testing.assert_allclose(d2, np.sort(ref, axis=1)[:, 1], atol=1e-12)


def test_nearest_centroid_exact_hits_and_ties():
    rng = np.random.default_rng(5)
    C = rng.standard_normal((16, 8))
    idx, d1, _ = oracle.nearest_centroid(C.copy(), C)
    assert np.array_equal(idx, np.arange(16)) and np.all(np.abs(d1) < 1e-12)
    Cd = np.concatenate([C, C[3:4]])          # index 16 duplicates 3 -> 3 must win
    idx2, dist = oracle.nearest_centroid_bruteforce(C[3:4] + 1e-3, Cd)
    assert idx2[0] == 3 and dist[0, 3] == dist[0, 16]
    idx3, _, _ = oracle.nearest_centroid(C[3:4] + 1e-3, Cd)
    assert idx3[0] == 3


def test_near_tie_tau_is_small_and_positive():
    t = oracle.near_tie_tau(np.array([0.5]), np.array([0.7]), 4.0, 16.0)
    assert 0 < t[0] < 1e-3


# ---------------------------------------------------------------- scale adjustment
def test_scale_adjust_parallel_component():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((50, 32))
    wh = w + 0.3 * rng.standard_normal((50, 32))
    a = oracle.scale_adjust(w, wh)
    np.testing.assert_allclose(np.sum(w * (a[:, None] * wh), axis=1), np.sum(w * w, axis=1), rtol=1e-12)
    err = w - a[:, None] * wh                       # the residual error is orthogonal to w
    np.testing.assert_allclose(np.sum(err * w, axis=1), 0.0, atol=1e-11)
    np.testing.assert_allclose(oracle.scale_adjust(w, w), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.scale_adjust(w, 2 * w), 0.5, rtol=1e-14)
    assert oracle.scale_adjust(w[:1], -w[:1])[0] == 1.0     # guard: non-positive projection
    assert oracle.scale_adjust(np.zeros((1, 4)), np.ones((1, 4)))[0] == 1.0


def test_fp16_rounding_is_nearest_even():
    assert oracle.to_f16(1 + 2 ** -11)[()] == 1.0
    assert oracle.to_f16(1 + 3 * 2 ** -11)[()] == 1 + 2 ** -9
    assert oracle.to_f16(65504.0)[()] == 65504.0


# ---------------------------------------------------------------- encode / dequantize
def test_encode_lossless_codebook_round_trip():
    """With a codebook that holds every rotated sub-vector exactly, encode picks
    them (distance 0), alpha = 1, and dequantize returns x."""
    rng = np.random.default_rng(7)
    L, d, g = 6, 16, 4
    x = rng.standard_normal((L, d)) + 0.5
    w = oracle.rotate(oracle.nsn_forward(x)["u"])
    C = oracle.subvectors(w, g).reshape(-1, g)
    assert C.shape[0] <= 256
    r = oracle.encode_head(x, C, g)
    np.testing.assert_allclose(C[r["idx"]].reshape(L, d), w, atol=1e-13)
    np.testing.assert_allclose(r["alpha"], 1.0, rtol=1e-12)
    xr = oracle.dequantize_head(r["idx"], r["s1_exact"], r["s2p_exact"], r["o_exact"], C, g)
    np.testing.assert_allclose(xr, x, rtol=1e-11, atol=1e-11)


def test_encode_matches_bruteforce_on_its_own_rotation():
    rng = np.random.default_rng(8)
    C = oracle.to_f16(rng.standard_normal((256, 8)))
    x = rng.standard_normal((40, 128)) * 3 + 1
    r = oracle.encode_head(x, C, 8)
    ib, _ = oracle.nearest_centroid_bruteforce(oracle.subvectors(r["w"], 8).reshape(-1, 8), C)
    assert np.array_equal(r["idx"].reshape(-1), ib)
    np.testing.assert_allclose(r["s1"], oracle.to_f16(np.linalg.norm(x, axis=1) / math.sqrt(128)), rtol=0)
    # stored s2' = fp16(s2 * alpha); the reconstruction keeps the parallel component
    wh = C[r["idx"]].reshape(40, 128)
    np.testing.assert_allclose(np.sum(r["w"] * r["alpha"][:, None] * wh, axis=1), 128.0, rtol=1e-12)


def test_dequantize_hand_example():
    # d = 4, g = 2: idx picks [1,0] and [0,1]; s1 = 2, s2' = 0.5, o = [1 0 0 0]
    C = np.array([[1.0, 0.0], [0.0, 1.0]])
    idx = np.array([[0, 1]])
    # w_hat = [1 0 0 1]; H4/2 w_hat = [1 0 0 1]; x = 2 (0.5 [1 0 0 1] + [1 0 0 0]) = [3 0 0 1]
    xr = oracle.dequantize_head(idx, np.array([2.0]), np.array([0.5]), np.array([1.0, 0, 0, 0]), C, 2)
    np.testing.assert_allclose(xr, [[3.0, 0.0, 0.0, 1.0]], atol=1e-15)


# ---------------------------------------------------------------- attention
def _random_cache(rng, B, Hkv, S, d, g, K=256):
    C = oracle.to_f16(rng.standard_normal((K, g)))
    m = d // g
    mk = lambda: dict(idx=rng.integers(0, K, (B, Hkv, S, m)), s1=oracle.to_f16(rng.uniform(0.5, 2, (B, Hkv, S))),
                      s2p=oracle.to_f16(rng.uniform(0.5, 1.5, (B, Hkv, S))),
                      o=oracle.to_f32(rng.standard_normal((B, Hkv, d))))
    return C, mk(), mk()


def _args(kc, vc):
    return (kc["idx"], kc["s1"], kc["s2p"], kc["o"], vc["idx"], vc["s1"], vc["s2p"], vc["o"])


def test_attention_special_cases():
    rng = np.random.default_rng(9)
    V = rng.standard_normal((7, 8))
    K = rng.standard_normal((7, 8))
    np.testing.assert_allclose(oracle.attention_dense(np.zeros(8), K, V), V.mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(oracle.attention_dense(rng.standard_normal(8), K[:1], V[:1]), V[0], atol=1e-14)
    q = 50.0 * K[4] / np.linalg.norm(K[4])
    Kd = K.copy()
    Kd[4] = 10 * q
    np.testing.assert_allclose(oracle.attention_dense(q, Kd, V), V[4], atol=1e-12)
    perm = rng.permutation(7)
    qq = rng.standard_normal(8)
    np.testing.assert_allclose(oracle.attention_dense(qq, K[perm], V[perm]), oracle.attention_dense(qq, K, V), atol=1e-14)
    p = scipy.special.softmax(K @ qq / math.sqrt(8))
    np.testing.assert_allclose(oracle.attention_dense(qq, K, V), p @ V, atol=1e-14)


def test_decode_attention_gqa_mapping_and_lut_form():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, S, d, g = 2, 4, 2, 37, 32, 4
    C, kc, vc = _random_cache(rng, B, Hkv, S, d, g)
    q = oracle.to_f16(rng.standard_normal((B, Hq, d)))
    out = oracle.decode_attention(q, *_args(kc, vc), C, g)
    for b in range(B):
        for h in range(Hq):
            hk = h // 2
            Kh = oracle.dequantize_head(kc["idx"][b, hk], kc["s1"][b, hk], kc["s2p"][b, hk], kc["o"][b, hk], C, g)
            Vh = oracle.dequantize_head(vc["idx"][b, hk], vc["s1"][b, hk], vc["s2p"][b, hk], vc["o"][b, hk], C, g)
            p = scipy.special.softmax(Kh @ q[b, h] / math.sqrt(d))
            np.testing.assert_allclose(out[b, h], p @ Vh, atol=1e-12)
    lut = oracle.decode_attention_lut(q, *_args(kc, vc), C, g)
    np.testing.assert_allclose(lut, out, atol=1e-12)


def test_decode_attention_blocks_reductions():
    """Per-block o: no blocks is the plain decode (with a window: the residual
    decode); blocks whose o equal the prefix's are the single-o decode over the
    whole cache, however the tokens are cut into blocks; shifting one block's o_V by
    delta moves the output by (sum over that block's tokens of p_i s1_i) delta, the
    weights p from the scipy softmax of the dequantized keys."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, d, g = 2, 4, 2, 32, 4
    S0, Rb, nblk = 11, 5, 3
    S = S0 + Rb * nblk
    C, kc, vc = _random_cache(rng, B, Hkv, S, d, g)
    q = oracle.to_f16(rng.standard_normal((B, Hq, d)))
    kr = oracle.to_f16(rng.standard_normal((B, Hkv, 4, d)))
    vr = oracle.to_f16(rng.standard_normal((B, Hkv, 4, d)))
    kob = oracle.to_f32(rng.standard_normal((nblk, B, Hkv, d)))
    vob = oracle.to_f32(rng.standard_normal((nblk, B, Hkv, d)))

    def blocks(kc_, vc_, ko, vo, s0, rb, **kw):
        return oracle.decode_attention_blocks(q, kc_["idx"], kc_["s1"], kc_["s2p"], kc_["o"], ko, vc_["idx"], vc_["s1"],
                                              vc_["s2p"], vc_["o"], vo, C, g, s0, rb, **kw)

    np.testing.assert_allclose(blocks(kc, vc, None, None, S, 1), oracle.decode_attention(q, *_args(kc, vc), C, g),
                               atol=1e-13)
    np.testing.assert_allclose(blocks(kc, vc, None, None, S, 1, k_res=kr, v_res=vr),
                               oracle.decode_attention_residual(q, *_args(kc, vc), C, g, kr, vr), atol=1e-13)
    same_k = np.broadcast_to(kc["o"], (nblk,) + kc["o"].shape)
    same_v = np.broadcast_to(vc["o"], (nblk,) + vc["o"].shape)
    ref = oracle.decode_attention(q, *_args(kc, vc), C, g)
    np.testing.assert_allclose(blocks(kc, vc, same_k, same_v, S0, Rb), ref, atol=1e-13)
    n1 = S - S0 - 2  # the same tokens cut into one-token blocks after a longer prefix
    same_k1 = np.broadcast_to(kc["o"], (n1,) + kc["o"].shape)
    same_v1 = np.broadcast_to(vc["o"], (n1,) + vc["o"].shape)
    np.testing.assert_allclose(blocks(kc, vc, same_k1, same_v1, S0 + 2, 1), ref, atol=1e-13)
    base = blocks(kc, vc, kob, vob, S0, Rb)
    j, delta = 1, rng.standard_normal(d)
    vob2 = vob.copy()
    vob2[j] += delta
    moved = blocks(kc, vc, kob, vob2, S0, Rb)
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            segs = [(0, S0, kc["o"][b, hk])] + [(S0 + i * Rb, S0 + (i + 1) * Rb, kob[i, b, hk]) for i in range(nblk)]
            K = np.concatenate([oracle.dequantize_head(kc["idx"][b, hk, t0:t1], kc["s1"][b, hk, t0:t1],
                                                       kc["s2p"][b, hk, t0:t1], o, C, g) for t0, t1, o in segs])
            p = scipy.special.softmax(K @ q[b, h] / math.sqrt(d))
            t0, t1 = S0 + j * Rb, S0 + (j + 1) * Rb
            w = float(np.sum(p[t0:t1] * vc["s1"][b, hk, t0:t1]))
            np.testing.assert_allclose(moved[b, h] - base[b, h], w * delta, atol=1e-12)


def test_decode_attention_residual_reductions():
    """Residual window: R = 0 is the quantized-only decode; S = 0 is plain
    attention over the raw tokens (scipy softmax); in between, the one softmax
    over S + R tokens equals the log-sum-exp merge of the two separate softmaxes,
    and a dominant residual key selects its value."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, S, R, d, g = 2, 4, 2, 29, 6, 32, 4
    C, kc, vc = _random_cache(rng, B, Hkv, S, d, g)
    q = oracle.to_f16(rng.standard_normal((B, Hq, d)))
    kr = oracle.to_f16(rng.standard_normal((B, Hkv, R, d)))
    vr = oracle.to_f16(rng.standard_normal((B, Hkv, R, d)))
    empty = np.zeros((B, Hkv, 0, d))
    np.testing.assert_allclose(oracle.decode_attention_residual(q, *_args(kc, vc), C, g, empty, empty),
                               oracle.decode_attention(q, *_args(kc, vc), C, g), atol=1e-13)
    none = dict(idx=kc["idx"][:, :, :0], s1=kc["s1"][:, :, :0], s2p=kc["s2p"][:, :, :0], o=kc["o"])
    only_r = oracle.decode_attention_residual(q, *_args(none, none), C, g, kr, vr)
    both = oracle.decode_attention_residual(q, *_args(kc, vc), C, g, kr, vr)
    quant = oracle.decode_attention(q, *_args(kc, vc), C, g)
    for b in range(B):
        for h in range(Hq):
            hk = h // 2
            sr = kr[b, hk] @ q[b, h] / math.sqrt(d)
            np.testing.assert_allclose(only_r[b, h], scipy.special.softmax(sr) @ vr[b, hk], atol=1e-13)
            Kh = oracle.dequantize_head(kc["idx"][b, hk], kc["s1"][b, hk], kc["s2p"][b, hk], kc["o"][b, hk], C, g)
            lq = scipy.special.logsumexp(Kh @ q[b, h] / math.sqrt(d))
            lr = scipy.special.logsumexp(sr)
            wq = 1.0 / (1.0 + math.exp(lr - lq))
            np.testing.assert_allclose(both[b, h], wq * quant[b, h] + (1 - wq) * only_r[b, h], atol=1e-12)
    kd = kr.copy()
    kd[0, 1, 3] = 400.0 * q[0, 2] / np.linalg.norm(q[0, 2])
    dom = oracle.decode_attention_residual(q, *_args(kc, vc), C, g, kd, vr)
    np.testing.assert_allclose(dom[0, 2], vr[0, 1, 3], atol=1e-12)


# ---------------------------------------------------------------- RNG + codebook
def test_splitmix64_published_vector():
    # first outputs of SplitMix64 seeded with 1234567 (reference test vector)
    assert [int(v) for v in oracle.splitmix64(1234567, 0, 5)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]
    assert np.array_equal(oracle.splitmix64(99, 7, 3), oracle.splitmix64(99, 0, 10)[7:])


def test_normal_stream_is_standard_normal_and_sliceable():
    z = oracle.normal_stream(12345, 0, 1 << 18)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert scipy.stats.kstest(z[:50000], "norm").pvalue > 1e-3
    assert np.array_equal(oracle.normal_stream(12345, 5, 9), z[5:14])
    assert np.array_equal(oracle.normal_stream(12345, 6, 4), z[6:10])


def test_kmeans_scalar_lloyd_max_levels():
    """g = 1 k-means on N(0,1) approaches the Lloyd-Max quantizers:
    2 levels +-sqrt(2/pi) (MSE 1 - 2/pi); 4 levels +-0.4528, +-1.5104 (MSE 0.1175)."""
    X = oracle.normal_stream(2024, 0, 1 << 20).reshape(-1, 1)
    C, it, _ = oracle.kmeans(X, 2, 100)
    np.testing.assert_allclose(np.sort(C[:, 0]), [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=4e-3)
    # sampling error of a 2^20-sample second moment is ~1.4e-3
    assert abs(oracle.codebook_distortion(X, C) - (1 - 2 / math.pi)) < 5e-3
    C4, _, _ = oracle.kmeans(X, 4, 300)
    np.testing.assert_allclose(np.sort(C4[:, 0]), [-1.5104, -0.4528, 0.4528, 1.5104], atol=1e-2)
    assert abs(oracle.codebook_distortion(X, C4) - 0.1175) < 4e-3


def test_kmeans_blobs_and_fixed_point():
    rng = np.random.default_rng(11)
    centers = np.array([[5.0, 0], [-5, 0], [0, 5]])
    X = np.concatenate([c + 0.1 * rng.standard_normal((100, 2)) for c in centers])
    X = X[rng.permutation(300)]
    C, it, conv = oracle.kmeans(X, 3, 50)
    assert conv
    got = C[np.argsort(C[:, 0] + 10 * C[:, 1])]
    ref = centers[np.argsort(centers[:, 0] + 10 * centers[:, 1])]
    np.testing.assert_allclose(got, ref, atol=0.05)
    idx, _, _ = oracle.nearest_centroid(X, C)
    for k in range(3):                                 # every centroid is its cell mean
        np.testing.assert_allclose(C[k], X[idx == k].mean(axis=0), atol=1e-12)


def test_kmeans_empty_cell_reseeded_with_farthest_sample():
    X = np.array([[0.0], [0.0], [0.1], [10.0]])       # first 2 samples coincide -> cell 1 empty
    C, it, _ = oracle.kmeans(X, 2, 1)
    assert C[1, 0] == 10.0


@pytest.mark.parametrize("g,lo,hi", [(4, 2.0 ** -4, 0.1175), (8, 0.25, 1 - 2 / math.pi)])
def test_stored_codebooks_distortion_bounds(g, lo, hi):
    """Shannon's Gaussian bound D >= 2^-2R (R = 8/g bits/dim) is a hard floor; the
    product of scalar Lloyd-Max codebooks (a valid 256-entry code) is beaten."""
    path = os.path.join(GOLDEN, f"codebook_g{g}.txt")
    if not os.path.exists(path):
        pytest.skip("stored codebook not generated yet")
    C, meta = load_codebook(g)
    assert C.shape == (256, g)
    assert np.array_equal(C, oracle.to_f16(C))             # fp16-exact entries
    X = oracle.normal_stream(777, 0, (1 << 16) * g).reshape(-1, g)   # held-out samples
    D = oracle.codebook_distortion(X, C)
    assert lo < D < hi
    assert abs(float(meta["distortion_per_dim"]) - D) < 5e-3


# ---------------------------------------------------------------- cosine fine-tune
def test_cosine_loss_hand_example():
    # w = (3, 4, 0, 0) with g = 2: blocks (3, 4) -> centroid 0 = (1, 1), (0, 0) -> centroid 1 = (0, 1)
    # w_hat = (1, 1, 0, 1): <w, w_hat> = 7, |w| = 5, |w_hat| = sqrt(3): distance 1 - 7 / (5 sqrt 3)
    C = np.array([[1.0, 1.0], [0.0, 1.0]])
    W = np.array([[3.0, 4.0, 0.0, 0.0]])
    loss, _ = oracle.cosine_loss_grad(W, C, 2, np.array([[0, 1]]))
    assert abs(loss - (1 - 7 / (5 * math.sqrt(3)))) < 1e-15
    # nearest centroids: (3, 4) -> 0 (13 < 18), (0, 0) -> 1 (1 < 2)
    assert oracle.mean_cosine_distance(W, C, 2) == pytest.approx(loss, abs=1e-15)


def test_cosine_gradient_matches_finite_differences():
    """The analytic gradient (assignment held fixed) against central differences
    of the loss along random directions."""
    rng = np.random.default_rng(21)
    g, d, K, N = 4, 32, 16, 40
    W = rng.standard_normal((N, d))
    C = rng.standard_normal((K, g))
    idx = oracle.nearest_centroid(W.reshape(-1, g), C)[0].reshape(N, d // g)
    _, grad = oracle.cosine_loss_grad(W, C, g, idx)
    eps = 1e-6
    for _ in range(6):
        E = rng.standard_normal((K, g))
        lp, _ = oracle.cosine_loss_grad(W, C + eps * E, g, idx)
        lm, _ = oracle.cosine_loss_grad(W, C - eps * E, g, idx)
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - np.sum(grad * E)) < 1e-8 * max(1.0, abs(fd))


def test_cosine_gradient_is_scale_free():
    """The cosine is invariant to scaling the codebook, so the gradient is
    orthogonal to it: sum_k <grad_k, C_k> = 0."""
    rng = np.random.default_rng(22)
    W = rng.standard_normal((64, 128))
    C, _ = load_codebook(4)
    idx = oracle.nearest_centroid(W.reshape(-1, 4), C)[0].reshape(64, 32)
    _, grad = oracle.cosine_loss_grad(W, C, 4, idx)
    assert abs(np.sum(grad * C)) < 1e-14 * np.linalg.norm(grad) * np.linalg.norm(C) + 1e-18
    l1, _ = oracle.cosine_loss_grad(W, C, 4, idx)
    l2, _ = oracle.cosine_loss_grad(W, 3.7 * C, 4, idx)
    assert abs(l1 - l2) < 1e-14


def test_sign_quantizer_mean_cosine_closed_form():
    """g = 1, K = 2 with centroids -c, +c quantizes w to c sign(w) for any c > 0; its
    cosine to w is |w|_1 / (sqrt(d) |w|_2), whose mean over N(0, I_d) is
    sqrt(d) E|u_1| = sqrt(d) Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)) (u uniform on
    the sphere)."""
    d, N = 128, 4096
    W = oracle.normal_stream(31, 0, N * d).reshape(N, d)
    expect = 1 - math.sqrt(d) * math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    for c in (0.5, 2.0):
        got = oracle.mean_cosine_distance(W, np.array([[-c], [c]]), 1)
        # the per-vector cosine has std ~ 0.034 at d = 128: 5 sigma of the mean of N
        assert abs(got - expect) < 5 * 0.034 / math.sqrt(N)


def test_cosine_finetune_descends():
    """Small steps of the fine-tune lower the training loss monotonically, and the
    step taken is -lr times the gradient of the first iterate."""
    C0, _ = load_codebook(8)
    C, _, losses = oracle.cosine_finetune(C0, 8, 5, 2048, 6, 100.0)
    assert np.all(np.diff(losses) < 0)
    C1, _, _ = oracle.cosine_finetune(C0, 8, 5, 2048, 1, 100.0)
    W = oracle.normal_stream(5, 0, 2048 * 128).reshape(2048, 128)
    idx = oracle.nearest_centroid(W.reshape(-1, 8), C0)[0].reshape(2048, 16)
    np.testing.assert_allclose(C1, C0 - 100.0 * oracle.cosine_loss_grad(W, C0, 8, idx)[1], atol=1e-15)


@pytest.mark.parametrize("g", [4, 8])
def test_stored_finetuned_codebook_lowers_heldout_cosine(g):
    """The stored fine-tuned codebook beats the k-means one it started from on
    held-out vectors (a stream seed neither step saw), and keeps the distortion
    bounds of the k-means codebook."""
    Ck, _ = load_codebook(g)
    Cf, meta = load_codebook(g, finetuned=True)
    assert int(meta["seed"]) != 4242
    Wh = oracle.normal_stream(4242, 0, 16384 * 128).reshape(16384, 128)
    dk = oracle.mean_cosine_distance(Wh, Ck, g)
    df = oracle.mean_cosine_distance(Wh, Cf, g)
    assert df < dk
    X = oracle.normal_stream(4243, 0, (1 << 16) * g).reshape(-1, g)
    D = oracle.codebook_distortion(X, Cf)
    assert 2.0 ** (-2 * 8 / g) < D < (0.1175 if g == 4 else 0.3634)


# ---------------------------------------------------------------- double quantization
def test_f16_bits_known_patterns():
    assert list(oracle.f16_bits([1.0, 2.0, 0.5, 65504.0, 2.0 ** -24, 0.0])) == [0x3C00, 0x4000, 0x3800, 0x7BFF, 1, 0]
    assert list(oracle.f16_from_bits([0x3C00, 0x3555])) == [1.0, float(np.float16(1.0 / 3.0))]


def test_dq_o_grid_and_bounds():
    # o on the grid of its own scale comes back exactly; the extreme maps to +-7
    o = np.array([7.0, -3.0, 0.0, 1.0, -7.0]) * 0.25
    codes, scale, oq = oracle.dq_o(o)
    assert scale == 0.25 and list(codes) == [7, -3, 0, 1, -7] and np.array_equal(oq, o)
    rng = np.random.default_rng(41)
    o = rng.standard_normal(128)
    codes, scale, oq = oracle.dq_o(o)
    assert np.max(np.abs(codes)) == 7 and np.all(np.abs(codes) <= 7)
    assert np.max(np.abs(oq - o)) <= scale / 2 * (1 + 1e-6)
    assert oracle.dq_o(np.zeros(8))[1] == 0.0
    # exact midpoints (decided in fp64) go to the even code
    codes, scale, _ = oracle.dq_o(np.array([7.0, 2.5, 0.5, -1.5, -2.5]) * 0.25)
    assert scale == 0.25 and list(codes) == [7, 2, 0, -2, -2]


def test_dq_s1_grid():
    # equal scales: stride 1 and the fp16 value itself; zero token -> code 0
    c = oracle.dq_s1_codes(np.array([1.5, 1.5, 0.0]), *oracle.dq_s1_params(np.array([1.5, 1.5, 0.0])))
    assert list(c) == [1, 1, 0]
    base, stride = oracle.dq_s1_params(np.array([1.5, 0.0]))
    assert oracle.dq_s1_values(np.array([1, 0]), base, stride).tolist() == [1.5, 0.0]
    # hand example: patterns 0x3C00 (1.0) .. 0x4000 (2.0) span 1024: stride ceil(1024/14) = 74
    s1 = np.array([1.0, 2.0, 1.25])
    base, stride = oracle.dq_s1_params(s1)
    assert (base, stride) == (0x3C00, 74)
    codes = oracle.dq_s1_codes(s1, base, stride)
    # 1.25 = 0x3D00: offset 256 = 3.46 strides -> code 1 + 3 = 4 (value pattern 0x3C00 + 222)
    assert list(codes) == [1, 15, 4]
    vals = oracle.dq_s1_values(codes, base, stride)
    assert vals[0] == 1.0 and vals[2] == float(oracle.f16_from_bits([0x3C00 + 3 * 74])[0])
    assert vals[1] >= 2.0 and int(oracle.f16_bits(vals[1])) == 0x3C00 + 14 * 74
    # monotone, clamped for values outside the range (appended tokens)
    s = np.geomspace(0.1, 40.0, 200)
    cs = oracle.dq_s1_codes(s, 0x3C00, 74)
    assert np.all(np.diff(cs) >= 0) and cs[0] == 1 and cs[-1] == 15


def test_dq_codebook_levels():
    rng = np.random.default_rng(42)
    C = rng.standard_normal((256, 4))
    k, D, Cq = oracle.dq_codebook(C)
    assert k.min() >= 0 and k.max() <= 15 and len(np.unique(k)) <= 16
    assert D == pytest.approx(np.max(np.abs(C)) / 7.5, rel=1e-7)
    # nearest mid-rise level, up to the fp16 rounding of the level value
    assert np.max(np.abs(Cq - C)) <= D / 2 * (1 + 1e-6) + 2.0 ** -11 * 4
    # idempotent: the levels of the quantized codebook are themselves
    k2, D2, Cq2 = oracle.dq_codebook(Cq)
    assert np.array_equal(Cq2, Cq)


def test_dq_encode_reconstructs_before_vq():
    """With the quantized s1 and o used by the encoding, x = s1_q (s2 u + o_q)
    holds exactly before the vector quantization, for computed and reused
    parameters, zero and degenerate tokens included."""
    rng = np.random.default_rng(43)
    x = rng.standard_normal((60, 128)) * rng.uniform(0.1, 30, (60, 1)) + 2.0
    x[5] = 0.0
    C, _ = load_codebook(4)
    r = oracle.encode_head_dq(x, C, 4)
    xr = r["s1q"][:, None] * (r["s2"][:, None] * r["u"] + r["o_q"][None, :])
    assert np.max(np.abs(xr - x)) < 1e-12 * np.max(np.abs(x))
    assert r["s1c"][5] == 0 and np.all(r["s1c"][np.arange(60) != 5] >= 1)
    # append with the stored parameters, including a token far outside the s1 range
    xa = np.concatenate([rng.standard_normal((3, 128)), 500 * rng.standard_normal((1, 128))])
    ra = oracle.encode_head_dq(xa, C, 4, dq=r["dq"])
    xr = ra["s1q"][:, None] * (ra["s2"][:, None] * ra["u"] + ra["o_q"][None, :])
    assert np.max(np.abs(xr - xa)) < 1e-12 * np.max(np.abs(xa))
    # dequantization from the stored fields uses the same parameters
    xh = oracle.dequantize_head_dq(r["idx"], r["s1c"], r["s2p"], r["dq"], C, 4)
    np.testing.assert_allclose(xh, oracle.dequantize_head(r["idx"], r["s1q"], r["s2p"], r["o_q"], C, 4), atol=1e-13)
    # the quantization error is the VQ error of the same order as without DQ
    e_dq = np.linalg.norm(xh - x) / np.linalg.norm(x)
    p = oracle.encode_head(x, C, 4)
    e = np.linalg.norm(oracle.dequantize_head(p["idx"], p["s1"], p["s2p"], p["o"], C, 4) - x) / np.linalg.norm(x)
    assert e_dq < 1.3 * e


def test_dq_decode_attention_equals_plain_decode_on_dequantized_parameters():
    rng = np.random.default_rng(44)
    C, _ = load_codebook(8)
    B, Hkv, Hq, S = 1, 2, 4, 40
    X = [rng.standard_normal((B, Hkv, S, 128)) * 2 + 1 for _ in range(2)]
    enc = [[oracle.encode_head_dq(X[t][0, h], C, 8) for h in range(Hkv)] for t in range(2)]
    st = lambda t, key: np.stack([enc[t][h][key] for h in range(Hkv)])[None]
    q = oracle.to_f16(rng.standard_normal((B, Hq, 128)))
    out = oracle.decode_attention_dq(q, st(0, "idx"), st(0, "s1c"), st(0, "s2p"), [[e["dq"] for e in enc[0]]],
                                     st(1, "idx"), st(1, "s1c"), st(1, "s2p"), [[e["dq"] for e in enc[1]]], C, 8)
    oq = lambda t: np.stack([enc[t][h]["o_q"] for h in range(Hkv)])[None]
    ref = oracle.decode_attention(q, st(0, "idx"), st(0, "s1q"), st(0, "s2p"), oq(0),
                                  st(1, "idx"), st(1, "s1q"), st(1, "s2p"), oq(1), C, 8)
    np.testing.assert_allclose(out, ref, atol=1e-12)


# ---------------------------------------------------------------- keys before RoPE
def test_rope_hand_example_and_identities():
    # d = 4, base 100: theta = (1, 0.1); x = (1, 2, 3, 4) at position 1:
    # pair (x0, x2) by 1 rad, pair (x1, x3) by 0.1 rad
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    r = oracle.rope(x, [1], base=100.0)
    c1, s1, c2, s2 = math.cos(1), math.sin(1), math.cos(0.1), math.sin(0.1)
    np.testing.assert_allclose(r[0], [1 * c1 - 3 * s1, 2 * c2 - 4 * s2, 3 * c1 + 1 * s1, 4 * c2 + 2 * s2], atol=1e-15)
    rng = np.random.default_rng(61)
    X = rng.standard_normal((5, 128))
    np.testing.assert_allclose(oracle.rope(X, np.zeros(5)), X, atol=0)  # position 0 is the identity
    P = rng.integers(0, 100000, 5)
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(X, P), axis=1), np.linalg.norm(X, axis=1), rtol=1e-13)
    # composition and the relative-position property that RoPE exists for
    np.testing.assert_allclose(oracle.rope(oracle.rope(X, P), P + 7), oracle.rope(X, 2 * P + 7), atol=1e-9)
    q, k = rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    a = float(oracle.rope(q, [1000])[0] @ oracle.rope(k, [990])[0])
    b = float(oracle.rope(q, [10])[0] @ oracle.rope(k, [0])[0])
    assert abs(a - b) < 1e-10


def test_decode_attention_rope_reductions():
    """With every key position 0 the rotary score is the plain one; rotating the
    query back by p equals rotating every key forward by p."""
    rng = np.random.default_rng(62)
    B, Hq, Hkv, S, d, g = 1, 4, 2, 21, 128, 4
    C, kc, vc = _random_cache(rng, B, Hkv, S, d, g)
    q = oracle.to_f16(rng.standard_normal((B, Hq, d)))
    out = oracle.decode_attention_rope(q, *_args(kc, vc), C, g)
    for h in range(Hq):
        hk = h // 2
        K = oracle.dequantize_head(kc["idx"][0, hk], kc["s1"][0, hk], kc["s2p"][0, hk], kc["o"][0, hk], C, g)
        V = oracle.dequantize_head(vc["idx"][0, hk], vc["s1"][0, hk], vc["s2p"][0, hk], vc["o"][0, hk], C, g)
        sc = np.array([float(oracle.rope(q[0, h][None], [-i])[0] @ K[i]) for i in range(S)]) / math.sqrt(d)
        np.testing.assert_allclose(out[0, h], scipy.special.softmax(sc) @ V, atol=1e-12)
    one = {k_: v_[:, :, :1] for k_, v_ in kc.items() if k_ != "o"} | {"o": kc["o"]}
    onev = {k_: v_[:, :, :1] for k_, v_ in vc.items() if k_ != "o"} | {"o": vc["o"]}
    np.testing.assert_allclose(oracle.decode_attention_rope(q, *_args(one, onev), C, g),
                               oracle.decode_attention(q, *_args(one, onev), C, g), atol=1e-13)


# ---------------------------------------------------------------- randomized Hadamard (random signs)
def test_signs_from_mask_bit_order():
    mask = bytes([0b00000101] + [0] * 14 + [0b10000000])
    s = oracle.signs_from_mask(mask)
    neg = np.flatnonzero(s < 0)
    assert list(neg) == [0, 2, 127]
    assert np.all(np.abs(s) == 1.0)
    assert np.array_equal(oracle.signs_from_mask(bytes(16)), np.ones(128))
    assert np.array_equal(oracle.signs_from_mask(bytes([255] * 16)), -np.ones(128))


def test_randomized_rotation_is_orthonormal_and_inverted():
    rng = np.random.default_rng(71)
    s = oracle.signs_from_mask(rng.integers(0, 256, 16, dtype=np.uint8))
    H = oracle.hadamard_orthonormal(128)
    M = H @ np.diag(s)  # w = H D u
    np.testing.assert_allclose(M @ M.T, np.eye(128), atol=1e-14)
    u = rng.standard_normal((6, 128))
    w = oracle.rotate(u, s)
    np.testing.assert_allclose(w, (M @ u.T).T, atol=1e-13)
    np.testing.assert_allclose(oracle.unrotate(w, s), u, atol=1e-13)
    np.testing.assert_allclose(oracle.rotate(u, np.ones(128)), oracle.rotate(u), atol=0)
    # a sign pattern that is not symmetric under H: D H != H D
    assert np.max(np.abs(oracle.unrotate(w, s) - oracle.rotate(w, s))) > 1e-3


def test_randomized_encode_equals_plain_encode_of_sign_flipped_input():
    """H D (NSN(x)) = H NSN(D x): the two norms are unchanged by D and the
    channel mean flips with it, so the codes and scales of encode(x, D) are those
    of plain encode(D x) and the stored shift is D times that one's."""
    rng = np.random.default_rng(72)
    C, _ = load_codebook(4)
    s = oracle.signs_from_mask(rng.integers(0, 256, 16, dtype=np.uint8))
    x = rng.standard_normal((30, 128)) * 2 + rng.standard_normal(128)
    r = oracle.encode_head(x, C, 4, signs=s)
    p = oracle.encode_head(x * s, C, 4)
    assert np.array_equal(r["idx"], p["idx"])
    np.testing.assert_array_equal(r["s1"], p["s1"])
    np.testing.assert_array_equal(r["s2p"], p["s2p"])
    np.testing.assert_array_equal(r["o"], p["o"] * s)
    # dequantization inverts the rotation with D H: x_hat(x, D) = D x_hat_plain(D x)
    xr = oracle.dequantize_head(r["idx"], r["s1"], r["s2p"], r["o"], C, 4, s)
    xp = oracle.dequantize_head(p["idx"], p["s1"], p["s2p"], p["o"], C, 4)
    np.testing.assert_allclose(xr, xp * s, atol=1e-12)
    # and with the lossless codebook the round trip returns x
    w = oracle.rotate(oracle.nsn_forward(x[:8, :16])["u"], s[:16])
    Cl = oracle.subvectors(w, 4).reshape(-1, 4)
    rl = oracle.encode_head(x[:8, :16], Cl, 4, signs=s[:16])
    np.testing.assert_allclose(oracle.dequantize_head(rl["idx"], rl["s1_exact"], rl["s2p_exact"], rl["o_exact"],
                                                      Cl, 4, s[:16]), x[:8, :16], rtol=1e-11, atol=1e-11)


def test_randomized_decode_equals_plain_decode_of_flipped_query():
    """With x_hat = D (s1 (s2' H w_hat + D o)), the rotated cache is D times the
    plain cache whose shift is D o: scores q . D k = (D q) . k and the output is D
    times the plain output."""
    rng = np.random.default_rng(73)
    B, Hq, Hkv, S, d, g = 1, 4, 2, 23, 128, 4
    C, kc, vc = _random_cache(rng, B, Hkv, S, d, g)
    s = oracle.signs_from_mask(rng.integers(0, 256, 16, dtype=np.uint8))
    q = oracle.to_f16(rng.standard_normal((B, Hq, d)))
    out = oracle.decode_attention(q, *_args(kc, vc), C, g, signs=s)
    flip = lambda c: {k_: v_ for k_, v_ in c.items() if k_ != "o"} | {"o": c["o"] * s}
    ref = oracle.decode_attention(q * s, *_args(flip(kc), flip(vc)), C, g) * s
    np.testing.assert_allclose(out, ref, atol=1e-12)
    for h in range(Hq):
        K = oracle.dequantize_head(kc["idx"][0, h // 2], kc["s1"][0, h // 2], kc["s2p"][0, h // 2],
                                   kc["o"][0, h // 2], C, g, s)
        V = oracle.dequantize_head(vc["idx"][0, h // 2], vc["s1"][0, h // 2], vc["s2p"][0, h // 2],
                                   vc["o"][0, h // 2], C, g, s)
        np.testing.assert_allclose(out[0, h], scipy.special.softmax(K @ q[0, h] / math.sqrt(d)) @ V, atol=1e-12)
    rr = oracle.decode_attention_rope(q, *_args(kc, vc), C, g, signs=s)
    one = {k_: v_[:, :, :1] for k_, v_ in kc.items() if k_ != "o"} | {"o": kc["o"]}
    onev = {k_: v_[:, :, :1] for k_, v_ in vc.items() if k_ != "o"} | {"o": vc["o"]}
    np.testing.assert_allclose(oracle.decode_attention_rope(q, *_args(one, onev), C, g, signs=s),
                               oracle.decode_attention(q, *_args(one, onev), C, g, signs=s), atol=1e-13)
    assert not np.allclose(rr, out)
    # the residual window holds raw tokens: the signs touch only the quantized part
    empty = np.zeros((B, Hkv, 0, d))
    np.testing.assert_allclose(oracle.decode_attention_residual(q, *_args(kc, vc), C, g, empty, empty, signs=s),
                               out, atol=1e-13)
    kr = oracle.to_f16(rng.standard_normal((B, Hkv, 5, d)))
    vr = oracle.to_f16(rng.standard_normal((B, Hkv, 5, d)))
    none = dict(idx=kc["idx"][:, :, :0], s1=kc["s1"][:, :, :0], s2p=kc["s2p"][:, :, :0], o=kc["o"])
    np.testing.assert_allclose(oracle.decode_attention_residual(q, *_args(none, none), C, g, kr, vr, signs=s),
                               oracle.decode_attention_residual(q, *_args(none, none), C, g, kr, vr), atol=0)


def test_randomized_dq_encode_and_decode_follow_the_plain_ones():
    rng = np.random.default_rng(74)
    C, _ = load_codebook(8)
    s = oracle.signs_from_mask(rng.integers(0, 256, 16, dtype=np.uint8))
    x = rng.standard_normal((25, 128)) * 2 + 1
    r = oracle.encode_head_dq(x, C, 8, signs=s)
    p = oracle.encode_head_dq(x * s, C, 8)
    assert np.array_equal(r["idx"], p["idx"])
    np.testing.assert_array_equal(r["s2p"], p["s2p"])
    np.testing.assert_array_equal(r["s1c"], p["s1c"])
    np.testing.assert_array_equal(np.asarray(r["dq"]["o_codes"]), np.asarray(p["dq"]["o_codes"]) * s)
    xr = oracle.dequantize_head_dq(r["idx"], r["s1c"], r["s2p"], r["dq"], C, 8, s)
    xp = oracle.dequantize_head_dq(p["idx"], p["s1c"], p["s2p"], p["dq"], C, 8)
    np.testing.assert_allclose(xr, xp * s, atol=1e-12)
