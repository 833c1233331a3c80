"""GPU parity of the randomized Hadamard option (rotation H D, D = diag(+-1) from
a 16-byte channel mask) against the fp64 oracle, through the C ABI.

The signs are a seeded random draw passed as input.  Every call that takes the
codebook handle uses them: encode (plain and double-quantized), dequantize,
decode attention (plain, with a residual window, double-quantized, rotary) and
the fused append + decode step.  An all-zero mask must give the plain path's
bytes exactly.
"""

import numpy as np
import pytest

import oracle
import synthetic
from golden_io import have_codebook, load_codebook
from oracle.parity import (attention_ref_group, check_attention_rows, check_encode_head, check_encode_head_dq,
                           dq_head_from_bytes, gpu_to_np, s1_codes_from_bytes)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import kv_cache_vector_nsn_amd as nsn  # noqa: E402


def _log(msg):
    print(msg, flush=True)


MASK = bytes(np.random.default_rng(20250523).integers(0, 256, 16, dtype=np.uint8))
SIGNS = oracle.signs_from_mask(MASK)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsn.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def books(dev):
    out = {}
    for g in (4, 8):
        if not have_codebook(g):
            pytest.skip("stored codebooks missing")
        C, _ = load_codebook(g)
        out[g] = (C, nsn.nsn_codebook_create_rht(C.astype(np.float32), MASK, g),
                  nsn.nsn_codebook_create(C.astype(np.float32), g),
                  nsn.nsn_codebook_create_rht(C.astype(np.float32), bytes(16), g))
    return out


def _encode(cb, X, g, L_cap, garbage=True):
    B, H, L, d = X.shape
    if garbage:
        idx = torch.randint(0, 256, (B, H, L_cap, d // g), dtype=torch.uint8, device=X.device)
        sc = torch.full((B, H, L_cap, 2), float("nan"), dtype=torch.float16, device=X.device)
    else:
        idx = torch.zeros((B, H, L_cap, d // g), dtype=torch.uint8, device=X.device)
        sc = torch.zeros((B, H, L_cap, 2), dtype=torch.float16, device=X.device)
    o = torch.zeros((B, H, d), dtype=torch.float32, device=X.device)
    nsn.nsn_encode(cb, X, o, idx, sc)
    return idx, sc, o


def _host(idx, sc, o, S):
    s = gpu_to_np(sc)
    return (idx.cpu().numpy().astype(np.int64)[:, :, :S], s[:, :, :S, 0], s[:, :, :S, 1], gpu_to_np(o))


def test_sign_mask_round_trip(dev, books):
    _, cb, plain, zero = books[4]
    assert nsn.nsn_codebook_sign_mask(cb) == MASK
    assert nsn.nsn_codebook_sign_mask(plain) == bytes(16)
    assert nsn.nsn_codebook_sign_mask(zero) == bytes(16)
    assert 40 < int(np.sum(SIGNS < 0)) < 88  # a real mix of signs


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_rht_encode_matches_oracle(dev, books, g, dtype):
    """Ragged lengths, a zero token, tokens equal up to scale, a tensor of equal
    tokens (every shifted token degenerate); indices and scales as for the plain
    encode, against the oracle's H D rotation."""
    C, cb, _, _ = books[g]
    rep = {}
    for L in (1, 7, 33, 257, 1000):
        K, _ = synthetic.make_kv_numpy(2000 + L, 2, 2, L, 128, "outlier", dtype)
        if L >= 9:
            K[0, 1, 3] = 0
            K[1, 0, 6] = (2 * K[1, 0, 5].astype(np.float32)).astype(K.dtype)
        idx, sc, o = _encode(cb, torch.from_numpy(K).to(dev), g, L + 3)
        torch.cuda.synchronize()
        hc = _host(idx, sc, o, L)
        for b in range(2):
            for h in range(2):
                check_encode_head(K[b, h].astype(np.float64), C, g, hc[0][b, h], hc[1][b, h], hc[2][b, h],
                                  hc[3][b, h], report=rep, signs=SIGNS)
    x = np.tile(np.random.default_rng(3).standard_normal(128).astype(np.float16), (1, 1, 12, 1))
    idx, sc, o = _encode(cb, torch.from_numpy(x).to(dev), g, 12)
    torch.cuda.synchronize()
    hc = _host(idx, sc, o, 12)
    r = check_encode_head(x[0, 0].astype(np.float64), C, g, hc[0][0, 0], hc[1][0, 0], hc[2][0, 0], hc[3][0, 0],
                          signs=SIGNS)
    assert r["degenerate"] == 12
    _log(f"rht encode g={g} {dtype}: {rep}")


@pytest.mark.parametrize("g", [4, 8])
def test_zero_mask_is_the_plain_path(dev, books, g):
    """An all-zero mask writes the plain codebook's bytes and decodes to the same
    bits; the random mask changes the codes."""
    C, cb, plain, zero = books[g]
    K, V = synthetic.make_kv_numpy(77 + g, 1, 2, 300, 128, "outlier", "f16")
    Xk, Xv = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    a = [_encode(plain, X, g, 300, garbage=False) for X in (Xk, Xv)]
    z = [_encode(zero, X, g, 300, garbage=False) for X in (Xk, Xv)]
    r = [_encode(cb, X, g, 300, garbage=False) for X in (Xk, Xv)]
    q = synthetic.make_queries(5, 1, 8, 128, dev)
    outs = []
    for book, caches in ((plain, a), (zero, z)):
        out = torch.empty((1, 8, 128), dtype=torch.float32, device=dev)
        nsn.nsn_decode_attention(book, q, caches[0], caches[1], out, 300)
        outs.append(out)
    torch.cuda.synchronize()
    for ta, tz in zip(a[0] + a[1], z[0] + z[1]):
        assert torch.equal(ta.view(torch.uint8) if ta.dtype != torch.uint8 else ta,
                           tz.view(torch.uint8) if tz.dtype != torch.uint8 else tz)
    assert torch.equal(outs[0], outs[1])
    assert not torch.equal(a[0][0], r[0][0])


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("GQ", [1, 4, 8])
def test_rht_decode_and_dequantize_match_oracle(dev, books, g, GQ):
    """Decode attention and dequantization over caches written with the signs;
    ragged S, garbage past S."""
    C, cb, _, _ = books[g]
    B, Hkv = 2, 2
    Hq = GQ * Hkv
    for S in (1, 33, 1000, 4099):
        _log(f"rht decode g={g} GQ={GQ} S={S}")
        K, V = synthetic.make_kv_numpy(3000 + S + GQ, B, Hkv, S, 128, "outlier", "f16")
        caches = [_encode(cb, torch.from_numpy(X).to(dev), g, S + 20) for X in (K, V)]
        q = synthetic.make_queries(S + GQ, B, Hq, 128, dev)
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        nsn.nsn_decode_attention(cb, q, caches[0], caches[1], out, S)
        xh = torch.empty((B, Hkv, S, 128), dtype=torch.float32, device=dev)
        nsn.nsn_dequantize(cb, caches[0][0], caches[0][1], caches[0][2], S, xh)
        torch.cuda.synchronize()
        kc, vc = _host(*caches[0], S), _host(*caches[1], S)
        on, qn = gpu_to_np(out), gpu_to_np(q)
        for b in range(B):
            for hk in range(Hkv):
                check_attention_rows(on[b, hk * GQ:(hk + 1) * GQ],
                                     attention_ref_group(qn, kc, vc, C, g, b, hk, GQ, S, signs=SIGNS))
        xr = oracle.dequantize_head(kc[0][1, 1], kc[1][1, 1], kc[2][1, 1], kc[3][1, 1], C, g, SIGNS)
        xg = gpu_to_np(xh)[1, 1]
        assert np.max(np.abs(xg - xr)) <= 1e-5 * max(1.0, np.max(np.abs(xr))), np.max(np.abs(xg - xr))


@pytest.mark.parametrize("g", [4, 8])
def test_rht_residual_window_and_step(dev, books, g):
    """A residual window in the same softmax (the window's raw tokens take no
    signs), then a fused append + decode step."""
    C, cb, _, _ = books[g]
    B, Hkv, GQ, S, R, R_cap = 2, 2, 4, 700, 19, 32
    Hq = GQ * Hkv
    K, V = synthetic.make_kv_numpy(4000 + g, B, Hkv, S + 1, 128, "outlier", "f16")
    caches = [_encode(cb, torch.from_numpy(np.ascontiguousarray(X[:, :, :S])).to(dev), g, S + 8) for X in (K, V)]
    Kr, Vr = synthetic.make_kv_numpy(4100 + g, B, Hkv, R_cap, 128, "normal", "f16")
    Kr[:, :, R:] = np.nan
    Vr[:, :, R:] = np.nan
    q = synthetic.make_queries(4000 + g, B, Hq, 128, dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    nsn.nsn_decode_attention_residual(cb, q, caches[0], caches[1], torch.from_numpy(Kr).to(dev),
                                      torch.from_numpy(Vr).to(dev), out, S, R)
    torch.cuda.synchronize()
    kc, vc = _host(*caches[0], S), _host(*caches[1], S)
    ref = oracle.decode_attention_residual(gpu_to_np(q), *kc, *vc, C, g, Kr[:, :, :R].astype(np.float64),
                                           Vr[:, :, :R].astype(np.float64), signs=SIGNS)
    on = gpu_to_np(out)
    for b in range(B):
        check_attention_rows(on[b], ref[b])
    # append token S (stored o reused) and attend over S + 1
    kn = torch.from_numpy(np.ascontiguousarray(K[:, :, S])).to(dev)
    vn = torch.from_numpy(np.ascontiguousarray(V[:, :, S])).to(dev)
    nsn.nsn_decode_step(cb, q, kn, vn, caches[0], caches[1], out, S)
    torch.cuda.synchronize()
    kc, vc = _host(*caches[0], S + 1), _host(*caches[1], S + 1)
    for X, hc in ((K, kc), (V, vc)):
        for b in range(B):
            for h in range(Hkv):
                check_encode_head(X[b, h, S:S + 1].astype(np.float64), C, g, hc[0][b, h, S:], hc[1][b, h, S:],
                                  hc[2][b, h, S:], hc[3][b, h], o_given=hc[3][b, h], signs=SIGNS)
    on, qn = gpu_to_np(out), gpu_to_np(q)
    for b in range(B):
        for hk in range(Hkv):
            check_attention_rows(on[b, hk * GQ:(hk + 1) * GQ],
                                 attention_ref_group(qn, kc, vc, C, g, b, hk, GQ, S + 1, signs=SIGNS))


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("GQ", [1, 4])
def test_rht_rope_matches_oracle(dev, books, g, GQ):
    C, cb, _, _ = books[g]
    B, Hkv = 1, 2
    Hq = GQ * Hkv
    for S, base in ((1, 10000.0), (300, 1e6), (2049, 10000.0)):
        _log(f"rht rope g={g} GQ={GQ} S={S}")
        K, V = synthetic.make_kv_numpy(5000 + S + GQ, B, Hkv, S, 128, "normal", "f16")
        caches = [_encode(cb, torch.from_numpy(X).to(dev), g, S + 5) for X in (K, V)]
        q = synthetic.make_queries(S, B, Hq, 128, dev)
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
        nsn.nsn_decode_attention_rope(cb, q, caches[0], caches[1], out, S, rope_base=base)
        torch.cuda.synchronize()
        kc, vc = _host(*caches[0], S), _host(*caches[1], S)
        ref = oracle.decode_attention_rope(gpu_to_np(q), *kc, *vc, C, g, base, signs=SIGNS)
        on = gpu_to_np(out)
        for b in range(B):
            check_attention_rows(on[b], ref[b])


def _dq_cache(dev, B, H, L_cap, g):
    idx = torch.randint(0, 256, (B, H, L_cap, 128 // g), dtype=torch.uint8, device=dev)
    s2 = torch.full((B, H, L_cap), float("nan"), dtype=torch.float16, device=dev)
    s1c = torch.randint(0, 256, (B, H, (L_cap + 1) // 2), dtype=torch.uint8, device=dev)
    head = torch.randint(0, 256, (B, H, nsn.DQ_HEAD_BYTES), dtype=torch.uint8, device=dev)
    return idx, s2, s1c, head


def _dq_host(cache, L):
    idx, s2, s1c, head = cache
    B, H = idx.shape[:2]
    hb, cbytes = head.cpu().numpy(), s1c.cpu().numpy()
    heads = [[dq_head_from_bytes(hb[b, h]) for h in range(H)] for b in range(B)]
    codes = np.stack([np.stack([s1_codes_from_bytes(cbytes[b, h], L) for h in range(H)]) for b in range(B)])
    return idx.cpu().numpy().astype(np.int64)[:, :, :L], codes, gpu_to_np(s2)[:, :, :L], heads


@pytest.mark.parametrize("g", [4, 8])
def test_rht_dq_encode_and_decode_match_oracle(dev, books, g):
    C, cb, _, _ = books[g]
    B, Hkv, GQ = 1, 2, 4
    for S in (33, 1500):
        _log(f"rht dq g={g} S={S}")
        K, V = synthetic.make_kv_numpy(6000 + S, B, Hkv, S, 128, "outlier", "f16")
        caches = []
        for X in (K, V):
            c = _dq_cache(dev, B, Hkv, S + 7, g)
            nsn.nsn_encode_dq(cb, torch.from_numpy(X).to(dev), c)
            caches.append(c)
        q = synthetic.make_queries(S, B, GQ * Hkv, 128, dev)
        out = torch.empty((B, GQ * Hkv, 128), dtype=torch.float32, device=dev)
        nsn.nsn_decode_attention_dq(cb, q, caches[0], caches[1], out, S)
        torch.cuda.synchronize()
        kh, vh = _dq_host(caches[0], S), _dq_host(caches[1], S)
        for X, hh in ((K, kh), (V, vh)):
            for h in range(Hkv):
                check_encode_head_dq(X[0, h].astype(np.float64), C, g, hh[0][0, h], hh[1][0, h], hh[2][0, h],
                                     hh[3][0][h], signs=SIGNS)
        ref = oracle.decode_attention_dq(gpu_to_np(q), *kh, *vh, C, g, signs=SIGNS)
        check_attention_rows(gpu_to_np(out)[0], ref[0])


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("GQ", [1, 4])
def test_rope_prepared_tables_match_per_call(dev, books, g, GQ):
    """cos / sin tables built once (nsn_rope_tables) and passed to the decode give
    the per-call decode's output bit for bit, for tables sized exactly to S and
    longer ones (more coarse rows than S reads), shared by a codebook with a sign
    mask and one without; the masked codebook's output also against the oracle."""
    C, cb_r, cb_p, _ = books[g]
    B, Hkv = 2, 2
    Hq = GQ * Hkv
    base = 5e5
    tabs = {S_tab: nsn.nsn_rope_tables(S_tab, rope_base=base, device=dev) for S_tab in (300, 2049, 4096)}
    for S in (1, 257, 300, 2049):
        K, V = synthetic.make_kv_numpy(6000 + S + GQ, B, Hkv, S, 128, "normal", "f16")
        q = synthetic.make_queries(S + 1, B, Hq, 128, dev)
        for cb, signs in ((cb_r, SIGNS), (cb_p, None)):
            caches = [_encode(cb, torch.from_numpy(X).to(dev), g, S + 3) for X in (K, V)]
            ref_out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
            nsn.nsn_decode_attention_rope(cb, q, caches[0], caches[1], ref_out, S, rope_base=base)
            for S_tab, tab in tabs.items():
                if S_tab < S:
                    continue
                _log(f"rope tables g={g} GQ={GQ} S={S} S_tab={S_tab} signs={signs is not None}")
                out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev)
                nsn.nsn_decode_attention_rope_tables(cb, q, caches[0], caches[1], out, S, tab, S_tab)
                torch.cuda.synchronize()
                assert torch.equal(out, ref_out), (S, S_tab)
            if signs is not None:
                kc, vc = _host(*caches[0], S), _host(*caches[1], S)
                ref = oracle.decode_attention_rope(gpu_to_np(q), *kc, *vc, C, g, base, signs=signs)
                on = gpu_to_np(ref_out)
                for b in range(B):
                    check_attention_rows(on[b], ref[b])
