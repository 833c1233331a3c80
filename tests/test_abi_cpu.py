"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and its host-side validation returns the documented status codes
before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_vector_nsn_amd as nsn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsn.h")

OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nsn_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nsn.LIB_PATH):
        pytest.skip("libnsn.so not built")
    return nsn.lib()


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for n in ["nsn_build_codebook", "nsn_codebook_create", "nsn_encode", "nsn_decode_attention",
              "nsn_decode_attention_residual", "nsn_decode_step", "nsn_dequantize", "nsn_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert L.nsn_version() == 10000


def test_search_grid_edges(L):
    """The g = 4 candidate grid: 21 ascending edges over [-4, 4], mirror
    symmetric, a step of 0.4; a short buffer is rejected."""
    e = np.asarray(nsn.nsn_search_grid_edges())
    assert len(e) == 21 and e[0] == -4.0 and e[-1] == 4.0 and e[10] == 0.0
    assert np.array_equal(e, -e[::-1])
    assert np.allclose(np.diff(e), 0.4, rtol=0, atol=1e-6)
    buf = (ctypes.c_float * 20)()
    assert L.nsn_search_grid_edges(buf, 20) == EINVAL
    assert L.nsn_search_grid_edges(None, 64) == EINVAL


def test_codebook_create_rejects_bad_input_before_hip(L):
    h = ctypes.c_void_p()
    c = np.zeros((256, 4), np.float32)
    assert L.nsn_codebook_create(None, 4, 256, ctypes.byref(h)) == EINVAL
    assert L.nsn_codebook_create(c.ctypes.data, 5, 256, ctypes.byref(h)) == EUNSUP
    assert L.nsn_codebook_create(c.ctypes.data, 4, 128, ctypes.byref(h)) == EUNSUP
    c[3, 1] = 0.1  # 0.1 is not an fp16 value
    assert L.nsn_codebook_create(c.ctypes.data, 4, 256, ctypes.byref(h)) == EINVAL
    assert b"fp16" in L.nsn_last_error()
    c[3, 1] = np.nan
    assert L.nsn_codebook_create(c.ctypes.data, 4, 256, ctypes.byref(h)) == EINVAL
    # the randomized-Hadamard variant: a missing mask, then the same centroid checks
    mask = (ctypes.c_uint8 * 16)()
    assert L.nsn_codebook_create_rht(c.ctypes.data, 4, 256, None, ctypes.byref(h)) == EINVAL
    assert L.nsn_codebook_create_rht(c.ctypes.data, 4, 256, mask, None) == EINVAL
    assert L.nsn_codebook_create_rht(c.ctypes.data, 4, 256, mask, ctypes.byref(h)) == EINVAL  # the NaN entry
    c[3, 1] = 0.0
    assert L.nsn_codebook_create_rht(c.ctypes.data, 5, 256, mask, ctypes.byref(h)) == EUNSUP
    assert L.nsn_codebook_sign_mask(None, mask) == EINVAL


def test_build_codebook_rejects_bad_input(L):
    c = np.zeros((256, 8), np.float32)
    assert L.nsn_build_codebook(1, 8, 256, 1 << 10, 10, None, None, None) == EINVAL
    assert L.nsn_build_codebook(1, 6, 256, 1 << 10, 10, c.ctypes.data, None, None) == EUNSUP
    assert L.nsn_build_codebook(1, 8, 255, 1 << 10, 10, c.ctypes.data, None, None) == EUNSUP
    assert L.nsn_build_codebook(1, 8, 256, 100, 10, c.ctypes.data, None, None) == EINVAL
    assert L.nsn_build_codebook(1, 8, 256, 1 << 10, 0, c.ctypes.data, None, None) == EINVAL


def test_finetune_codebook_rejects_bad_input(L):
    C = np.zeros((256, 4), dtype=np.float32)
    out = np.zeros((256, 4), dtype=np.float32)
    f = lambda c=C.ctypes.data, g=4, K=256, n=1024, it=3, lr=1.0, o=out.ctypes.data: L.nsn_finetune_codebook(
        c, g, K, 1, n, it, lr, o, None, None)
    assert f(c=None) == EINVAL and f(o=None) == EINVAL
    assert f(g=5) == EUNSUP and f(K=128) == EUNSUP
    assert f(n=0) == EINVAL and f(n=(1 << 22) + 1) == EUNSUP
    assert f(it=-1) == EINVAL and f(lr=-1.0) == EINVAL and f(lr=float("nan")) == EINVAL
    bad = C.copy()
    bad[3, 1] = np.inf
    assert f(c=bad.ctypes.data) == EINVAL


def test_codebook_dq4_matches_oracle(L):
    """The library's 4-bit codebook routine (host code) against the oracle's, bit
    for bit, on the stored codebooks and a random one with exact level ties."""
    import oracle
    from golden_io import load_codebook

    rng = np.random.default_rng(5)
    Cr = rng.standard_normal((256, 4))
    D = float(np.float32(np.max(np.abs(Cr)) / 7.5))
    Cr[:8, 0] = (np.arange(8) - 3.0) * D  # entries on level boundaries (k - 8) D
    for C in (load_codebook(4)[0], load_codebook(8)[0], oracle.to_f32(Cr)):
        codes, step, Cq = nsn.nsn_codebook_dq4(C.astype(np.float32))
        k, Do, Cqo = oracle.dq_codebook(C)
        assert step == Do and np.array_equal(codes, k) and np.array_equal(Cq.astype(np.float64), Cqo)
    with pytest.raises(nsn.NSNError):
        nsn.nsn_codebook_dq4(np.full((4, 4), np.nan, dtype=np.float32))


def test_workspace_queries(L):
    assert L.nsn_encode_workspace_size(1, 8, 4096, 128) > 0
    assert L.nsn_encode_workspace_size(1, 8, 4096, 64) == 0
    assert L.nsn_encode_workspace_size(0, 8, 4096, 128) == 0
    assert L.nsn_decode_workspace_size(16, 32, 8, 32768, 128) > 0
    assert L.nsn_decode_workspace_size(16, 30, 8, 32768, 128) == 0
    # grows with the batch (per-query-head partials)
    assert L.nsn_decode_workspace_size(32, 32, 8, 32768, 128) >= L.nsn_decode_workspace_size(16, 32, 8, 32768, 128)


P = 0x1000  # any non-NULL pointer value; the checks never dereference it


def enc(L, g=4, x=P, dt=0, B=1, H=8, Lt=64, Lc=64, pos0=0, d=128, om=0, o=P, idx=P, sc=P, ws=P, wsb=1 << 30):
    return L.nsn_check_encode_args(g, x, dt, B, H, Lt, Lc, pos0, d, om, o, idx, sc, ws, wsb)


def test_encode_validation_codes(L):
    assert enc(L) == OK
    assert enc(L, B=255, H=257, Lt=1, Lc=1, ws=P) == OK       # B*H = 65535 grid rows
    assert enc(L, B=256, H=256, Lt=1, Lc=1, ws=P) == EUNSUP
    assert enc(L, g=8, dt=1) == OK
    assert enc(L, x=None) == EINVAL
    assert enc(L, o=None) == EINVAL
    assert enc(L, idx=None) == EINVAL
    assert enc(L, sc=None) == EINVAL
    assert enc(L, B=0) == EINVAL
    assert enc(L, Lt=0) == EINVAL
    assert enc(L, d=64) == EUNSUP
    assert enc(L, g=2) == EUNSUP
    assert enc(L, dt=7) == EINVAL
    assert enc(L, om=3) == EINVAL
    assert enc(L, Lt=65, Lc=64) == EINVAL                 # tokens beyond capacity
    assert enc(L, pos0=1, Lt=8, Lc=64) == OK              # COMPUTE at any pos0: a block encoded on its own
    assert enc(L, pos0=57, Lt=8, Lc=64) == EINVAL
    assert enc(L, om=1, pos0=63, Lt=1, Lc=64, ws=None, wsb=0) == OK   # REUSE append needs no workspace
    assert enc(L, om=1, pos0=64, Lt=1, Lc=64, ws=None, wsb=0) == EINVAL
    assert enc(L, ws=None) == EWS
    need = L.nsn_encode_workspace_size(1, 8, 64, 128)
    assert enc(L, wsb=need - 1) == EWS and enc(L, wsb=need) == OK


def dec(L, g=4, q=P, B=2, Hq=8, Hkv=2, S=100, Sc=128, d=128, ptrs=(P,) * 7, ws=P, wsb=1 << 30):
    return L.nsn_check_decode_args(g, q, B, Hq, Hkv, S, Sc, d, *ptrs, ws, wsb)


def test_decode_validation_codes(L):
    assert dec(L) == OK
    assert dec(L, q=None) == EINVAL
    for i in range(7):
        p = [P] * 7
        p[i] = None
        assert dec(L, ptrs=tuple(p)) == EINVAL
    assert dec(L, S=0) == EINVAL
    assert dec(L, S=129) == EINVAL                        # S > S_cap
    assert dec(L, Hq=6, Hkv=4) == EINVAL                  # Hq % Hkv
    assert dec(L, Hq=12, Hkv=4) == EUNSUP                 # group of 3
    assert dec(L, Hq=32, Hkv=2) == EUNSUP                 # group of 16
    assert dec(L, d=256) == EUNSUP
    assert dec(L, ws=None) == EWS
    need = L.nsn_decode_workspace_size(2, 8, 2, 100, 128)
    assert dec(L, wsb=need - 1) == EWS and dec(L, wsb=need) == OK
    assert dec(L, g=5) == EUNSUP
    # one (batch, KV head) index slab must stay below 2^31 bytes: S_cap * d / g
    assert dec(L, B=1, Hkv=1, Hq=4, S=100, Sc=2 ** 26 - 1) == OK
    assert dec(L, B=1, Hkv=1, Hq=4, S=100, Sc=2 ** 26) == EUNSUP
    assert dec(L, g=8, B=1, Hkv=1, Hq=4, S=100, Sc=2 ** 27 - 1) == OK
    assert dec(L, g=8, B=1, Hkv=1, Hq=4, S=100, Sc=2 ** 27) == EUNSUP


def res(L, g=4, q=P, B=2, Hq=8, Hkv=2, S=100, Sc=128, d=128, ptrs=(P,) * 7, kr=P, vr=P, R=5, Rc=32, ws=P,
        wsb=1 << 30):
    return L.nsn_check_decode_residual_args(g, q, B, Hq, Hkv, S, Sc, d, *ptrs[:6], kr, vr, R, Rc, ptrs[6], ws, wsb)


def test_decode_residual_validation_codes(L):
    assert res(L) == OK
    assert res(L, R=0) == OK                                # quantized part only
    need0 = L.nsn_decode_workspace_size(2, 8, 2, 0, 128)     # residual only: the window's partials
    assert need0 == 2 * 8 * 132 * 4
    assert res(L, S=0, Sc=0, ptrs=(None,) * 6 + (P,), wsb=need0) == OK  # no cache arrays
    assert res(L, S=0, Sc=0, ptrs=(None,) * 6 + (P,), ws=None, wsb=0) == EWS
    assert res(L, S=0, Sc=0, ptrs=(None,) * 6 + (P,), wsb=need0 - 1) == EWS
    assert res(L, S=0, R=0) == EINVAL                       # nothing to attend to
    assert res(L, R=33) == EINVAL and res(L, Rc=0, R=0) == EINVAL
    assert res(L, S=-1) == EINVAL and res(L, R=-1) == EINVAL
    assert res(L, kr=None) == EINVAL and res(L, vr=None) == EINVAL
    assert res(L, R=0, kr=None, vr=None) == OK              # residual pointers unused when R = 0
    assert res(L, S=0, q=None) == EINVAL
    assert res(L, S=0, Hq=12, Hkv=4) == EUNSUP and res(L, S=0, d=64) == EUNSUP
    assert res(L, ptrs=(P,) * 6 + (None,)) == EINVAL        # out
    assert res(L, ws=None) == EWS                           # S > 0 needs the decode workspace
    assert res(L, S=129) == EINVAL


def blk(L, g=4, q=P, B=2, Hq=8, Hkv=2, S0=100, nb=3, Rb=8, nbc=4, Sc=128, d=128, ptrs=(P,) * 9, kr=P, vr=P, R=5,
        Rc=32, ws=P, wsb=1 << 30):
    ki, ks, ko, kob, vi, vs, vo, vob, out = ptrs
    return L.nsn_check_decode_blocks_args(g, q, B, Hq, Hkv, S0, nb, Rb, nbc, Sc, d, ki, ks, ko, kob, vi, vs, vo, vob,
                                          kr, vr, R, Rc, out, ws, wsb)


def test_decode_blocks_validation_codes(L):
    """Per-block o decode: sizes of the prefix and the blocks against the capacity,
    the block o table against nblk_cap, pointers that must or need not be given,
    the workspace (nsn_decode_blocks_workspace_size)."""
    assert blk(L) == OK
    assert blk(L, R=0, kr=None, vr=None) == OK
    assert blk(L, S0=0, ptrs=(P, P, None, P, P, P, None, P, P)) == OK   # no prefix: its o unused
    assert blk(L, S0=5, ptrs=(P, P, None, P, P, P, None, P, P)) == EINVAL
    assert blk(L, nb=0, Rb=0, ptrs=(P, P, P, None, P, P, P, None, P)) == OK   # no blocks: no table
    assert blk(L, ptrs=(P, P, P, None, P, P, P, P, P)) == EINVAL
    assert blk(L, nb=5) == EINVAL                             # beyond nblk_cap
    assert blk(L, Rb=0) == EINVAL
    assert blk(L, S0=105) == EINVAL                           # 105 + 3 * 8 > 128
    assert blk(L, S0=104) == OK
    assert blk(L, S0=-1) == EINVAL and blk(L, nb=-1) == EINVAL and blk(L, R=-1) == EINVAL
    assert blk(L, S0=0, nb=0, R=0) == EINVAL                  # nothing to attend to
    assert blk(L, R=33) == EINVAL and blk(L, kr=None) == EINVAL
    assert blk(L, q=None) == EINVAL and blk(L, ptrs=(P,) * 8 + (None,)) == EINVAL
    assert blk(L, Hq=12, Hkv=4) == EUNSUP and blk(L, d=64) == EUNSUP and blk(L, g=2) == EUNSUP
    need = L.nsn_decode_blocks_workspace_size(2, 8, 2, 100, 3, 128)
    assert need > 0 and blk(L, wsb=need) == OK and blk(L, wsb=need - 1) == EWS and blk(L, ws=None) == EWS
    assert L.nsn_decode_blocks_workspace_size(2, 8, 2, 100, 3, 64) == 0


def test_rope_and_dq_entry_points_reject_bad_input(L):
    """Argument errors that these entry points report before any device access
    (the handle is never dereferenced on these paths)."""
    fake = P
    assert L.nsn_decode_attention_rope(fake, P, 1, 4, 2, 10, 16, 128, 1.0, *(P,) * 7, P, 1 << 30, None) == EINVAL
    assert L.nsn_decode_attention_rope(fake, P, 1, 4, 2, 10, 16, 128, float("nan"), *(P,) * 7, P, 1 << 30,
                                       None) == EINVAL
    assert L.nsn_decode_attention_rope(None, P, 1, 4, 2, 10, 16, 128, 1e4, *(P,) * 7, P, 1 << 30, None) == EINVAL
    assert L.nsn_decode_attention_rope(fake, P, 1, 4, 2, 10, 16, 128, 1e4, *(P,) * 7, P, 0, None) == EWS
    assert L.nsn_decode_rope_workspace_size(1, 4, 2, 10, 128) > L.nsn_decode_workspace_size(1, 4, 2, 10, 128)
    # prepared RoPE tables: sizes, then argument errors raised before any launch
    assert L.nsn_rope_tables_size(0) == 0 and L.nsn_rope_tables_size(-3) == 0
    assert L.nsn_rope_tables_size(256) == (1 + 256) * 64 * 8  # coarse row, then the 256 fine rows
    assert L.nsn_rope_tables_size(257) == (2 + 256) * 64 * 8
    n = L.nsn_rope_tables_size(1000)
    assert L.nsn_rope_tables(1.0, 1000, P, n, None) == EINVAL
    assert L.nsn_rope_tables(float("inf"), 1000, P, n, None) == EINVAL
    assert L.nsn_rope_tables(1e4, 0, P, n, None) == EINVAL
    assert L.nsn_rope_tables(1e4, 1000, None, n, None) == EINVAL
    assert L.nsn_rope_tables(1e4, 1000, P + 8, n, None) == EINVAL  # not 16-byte aligned
    assert L.nsn_rope_tables(1e4, 1000, P, n - 1, None) == EINVAL
    assert "bytes" in nsn.nsn_last_error()
    need = L.nsn_decode_rope_tables_workspace_size(1, 4, 2, 10, 128)
    assert 0 < need == L.nsn_decode_rope_workspace_size(1, 4, 2, 10, 128) - L.nsn_rope_tables_size(10)
    assert L.nsn_decode_rope_tables_workspace_size(1, 4, 2, 10, 64) == 0

    def rt(tables=P, S=10, S_tab=16, wsb=1 << 30, cb=fake):
        return L.nsn_decode_attention_rope_tables(cb, P, 1, 4, 2, S, 16, 128, tables, S_tab, *(P,) * 7, P, wsb, None)

    assert rt(S=17, S_tab=16) == EINVAL and "tables" in nsn.nsn_last_error()
    assert rt(tables=None) == EINVAL and rt(tables=P + 4) == EINVAL and rt(S_tab=0) == EINVAL
    assert rt(cb=None) == EINVAL
    assert rt(wsb=need - 1) == EWS
    # double-quantized decode: the s1 code arrays are required
    assert L.nsn_decode_attention_dq(fake, P, 1, 4, 2, 10, 16, 128, P, P, None, P, P, P, P, P, P, P,
                                     1 << 30, None) == EINVAL
    assert L.nsn_encode_dq_workspace_size(1, 2, 100, 128) > L.nsn_encode_workspace_size(1, 2, 100, 128)
    assert L.nsn_encode_dq_workspace_size(1, 2, 100, 64) == 0


def test_binding_raises_with_status_text(L):
    with pytest.raises(nsn.NSNError) as ei:
        nsn.nsn_codebook_create(np.full((256, 4), 0.1, np.float32))
    assert ei.value.code == EINVAL


class _FakeGPUTensor:
    """Stands in for a GPU tensor in the binding's checks (no device needed)."""

    def __init__(self, shape, dtype, contiguous=True, cuda=True):
        self.shape, self._dtype, self._contig, self.is_cuda = tuple(shape), dtype, contiguous, cuda

    @property
    def dtype(self):
        return f"torch.{self._dtype}"

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        return P


def test_binding_checks_tensors_before_any_call(L):
    """The binding refuses host, strided, mistyped or misshapen tensors with a
    ValueError naming the argument, before the library is called."""
    cb = nsn.Codebook(P, 4)
    try:
        _binding_cases(cb)
    finally:
        cb.handle = None  # a stand-in handle: never destroyed


def _binding_cases(cb):
    F = _FakeGPUTensor
    B, H, Lt, d = 1, 2, 16, 128
    good = dict(x=F((B, H, Lt, d), "float16"), o=F((B, H, d), "float32"), idx=F((B, H, Lt, 32), "uint8"),
                scales=F((B, H, Lt, 2), "float16"))
    cases = [("x", F((B, H, Lt, d), "float16", cuda=False), "GPU tensor"),
             ("x", F((B, H, Lt, d), "float16", contiguous=False), "contiguous"),
             ("x", F((B, H, Lt, d), "bfloat16"), "dtype"),
             ("o", F((B, H, d), "float16"), "dtype"),
             ("idx", F((B, H, Lt, 16), "uint8"), "shape"),
             ("scales", F((B, H, Lt + 1, 2), "float16"), "shape")]
    for name, bad, msg in cases:
        args = dict(good, **{name: bad})
        with pytest.raises(ValueError, match=msg):
            nsn.nsn_encode(cb, args["x"], args["o"], args["idx"], args["scales"], o_mode=nsn.NSN_O_REUSE)
    cache = (good["idx"], good["scales"], good["o"])
    with pytest.raises(ValueError, match="q"):
        nsn.nsn_decode_attention(cb, F((B, 8, d), "float32"), cache, cache, F((B, 8, d), "float32"), Lt)
    with pytest.raises(ValueError, match="out"):
        nsn.nsn_decode_attention(cb, F((B, 8, d), "float16"), cache, cache, F((B, 8, 64), "float32"), Lt)
    with pytest.raises(ValueError, match="v_cache scales"):
        nsn.nsn_decode_attention(cb, F((B, 8, d), "float16"), cache, (good["idx"], F((B, H, Lt, 2), "float32"),
                                                                      good["o"]), F((B, 8, d), "float32"), Lt)
    # a V cache (or its scales) of another capacity than the K cache: the library
    # indexes both with K's capacity, so every decode entry point refuses it
    small = (F((B, H, Lt - 4, 32), "uint8"), F((B, H, Lt - 4, 2), "float16"), good["o"])
    q8, out8 = F((B, 8, d), "float16"), F((B, 8, d), "float32")
    with pytest.raises(ValueError, match="v_cache idx"):
        nsn.nsn_decode_attention(cb, q8, cache, small, out8, Lt - 4)
    with pytest.raises(ValueError, match="v_cache scales"):
        nsn.nsn_decode_attention(cb, q8, cache, (good["idx"], small[1], good["o"]), out8, Lt - 4)
    with pytest.raises(ValueError, match="v_cache idx"):
        nsn.nsn_decode_attention_rope(cb, q8, cache, small, out8, Lt - 4)
    res = F((B, H, 8, d), "float16")
    with pytest.raises(ValueError, match="v_cache idx"):
        nsn.nsn_decode_attention_residual(cb, q8, cache, small, res, res, out8, Lt - 4, 8)
    with pytest.raises(ValueError, match="both"):
        nsn.nsn_decode_attention_residual(cb, q8, cache, None, res, res, out8, 0, 8)
    new = F((B, H, d), "float16")
    with pytest.raises(ValueError, match="v_cache idx"):
        nsn.nsn_decode_step(cb, q8, new, new, cache, small, out8, Lt - 5)
    dq = (good["idx"], F((B, H, Lt), "float16"), F((B, H, Lt // 2), "uint8"), F((B, H, 80), "uint8"))
    dq_small = (small[0], F((B, H, Lt - 4), "float16"), F((B, H, (Lt - 4) // 2), "uint8"), F((B, H, 80), "uint8"))
    with pytest.raises(ValueError, match="v_cache idx"):
        nsn.nsn_decode_attention_dq(cb, q8, dq, dq_small, out8, Lt - 4)
    with pytest.raises(ValueError, match="v_cache s1c"):
        nsn.nsn_decode_attention_dq(cb, q8, dq, (dq[0], dq[1], dq_small[2], dq[3]), out8, Lt - 4)


def test_decode_noalloc_refuses_sizes_beyond_its_static_workspace(L):
    """The no-allocation decode checks its arguments like nsn_decode_attention and
    refuses a size whose workspace exceeds its 4 MiB static array (NSN_EWORKSPACE)
    before any HIP call; a NULL tensor pointer is NSN_EINVAL."""
    cb = P  # a stand-in handle: the checks above the size limit never read it
    need = L.nsn_decode_workspace_size(64, 256, 32, 4096, 128)
    assert need > 4 << 20
    rc = L.nsn_decode_attention_noalloc(cb, P, 64, 256, 32, 4096, 4096, 128, P, P, P, P, P, P, P, None)
    assert rc == -3 and b"static scratch" in L.nsn_last_error()
    rc = L.nsn_decode_attention_noalloc(cb, P, 1, 4, 2, 100, 100, 128, P, None, P, P, P, P, P, None)
    assert rc == -1 and b"NULL" in L.nsn_last_error()
