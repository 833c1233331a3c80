"""Python binding of the NSNQuant gfx950 library (libnsn.so).

Argument marshalling only: every step of the path runs in the HIP kernels of
libnsn.so.  The functions keep the C names; tensors are torch tensors on the
GPU (device memory and streams come from PyTorch).  If the shared library has
not been built the first call raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "NSNError", "Codebook", "lib", "nsn_version", "nsn_last_error", "nsn_build_codebook", "nsn_finetune_codebook",
    "nsn_codebook_create", "nsn_codebook_create_rht", "nsn_codebook_sign_mask", "nsn_encode_workspace_size", "nsn_encode", "nsn_decode_workspace_size",
    "nsn_decode_attention", "nsn_decode_attention_noalloc", "nsn_decode_attention_residual", "nsn_residual_flush", "nsn_decode_step",
    "nsn_decode_blocks_workspace_size", "nsn_decode_attention_blocks", "nsn_block_flush",
    "nsn_decode_rope_workspace_size", "nsn_decode_attention_rope", "nsn_rope_tables_size", "nsn_rope_tables",
    "nsn_decode_rope_tables_workspace_size", "nsn_decode_attention_rope_tables",
    "nsn_codebook_dq4", "nsn_encode_dq_workspace_size", "nsn_encode_dq", "nsn_decode_attention_dq", "DQ_HEAD_BYTES",
    "nsn_dequantize", "NSN_F16", "NSN_F32",
    "NSN_O_COMPUTE", "NSN_O_REUSE", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnsn.so")
NSN_OK, NSN_EINVAL, NSN_EUNSUPPORTED, NSN_EWORKSPACE, NSN_EHIP, NSN_ENOMEM = 0, -1, -2, -3, -4, -5
NSN_F16, NSN_F32 = 0, 1
NSN_O_COMPUTE, NSN_O_REUSE = 0, 1
DQ_HEAD_BYTES = 80  # sizeof(nsn_dq_head)

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


class NSNError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"nsn status {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libnsn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run kv_cache_vector_nsn_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "nsn_version": (_I, []),
        "nsn_last_error": (ctypes.c_char_p, []),
        "nsn_build_codebook": (_I, [ctypes.c_uint64, _I, _I, ctypes.c_int64, _I, _P, _P, _P]),
        "nsn_finetune_codebook": (_I, [_P, _I, _I, ctypes.c_uint64, ctypes.c_int64, _I, ctypes.c_double, _P, _P,
                                       _P]),
        "nsn_codebook_create": (_I, [_P, _I, _I, ctypes.POINTER(_P)]),
        "nsn_codebook_create_rht": (_I, [_P, _I, _I, _P, ctypes.POINTER(_P)]),
        "nsn_codebook_sign_mask": (_I, [_P, _P]),
        "nsn_codebook_destroy": (None, [_P]),
        "nsn_codebook_g": (_I, [_P]),
        "nsn_codebook_search_stats": (_I, [_P, _P, _P]),
        "nsn_search_grid_edges": (_I, [_P, _I]),
        "nsn_encode_workspace_size": (_SZ, [_I, _I, _I, _I]),
        "nsn_encode": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
        "nsn_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
        "nsn_decode_attention": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "nsn_decode_attention_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
        "nsn_decode_attention_residual": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                                               _I, _P, _P, _SZ, _P]),
        "nsn_decode_rope_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
        "nsn_decode_attention_rope": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_double, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _SZ, _P]),
        "nsn_rope_tables_size": (_SZ, [_I]),
        "nsn_rope_tables": (_I, [ctypes.c_double, _I, _P, _SZ, _P]),
        "nsn_decode_rope_tables_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
        "nsn_decode_attention_rope_tables": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P,
                                                  _P, _P, _SZ, _P]),
        "nsn_codebook_dq4": (_I, [_P, _I, _I, _P, _P, _P]),
        "nsn_encode_dq_workspace_size": (_SZ, [_I, _I, _I, _I]),
        "nsn_encode_dq": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
        "nsn_decode_attention_dq": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                         _P]),
        "nsn_decode_step": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "nsn_dequantize": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
        "nsn_check_encode_args": (_I, [_I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ]),
        "nsn_check_decode_args": (_I, [_I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ]),
        "nsn_check_decode_residual_args": (_I, [_I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                                                _I, _P, _P, _SZ]),
        "nsn_decode_blocks_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
        "nsn_decode_attention_blocks": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
        "nsn_check_decode_blocks_args": (_I, [_I, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                              _P, _P, _P, _P, _I, _I, _P, _P, _SZ]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != NSN_OK:
        raise NSNError(rc, lib().nsn_last_error().decode())


def _t(t, name, dtypes, shape=None):
    """Device pointer of `t` after checking that it is a contiguous GPU tensor of
    one of `dtypes` (names of torch dtypes) and, if given, of exactly `shape`; the
    kernels index the memory as that dense layout.  An int passes through as a raw
    device pointer; None stays None."""
    if t is None or isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (the kernels read it as a dense row-major array)")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


_F16, _F32, _U8 = ("float16",), ("float32",), ("uint8",)


def _cache_ptrs(cache, name, B, H, d, g, cap=None):
    """(idx, scales, o) of a plain K or V cache, checked: idx [B,H,S_cap,d/g] uint8,
    scales [B,H,S_cap,2] fp16, o [B,H,d] fp32.  cap: the capacity S_cap the library
    is given (it indexes K and V alike with it); None takes idx's own."""
    idx, sc, o = cache
    cap = idx.shape[2] if cap is None else cap
    return (_t(idx, f"{name} idx", _U8, (B, H, cap, d // g)), _t(sc, f"{name} scales", _F16, (B, H, cap, 2)),
            _t(o, f"{name} o", _F32, (B, H, d)))


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _ws(nbytes, like, ws):
    if ws is not None:
        return ws
    import torch

    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=like.device)


def nsn_version() -> int:
    return lib().nsn_version()


def nsn_last_error() -> str:
    return lib().nsn_last_error().decode()


def nsn_build_codebook(seed: int, g: int, K: int = 256, n_samples: int = 1 << 20, max_iters: int = 200):
    """GPU k-means codebook -> (centroids float32 [K, g] numpy, distortion/dim, iterations)."""
    import numpy as np

    c = np.zeros((K, g), dtype=np.float32)
    dist = ctypes.c_double()
    it = ctypes.c_int()
    _check(lib().nsn_build_codebook(seed, g, K, n_samples, max_iters, c.ctypes.data, ctypes.addressof(dist),
                                    ctypes.addressof(it)))
    return c, dist.value, it.value


def nsn_finetune_codebook(centroids, seed: int, n_vectors: int, iters: int, lr: float, g: int | None = None):
    """GPU cosine fine-tune -> (centroids float32 [K, g] fp16-exact, raw float64 [K, g],
    mean cosine distance before each step and of the rounded result (iters + 1,))."""
    import numpy as np

    cin = np.ascontiguousarray(centroids, dtype=np.float32)
    K, gg = cin.shape
    g = gg if g is None else g
    cout = np.zeros((K, g), dtype=np.float32)
    raw = np.zeros((K, g), dtype=np.float64)
    cd = np.zeros(iters + 1, dtype=np.float64)
    _check(lib().nsn_finetune_codebook(cin.ctypes.data, g, K, seed, n_vectors, iters, lr, cout.ctypes.data,
                                       raw.ctypes.data, cd.ctypes.data))
    return cout, raw, cd


class Codebook:
    """Owning wrapper of an nsn_codebook handle."""

    def __init__(self, handle: int, g: int):
        self.handle = handle
        self.g = g

    def close(self):
        if self.handle:
            lib().nsn_codebook_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def nsn_codebook_create(centroids, g: int | None = None) -> Codebook:
    import numpy as np

    c = np.ascontiguousarray(centroids, dtype=np.float32)
    g = c.shape[1] if g is None else g
    h = _P()
    _check(lib().nsn_codebook_create(c.ctypes.data, g, c.shape[0], ctypes.byref(h)))
    return Codebook(h.value, g)


def nsn_codebook_create_rht(centroids, sign_mask, g: int | None = None) -> Codebook:
    """Codebook whose calls rotate by H D (D = diag(+-1) from the 16-byte mask:
    bit c % 8 of byte c // 8 set negates channel c)."""
    import numpy as np

    c = np.ascontiguousarray(centroids, dtype=np.float32)
    m = np.ascontiguousarray(np.frombuffer(bytes(sign_mask), dtype=np.uint8))
    if m.size != 16:
        raise ValueError("sign_mask must be 16 bytes")
    g = c.shape[1] if g is None else g
    h = _P()
    _check(lib().nsn_codebook_create_rht(c.ctypes.data, g, c.shape[0], m.ctypes.data, ctypes.byref(h)))
    return Codebook(h.value, g)


def nsn_codebook_sign_mask(cb: Codebook) -> bytes:
    buf = (ctypes.c_uint8 * 16)()
    _check(lib().nsn_codebook_sign_mask(cb.handle, buf))
    return bytes(buf)


def nsn_codebook_search_stats(cb: Codebook):
    """(longest candidate list, overflowing cells) of the g = 4 search grid."""
    mx, ov = ctypes.c_int(), ctypes.c_int()
    _check(lib().nsn_codebook_search_stats(cb.handle, ctypes.byref(mx), ctypes.byref(ov)))
    return mx.value, ov.value


def nsn_search_grid_edges():
    """Bin edges (ascending, the same on every coordinate) of the g = 4 search grid."""
    buf = (ctypes.c_float * 64)()
    n = lib().nsn_search_grid_edges(buf, 64)
    _check(min(n, 0))
    return [float(buf[i]) for i in range(n)]


def nsn_encode_workspace_size(B, H, L, d=128) -> int:
    return lib().nsn_encode_workspace_size(B, H, L, d)


def nsn_encode(cb: Codebook, x, o, idx, scales, *, o_mode=NSN_O_COMPUTE, pos0=0, ws=None, stream=None):
    """x [B,H,L,d] fp16/fp32; o [B,H,d] fp32; idx [B,H,L_cap,d/g] uint8; scales [B,H,L_cap,2] fp16."""
    import torch

    B, H, L, d = x.shape
    L_cap = idx.shape[2]
    xdt = NSN_F16 if x.dtype == torch.float16 else NSN_F32
    px = _t(x, "x", ("float16", "float32"))
    pi, ps, po = _cache_ptrs((idx, scales, o), "cache", B, H, d, cb.g)
    if o_mode == NSN_O_COMPUTE:
        ws = _ws(nsn_encode_workspace_size(B, H, L, d), x, ws)
    _check(lib().nsn_encode(cb.handle, px, xdt, B, H, L, L_cap, pos0, d, o_mode, po, pi, ps, _t(ws, "ws", _U8),
                            0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def nsn_decode_workspace_size(B, Hq, Hkv, S, d=128) -> int:
    return lib().nsn_decode_workspace_size(B, Hq, Hkv, S, d)


def nsn_decode_attention(cb: Codebook, q, k_cache, v_cache, out, S, *, ws=None, stream=None):
    """q [B,Hq,d] fp16; caches are (idx, scales, o) triples; out [B,Hq,d] fp32."""
    B, Hq, d = q.shape
    Hkv, S_cap = k_cache[0].shape[1], k_cache[0].shape[2]
    kp = _cache_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap)
    vp = _cache_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap)
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    ws = _ws(nsn_decode_workspace_size(B, Hq, Hkv, S, d), q, ws)
    _check(lib().nsn_decode_attention(cb.handle, pq, B, Hq, Hkv, S, S_cap, d, *kp, *vp, pout, _t(ws, "ws", _U8),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def nsn_decode_attention_noalloc(cb: Codebook, q, k_cache, v_cache, out, S, *, stream=None):
    """nsn_decode_attention with the library's static per-device workspace (no
    allocation anywhere); q [B,Hq,d] fp16; caches are (idx, scales, o); out fp32."""
    B, Hq, d = q.shape
    Hkv, S_cap = k_cache[0].shape[1], k_cache[0].shape[2]
    kp = _cache_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap)
    vp = _cache_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap)
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    _check(lib().nsn_decode_attention_noalloc(cb.handle, pq, B, Hq, Hkv, S, S_cap, d, *kp, *vp, pout,
                                              _stream(stream)))


def nsn_decode_attention_residual(cb: Codebook, q, k_cache, v_cache, k_res, v_res, out, S, R, *, ws=None,
                                  stream=None):
    """Attention over S quantized tokens plus R fp16 residual tokens.

    q [B,Hq,d] fp16; caches are (idx, scales, o) triples (None when S = 0);
    k_res, v_res [B,Hkv,R_cap,d] fp16; out [B,Hq,d] fp32."""
    B, Hq, d = q.shape
    Hkv, R_cap = k_res.shape[1], k_res.shape[2]
    S_cap = k_cache[0].shape[2] if k_cache is not None else 0
    if (k_cache is None) != (v_cache is None):
        raise ValueError("k_cache and v_cache must both be given or both be None")
    kp = _cache_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap) if k_cache is not None else (None, None, None)
    vp = _cache_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap) if v_cache is not None else (None, None, None)
    pr = (_t(k_res, "k_res", _F16, (B, Hkv, R_cap, d)), _t(v_res, "v_res", _F16, (B, Hkv, R_cap, d)))
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    ws = _ws(nsn_decode_workspace_size(B, Hq, Hkv, S, d), q, ws)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().nsn_decode_attention_residual(cb.handle, pq, B, Hq, Hkv, S, S_cap, d, *kp, *vp, *pr, R, R_cap,
                                               pout, _t(ws, "ws", _U8), nbytes, _stream(stream)))


def nsn_residual_flush(cb: Codebook, k_res, v_res, k_cache, v_cache, S, *, ws=None, stream=None):
    """Quantize a full residual window (R_cap tokens) into cache positions S ..
    S + R_cap - 1: two nsn_encode calls, reusing the stored o when S > 0 and
    computing it from the window when S = 0."""
    B, Hkv, R_cap, d = k_res.shape
    mode = NSN_O_REUSE if S > 0 else NSN_O_COMPUTE
    if mode == NSN_O_COMPUTE and ws is None:
        ws = _ws(nsn_encode_workspace_size(B, Hkv, R_cap, d), k_res, None)
    for x, (idx, sc, o) in ((k_res, k_cache), (v_res, v_cache)):
        nsn_encode(cb, x, o, idx, sc, o_mode=mode, pos0=S, ws=ws, stream=stream)


def nsn_decode_blocks_workspace_size(B, Hq, Hkv, S0, nblk, d=128) -> int:
    return lib().nsn_decode_blocks_workspace_size(B, Hq, Hkv, S0, nblk, d)


def nsn_decode_attention_blocks(cb: Codebook, q, k_cache, v_cache, k_ob, v_ob, out, S0, nblk, Rb, *, k_res=None,
                                v_res=None, R=0, ws=None, stream=None):
    """Attention over a prefix of S0 tokens (the caches' own o) and nblk flushed
    blocks of Rb tokens, block j with o k_ob[j] / v_ob[j] ([nblk_cap,B,Hkv,d] fp32),
    plus R fp16 residual rows (k_res/v_res [B,Hkv,R_cap,d], optional)."""
    B, Hq, d = q.shape
    Hkv, S_cap = k_cache[0].shape[1], k_cache[0].shape[2]
    kp = _cache_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap)
    vp = _cache_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap)
    nblk_cap = k_ob.shape[0]
    pob = (_t(k_ob, "k_ob", _F32, (nblk_cap, B, Hkv, d)), _t(v_ob, "v_ob", _F32, (nblk_cap, B, Hkv, d)))
    if (k_res is None) != (v_res is None):
        raise ValueError("k_res and v_res must both be given or both be None")
    if k_res is not None:
        R_cap = k_res.shape[2]
        pr = (_t(k_res, "k_res", _F16, (B, Hkv, R_cap, d)), _t(v_res, "v_res", _F16, (B, Hkv, R_cap, d)))
    else:
        R_cap, pr = 0, (None, None)
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    ws = _ws(nsn_decode_blocks_workspace_size(B, Hq, Hkv, S0, nblk, d), q, ws)
    _check(lib().nsn_decode_attention_blocks(cb.handle, pq, B, Hq, Hkv, S0, nblk, Rb, nblk_cap, S_cap, d, kp[0], kp[1],
                                             kp[2], pob[0], vp[0], vp[1], vp[2], pob[1], *pr, R, R_cap, pout,
                                             _t(ws, "ws", _U8), ws.numel() * ws.element_size(), _stream(stream)))


def nsn_block_flush(cb: Codebook, k_res, v_res, k_cache, v_cache, k_ob, v_ob, S0, j, *, ws=None, stream=None):
    """Quantize a full residual window (Rb = R_cap tokens) as block j of the cache:
    each tensor encoded on its own (NSN_O_COMPUTE), records at positions
    S0 + j Rb .., its o written to k_ob[j] / v_ob[j]."""
    B, Hkv, Rb, d = k_res.shape
    if ws is None:
        ws = _ws(nsn_encode_workspace_size(B, Hkv, Rb, d), k_res, None)
    for x, (idx, sc, _), ob in ((k_res, k_cache, k_ob), (v_res, v_cache, v_ob)):
        nsn_encode(cb, x, ob[j], idx, sc, o_mode=NSN_O_COMPUTE, pos0=S0 + j * Rb, ws=ws, stream=stream)


def nsn_decode_rope_workspace_size(B, Hq, Hkv, S, d=128) -> int:
    return lib().nsn_decode_rope_workspace_size(B, Hq, Hkv, S, d)


def nsn_decode_attention_rope(cb: Codebook, q, k_cache, v_cache, out, S, *, rope_base=10000.0, ws=None, stream=None):
    """Keys cached before RoPE: q [B,Hq,d] fp16 (rotated to its position); caches as in
    nsn_decode_attention; cached token i is rotated by position i inside the score."""
    B, Hq, d = q.shape
    Hkv, S_cap = k_cache[0].shape[1], k_cache[0].shape[2]
    kp = _cache_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap)
    vp = _cache_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap)
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    ws = _ws(nsn_decode_rope_workspace_size(B, Hq, Hkv, S, d), q, ws)
    _check(lib().nsn_decode_attention_rope(cb.handle, pq, B, Hq, Hkv, S, S_cap, d, rope_base, *kp, *vp, pout,
                                           _t(ws, "ws", _U8), ws.numel() * ws.element_size(), _stream(stream)))


def nsn_rope_tables_size(S_tab) -> int:
    return lib().nsn_rope_tables_size(S_tab)


def nsn_rope_tables(S_tab, *, rope_base=10000.0, tables=None, device=None, stream=None):
    """The cos / sin tables of every position below S_tab, built once on the GPU for
    nsn_decode_attention_rope_tables; returns the (uint8) tables tensor, allocated on
    `device` (default: the current GPU) unless one is passed."""
    import torch

    nbytes = nsn_rope_tables_size(S_tab)
    if tables is None:
        tables = torch.empty(max(1, nbytes), dtype=torch.uint8, device=device if device is not None else "cuda")
    _check(lib().nsn_rope_tables(rope_base, S_tab, _t(tables, "tables", _U8), tables.numel() * tables.element_size(),
                                 _stream(stream)))
    return tables


def nsn_decode_rope_tables_workspace_size(B, Hq, Hkv, S, d=128) -> int:
    return lib().nsn_decode_rope_tables_workspace_size(B, Hq, Hkv, S, d)


def nsn_decode_attention_rope_tables(cb: Codebook, q, k_cache, v_cache, out, S, tables, S_tab, *, ws=None,
                                     stream=None):
    """nsn_decode_attention_rope with tables from nsn_rope_tables(S_tab, rope_base=...)
    (S <= S_tab); the workspace holds only the chunk partials."""
    B, Hq, d = q.shape
    Hkv, S_cap = k_cache[0].shape[1], k_cache[0].shape[2]
    kp = _cache_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap)
    vp = _cache_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap)
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    ws = _ws(nsn_decode_rope_tables_workspace_size(B, Hq, Hkv, S, d), q, ws)
    _check(lib().nsn_decode_attention_rope_tables(cb.handle, pq, B, Hq, Hkv, S, S_cap, d, _t(tables, "tables", _U8),
                                                  S_tab, *kp, *vp, pout, _t(ws, "ws", _U8),
                                                  ws.numel() * ws.element_size(), _stream(stream)))


def nsn_codebook_dq4(centroids):
    """4-bit codebook -> (codes uint8 [K, g], step D, centroids_q float32 [K, g] fp16-exact)."""
    import numpy as np

    c = np.ascontiguousarray(centroids, dtype=np.float32)
    K, g = c.shape
    codes = np.zeros((K, g), dtype=np.uint8)
    cq = np.zeros((K, g), dtype=np.float32)
    step = ctypes.c_float()
    _check(lib().nsn_codebook_dq4(c.ctypes.data, K, g, codes.ctypes.data, ctypes.addressof(step), cq.ctypes.data))
    return codes, step.value, cq


def nsn_encode_dq_workspace_size(B, H, L, d=128) -> int:
    return lib().nsn_encode_dq_workspace_size(B, H, L, d)


def _dq_ptrs(cache, name, B, H, d, g, cap=None):
    """(idx, s2, s1c, head) of a double-quantized cache, checked (cap as in _cache_ptrs)."""
    idx, s2, s1c, head = cache
    cap = idx.shape[2] if cap is None else cap
    return (_t(idx, f"{name} idx", _U8, (B, H, cap, d // g)), _t(s2, f"{name} s2", _F16, (B, H, cap)),
            _t(s1c, f"{name} s1c", _U8, (B, H, (cap + 1) // 2)), _t(head, f"{name} head", _U8, (B, H, DQ_HEAD_BYTES)))


def nsn_encode_dq(cb: Codebook, x, cache, *, o_mode=NSN_O_COMPUTE, pos0=0, ws=None, stream=None):
    """x [B,H,L,d] fp16/fp32; cache = (idx [B,H,L_cap,d/g] u8, s2 [B,H,L_cap] fp16,
    s1c [B,H,(L_cap+1)//2] u8, head [B,H,80] u8 (nsn_dq_head records))."""
    import torch

    B, H, L, d = x.shape
    L_cap = cache[0].shape[2]
    xdt = NSN_F16 if x.dtype == torch.float16 else NSN_F32
    pi, p2, pc, ph = _dq_ptrs(cache, "cache", B, H, d, cb.g)
    px = _t(x, "x", ("float16", "float32"))
    ws = _ws(nsn_encode_dq_workspace_size(B, H, L, d), x, ws)
    _check(lib().nsn_encode_dq(cb.handle, px, xdt, B, H, L, L_cap, pos0, d, o_mode, ph, pi, p2, pc,
                               _t(ws, "ws", _U8), ws.numel() * ws.element_size(), _stream(stream)))


def nsn_decode_attention_dq(cb: Codebook, q, k_cache, v_cache, out, S, *, ws=None, stream=None):
    """q [B,Hq,d] fp16; caches are (idx, s2, s1c, head) as in nsn_encode_dq; out [B,Hq,d] fp32."""
    B, Hq, d = q.shape
    Hkv, S_cap = k_cache[0].shape[1], k_cache[0].shape[2]
    kp = _dq_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap)
    vp = _dq_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap)
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    ws = _ws(nsn_decode_workspace_size(B, Hq, Hkv, S, d), q, ws)
    _check(lib().nsn_decode_attention_dq(cb.handle, pq, B, Hq, Hkv, S, S_cap, d, *kp, *vp, pout, _t(ws, "ws", _U8),
                                         ws.numel() * ws.element_size(), _stream(stream)))


def nsn_decode_step(cb: Codebook, q, k_new, v_new, k_cache, v_cache, out, S, *, ws=None, stream=None):
    """Append k_new/v_new [B,Hkv,d] fp16 at position S (encoded inside the decode
    kernel) and attend over S + 1 tokens."""
    B, Hq, d = q.shape
    Hkv, S_cap = k_cache[0].shape[1], k_cache[0].shape[2]
    kp = _cache_ptrs(k_cache, "k_cache", B, Hkv, d, cb.g, S_cap)
    vp = _cache_ptrs(v_cache, "v_cache", B, Hkv, d, cb.g, S_cap)
    pn = (_t(k_new, "k_new", _F16, (B, Hkv, d)), _t(v_new, "v_new", _F16, (B, Hkv, d)))
    pq, pout = _t(q, "q", _F16, (B, Hq, d)), _t(out, "out", _F32, (B, Hq, d))
    ws = _ws(nsn_decode_workspace_size(B, Hq, Hkv, S + 1, d), q, ws)
    _check(lib().nsn_decode_step(cb.handle, pq, *pn, B, Hq, Hkv, S, S_cap, d, *kp, *vp, pout, _t(ws, "ws", _U8),
                                 ws.numel() * ws.element_size(), _stream(stream)))


def nsn_dequantize(cb: Codebook, idx, scales, o, L, x_hat, *, stream=None):
    """x_hat [B,H,L,d] fp32 from idx [B,H,L_cap,m], scales [B,H,L_cap,2], o [B,H,d]."""
    B, H, L_cap, _ = idx.shape
    pi, ps, po = _cache_ptrs((idx, scales, o), "cache", B, H, 128, cb.g)
    _check(lib().nsn_dequantize(cb.handle, pi, ps, po, B, H, L, L_cap, 128, _t(x_hat, "x_hat", _F32, (B, H, L, 128)),
                                _stream(stream)))
