"""GPU test of nsn_decode_attention_noalloc (the decode for callers that cannot
allocate): through the C ABI, its output equals nsn_decode_attention's on the
same inputs, on two calls in a row (the second smaller), each checked as well
against the oracle's dense attention on the dequantized cache (1e-3)."""

import numpy as np
import pytest

import synthetic
from golden_io import load_codebook
from oracle.parity import attention_ref_group, check_attention_rows, gpu_to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import kv_cache_vector_nsn_amd as nsn  # noqa: E402


def _case(dev, cb, C, g, seed, B, Hkv, GQ, S):
    K, V = synthetic.make_kv(seed, B, Hkv, S, 128, "normal", "f16", dev)
    caches, hosts = [], []
    for X in (K, V):
        idx = torch.zeros((B, Hkv, S + 24, 128 // g), dtype=torch.uint8, device=dev)
        sc = torch.zeros((B, Hkv, S + 24, 2), dtype=torch.float16, device=dev)
        o = torch.zeros((B, Hkv, 128), dtype=torch.float32, device=dev)
        nsn.nsn_encode(cb, X, o, idx, sc)
        caches.append((idx, sc, o))
    torch.cuda.synchronize()
    for idx, sc, o in caches:
        s = gpu_to_np(sc)
        hosts.append((idx.cpu().numpy().astype(np.int64), s[..., 0], s[..., 1], gpu_to_np(o)))
    q = synthetic.make_queries(seed, B, Hkv * GQ, 128, dev)
    ref_out = torch.empty((B, Hkv * GQ, 128), dtype=torch.float32, device=dev)
    got = torch.full((B, Hkv * GQ, 128), float("nan"), dtype=torch.float32, device=dev)
    nsn.nsn_decode_attention(cb, q, caches[0], caches[1], ref_out, S)
    nsn.nsn_decode_attention_noalloc(cb, q, caches[0], caches[1], got, S)
    torch.cuda.synchronize()
    assert torch.equal(got, ref_out), float((got - ref_out).abs().max())
    qn, on = gpu_to_np(q), gpu_to_np(got)
    for b in range(B):
        for hk in range(Hkv):
            check_attention_rows(on[b, hk * GQ:(hk + 1) * GQ],
                                 attention_ref_group(qn, hosts[0], hosts[1], C, g, b, hk, GQ, S))


@pytest.mark.parametrize("g", [4, 8])
def test_decode_noalloc_matches_decode(g):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    C, _ = load_codebook(g)
    cb = nsn.nsn_codebook_create(C.astype(np.float32), g)
    # the larger call first, then a smaller one that reuses the same static array
    _case(dev, cb, C, g, 911, B=2, Hkv=4, GQ=4, S=3000)
    _case(dev, cb, C, g, 912, B=1, Hkv=2, GQ=2, S=700)
