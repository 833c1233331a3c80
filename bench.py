"""Benchmark of the NSNQuant hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
encode K and V of every KV head (NSN + Hadamard + nearest centroid + scale),
then decode attention of every query head over the freshly quantized cache.
Default workload: the Mistral-7B-like long-context layer (batch 1, 32 query /
8 KV heads, 131072 tokens, head_dim 128, fp16 inputs with Student-t(3) channel
offsets, 2-bit VQ = 4-dim sub-vectors x 256 centroids).

Prints ONE JSON line.  `value` is encode tokens per second of the whole step
(tokens = K and V of all KV heads of the layer).  Extra keys carry:
  * the per-phase figures of the step's layer (encode tokens/s, decode GB/s over
    the algorithmic cache bytes, the roofline of the dominant kernel);
  * `configs`: the other workloads at their own shapes -- the LLaMA-8B-like
    layer encode, the batch-16 32k-token 2-bit decode, the batch-64 8k-token
    1-bit decode step (append + attention) and the single-head fp32 round trip --
    each timed per call (median, p10, p90 of event pairs around single calls) and
    back to back (one event pair around many calls), over input copies rotated
    so that the 256 MB last-level cache cannot serve repeats;
  * the measured device copy and streaming-read rates beside the 8 TB/s peak;
  * the oracle's CPU rate on a bounded sample (`cpu_baseline`).
"""

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encode tokens/s and decode-attn GB/s (% HBM roofline) at 1/2-bit, head_dim 128"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 600_000_000      # rotated input footprint: > 2 x the 256 MB last-level cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mistral7b-long-2bit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample duration")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extension timings (residual window, double quantization, RoPE, 1 bit, RHT)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' lines")
    ap.add_argument("--only", default=None,
                    help="profiling aid: run only one part and print its timings "
                         "(encode | decode | rope | config2 | config3 | config4 | copy)")
    return ap.parse_args()


def algorithmic(w):
    """Algorithmic bytes / flops / candidate compares per unit: per head-vector for
    encode (x read once, indices and the scale pair written), per cached
    token-head for decode (K and V indices and scale pairs read once)."""
    m = w.d // w.g
    enc_bytes_per_vec = (2 if w.dtype == "f16" else 4) * w.d + m + 4          # x read + idx + (s1, s2') written
    dec_bytes_per_tokhead = 2 * (m + 4)                                        # K and V idx + scales
    enc_flop_per_vec = 2 * 256 * w.d                                           # distance contraction
    enc_cmp_per_vec = m * 256                                                  # one compare per candidate
    return enc_bytes_per_vec, dec_bytes_per_tokhead, enc_flop_per_vec, enc_cmp_per_vec


def measured_traffic():
    """HBM bytes per launch of the encode kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, if it was taken on the current kernel sources
    (matching hash), else None."""
    import hashlib
    import re

    src = os.path.join(ROOT, "kv_cache_vector_nsn_amd", "csrc")
    h = hashlib.sha256()
    for f in ("nsn_encode.hip", "nsn_cells.hip", "nsn_device.h", "nsn_internal.h"):
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    prof = os.path.join(ROOT, "profiles", "k_encode4_mistral7b-long-2bit_traffic.md")
    if not os.path.exists(prof):
        return None
    txt = open(prof).read()
    m = re.search(r"source_sha256_16: ([0-9a-f]+)", txt)
    t = re.search(r"traffic_bytes_per_launch: ([0-9.e+]+)", txt)
    if not m or not t or m.group(1) != h.hexdigest()[:16]:
        return None
    return float(t.group(1))


def timed(fn, iters, torch):
    """Back-to-back: one event pair around `iters` calls on the current stream (ms per call)."""
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(iters):
        fn(i)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def timing(fn, iters, torch, warm=3):
    """Per-call (an event pair around each single call: median, p10, p90) and
    steady-state (one event pair around `iters` back-to-back calls) times, ms."""
    import numpy as np

    st = torch.cuda.current_stream()
    for i in range(warm):
        fn(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(st)
        fn(i)
        b.record(st)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in evs])
    steady = timed(fn, iters, torch)
    return {"median_ms": float(np.median(per)), "p10_ms": float(np.percentile(per, 10)),
            "p90_ms": float(np.percentile(per, 90)), "steady_ms": steady}


def rates(t, nbytes, tokens=None):
    """GB/s and HBM fraction of a timing dict at its median and steady-state times."""
    out = dict(t)
    out["GBps"] = nbytes / (t["median_ms"] * 1e-3) / 1e9
    out["GBps_steady"] = nbytes / (t["steady_ms"] * 1e-3) / 1e9
    out["hbm_frac"] = out["GBps"] / HBM_PEAK_GBPS
    out["hbm_frac_steady"] = out["GBps_steady"] / HBM_PEAK_GBPS
    out["algorithmic_bytes"] = int(nbytes)
    if tokens is not None:
        out["tokens_per_s"] = tokens / (t["median_ms"] * 1e-3)
    return out


def copy_rates(torch, dev):
    """A plain 1 GiB device copy (read + write bytes) and a 2 GiB streaming read
    (sums of 1024-element rows: the fastest read-only pattern among torch's
    reductions here, 2 MB written), the measured denominators beside the 8 TB/s
    spec."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    tc = timing(lambda i: dst.copy_(src), 10, torch)
    del dst
    big = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    rows = torch.empty(big.numel() // 1024, dtype=torch.float32, device=dev)
    tr = timing(lambda i: torch.sum(big.view(-1, 1024), 1, out=rows), 10, torch)
    r = {"copy_GBps": 2 * src.numel() * 4 / (tc["median_ms"] * 1e-3) / 1e9,
         "read_GBps": big.numel() * 4 / (tr["median_ms"] * 1e-3) / 1e9, "copy_bytes": 2 * src.numel() * 4,
         "read_bytes": big.numel() * 4}
    del src, big
    torch.cuda.empty_cache()
    return r


def cpu_baseline(w, C, target_s):
    """Time the fp64 oracle on a bounded sample of the same workload: for KV head
    after KV head (up to all of them), K and V of that head (NSN over all sample
    tokens, nearest centroid, scale) plus the decode attention of its query heads
    over the sample, until about target_s seconds have run; scaled to the layer.
    Also one KV head of 8192 tokens with the BLAS pinned to one thread."""
    import numpy as np

    import oracle
    import synthetic

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = os.cpu_count() or 1
    GQ = w.Hq // w.Hkv
    enc_b, dec_b, _, _ = algorithmic(w)

    def one_head(seed, Ls):
        K, V = synthetic.make_kv_numpy(seed, 1, 1, Ls, w.d, w.kind, w.dtype)
        q = np.random.default_rng(seed).standard_normal((1, GQ, w.d)).astype(np.float16).astype(np.float64)
        t = time.perf_counter()
        rk = oracle.encode_head(K[0, 0].astype(np.float64), C, w.g)
        rv = oracle.encode_head(V[0, 0].astype(np.float64), C, w.g)
        kc = tuple(a[None, None] for a in (rk["idx"], rk["s1"], rk["s2p"])) + (rk["o"][None, None],)
        vc = tuple(a[None, None] for a in (rv["idx"], rv["s1"], rv["s2p"])) + (rv["o"][None, None],)
        oracle.decode_attention(q, *kc, *vc, C, w.g)
        return time.perf_counter() - t

    Ls = min(w.L, 65536)
    spent, heads = 0.0, 0
    while heads < w.Hkv and spent < target_s:
        spent += one_head(99 + heads, Ls)
        heads += 1
    per_token_s = spent / heads * w.Hkv / Ls  # all KV heads of the layer
    tok_s = 1.0 / per_token_s
    # bytes per layer token: K and V of every KV head encoded, and read once by the decode
    bytes_per_token = w.Hkv * (2 * enc_b + dec_b)
    out = {"value": tok_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{heads} KV head(s) x {Ls} tokens (K+V encode, {GQ}-head decode each) in {spent:.1f} s, "
                     f"scaled to {w.Hkv} KV heads",
           "GBps": tok_s * bytes_per_token / 1e9, "bytes_per_token": bytes_per_token}
    if threadpool_limits is not None:
        Ls1 = min(w.L, 8192)
        with threadpool_limits(limits=1):
            t1 = one_head(199, Ls1)
        out["one_core_tokens_per_s"] = Ls1 / (t1 * w.Hkv)
        out["one_core_sample"] = f"1 KV head x {Ls1} tokens in {t1:.2f} s, one BLAS thread, scaled to {w.Hkv} KV heads"
    return out


# ---------------------------------------------------------------- other workloads
def config_encode(nsn, torch, dev, name, iters, books):
    """LLaMA-8B-like layer: encode of K and V of the 8 KV heads (one call on a
    [2B, Hkv, L, d] tensor), over rotated input copies; and the per-token kernel
    alone (reused o)."""
    import synthetic

    w = synthetic.WORKLOADS[name]
    cb = books[w.g]
    m = w.d // w.g
    K, V = synthetic.make_kv(21, w.B, w.Hkv, w.L, w.d, w.kind, w.dtype, dev)
    x = torch.cat([K, V], 0).contiguous()
    del K, V
    ncopy = max(2, -(-ROTATE_BYTES // (x.numel() * x.element_size())))
    xs = [x.clone() for _ in range(ncopy)]
    idx = torch.empty((2 * w.B, w.Hkv, w.L, m), dtype=torch.uint8, device=dev)
    sc = torch.empty((2 * w.B, w.Hkv, w.L, 2), dtype=torch.float16, device=dev)
    o = torch.empty((2 * w.B, w.Hkv, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(nsn.nsn_encode_workspace_size(2 * w.B, w.Hkv, w.L), dtype=torch.uint8, device=dev)
    enc_b = algorithmic(w)[0]
    nbytes = 2 * w.B * w.Hkv * w.L * enc_b
    t = timing(lambda i: nsn.nsn_encode(cb, xs[i % ncopy], o, idx, sc, ws=ws), iters, torch)
    tk = timing(lambda i: nsn.nsn_encode(cb, xs[i % ncopy], o, idx, sc, o_mode=nsn.NSN_O_REUSE), iters, torch)
    return {"workload": name, "op": "encode K and V (statistics + per-token kernel)",
            **rates(t, nbytes, tokens=w.B * w.L),
            "per_token_kernel": rates(tk, nbytes, tokens=w.B * w.L), "rotated_copies": ncopy}


def _encoded_cache(nsn, torch, dev, w, cb, seed, L_cap):
    import synthetic

    m = w.d // w.g
    K, V = synthetic.make_kv(seed, w.B, w.Hkv, w.L, w.d, w.kind, w.dtype, dev)
    caches = []
    for X in (K, V):
        idx = torch.zeros((w.B, w.Hkv, L_cap, m), dtype=torch.uint8, device=dev)
        sc = torch.zeros((w.B, w.Hkv, L_cap, 2), dtype=torch.float16, device=dev)
        o = torch.empty((w.B, w.Hkv, w.d), dtype=torch.float32, device=dev)
        nsn.nsn_encode(cb, X, o, idx, sc)
        caches.append((idx, sc, o))
    del K, V
    torch.cuda.synchronize()
    return caches


def config_decode(nsn, torch, dev, name, iters, books):
    """Batch-16, 32k-token, 2-bit cache: decode attention of the 32 query heads
    over rotated cache copies (K and V indices and scale pairs, 72 B per
    token-head)."""
    import synthetic

    w = synthetic.WORKLOADS[name]
    cb = books[w.g]
    kc, vc = _encoded_cache(nsn, torch, dev, w, cb, 31, w.L)
    dec_b = algorithmic(w)[1]
    cache_bytes = w.B * w.Hkv * w.L * dec_b
    ncopy = max(2, -(-ROTATE_BYTES // cache_bytes))
    copies = [(tuple(t.clone() for t in kc), tuple(t.clone() for t in vc)) for _ in range(ncopy)]
    del kc, vc
    q = synthetic.make_queries(31, w.B, w.Hq, w.d, dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(nsn.nsn_decode_workspace_size(w.B, w.Hq, w.Hkv, w.L), dtype=torch.uint8, device=dev)
    t = timing(lambda i: nsn.nsn_decode_attention(cb, q, copies[i % ncopy][0], copies[i % ncopy][1], out, w.L, ws=ws),
               max(iters, 2 * ncopy), torch)
    extra = w.B * w.Hq * w.d * (2 + 4) + 2 * w.B * w.Hkv * w.d * 4  # q in, out written, o_K and o_V read
    return {"workload": name, "op": "decode attention (all query heads, split-KV + combine)",
            **rates(t, cache_bytes + extra), "cache_bytes": cache_bytes, "rotated_copies": ncopy}


def config_step(nsn, torch, dev, name, iters, books):
    """Batch-64, 8k-token, 1-bit cache: the decode step -- one new K and V token
    per (batch, KV head) encoded with the stored o and written at slot S, then
    attention over S + 1 tokens -- over rotated cache copies."""
    import synthetic

    w = synthetic.WORKLOADS[name]
    cb = books[w.g]
    S = w.L
    kc, vc = _encoded_cache(nsn, torch, dev, w, cb, 41, S + 1)
    m = w.d // w.g
    dec_b = algorithmic(w)[1]
    cache_bytes = w.B * w.Hkv * (S + 1) * dec_b
    ncopy = max(2, -(-ROTATE_BYTES // cache_bytes))
    copies = [(tuple(t.clone() for t in kc), tuple(t.clone() for t in vc)) for _ in range(ncopy)]
    del kc, vc
    Kn, Vn = synthetic.make_kv(42, w.B, w.Hkv, 1, w.d, w.kind, w.dtype, dev)
    kn, vn = Kn[:, :, 0].contiguous(), Vn[:, :, 0].contiguous()
    q = synthetic.make_queries(41, w.B, w.Hq, w.d, dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(nsn.nsn_decode_workspace_size(w.B, w.Hq, w.Hkv, S + 1), dtype=torch.uint8, device=dev)
    t = timing(lambda i: nsn.nsn_decode_step(cb, q, kn, vn, copies[i % ncopy][0], copies[i % ncopy][1], out, S,
                                             ws=ws), max(iters, 2 * ncopy), torch)
    append_bytes = 2 * w.B * w.Hkv * (2 * w.d + m + 4)  # new K/V rows read, their records written
    extra = w.B * w.Hq * w.d * (2 + 4) + 2 * w.B * w.Hkv * w.d * 4
    return {"workload": name, "op": "decode step: append-encode of the new token + attention over S + 1",
            **rates(t, cache_bytes + append_bytes + extra), "cache_bytes": cache_bytes, "rotated_copies": ncopy}


def config_single(nsn, torch, dev, name, iters, books):
    """Single fp32 head of 256 tokens at 1 bit: encode of K and V, then one
    query's attention (launch-bound: reported as latency)."""
    import synthetic

    w = synthetic.WORKLOADS[name]
    cb = books[w.g]
    m = w.d // w.g
    K, V = synthetic.make_kv(51, w.B, w.Hkv, w.L, w.d, w.kind, w.dtype, dev)
    x = torch.cat([K, V], 0).contiguous()
    idx = torch.empty((2, 1, w.L, m), dtype=torch.uint8, device=dev)
    sc = torch.empty((2, 1, w.L, 2), dtype=torch.float16, device=dev)
    o = torch.empty((2, 1, w.d), dtype=torch.float32, device=dev)
    q = synthetic.make_queries(51, 1, 1, w.d, dev)
    out = torch.empty((1, 1, w.d), dtype=torch.float32, device=dev)
    ews = torch.empty(nsn.nsn_encode_workspace_size(2, 1, w.L), dtype=torch.uint8, device=dev)
    dws = torch.empty(nsn.nsn_decode_workspace_size(1, 1, 1, w.L), dtype=torch.uint8, device=dev)

    def run(i):
        nsn.nsn_encode(cb, x, o, idx, sc, ws=ews)
        nsn.nsn_decode_attention(cb, q, (idx[:1], sc[:1], o[:1]), (idx[1:], sc[1:], o[1:]), out, w.L, ws=dws)

    t = timing(run, iters, torch)
    return {"workload": name, "op": "encode K and V + one query's attention (latency)", **t}


def _layer_inputs(nsn, torch, dev, w):
    import synthetic

    m = w.d // w.g
    K, V = synthetic.make_kv(7, w.B, w.Hkv, w.L, w.d, w.kind, w.dtype, dev)
    x = torch.cat([K, V], 0).contiguous()
    del K, V
    idx = torch.empty((2 * w.B, w.Hkv, w.L, m), dtype=torch.uint8, device=dev)
    sc = torch.empty((2 * w.B, w.Hkv, w.L, 2), dtype=torch.float16, device=dev)
    o = torch.empty((2 * w.B, w.Hkv, w.d), dtype=torch.float32, device=dev)
    return x, idx, sc, o


def layer_encode(nsn, torch, dev, w, cb, iters):
    """Profiling aid: the step layer's encode (statistics + per-token kernel) and
    its per-token kernel alone (reused o)."""
    x, idx, sc, o = _layer_inputs(nsn, torch, dev, w)
    ws = torch.empty(nsn.nsn_encode_workspace_size(2 * w.B, w.Hkv, w.L), dtype=torch.uint8, device=dev)
    nbytes = 2 * w.B * w.Hkv * w.L * algorithmic(w)[0]
    t = timing(lambda i: nsn.nsn_encode(cb, x, o, idx, sc, ws=ws), iters, torch)
    tk = timing(lambda i: nsn.nsn_encode(cb, x, o, idx, sc, o_mode=nsn.NSN_O_REUSE), iters, torch)
    return {"encode": rates(t, nbytes), "per_token_kernel": rates(tk, nbytes)}


def layer_decode(nsn, torch, dev, w, cb, iters):
    """Profiling aid: the step layer's decode over two rotated cache copies."""
    import synthetic

    x, idx, sc, o = _layer_inputs(nsn, torch, dev, w)
    nsn.nsn_encode(cb, x, o, idx, sc)
    del x
    q = synthetic.make_queries(7, w.B, w.Hq, w.d, dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(nsn.nsn_decode_workspace_size(w.B, w.Hq, w.Hkv, w.L), dtype=torch.uint8, device=dev)
    cache_bytes = w.B * w.Hkv * w.L * algorithmic(w)[1]
    ncopy = max(2, -(-ROTATE_BYTES // cache_bytes))
    copies = [(idx.clone(), sc.clone(), o.clone()) for _ in range(ncopy)]
    B = w.B

    def dec(i):
        c = copies[i % ncopy]
        nsn.nsn_decode_attention(cb, q, (c[0][:B], c[1][:B], c[2][:B]), (c[0][B:], c[1][B:], c[2][B:]), out, w.L,
                                 ws=ws)

    return {"decode": rates(timing(dec, max(iters, ncopy), torch), cache_bytes), "rotated_copies": ncopy}


def layer_rope(nsn, torch, dev, w, cb, iters):
    """Profiling aid: the step layer's decode over pre-RoPE keys (rotated cache copies)."""
    import synthetic

    x, idx, sc, o = _layer_inputs(nsn, torch, dev, w)
    nsn.nsn_encode(cb, x, o, idx, sc)
    del x
    q = synthetic.make_queries(7, w.B, w.Hq, w.d, dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(nsn.nsn_decode_rope_workspace_size(w.B, w.Hq, w.Hkv, w.L), dtype=torch.uint8, device=dev)
    cache_bytes = w.B * w.Hkv * w.L * algorithmic(w)[1]
    ncopy = max(2, -(-ROTATE_BYTES // cache_bytes))
    copies = [(idx.clone(), sc.clone(), o.clone()) for _ in range(ncopy)]
    B = w.B

    def dec(i):
        c = copies[i % ncopy]
        nsn.nsn_decode_attention_rope(cb, q, (c[0][:B], c[1][:B], c[2][:B]), (c[0][B:], c[1][B:], c[2][B:]), out,
                                      w.L, ws=ws)

    tab = nsn.nsn_rope_tables(w.L, device=dev)

    def dec_t(i):
        c = copies[i % ncopy]
        nsn.nsn_decode_attention_rope_tables(cb, q, (c[0][:B], c[1][:B], c[2][:B]), (c[0][B:], c[1][B:], c[2][B:]),
                                             out, w.L, tab, w.L, ws=ws)

    return {"decode": rates(timing(dec, max(iters, ncopy), torch), cache_bytes),
            "decode_prepared_tables": rates(timing(dec_t, max(iters, ncopy), torch), cache_bytes),
            "rotated_copies": ncopy}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "single-GPU build: this path runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import kv_cache_vector_nsn_amd as nsn
    import synthetic
    from tests.golden_io import load_codebook  # stored N(0,1) k-means codebooks (inputs)

    w = synthetic.WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    C, _ = load_codebook(w.g)
    # every codebook handle is built before any timed region (the candidate table
    # of a g = 4 handle is built by a kernel when the handle is created)
    books = {g: nsn.nsn_codebook_create(load_codebook(g)[0].astype(np.float32), g) for g in (4, 8)}
    cb = books[w.g]
    cb8 = books[8]
    cbr = None if a.no_extras else nsn.nsn_codebook_create_rht(
        C.astype(np.float32), bytes(np.random.default_rng(20250523).integers(0, 256, 16, dtype=np.uint8)), w.g)
    it = max(a.steps, 20) if a.only is None else max(a.steps, 3)

    if a.only is not None:  # profiling aid: the listed parts only, in order
        parts = {"config2": lambda: config_encode(nsn, torch, dev, "llama8b-layer-encode-2bit", it, books),
                 "config3": lambda: config_decode(nsn, torch, dev, "decode-2bit-b16-s32k", it, books),
                 "config4": lambda: config_step(nsn, torch, dev, "decode-step-1bit-b64-s8k", it, books),
                 "encode": lambda: layer_encode(nsn, torch, dev, w, cb, it),
                 "decode": lambda: layer_decode(nsn, torch, dev, w, cb, it),
                 "rope": lambda: layer_rope(nsn, torch, dev, w, cb, it),
                 "encode8": lambda: layer_encode(nsn, torch, dev, dataclasses.replace(w, g=8), cb8, it),
                 "copy": lambda: copy_rates(torch, dev)}
        res = {}
        for p in a.only.split(","):
            res[p] = parts[p]()
            torch.cuda.empty_cache()
        print(json.dumps(res), flush=True)
        return

    # the other workloads first: each at its own shape, per-call and back-to-back
    configs = {}
    if not a.no_configs:
        configs["llama8b-layer-encode-2bit"] = config_encode(nsn, torch, dev, "llama8b-layer-encode-2bit", it, books)
        print(f"# config llama8b encode: {configs['llama8b-layer-encode-2bit']['median_ms']:.4f} ms", file=sys.stderr,
              flush=True)
        configs["decode-2bit-b16-s32k"] = config_decode(nsn, torch, dev, "decode-2bit-b16-s32k", it, books)
        print(f"# config b16 s32k decode: {configs['decode-2bit-b16-s32k']['median_ms']:.4f} ms", file=sys.stderr,
              flush=True)
        configs["decode-step-1bit-b64-s8k"] = config_step(nsn, torch, dev, "decode-step-1bit-b64-s8k", it, books)
        print(f"# config b64 s8k step: {configs['decode-step-1bit-b64-s8k']['median_ms']:.4f} ms", file=sys.stderr,
              flush=True)
        configs["single-head-fp32-1bit"] = config_single(nsn, torch, dev, "single-head-fp32-1bit", it, books)
        torch.cuda.empty_cache()

    m = w.d // w.g
    BH = w.B * w.Hkv

    # inputs resident in HBM: K and V of the layer stacked as one [2B, Hkv, L, d]
    # tensor so one encode call covers both; two copies rotate between steps.
    xs = []
    for r in range(2):
        K, V = synthetic.make_kv(7 + r, w.B, w.Hkv, w.L, w.d, w.kind, w.dtype, dev)
        xs.append(torch.cat([K, V], 0).contiguous())
        del K, V
    q = synthetic.make_queries(7, w.B, w.Hq, w.d, dev)
    idx = torch.empty((2 * w.B, w.Hkv, w.L, m), dtype=torch.uint8, device=dev)
    sc = torch.empty((2 * w.B, w.Hkv, w.L, 2), dtype=torch.float16, device=dev)
    o = torch.empty((2 * w.B, w.Hkv, w.d), dtype=torch.float32, device=dev)
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=dev)
    ews = torch.empty(nsn.nsn_encode_workspace_size(2 * w.B, w.Hkv, w.L), dtype=torch.uint8, device=dev)
    dws = torch.empty(nsn.nsn_decode_workspace_size(w.B, w.Hq, w.Hkv, w.L), dtype=torch.uint8, device=dev)

    def kv_views(i, s, oo):
        return (i[:w.B], s[:w.B], oo[:w.B]), (i[w.B:], s[w.B:], oo[w.B:])

    def step(i):
        nsn.nsn_encode(cb, xs[i % 2], o, idx, sc, ws=ews)
        kc, vc = kv_views(idx, sc, o)
        nsn.nsn_decode_attention(cb, q, kc, vc, out, w.L, ws=dws)

    for i in range(a.warmup):
        step(i)
    ms_step = timed(step, a.steps, torch)
    print(f"# step {ms_step:.4f} ms", file=sys.stderr, flush=True)

    # phase timings: encode alone; the per-token kernel alone (reused o skips the
    # two mean kernels); decode alone over rotated cache copies
    t_enc = timing(lambda i: nsn.nsn_encode(cb, xs[i % 2], o, idx, sc, ws=ews), it, torch)
    t_kenc = timing(lambda i: nsn.nsn_encode(cb, xs[i % 2], o, idx, sc, o_mode=nsn.NSN_O_REUSE), it, torch)
    cache_bytes = BH * w.L * 2 * (m + 4)
    ncopy = max(2, -(-ROTATE_BYTES // cache_bytes))
    copies = [(idx.clone(), sc.clone(), o.clone()) for _ in range(ncopy)]

    def dec(i):
        kc, vc = kv_views(*copies[i % ncopy])
        nsn.nsn_decode_attention(cb, q, kc, vc, out, w.L, ws=dws)

    t_dec = timing(dec, max(it, 2 * ncopy), torch)
    ms_enc, ms_k_encode, ms_dec = t_enc["steady_ms"], t_kenc["steady_ms"], t_dec["steady_ms"]
    print(f"# encode {ms_enc:.4f} ms (per-token kernel {ms_k_encode:.4f} ms), decode {ms_dec:.4f} ms", file=sys.stderr,
          flush=True)
    del copies

    # the NEXT rows on the same layer: decode with a 128-token fp16 residual window,
    # and the double-quantized cache (encode of the step input, decode over rotated
    # copies); decode bytes are algorithmic (cache records, plus the residual rows)
    extra = {}
    if not a.no_extras:
        R = 128
        kres = torch.randn((w.B, w.Hkv, R, w.d), device=dev).to(torch.float16)
        vres = torch.randn((w.B, w.Hkv, R, w.d), device=dev).to(torch.float16)
        copies = [(idx.clone(), sc.clone(), o.clone()) for _ in range(ncopy)]

        def dec_res(i):
            kc, vc = kv_views(*copies[i % ncopy])
            nsn.nsn_decode_attention_residual(cb, q, kc, vc, kres, vres, out, w.L, R, ws=dws)

        for i in range(3):
            dec_res(i)
        ms_res = timed(dec_res, max(a.steps, 2 * ncopy), torch)
        del copies
        capb = (w.L + 1) // 2
        dq = (torch.empty((2 * w.B, w.Hkv, w.L, m), dtype=torch.uint8, device=dev),
              torch.empty((2 * w.B, w.Hkv, w.L), dtype=torch.float16, device=dev),
              torch.empty((2 * w.B, w.Hkv, capb), dtype=torch.uint8, device=dev),
              torch.empty((2 * w.B, w.Hkv, nsn.DQ_HEAD_BYTES), dtype=torch.uint8, device=dev))
        dws_dq = torch.empty(nsn.nsn_encode_dq_workspace_size(2 * w.B, w.Hkv, w.L), dtype=torch.uint8, device=dev)
        nsn.nsn_encode_dq(cb, xs[0], dq, ws=dws_dq)
        ms_dq_enc = timed(lambda i: nsn.nsn_encode_dq(cb, xs[i % 2], dq, ws=dws_dq), a.steps, torch)
        dq_bytes = BH * w.L * 2 * (m + 2.5)
        ncopy_dq = max(2, -(-ROTATE_BYTES // int(dq_bytes)))
        dq_copies = [tuple(t.clone() for t in dq) for _ in range(ncopy_dq)]

        def dec_dq(i):
            c = dq_copies[i % ncopy_dq]
            nsn.nsn_decode_attention_dq(cb, q, tuple(t[:w.B] for t in c), tuple(t[w.B:] for t in c), out, w.L,
                                        ws=dws)

        for i in range(3):
            dec_dq(i)
        ms_dq_dec = timed(dec_dq, max(a.steps, 2 * ncopy_dq), torch)
        del dq_copies
        # keys quantized before RoPE: the same cache scored with each key rotated by its position
        rws = torch.empty(nsn.nsn_decode_rope_workspace_size(w.B, w.Hq, w.Hkv, w.L), dtype=torch.uint8, device=dev)
        copies = [(idx.clone(), sc.clone(), o.clone()) for _ in range(ncopy)]

        def dec_rope(i):
            kc, vc = kv_views(*copies[i % ncopy])
            nsn.nsn_decode_attention_rope(cb, q, kc, vc, out, w.L, ws=rws)

        for i in range(3):
            dec_rope(i)
        ms_rope = timed(dec_rope, max(a.steps, 2 * ncopy), torch)
        # the same decode with the cos / sin tables built once for the cache length
        rtab = nsn.nsn_rope_tables(w.L, device=dev)
        rws_t = torch.empty(nsn.nsn_decode_rope_tables_workspace_size(w.B, w.Hq, w.Hkv, w.L), dtype=torch.uint8,
                            device=dev)

        def dec_rope_t(i):
            kc, vc = kv_views(*copies[i % ncopy])
            nsn.nsn_decode_attention_rope_tables(cb, q, kc, vc, out, w.L, rtab, w.L, ws=rws_t)

        for i in range(3):
            dec_rope_t(i)
        ms_rope_t = timed(dec_rope_t, max(a.steps, 2 * ncopy), torch)
        del copies, rtab
        # the same layer at 1 bit (8-dimensional sub-vectors, the g = 8 codebook)
        m8 = w.d // 8
        idx8 = torch.empty((2 * w.B, w.Hkv, w.L, m8), dtype=torch.uint8, device=dev)
        sc8, o8 = torch.empty_like(sc), torch.empty_like(o)
        nsn.nsn_encode(cb8, xs[0], o8, idx8, sc8, ws=ews)
        ms_enc8 = timed(lambda i: nsn.nsn_encode(cb8, xs[i % 2], o8, idx8, sc8, ws=ews), a.steps, torch)
        ms_k8 = timed(lambda i: nsn.nsn_encode(cb8, xs[i % 2], o8, idx8, sc8, o_mode=nsn.NSN_O_REUSE), a.steps,
                      torch)
        bytes8 = BH * w.L * 2 * (m8 + 4)
        ncopy8 = max(2, -(-ROTATE_BYTES // bytes8))
        copies = [(idx8.clone(), sc8.clone(), o8.clone()) for _ in range(ncopy8)]

        def dec8(i):
            kc, vc = kv_views(*copies[i % ncopy8])
            nsn.nsn_decode_attention(cb8, q, kc, vc, out, w.L, ws=dws)

        for i in range(3):
            dec8(i)
        ms_dec8 = timed(dec8, max(a.steps, 2 * ncopy8), torch)
        del copies
        # the randomized Hadamard option (a seeded 16-byte channel-sign mask) on the same layer
        nsn.nsn_encode(cbr, xs[0], o, idx, sc, ws=ews)
        ms_enc_r = timed(lambda i: nsn.nsn_encode(cbr, xs[i % 2], o, idx, sc, ws=ews), a.steps, torch)
        copies = [(idx.clone(), sc.clone(), o.clone()) for _ in range(ncopy)]

        def dec_r(i):
            kc, vc = kv_views(*copies[i % ncopy])
            nsn.nsn_decode_attention(cbr, q, kc, vc, out, w.L, ws=dws)

        for i in range(3):
            dec_r(i)
        ms_dec_r = timed(dec_r, max(a.steps, 2 * ncopy), torch)
        del copies
        res_bytes = BH * w.L * 2 * (m + 4) + BH * R * 2 * w.d * 2
        extra = {
            "randomized_hadamard": {"encode_ms": ms_enc_r,
                                    "encode_tokens_per_s": w.B * w.L / (ms_enc_r * 1e-3),
                                    "decode_ms": ms_dec_r,
                                    "decode_GBps": BH * w.L * 2 * (m + 4) / (ms_dec_r * 1e-3) / 1e9},
            "one_bit": {"encode_ms": ms_enc8, "encode_tokens_per_s": w.B * w.L / (ms_enc8 * 1e-3),
                        "kernel_ms": ms_k8,
                        "kernel_hbm_frac": 2 * BH * w.L * (256 + m8 + 4) / (ms_k8 * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                        "decode_ms": ms_dec8, "decode_GBps": bytes8 / (ms_dec8 * 1e-3) / 1e9,
                        "decode_hbm_frac": bytes8 / (ms_dec8 * 1e-3) / 1e9 / HBM_PEAK_GBPS},
            "residual_window": {"R": R, "decode_ms": ms_res,
                                "decode_GBps": res_bytes / (ms_res * 1e-3) / 1e9},
            "double_quant": {"encode_ms": ms_dq_enc, "encode_tokens_per_s": w.B * w.L / (ms_dq_enc * 1e-3),
                             "decode_ms": ms_dq_dec, "decode_GBps": dq_bytes / (ms_dq_dec * 1e-3) / 1e9,
                             "decode_bytes_per_token_head": 2 * (m + 2.5),
                             "scale_bits_per_element": 20 / w.d},
            "keys_pre_rope": {"decode_ms": ms_rope,
                              "decode_GBps": BH * w.L * 2 * (m + 4) / (ms_rope * 1e-3) / 1e9,
                              "prepared_tables_decode_ms": ms_rope_t,
                              "prepared_tables_decode_GBps": BH * w.L * 2 * (m + 4) / (ms_rope_t * 1e-3) / 1e9},
        }
        print(f"# residual decode (R={R}) {ms_res:.4f} ms; DQ encode {ms_dq_enc:.4f} ms, DQ decode {ms_dq_dec:.4f} ms;"
              f" pre-RoPE-key decode {ms_rope:.4f} ms ({ms_rope_t:.4f} ms with prepared tables)", file=sys.stderr,
              flush=True)
        print(f"# 1-bit: encode {ms_enc8:.4f} ms (per-token kernel {ms_k8:.4f} ms), decode {ms_dec8:.4f} ms",
              file=sys.stderr, flush=True)
        print(f"# randomized Hadamard: encode {ms_enc_r:.4f} ms, decode {ms_dec_r:.4f} ms", file=sys.stderr,
              flush=True)
    del xs
    torch.cuda.empty_cache()
    measured = copy_rates(torch, dev)
    print(f"# copy {measured['copy_GBps']:.0f} GB/s, streaming read {measured['read_GBps']:.0f} GB/s", file=sys.stderr,
          flush=True)

    enc_b, dec_b, enc_f, enc_c = algorithmic(w)
    nvec = 2 * BH * w.L
    tokens = w.B * w.L
    enc_tok_s = tokens / (ms_enc * 1e-3)
    dec_bytes = BH * w.L * dec_b
    dec_gbps = dec_bytes / (ms_dec * 1e-3) / 1e9
    # dominant kernel: the per-token encode kernel, against HBM on its algorithmic
    # bytes (x read once, indices and the scale pair written), timed alone (the
    # reused-o mode launches only it) on the stream it runs on
    k_bytes = nvec * enc_b
    achieved = k_bytes / (ms_k_encode * 1e-3) / 1e9
    k_ops = nvec * enc_c
    line = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "seq_len": w.L,
                   "head_dim": w.d, "bits": w.bits, "subvector": w.g, "codebook": 256, "input": w.dtype,
                   "parallelism": "none (1 GPU)"},
        "encode_tokens_per_s": enc_tok_s,
        "encode_ms": ms_enc,
        "encode_hbm_frac": nvec * enc_b / (ms_enc * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "encode_timing": t_enc,
        "decode_ms": ms_dec,
        "decode_GBps": dec_gbps,
        "decode_hbm_frac": dec_gbps / HBM_PEAK_GBPS,
        "decode_hbm_frac_of_measured_read": dec_gbps / measured["read_GBps"],
        "decode_timing": t_dec,
        "roofline": {"bound": "hbm", "kernel": "k_encode (NSN + Hadamard + nearest centroid + alpha)",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic() if a.workload == "mistral7b-long-2bit" else None,
                     "bytes_per_launch": k_bytes, "kernel_ms": ms_k_encode, "kernel_timing": t_kenc,
                     "frac_of_measured_read": achieved / measured["read_GBps"],
                     "exhaustive_equiv_compares_per_s": k_ops / (ms_k_encode * 1e-3)},
        "measured_peaks": measured,
        "configs": configs,
    }
    line.update(extra)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, C, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
