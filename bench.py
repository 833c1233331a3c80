"""Benchmark of the NSNQuant hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
encode K and V of every KV head (NSN + Hadamard + nearest centroid + scale),
then decode attention of every query head over the freshly quantized cache.
Default workload: the Mistral-7B-like long-context layer (batch 1, 32 query /
8 KV heads, 131072 tokens, head_dim 128, fp16 inputs with Student-t(3) channel
offsets, 2-bit VQ = 4-dim sub-vectors x 256 centroids).

Prints ONE JSON line.  `value` is encode tokens per second of the whole step
(tokens = K and V of all KV heads of the layer).  Extra keys carry the
per-phase figures: encode tokens/s, decode GB/s over the algorithmic cache
bytes (measured on rotated caches so that the 256 MB last-level cache cannot
serve repeats), the roofline of the dominant kernel and the oracle's CPU rate.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encode tokens/s and decode-attn GB/s (% HBM roofline) at 1/2-bit, head_dim 128"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="mistral7b-long-2bit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample duration")
    ap.add_argument("--copy-probe", action="store_true", help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the residual-window and double-quantization timings")
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


def tokens_step(w):
    return w.B * w.L


def timed(fn, iters, torch):
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(iters):
        fn(i)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters  # ms


def cpu_baseline(w, C, target_s):
    """Time the fp64 oracle on a bounded sample of the same workload: for KV head
    after KV head (up to all of them), K and V of that head (NSN over all sample
    tokens, nearest centroid, scale) plus the decode attention of its query heads
    over the sample, until about target_s seconds have run; scaled to the layer."""
    import numpy as np

    import oracle
    import synthetic

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    GQ = w.Hq // w.Hkv
    Ls = min(w.L, 65536)
    spent, heads = 0.0, 0
    while heads < w.Hkv and spent < target_s:
        K, V = synthetic.make_kv_numpy(99 + heads, 1, 1, Ls, w.d, w.kind, w.dtype)
        q = np.random.default_rng(99 + heads).standard_normal((1, GQ, w.d)).astype(np.float16).astype(np.float64)
        t = time.perf_counter()
        rk = oracle.encode_head(K[0, 0].astype(np.float64), C, w.g)
        rv = oracle.encode_head(V[0, 0].astype(np.float64), C, w.g)
        kc = tuple(a[None, None] for a in (rk["idx"], rk["s1"], rk["s2p"])) + (rk["o"][None, None],)
        vc = tuple(a[None, None] for a in (rv["idx"], rv["s1"], rv["s2p"])) + (rv["o"][None, None],)
        oracle.decode_attention(q, *kc, *vc, C, w.g)
        spent += time.perf_counter() - t
        heads += 1
    per_token_s = spent / heads * w.Hkv / Ls  # all KV heads of the layer
    return {"value": 1.0 / per_token_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} KV head(s) x {Ls} tokens (K+V encode, {GQ}-head decode each) in {spent:.1f} s, "
                      f"scaled to {w.Hkv} KV heads"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "single-GPU build: this path runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import kv_cache_vector_nsn_amd as nsn
    import synthetic
    from tests.golden_io import load_codebook  # stored N(0,1) k-means codebook (an input)

    w = synthetic.WORKLOADS[a.workload]
    dev = torch.device("cuda:0")
    C, _ = load_codebook(w.g)
    cb = nsn.nsn_codebook_create(C.astype(np.float32), w.g)
    # the randomized Hadamard option's handle (a seeded 16-byte channel-sign mask), built
    # here so that its candidate-table kernel runs before any timed region
    cbr = None if a.no_extras else nsn.nsn_codebook_create_rht(
        C.astype(np.float32), bytes(np.random.default_rng(20250523).integers(0, 256, 16, dtype=np.uint8)), w.g)
    cb8 = None if a.no_extras else nsn.nsn_codebook_create(load_codebook(8)[0].astype(np.float32), 8)
    m = w.d // w.g
    GQ = w.Hq // w.Hkv
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
    ms_enc = timed(lambda i: nsn.nsn_encode(cb, xs[i % 2], o, idx, sc, ws=ews), a.steps, torch)
    ms_k_encode = timed(lambda i: nsn.nsn_encode(cb, xs[i % 2], o, idx, sc, o_mode=nsn.NSN_O_REUSE), a.steps, torch)
    cache_bytes = BH * w.L * 2 * (m + 4)
    ncopy = max(2, -(-600_000_000 // cache_bytes))
    copies = [(idx.clone(), sc.clone(), o.clone()) for _ in range(ncopy)]

    def dec(i):
        kc, vc = kv_views(*copies[i % ncopy])
        nsn.nsn_decode_attention(cb, q, kc, vc, out, w.L, ws=dws)

    for i in range(3):
        dec(i)
    ms_dec = timed(dec, max(a.steps, 2 * ncopy), torch)
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
        ncopy_dq = max(2, -(-600_000_000 // int(dq_bytes)))
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
        del copies
        # the same layer at 1 bit (8-dimensional sub-vectors, the g = 8 codebook)
        m8 = w.d // 8
        idx8 = torch.empty((2 * w.B, w.Hkv, w.L, m8), dtype=torch.uint8, device=dev)
        sc8, o8 = torch.empty_like(sc), torch.empty_like(o)
        nsn.nsn_encode(cb8, xs[0], o8, idx8, sc8, ws=ews)
        ms_enc8 = timed(lambda i: nsn.nsn_encode(cb8, xs[i % 2], o8, idx8, sc8, ws=ews), a.steps, torch)
        ms_k8 = timed(lambda i: nsn.nsn_encode(cb8, xs[i % 2], o8, idx8, sc8, o_mode=nsn.NSN_O_REUSE), a.steps,
                      torch)
        bytes8 = BH * w.L * 2 * (m8 + 4)
        ncopy8 = max(2, -(-600_000_000 // bytes8))
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
                                    "encode_tokens_per_s": tokens_step(w) / (ms_enc_r * 1e-3),
                                    "decode_ms": ms_dec_r,
                                    "decode_GBps": BH * w.L * 2 * (m + 4) / (ms_dec_r * 1e-3) / 1e9},
            "one_bit": {"encode_ms": ms_enc8, "encode_tokens_per_s": tokens_step(w) / (ms_enc8 * 1e-3),
                        "kernel_ms": ms_k8,
                        "kernel_hbm_frac": 2 * BH * w.L * (256 + m8 + 4) / (ms_k8 * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                        "decode_ms": ms_dec8, "decode_GBps": bytes8 / (ms_dec8 * 1e-3) / 1e9,
                        "decode_hbm_frac": bytes8 / (ms_dec8 * 1e-3) / 1e9 / HBM_PEAK_GBPS},
            "residual_window": {"R": R, "decode_ms": ms_res,
                                "decode_GBps": res_bytes / (ms_res * 1e-3) / 1e9},
            "double_quant": {"encode_ms": ms_dq_enc, "encode_tokens_per_s": tokens_step(w) / (ms_dq_enc * 1e-3),
                             "decode_ms": ms_dq_dec, "decode_GBps": dq_bytes / (ms_dq_dec * 1e-3) / 1e9,
                             "decode_bytes_per_token_head": 2 * (m + 2.5),
                             "scale_bits_per_element": 20 / w.d},
            "keys_pre_rope": {"decode_ms": ms_rope,
                              "decode_GBps": BH * w.L * 2 * (m + 4) / (ms_rope * 1e-3) / 1e9},
        }
        print(f"# residual decode (R={R}) {ms_res:.4f} ms; DQ encode {ms_dq_enc:.4f} ms, DQ decode {ms_dq_dec:.4f} ms;"
              f" pre-RoPE-key decode {ms_rope:.4f} ms", file=sys.stderr, flush=True)
        print(f"# 1-bit: encode {ms_enc8:.4f} ms (per-token kernel {ms_k8:.4f} ms), decode {ms_dec8:.4f} ms",
              file=sys.stderr, flush=True)
        print(f"# randomized Hadamard: encode {ms_enc_r:.4f} ms, decode {ms_dec_r:.4f} ms", file=sys.stderr,
              flush=True)
    if a.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        ms_copy = timed(lambda i: dst.copy_(src), 5, torch)
        print(f"# copy 1 GiB: {ms_copy:.4f} ms ({2 * src.numel() * 4 / ms_copy / 1e6:.0f} GB/s)", file=sys.stderr)

    enc_b, dec_b, enc_f, enc_c = algorithmic(w)
    nvec = 2 * BH * w.L
    tokens = w.B * w.L
    enc_tok_s = tokens / (ms_enc * 1e-3)
    dec_bytes = BH * w.L * dec_b
    dec_gbps = dec_bytes / (ms_dec * 1e-3) / 1e9
    # dominant kernel: the per-token encode kernel, against HBM on its algorithmic
    # bytes (x read once, indices and scale pair written); the exhaustive-search
    # equivalent compare rate is reported beside it for context
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
        "decode_ms": ms_dec,
        "decode_GBps": dec_gbps,
        "decode_hbm_frac": dec_gbps / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "kernel": "k_encode (NSN + Hadamard + nearest centroid + alpha)",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic() if a.workload == "mistral7b-long-2bit" else None,
                     "bytes_per_launch": k_bytes, "kernel_ms": ms_k_encode,
                     "exhaustive_equiv_compares_per_s": k_ops / (ms_k_encode * 1e-3)},
    }
    line.update(extra)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, C, a.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
