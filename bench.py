#!/usr/bin/env python3
"""Benchmark of the DF11 decode hot path on one MI355X.

Default workload: one Llama-3-8B-shaped decoder layer of synthetic
N(0, 0.02) BF16 weights (q, k, v, o, gate, up, down: 218,103,808 elements)
with one codebook for the layer, compressed and resident in HBM.  One step
decodes all seven matrices in one launch (df11_decode_batch), each into its
slice of one reused layer-sized BF16 buffer.

Also reported: the seven matrices one launch each into one reused
matrix-sized buffer (eager, and replayed as one HIP graph), the whole
8B-parameter model (226 matrices) per pass, compressed CPU offload, the GPU
encoder, and the fused decode+GEMM on up_proj at B in {1, 8, 64, 256}.

Prints one JSON line:
  value     decoded BF16 GB/s (2 bytes per element / step time)
  roofline  the decode kernel's algorithmic HBM bytes per launch / its
            average launch time (HIP events on the launch stream; one launch
            per step), against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle's bit-serial decode of the same layer, timed
            on this host's allowed cores (one thread each; also on one core)

    python bench.py [--steps K] [--warmup W] [--no-model] [--no-fused] [--no-shard] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(enc) -> int:
    """Bytes a decode must move: the exponent stream, one sign+mantissa byte
    per element, the per-lane gaps and code counts, the per-segment records,
    and the BF16 output (2 bytes per element)."""
    stream = (enc.total_bits + 7) // 8
    return stream + enc.n + enc.n_segments * 128 + (enc.n_segments + 1) * 16 + 2 * enc.n


def measured_traffic(profile: str, sources) -> float | None:
    """HBM bytes per decode launch from the committed rocprofv3 summary
    (FETCH_SIZE and WRITE_SIZE, calibrated against a plain copy), or None
    when the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("|", "#", "(", "`")):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


DECODE_SOURCES = ("huffman_decode_df11_amd/csrc/decode.hip", "huffman_decode_df11_amd/csrc/df11_device.h")


def build_layer(seed: int = 0):
    from huffman_decode_df11_amd import api, synth
    t0 = time.time()
    mats = synth.llama_layer(seed=seed, layer=0)
    hist = None
    for _, m in mats:
        hist = api.hist_accumulate(m, hist)
    cb = api.build_codebook(hist)
    encs = [(name, m, api.encode(m, codebook=cb)) for name, m in mats]
    log("layer generated and encoded in %.1f s" % (time.time() - t0))
    return encs


def _hold_queue(ms: float):
    """Put a bounded spin kernel at the head of the stream, so that the host
    enqueues the timed launches while the GPU is busy and the events then
    see kernel durations, not host launch gaps."""
    import torch
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is not None:
        sleep(int(ms * 1e-3 * 2.4e9))


def time_decode(dts, outbuf, steps: int, warmup: int):
    """Per-matrix launch durations and the eager layer loop.

    For each matrix, `steps` back-to-back launches into the reused buffer
    between two events on the launch stream, with the queue held busy so
    that the host runs ahead: the average is the kernel duration plus the
    dispatch gap between consecutive kernels.  Then `steps` passes of the
    seven launches issued one by one from Python, without the hold.
    Returns ([tensors] per-launch ms, eager ms per pass)."""
    import torch
    from huffman_decode_df11_amd import api
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for dt in dts:
            api.decode(dt, out=outbuf, stream=stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in dts]
    _hold_queue(2.0 + 0.05 * steps * len(dts))
    for (a, b), dt in zip(ev, dts):
        a.record(stream)
        for _ in range(steps):
            api.decode(dt, out=outbuf, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([a.elapsed_time(b) / steps for a, b in ev])
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        for dt in dts:
            api.decode(dt, out=outbuf, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    return per_launch, start.elapsed_time(stop) / steps


def time_batched(dts, steps: int, warmup: int):
    """One df11_decode_batch launch per step over all tensors, each into its
    own slice of one reused layer-sized buffer.  The queue is held busy
    while the host enqueues the timed launches (as for the per-matrix
    times), so the events bracket back-to-back launches and not the wake-up
    of an idle GPU after the synchronize."""
    import torch
    from huffman_decode_df11_amd import api
    total = sum(((dt.n + 7) // 8) * 8 for dt in dts)
    buf = torch.empty(total, dtype=torch.bfloat16, device="cuda")
    outs, off = [], 0
    for dt in dts:
        outs.append(buf[off:off + dt.n])
        off += ((dt.n + 7) // 8) * 8
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        api.decode_batch(dts, outs=outs, stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _hold_queue(2.0 + 0.2 * steps)
    a.record(stream)
    for _ in range(steps):
        api.decode_batch(dts, outs=outs, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps, outs


def time_graph(dts, outbuf, steps: int, warmup: int):
    """The per-matrix launches captured once in a HIP graph and replayed."""
    import torch
    from huffman_decode_df11_amd import api
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for dt in dts:
            api.decode(dt, out=outbuf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for dt in dts:
            api.decode(dt, out=outbuf)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def model_pass(steps: int, warmup: int, seed: int = 0):
    """The 8B-parameter model (32 layers, embedding, LM head; 226 matrices,
    8,029,995,008 elements, one codebook per layer): every matrix decoded
    into one reused buffer, as eager launches, as one HIP graph, and as one
    batched launch per layer."""
    import torch
    from huffman_decode_df11_amd import model as mdl
    t0 = time.time()
    m = mdl.synthetic_llama3_8b(seed=seed, device="cuda")
    t_build = time.time() - t0
    checked = mdl.verify_pass(m, seed)
    log("8B model built in %.1f s; all %d elements decoded and verified" % (t_build, checked))
    alg = sum((t.total_bits + 7) // 8 + t.n + t.n_segments * 144 + 16 + 2 * t.n for _, _, t in m.matrices)

    def timeit(f, n):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n = max(3, steps // 4)
    t_eager = timeit(m.decode_pass, n)
    t_graph = timeit(m.capture(), n)
    t_batched = timeit(m.decode_pass_batched, n)
    out = {
        "workload": "llama3-8b model: embedding, 32 layers, LM head, bf16 N(0,0.02), "
                    "%d elements in %d matrices, one codebook per layer, one reused buffer" % (
                        m.n_elements, len(m.matrices)),
        "elements": m.n_elements,
        "compressed_bytes": m.compressed_nbytes(),
        "bf16_bytes": 2 * m.n_elements,
        "bits_per_weight": round(8.0 * m.compressed_nbytes() / m.n_elements, 4),
        "build_s": round(t_build, 1),
        "verified_elements": checked,
        "passes_timed": n,
    }
    for name, t, launches in (("graph", t_graph, len(m.matrices)), ("eager", t_eager, len(m.matrices)),
                              ("batched_per_layer", t_batched, len(m.groups))):
        out[name] = {"ms_per_pass": round(t, 3), "launches": launches,
                     "decoded_gbs": round(2.0 * m.n_elements / (t * 1e-3) / 1e9, 1),
                     "hbm_frac": round(alg / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del m
    torch.cuda.empty_cache()
    return out


def offload_pass(steps: int, warmup: int, seed: int = 0, layers: int = 4):
    """Compressed CPU offload: `layers` decoder layers of the 8B model held in
    pinned host memory, each streamed to the GPU one layer ahead of its
    decode; next to a plain host-to-device copy of the same layers in BF16."""
    import torch
    from huffman_decode_df11_amd import model as mdl
    from huffman_decode_df11_amd.offload import OffloadedModel
    groups = mdl.encode_llama3_8b(seed=seed, device="cuda", layers=layers, embed_and_head=False)
    off = OffloadedModel(groups)
    out = torch.empty(off.max_elements, dtype=torch.bfloat16, device="cuda")
    got = []
    off.decode_pass(out, on_matrix=lambda g, name, o: got.append(o.view(torch.int16)[:16].clone()))
    torch.cuda.synchronize()
    specs = [sp for sp in __import__("huffman_decode_df11_amd.synth", fromlist=["x"]).llama3_8b_tensors(layers)
             if sp[0] not in ("embed", "head")]
    # spot check: the first 16 elements of every matrix against the generator
    from huffman_decode_df11_amd import synth
    for k, ((g, name, r, c), o) in enumerate(zip(specs, got)):
        want = synth.normal_bf16_torch(r, c, seed, k + 1, "cuda").view(torch.int16).reshape(-1)[:16]
        if not torch.equal(o, want):
            raise SystemExit("offload parity check failed at %s %s" % (g, name))

    def timeit(f, n):
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    n = max(2, steps // 5)
    t_off = timeit(lambda: off.decode_pass(out), n)
    host = off.host_nbytes()
    bf16_bytes = 2 * off.n_elements
    src = torch.empty(bf16_bytes // 2, dtype=torch.int16, pin_memory=True)
    dst = torch.empty(bf16_bytes // 2, dtype=torch.int16, device="cuda")
    t_bf16 = timeit(lambda: dst.copy_(src, non_blocking=True), n)
    res = {
        "workload": "%d llama3-8b layers (%d elements) compressed in pinned host memory, "
                    "streamed layer by layer through two device slots" % (layers, off.n_elements),
        "host_bytes_per_pass": host,
        "ms_per_pass": round(t_off, 3),
        "pcie_gbs": round(host / (t_off * 1e-3) / 1e9, 2),
        "decoded_gbs": round(bf16_bytes / (t_off * 1e-3) / 1e9, 2),
        "bf16_copy_ms": round(t_bf16, 3),
        "bf16_copy_gbs": round(bf16_bytes / (t_bf16 * 1e-3) / 1e9, 2),
        "bytes_saved_vs_bf16": round(1 - host / bf16_bytes, 4),
    }
    del off, out, src, dst, groups
    torch.cuda.empty_cache()
    return res


def encode_rate(seed: int = 0):
    """Encoding up_proj (14336 x 4096) on the GPU (histogram, codebook on the
    host, df11_encode_device) next to the host encoder on one thread."""
    import torch
    from huffman_decode_df11_amd import api, synth
    N, K = 14336, 4096
    w = synth.normal_bf16_torch(N, K, seed, 99, "cuda")
    api.encode_device(w)      # warm-up (library load, kernels)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        d = api.encode_device(w)
    torch.cuda.synchronize()
    t_dev = (time.perf_counter() - t0) / reps
    u = w.view(torch.int16).cpu().numpy().view(np.uint16)
    t0 = time.perf_counter()
    h = api.encode(u)
    t_host = time.perf_counter() - t0
    same = all(np.array_equal(h.arrays[k], d.to_host().arrays[k]) for k in ("exp_words", "sm", "gaps", "segs"))
    return {"workload": "encode up_proj 14336x4096 bf16 N(0,0.02), codebook from its own histogram",
            "device_ms": round(t_dev * 1e3, 2), "device_bf16_gbs": round(2 * N * K / t_dev / 1e9, 1),
            "host_one_thread_ms": round(t_host * 1e3, 1), "identical_to_host_encoder": bool(same)}


def fused_up_proj(steps: int, warmup: int, seed: int = 0, copies: int = 8, rows: int = 14336):
    """df11_decode_gemm on the up_proj weight (14336 x 4096; or its first
    `rows` rows, one GPU's share of a row split) for B in {1, 8, 64, 256},
    next to torch.matmul on the BF16 weight and to the unfused path
    (df11_decode of a row-major encoding, then torch.matmul).  Every variant
    cycles through `copies` copies of its weight (> 256 MB in all), so
    weights come from HBM and not from the 256 MB Infinity Cache; x and y
    stay small and warm, as activations do."""
    import torch
    from huffman_decode_df11_amd import api, synth
    N, K = rows, 4096
    W = synth.normal_bf16(14336 * K, 0.02, seed=seed, index=5, count=7).reshape(14336, K)[:N].copy()
    enc = api.encode(W, layout=api.gemm_layout(N, K))
    enc_rm = api.encode(W, codebook=enc.codebook)
    dts = [enc.to("cuda") for _ in range(copies)]
    dts_rm = [enc_rm.to("cuda") for _ in range(copies)]
    w0 = torch.from_numpy(W.view(np.int16)).cuda().view(torch.bfloat16)
    wts = [w0] + [w0.clone() for _ in range(copies - 1)]
    wbuf = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    w_bytes = enc.compressed_nbytes()

    def timeit(f):
        for i in range(max(warmup, copies)):   # every copy touched before timing
            f(i % copies)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            f(i % copies)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    by_b = {}
    for B in (1, 8, 64, 256):
        X = synth.activations_bf16(B, K, seed=1)
        x = torch.from_numpy(X.view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty(B, N, dtype=torch.float32, device="cuda")
        api.decode_gemm(dts[0], x, out=y)
        yt = x.float() @ w0.float().T
        torch.cuda.synchronize()
        rel = float((y - yt).norm() / yt.norm())
        if not rel < 2e-3:
            raise SystemExit("fused decode+GEMM parity failed at B=%d (rel %.3g)" % (B, rel))
        t_fused = timeit(lambda i: api.decode_gemm(dts[i], x, out=y))
        t_plain = timeit(lambda i: torch.matmul(x, wts[i].T))
        t_unfused = timeit(lambda i: torch.matmul(x, api.decode(dts_rm[i], out=wbuf).T))
        flops = 2.0 * B * N * K
        alg = w_bytes + B * K * 2 + B * N * 4
        mfma_bound = flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) > alg / (HBM_PEAK_GBS * 1e9)
        by_b[str(B)] = {
            "fused_ms": round(t_fused, 4),
            "fused_tflops": round(flops / t_fused / 1e9, 2),
            "plain_bf16_matmul_ms": round(t_plain, 4),
            "decode_then_matmul_ms": round(t_unfused, 4),
            "fused_over_plain": round(t_fused / t_plain, 3),
            "rel_err_vs_fp32": rel,
            "roofline": ({"bound": "mfma", "achieved": round(flops / t_fused / 1e9, 2),
                          "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(flops / t_fused / 1e9 / BF16_MFMA_PEAK_TFLOPS, 4)}
                         if mfma_bound else
                         {"bound": "hbm", "achieved": round(alg / t_fused / 1e6, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(alg / t_fused / 1e6 / HBM_PEAK_GBS, 4)}),
        }
    what = "up_proj 14336x4096" if N == 14336 else "rows 0..%d of up_proj 14336x4096 (one GPU's share of an %d-way row split)" % (N - 1, 14336 // N)
    return {"workload": what + " bf16 N(0,0.02), x[B,4096] N(0,1), y float32; each variant cycles "
                        "through %d copies of its weight" % copies,
            "compressed_weight_bytes": w_bytes, "by_batch": by_b}


def other_configs(steps: int, warmup: int, seed: int = 0):
    """The two other decode workloads, one df11_decode launch per step: a
    1024 x 1024 N(0, 0.02) tensor (launch-bound; the same tensor again and
    again) and 16,777,216 elements of 99% Student-t(3) x 0.02 plus 1% random
    16-bit patterns (every exponent, the longest codes; 12 copies cycled so
    the compressed data comes from HBM).  Parity is checked in full first."""
    import torch
    from huffman_decode_df11_amd import api, synth
    out = {}
    for name, u, copies in (("tensor_1024x1024", synth.tensor_1024(seed=seed).reshape(-1), 1),
                            ("adversarial_16m", synth.adversarial_bf16(1 << 24, seed=seed), 12)):
        enc = api.encode(u)
        dts = [enc.to("cuda") for _ in range(copies)]
        buf = torch.empty(u.size, dtype=torch.bfloat16, device="cuda")
        api.decode(dts[0], out=buf)
        torch.cuda.synchronize()
        if not np.array_equal(buf.view(torch.int16).cpu().numpy().view(np.uint16), u):
            raise SystemExit("parity failed on " + name)
        for i in range(max(warmup, copies)):
            api.decode(dts[i % copies], out=buf)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_launch = max(steps, 50)
        _hold_queue(2.0 + 0.05 * n_launch)
        a.record()
        for i in range(n_launch):
            api.decode(dts[i % copies], out=buf)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / n_launch
        alg = algorithmic_bytes(dts[0])
        out[name] = {"elements": int(u.size), "us_per_launch": round(ms * 1e3, 2),
                     "decoded_gbs": round(2.0 * u.size / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "bits_per_weight": round(enc.compressed_nbytes() * 8.0 / u.size, 3),
                     "copies_cycled": copies}
    return out


def embedding_lookup(steps: int, warmup: int, seed: int = 0, vocab: int = 128256, dim: int = 4096):
    """df11_decode_rows (the DF11Embedding lookup) on a vocabulary-sized table,
    128256 x 4096 bf16 N(0, 0.02) in the row-major layout: B random token ids
    per call (B = 1, 32, 2048), every returned row checked bit-exactly, timed
    against torch's embedding gather on the BF16 table.  Algorithmic bytes
    per row: the row's compressed bytes (exponent bits at the table's mean
    code length plus one sign+mantissa byte per element) and its BF16 output."""
    import torch
    from huffman_decode_df11_amd import api, synth
    W = synth.normal_bf16_torch(vocab, dim, seed=seed, index=900, device="cuda")
    dt = api.encode_device(W, layout=api.make_layout(rows=vocab, cols=dim))
    row_alg = dim * (dt.total_bits / dt.n / 8.0 + 1.0) + 2.0 * dim
    rng = np.random.default_rng(seed + 77)

    def timeit(f, n):
        for _ in range(max(warmup, 3)):
            f()
        torch.cuda.synchronize()
        _hold_queue(2.0 + 0.05 * n)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    out = {"workload": "embedding table %dx%d bf16 N(0,0.02), row-major layout, B random token ids per call"
                       % (vocab, dim),
           "bits_per_weight": round(dt.compressed_nbytes() * 8.0 / dt.n, 4), "by_tokens": {}}
    for B in (1, 32, 2048):
        ids = torch.from_numpy(rng.integers(0, vocab, B)).cuda()
        buf = torch.empty(B, dim, dtype=torch.bfloat16, device="cuda")
        api.decode_rows(dt, ids, out=buf)
        torch.cuda.synchronize()
        if not torch.equal(buf.view(torch.int16), W[ids].view(torch.int16)):
            raise SystemExit("embedding lookup parity failed at B=%d" % B)
        n = max(steps, 50)
        us = timeit(lambda: api.decode_rows(dt, ids, out=buf), n)
        us_t = timeit(lambda: torch.nn.functional.embedding(ids, W), n)
        out["by_tokens"][str(B)] = {"us_per_call": round(us, 2), "torch_bf16_gather_us": round(us_t, 2),
                                    "rows_per_s": round(B / (us * 1e-6), 1),
                                    "hbm_frac": round(B * row_alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del W, dt
    torch.cuda.empty_cache()
    return out


def shard_layer_decode(steps: int, warmup: int, ways: int = 8, copies: int = 4, seed: int = 0):
    """One GPU's share of the layer under an `ways`-way row split: the first
    1/ways of the rows of each of the seven matrices, one codebook, decoded
    in one df11_decode_batch launch per step; the step cycles through
    `copies` copies of the encodings so the compressed data (> 256 MB in
    all) comes from HBM."""
    import torch
    from huffman_decode_df11_amd import api, synth
    mats = [(name, m[: m.shape[0] // ways].copy()) for name, m in synth.llama_layer(seed=seed, layer=0)]
    hist = None
    for _, m in mats:
        hist = api.hist_accumulate(m, hist)
    cb = api.build_codebook(hist)
    encs = [api.encode(m, codebook=cb) for _, m in mats]
    sets = [[e.to("cuda") for e in encs] for _ in range(copies)]
    n = sum(m.size for _, m in mats)
    outs = [torch.empty(m.size, dtype=torch.bfloat16, device="cuda") for _, m in mats]
    api.decode_batch(sets[0], outs=outs)
    torch.cuda.synchronize()
    for (_, m), o in zip(mats, outs):
        if not np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), m.reshape(-1)):
            raise SystemExit("shard decode parity failed")
    for i in range(max(warmup, copies)):
        api.decode_batch(sets[i % copies], outs=outs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _hold_queue(2.0 + 0.05 * steps)
    a.record()
    for i in range(steps):
        api.decode_batch(sets[i % copies], outs=outs)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    alg = sum(algorithmic_bytes(dt) for dt in sets[0])
    return {"workload": "rows 0..R/%d-1 of each of the seven llama3-8b layer matrices (%d elements), one launch"
                        % (ways, n), "elements": n, "ms_per_step": round(ms, 4),
            "decoded_gbs": round(2.0 * n / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def copy_peak(nbytes: int = 512 << 20, reps: int = 10):
    """Device-to-device copy rate (read + write bytes per second) of a
    buffer larger than the Infinity Cache: the practical HBM ceiling."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def verify(dts, mats, outbuf):
    import torch
    from huffman_decode_df11_amd import api
    for dt, m in zip(dts, mats):
        api.decode(dt, out=outbuf)
        torch.cuda.synchronize()
        got = outbuf.view(torch.int16)[:m.size].cpu().numpy().view(np.uint16)
        if not np.array_equal(got, m.reshape(-1)):
            raise SystemExit("parity check failed before timing")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_layer(mats, one_core_s: float = 12.0, all_cores_s: float = 10.0):
    """The oracle's serial decode on the host over the layer's matrices:
    first on one core (the loop pinned to the first CPU this process may
    use), then on every allowed core, one thread per core, each thread
    decoding whole matrices in turn (independent tensors; the oracle's C
    decode runs without the interpreter lock).  Returns (all cores, one
    core) baseline records."""
    from concurrent.futures import ThreadPoolExecutor
    import itertools
    from oracle import oracle as orc
    hist = None
    for m in mats:
        hist = orc.histogram(m) if hist is None else hist + orc.histogram(m)
    ln = orc.code_lengths(hist, 32)
    refs = [orc.encode(m, lengths=ln) for m in mats]
    allowed = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    cpu = _cpu_model()

    # one core
    if allowed:
        os.sched_setaffinity(0, {allowed[0]})
    elems, secs, passes = 0, 0.0, 0
    try:
        while passes == 0 or secs < one_core_s:
            for m, ref in zip(mats, refs):
                t0 = time.perf_counter()
                out = orc.decode(ref.E, ref.total_bits, ref.sm, ref.n, ln)
                secs += time.perf_counter() - t0
                elems += m.size
                if passes == 0 and not np.array_equal(out, m.reshape(-1)):
                    raise SystemExit("oracle round trip failed")
                del out
            passes += 1
    finally:
        if allowed:
            os.sched_setaffinity(0, set(allowed))
    one = {"value": round(2.0 * elems / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "bit-serial oracle decode of the layer's 7 matrices, %d passes (%d elements, %.1f s), "
                     "one host thread pinned to CPU %s of %d allowed (%s)" % (
                         passes, elems, secs, allowed[0] if allowed else "?", len(allowed), cpu)}

    # every allowed core: threads take matrices in turn until the budget is used
    threads = max(1, len(allowed))
    order = itertools.count()
    t_start = time.perf_counter()
    deadline = t_start + all_cores_s

    def worker(_):
        done = 0
        while True:
            i = next(order)
            if i >= threads and time.perf_counter() >= deadline:
                return done
            ref = refs[i % len(refs)]
            orc.decode(ref.E, ref.total_bits, ref.sm, ref.n, ln)
            done += ref.n
    with ThreadPoolExecutor(max_workers=threads) as ex:
        total = sum(ex.map(worker, range(threads)))
    wall = time.perf_counter() - t_start
    allc = {"value": round(2.0 * total / wall / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "bit-serial oracle decode of the layer's 7 matrices (whole matrices, in turn) on %d host "
                      "threads, one per allowed CPU, %.1f s wall, %d elements (%s)" % (threads, wall, total, cpu)}
    return allc, one


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer", choices=["layer"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-shard", action="store_true")
    ap.add_argument("--no-model", action="store_true", help="skip the 8B-parameter model pass")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no cross-GPU step; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from huffman_decode_df11_amd import api
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")

    encs = build_layer(args.seed)
    mats = [m for _, m, _ in encs]
    dts = [e.to("cuda") for _, _, e in encs]
    n_total = sum(e.n for _, _, e in encs)
    biggest = max(e.n for _, _, e in encs)
    outbuf = torch.empty(biggest, dtype=torch.bfloat16, device="cuda")
    verify(dts, mats, outbuf)
    log("parity verified on all %d matrices" % len(dts))

    alg = [algorithmic_bytes(e) for _, _, e in encs]
    compressed = sum(e.compressed_nbytes() for _, _, e in encs)
    stream_bits = sum(e.total_bits for _, _, e in encs)

    # the step: the layer's seven matrices in one launch, each into its own
    # slice of one reused layer-sized buffer
    ms_per_step, outs = time_batched(dts, args.steps, args.warmup)
    for o, m in zip(outs, mats):
        if not np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), m.reshape(-1)):
            raise SystemExit("batched parity check failed")
    del outs
    achieved = sum(alg) / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": "decoded BF16 GB/s (df11_decode, Llama-3-8B layer)",
        "value": round(2.0 * n_total / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": "llama3-8b-layer: q,k,v,o,gate,up,down bf16 N(0,0.02), 218,103,808 elements, "
                        "one codebook, the seven matrices decoded in one launch (df11_decode_batch), each "
                        "into its slice of one reused layer-sized buffer",
            "elements": n_total,
            "launches_per_step": 1,
            "bits_per_weight": round(8.0 * compressed / n_total, 4),
            "exponent_bits_per_weight": round(stream_bits / n_total, 4),
            "parallelism": "1 GPU",
        },
        "elements_per_s": round(n_total / (ms_per_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_kernel_llama3_8b_layer.md", DECODE_SOURCES),
            "kernel": "decode_kernel",
            "algorithmic_bytes_per_launch": int(sum(alg)),
            "algorithmic_bytes_per_element": round(sum(alg) / n_total, 4),
            "timing": "events around the timed back-to-back launches on the launch stream, enqueued "
                      "behind a short spin kernel; one launch per step, so the average launch duration "
                      "is the step time",
        },
    }
    copy_gbs = copy_peak()
    result["roofline"]["copy_peak_gbs"] = round(copy_gbs, 1)
    result["roofline"]["frac_of_copy_peak"] = round(achieved / copy_gbs, 4)
    # the same matrices one launch each into one matrix-sized reused buffer
    launch_ms, eager_ms = time_decode(dts, outbuf, args.steps, args.warmup)
    graph_ms = time_graph(dts, outbuf, args.steps, args.warmup)
    # after the replays the buffer holds the last matrix of the layer
    last = outbuf.view(torch.int16)[:mats[-1].size].cpu().numpy().view(np.uint16)
    if not np.array_equal(last, mats[-1].reshape(-1)):
        raise SystemExit("graph replay parity check failed")
    result["per_matrix_layer"] = {
        "buffer": "one reused buffer of the largest matrix",
        "graph": {"launches_per_step": len(dts), "ms_per_step": round(graph_ms, 4),
                  "decoded_gbs": round(2.0 * n_total / (graph_ms * 1e-3) / 1e9, 2),
                  "hbm_frac": round(sum(alg) / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "eager": {"launches_per_step": len(dts), "ms_per_step": round(eager_ms, 4),
                  "decoded_gbs": round(2.0 * n_total / (eager_ms * 1e-3) / 1e9, 2)},
        "repeated_launch_ms": {name: round(float(t), 4) for (name, _, _), t in zip(encs, launch_ms)},
        "repeated_launch_note": "each matrix decoded again and again into the same buffer; its 100-200 MB "
                                "of traffic partly stays in the 256 MB Infinity Cache, so these are warm-cache "
                                "kernel times",
    }
    if not args.no_model:
        result["model_pass"] = model_pass(args.steps, args.warmup, args.seed)
        result["offload_pass"] = offload_pass(args.steps, args.warmup, args.seed)
        result["encode"] = encode_rate(args.seed)
    if not args.no_fused:
        result["fused_up_proj"] = fused_up_proj(args.steps, args.warmup, args.seed)
    if not args.no_model:
        result["other_configs"] = other_configs(args.steps, args.warmup, args.seed)
        result["embedding_lookup"] = embedding_lookup(args.steps, args.warmup, args.seed)
    if not args.no_shard:
        # what one GPU does under an 8-way row split of each matrix (no collective)
        result["shard_8way"] = {
            "layer_decode": shard_layer_decode(args.steps, args.warmup, ways=8, seed=args.seed),
            "fused_up_proj": fused_up_proj(args.steps, args.warmup, args.seed, copies=32, rows=14336 // 8),
        }
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = 256 << 20
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["cpu_baseline_one_core"] = cpu_baseline_layer(mats)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
