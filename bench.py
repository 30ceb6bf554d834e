#!/usr/bin/env python3
"""Benchmark of the DF11 decode hot path on one MI355X.

The step: one pass over an 8B-parameter model of synthetic N(0, 0.02) BF16
weights shaped like Llama-3-8B (embedding 128256 x 4096, 32 decoder layers
of q, k, v, o, gate, up, down, LM head: 8,029,995,008 elements in 226
matrices), compressed with one codebook per layer and resident in HBM.  A
pass decodes each layer (and the embedding, and the head) in one
df11_decode_batch launch into one reused buffer: 34 launches.  Every
element is checked against its generator through those launches before
timing.

Also reported: the same pass as 226 per-matrix launches (eager and as one
HIP graph), one decoder layer on its own, the 1024 x 1024 tensor and the
16M adversarial mix, compressed CPU offload, the GPU encoder, the embedding
row gather, the fused decode+GEMM on up_proj at B in {1, 8, 64, 256}, and
one GPU's share of an 8-way row split.

Prints one JSON line:
  value     decoded BF16 GB/s (2 bytes per element / pass time)
  roofline  the decode kernel's algorithmic HBM bytes per launch / its
            average launch duration (HIP events around every launch on the
            launch stream), against the 8 TB/s HBM peak
  cpu_baseline  the CPU oracle's bit-serial decode on this host's allowed
            cores over a bounded sample of the model (one layer and 8,192
            embedding rows), extrapolated to the pass; cpu_baseline_legs
            holds the other oracle timings (one core)

    python bench.py [--steps K] [--warmup W] [--headline-only] [--no-extras] [--no-fused] [--no-shard]
                    [--no-cpu-baseline]
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


def model_headline(steps: int, warmup: int, seed: int = 0):
    """The step: one pass over the 8B-parameter model (embedding, 32 decoder
    layers, LM head: 226 matrices, 8,029,995,008 elements, one codebook per
    layer, compressed and resident in HBM), each group of matrices (a layer,
    the embedding, the head) decoded in one df11_decode_batch launch into one
    reused group-sized buffer, 34 launches per pass.  Every element of every
    matrix is checked against its generator through those launches first.

    Timed twice, each time `steps` passes back to back behind a short spin
    kernel on the launch stream: between two events (ms per pass, the
    step; with nothing else on the stream, pass time / launches is the
    average launch duration, the gaps between launches included), and again
    with an event pair around every launch (the split of the pass over the
    embedding, the layers and the head; each pair adds a few microseconds
    around its launch, so neither the step nor the average comes from this
    run).  Returns (model, record)."""
    import torch
    from huffman_decode_df11_amd import model as mdl
    t0 = time.time()
    m = mdl.synthetic_llama3_8b(seed=seed, device="cuda")
    t_build = time.time() - t0
    checked = mdl.verify_pass_batched(m, seed)
    log("8B model built in %.1f s; all %d elements decoded through the batched launches and verified"
        % (t_build, checked))
    alg_launch = [sum(algorithmic_bytes(t) for _, t in mats) for _, mats in m.groups]
    alg = sum(alg_launch)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        m.decode_pass_batched(stream)
    torch.cuda.synchronize()
    ng = len(m.groups)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a, b = ev(), ev()
    _hold_queue(5.0)
    a.record(stream)
    for s in range(steps):
        for i in range(ng):
            m.decode_group(i, stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms_pass = a.elapsed_time(b) / steps
    evs = [[(ev(), ev()) for _ in range(ng)] for _ in range(steps)]
    _hold_queue(5.0)
    for s in range(steps):
        for i in range(ng):
            evs[s][i][0].record(stream)
            m.decode_group(i, stream)
            evs[s][i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([[e0.elapsed_time(e1) for e0, e1 in row] for row in evs])
    kernel_ms = float(launch_ms.sum(axis=1).mean())
    # the buffers hold the last pass's head: check it again after the timing
    from huffman_decode_df11_amd import synth
    spec = synth.llama3_8b_tensors(len(m.groups) - 2)[-1]
    want = synth.normal_bf16_torch(spec[2], spec[3], seed, len(m.matrices) - 1, "cuda").view(torch.int16)
    if not torch.equal(m._layer_outs[ng - 1][0].view(torch.int16), want.reshape(-1)):
        raise SystemExit("model pass parity check after timing failed")
    n = m.n_elements
    layer_ms = launch_ms[:, 1:ng - 1].mean()
    rec = {
        "elements": n,
        "matrices": len(m.matrices),
        "launches_per_step": ng,
        "compressed_bytes": m.compressed_nbytes(),
        "bits_per_weight": round(8.0 * m.compressed_nbytes() / n, 4),
        "exponent_bits_per_weight": round(m.stream_bits() / n, 4),
        "build_s": round(t_build, 1),
        "verified_elements": checked,
        "ms_per_step": ms_pass,
        "kernel_ms_per_step": kernel_ms,
        "algorithmic_bytes_per_step": int(alg),
        "launch_us": {"embedding": round(float(launch_ms[:, 0].mean()) * 1e3, 2),
                      "decoder_layer_mean": round(float(layer_ms) * 1e3, 2),
                      "decoder_layer_min": round(float(launch_ms[:, 1:ng - 1].min()) * 1e3, 2),
                      "decoder_layer_max": round(float(launch_ms[:, 1:ng - 1].max()) * 1e3, 2),
                      "lm_head": round(float(launch_ms[:, ng - 1].mean()) * 1e3, 2)},
        "layer_launch_hbm_frac": round(float(np.mean(alg_launch[1:ng - 1])) / (layer_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    return m, rec


def model_other_modes(m, steps: int, warmup: int):
    """The same model pass as 226 eager launches (one per matrix into one
    reused matrix-sized buffer) and as those launches captured once in a HIP
    graph and replayed."""
    import torch
    alg = sum(algorithmic_bytes(t) for _, _, t in m.matrices)

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
    out = {"passes_timed": n}
    for name, f in (("eager", m.decode_pass), ("graph", m.capture())):
        t = timeit(f, n)
        out[name] = {"ms_per_pass": round(t, 3), "launches": len(m.matrices),
                     "decoded_gbs": round(2.0 * m.n_elements / (t * 1e-3) / 1e9, 1),
                     "hbm_frac": round(alg / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
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
    `rows` rows, one GPU's share of a row split) for B in {1, 8, 64, 256}
    (and 2, 32, 128),
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
    for B in (1, 2, 8, 32, 64, 128, 256):
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
    the compressed data comes from HBM), each in the default 16-byte chunks
    and in 8-byte chunks (twice the segments: shorter per-wave work for
    tensors too small to fill the GPU many times over).  Parity is checked
    in full first."""
    import torch
    from huffman_decode_df11_amd import api, synth
    out = {}
    for name, u, copies, chunk in (("tensor_1024x1024", synth.tensor_1024(seed=seed).reshape(-1), 1, 16),
                                   ("tensor_1024x1024_chunk8", synth.tensor_1024(seed=seed).reshape(-1), 1, 8),
                                   ("adversarial_16m", synth.adversarial_bf16(1 << 24, seed=seed), 12, 16),
                                   ("adversarial_16m_chunk8", synth.adversarial_bf16(1 << 24, seed=seed), 12, 8)):
        enc = api.encode(u, layout=api.make_layout(chunk_bytes=chunk))
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
        copy_us = _copy_same_traffic_us(alg, copies, n_launch)
        out[name] = {"elements": int(u.size), "us_per_launch": round(ms * 1e3, 2),
                     "decoded_gbs": round(2.0 * u.size / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "copy_same_traffic_us": round(copy_us, 2),
                     "copy_same_traffic_hbm_frac": round(alg / (copy_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "bits_per_weight": round(enc.compressed_nbytes() * 8.0 / u.size, 3),
                     "chunk_bytes": chunk, "copies_cycled": copies}
    return out


def _copy_same_traffic_us(alg_bytes: int, copies: int, n: int) -> float:
    """A plain device copy moving the same bytes as one decode launch (reads
    alg/2, writes alg/2), timed the same way (back-to-back calls behind a
    spin kernel, `copies` sources cycled): what HBM gives a kernel of this
    size with no decoding at all."""
    import torch
    nb = max(16, int(alg_bytes // 2) // 16 * 16)
    srcs = [torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(i) for i in range(copies)]
    dst = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for i in range(copies):
        dst.copy_(srcs[i])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _hold_queue(2.0 + 0.05 * n)
    a.record()
    for i in range(n):
        dst.copy_(srcs[i % copies])
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e3


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

    out = {"workload": "embedding table %dx%d bf16 N(0,0.02), row-major layout (8-byte chunks, the DF11Embedding "
                       "default; and 16-byte chunks), B random token ids per call" % (vocab, dim), "by_tokens": {}}
    ids_by_b = {B: torch.from_numpy(rng.integers(0, vocab, B)).cuda() for B in (1, 32, 2048)}
    for chunk in (8, 16):
        dt = api.encode_device(W, layout=api.make_layout(rows=vocab, cols=dim, chunk_bytes=chunk))
        row_alg = dim * (dt.total_bits / dt.n / 8.0 + 1.0) + 2.0 * dim
        out["bits_per_weight_chunk%d" % chunk] = round(dt.compressed_nbytes() * 8.0 / dt.n, 4)
        for B, ids in ids_by_b.items():
            buf = torch.empty(B, dim, dtype=torch.bfloat16, device="cuda")
            api.decode_rows(dt, ids, out=buf)
            torch.cuda.synchronize()
            if not torch.equal(buf.view(torch.int16), W[ids].view(torch.int16)):
                raise SystemExit("embedding lookup parity failed at B=%d" % B)
            n = max(steps, 50)
            us = timeit(lambda: api.decode_rows(dt, ids, out=buf), n)
            rec = out["by_tokens"].setdefault(str(B), {})
            if chunk == 8:
                rec["torch_bf16_gather_us"] = round(timeit(lambda: torch.nn.functional.embedding(ids, W), n), 2)
            rec["us_per_call_chunk%d" % chunk] = round(us, 2)
            rec["rows_per_s_chunk%d" % chunk] = round(B / (us * 1e-6), 1)
            rec["hbm_frac_chunk%d" % chunk] = round(B * row_alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        del dt
    del W
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


def copy_peak(nbytes: int = 512 << 20, reps: int = 5, groups: int = 3):
    """Device-to-device copy rate (read + write bytes per second) of a
    buffer larger than the Infinity Cache: the practical HBM ceiling.  The
    best of `groups` timed groups of `reps` copies (a single group has read
    low now and then, which would overstate the fraction of it reached)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(groups):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        best = max(best, 2.0 * nbytes / (ms * 1e-3) / 1e9)
    del src, dst
    return best


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


def _pinned_one_core(f):
    """Run f() with this process pinned to the first CPU it may use."""
    allowed = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    if allowed:
        os.sched_setaffinity(0, {allowed[0]})
    try:
        return f()
    finally:
        if allowed:
            os.sched_setaffinity(0, set(allowed))


def _repeat(f, min_s: float):
    """Call f() until min_s seconds have passed (at least once); returns
    (calls, seconds)."""
    calls, secs = 0, 0.0
    while calls == 0 or secs < min_s:
        t0 = time.perf_counter()
        f()
        secs += time.perf_counter() - t0
        calls += 1
    return calls, secs


def cpu_baselines(seed: int = 0, all_cores_s: float = 10.0):
    """The oracle as written (plain serial C: bit-serial decode, serial
    encode, scalar float32 GEMM) timed on this host.  Returns (headline,
    legs).

    Headline: the 8B model pass extrapolated from a bounded sample -- layer
    0's seven matrices (218,103,808 elements) and the first 8,192 rows of the
    embedding (33,554,432 elements), generated exactly as the model's -- the
    oracle decoding whole tensors in turn on every allowed CPU (one thread
    each; its C decode runs outside the interpreter lock) for about
    all_cores_s seconds.  Decoded GB/s over that mix = 2 x elements / wall;
    the pass would take 8,029,995,008 / (elements/s).

    Legs, on one core pinned: the 1024 x 1024 tensor, the 16M adversarial
    mix, the layer's matrices, the oracle encoder on up_proj, and the scalar
    GEMM on up_proj at each B (a sample of W's rows, extrapolated by flops)."""
    import itertools
    from concurrent.futures import ThreadPoolExecutor
    import torch
    from oracle import oracle as orc
    from huffman_decode_df11_amd import synth
    cpu = _cpu_model()
    allowed = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else [0]
    threads = max(1, len(allowed))
    specs = synth.llama3_8b_tensors()
    t_setup = time.perf_counter()

    def host(idx, rows=None):
        g, name, r, c = specs[idx]
        t = synth.normal_bf16_torch(r, c, seed, idx, "cuda")
        if rows is not None:
            t = t[:rows]
        return name, t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)

    layer = [host(i) for i in range(1, 8)]
    emb = host(0, rows=8192)
    torch.cuda.empty_cache()
    hist = None
    for _, u in layer:
        hist = orc.histogram(u) if hist is None else hist + orc.histogram(u)
    ln_layer = orc.code_lengths(hist, 32)
    ln_emb = orc.code_lengths(orc.histogram(emb[1]), 32)
    jobs = [(name, u, ln_layer) for name, u in layer] + [("embed_tokens[:8192]", emb[1], ln_emb)]
    with ThreadPoolExecutor(max_workers=min(threads, len(jobs))) as ex:
        refs = list(ex.map(lambda j: orc.encode(j[1], lengths=j[2]), jobs))
    for (name, u, ln), ref in zip(jobs, refs):
        if not np.array_equal(orc.decode(ref.E, ref.total_bits, ref.sm, ref.n, ln), u):
            raise SystemExit("oracle round trip failed on " + name)
    t_setup = time.perf_counter() - t_setup

    # headline: every allowed core, whole tensors in turn until the budget is used
    order = itertools.count()
    t_start = time.perf_counter()
    deadline = t_start + all_cores_s

    def worker(_):
        done = 0
        while True:
            i = next(order)
            if i >= threads and time.perf_counter() >= deadline:
                return done
            (name, u, ln), ref = jobs[i % len(jobs)], refs[i % len(jobs)]
            orc.decode(ref.E, ref.total_bits, ref.sm, ref.n, ln)
            done += ref.n
    with ThreadPoolExecutor(max_workers=threads) as ex:
        total = sum(ex.map(worker, range(threads)))
    wall = time.perf_counter() - t_start
    model_n = sum(r * c for _, _, r, c in specs)
    rate = total / wall
    headline = {"value": round(2.0 * rate / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": "bit-serial oracle decode, whole tensors in turn on %d host threads (one per allowed CPU, "
                          "%s) for %.1f s wall, %d elements: layer 0's 7 matrices and embedding rows 0..8191 of the "
                          "8B model (same generator); the model pass (%d elements) extrapolates to %.1f s"
                          % (threads, cpu, wall, total, model_n, model_n / rate)}

    legs = {"host_cpu": cpu, "allowed_cpus": threads, "setup_s": round(t_setup, 1)}

    def one_core_decode(u, ln, ref, min_s):
        calls, secs = _pinned_one_core(lambda: _repeat(lambda: orc.decode(ref.E, ref.total_bits, ref.sm, ref.n, ln),
                                                          min_s))
        return {"value": round(2.0 * ref.n * calls / secs / 1e9, 4), "unit": "GB/s decoded", "cores": 1,
                "elements": int(ref.n), "calls": calls, "seconds": round(secs, 2)}

    u0 = synth.tensor_1024(seed=seed).reshape(-1)
    ln0 = orc.code_lengths(orc.histogram(u0), 32)
    legs["decode_1024x1024"] = one_core_decode(u0, ln0, orc.encode(u0, lengths=ln0), 1.0)
    u2 = synth.adversarial_bf16(1 << 24, seed=seed)
    ln2 = orc.code_lengths(orc.histogram(u2), 32)
    legs["decode_adversarial_16m"] = one_core_decode(u2, ln2, orc.encode(u2, lengths=ln2), 1.5)
    calls, secs = _pinned_one_core(lambda: _repeat(
        lambda: [orc.decode(r.E, r.total_bits, r.sm, r.n, j[2]) for j, r in zip(jobs[:7], refs[:7])], 2.0))
    n_layer = sum(r.n for r in refs[:7])
    legs["decode_llama3_8b_layer"] = {"value": round(2.0 * n_layer * calls / secs / 1e9, 4), "unit": "GB/s decoded",
                                      "cores": 1, "elements": n_layer, "passes": calls, "seconds": round(secs, 2)}
    legs["decode_model_pass_one_core_extrapolated_s"] = round(model_n * secs / (n_layer * calls), 1)
    up = dict(layer)["up_proj"]
    t0 = time.perf_counter()
    _pinned_one_core(lambda: orc.encode(up, lengths=ln_layer))
    te = time.perf_counter() - t0
    legs["encode_up_proj"] = {"value": round(2.0 * up.size / te / 1e9, 4), "unit": "GB/s of BF16 input", "cores": 1,
                              "elements": int(up.size), "seconds": round(te, 2)}
    W = up.reshape(14336, 4096)
    X = synth.activations_bf16(256, 4096, seed=1)
    gemm = {}
    for B in (1, 8, 64, 256):
        rows = int(min(14336, max(16, (1e9 / (2 * B * 4096)) // 16 * 16)))
        t0 = time.perf_counter()
        _pinned_one_core(lambda: orc.gemm_f32(X[:B], W[:rows]))
        tg = time.perf_counter() - t0
        flops = 2.0 * B * rows * 4096
        gemm[str(B)] = {"tflops": round(flops / tg / 1e12, 6), "rows_sampled": rows,
                        "seconds": round(tg, 3), "full_up_proj_s_extrapolated": round(tg * 14336 / rows, 2)}
    legs["gemm_up_proj_scalar_f32"] = {"unit": "TFLOP/s", "cores": 1, "by_batch": gemm}
    return headline, legs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--headline-only", action="store_true",
                    help="only the model pass (build, verify, warm-up, timed passes): the profiled command")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-shard", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--only", default="",
                    help="comma-separated sections to run instead of the step (for profiling): fused, other_configs, "
                         "embedding_lookup, encode, llama3_8b_layer")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path has no cross-GPU step (the row-split shard of one "
              "GPU is reported as shard_8way); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.only:
        sections = {"fused": lambda: fused_up_proj(args.steps, args.warmup, args.seed),
                    "other_configs": lambda: other_configs(args.steps, args.warmup, args.seed),
                    "embedding_lookup": lambda: embedding_lookup(args.steps, args.warmup, args.seed),
                    "encode": lambda: encode_rate(args.seed),
                    "llama3_8b_layer": lambda: layer_workload(args.steps, args.warmup, args.seed)}
        out = {}
        for name in args.only.split(","):
            log("section", name)
            out[name] = sections[name]()
        if args.calibrate_copy:
            out["calibration_copy_bytes"] = calibration_copy()
        print(json.dumps(out), flush=True)
        return

    m, rec = model_headline(args.steps, args.warmup, args.seed)
    n = rec["elements"]
    ms = rec["ms_per_step"]
    alg = rec["algorithmic_bytes_per_step"]
    ng = rec["launches_per_step"]
    # (alg / ng) bytes per launch over (ms / ng) per launch
    achieved = alg / (ms * 1e-3) / 1e9
    result = {
        "metric": "decoded BF16 GB/s (df11_decode_batch, 8B-parameter model pass)",
        "value": round(2.0 * n / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": "llama3-8b-sized model pass: embedding 128256x4096, 32 decoder layers (q,k,v,o,gate,up,down), "
                        "LM head; bf16 N(0,0.02), %d elements in %d matrices, one codebook per layer; each layer "
                        "(and the embedding, the head) decoded in one launch into one reused buffer" % (n, rec["matrices"]),
            "elements": n,
            "launches_per_step": ng,
            "bits_per_weight": rec["bits_per_weight"],
            "exponent_bits_per_weight": rec["exponent_bits_per_weight"],
            "parallelism": "1 GPU",
        },
        "elements_per_s": round(n / (ms * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_kernel_llama3_8b_model_pass.md", DECODE_SOURCES),
            "kernel": "decode_kernel",
            "launches_per_step": ng,
            "avg_launch_us": round(ms / ng * 1e3, 2),
            "algorithmic_bytes_per_launch": int(alg / ng),
            "algorithmic_bytes_per_element": round(alg / n, 4),
            "timing": "HIP events on the launch stream around `steps` back-to-back passes of %d decode launches "
                      "(queued behind a short spin kernel, nothing else on the stream); average launch duration = "
                      "pass time / %d, gaps between launches included; achieved = algorithmic bytes per launch / "
                      "that duration" % (ng, ng),
        },
        "model_pass": {k: rec[k] for k in ("verified_elements", "build_s", "compressed_bytes", "launch_us",
                                           "layer_launch_hbm_frac")},
    }
    result["model_pass"]["launch_events_ms_per_pass"] = round(rec["kernel_ms_per_step"], 4)
    headline_only = args.headline_only
    if not headline_only:
        copy_gbs = copy_peak()
        result["roofline"]["copy_peak_gbs"] = round(copy_gbs, 1)
        result["roofline"]["frac_of_copy_peak"] = round(achieved / copy_gbs, 4)
        if not args.no_extras:
            result["model_pass"].update(model_other_modes(m, args.steps, args.warmup))
    del m
    torch.cuda.empty_cache()
    if not headline_only and not args.no_extras:
        result["llama3_8b_layer"] = layer_workload(args.steps, args.warmup, args.seed)
        result["offload_pass"] = offload_pass(args.steps, args.warmup, args.seed)
        result["encode"] = encode_rate(args.seed)
        result["other_configs"] = other_configs(args.steps, args.warmup, args.seed)
        result["embedding_lookup"] = embedding_lookup(args.steps, args.warmup, args.seed)
    if not headline_only and not args.no_fused:
        result["fused_up_proj"] = fused_up_proj(args.steps, args.warmup, args.seed)
    if not headline_only and not args.no_shard and not args.no_extras:
        # what one GPU does under an 8-way row split of each matrix (no collective)
        result["shard_8way"] = {
            "layer_decode": shard_layer_decode(args.steps, args.warmup, ways=8, seed=args.seed),
            "fused_up_proj": fused_up_proj(args.steps, args.warmup, args.seed, copies=32, rows=14336 // 8),
        }
    if args.calibrate_copy:
        result["calibration_copy_bytes"] = calibration_copy()
    if not headline_only and not args.no_cpu_baseline:
        result["cpu_baseline"], result["cpu_baseline_legs"] = cpu_baselines(args.seed)
    print(json.dumps(result), flush=True)


def calibration_copy(nbytes: int = 256 << 20) -> int:
    """Three plain device-to-device copies of nbytes, whose HBM counters
    calibrate FETCH_SIZE and WRITE_SIZE in the profiles."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return nbytes


def layer_workload(steps: int, warmup: int, seed: int = 0):
    """One Llama-3-8B-shaped decoder layer (218,103,808 elements, one
    codebook): the seven matrices in one batched launch into a layer-sized
    buffer, and one launch each into one reused matrix-sized buffer (eager,
    and as one HIP graph).  Parity checked in full first."""
    import torch
    from huffman_decode_df11_amd import api
    encs = build_layer(seed)
    mats = [m for _, m, _ in encs]
    dts = [e.to("cuda") for _, _, e in encs]
    n_total = sum(e.n for _, _, e in encs)
    outbuf = torch.empty(max(e.n for _, _, e in encs), dtype=torch.bfloat16, device="cuda")
    verify(dts, mats, outbuf)
    alg = [algorithmic_bytes(e) for _, _, e in encs]
    ms, outs = time_batched(dts, steps, warmup)
    for o, m in zip(outs, mats):
        if not np.array_equal(o.view(torch.int16).cpu().numpy().view(np.uint16), m.reshape(-1)):
            raise SystemExit("batched parity check failed")
    del outs
    launch_ms, eager_ms = time_decode(dts, outbuf, steps, warmup)
    graph_ms = time_graph(dts, outbuf, steps, warmup)
    last = outbuf.view(torch.int16)[:mats[-1].size].cpu().numpy().view(np.uint16)
    if not np.array_equal(last, mats[-1].reshape(-1)):
        raise SystemExit("graph replay parity check failed")
    per = lambda t: {"ms_per_step": round(t, 4), "decoded_gbs": round(2.0 * n_total / (t * 1e-3) / 1e9, 2),
                     "hbm_frac": round(sum(alg) / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # the four smaller matrices (q, k, v, o: 1,328-5,306 segments, too few to
    # fill the GPU many times over) in 8-byte chunks, the others in 16
    cb = encs[0][2].codebook
    small = {"q_proj", "k_proj", "v_proj", "o_proj"}
    encs8 = [api.encode(m, codebook=cb, layout=api.make_layout(chunk_bytes=8 if name in small else 16))
             for name, m, _ in encs]
    dts8 = [e.to("cuda") for e in encs8]
    verify(dts8, mats, outbuf)
    _, eager8_ms = time_decode(dts8, outbuf, steps, warmup)
    alg8 = sum(algorithmic_bytes(e) for e in encs8)
    return {
        "workload": "llama3-8b layer: q,k,v,o,gate,up,down bf16 N(0,0.02), %d elements, one codebook" % n_total,
        "batched_one_launch": per(ms),
        "per_matrix_graph": dict(per(graph_ms), launches_per_step=len(dts)),
        "per_matrix_eager": dict(per(eager_ms), launches_per_step=len(dts)),
        "per_matrix_eager_small_chunk8": {
            "ms_per_step": round(eager8_ms, 4), "decoded_gbs": round(2.0 * n_total / (eager8_ms * 1e-3) / 1e9, 2),
            "hbm_frac": round(alg8 / (eager8_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bits_per_weight": round(8.0 * sum(e.compressed_nbytes() for e in encs8) / n_total, 4),
            "note": "q, k, v, o encoded with 8-byte chunks, gate, up, down with 16"},
        "repeated_launch_ms": {name: round(float(t), 4) for (name, _, _), t in zip(encs, launch_ms)},
        "repeated_launch_note": "each matrix decoded again and again into the same buffer; its 100-200 MB "
                                "of traffic partly stays in the 256 MB Infinity Cache, so these are warm-cache "
                                "kernel times",
    }


if __name__ == "__main__":
    main()
