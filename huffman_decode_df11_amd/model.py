"""Whole-model decode: every weight matrix of a model held DF11-compressed in
device memory and restored, one matrix at a time, into one reused BF16
buffer right before it would be used.

[P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" 2.2
     item 3: the compressed weights stay resident on the GPU and each is
     decompressed just before its matrix multiplication, then discarded, so
     the decompression runs once per forward pass for every matrix.
[P1] 2.2 item 1: one code per group of weights (here one per decoder layer,
     one for the embedding and one for the LM head).

A pass is the plain sequence of per-matrix decode launches (226 for the
8B-parameter model); it can also be captured once as a HIP graph and
replayed, or run as one batched launch per decoder layer into a layer-sized
buffer.  The matmuls that would consume the weights are not part of a pass.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from typing import List, Tuple

import numpy as np

from . import api, synth


class CompressedModel:
    """Groups of DF11Tensors (each group shares one codebook), decoded in
    order into one reused buffer of the largest matrix's size."""

    def __init__(self, groups: List[Tuple[str, List[Tuple[str, "api.DF11Tensor"]]]], device="cuda"):
        import torch
        self.groups = groups
        self.device = torch.device(device)
        self.matrices = [(g, name, t) for g, mats in groups for name, t in mats]
        self.n_elements = sum(t.n for _, _, t in self.matrices)
        self.max_elements = max(t.n for _, _, t in self.matrices)
        self.buffer = torch.empty(self.max_elements, dtype=torch.bfloat16, device=self.device)
        self._graph = None
        self._layer_buffer = None

    # ------------------------------------------------------------ passes
    def decode_pass(self, stream=None):
        """One launch per matrix into the reused buffer."""
        for _, _, t in self.matrices:
            api.decode(t, out=self.buffer, stream=stream)

    def decode_pass_batched(self, stream=None):
        """One launch per group (all matrices of a decoder layer at once) into
        one reused buffer sized for the largest group."""
        for i in range(len(self.groups)):
            self.decode_group(i, stream)

    def decode_group(self, i: int, stream=None):
        """Decode group i in one launch; returns its outputs (slices of the
        reused group buffer, valid until the next group is decoded)."""
        import torch
        if self._layer_buffer is None:
            need = max(sum(_round8(t.n) for _, t in mats) for _, mats in self.groups)
            self._layer_buffer = torch.empty(need, dtype=torch.bfloat16, device=self.device)
            self._layer_outs = []
            for _, mats in self.groups:
                outs, off = [], 0
                for _, t in mats:
                    outs.append(self._layer_buffer[off:off + t.n])
                    off += _round8(t.n)
                self._layer_outs.append(outs)
        api.decode_batch([t for _, t in self.groups[i][1]], outs=self._layer_outs[i], stream=stream)
        return self._layer_outs[i]

    def capture(self):
        """Capture decode_pass as a HIP graph (once); returns replay()."""
        import torch
        if self._graph is None:
            side = torch.cuda.Stream(device=self.device)
            side.wait_stream(torch.cuda.current_stream(self.device))
            with torch.cuda.stream(side):
                self.decode_pass()           # warm-up launches outside the capture
            torch.cuda.current_stream(self.device).wait_stream(side)
            torch.cuda.synchronize(self.device)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.decode_pass()
            self._graph = g
        return self._graph.replay

    # ------------------------------------------------------------ sizes
    def compressed_nbytes(self) -> int:
        return sum(t.compressed_nbytes() for _, _, t in self.matrices)

    def stream_bits(self) -> int:
        return sum(t.total_bits for _, _, t in self.matrices)


def _round8(n: int) -> int:
    return (n + 7) // 8 * 8


def encode_llama3_8b(seed: int = 0, device="cuda", layers: int = synth.LLAMA3_8B_LAYERS, threads: int = 0,
                     embed_and_head: bool = True, on_group=None):
    """Generate the model's matrices on `device` (torch Philox, N(0, 0.02)
    rounded to BF16) and encode each group (a decoder layer, the embedding,
    the head) on host threads with the group's own codebook.  on_group(g,
    [(name, Encoded)]) is called as each group is done (in completion
    order); returns the groups in model order when on_group is None."""
    import torch
    specs = synth.llama3_8b_tensors(layers)
    by_group = {}
    for idx, (g, name, r, c) in enumerate(specs):
        if not embed_and_head and g in ("embed", "head"):
            continue
        by_group.setdefault(g, []).append((idx, name, r, c))
    order = list(by_group)
    threads = threads or min(16, os.cpu_count() or 4)
    lock = __import__("threading").Lock()

    def encode_group(g):
        host = []
        for idx, name, r, c in by_group[g]:
            with lock:   # generation and download on the device, one group at a time
                x = synth.normal_bf16_torch(r, c, seed, idx, device)
                host.append((name, x.view(torch.int16).cpu().numpy().view(np.uint16)))
                del x
        hist = None
        for _, u in host:
            hist = api.hist_accumulate(u, hist)
        cb = api.build_codebook(hist)
        return g, [(name, api.encode(u, codebook=cb)) for name, u in host]

    done = {}
    with cf.ThreadPoolExecutor(threads) as ex:
        for fut in cf.as_completed([ex.submit(encode_group, g) for g in order]):
            g, encs = fut.result()
            if on_group is not None:
                on_group(g, encs)
            else:
                done[g] = encs
    return None if on_group is not None else [(g, done[g]) for g in order]


def synthetic_llama3_8b(seed: int = 0, device="cuda", layers: int = synth.LLAMA3_8B_LAYERS,
                        threads: int = 0, log=None, encoder: str = "device") -> CompressedModel:
    """The 8B-parameter model, only the compressed tensors kept on `device`.
    encoder "device": each group generated, counted and encoded on the GPU
    (df11_hist_device, df11_encode_device; the 256-symbol codebook is built
    on the host); "host": encode_llama3_8b on host threads."""
    order = [g for g, _, _, _ in synth.llama3_8b_tensors(layers)]
    order = list(dict.fromkeys(order))
    if encoder == "device":
        return CompressedModel(_encode_on_device(seed, device, layers, log), device=device)
    resident = {}

    def upload(g, encs):
        resident[g] = [(name, e.to(device)) for name, e in encs]
        if log:
            log("encoded %s (%d/%d groups)" % (g, len(resident), len(order)))

    encode_llama3_8b(seed, device, layers, threads, on_group=upload)
    return CompressedModel([(g, resident[g]) for g in order], device=device)


def _encode_on_device(seed: int, device, layers: int, log=None):
    specs = synth.llama3_8b_tensors(layers)
    by_group = {}
    for idx, (g, name, r, c) in enumerate(specs):
        by_group.setdefault(g, []).append((idx, name, r, c))
    groups = []
    for g, mats in by_group.items():
        hist = None
        for idx, name, r, c in mats:
            hist = api.hist_device(synth.normal_bf16_torch(r, c, seed, idx, device), hist)
        cb = api.build_codebook(hist)
        encs = []
        for idx, name, r, c in mats:
            # generated again rather than kept: one matrix at a time in device memory
            encs.append((name, api.encode_device(synth.normal_bf16_torch(r, c, seed, idx, device), codebook=cb)))
        groups.append((g, encs))
        if log:
            log("encoded %s on the device (%d/%d groups)" % (g, len(groups), len(by_group)))
    return groups


def verify_pass(model: CompressedModel, seed: int, stream=None) -> int:
    """Decode every matrix and compare it, on the device, with the same
    matrix generated again from its seed.  Returns the number of elements
    checked; raises on the first mismatch."""
    import torch
    specs = synth.llama3_8b_tensors(len(model.groups) - 2)
    assert len(specs) == len(model.matrices)
    checked = 0
    for idx, ((g, name, r, c), (g2, name2, t)) in enumerate(zip(specs, model.matrices)):
        assert (g, name) == (g2, name2)
        api.decode(t, out=model.buffer, stream=stream)
        want = synth.normal_bf16_torch(r, c, seed, idx, model.device).view(torch.int16).reshape(-1)
        got = model.buffer[:t.n].view(torch.int16)
        if not torch.equal(got, want):
            bad = int((got != want).nonzero()[0])
            raise RuntimeError("model pass: %s %s differs at element %d" % (g, name, bad))
        checked += t.n
    return checked


def verify_pass_batched(model: CompressedModel, seed: int, stream=None) -> int:
    """Decode every group in one launch each (decode_group, the launches of
    decode_pass_batched) and compare every output, on the device, with the
    same matrix generated again from its seed.  Returns the number of
    elements checked; raises on the first mismatch."""
    import torch
    specs = synth.llama3_8b_tensors(len(model.groups) - 2)
    assert len(specs) == len(model.matrices)
    checked, idx = 0, 0
    for i, (g, mats) in enumerate(model.groups):
        outs = model.decode_group(i, stream)
        for (name, t), out in zip(mats, outs):
            sg, sname, r, c = specs[idx]
            assert (sg, sname) == (g, name)
            want = synth.normal_bf16_torch(r, c, seed, idx, model.device).view(torch.int16).reshape(-1)
            got = out.view(torch.int16)
            if not torch.equal(got, want):
                bad = int((got != want).nonzero()[0])
                raise RuntimeError("model pass: %s %s differs at element %d" % (g, name, bad))
            checked += t.n
            idx += 1
    return checked
