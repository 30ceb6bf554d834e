"""Compressed CPU offload: layers kept DF11-compressed in pinned host memory
and streamed to the GPU one layer ahead of their decode.

[P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" and
[P2] "DFloat11：用于高效 GPU 推理的 LLM 和扩散模型无损压缩" describe an offload
mode for small GPUs: the compressed weights live in CPU memory and only the
block being computed is on the GPU.  Moving compressed blocks instead of
BF16 ones moves ~30% fewer bytes over PCIe.

Per group (a decoder layer): its streamed arrays (exponent words,
sign+mantissa bytes, gaps, chunk counts, segment records) are one pinned
host blob; a
copy stream moves the blob into one of two device slots while the compute
stream decodes the previous group from the other slot; events order slot
reuse.  The code tables (a few KB per codebook) stay resident on the GPU.
"""
from __future__ import annotations

import ctypes
from typing import List, Tuple

import numpy as np

from . import api
from ._lib import VIEW_ARRAYS, View

_STREAMED = ("exp_words", "sm", "gaps", "counts", "segs", "block_seg")
_ALIGN = 256


def _round(n: int) -> int:
    return (n + _ALIGN - 1) // _ALIGN * _ALIGN


def _same_tables(a, b) -> bool:
    """Two codebooks decode alike: the same object, or equal code lengths and
    lookup tables."""
    if a is b:
        return True
    if (a.n_tables, a.fast_bits, a.min_len, a.max_len) != (b.n_tables, b.fast_bits, b.min_len, b.max_len):
        return False
    nt, nf = a.n_tables * 256, 2 << a.fast_bits
    return (bytes(a.len) == bytes(b.len) and
            np.array_equal(np.ctypeslib.as_array(a.chain)[:nt], np.ctypeslib.as_array(b.chain)[:nt]) and
            np.array_equal(np.ctypeslib.as_array(a.fast)[:nf], np.ctypeslib.as_array(b.fast)[:nf]))


class OffloadedModel:
    """Groups [(name, [(matrix, Encoded)])] held in pinned host memory."""

    def __init__(self, groups: List[Tuple[str, list]], device="cuda"):
        import torch
        self.device = torch.device(device)
        self.groups = []
        max_blob = 0
        self.n_elements = 0
        for gname, mats in groups:
            # the group's matrices decode through the first one's device tables
            cb0 = mats[0][1].codebook
            for name, enc in mats[1:]:
                if not _same_tables(enc.codebook, cb0):
                    raise ValueError("group %s: %s has another codebook than %s; a group shares one"
                                     % (gname, name, mats[0][0]))
            layout, off = [], 0
            for name, enc in mats:
                offs = {}
                for a in _STREAMED:
                    offs[a] = off
                    off = _round(off + enc.arrays[a].nbytes)
                layout.append((name, enc, offs))
                self.n_elements += enc.n
            blob = torch.empty(max(off, _ALIGN), dtype=torch.uint8, pin_memory=True)
            hb = blob.numpy()
            for name, enc, offs in layout:
                for a in _STREAMED:
                    src = enc.arrays[a].view(np.uint8).reshape(-1)
                    hb[offs[a]:offs[a] + src.size] = src
            tables = api._device_tables(mats[0][1], self.device)
            self.groups.append((gname, layout, blob, off, tables))
            max_blob = max(max_blob, off)
        self.slots = [torch.empty(max(max_blob, _ALIGN), dtype=torch.uint8, device=self.device) for _ in range(2)]
        # one device view per (group, matrix, slot): pointers into the slot
        self.views = []
        for gname, layout, blob, size, tables in self.groups:
            per_slot = []
            for slot in self.slots:
                vs = []
                for name, enc, offs in layout:
                    v = View()
                    ctypes.memmove(ctypes.byref(v), ctypes.byref(enc.view), ctypes.sizeof(View))
                    for a, _ in VIEW_ARRAYS:
                        if a in offs:
                            setattr(v, a, slot.data_ptr() + offs[a])
                        else:
                            setattr(v, a, tables[a].data_ptr())
                    vs.append((name, enc.n, v))
                per_slot.append(vs)
            self.views.append(per_slot)
        self.max_elements = max(enc.n for _, layout, _, _, _ in self.groups for _, enc, _ in layout)
        self.copy_stream = torch.cuda.Stream(device=self.device)
        self.copied = [torch.cuda.Event() for _ in range(2)]
        self.freed = [torch.cuda.Event() for _ in range(2)]

    def host_nbytes(self) -> int:
        return sum(size for _, _, _, size, _ in self.groups)

    def _copy(self, i: int):
        import torch
        _, _, blob, size, _ = self.groups[i]
        slot = i % 2
        with torch.cuda.stream(self.copy_stream):
            self.copy_stream.wait_event(self.freed[slot])
            self.slots[slot][:size].copy_(blob[:size], non_blocking=True)
            self.copied[slot].record(self.copy_stream)

    def decode_pass(self, out, on_matrix=None):
        """Stream every group in and decode its matrices into `out` (one
        reused buffer of at least max_elements BF16) on the current stream.
        on_matrix(group, name, out_view) runs after each decode is enqueued
        (the consumer of the decoded weight)."""
        import torch
        compute = torch.cuda.current_stream(self.device)
        for slot in range(2):
            self.freed[slot].record(compute)
        if self.groups:
            self._copy(0)
        for i, (gname, layout, _, _, _) in enumerate(self.groups):
            if i + 1 < len(self.groups):
                self._copy(i + 1)
            slot = i % 2
            compute.wait_event(self.copied[slot])
            for name, n, v in self.views[i][slot]:
                api.check(api.lib().df11_decode(ctypes.byref(v), out.data_ptr(), api._stream_handle(compute)),
                          "df11_decode")
                if on_matrix is not None:
                    on_matrix(gname, name, out[:n])
            self.freed[slot].record(compute)
