"""torch.nn modules whose weights stay DFloat11-compressed on the GPU.

[P1] "DFloat11无损压缩技术：基于哈夫曼编码的BFloat16大模型显存优化方案" 2.2
     item 3, [P2] "DFloat11：用于高效 GPU 推理的 LLM 和扩散模型无损压缩"
     "工作原理": the compressed weights stay in GPU memory and each matrix is
     restored to BF16 right before its product, then discarded.

DF11Linear computes y = x W^T (+ b) either with the fused kernel
(df11_decode_gemm: W decoded tile by tile inside the matrix-core kernel,
never written to HBM) or by decoding W into a buffer shared by all modules
on the device and calling torch.matmul.  DF11Embedding restores only the
rows a lookup needs (df11_decode_rows).  Every weight byte is decoded by the
HIP library; nothing falls back to the CPU.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import api

_BUFFERS = {}


def _shared_buffer(device: torch.device, numel: int) -> torch.Tensor:
    """One BF16 buffer per device, grown to the largest weight decoded into it."""
    key = str(device)
    buf = _BUFFERS.get(key)
    if buf is None or buf.numel() < numel:
        buf = torch.empty(numel, dtype=torch.bfloat16, device=device)
        _BUFFERS[key] = buf
    return buf


def _bits(weight) -> np.ndarray:
    if isinstance(weight, torch.Tensor):
        assert weight.dtype == torch.bfloat16
        return weight.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    a = np.asarray(weight)
    assert a.dtype == np.uint16
    return a


class DF11Linear(torch.nn.Module):
    """A linear layer y = x W^T + b with W [out_features, in_features] held
    compressed.  mode "fused" (needs out % 32 == 0 and in % 512 == 0) runs
    the fused product (x packed in operand order above 32 rows) for up to
    fused_max_rows rows of x and decode + matmul above (default 256, the
    fused kernels' limit: on an up_proj-shaped weight, 14336 x 4096, the
    fused call measured about 37 / 45 / 62 / 85 us at 1 / 64 / 128 / 256
    rows against about 60 / 79 / 82 / 105 us for decoding the tile-ordered
    weight and calling torch.matmul); mode "decode" always decodes into the
    shared buffer and calls torch.matmul.  "auto" picks "fused" when the shape allows it.
    deterministic=True asks the fused kernels for one writer per element of
    y (df11_gemm_tuning one_writer): the same output on every run, where
    weights with few 32-row blocks (4096 x 4096, 4096 x 14336) otherwise
    split a row block's work and add float32 partial sums atomically."""

    fused_max_rows = 256

    def __init__(self, weight, bias: Optional[torch.Tensor] = None, mode: str = "auto", device="cuda",
                 codebook=None, deterministic: bool = False):
        super().__init__()
        self.deterministic = bool(deterministic)
        w = _bits(weight)
        assert w.ndim == 2
        self.out_features, self.in_features = (int(v) for v in w.shape)
        fits = self.out_features % api.gemm_tile()[0] == 0 and self.in_features % api.gemm_tile()[1] == 0
        if mode == "auto":
            mode = "fused" if fits else "decode"
        if mode == "fused" and not fits:
            raise ValueError("fused mode needs out_features %% 32 == 0 and in_features %% 512 == 0")
        if mode not in ("fused", "decode"):
            raise ValueError("mode must be auto, fused or decode")
        self.mode = mode
        layout = (api.gemm_layout(self.out_features, self.in_features) if mode == "fused"
                  else api.make_layout(rows=self.out_features, cols=self.in_features))
        self.weight_df11 = api.encode(w, codebook=codebook, layout=layout).to(device)
        self.device = self.weight_df11.device
        self.bias = (torch.nn.Parameter(bias.detach().to(self.device, torch.bfloat16), requires_grad=False)
                     if bias is not None else None)

    @classmethod
    def from_linear(cls, lin: torch.nn.Linear, mode: str = "auto", device="cuda",
                    deterministic: bool = False) -> "DF11Linear":
        return cls(lin.weight.detach().to(torch.bfloat16), lin.bias, mode=mode, device=device,
                   deterministic=deterministic)

    def decoded_weight(self) -> torch.Tensor:
        """W restored into the shared buffer (valid until the next decode on
        this device), as an [out, in] BF16 view."""
        n = self.out_features * self.in_features
        buf = _shared_buffer(self.device, n)
        api.decode(self.weight_df11, out=buf)
        return buf[:n].view(self.out_features, self.in_features)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        shape = x.shape
        x2 = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        B = x2.shape[0]
        if self.mode == "fused" and 1 <= B <= min(256, self.fused_max_rows):
            y = api.decode_gemm(self.weight_df11, x2,
                                tuning=api.gemm_tuning(one_writer=1) if self.deterministic else None)
            if self.bias is not None:
                y = y + self.bias.float()
            y = y.to(torch.bfloat16)
        else:
            y = torch.matmul(x2, self.decoded_weight().t())
            if self.bias is not None:
                y = y + self.bias
        return y.reshape(*shape[:-1], self.out_features)

    def extra_repr(self) -> str:
        return "in_features=%d, out_features=%d, mode=%s, bits_per_weight=%.2f" % (
            self.in_features, self.out_features, self.mode,
            8.0 * self.weight_df11.compressed_nbytes() / (self.in_features * self.out_features))


class DF11Embedding(torch.nn.Module):
    """An embedding table [num_embeddings, embedding_dim] held compressed;
    a lookup decodes only the rows it returns.  Ids must lie in
    [0, num_embeddings) (an id outside leaves its output row unwritten).
    chunk_bytes 8 (the default) halves the segments a looked-up row decodes
    (128256 x 4096 table: 6.7 against 8.7 us for one id, 7.2 against 9.3 us
    for 32) for 0.37 more bits per weight; 16 is the smaller encoding."""

    def __init__(self, weight, device="cuda", codebook=None, chunk_bytes: int = 8):
        super().__init__()
        w = _bits(weight)
        assert w.ndim == 2
        self.num_embeddings, self.embedding_dim = (int(v) for v in w.shape)
        if self.embedding_dim % 8:
            raise ValueError("embedding_dim must be a multiple of 8")
        layout = api.make_layout(rows=self.num_embeddings, cols=self.embedding_dim, chunk_bytes=chunk_bytes)
        self.weight_df11 = api.encode(w, codebook=codebook, layout=layout).to(device)
        self.device = self.weight_df11.device

    @classmethod
    def from_embedding(cls, emb: torch.nn.Embedding, device="cuda") -> "DF11Embedding":
        return cls(emb.weight.detach().to(torch.bfloat16), device=device)

    def forward(self, ids: torch.Tensor) -> torch.Tensor:
        flat = ids.reshape(-1).to(self.device, torch.int64)
        out = api.decode_rows(self.weight_df11, flat)
        return out.view(*ids.shape, self.embedding_dim)
