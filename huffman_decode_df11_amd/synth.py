"""Seeded synthetic BF16 workloads.

This module only draws random numbers and rounds them to BF16 bit patterns.
It holds none of the codec's arithmetic, so both the CPU oracle and the HIP
path can take their inputs from here.

Recipe (the pages publish no weights, so every workload is synthetic):

* ``normal``: values ~ N(0, sigma) drawn in float64, cast to float32 and then
  rounded to BF16 with round-to-nearest-even. sigma = 0.02 stands in for
  trained transformer weights.
* ``adversarial``: 99% Student-t with 3 degrees of freedom scaled by 0.02, and
  1% uniformly random 16-bit patterns, so every exponent value (zero,
  subnormal, Inf, NaN) occurs.
* ``fibonacci``: exponent counts follow the Fibonacci numbers over 34
  exponent values, which makes an unrestricted Huffman code 33 bits deep;
  sign and mantissa bits are uniform.
* ``exhaustive``: all 65,536 BF16 bit patterns once each, in order.

Every tensor draws from its own stream: ``SeedSequence(seed).spawn(k)[i]``
for the i-th of k tensors of a workload.

The 8B-parameter model (32 layers, embedding, head: 8.03e9 elements) is
drawn on the device with torch's Philox generator instead, seeded with
``model_stream_seed(seed, tensor_index)``, so that it can be generated, and
regenerated for checking, in seconds: same N(0, 0.02) float32 values
rounded to BF16 with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np

LLAMA3_8B_LAYER = (
    ("q_proj", 4096, 4096),
    ("k_proj", 1024, 4096),
    ("v_proj", 1024, 4096),
    ("o_proj", 4096, 4096),
    ("gate_proj", 14336, 4096),
    ("up_proj", 14336, 4096),
    ("down_proj", 4096, 14336),
)
LLAMA3_8B_VOCAB = 128256
LLAMA3_8B_HIDDEN = 4096
LLAMA3_8B_LAYERS = 32


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def streams(seed: int, k: int):
    """k independent generators spawned from one seed."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(k)]


def _normal_bits(rng, n: int, sigma: float, block: int = 1 << 24) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    for lo in range(0, n, block):
        hi = min(n, lo + block)
        v = rng.standard_normal(hi - lo) * sigma
        out[lo:hi] = f32_to_bf16_bits(v.astype(np.float32))
    return out


def normal_bf16(n: int, sigma: float = 0.02, seed: int = 0, index: int = 0,
                count: int = 1) -> np.ndarray:
    """n BF16 bit patterns of N(0, sigma) from stream ``index`` of ``count``."""
    return _normal_bits(streams(seed, count)[index], n, sigma)


def tensor_1024(seed: int = 0) -> np.ndarray:
    """One 1024 x 1024 N(0, 0.02) tensor (1,048,576 elements)."""
    return normal_bf16(1024 * 1024, 0.02, seed).reshape(1024, 1024)


def llama_layer(seed: int = 0, layer: int = 0, sigma: float = 0.02):
    """The seven weight matrices of one Llama-3-8B-shaped decoder layer.

    Returns a list of (name, uint16[rows, cols]) in the fixed order above.
    Layer ``layer`` of a model uses ``SeedSequence(seed).spawn(layers)``'s
    entry as its own seed so that layers differ.
    """
    base = int(np.random.SeedSequence(seed).spawn(layer + 1)[layer].generate_state(1)[0])
    gens = streams(base, len(LLAMA3_8B_LAYER))
    return [(name, _normal_bits(g, r * c, sigma).reshape(r, c))
            for g, (name, r, c) in zip(gens, LLAMA3_8B_LAYER)]


def adversarial_bf16(n: int = 1 << 24, seed: int = 0, frac_random: float = 0.01) -> np.ndarray:
    """99% t(3) * 0.02 and 1% uniformly random 16-bit patterns."""
    rng = streams(seed, 1)[0]
    v = (rng.standard_t(3, size=n) * 0.02).astype(np.float32)
    bits = f32_to_bf16_bits(v)
    mask = rng.random(n) < frac_random
    bits[mask] = rng.integers(0, 65536, size=int(mask.sum()), dtype=np.uint32).astype(np.uint16)
    return bits


def fibonacci_bf16(seed: int = 0, nsym: int = 34, first_exp: int = 100) -> np.ndarray:
    """Exponent counts F(1), F(2), ..., F(nsym) (F(1) = F(2) = 1) over exponents
    first_exp .. first_exp + nsym - 1, shuffled, with uniform sign and mantissa."""
    fib = [1, 1]
    while len(fib) < nsym:
        fib.append(fib[-1] + fib[-2])
    counts = np.array(fib[:nsym], dtype=np.int64)
    exps = np.repeat(np.arange(first_exp, first_exp + nsym, dtype=np.uint16), counts)
    rng = streams(seed, 1)[0]
    rng.shuffle(exps)
    low = rng.integers(0, 256, size=exps.size, dtype=np.uint16)
    return (((low & 0x80) << 8) | (exps << 7) | (low & 0x7F)).astype(np.uint16)


def exhaustive_bf16() -> np.ndarray:
    """Every 16-bit pattern once: 256 exponents x 256 sign/mantissa bytes."""
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def activations_bf16(batch: int, k: int = 4096, seed: int = 1) -> np.ndarray:
    """X[batch, k] ~ N(0, 1) as BF16 bits."""
    return normal_bf16(batch * k, 1.0, seed).reshape(batch, k)


# ---------------------------------------------------------------- 8B model

def llama3_8b_tensors(layers: int = LLAMA3_8B_LAYERS):
    """(group, name, rows, cols) of every weight matrix of the model in
    decode order: the embedding, the decoder layers, the LM head.  One
    group shares one codebook."""
    out = [("embed", "embed_tokens", LLAMA3_8B_VOCAB, LLAMA3_8B_HIDDEN)]
    for i in range(layers):
        out += [("layer%d" % i, name, r, c) for name, r, c in LLAMA3_8B_LAYER]
    out.append(("head", "lm_head", LLAMA3_8B_VOCAB, LLAMA3_8B_HIDDEN))
    return out


def model_stream_seed(seed: int, index: int) -> int:
    return (seed * 1000003 + index * 7919 + 17) & 0x7FFFFFFFFFFFFFFF


def normal_bf16_torch(rows: int, cols: int, seed: int, index: int, device, sigma: float = 0.02):
    """A [rows, cols] torch.bfloat16 tensor of N(0, sigma) drawn on `device`
    from the Philox stream model_stream_seed(seed, index)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(model_stream_seed(seed, index))
    x = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    x.mul_(sigma)
    return x.to(torch.bfloat16)
