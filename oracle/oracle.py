"""Python face of the DF11 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It wraps the plain C in ``df11_oracle.c`` (built with
gcc on first use) and adds a pure-Python brute force for tiny alphabets.
It imports nothing from the HIP library, and the library imports nothing
from here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "df11_oracle.c")
_SO = os.path.join(_HERE, "_build", "liborc.so")
_lock = threading.Lock()
_lib = None

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_u64 = ctypes.c_uint64


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, -O2) into oracle/_build."""
    with _lock:
        if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            os.makedirs(os.path.dirname(_SO), exist_ok=True)
            tmp = _SO + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-shared", "-fPIC",
                                   "-o", tmp, _SRC])
            os.replace(tmp, _SO)
    return _SO


def build_sanitized() -> str:
    """The oracle with AddressSanitizer and UndefinedBehaviorSanitizer
    (clang, shared sanitizer runtime) into oracle/_build_san, for the CPU
    tests run under the sanitizers (DF11_ORACLE_LIBRARY points at it)."""
    so = os.path.join(os.path.dirname(os.path.dirname(_SO)), "_build_san", "liborc.so")
    os.makedirs(os.path.dirname(so), exist_ok=True)
    subprocess.check_call(["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-std=c99", "-Wall", "-shared", "-fPIC",
                           "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                           "-shared-libsan", "-fno-omit-frame-pointer", "-o", so, _SRC])
    return so


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("DF11_ORACLE_LIBRARY") or build()
        L = ctypes.CDLL(path)
        L.orc_histogram.argtypes = [_u16p, _u64, _u64p]
        L.orc_huffman_lengths.argtypes = [_u64p, _u8p]
        L.orc_huffman_lengths.restype = ctypes.c_int
        L.orc_package_merge.argtypes = [_u64p, ctypes.c_int, _u8p]
        L.orc_package_merge.restype = ctypes.c_int
        L.orc_code_lengths.argtypes = [_u64p, ctypes.c_int, _u8p]
        L.orc_code_lengths.restype = ctypes.c_int
        L.orc_canonical_codes.argtypes = [_u8p, _u32p]
        L.orc_sign_mantissa.argtypes = [_u16p, _u64, _u8p]
        L.orc_code_starts.argtypes = [_u16p, _u64, _u8p, _u64, _u64, _u64p]
        L.orc_code_starts.restype = _u64
        L.orc_write_stream.argtypes = [_u16p, _u64, _u8p, _u32p, _u64p, _u8p]
        L.orc_decode.argtypes = [_u8p, _u64, _u8p, _u64, _u8p, _u64, _u64, _u16p]
        L.orc_decode.restype = ctypes.c_int
        L.orc_metadata.argtypes = [_u64p, _u16p, _u64, _u8p, _u64, _u64, _u64,
                                   _u8p, _u64p, _u32p]
        L.orc_chunk_counts.argtypes = [_u64p, _u64, _u64, _u64, _u8p]
        L.orc_chunk_counts.restype = ctypes.c_int
        L.orc_gemm_f32.argtypes = [_u16p, _u16p, _u64, _u64, _u64, _f32p]
        L.orc_gemm_f64.argtypes = [_u16p, _u16p, _u64, _u64, _u64, _f64p]
        L.orc_tile_order.argtypes = [_u16p, _u64, _u64, _u64, _u64, _u64, _u16p]
        _lib = L
    return _lib


def _u16(u) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(u).reshape(-1), dtype=np.uint16)


def histogram(u) -> np.ndarray:
    u = _u16(u)
    h = np.zeros(256, np.uint64)
    lib().orc_histogram(u, u.size, h)
    return h


def huffman_lengths(hist) -> np.ndarray:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(256, np.uint8)
    lib().orc_huffman_lengths(h, ln)
    return ln


def package_merge(hist, lmax: int) -> np.ndarray:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(256, np.uint8)
    if lib().orc_package_merge(h, int(lmax), ln) < 0:
        raise ValueError("too many symbols for lmax")
    return ln


def code_lengths(hist, lmax: int = 32) -> np.ndarray:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(256, np.uint8)
    if lib().orc_code_lengths(h, int(lmax), ln) < 0:
        raise ValueError("too many symbols for lmax")
    return ln


def canonical_codes(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    c = np.zeros(256, np.uint32)
    lib().orc_canonical_codes(ln, c)
    return c


def sign_mantissa(u) -> np.ndarray:
    u = _u16(u)
    sm = np.zeros(u.size, np.uint8)
    lib().orc_sign_mantissa(u, u.size, sm)
    return sm


class Encoded:
    """The oracle's encoding of one tensor: stream bytes (MSB first), total
    bits, sign+mantissa bytes, and the segment metadata for one layout."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def encode(u, lengths=None, lmax: int = 32, chunk_bytes: int = 16, seg_lanes: int = 64,
           align_elems: int = 0) -> Encoded:
    """Encode BF16 bits u with the given code lengths (default: this tensor's
    own histogram), laying the stream out in segments of seg_lanes chunks of
    chunk_bytes bytes."""
    u = _u16(u)
    n = u.size
    if lengths is None:
        lengths = code_lengths(histogram(u), lmax)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    codes = canonical_codes(ln)
    chunk_bits = chunk_bytes * 8
    seg_bits = chunk_bits * seg_lanes
    start = np.zeros(max(n, 1), np.uint64)
    total = int(lib().orc_code_starts(u, n, ln, seg_bits, align_elems, start))
    E = np.zeros((total + 7) // 8 + 8, np.uint8)
    lib().orc_write_stream(u, n, ln, codes, start, E)
    sm = sign_mantissa(u)
    nseg = (total + seg_bits - 1) // seg_bits
    gaps = np.zeros(max(nseg * seg_lanes, 1), np.uint8)
    seg_elem = np.zeros(nseg + 1, np.uint64)
    seg_nbits = np.zeros(max(nseg, 1), np.uint32)
    lib().orc_metadata(start, u, n, ln, chunk_bits, seg_bits, nseg, gaps, seg_elem, seg_nbits)
    counts = np.zeros(max(nseg * seg_lanes, 1), np.uint8)
    if lib().orc_chunk_counts(start, n, chunk_bits, nseg * seg_lanes, counts) != 0:
        raise ValueError("a chunk holds more than 255 codes: its count does not fit in a byte")
    return Encoded(n=n, lengths=ln, codes=codes, starts=start[:n], total_bits=total,
                   E=E[:(total + 7) // 8], sm=sm, n_segments=nseg,
                   gaps=gaps[:nseg * seg_lanes], counts=counts[:nseg * seg_lanes],
                   seg_elem=seg_elem, seg_nbits=seg_nbits[:nseg],
                   chunk_bytes=chunk_bytes, seg_lanes=seg_lanes, align_elems=align_elems)


def decode(E, total_bits: int, sm, n: int, lengths, seg_bits: int = 0,
           align_elems: int = 0) -> np.ndarray:
    """Bit-serial canonical decode of n elements."""
    E = np.ascontiguousarray(E, dtype=np.uint8)
    sm = np.ascontiguousarray(sm, dtype=np.uint8)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    out = np.zeros(max(n, 1), np.uint16)
    if E.size == 0:
        E = np.zeros(1, np.uint8)
    if sm.size == 0:
        sm = np.zeros(1, np.uint8)
    rc = lib().orc_decode(E, int(total_bits), sm, int(n), ln, int(seg_bits), int(align_elems), out)
    if rc != 0:
        raise ValueError("bit pattern is no code")
    return out[:n]


def gemm_f32(X, W) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    B, K = X.shape
    N = W.shape[0]
    assert W.shape[1] == K
    Y = np.zeros((B, N), np.float32)
    lib().orc_gemm_f32(X.reshape(-1), W.reshape(-1), B, N, K, Y.reshape(-1))
    return Y


def gemm_f64(X, W) -> np.ndarray:
    X = np.ascontiguousarray(X, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    B, K = X.shape
    N = W.shape[0]
    Y = np.zeros((B, N), np.float64)
    lib().orc_gemm_f64(X.reshape(-1), W.reshape(-1), B, N, K, Y.reshape(-1))
    return Y


def round_bf16(x) -> np.ndarray:
    """BF16 bit patterns of float32 values x, each the nearer of its two
    neighbouring BF16 values, ties to the one whose last mantissa bit is 0
    (IEEE 754 round-to-nearest-even; BF16 is binary32 with the low 16
    mantissa bits dropped: 1 sign, 8 exponent, 7 mantissa bits, as the
    pages give the format).  A value at or past the midpoint between the
    largest finite BF16 and 2^128 becomes infinity; NaN becomes a quiet NaN
    (the quiet bit set on the truncated pattern).

    Written from that definition with exact float64 distances, not with the
    integer rounding trick."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lo = (bits >> 16).astype(np.int64)               # toward zero, same sign
    e = (lo >> 7) & 0xFF
    sign = np.where(lo & 0x8000, -1.0, 1.0)
    with np.errstate(invalid="ignore"):              # NaN and Inf are settled below
        vlo = ((lo.astype(np.uint32) << 16)).view(np.float32).astype(np.float64)
        ulp = np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)  # BF16 spacing at this exponent
        vhi = vlo + sign * ulp                       # next BF16 away from zero (2^128 past the top)
        xv = x.astype(np.float64)
        dlo = np.abs(xv - vlo)
        dhi = np.abs(vhi - xv)
        up = (dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1))
    out = np.where(up, lo + 1, lo)
    out = np.where(np.isinf(x), lo, out)
    out = np.where(np.isnan(x), lo | 0x40, out)
    return out.astype(np.uint16)


def tile_order(u, rows: int, cols: int, tile_rows: int, tile_cols: int, kchunk: int = 0) -> np.ndarray:
    u = _u16(u)
    out = np.zeros(u.size, np.uint16)
    lib().orc_tile_order(u, rows, cols, tile_rows, tile_cols, kchunk, out)
    return out


# ---------------------------------------------------------------------------
# pure-Python brute force for tiny alphabets

def brute_min_cost(weights, lmax: int = 32) -> int:
    """Least sum(w_i * l_i) over all length vectors with 1 <= l_i <= lmax and
    Kraft sum <= 1 (every such vector is a prefix code).  Exhaustive; meant
    for at most 7 symbols."""
    w = [int(x) for x in weights]
    k = len(w)
    if k == 0:
        return 0
    if k == 1:
        return w[0]
    top = min(lmax, k - 1)
    best = None

    def rec(i, kraft_num, cost):
        nonlocal best
        if i == k:
            if best is None or cost < best:
                best = cost
            return
        for l in range(1, top + 1):
            kn = kraft_num + (1 << (top - l))
            if kn <= (1 << top):
                rec(i + 1, kn, cost + w[i] * l)

    rec(0, 0, 0)
    return best


def entropy_bits(hist) -> float:
    h = np.asarray(hist, dtype=np.float64)
    p = h[h > 0] / h.sum()
    return float(-(p * np.log2(p)).sum())
