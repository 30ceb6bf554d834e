"""Thin Python binding over libdf11.so: argument marshalling only.

Every step of the codec runs in the library -- the host encoder in C++ and
the decode paths in HIP kernels on the GPU.  PyTorch provides device memory
and streams.  There is no Python or CPU fallback: if the library is missing
the calls raise.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from . import _lib
from ._lib import DF11_Y_BF16, DF11_Y_F32, Codebook, DecodeTuning, GemmTuning, Layout, View, check, lib

DEFAULT_MAX_LEN = 32
DEFAULT_FAST_BITS = _lib.DF11_FAST_BITS_DEFAULT


def _u16(bits) -> np.ndarray:
    try:
        import torch
        if isinstance(bits, torch.Tensor):
            if bits.is_cuda:
                raise ValueError("the encoder runs on the host: pass a CPU tensor or numpy array")
            bits = bits.contiguous().view(torch.int16).numpy()
    except ImportError:
        pass
    a = np.asarray(bits)
    if a.dtype not in (np.uint16, np.int16):
        raise TypeError("BF16 weights are passed as their 16-bit patterns (uint16/int16), got %s" % a.dtype)
    return np.ascontiguousarray(a.reshape(-1)).view(np.uint16)


def hist_accumulate(bits, hist: Optional[np.ndarray] = None) -> np.ndarray:
    """Add the exponent counts of `bits` to `hist` (new zeros if None)."""
    u = _u16(bits)
    if hist is None:
        hist = np.zeros(256, np.uint64)
    assert hist.dtype == np.uint64 and hist.size == 256 and hist.flags.c_contiguous
    check(lib().df11_hist_accumulate(u.ctypes.data, u.size, hist.ctypes.data), "df11_hist_accumulate")
    return hist


def build_codebook(hist, max_len: int = DEFAULT_MAX_LEN, fast_bits: int = DEFAULT_FAST_BITS) -> Codebook:
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    cb = Codebook()
    check(lib().df11_codebook_build(h.ctypes.data, max_len, fast_bits, ctypes.byref(cb)), "df11_codebook_build")
    return cb


def codebook_lengths(cb: Codebook) -> np.ndarray:
    return np.frombuffer(bytes(cb.len), dtype=np.uint8).copy()


def codebook_codes(cb: Codebook) -> np.ndarray:
    return np.ctypeslib.as_array(cb.code).astype(np.uint32).copy()


def make_layout(chunk_bytes: int = 16, align_elems: int = 0, rows: int = 0, cols: int = 0,
                tile_rows: int = 0, tile_cols: int = 0, tile_kchunk: int = 0) -> Layout:
    return Layout(chunk_bytes=chunk_bytes, seg_lanes=64, align_elems=align_elems, rows=rows,
                  cols=cols, tile_rows=tile_rows, tile_cols=tile_cols, tile_kchunk=tile_kchunk)


def gemm_layout(rows: int, cols: int) -> Layout:
    lay = Layout()
    check(lib().df11_gemm_layout(rows, cols, ctypes.byref(lay)), "df11_gemm_layout")
    return lay


def gemm_tile() -> tuple:
    L = lib()
    return int(L.df11_gemm_tile_rows()), int(L.df11_gemm_tile_cols())


class Encoded:
    """A host encoding owned by the library (freed with the object)."""

    def __init__(self, handle: int, codebook: Codebook, shape: tuple):
        self._handle = ctypes.c_void_p(handle)
        self.codebook = codebook
        self.shape = shape
        self.view = View()
        check(lib().df11_encoded_view(self._handle, ctypes.byref(self.view)), "df11_encoded_view")
        self.arrays = {}
        for name, ct in _lib.VIEW_ARRAYS:
            count = int(getattr(self.view, "n_" + name))
            ptr = getattr(self.view, name)
            nbytes = count * ctypes.sizeof(ct)
            if nbytes:
                buf = (ctypes.c_uint8 * nbytes).from_address(ptr)
                buf._owner = self   # the arrays keep the library-owned encoding alive
                self.arrays[name] = np.frombuffer(buf, dtype=np.uint8)
            else:
                self.arrays[name] = np.zeros(0, np.uint8)

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h is not None and h.value:
            try:
                lib().df11_encoded_free(h)
            except Exception:   # interpreter shutdown: the module may be gone
                pass
            self._handle = None

    # typed views of the host arrays
    @property
    def exp_words(self): return self.arrays["exp_words"].view(np.uint32)
    @property
    def sm(self): return self.arrays["sm"]
    @property
    def gaps(self): return self.arrays["gaps"]
    @property
    def counts(self): return self.arrays["counts"]
    @property
    def seg_elem(self): return self.arrays["segs"].view(np.uint64).reshape(-1, 2)[:, 0]
    @property
    def seg_nbits(self): return self.arrays["segs"].view(np.uint32).reshape(-1, 4)[:, 2]
    @property
    def chain(self): return self.arrays["chain"].view(np.uint16)
    @property
    def fast(self): return self.arrays["fast"].view(np.uint32)
    @property
    def block_seg(self): return self.arrays["block_seg"].view(np.uint64)

    @property
    def n(self) -> int: return int(self.view.n)
    @property
    def total_bits(self) -> int: return int(self.view.total_bits)
    @property
    def n_segments(self) -> int: return int(self.view.n_segments)

    def stream_bytes_msb_first(self) -> np.ndarray:
        """The exponent stream as a byte sequence, first bit in bit 7 of byte 0."""
        nbytes = (self.total_bits + 7) // 8
        return self.exp_words.byteswap().view(np.uint8)[:nbytes]

    def compressed_nbytes(self) -> int:
        """Bytes a decode reads: stream, sign+mantissa, gaps, segment records, tables."""
        return sum(a.size for k, a in self.arrays.items() if k != "block_seg")

    def bits_per_weight(self) -> float:
        return 8.0 * self.compressed_nbytes() / max(self.n, 1)

    def validate(self) -> None:
        check(lib().df11_validate(ctypes.byref(self.view), ctypes.byref(self.codebook)), "df11_validate")

    def to(self, device="cuda") -> "DF11Tensor":
        return DF11Tensor(self, device)


def encode(bits, codebook: Optional[Codebook] = None, layout: Optional[Layout] = None,
           max_len: int = DEFAULT_MAX_LEN, fast_bits: int = DEFAULT_FAST_BITS) -> Encoded:
    """Encode BF16 bit patterns on the host.  Without a codebook one is built
    from this tensor's own exponent histogram."""
    shape = tuple(np.shape(bits)) if not hasattr(bits, "shape") else tuple(bits.shape)
    u = _u16(bits)
    if codebook is None:
        codebook = build_codebook(hist_accumulate(u), max_len, fast_bits)
    h = ctypes.c_void_p()
    lay = ctypes.byref(layout) if layout is not None else None
    check(lib().df11_encode(u.ctypes.data, u.size, ctypes.byref(codebook), lay, ctypes.byref(h)), "df11_encode")
    return Encoded(h.value, codebook, shape)


def hist_device(bits, hist: Optional[np.ndarray] = None, stream=None) -> np.ndarray:
    """Exponent counts of a device BF16 tensor (computed on the GPU), added
    into `hist` (new zeros if None)."""
    if hist is None:
        hist = np.zeros(256, np.uint64)
    assert hist.dtype == np.uint64 and hist.size == 256 and hist.flags.c_contiguous
    t = bits.contiguous()
    assert t.is_cuda and t.element_size() == 2
    check(lib().df11_hist_device(t.data_ptr(), t.numel(), hist.ctypes.data, _stream_handle(stream)),
          "df11_hist_device")
    return hist


class DeviceEncoded:
    """An encoding made on the GPU (df11_encode_device); every array lives in
    device memory owned by the library.  Usable wherever a DF11Tensor is
    (decode, decode_rows, decode_gemm)."""

    def __init__(self, handle: int, codebook: Codebook, shape: tuple, device):
        self._handle = ctypes.c_void_p(handle)
        self.codebook = codebook
        self.shape = shape
        self.device = device
        self.view = View()
        check(lib().df11_device_encoded_view(self._handle, ctypes.byref(self.view)), "df11_device_encoded_view")
        self.host_view = self.view      # only its scalar fields are read on the host
        # decode through the codebook's shared device tables (the library's
        # own copy stays allocated), so that tensors of one codebook can be
        # decoded in one batched launch
        shared = _codebook_tables(codebook, device)
        self.view.chain = shared["chain"].data_ptr()
        self.view.fast = shared["fast"].data_ptr()
        self._tables = shared
        self.n = int(self.view.n)
        self.total_bits = int(self.view.total_bits)
        self.n_segments = int(self.view.n_segments)

    def compressed_nbytes(self) -> int:
        return sum(int(getattr(self.view, "n_" + name)) * ctypes.sizeof(ct)
                   for name, ct in _lib.VIEW_ARRAYS if name != "block_seg")

    def to_host(self) -> Encoded:
        h = ctypes.c_void_p()
        check(lib().df11_device_encoded_to_host(self._handle, ctypes.byref(h)), "df11_device_encoded_to_host")
        return Encoded(h.value, self.codebook, self.shape)

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h is not None and h.value:
            try:
                lib().df11_device_encoded_free(h)
            except Exception:   # interpreter shutdown: the module may be gone
                pass
            self._handle = None


def encode_device(bits, codebook: Optional[Codebook] = None, layout: Optional[Layout] = None,
                  max_len: int = DEFAULT_MAX_LEN, fast_bits: int = DEFAULT_FAST_BITS, stream=None) -> DeviceEncoded:
    """Encode a device BF16 tensor on the GPU.  Without a codebook one is
    built (on the host, 256 symbols) from the tensor's device histogram."""
    t = bits.contiguous()
    assert t.is_cuda and t.element_size() == 2
    if codebook is None:
        codebook = build_codebook(hist_device(t, stream=stream), max_len, fast_bits)
    h = ctypes.c_void_p()
    lay = ctypes.byref(layout) if layout is not None else None
    check(lib().df11_encode_device(t.data_ptr(), t.numel(), ctypes.byref(codebook), lay, _stream_handle(stream),
                                   ctypes.byref(h)), "df11_encode_device")
    return DeviceEncoded(h.value, codebook, tuple(t.shape), t.device)


_TABLE_ARRAYS = ("chain", "fast")


def _codebook_tables(cb: Codebook, device):
    """The codebook's chain and fast tables on `device`, uploaded once per
    codebook and device (the same cache the host encodings use)."""
    import torch
    cache = getattr(cb, "_device_tables", None)
    if cache is None:
        cache = {}
        cb._device_tables = cache
    key = str(torch.device(device))
    if key not in cache:
        chain = np.ctypeslib.as_array(cb.chain)[:cb.n_tables * 256].astype(np.uint16).view(np.uint8)
        fast = np.ctypeslib.as_array(cb.fast)[:2 << cb.fast_bits].astype(np.uint32).view(np.uint8)
        cache[key] = {"chain": torch.from_numpy(chain.copy()).to(device),
                      "fast": torch.from_numpy(fast.copy()).to(device)}
    return cache[key]


def _device_tables(enc: Encoded, device):
    """The codebook's tables on `device`, uploaded once per codebook and
    device, so that tensors sharing a codebook share device tables (which a
    batched decode requires)."""
    return _codebook_tables(enc.codebook, device)


class DF11Tensor:
    """An encoded tensor resident in device memory, plus its device view."""

    def __init__(self, enc: Encoded, device="cuda"):
        import torch
        self.shape = enc.shape
        self.n = enc.n
        self.codebook = enc.codebook
        self.host_view = enc.view
        self.tensors = {}
        shared = _device_tables(enc, device)
        for name, _ in _lib.VIEW_ARRAYS:
            if name in shared:
                self.tensors[name] = shared[name]
                continue
            a = enc.arrays[name]
            t = torch.from_numpy(a.copy() if a.size else np.zeros(16, np.uint8)).to(device)
            self.tensors[name] = t
        self.view = View()
        ctypes.memmove(ctypes.byref(self.view), ctypes.byref(enc.view), ctypes.sizeof(View))
        for name, _ in _lib.VIEW_ARRAYS:
            setattr(self.view, name, self.tensors[name].data_ptr())
        self.device = self.tensors["sm"].device
        self.total_bits = int(enc.view.total_bits)
        self.n_segments = int(enc.view.n_segments)
        self._compressed = enc.compressed_nbytes()

    def compressed_nbytes(self) -> int:
        """Bytes of the encoding a decode reads (same count as Encoded's)."""
        return self._compressed

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors.values())


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def decode(t: DF11Tensor, out=None, stream=None):
    """Decode to BF16 on the GPU (bit-exact).  Returns `out` (a new
    torch.bfloat16 tensor of t.shape when None)."""
    import torch
    if out is None:
        out = torch.empty(t.shape if t.shape else (t.n,), dtype=torch.bfloat16, device=t.device)
    assert out.is_cuda and out.is_contiguous() and out.numel() >= t.n and out.element_size() == 2
    check(lib().df11_decode(ctypes.byref(t.view), out.data_ptr(), _stream_handle(stream)), "df11_decode")
    return out


def decode_tuning(waves: int = 0, stores: int = 0, groups: int = 0) -> DecodeTuning:
    """Explicit launch choices for decode_batch (0 = the library's choice)."""
    return DecodeTuning(waves=waves, stores=stores, groups=groups)


def gemm_tuning(kernel: int = 0, row_blocks: int = 0, parts: int = 0, split: int = 0,
                one_writer: int = 0, tiles_per_wave: int = 0, k_slices: int = 0) -> GemmTuning:
    """Explicit kernel choices for decode_gemm (0 = the library's choice);
    one_writer=1: y summed in a fixed order, the same on every run;
    tiles_per_wave: batch tiles per matrix-core wave of the pipelined kernel;
    k_slices: matrix-core waves per batch tile of the exponent-ring kernel."""
    return GemmTuning(kernel=kernel, row_blocks=row_blocks, parts=parts, split=split, one_writer=one_writer,
                      tiles_per_wave=tiles_per_wave, k_slices=k_slices)


def decode_batch(tensors: Sequence[DF11Tensor], outs=None, stream=None, tuning: Optional[DecodeTuning] = None):
    """Decode several tensors that share a codebook in one launch.  Returns
    the list of outputs (new torch.bfloat16 tensors where outs is None)."""
    import torch
    tensors = list(tensors)
    if outs is None:
        outs = [torch.empty(t.shape if t.shape else (t.n,), dtype=torch.bfloat16, device=t.device)
                for t in tensors]
    assert len(outs) == len(tensors)
    views = (View * max(len(tensors), 1))()
    ptrs = (ctypes.c_void_p * max(len(tensors), 1))()
    for i, (t, o) in enumerate(zip(tensors, outs)):
        assert o.is_cuda and o.is_contiguous() and o.numel() >= t.n and o.element_size() == 2
        ctypes.memmove(ctypes.byref(views, i * ctypes.sizeof(View)), ctypes.byref(t.view), ctypes.sizeof(View))
        ptrs[i] = o.data_ptr()
    if tuning is None:
        check(lib().df11_decode_batch(views, ptrs, len(tensors), _stream_handle(stream)), "df11_decode_batch")
    else:
        check(lib().df11_decode_batch_tuned(views, ptrs, len(tensors), ctypes.byref(tuning), _stream_handle(stream)),
              "df11_decode_batch_tuned")
    return outs


def decode_rows(t: DF11Tensor, rows, out=None, stream=None):
    """Decode only the rows `rows` (a device int64 tensor of row ids) of a
    row-major [R, C] tensor into out [len(rows), C] (new when None)."""
    import torch
    C = int(t.host_view.cols)
    rows = rows.reshape(-1)
    assert rows.is_cuda and rows.dtype == torch.int64
    rows = rows.contiguous()
    if out is None:
        out = torch.empty((rows.numel(), C), dtype=torch.bfloat16, device=rows.device)
    assert out.is_contiguous() and out.numel() >= rows.numel() * C and out.element_size() == 2
    check(lib().df11_decode_rows(ctypes.byref(t.view), rows.data_ptr(), rows.numel(), out.data_ptr(),
                                 _stream_handle(stream)), "df11_decode_rows")
    return out


def gemm_workspace_bytes(w: DF11Tensor, B: int) -> int:
    """Bytes of the packed-x workspace decode_gemm uses for B rows of x."""
    return int(lib().df11_decode_gemm_workspace_bytes(ctypes.byref(w.view), B))


def decode_gemm(w: DF11Tensor, x, out=None, w_debug=None, stream=None, out_dtype=None,
                tuning: Optional[GemmTuning] = None, workspace="auto"):
    """y = x @ W^T with W decoded tile by tile inside the kernel.  x: [B, K]
    bf16 on the GPU; returns y [B, N], float32 (default) or bfloat16
    (out_dtype=torch.bfloat16, or an `out` of that type: the float32 sum
    rounded once, ties to even).  tuning: explicit kernel choices.
    workspace: "auto" (above 32 rows of x, a device buffer from torch's
    allocator for x in operand order), None (x read in place), or a uint8
    device tensor of at least gemm_workspace_bytes(w, B) bytes."""
    import torch
    N, K = int(w.host_view.rows), int(w.host_view.cols)
    assert x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2 and x.shape[1] == K
    x = x.contiguous()
    B = x.shape[0]
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    assert out_dtype in (torch.float32, torch.bfloat16)
    if out is None:
        out = torch.empty((B, N), dtype=out_dtype, device=x.device)
    assert out.is_contiguous() and out.dtype == out_dtype and out.numel() == B * N
    wd = 0
    if w_debug is not None:
        assert w_debug.is_contiguous() and w_debug.numel() == N * K and w_debug.element_size() == 2
        wd = w_debug.data_ptr()
    y_dtype = DF11_Y_BF16 if out_dtype == torch.bfloat16 else DF11_Y_F32
    ws_ptr, ws_bytes = None, 0
    if isinstance(workspace, str):
        assert workspace == "auto"
        ws_bytes = gemm_workspace_bytes(w, B)
        if ws_bytes:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
            ws_ptr = workspace.data_ptr()
    elif workspace is not None:
        assert workspace.is_cuda and workspace.is_contiguous()
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().df11_decode_gemm_ex(ctypes.byref(w.view), x.data_ptr(), B, out.data_ptr(), y_dtype, wd,
                                    ctypes.byref(tuning) if tuning is not None else None, ws_ptr, ws_bytes,
                                    _stream_handle(stream)), "df11_decode_gemm_ex")
    return out
