"""ctypes declarations for libdf11.so (include/df11.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# DF11_LIBRARY names another build of the same library (the sanitizer build
# of `python -m huffman_decode_df11_amd.build --sanitize`)
LIB_PATH = os.environ.get("DF11_LIBRARY") or os.path.join(_PKG, "_build", "libdf11.so")

DF11_OK = 0
DF11_MAX_TABLES = 64
DF11_FAST_BITS_MAX = 12
DF11_FAST_BITS_DEFAULT = 11
DF11_Y_F32 = 0
DF11_Y_BF16 = 1
DF11_STORES_AUTO, DF11_STORES_CACHED, DF11_STORES_STREAMING = 0, 1, 2
DF11_GEMM_AUTO, DF11_GEMM_SEGMENT, DF11_GEMM_WIDE, DF11_GEMM_TILED, DF11_GEMM_VECTOR, DF11_GEMM_PIPE, DF11_GEMM_RING = \
    0, 1, 2, 3, 4, 5, 6

u32, u64 = ctypes.c_uint32, ctypes.c_uint64


class Codebook(ctypes.Structure):
    _fields_ = [
        ("max_len", u32), ("min_len", u32), ("n_symbols", u32), ("n_tables", u32),
        ("fast_bits", u32), ("reserved", u32 * 3),
        ("len", ctypes.c_uint8 * 256),
        ("code", u32 * 256),
        ("chain", ctypes.c_uint16 * (DF11_MAX_TABLES * 256)),
        ("fast", u32 * (2 << DF11_FAST_BITS_MAX)),
    ]


class Layout(ctypes.Structure):
    _fields_ = [
        ("chunk_bytes", u32), ("seg_lanes", u32), ("align_elems", u64),
        ("rows", u64), ("cols", u64), ("tile_rows", u32), ("tile_cols", u32),
        ("tile_kchunk", u32), ("reserved", u32),
    ]


class Segment(ctypes.Structure):
    _fields_ = [("elem_off", u64), ("nbits", u32), ("reserved", u32)]


class View(ctypes.Structure):
    _fields_ = [
        ("n", u64), ("total_bits", u64), ("n_segments", u64),
        ("chunk_bytes", u32), ("seg_lanes", u32),
        ("rows", u64), ("cols", u64),
        ("tile_rows", u32), ("tile_cols", u32),
        ("tile_kchunk", u32), ("row_win_lo", ctypes.c_int32),
        ("align_elems", u64),
        ("min_len", u32), ("max_len", u32), ("n_tables", u32), ("fast_bits", u32),
        ("max_seg_elems", u32), ("row_win_span", u32),
        ("exp_words", ctypes.c_void_p), ("n_exp_words", u64),
        ("sm", ctypes.c_void_p), ("n_sm", u64),
        ("gaps", ctypes.c_void_p), ("n_gaps", u64),
        ("segs", ctypes.c_void_p), ("n_segs", u64),
        ("chain", ctypes.c_void_p), ("n_chain", u64),
        ("fast", ctypes.c_void_p), ("n_fast", u64),
        ("block_seg", ctypes.c_void_p), ("n_block_seg", u64),
        ("counts", ctypes.c_void_p), ("n_counts", u64),
    ]


class DecodeTuning(ctypes.Structure):
    _fields_ = [("waves", u32), ("stores", u32), ("groups", u32), ("reserved", u32 * 5)]


class GemmTuning(ctypes.Structure):
    _fields_ = [("kernel", u32), ("row_blocks", u32), ("parts", u32), ("split", u32), ("one_writer", u32),
                ("tiles_per_wave", u32), ("k_slices", u32), ("reserved", u32)]


# (field, element ctype) of every array in a view
VIEW_ARRAYS = (
    ("exp_words", ctypes.c_uint32),
    ("sm", ctypes.c_uint8),
    ("gaps", ctypes.c_uint8),
    ("segs", Segment),
    ("chain", ctypes.c_uint16),
    ("fast", ctypes.c_uint32),
    ("block_seg", ctypes.c_uint64),
    ("counts", ctypes.c_uint8),
)

EXPORTS = (
    "df11_hist_accumulate", "df11_codebook_build", "df11_encode", "df11_encoded_free",
    "df11_encoded_view", "df11_gemm_layout", "df11_gemm_tile_rows", "df11_gemm_tile_cols",
    "df11_validate", "df11_decode", "df11_decode_batch", "df11_decode_batch_tuned", "df11_decode_rows",
    "df11_decode_gemm", "df11_decode_gemm_out", "df11_decode_gemm_ex", "df11_decode_gemm_noalloc", "df11_decode_gemm_workspace_bytes", "df11_decode_gemm_noalloc", "df11_hist_device", "df11_encode_device", "df11_device_encoded_free", "df11_device_encoded_view",
    "df11_device_encoded_to_host",
    "df11_status_string", "df11_last_error", "df11_version",
)

_lib = None


class DF11Error(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        msg = "%s failed: %s (%d): %s" % (
            where, L.df11_status_string(status).decode(), status, L.df11_last_error().decode())
        super().__init__(msg)
        self.status = status


def lib():
    """Load libdf11.so.  Raises if the HIP library has not been built: there is
    no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libdf11.so not found at %s; build it with "
                          "`python -m huffman_decode_df11_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    L.df11_hist_accumulate.argtypes = [vp, u64, vp]
    L.df11_codebook_build.argtypes = [vp, u32, u32, ctypes.POINTER(Codebook)]
    L.df11_encode.argtypes = [vp, u64, ctypes.POINTER(Codebook), ctypes.POINTER(Layout), ctypes.POINTER(vp)]
    L.df11_encoded_free.argtypes = [vp]
    L.df11_encoded_free.restype = None
    L.df11_encoded_view.argtypes = [vp, ctypes.POINTER(View)]
    L.df11_gemm_layout.argtypes = [u64, u64, ctypes.POINTER(Layout)]
    L.df11_gemm_tile_rows.restype = u32
    L.df11_gemm_tile_cols.restype = u32
    L.df11_validate.argtypes = [ctypes.POINTER(View), ctypes.POINTER(Codebook)]
    L.df11_decode.argtypes = [ctypes.POINTER(View), vp, vp]
    L.df11_decode_batch.argtypes = [ctypes.POINTER(View), ctypes.POINTER(vp), u32, vp]
    L.df11_decode_batch_tuned.argtypes = [ctypes.POINTER(View), ctypes.POINTER(vp), u32,
                                          ctypes.POINTER(DecodeTuning), vp]
    L.df11_decode_rows.argtypes = [ctypes.POINTER(View), vp, u64, vp, vp]
    L.df11_decode_gemm.argtypes = [ctypes.POINTER(View), vp, u32, vp, vp, vp]
    L.df11_decode_gemm_out.argtypes = [ctypes.POINTER(View), vp, u32, vp, ctypes.c_int, vp, vp]
    L.df11_decode_gemm_ex.argtypes = [ctypes.POINTER(View), vp, u32, vp, ctypes.c_int, vp,
                                      ctypes.POINTER(GemmTuning), vp, u64, vp]
    L.df11_decode_gemm_workspace_bytes.argtypes = [ctypes.POINTER(View), u32]
    L.df11_decode_gemm_noalloc.argtypes = [ctypes.POINTER(View), vp, u32, vp, ctypes.c_int, vp,
                                           ctypes.POINTER(GemmTuning), vp]
    L.df11_decode_gemm_workspace_bytes.restype = u64
    L.df11_hist_device.argtypes = [vp, u64, vp, vp]
    L.df11_encode_device.argtypes = [vp, u64, ctypes.POINTER(Codebook), ctypes.POINTER(Layout), vp,
                                     ctypes.POINTER(vp)]
    L.df11_device_encoded_free.argtypes = [vp]
    L.df11_device_encoded_free.restype = None
    L.df11_device_encoded_view.argtypes = [vp, ctypes.POINTER(View)]
    L.df11_device_encoded_to_host.argtypes = [vp, ctypes.POINTER(vp)]
    L.df11_status_string.argtypes = [ctypes.c_int]
    L.df11_status_string.restype = ctypes.c_char_p
    L.df11_last_error.restype = ctypes.c_char_p
    L.df11_version.restype = ctypes.c_char_p
    for name in ("df11_hist_accumulate", "df11_codebook_build", "df11_encode", "df11_encoded_view",
                 "df11_gemm_layout", "df11_validate", "df11_decode", "df11_decode_batch", "df11_decode_batch_tuned",
                 "df11_decode_rows", "df11_decode_gemm", "df11_decode_gemm_out", "df11_decode_gemm_ex", "df11_decode_gemm_noalloc",
                 "df11_hist_device", "df11_encode_device",
                 "df11_device_encoded_view", "df11_device_encoded_to_host"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != DF11_OK:
        raise DF11Error(status, where)
