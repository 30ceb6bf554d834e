"""Host-side checks of the device entry points, with no GPU work:

- the decode kernels' per-segment address arithmetic (segment_plan.h,
  compiled for the CPU into df11_segment_bounds_check) keeps every store,
  staging access and sign+mantissa load of a segment inside its array for
  random and corrupt segment records, and covers each element once;
- the argument checks that refuse a call before anything is launched:
  views whose max_seg_elems or code lengths are out of range, chunk sizes
  the kernels do not read, tuning choices that do not apply, and the fused
  product's segment-parallel kernel for weights whose segments would not fit
  its staging (all-zero and 95%-zero weights).  The views are host views:
  their pointers are never dereferenced, because every call here is refused
  first."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from huffman_decode_df11_amd import _lib, api, synth
from huffman_decode_df11_amd.build import BOUNDS_CHECK


def test_segment_address_arithmetic_stays_in_bounds():
    if not os.path.exists(BOUNDS_CHECK):
        pytest.skip("df11_segment_bounds_check is built by huffman_decode_df11_amd.build")
    for seed in (1, 2, 3):
        r = subprocess.run([BOUNDS_CHECK, "60000", str(seed)], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert r.stdout.startswith("ok:"), r.stdout


def _copy(view):
    v = _lib.View()
    ctypes.memmove(ctypes.byref(v), ctypes.byref(view), ctypes.sizeof(_lib.View))
    return v


def _aligned(nbytes):
    raw = np.zeros(nbytes + 64, np.uint8)
    off = (-raw.ctypes.data) % 64
    return raw, raw.ctypes.data + off


@pytest.fixture(scope="module")
def enc():
    return api.encode(synth.normal_bf16(200_000, 0.02, seed=1))


@pytest.mark.parametrize("field,value", [("max_seg_elems", 0), ("max_seg_elems", 8193), ("min_len", 0),
                                         ("max_len", 33), ("chunk_bytes", 32), ("chunk_bytes", 4)])
def test_decode_refuses_bad_views(enc, field, value):
    v = _copy(enc.view)
    setattr(v, field, value)
    if field == "max_seg_elems" and value > 0:
        v.min_len = 1       # 8192 bits of 1-bit codes: at most 8192 per segment
    _, out = _aligned(2 * enc.n)
    rc = _lib.lib().df11_decode(ctypes.byref(v), out, None)
    assert rc == -1, _lib.lib().df11_last_error()


def test_decode_refuses_bad_tuning(enc):
    _, out = _aligned(2 * enc.n)
    outs = (ctypes.c_void_p * 1)(out)
    L = _lib.lib()
    for t in (api.decode_tuning(waves=5), api.decode_tuning(waves=18), api.decode_tuning(stores=3)):
        rc = L.df11_decode_batch_tuned(ctypes.byref(enc.view), outs, 1, ctypes.byref(t), None)
        assert rc == -1, L.df11_last_error()


def _gemm_call(view, B, tune, y_dtype=_lib.DF11_Y_F32, w_debug=False):
    N, K = int(view.rows), int(view.cols)
    _x, x = _aligned(2 * B * K)
    _y, y = _aligned(4 * B * N)
    _w, w = _aligned(2 * N * K)
    rc = _lib.lib().df11_decode_gemm_ex(ctypes.byref(view), x, B, y, y_dtype, w if w_debug else None,
                                        ctypes.byref(tune), None, 0, None)
    return rc, _lib.lib().df11_last_error().decode()


@pytest.mark.parametrize("kind", ["zero", "sparse95"])
def test_fused_segment_kernel_refused_when_staging_exceeds_64k(kind):
    """Segments of 1-bit codes hold up to 8,192 weights (all-zero weight) or
    ~7,300 (95% zeros): eight waves' staging would pass the 64 KB that the
    emit loop can address, so the segment-parallel kernel is refused (the
    automatic choice takes the tile-synchronous or wide kernel instead,
    checked on the GPU)."""
    N, K = 64, 4096
    if kind == "zero":
        W = np.zeros((N, K), np.uint16)
    else:
        W = synth.normal_bf16(N * K, 0.02, seed=78).reshape(N, K)
        W[np.random.default_rng(77).random((N, K)) < 0.95] = 0
    e = api.encode(W, layout=api.gemm_layout(N, K))
    assert 16 + 8 * (e.view.max_seg_elems + 1024 + 31) > 65520
    for B in (1, 33):
        rc, msg = _gemm_call(e.view, B, api.gemm_tuning(kernel=_lib.DF11_GEMM_SEGMENT))
        assert rc == -7 and "staging" in msg, msg
    # the vector kernel (one or two rows of x) keeps the same staging, 8 or 12 waves
    rc, msg = _gemm_call(e.view, 1, api.gemm_tuning(kernel=_lib.DF11_GEMM_VECTOR))
    assert rc == -7 and "staging" in msg, msg


@pytest.mark.parametrize("B,tune,bf16,wd", [
    (8, dict(kernel=_lib.DF11_GEMM_SEGMENT), False, True),          # no w_debug on the segment kernel
    (65, dict(kernel=_lib.DF11_GEMM_SEGMENT), False, False),        # at most two batch tiles
    (8, dict(kernel=_lib.DF11_GEMM_WIDE), False, False),            # the wide kernel takes > 32 rows
    (8, dict(kernel=_lib.DF11_GEMM_TILED, row_blocks=2), False, False),
    (8, dict(parts=2), False, False),                               # parts without the segment kernel
    (8, dict(kernel=_lib.DF11_GEMM_SEGMENT, parts=2), True, False), # BF16 y: one writer per element
    (64, dict(kernel=_lib.DF11_GEMM_WIDE, split=2), True, False),
    (3, dict(kernel=_lib.DF11_GEMM_VECTOR), False, False),          # the vector kernel takes 1 or 2 rows
    (1, dict(kernel=_lib.DF11_GEMM_VECTOR), False, True),           # and no w_debug
    (2, dict(kernel=_lib.DF11_GEMM_VECTOR, parts=2), True, False),  # BF16 y: one writer per element
    (8, dict(kernel=7), False, False),                              # no such kernel
    (129, dict(kernel=_lib.DF11_GEMM_RING), False, False),          # the exponent ring takes up to 128 rows
    (65, dict(kernel=_lib.DF11_GEMM_RING, k_slices=2), False, False),  # two k-slices up to 64 rows
    (8, dict(kernel=_lib.DF11_GEMM_RING, k_slices=3), False, False),
    (8, dict(kernel=_lib.DF11_GEMM_PIPE, k_slices=2), False, False),   # k_slices only on the exponent ring
    (8, dict(kernel=_lib.DF11_GEMM_PIPE, parts=2), False, False),   # parts without the segment kernels
    (64, dict(kernel=_lib.DF11_GEMM_PIPE, split=2), True, False),   # BF16 y: one writer per element
    (64, dict(kernel=_lib.DF11_GEMM_PIPE, split=2, one_writer=1), False, False),
    (64, dict(kernel=_lib.DF11_GEMM_PIPE, tiles_per_wave=3), False, False),   # 1 or 2 batch tiles per wave
    (64, dict(kernel=_lib.DF11_GEMM_WIDE, tiles_per_wave=2), False, False),   # only on the pipelined kernel
    (64, dict(tiles_per_wave=1), False, False),
    (8, dict(kernel=_lib.DF11_GEMM_SEGMENT, parts=2, one_writer=1), False, False),  # one writer: parts 1
    (64, dict(kernel=_lib.DF11_GEMM_WIDE, split=2, one_writer=1), False, False),    # and split 1
])
def test_fused_refuses_choices_that_do_not_apply(B, tune, bf16, wd):
    N, K = 64, 1024
    e = api.encode(synth.normal_bf16(N * K, 0.02, seed=2).reshape(N, K), layout=api.gemm_layout(N, K))
    rc, msg = _gemm_call(e.view, B, api.gemm_tuning(**tune), _lib.DF11_Y_BF16 if bf16 else _lib.DF11_Y_F32, wd)
    assert rc == -1, msg


def test_encoders_write_only_layouts_the_decoders_read():
    u = synth.normal_bf16(10_000, 0.02, seed=3)
    for cb in (4, 12, 20, 24, 32):
        with pytest.raises(_lib.DF11Error) as ei:
            api.encode(u, layout=api.make_layout(chunk_bytes=cb))
        assert ei.value.status == -1
    for cb in (8, 16):
        assert api.encode(u, layout=api.make_layout(chunk_bytes=cb)).view.chunk_bytes == cb


def test_offload_group_refuses_mixed_codebooks():
    """A compressed-offload group decodes every matrix through the first
    matrix's device tables, so matrices encoded with other codebooks are
    refused (before any pinned or device memory is allocated); matrices
    that share a codebook, or carry equal tables, are accepted up to that
    point."""
    from huffman_decode_df11_amd.offload import OffloadedModel, _same_tables
    a = synth.normal_bf16(50_000, 0.02, seed=4)
    b = synth.normal_bf16(50_000, 0.05, seed=5)
    ea, eb = api.encode(a), api.encode(b)
    with pytest.raises(ValueError, match="codebook"):
        OffloadedModel([("layer0", [("a", ea), ("b", eb)])], device="cpu")
    assert _same_tables(ea.codebook, api.encode(a).codebook)     # rebuilt from the same histogram
    assert not _same_tables(ea.codebook, eb.codebook)


def test_fused_workspace_size_and_refusals():
    """The packed-x workspace: none up to 32 rows of x, 32 T rows of x
    ((K / 16) x T kilobytes) for T = 2, 4, 8 batch tiles above; a call with a workspace that is
    too small or not 256-byte aligned is refused before any GPU work."""
    N, K = 64, 1024
    e = api.encode(synth.normal_bf16(N * K, 0.02, seed=5).reshape(N, K), layout=api.gemm_layout(N, K))
    L = _lib.lib()
    size = lambda B: int(L.df11_decode_gemm_workspace_bytes(ctypes.byref(e.view), B))
    assert [size(B) for B in (1, 32, 33, 64, 65, 128, 129, 256)] == \
        [0, 0] + [K // 16 * T * 1024 for T in (2, 2, 4, 4, 8, 8)]
    assert int(L.df11_decode_gemm_workspace_bytes(ctypes.byref(api.encode(synth.normal_bf16(1000, 0.02)).view), 64)) == 0
    _x, x = _aligned(2 * 64 * K)
    _y, y = _aligned(4 * 64 * N)
    _w, w = _aligned(size(64) + 512)
    for ptr, nbytes in ((w, size(64) - 16), (w + 16, size(64))):
        rc = L.df11_decode_gemm_ex(ctypes.byref(e.view), x, 64, y, _lib.DF11_Y_F32, None, None, ptr, nbytes, None)
        assert rc == -1, L.df11_last_error()
