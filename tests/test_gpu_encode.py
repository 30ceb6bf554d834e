"""GPU encoder (df11_hist_device, df11_encode_device) against the host
encoder, byte for byte, on every layout and workload; the host encoder is
itself checked against the oracle (test_host_library.py), and decoding the
device encoding must give the input back."""
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import _lib, api, synth
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(u):
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).cuda().view(torch.bfloat16)


def _same(h, d):
    for name in ("exp_words", "sm", "gaps", "counts", "segs", "chain", "fast", "block_seg"):
        a, b = h.arrays[name], d.arrays[name]
        assert a.size == b.size, name
        bad = np.nonzero(a != b)[0]
        assert bad.size == 0, "%s differs at byte %d" % (name, bad[0])
    for f in ("n", "total_bits", "n_segments", "max_seg_elems", "min_len", "max_len", "n_tables", "fast_bits",
              "row_win_lo", "row_win_span"):
        assert getattr(h.view, f) == getattr(d.view, f), f


WORKLOADS = {
    "normal": lambda: synth.normal_bf16(1_000_003, 0.02, seed=50),
    "adversarial": lambda: synth.adversarial_bf16(300_000, seed=51),
    "fibonacci": lambda: synth.fibonacci_bf16(seed=52),
    "exhaustive": lambda: synth.exhaustive_bf16(),
    "one": lambda: np.array([0x3F80], np.uint16),
    "ragged": lambda: synth.normal_bf16(4097, 0.02, seed=53),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("lay", ["default", "chunk8", "chunk32", "aligned"])
def test_device_encoder_matches_host(name, lay):
    u = WORKLOADS[name]()
    _say("case encode_device %s %s n=%d" % (name, lay, u.size))
    layout = {"default": None, "chunk8": api.make_layout(chunk_bytes=8),
              "chunk32": api.make_layout(chunk_bytes=32), "aligned": api.make_layout(align_elems=4112)}[lay]
    cb = api.build_codebook(api.hist_accumulate(u))
    if lay == "chunk32":
        # the decoders read 8- and 16-byte chunks only: both encoders refuse others
        for f in (lambda: api.encode(u, codebook=cb, layout=layout),
                  lambda: api.encode_device(_dev(u), codebook=cb, layout=layout)):
            with pytest.raises(_lib.DF11Error) as ei:
                f()
            assert ei.value.status == -1
        return
    h = api.encode(u, codebook=cb, layout=layout)
    d = api.encode_device(_dev(u), codebook=cb, layout=layout)
    _same(h, d.to_host())
    d.to_host().validate()


@pytest.mark.parametrize("kc", [0, 8])
def test_device_encoder_tile_orders(kc):
    rows, cols = 96, 1536
    _say("case encode_device tiles kc=%d" % kc)
    u = synth.normal_bf16(rows * cols, 0.02, seed=54).reshape(rows, cols)
    layout = (api.gemm_layout(rows, cols) if kc else
              api.make_layout(rows=rows, cols=cols, tile_rows=32, tile_cols=512, align_elems=32 * 512))
    cb = api.build_codebook(api.hist_accumulate(u))
    _same(api.encode(u, codebook=cb, layout=layout), api.encode_device(_dev(u), codebook=cb, layout=layout).to_host())


def test_device_histogram_and_default_codebook():
    u = synth.adversarial_bf16(2_000_000, seed=55)
    _say("case hist_device")
    assert np.array_equal(api.hist_device(_dev(u)), orc.histogram(u))
    d = api.encode_device(_dev(u))          # codebook from the device histogram
    out = api.decode(d)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), u)


def test_device_encode_full_size_up_proj_decodes():
    N, K = 14336, 4096
    _say("case encode_device up_proj")
    w = synth.normal_bf16_torch(N, K, seed=5, index=1, device="cuda")
    d = api.encode_device(w, layout=api.gemm_layout(N, K))
    x = torch.randn(8, K, device="cuda").to(torch.bfloat16)
    dbg = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    api.decode_gemm(d, x, w_debug=dbg)
    out = api.decode(d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16).reshape(N, K), w.view(torch.int16))
    assert torch.equal(dbg.view(torch.int16), w.view(torch.int16))


def test_device_encode_errors():
    u = synth.normal_bf16(1000, 0.02, seed=56)
    cb = api.build_codebook(api.hist_accumulate(u))
    v = u.copy()
    v[3] = 0x7F80                      # an exponent the codebook has no code for
    with pytest.raises(_lib.DF11Error) as ei:
        api.encode_device(_dev(v), codebook=cb)
    assert ei.value.status == -2
    with pytest.raises(_lib.DF11Error) as ei:
        api.encode_device(_dev(u), codebook=cb, layout=api.make_layout(align_elems=10))
    assert ei.value.status == -1
    e = api.encode_device(_dev(np.zeros(0, np.uint16)), codebook=cb)
    assert e.n == 0 and e.n_segments == 0


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("lay", ["default", "chunk8", "aligned"])
def test_device_encoder_matches_oracle(name, lay):
    """The GPU encoder against the oracle directly (not through the host
    encoder): stream bytes, sign+mantissa bytes, gaps, code counts and
    segment records on the same inputs and code lengths, including the
    exhaustive 65,536-pattern tensor and the Fibonacci histogram whose
    32-bit length limit binds."""
    u = WORKLOADS[name]()
    _say("case encode_device vs oracle %s %s n=%d" % (name, lay, u.size))
    kw = {"default": {}, "chunk8": dict(chunk_bytes=8), "aligned": dict(align_elems=4112)}[lay]
    d = api.encode_device(_dev(u), layout=api.make_layout(**kw)).to_host()
    ln = api.codebook_lengths(d.codebook)
    ref = orc.encode(u, lengths=ln, chunk_bytes=kw.get("chunk_bytes", 16), seg_lanes=64,
                     align_elems=kw.get("align_elems", 0))
    assert d.total_bits == ref.total_bits
    assert np.array_equal(d.stream_bytes_msb_first(), ref.E)
    assert np.array_equal(d.sm[:d.n], ref.sm)
    assert d.n_segments == ref.n_segments
    assert np.array_equal(d.gaps, ref.gaps)
    assert np.array_equal(d.counts, ref.counts)
    assert np.array_equal(d.seg_elem, ref.seg_elem)
    assert np.array_equal(d.seg_nbits[:-1], ref.seg_nbits)
    # and the code itself is optimal for the tensor's histogram (oracle cost)
    hist = orc.histogram(u)
    cost = lambda lens: int(sum(int(h) * int(l) for h, l in zip(hist, lens)))
    assert cost(ln) == cost(orc.code_lengths(hist, 32))


@pytest.mark.parametrize("chunk", [8, 16])
def test_device_encoder_row_window(chunk):
    """A row-major table with rows and cols set: the GPU encoder records the
    same row window (row_win_lo, row_win_span) as the host encoder, with
    every other array byte-identical."""
    rows, cols = 4096, 4096
    _say("case encode_device row window chunk %d" % chunk)
    u = synth.normal_bf16(rows * cols, 0.02, seed=57).reshape(rows, cols)
    layout = api.make_layout(rows=rows, cols=cols, chunk_bytes=chunk)
    cb = api.build_codebook(api.hist_accumulate(u))
    h = api.encode(u, codebook=cb, layout=layout)
    d = api.encode_device(_dev(u.reshape(-1)), codebook=cb, layout=layout)
    assert h.view.row_win_span > 0
    _same(h, d.to_host())
    assert (d.view.row_win_lo, d.view.row_win_span) == (h.view.row_win_lo, h.view.row_win_span)
