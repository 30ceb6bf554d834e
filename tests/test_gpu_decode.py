"""GPU parity of df11_decode against the oracle (bit-exact), through the C ABI.

The oracle's decode of its own encoding is the input itself (pinned by the
round-trip tests), so the expected output of every case is the oracle's
decode; for large inputs it is the input bits, which the oracle reproduces
exactly, checked on sampled segments."""
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import api, synth
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

SENTINELS = (0x5555, 0xAAAA)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _to_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def _decode_checked(dt, n, margin=64):
    """Decode twice into buffers pre-filled with two different sentinels and
    a guard margin: every element must be written (both runs agree) and no
    element past n may change."""
    outs = []
    for s in SENTINELS:
        buf = torch.full((n + margin,), s - 65536 if s >= 32768 else s, dtype=torch.int16, device="cuda")
        api.decode(dt, out=buf.view(torch.bfloat16))
        torch.cuda.synchronize()
        b = _to_bits(buf)
        assert (b[n:] == s).all(), "decode wrote past the end of the output"
        outs.append(b[:n])
    assert np.array_equal(outs[0], outs[1]), "some outputs were not written"
    return outs[0]


def _check(u, layout=None, fast_bits=11, max_len=32, oracle=True, tag=""):
    u = np.ascontiguousarray(u).reshape(-1)
    cb_bytes = layout.chunk_bytes if layout is not None and layout.chunk_bytes else 16
    _say("case", tag, "n=%d fast_bits=%d chunk=%d" % (u.size, fast_bits, cb_bytes))
    enc = api.encode(u, layout=layout, fast_bits=fast_bits, max_len=max_len)
    dt = enc.to("cuda")
    got = _decode_checked(dt, u.size)
    if oracle:
        ln = api.codebook_lengths(enc.codebook)
        ref = orc.encode(u, lengths=ln, chunk_bytes=cb_bytes, align_elems=layout.align_elems if layout else 0)
        assert np.array_equal(enc.stream_bytes_msb_first(), ref.E)
        assert np.array_equal(enc.counts, ref.counts) and np.array_equal(enc.gaps, ref.gaps)
        want = orc.decode(ref.E, ref.total_bits, ref.sm, ref.n, ln,
                          seg_bits=cb_bytes * 8 * 64, align_elems=layout.align_elems if layout else 0)
    else:
        want = u
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%d mismatches, first at %s: got %04x want %04x" % (
        bad.size, bad[:5], got[bad[0]], want[bad[0]])
    return enc


@pytest.mark.parametrize("fast_bits", [8, 9, 10, 11, 12])
def test_tensor_1024x1024(fast_bits):
    _check(synth.tensor_1024(seed=0), fast_bits=fast_bits, tag="1024x1024")


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 255, 1000, 4097, 65537, 1_000_003])
def test_ragged_sizes(n):
    _check(synth.normal_bf16(n, 0.02, seed=n), tag="ragged")


def test_exhaustive_all_patterns():
    _check(synth.exhaustive_bf16(), tag="exhaustive")


def test_adversarial_small():
    _check(synth.adversarial_bf16(1 << 20, seed=1), tag="adversarial-1M")


def test_adversarial_full_16m():
    u = synth.adversarial_bf16(1 << 24, seed=0)
    enc = _check(u, oracle=False, tag="adversarial-16M")
    _oracle_sampled(enc, u)


def test_fibonacci_32bit_codes():
    u = synth.fibonacci_bf16()
    enc = _check(u, oracle=False, tag="fibonacci")
    assert enc.codebook.max_len == 32     # the 32-bit limit binds (Huffman would need 33)


@pytest.mark.parametrize("lmax", [12, 16])
def test_length_limited(lmax):
    _check(synth.adversarial_bf16(1 << 20, seed=2), max_len=lmax, tag="lmax%d" % lmax)


def test_one_and_two_symbols():
    one = (np.full(100_003, 0x3F80, np.uint16) | (np.arange(100_003) % 256).astype(np.uint16)).astype(np.uint16)
    _check(one, tag="one-symbol")
    two = np.where(np.arange(77_777) % 5 == 0, 0xBF80, 0x4000).astype(np.uint16)
    _check(two, tag="two-symbols")


def test_aligned_layout():
    _check(synth.normal_bf16(500_000, 0.02, seed=3), layout=api.make_layout(align_elems=4096), tag="aligned")


@pytest.mark.parametrize("kc", [0, 8, 16])
def test_tile_order_decodes_row_major(kc):
    """Tile order with and without column groups: the decode writes row-major
    BF16, which must be the input (the oracle's encode/decode round trip is
    the identity); the stream itself equals the oracle's encoding of the
    oracle's permutation."""
    rows, cols = 128, 2048
    u = synth.normal_bf16(rows * cols, 0.02, seed=4).reshape(rows, cols)
    lay = api.make_layout(rows=rows, cols=cols, tile_rows=32, tile_cols=512, align_elems=32 * 512,
                          tile_kchunk=kc)
    _say("case tile order kc=%d" % kc)
    enc = api.encode(u, layout=lay)
    ref = orc.encode(orc.tile_order(u, rows, cols, 32, 512, kc), lengths=api.codebook_lengths(enc.codebook),
                     align_elems=32 * 512)
    assert np.array_equal(enc.stream_bytes_msb_first(), ref.E)
    got = _decode_checked(enc.to("cuda"), u.size)
    assert np.array_equal(got, u.reshape(-1))


def test_gemm_layout_decodes_row_major():
    rows, cols = 96, 1536
    u = synth.adversarial_bf16(rows * cols, seed=5).reshape(rows, cols)
    _say("case gemm layout plain decode")
    enc = api.encode(u, layout=api.gemm_layout(rows, cols))
    got = _decode_checked(enc.to("cuda"), u.size)
    assert np.array_equal(got, u.reshape(-1))


def test_empty():
    enc = api.encode(np.zeros(0, np.uint16))
    dt = enc.to("cuda")
    out = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    api.decode(dt, out=out)
    torch.cuda.synchronize()
    assert (_to_bits(out) == 0).all()


def _oracle_sampled(enc, u, nseg=24, seed=0):
    """The oracle decodes sampled segments of the library's stream on its own
    (bit-serial) and must reproduce the same elements."""
    ln = api.codebook_lengths(enc.codebook)
    stream = enc.stream_bytes_msb_first()
    rng = np.random.default_rng(seed)
    segs = rng.choice(enc.n_segments, size=min(nseg, enc.n_segments), replace=False)
    seg_bits = 16 * 8 * 64
    for s in segs:
        g0, g1 = int(enc.seg_elem[s]), int(enc.seg_elem[s + 1])
        if g1 == g0:
            continue
        # first code of segment s starts at s*seg_bits + gap of its first lane
        start = int(s) * seg_bits + int(enc.gaps[int(s) * 64])
        # the segment's codes, re-aligned so the first one starts at bit 0
        sub = np.zeros(seg_bits // 8 + 16, np.uint8)
        b0 = start // 8
        chunk = stream[b0:b0 + seg_bits // 8 + 8]
        sub[:chunk.size] = chunk
        bits = np.unpackbits(sub)[start - 8 * b0:]
        packed = np.packbits(bits)
        out = orc.decode(packed, bits.size, enc.sm[g0:g1], g1 - g0, ln)
        assert np.array_equal(out, u[g0:g1]), "segment %d" % s


def test_llama_layer_full_size_reused_buffer():
    """The seven Llama-3-8B-shaped matrices of one layer, one codebook for the
    layer, each decoded into one reused BF16 buffer."""
    mats = synth.llama_layer(seed=0, layer=0)
    hist = None
    for _, m in mats:
        hist = api.hist_accumulate(m, hist)
    cb = api.build_codebook(hist)
    biggest = max(m.size for _, m in mats)
    buf = torch.empty(biggest + 64, dtype=torch.int16, device="cuda")
    for name, m in mats:
        _say("case llama", name, m.shape)
        enc = api.encode(m, codebook=cb)
        dt = enc.to("cuda")
        buf.fill_(0x5555)
        api.decode(dt, out=buf.view(torch.bfloat16))
        torch.cuda.synchronize()
        got = _to_bits(buf)
        assert np.array_equal(got[:m.size], m.reshape(-1)), name
        assert (got[m.size:] == 0x5555).all()
        if name in ("up_proj", "k_proj"):
            _oracle_sampled(enc, m.reshape(-1), nseg=8)
        del dt, enc


def test_batch_llama_layer_one_launch():
    """All seven matrices of a layer in one launch, each into its own output."""
    mats = synth.llama_layer(seed=0, layer=1)
    hist = None
    for _, m in mats:
        hist = api.hist_accumulate(m, hist)
    cb = api.build_codebook(hist)
    dts = [api.encode(m, codebook=cb).to("cuda") for _, m in mats]
    _say("case batch llama layer")
    outs = [torch.full((m.size + 32,), 0x5555, dtype=torch.int16, device="cuda") for _, m in mats]
    api.decode_batch(dts, outs=[o.view(torch.bfloat16) for o in outs])
    torch.cuda.synchronize()
    for (name, m), o in zip(mats, outs):
        got = _to_bits(o)
        assert np.array_equal(got[:m.size], m.reshape(-1)), name
        assert (got[m.size:] == 0x5555).all(), name


def test_batch_streaming_launch_with_ragged_views():
    """A launch whose output exceeds the last-level cache takes the streaming
    (nontemporal) loads and stores: a 135M-element tensor and ragged small
    ones in one batch, each bit-exact with its neighbours untouched."""
    sizes = [1, 135_000_001, 17, 1_000_003]
    tensors = [synth.normal_bf16(n, 0.02, seed=300 + i) for i, n in enumerate(sizes)]
    hist = None
    for t in tensors:
        hist = api.hist_accumulate(t, hist)
    cb = api.build_codebook(hist)
    dts = [api.encode(t, codebook=cb).to("cuda") for t in tensors]
    assert 2 * sum(sizes) > 256 << 20
    _say("case batch streaming", sizes)
    outs = [torch.full((t.size + 16,), 0x5555, dtype=torch.int16, device="cuda") for t in tensors]
    api.decode_batch(dts, outs=[o.view(torch.bfloat16) for o in outs])
    torch.cuda.synchronize()
    for t, o in zip(tensors, outs):
        got = _to_bits(o)
        assert np.array_equal(got[:t.size], t)
        assert (got[t.size:] == 0x5555).all()


def test_streaming_launch_tile_order_output():
    """A weight in the fused kernel's tile order (8-column groups) whose BF16
    output exceeds the last-level cache, decoded to row-major by
    df11_decode: the streaming stores go through the tile-order placement."""
    rows, cols = 8224, 16384
    assert 2 * rows * cols > 256 << 20
    u = synth.normal_bf16(rows * cols, 0.02, seed=320).reshape(rows, cols)
    _say("case streaming tile order", rows, cols)
    dt = api.encode(u, layout=api.gemm_layout(rows, cols)).to("cuda")
    out = torch.full((rows * cols + 16,), 0x5555, dtype=torch.int16, device="cuda")
    api.decode(dt, out=out.view(torch.bfloat16))
    torch.cuda.synchronize()
    want = torch.from_numpy(u.reshape(-1).view(np.int16)).cuda()
    assert torch.equal(out[:rows * cols], want)
    assert (out[rows * cols:] == 0x5555).all()


def test_batch_many_small_and_empty():
    """More views than one launch takes (16), ragged sizes and an empty one."""
    rng = np.random.default_rng(7)
    sizes = [0, 1, 17, 4096, 100_000] + [int(x) for x in rng.integers(1, 300_000, size=17)]
    tensors = [synth.normal_bf16(n, 0.02, seed=100 + i) for i, n in enumerate(sizes)]
    hist = None
    for t in tensors:
        hist = api.hist_accumulate(t, hist)
    cb = api.build_codebook(hist)
    dts = [api.encode(t, codebook=cb).to("cuda") for t in tensors]
    _say("case batch small", len(dts))
    outs = [torch.full((max(t.size, 1) + 16,), 0x5555, dtype=torch.int16, device="cuda") for t in tensors]
    api.decode_batch(dts, outs=[o.view(torch.bfloat16) for o in outs])
    torch.cuda.synchronize()
    for t, o in zip(tensors, outs):
        got = _to_bits(o)
        assert np.array_equal(got[:t.size], t)
        assert (got[t.size:] == 0x5555).all()


def test_batch_rejects_different_codebooks():
    from huffman_decode_df11_amd import _lib
    a = api.encode(synth.normal_bf16(5000, 0.02, seed=1)).to("cuda")
    b = api.encode(synth.normal_bf16(5000, 0.03, seed=2)).to("cuda")
    with pytest.raises(_lib.DF11Error) as ei:
        api.decode_batch([a, b])
    assert ei.value.status == -1


@pytest.mark.parametrize("name", ["normal", "adversarial", "fibonacci"])
def test_locate_pass_without_stored_counts(name):
    """A view without chunk counts: the kernel finds each lane's codes with
    the locate pass; the output is the same bit-exact result."""
    u = {"normal": lambda: synth.normal_bf16(2_000_003, 0.02, seed=63),
         "adversarial": lambda: synth.adversarial_bf16(1_000_000, seed=64),
         "fibonacci": lambda: synth.fibonacci_bf16(seed=65)}[name]()
    _say("case locate pass", name)
    dt = api.encode(u).to("cuda")
    dt.view.counts = None
    dt.view.n_counts = 0
    got = _decode_checked(dt, u.size)
    assert np.array_equal(got, u)


def test_concurrent_streams():
    """Two streams decoding different tensors at the same time (different
    codebooks and sizes, 20 launches each, interleaved); every output
    bit-exact."""
    a = synth.normal_bf16(3_000_017, 0.02, seed=330)
    b = synth.adversarial_bf16(2_000_000, seed=331)
    da, db = api.encode(a).to("cuda"), api.encode(b).to("cuda")
    _say("case concurrent streams")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a = [torch.empty(a.size, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    outs_b = [torch.empty(b.size, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    for i in range(20):
        api.decode(da, out=outs_a[i % 4], stream=sa)
        api.decode(db, out=outs_b[i % 4], stream=sb)
    torch.cuda.synchronize()
    for o in outs_a:
        assert np.array_equal(_to_bits(o), a)
    for o in outs_b:
        assert np.array_equal(_to_bits(o), b)


def test_batch_mixed_layouts():
    """One launch over a weight in the fused kernel's tile order, a
    row-major tensor with a ragged size and a tile order with 16-column
    groups, sharing a codebook: the launch takes the kernel with the
    row-wise tile merge, which must still merge the other views in stream
    order; every output bit-exact, guards untouched."""
    gemm = synth.normal_bf16(256 * 2048, 0.02, seed=340).reshape(256, 2048)
    flat = synth.normal_bf16(1_000_003, 0.02, seed=341)
    kc16 = synth.normal_bf16(128 * 1024, 0.02, seed=342).reshape(128, 1024)
    hist = None
    for t in (gemm, flat, kc16):
        hist = api.hist_accumulate(t, hist)
    cb = api.build_codebook(hist)
    lay16 = api.make_layout(rows=128, cols=1024, tile_rows=32, tile_cols=512, align_elems=32 * 512, tile_kchunk=16)
    dts = [api.encode(gemm, codebook=cb, layout=api.gemm_layout(256, 2048)).to("cuda"),
           api.encode(flat, codebook=cb).to("cuda"),
           api.encode(kc16, codebook=cb, layout=lay16).to("cuda")]
    _say("case batch mixed layouts")
    srcs = (gemm, flat, kc16)
    outs = [torch.full((t.size + 16,), 0x5555, dtype=torch.int16, device="cuda") for t in srcs]
    api.decode_batch(dts, outs=[o.view(torch.bfloat16) for o in outs])
    torch.cuda.synchronize()
    for t, o in zip(srcs, outs):
        got = _to_bits(o)
        assert np.array_equal(got[:t.size], t.reshape(-1))
        assert (got[t.size:] == 0x5555).all()


# ------------------------------------------------------------ 8-byte chunks

C8 = dict(chunk_bytes=8)


@pytest.mark.parametrize("fast_bits", [8, 11, 12])
def test_chunk8_tensor_1024x1024(fast_bits):
    _check(synth.tensor_1024(seed=0), layout=api.make_layout(**C8), fast_bits=fast_bits, tag="chunk8 1024x1024")


@pytest.mark.parametrize("n", [1, 17, 1000, 65537, 1_000_003])
def test_chunk8_ragged_sizes(n):
    _check(synth.normal_bf16(n, 0.02, seed=n + 1), layout=api.make_layout(**C8), tag="chunk8 ragged")


@pytest.mark.parametrize("name", ["exhaustive", "adversarial", "fibonacci", "one", "aligned"])
def test_chunk8_workloads(name):
    u = {"exhaustive": synth.exhaustive_bf16,
         "adversarial": lambda: synth.adversarial_bf16(1 << 20, seed=6),
         "fibonacci": lambda: synth.fibonacci_bf16(seed=7),
         "one": lambda: (np.full(70_001, 0x3F80, np.uint16) | (np.arange(70_001) % 256)).astype(np.uint16),
         "aligned": lambda: synth.normal_bf16(300_000, 0.02, seed=8)}[name]()
    lay = api.make_layout(chunk_bytes=8, align_elems=2048 if name == "aligned" else 0)
    _check(u, layout=lay, tag="chunk8 " + name)


@pytest.mark.parametrize("kc", [0, 8])
def test_chunk8_tile_order_decodes_row_major(kc):
    rows, cols = 128, 2048
    u = synth.normal_bf16(rows * cols, 0.02, seed=9).reshape(rows, cols)
    lay = api.make_layout(chunk_bytes=8, rows=rows, cols=cols, tile_rows=32, tile_cols=512, align_elems=32 * 512,
                          tile_kchunk=kc)
    _say("case chunk8 tile order kc=%d" % kc)
    got = _decode_checked(api.encode(u, layout=lay).to("cuda"), u.size)
    assert np.array_equal(got, u.reshape(-1))


@pytest.mark.parametrize("name", ["normal", "fibonacci"])
def test_chunk8_locate_pass(name):
    u = {"normal": lambda: synth.normal_bf16(1_000_003, 0.02, seed=10),
         "fibonacci": lambda: synth.fibonacci_bf16(seed=11)}[name]()
    _say("case chunk8 locate pass", name)
    dt = api.encode(u, layout=api.make_layout(**C8)).to("cuda")
    dt.view.counts = None
    dt.view.n_counts = 0
    assert np.array_equal(_decode_checked(dt, u.size), u)


def test_chunk8_batch_and_mixed_chunk_sizes_refused():
    """A launch of 8-byte-chunk views decodes them all; views of different
    chunk sizes cannot share a launch."""
    from huffman_decode_df11_amd import _lib
    ts = [synth.normal_bf16(n, 0.02, seed=12 + n) for n in (5, 4_194_304, 77_777)]
    hist = None
    for t in ts:
        hist = api.hist_accumulate(t, hist)
    cb = api.build_codebook(hist)
    dts = [api.encode(t, codebook=cb, layout=api.make_layout(**C8)).to("cuda") for t in ts]
    _say("case chunk8 batch")
    outs = [torch.full((t.size + 16,), 0x5555, dtype=torch.int16, device="cuda") for t in ts]
    api.decode_batch(dts, outs=[o.view(torch.bfloat16) for o in outs])
    torch.cuda.synchronize()
    for t, o in zip(ts, outs):
        got = _to_bits(o)
        assert np.array_equal(got[:t.size], t) and (got[t.size:] == 0x5555).all()
    d16 = api.encode(ts[0], codebook=cb).to("cuda")
    with pytest.raises(_lib.DF11Error) as ei:
        api.decode_batch([dts[1], d16])
    assert ei.value.status == -1


# ------------------------------------------------------------ launch choices

@pytest.mark.parametrize("chunk", [16, 8])
def test_every_launch_choice_gives_the_same_output(chunk):
    """Explicit waves per workgroup and store kinds (tuning) on a Llama-sized
    k_proj and a ragged tensor in one launch: every choice bit-exact."""
    from huffman_decode_df11_amd import _lib
    ts = [synth.normal_bf16(1024 * 4096, 0.02, seed=20), synth.normal_bf16(300_001, 0.02, seed=21)]
    hist = api.hist_accumulate(ts[1], api.hist_accumulate(ts[0]))
    cb = api.build_codebook(hist)
    dts = [api.encode(t, codebook=cb, layout=api.make_layout(chunk_bytes=chunk)).to("cuda") for t in ts]
    for waves in (0, 4, 6, 8, 10, 12, 14, 16):
        for stores in (_lib.DF11_STORES_AUTO, _lib.DF11_STORES_CACHED, _lib.DF11_STORES_STREAMING):
            _say("case tuning chunk=%d waves=%d stores=%d" % (chunk, waves, stores))
            outs = [torch.full((t.size + 16,), 0x5555, dtype=torch.int16, device="cuda") for t in ts]
            api.decode_batch(dts, outs=[o.view(torch.bfloat16) for o in outs],
                             tuning=api.decode_tuning(waves=waves, stores=stores))
            torch.cuda.synchronize()
            for t, o in zip(ts, outs):
                got = _to_bits(o)
                assert np.array_equal(got[:t.size], t) and (got[t.size:] == 0x5555).all()
    with pytest.raises(_lib.DF11Error) as ei:
        api.decode_batch(dts, tuning=api.decode_tuning(waves=5))
    assert ei.value.status == -1


# ------------------------------------------------------------ corrupt streams

GUARD = 1024   # elements of guard band on either side of the output (16-byte aligned)


def _guarded_decode(dt, n, fill):
    buf = torch.full((n + 2 * GUARD,), fill, dtype=torch.int16, device="cuda")
    api.decode(dt, out=buf[GUARD:GUARD + n].view(torch.bfloat16))
    torch.cuda.synchronize()
    b = _to_bits(buf)
    return b[:GUARD], b[GUARD:GUARD + n], b[GUARD + n:]


@pytest.mark.parametrize("layout", ["row-major", "chunk8", "tile-order", "aligned", "no-counts"])
def test_corrupt_exponent_words_write_only_inside_the_output(layout):
    """Random bits flipped in the exponent words of the device copy (the
    other metadata intact): the decoded values are garbage, but every write
    stays inside out[0, n) -- the guard bands on both sides keep their
    sentinels -- and the call completes.  Without stored counts the locate
    pass reads the corrupt stream too (segments whose counts no longer add
    up to their records are skipped)."""
    rows, cols = 300, 2048
    u = synth.normal_bf16(rows * cols, 0.02, seed=90).reshape(rows, cols)
    lay = {"row-major": None, "chunk8": api.make_layout(chunk_bytes=8), "tile-order": api.gemm_layout(rows - 12, cols),
           "aligned": api.make_layout(align_elems=4096), "no-counts": None}[layout]
    if layout == "tile-order":
        u = u[:rows - 12]
    n = u.size
    dt = api.encode(u, layout=lay).to("cuda")
    if layout == "no-counts":
        dt.view.counts = None
        dt.view.n_counts = 0
    words = dt.tensors["exp_words"].view(torch.int32)
    gen = torch.Generator(device="cuda").manual_seed(91)
    for density in (0.01, 0.5):
        _say("case corrupt %s density %.2f" % (layout, density))
        flips = torch.randint(-2 ** 31, 2 ** 31 - 1, words.shape, generator=gen, device="cuda", dtype=torch.int32)
        keep = torch.rand(words.shape, generator=gen, device="cuda") >= density
        words ^= torch.where(keep, torch.zeros_like(flips), flips)
        for fill in (0x5555, -0x5556):
            lo, _, hi = _guarded_decode(dt, n, fill)
            s = fill & 0xFFFF
            assert (lo == s).all() and (hi == s).all(), "a write left out[0, n)"
