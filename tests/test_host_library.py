"""CPU tests of libdf11's host half against the oracle: exported symbols, code
optimality, canonical codes, stream, sign+mantissa bytes, gaps, segment
records, both lookup tables, the validator and the error paths."""
import ctypes
import os
import re

import numpy as np
import pytest

from huffman_decode_df11_amd import _lib, api, synth
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cost(hist, lengths):
    return int(sum(int(h) * int(l) for h, l in zip(hist, lengths)))


def _kraft_units(lengths):
    return sum(1 << (32 - int(l)) for l in lengths if l)


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "df11.h")) as f:
        text = f.read()
    declared = set(re.findall(r"\b(df11_[a-z_0-9]+)\s*\(", text))
    assert declared, "no declarations found"
    L = ctypes.CDLL(_lib.LIB_PATH)
    missing = [s for s in sorted(declared) if not hasattr(L, s)]
    assert not missing, missing
    assert set(_lib.EXPORTS) == declared


WORKLOADS = {
    "normal": lambda: synth.normal_bf16(300_000, 0.02, seed=11),
    "adversarial": lambda: synth.adversarial_bf16(300_000, seed=12),
    "exhaustive": synth.exhaustive_bf16,
    "fibonacci": lambda: synth.fibonacci_bf16(),
    "one_symbol": lambda: np.full(5000, 0x3F80, np.uint16) | np.arange(5000, dtype=np.uint16) % 128,
    "two_symbols": lambda: np.where(np.arange(7001) % 3 == 0, 0x3F80, 0x4000).astype(np.uint16),
}


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_codebook_is_optimal_and_canonical(name):
    u = WORKLOADS[name]()
    h = api.hist_accumulate(u)
    assert np.array_equal(h, orc.histogram(u))
    cb = api.build_codebook(h, 32)
    ln = api.codebook_lengths(cb)
    want = orc.code_lengths(h, 32)
    assert _cost(h, ln) == _cost(h, want)            # optimal (lengths themselves may differ)
    assert ln.max() <= 32
    assert all((ln[s] > 0) == (h[s] > 0) for s in range(256))
    if (h > 0).sum() >= 2:
        assert _kraft_units(ln) == 1 << 32
    assert np.array_equal(api.codebook_codes(cb), orc.canonical_codes(ln))
    assert cb.max_len == ln.max() and cb.min_len == ln[ln > 0].min()


@pytest.mark.parametrize("lmax", [10, 12, 16, 20])
def test_codebook_length_limit_matches_package_merge(lmax):
    u = synth.adversarial_bf16(200_000, seed=13)
    h = api.hist_accumulate(u)
    cb = api.build_codebook(h, lmax)
    ln = api.codebook_lengths(cb)
    assert ln.max() <= lmax
    assert _cost(h, ln) == _cost(h, orc.code_lengths(h, lmax))


def _chain_walk(chain, window):
    t = 0
    for level in range(4):
        e = int(chain[t * 256 + ((window >> (24 - 8 * level)) & 0xFF)])
        if not e & 0x8000:
            return e & 0xFF, (e >> 8) & 0x3F
        t = e & 0x7FFF
    return None


@pytest.mark.parametrize("name", ["normal", "adversarial", "fibonacci", "exhaustive"])
def test_lookup_tables_against_oracle_codes(name):
    u = WORKLOADS[name]()
    enc = api.encode(u)
    ln = api.codebook_lengths(enc.codebook)
    codes = orc.canonical_codes(ln)
    chain = enc.chain
    rng = np.random.default_rng(5)
    # every code, with random suffixes, walks to its own exponent and length
    for s in range(256):
        if not ln[s]:
            continue
        L = int(ln[s])
        for suf in rng.integers(0, 1 << 32, size=4, dtype=np.uint64):
            win = ((int(codes[s]) << (32 - L)) | (int(suf) >> L)) & 0xFFFFFFFF
            assert _chain_walk(chain, win) == (s, L)
    # the multi-code table: greedy decode of the window with the oracle's codes
    K = enc.codebook.fast_bits
    byprefix = {(int(codes[s]), int(ln[s])): s for s in range(256) if ln[s]}
    fast = enc.fast.reshape(-1, 2)
    for idx in range(1 << K):
        bits = format(idx, "0%db" % K)
        pos, syms = 0, []
        while len(syms) < 4:
            hit = None
            for L in range(1, K - pos + 1):
                key = (int(bits[pos:pos + L], 2), L)
                if key in byprefix:
                    hit = (byprefix[key], L)
                    break
            if hit is None:
                break
            syms.append(hit[0])
            pos += hit[1]
        want_meta = ((len(syms) << 16) - pos) & 0xFFFFFFFF if syms else 0
        want_syms = 0
        for i, e in enumerate(syms):
            want_syms |= (((e >> 1) | (e << 7)) & 0xFF) << (8 * i)
        assert int(fast[idx, 1]) == want_meta, idx
        assert int(fast[idx, 0]) == want_syms, idx


LAYOUTS = {
    "default": dict(),
    "chunk8": dict(chunk_bytes=8),
    "aligned": dict(align_elems=4096),
    "chunk8_aligned": dict(chunk_bytes=8, align_elems=2048),
}


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("name", ["normal", "adversarial", "fibonacci", "two_symbols", "one_symbol"])
def test_encoder_matches_oracle(name, layout):
    u = WORKLOADS[name]()
    kw = LAYOUTS[layout]
    cb = api.build_codebook(api.hist_accumulate(u))
    if 8 * kw.get("chunk_bytes", 16) // max(1, cb.min_len) > 255:
        # a chunk could hold more codes than a count byte records
        with pytest.raises(_lib.DF11Error) as ei:
            api.encode(u, codebook=cb, layout=api.make_layout(**kw))
        assert ei.value.status == -1
        return
    enc = api.encode(u, codebook=cb, layout=api.make_layout(**kw))
    ln = api.codebook_lengths(enc.codebook)
    ref = orc.encode(u, lengths=ln, chunk_bytes=kw.get("chunk_bytes", 16), seg_lanes=64,
                     align_elems=kw.get("align_elems", 0))
    assert enc.total_bits == ref.total_bits
    assert np.array_equal(enc.stream_bytes_msb_first(), ref.E)
    assert np.array_equal(enc.sm[:enc.n], ref.sm) and not enc.sm[enc.n:].any()
    assert enc.n_segments == ref.n_segments
    assert np.array_equal(enc.gaps, ref.gaps)
    assert np.array_equal(enc.counts, ref.counts)
    assert np.array_equal(enc.seg_elem, ref.seg_elem)
    assert np.array_equal(enc.seg_nbits[:-1], ref.seg_nbits)
    enc.validate()
    # the oracle's bit-serial decoder reads the library's stream back
    out = orc.decode(enc.stream_bytes_msb_first(), enc.total_bits, enc.sm[:enc.n], enc.n, ln,
                     seg_bits=8 * 64 * kw.get("chunk_bytes", 16), align_elems=kw.get("align_elems", 0))
    assert np.array_equal(out, u)


@pytest.mark.parametrize("kc", [0, 8, 16, 24])
def test_encoder_tile_order_matches_oracle_permutation(kc):
    rows, cols, tr, tc = 64, 1536 if kc == 24 else 1024, 32, 768 if kc == 24 else 512
    u = synth.normal_bf16(rows * cols, 0.02, seed=14).reshape(rows, cols)
    lay = api.make_layout(rows=rows, cols=cols, tile_rows=tr, tile_cols=tc, align_elems=tr * tc,
                          tile_kchunk=kc)
    enc = api.encode(u, layout=lay)
    ln = api.codebook_lengths(enc.codebook)
    perm = orc.tile_order(u, rows, cols, tr, tc, kc)
    ref = orc.encode(perm, lengths=ln, align_elems=tr * tc)
    assert np.array_equal(enc.stream_bytes_msb_first(), ref.E)
    assert np.array_equal(enc.sm[:enc.n], ref.sm)
    assert np.array_equal(enc.gaps, ref.gaps)
    assert np.array_equal(enc.seg_elem, ref.seg_elem)
    enc.validate()


def test_gemm_layout_shape_rules():
    tr, tc = api.gemm_tile()
    lay = api.gemm_layout(14336, 4096)
    assert lay.tile_rows == tr and lay.tile_cols == tc and lay.align_elems == tr * tc
    assert lay.tile_kchunk == 8
    with pytest.raises(_lib.DF11Error):
        api.gemm_layout(14336 + 1, 4096)


def test_empty_tensor_encodes():
    enc = api.encode(np.zeros(0, np.uint16))
    assert enc.n == 0 and enc.n_segments == 0 and enc.total_bits == 0
    enc.validate()


# --------------------------------------------------------------- error paths

def test_uncoded_exponent_rejected():
    u = synth.normal_bf16(1000, 0.02, seed=15)
    cb = api.build_codebook(api.hist_accumulate(u))
    v = u.copy()
    v[7] = 0x7F80   # Inf: exponent 255 never occurred
    with pytest.raises(_lib.DF11Error) as ei:
        api.encode(v, codebook=cb)
    assert ei.value.status == -2


@pytest.mark.parametrize("max_len", [0, 33])
def test_bad_max_len_rejected(max_len):
    with pytest.raises(_lib.DF11Error) as ei:
        api.build_codebook(np.ones(256, np.uint64), max_len)
    assert ei.value.status == -3


def test_too_many_tables_rejected():
    # 9-bit limit over ~256 exponents: every 8-bit prefix would need its own table
    h = api.hist_accumulate(synth.adversarial_bf16(200_000, seed=13))
    with pytest.raises(_lib.DF11Error) as ei:
        api.build_codebook(h, 9)
    assert ei.value.status == -3


def test_max_len_too_small_rejected():
    with pytest.raises(_lib.DF11Error) as ei:
        api.build_codebook(np.ones(256, np.uint64), 7)    # 256 symbols need 8 bits
    assert ei.value.status == -3


@pytest.mark.parametrize("kw", [dict(chunk_bytes=6), dict(chunk_bytes=64), dict(chunk_bytes=4), dict(chunk_bytes=12),
                                dict(chunk_bytes=32), dict(align_elems=10),
                                dict(rows=3, cols=5), dict(rows=100, cols=100, tile_rows=3, tile_cols=16),
                                dict(tile_kchunk=8),
                                dict(rows=64, cols=160, tile_rows=32, tile_cols=32, tile_kchunk=12),
                                dict(rows=64, cols=160, tile_rows=32, tile_cols=32, tile_kchunk=24),
                                dict(rows=63, cols=160, tile_rows=7, tile_cols=32, tile_kchunk=8)])
def test_bad_layout_rejected(kw):
    # the column-group cases have matching sizes, so only tile_kchunk is wrong
    n = kw["rows"] * kw["cols"] if "tile_kchunk" in kw and "rows" in kw else 10_000
    u = synth.normal_bf16(n, 0.02, seed=16)
    with pytest.raises(_lib.DF11Error) as ei:
        api.encode(u, layout=api.make_layout(**kw))
    assert ei.value.status == -1


def _corrupt_and_validate(enc, mutate):
    mutate(enc)
    with pytest.raises(_lib.DF11Error) as ei:
        enc.validate()
    assert ei.value.status in (-4, -1)


@pytest.mark.parametrize("what", ["stream_bit", "gap", "count", "seg_elem", "seg_nbits", "chain", "fast",
                                  "codebook_len", "n_segments"])
def test_validator_catches_corruption(what):
    u = synth.normal_bf16(200_000, 0.02, seed=17)
    enc = api.encode(u)
    enc.validate()

    def mutate(e):
        if what == "stream_bit":
            w = e.exp_words
            w[w.size // 3] ^= 0x00400000
        elif what == "gap":
            g = e.gaps
            g[100] = (int(g[100]) + 3) % 32
        elif what == "count":
            c = e.counts
            c[70] += 1
        elif what == "seg_elem":
            e.seg_elem[5] += 1
        elif what == "seg_nbits":
            e.seg_nbits[e.n_segments - 1] -= 1
        elif what == "chain":
            e.chain[3] ^= 1
        elif what == "fast":
            e.fast[10] ^= 1
        elif what == "codebook_len":
            e.codebook.len[121] += 1
        elif what == "n_segments":
            e.view.n_segments -= 1
    _corrupt_and_validate(enc, mutate)


def test_arrays_keep_their_encoding_alive():
    """A typed array taken from a temporary encoding stays valid: the array
    holds a reference to the library-owned memory's owner."""
    import gc
    u = synth.normal_bf16(50_000, 0.02, seed=60)
    ref = api.encode(u).arrays["exp_words"].copy()
    arr = api.encode(u).arrays["exp_words"]      # the Encoded object is a temporary
    gc.collect()
    _ = [api.encode(synth.normal_bf16(50_000, 0.02, seed=61)) for _ in range(3)]   # reuse freed memory
    assert np.array_equal(arr, ref)


def test_validator_accepts_a_view_without_counts():
    """Counts are optional in a view: without them the decoder (and the
    validator) find each lane's codes by walking the chunk."""
    enc = api.encode(synth.normal_bf16(100_000, 0.02, seed=62))
    enc.view.counts = None
    enc.view.n_counts = 0
    enc.validate()


def test_c_api_program_host_half():
    """The C ABI without Python: the example program built beside the library
    builds a codebook, encodes (row-major and tile order) and validates,
    and rejects a null input with a status (its device half runs in the GPU
    tests)."""
    import subprocess
    from huffman_decode_df11_amd import build as b
    assert os.path.exists(b.C_API_CHECK), "build the library first"
    r = subprocess.run([b.C_API_CHECK, "--host-only"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("c-api ok (host only)")


@pytest.mark.parametrize("chunk,rows,cols,kind", [(8, 600, 512, "normal"), (16, 600, 512, "normal"),
                                                   (8, 97, 1032, "skewed"), (16, 1, 4096, "normal"),
                                                   (16, 3000, 8, "normal")])
def test_row_window_matches_oracle_segments(chunk, rows, cols, kind):
    """The row window of a row-major encoding (df11_view row_win_lo and
    row_win_span) against the oracle's segment offsets on the same code:
    with g(r) = floor(r * cols * (segments / n)) in float64, every segment
    that overlaps row r (from the one holding the row's first element to the
    one holding its last) lies in [g + lo, g + lo + span), and the window is
    the tightest such (both ends reached by some row).  "skewed" rows differ
    tenfold in scale, so segments hold very different element counts."""
    n = rows * cols
    if kind == "normal":
        u = synth.normal_bf16(n, 0.02, seed=60).reshape(rows, cols)
    else:
        u = synth.normal_bf16(n, 0.02, seed=61).reshape(rows, cols)
        u[: rows // 2] = synth.adversarial_bf16(cols * (rows // 2), seed=62).reshape(rows // 2, cols)
    enc = api.encode(u, layout=api.make_layout(rows=rows, cols=cols, chunk_bytes=chunk))
    ref = orc.encode(u, lengths=api.codebook_lengths(enc.codebook), chunk_bytes=chunk, seg_lanes=64)
    nseg = ref.n_segments
    assert enc.n_segments == nseg
    starts = np.asarray(ref.seg_elem[:nseg], np.int64)
    e0 = np.arange(rows, dtype=np.int64) * cols
    first = np.searchsorted(starts, e0, side="right") - 1
    last = np.searchsorted(starts, e0 + cols - 1, side="right") - 1
    g = np.floor(e0.astype(np.float64) * (float(nseg) / float(n))).astype(np.int64)
    lo, span = int(enc.view.row_win_lo), int(enc.view.row_win_span)
    assert lo == int((first - g).min())
    assert span == int((last - g).max()) - lo + 1
    assert (first >= g + lo).all() and (last < g + lo + span).all()


def test_row_window_absent_without_rows_or_in_tile_order():
    u = synth.normal_bf16(96 * 1536, 0.02, seed=63)
    for layout in (api.make_layout(), api.gemm_layout(96, 1536)):
        e = api.encode(u.reshape(96, 1536), layout=layout)
        assert e.view.row_win_lo == 0 and e.view.row_win_span == 0
