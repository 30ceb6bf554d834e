"""GPU parity of df11_decode_gemm (fused decode + bf16 matrix cores) through
the C ABI: the decoded weights are bit-exact against the input (w_debug), and
y matches the oracle's float32 product within 2e-3 relative Frobenius error
(float32 accumulation differs only in summation order; BF16 products are
exact).  One or two rows of x take the vector kernel (dot products on the
vector ALU, no w_debug: its decode is checked through y with identity rows
of x, at full up_proj size).  Up to 40 rows of x take the segment-parallel kernel (one batch
tile of 32 rows up to 32, two above), which has no w_debug output: its
decode is checked bit-exactly through y with x = rows of the identity.
Above 40 rows (and for w_debug calls above 32) the wide kernel merges each
tile once into a BF16 plane in LDS, one row block per unit up to 112 rows
and two above (tuning.row_blocks forces either); up to 32 rows w_debug calls
take the tile-synchronous kernel.  Every case checks y of the call without w_debug
(the product path) as well as of the call with it."""
import ctypes
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import _lib, api, synth
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

TOL = 2e-3


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _x_to_gpu(X):
    return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda().view(torch.bfloat16)


def _run(W, X, with_debug=True, tuning=None):
    """y of the product call (no w_debug); with_debug: also the decoded
    weights and y of a second call that writes them.  Returns (y, wd, y_dbg)."""
    N, K = W.shape
    enc = api.encode(W, layout=api.gemm_layout(N, K))
    enc.validate()
    dt = enc.to("cuda")
    x = _x_to_gpu(X)
    y = torch.full((X.shape[0], N), float("nan"), dtype=torch.float32, device="cuda")
    api.decode_gemm(dt, x, out=y, tuning=tuning)
    wd = y_dbg = None
    if with_debug:
        wdbg = torch.full((N, K), 0x5555, dtype=torch.int16, device="cuda")
        yd = torch.full((X.shape[0], N), float("nan"), dtype=torch.float32, device="cuda")
        api.decode_gemm(dt, x, out=yd, w_debug=wdbg.view(torch.bfloat16), tuning=tuning)
        torch.cuda.synchronize()
        wd = wdbg.cpu().numpy().view(np.uint16)
        y_dbg = yd.cpu().numpy()
    torch.cuda.synchronize()
    return y.cpu().numpy(), wd, y_dbg


def _recover_by_identity(W, rows=32, counts=True, tuning=None):
    """W through y alone: x = rows of the identity placed at columns k0 ..
    k0 + rows - 1, for every k0, gives y[b, n] = W[n, k0 + b] exactly (one
    nonzero product per output).  counts=False drops the stored code counts
    (the kernel then runs the locate pass).  tuning: None, a tuning, or a
    function of the call's rows of x giving one.  Returns the recovered
    float32 W."""
    N, K = W.shape
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    if not counts:
        dt.view.counts = None
        dt.view.n_counts = 0
    got = np.empty((N, K), np.float32)
    for k0 in range(0, K, rows):
        b = min(rows, K - k0)
        X = np.zeros((b, K), np.uint16)
        X[np.arange(b), k0 + np.arange(b)] = 0x3F80
        y = api.decode_gemm(dt, _x_to_gpu(X), tuning=tuning(b) if callable(tuning) else tuning)
        got[:, k0:k0 + b] = y.cpu().numpy().T
    return got


def _legacy_tuning(rows):
    """The kernels that were the automatic choice before the ring kernels:
    segment-parallel up to 40 rows of x, wide above."""
    return api.gemm_tuning(kernel=_lib.DF11_GEMM_SEGMENT if rows <= 40 else _lib.DF11_GEMM_WIDE)


def _as_f32(W):
    return (W.astype(np.uint32) << 16).view(np.float32)


def _bf16_steps(a, b):
    """Distance in BF16 steps between two arrays of finite BF16 patterns."""
    def key(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def _rel(a, b):
    return float(np.linalg.norm(a.astype(np.float64) - b) / max(np.linalg.norm(b), 1e-30))


@pytest.mark.parametrize("B", [1, 3, 8, 31, 32, 33, 64, 100, 128, 200, 256])
def test_small_weight_all_batch_shapes(B):
    N, K = 96, 1536
    _say("case gemm small B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=20).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=21)
    y, wd, yd = _run(W, X)
    assert np.array_equal(wd, W), "decoded weights differ"
    ref = orc.gemm_f64(X, W)
    for got in (y, yd):
        assert np.isfinite(got).all()
        assert _rel(got, ref) < TOL
        assert _rel(got, orc.gemm_f32(X, W).astype(np.float64)) < TOL


@pytest.mark.parametrize("N,K,B", [(256, 14336, 5), (128, 4096, 40), (32, 512, 256), (128, 4096, 72),
                                   (64, 2048, 48)])
def test_k_split_shapes(N, K, B):
    """Few 32-row blocks: the K range is split across workgroups and the
    partial sums meet in y (28 tiles per row in 7 ranges of 4; 8 tiles in 8
    ranges; a single tile), through the automatic choice (the exponent ring
    up to 128 rows, the BF16 ring at 256) and, forced, the segment-parallel
    kernel (5 and 40 rows of x) and the wide one with 8, 4 and 2 batch tiles
    (256, 72 and 48 rows)."""
    _say("case gemm split N=%d K=%d B=%d" % (N, K, B))
    W = synth.normal_bf16(N * K, 0.02, seed=26).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=27)
    ref = orc.gemm_f64(X, W)
    for tune in (None, _legacy_tuning(B)):   # the segment-parallel kernel writes no w_debug
        y, wd, yd = _run(W, X, with_debug=tune is None or B > 40, tuning=tune)
        assert _rel(y, ref) < TOL
        if wd is not None:
            assert np.array_equal(wd, W), "decoded weights differ"
            assert _rel(yd, ref) < TOL


@pytest.mark.parametrize("rb", [1, 2])
@pytest.mark.parametrize("B", [64, 100, 256])
def test_wide_kernel_row_block_modes(B, rb):
    """The wide kernel with one and with two row blocks per unit, each
    forced (tuning.row_blocks) on a weight of three row blocks (so the last
    pair has one) and a weight split along K: decoded weights bit-exact, y
    within tolerance."""
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_WIDE, row_blocks=rb)
    for N, K, seed in ((96, 1536, 41), (64, 4096, 42)):
        _say("case gemm wide rb=%s B=%d N=%d K=%d" % (rb, B, N, K))
        W = synth.normal_bf16(N * K, 0.02, seed=seed).reshape(N, K)
        X = synth.activations_bf16(B, K, seed=seed + 1)
        y, wd, yd = _run(W, X, tuning=tune)
        assert np.array_equal(wd, W), "decoded weights differ"
        ref = orc.gemm_f64(X, W)
        assert _rel(y, ref) < TOL and _rel(yd, ref) < TOL


def test_identity_x_recovers_weights_exactly():
    # x = I: y[b, n] = W[n, b] exactly (one nonzero product per output)
    N, K, B = 64, 512, 256
    _say("case gemm identity")
    W = synth.normal_bf16(N * K, 0.02, seed=22).reshape(N, K)
    X = np.zeros((B, K), np.uint16)
    X[np.arange(B), np.arange(B)] = 0x3F80
    y, _, _ = _run(W, X, with_debug=False)
    assert np.array_equal(y, _as_f32(W)[:, :B].T)


@pytest.mark.parametrize("kernel", ["auto", "legacy"])
@pytest.mark.parametrize("rows", [32, 40, 48, 64])
@pytest.mark.parametrize("N,K,seed", [(96, 1536, 28), (256, 4096, 29)])
def test_identity_x_recovers_weights_segment_parallel(N, K, seed, rows, kernel):
    """Every weight through y alone, compared exactly: the automatic choice
    (the exponent ring, two k-slices per batch tile: their hand-over of
    partial sums) and, forced, the segment-parallel kernel at 32 and 40 rows
    of x (one batch tile, then two with the second a quarter full: masks at
    segment edges, rounds, the row block reduction per batch tile, the K
    split of y for the 8-row-block weight) and the wide kernel at 48 and 64
    rows (the merged BF16 plane, k-slice reduction)."""
    _say("case gemm identity %s N=%d K=%d rows=%d" % (kernel, N, K, rows))
    W = synth.normal_bf16(N * K, 0.02, seed=seed).reshape(N, K)
    tune = None if kernel == "auto" else _legacy_tuning   # per call: its rows of x
    assert np.array_equal(_recover_by_identity(W, rows=rows, tuning=tune), _as_f32(W))


def test_identity_x_recovers_long_code_weights():
    """Adversarial exponent mix (long codes, short segments) without the
    non-finite exponent 255, so that 0 * w stays 0: recovered exactly
    through y of the automatic choice and of the segment-parallel kernel."""
    N, K = 64, 1024
    _say("case gemm identity adversarial")
    W = synth.adversarial_bf16(N * K, seed=30).reshape(N, K)
    W = np.where((W >> 7) & 0xFF == 0xFF, W & 0x807F, W).astype(np.uint16)
    assert np.array_equal(_recover_by_identity(W), _as_f32(W))
    assert np.array_equal(_recover_by_identity(W, rows=64), _as_f32(W))
    assert np.array_equal(_recover_by_identity(W, tuning=_legacy_tuning), _as_f32(W))


def test_adversarial_weights_decode_exactly():
    # all exponents incl. Inf/NaN: w_debug must be bit-exact (y is not checked)
    N, K = 64, 1024
    _say("case gemm adversarial")
    W = synth.adversarial_bf16(N * K, seed=23).reshape(N, K)
    _, wd, _ = _run(W, synth.activations_bf16(4, K, seed=24))
    assert np.array_equal(wd, W)


@pytest.mark.parametrize("B", [1, 8, 64, 256])
def test_up_proj_full_size(B):
    """Wup 14336 x 4096, the fused workload: decoded weights compared in full
    on the GPU, y against the oracle on 48 sampled output features."""
    N, K = 14336, 4096
    _say("case gemm up_proj B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=0, index=5, count=7).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=1)
    enc = api.encode(W, layout=api.gemm_layout(N, K))
    dt = enc.to("cuda")
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = api.decode_gemm(dt, _x_to_gpu(X))
    yd = api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg)
    torch.cuda.synchronize()
    wt = torch.from_numpy(W.view(np.int16)).cuda()
    assert torch.equal(wdbg.view(torch.int16), wt), "decoded weights differ"
    cols = np.random.default_rng(B).choice(N, size=48, replace=False)
    ref = orc.gemm_f64(X, W[cols])
    # and the whole product against torch's float32 matmul of the same BF16 values
    yt = (_x_to_gpu(X).float() @ wt.view(torch.bfloat16).float().T)
    for out in (y, yd):
        assert _rel(out.cpu().numpy()[:, cols], ref) < TOL
        rel = float((out - yt).norm() / yt.norm())
        assert rel < TOL
    # BF16 y: the same float32 sums (448 row blocks fill the device, so both
    # calls write every element from one workgroup) rounded once
    y16 = api.decode_gemm(dt, _x_to_gpu(X), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, orc.round_bf16(y.cpu().numpy()))


@pytest.mark.parametrize("B", [1, 40, 64, 256])
def test_down_proj_full_size(B):
    """Wdown 4096 x 14336 (28 tiles per 32-row block, 128 row blocks, so the
    work of a row block is split across workgroups and y is accumulated):
    decoded weights compared in full, y against the oracle on 48 sampled
    output features and against torch's float32 matmul of the BF16 values."""
    N, K = 4096, 14336
    _say("case gemm down_proj B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=0, index=6, count=7).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=2)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = api.decode_gemm(dt, _x_to_gpu(X))
    yd = api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg)
    torch.cuda.synchronize()
    wt = torch.from_numpy(W.view(np.int16)).cuda()
    assert torch.equal(wdbg.view(torch.int16), wt), "decoded weights differ"
    cols = np.random.default_rng(B + 7).choice(N, size=48, replace=False)
    ref = orc.gemm_f64(X, W[cols])
    yt = (_x_to_gpu(X).float() @ wt.view(torch.bfloat16).float().T)
    for out in (y, yd):
        assert _rel(out.cpu().numpy()[:, cols], ref) < TOL
        assert float((out - yt).norm() / yt.norm()) < TOL


@pytest.mark.parametrize("B", [1, 8, 32, 64, 256])
def test_bf16_output_within_one_step_of_oracle(B):
    """y as BF16 (one rounding of the float32 sum) against the oracle's
    float64 product rounded to BF16: at most one BF16 step apart (the sums
    differ only in order, which can move a value across a rounding
    midpoint), on both kernels."""
    N, K = 96, 1536
    _say("case gemm bf16 out B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=31).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=32)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    ref = orc.round_bf16(orc.gemm_f64(X, W).astype(np.float32))
    y16 = api.decode_gemm(dt, _x_to_gpu(X), out_dtype=torch.bfloat16)
    wd = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y16d = api.decode_gemm(dt, _x_to_gpu(X), out_dtype=torch.bfloat16, w_debug=wd)
    torch.cuda.synchronize()
    for out in (y16, y16d):
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert _bf16_steps(got, ref).max() <= 1


def test_rejects_unknown_output_type():
    from huffman_decode_df11_amd import _lib
    N, K = 64, 512
    W = synth.normal_bf16(N * K, 0.02, seed=33).reshape(N, K)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    x = _x_to_gpu(synth.activations_bf16(2, K))
    y = torch.empty((2, N), dtype=torch.float32, device="cuda")
    rc = _lib.lib().df11_decode_gemm_out(ctypes.byref(dt.view), x.data_ptr(), 2, y.data_ptr(), 7, None,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -1


def test_rejects_row_major_layout():
    from huffman_decode_df11_amd import _lib
    W = synth.normal_bf16(64 * 512, 0.02, seed=25).reshape(64, 512)
    dt = api.encode(W, layout=api.make_layout(rows=64, cols=512)).to("cuda")
    with pytest.raises(_lib.DF11Error) as ei:
        api.decode_gemm(dt, _x_to_gpu(synth.activations_bf16(2, 512)))
    assert ei.value.status == -1


def test_fused_locate_pass_without_stored_counts():
    N, K, B = 96, 1536, 17
    _say("case gemm locate pass")
    W = synth.adversarial_bf16(N * K, seed=66).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=67)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    dt.view.counts = None
    dt.view.n_counts = 0
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg)
    y = api.decode_gemm(dt, _x_to_gpu(X))
    torch.cuda.synchronize()
    assert np.array_equal(wdbg.view(torch.int16).cpu().numpy().view(np.uint16), W)
    # the segment-parallel kernel's locate pass, exactly through y with x =
    # identity rows (no non-finite weights, so that 0 * w stays 0)
    Wf = np.where((W >> 7) & 0xFF == 0xFF, W & 0x807F, W).astype(np.uint16)
    assert np.array_equal(_recover_by_identity(Wf, counts=False), _as_f32(Wf))


def test_graph_replays_match_eager():
    """The fused product captured in a HIP graph (float32 y with the row
    blocks split into several runs, so the capture holds the fill kernel and
    the atomic adds; and BF16 y), replayed five times with the program's own
    eager work and synchronisations between replays; every replay equals the
    eager call."""
    N, K, B = 256, 4096, 8
    _say("case gemm graph replay")
    W = synth.normal_bf16(N * K, 0.02, seed=34).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=35)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    x = _x_to_gpu(X)
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    y16 = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        api.decode_gemm(dt, x, out=y)
        api.decode_gemm(dt, x, out=y16)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref32, ref16 = y.clone(), y16.clone()
    ref = orc.gemm_f64(X, W)
    assert _rel(ref32.cpu().numpy(), ref) < TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.decode_gemm(dt, x, out=y)
        api.decode_gemm(dt, x, out=y16)
    for i in range(5):
        y.fill_(float("nan"))
        y16.fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # float32 partial sums meet in y through atomics: their order may vary
        assert _rel(y.cpu().numpy(), ref) < TOL, i
        assert torch.allclose(y, ref32, rtol=1e-5, atol=1e-6), i
        assert torch.equal(y16.view(torch.int16), ref16.view(torch.int16)), i
        del junk


def _identity_recover_on_gpu(dt, N, K, rows, tuning=None):
    """W [N, K] as float32 through y alone, on the GPU: x = `rows` rows of
    the identity placed at columns k0 .. k0 + rows - 1, for every k0, gives
    y[b, n] = W[n, k0 + b] exactly (one nonzero product per output)."""
    got = torch.empty((K, N), dtype=torch.float32, device="cuda")
    for k0 in range(0, K, rows):
        b = min(rows, K - k0)
        X = torch.zeros((b, K), dtype=torch.int16, device="cuda")
        X[torch.arange(b), k0 + torch.arange(b)] = 0x3F80
        got[k0:k0 + b] = api.decode_gemm(dt, X.view(torch.bfloat16), tuning=tuning)
    torch.cuda.synchronize()
    return got.T


@pytest.mark.parametrize("kernel", ["auto", "segment"])
@pytest.mark.parametrize("rows", [32, 40])
def test_identity_x_recovers_up_proj_on_product_path(rows, kernel):
    """Wup 14336 x 4096 through the call the product path makes (no tuning:
    the exponent ring with two k-slices per batch tile), and through the
    segment-parallel kernel forced (its 448 row blocks fill the device's
    workgroup slots once, so each row block is one run and every wave walks
    about five segments, its accumulator carried from one to the next).
    x = 32 identity rows per call (one batch tile), or 40 (two batch tiles;
    the last call 16 rows, one tile): every one of the 58,720,256 weights
    comes back through y and is compared bit for bit."""
    N, K = 14336, 4096
    _say("case gemm identity up_proj product path rows=%d %s" % (rows, kernel))
    W = synth.normal_bf16(N * K, 0.02, seed=0, index=5, count=7).reshape(N, K)
    assert ((W & 0x7FFF) != 0).all()    # no zeros: 1 * w + 0 keeps every bit
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    got = _identity_recover_on_gpu(dt, N, K, rows,
                                   tuning=None if kernel == "auto" else api.gemm_tuning(kernel=_lib.DF11_GEMM_SEGMENT))
    want = (torch.from_numpy(W.view(np.int16)).cuda().to(torch.int32) << 16)
    bad = int((got.contiguous().view(torch.int32) != want).sum())
    assert bad == 0, "%d of %d weights differ" % (bad, N * K)


@pytest.mark.parametrize("B", [1, 33])
@pytest.mark.parametrize("kind", ["zero", "sparse95"])
def test_sparse_weights_take_a_kernel_whose_staging_fits(kind, B):
    """An all-zero weight (one exponent, 1-bit codes: 8,192 per segment) and
    a 95%-zero one (~7,300 per segment) make segments too large for the
    segment-parallel kernel's staging, whose LDS byte addresses must stay
    below 64 KB.  The call takes another kernel: decoded weights bit-exact,
    y equal to the oracle's (exactly zero for the all-zero weight)."""
    N, K = 64, 4096
    _say("case gemm sparse %s B=%d" % (kind, B))
    if kind == "zero":
        W = np.zeros((N, K), np.uint16)
    else:
        rng = np.random.default_rng(77)
        W = synth.normal_bf16(N * K, 0.02, seed=78).reshape(N, K)
        W[rng.random((N, K)) < 0.95] = 0
    enc = api.encode(W, layout=api.gemm_layout(N, K))
    assert enc.view.max_seg_elems > 7000
    X = synth.activations_bf16(B, K, seed=79)
    y, wd, yd = _run(W, X)
    assert np.array_equal(wd, W)
    ref = orc.gemm_f64(X, W)
    for got in (y, yd):
        if kind == "zero":
            assert (got == 0).all()
        else:
            assert _rel(got, ref) < TOL
    for code in (_lib.DF11_GEMM_SEGMENT, _lib.DF11_GEMM_VECTOR):
        if code == _lib.DF11_GEMM_VECTOR and B > 2:
            continue
        with pytest.raises(_lib.DF11Error) as ei:
            api.decode_gemm(enc.to("cuda"), _x_to_gpu(X), tuning=api.gemm_tuning(kernel=code))
        assert ei.value.status == -7


@pytest.mark.parametrize("kernel", ["auto", "tiled", "segment"])
def test_nonfinite_x_row(kernel):
    """A row of x holding +Inf: the other rows of y are as the oracle's
    product; that row of y is non-finite everywhere, as the oracle's is
    (+-Inf there: no weight in the Inf's column is zero), where the
    segment-parallel kernel may give NaN in place of +-Inf (it also
    multiplies neighbouring segments' weights, masked to +0, by that x).
    The automatic choice (the exponent ring) and the tile-synchronous kernel
    multiply whole decoded tiles: the signs of the plain product."""
    N, K, B = 96, 1536, 8
    _say("case gemm nonfinite x %s" % kernel)
    W = synth.normal_bf16(N * K, 0.02, seed=80).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=81)
    X[2, 700] = 0x7F80
    ref = orc.gemm_f64(X, W)
    assert np.isinf(ref[2]).all() and np.isfinite(np.delete(ref, 2, axis=0)).all()
    tune = {"auto": None, "tiled": api.gemm_tuning(kernel=_lib.DF11_GEMM_TILED),
            "segment": api.gemm_tuning(kernel=_lib.DF11_GEMM_SEGMENT)}[kernel]
    y, _, _ = _run(W, X, with_debug=False, tuning=tune)
    assert not np.isfinite(y[2]).any()
    assert _rel(np.delete(y, 2, axis=0), np.delete(ref, 2, axis=0)) < TOL
    if kernel != "segment":   # no masked neighbours: the signs of the plain product
        assert np.array_equal(y[2], ref[2])


@pytest.mark.parametrize("kernel,B,extra", [("segment", 8, dict(parts=2)), ("segment", 40, dict()),
                                            ("tiled", 8, dict(split=3)), ("wide", 64, dict(split=2)),
                                            ("wide", 100, dict(row_blocks=2)), ("vector", 1, dict()),
                                            ("vector", 2, dict()), ("vector", 2, dict(parts=3))])
def test_explicit_kernel_choices_agree(kernel, B, extra):
    """Every explicit kernel choice (tuning) gives the oracle's product."""
    N, K = 256, 4096
    _say("case gemm tuning %s B=%d %s" % (kernel, B, extra))
    W = synth.normal_bf16(N * K, 0.02, seed=82).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=83)
    code = {"segment": _lib.DF11_GEMM_SEGMENT, "tiled": _lib.DF11_GEMM_TILED, "wide": _lib.DF11_GEMM_WIDE,
            "vector": _lib.DF11_GEMM_VECTOR}[kernel]
    y, wd, yd = _run(W, X, with_debug=kernel not in ("segment", "vector"), tuning=api.gemm_tuning(kernel=code, **extra))
    ref = orc.gemm_f64(X, W)
    assert _rel(y, ref) < TOL
    if wd is not None:
        assert np.array_equal(wd, W) and _rel(yd, ref) < TOL


@pytest.mark.parametrize("B", [33, 40, 64, 65, 100, 128, 129, 200, 256])
def test_packed_x_workspace_and_in_place_x_agree(B):
    """Above 32 rows of x the product can read x packed in operand order
    from a workspace (filled first by a packing kernel; here a caller-owned
    buffer full of garbage, since every byte the product reads is written
    by the packing) or in place: both within tolerance of the oracle, the
    decoded weights bit-exact either way, on a weight split along K."""
    N, K = 96, 3072
    _say("case gemm packed x B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=84).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=85)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    x = _x_to_gpu(X)
    nb = api.gemm_workspace_bytes(dt, B)
    assert nb == K // 16 * (2 if B <= 64 else 4 if B <= 128 else 8) * 1024
    ws = torch.randint(0, 255, (nb + 256,), dtype=torch.uint8, device="cuda")
    ref = orc.gemm_f64(X, W)
    outs = []
    for workspace in (None, ws, "auto"):
        wd = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
        y = api.decode_gemm(dt, x, workspace=workspace)
        yd = api.decode_gemm(dt, x, workspace=workspace, w_debug=wd)
        torch.cuda.synchronize()
        assert np.array_equal(wd.view(torch.int16).cpu().numpy().view(np.uint16), W)
        for got in (y, yd):
            assert _rel(got.cpu().numpy(), ref) < TOL
        outs.append(y.cpu().numpy())
    assert _rel(outs[1], outs[0].astype(np.float64)) < 1e-5


@pytest.mark.parametrize("rows", [40, 64, 96])
def test_identity_x_recovers_up_proj_packed_x(rows):
    """Wup through y with x packed (the default above 32 rows): 40 rows of
    the identity per call (the exponent ring, two batch tiles of two
    k-slices each), 64 (two full batch tiles) and 96 (three batch tiles of
    one k-slice), every weight bit for bit."""
    N, K = 14336, 4096
    _say("case gemm identity up_proj packed rows=%d" % rows)
    W = synth.normal_bf16(N * K, 0.02, seed=0, index=5, count=7).reshape(N, K)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    got = _identity_recover_on_gpu(dt, N, K, rows)
    want = (torch.from_numpy(W.view(np.int16)).cuda().to(torch.int32) << 16)
    bad = int((got.contiguous().view(torch.int32) != want).sum())
    assert bad == 0, "%d of %d weights differ" % (bad, N * K)


@pytest.mark.parametrize("rows", [1, 2])
def test_identity_x_recovers_up_proj_vector_kernel(rows):
    """Wup 14336 x 4096 through the vector kernel (forced; the product path
    takes the exponent ring, covered at 32 and 40 rows above): x = identity
    rows, 4096 / rows calls, and every one of the 58,720,256 weights comes
    back through y bit for bit (one nonzero dot-product term per output,
    masked neighbours +0)."""
    N, K = 14336, 4096
    _say("case gemm identity up_proj vector kernel rows=%d" % rows)
    W = synth.normal_bf16(N * K, 0.02, seed=0, index=5, count=7).reshape(N, K)
    assert ((W & 0x7FFF) != 0).all()
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    got = _identity_recover_on_gpu(dt, N, K, rows, tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_VECTOR))
    want = (torch.from_numpy(W.view(np.int16)).cuda().to(torch.int32) << 16)
    bad = int((got.contiguous().view(torch.int32) != want).sum())
    assert bad == 0, "%d of %d weights differ" % (bad, N * K)


def test_vector_kernel_refuses_what_it_does_not_take():
    """The vector kernel takes one or two rows of x and no w_debug: an
    explicit request for more rows, or with w_debug, is an argument error."""
    N, K = 64, 1024
    W = synth.normal_bf16(N * K, 0.02, seed=84).reshape(N, K)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_VECTOR)
    with pytest.raises(_lib.DF11Error) as ei:
        api.decode_gemm(dt, _x_to_gpu(synth.activations_bf16(3, K, seed=85)), tuning=tune)
    assert ei.value.status == -1
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.DF11Error) as ei:
        api.decode_gemm(dt, _x_to_gpu(synth.activations_bf16(1, K, seed=85)), w_debug=wdbg, tuning=tune)
    assert ei.value.status == -1
    torch.cuda.synchronize()


def test_vector_kernel_nonfinite_x_row():
    """Two rows of x, the second holding +Inf: the first row of y is as the
    oracle's, the second non-finite everywhere (NaN where masked neighbours
    meet the Inf, as with the segment-parallel kernel)."""
    N, K = 96, 1536
    _say("case gemm vector nonfinite x")
    W = synth.normal_bf16(N * K, 0.02, seed=86).reshape(N, K)
    X = synth.activations_bf16(2, K, seed=87)
    X[1, 700] = 0x7F80
    ref = orc.gemm_f64(X, W)
    y, _, _ = _run(W, X, with_debug=False, tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_VECTOR))
    assert not np.isfinite(y[1]).any()
    assert _rel(y[:1], ref[:1]) < TOL


@pytest.mark.parametrize("B", [1, 8, 64, 200])
def test_one_writer_is_the_same_on_every_run(B):
    """A 4096 x 4096 weight has 128 row blocks, too few to fill the device:
    by default a row block's work is split (segment runs or K ranges) and
    float32 partial sums are added atomically.  With one_writer every
    element of y is summed by one workgroup in a fixed order: three calls
    give the same bits, within the oracle's tolerance."""
    N, K = 4096, 4096
    _say("case gemm one_writer B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=88).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=89)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    x = _x_to_gpu(X)
    tune = api.gemm_tuning(one_writer=1)
    ys = [api.decode_gemm(dt, x, tuning=tune) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int32), ys[0].view(torch.int32))
    assert _rel(ys[0].cpu().numpy(), orc.gemm_f64(X, W)) < TOL


# ---- pipelined kernel (DF11_GEMM_PIPE): decoder waves and matrix-core waves
# of one workgroup handing tiles over through a ring of BF16 planes in LDS

@pytest.mark.parametrize("N,K,B,extra", [(256, 4096, 1, dict()), (256, 4096, 8, dict()), (256, 4096, 33, dict()),
                                         (256, 4096, 64, dict(split=3)), (256, 4096, 100, dict(one_writer=1)),
                                         (256, 4096, 200, dict()), (256, 4096, 256, dict(one_writer=1)),
                                         (256, 4096, 160, dict(tiles_per_wave=1)),
                                         (256, 4096, 64, dict(tiles_per_wave=2)),
                                         (96, 1536, 17, dict()), (96, 1536, 250, dict(split=1))])
def test_pipelined_kernel_matches_oracle(N, K, B, extra):
    """Few row blocks (the K range of a row block split across workgroups,
    y added atomically, unless one_writer or split=1): decoded weights
    bit-exact through w_debug, y of both calls within the oracle's
    tolerance, and a BF16 y one rounding of the float32 one-writer sums."""
    _say("case gemm pipelined N=%d K=%d B=%d %s" % (N, K, B, extra))
    W = synth.normal_bf16(N * K, 0.02, seed=90).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=91)
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_PIPE, **extra)
    y, wd, yd = _run(W, X, tuning=tune)
    ref = orc.gemm_f64(X, W)
    assert np.array_equal(wd, W)
    assert _rel(y, ref) < TOL and _rel(yd, ref) < TOL
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    one = api.gemm_tuning(kernel=_lib.DF11_GEMM_PIPE, one_writer=1)
    y32 = api.decode_gemm(dt, _x_to_gpu(X), tuning=one)
    y16 = api.decode_gemm(dt, _x_to_gpu(X), out_dtype=torch.bfloat16, tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_PIPE))
    torch.cuda.synchronize()
    got16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, orc.round_bf16(y32.cpu().numpy()))


@pytest.mark.parametrize("B,tpw", [(33, 2), (96, 2), (160, 2), (230, 1), (256, 2)])
def test_pipelined_kernel_x_in_place(B, tpw):
    """x read in place (no workspace): rows past B, in the last batch tile
    and in a matrix-core wave's second tile beyond the rows of x, are
    clamped to row B - 1, and their sums are not stored.  y against the
    oracle; every element of a y prefilled with NaN written."""
    N, K = 128, 2048
    _say("case gemm pipelined x in place B=%d tiles_per_wave=%d" % (B, tpw))
    W = synth.normal_bf16(N * K, 0.02, seed=92).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=93)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    api.decode_gemm(dt, _x_to_gpu(X), out=y, workspace=None,
                    tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_PIPE, tiles_per_wave=tpw, one_writer=1))
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    assert _rel(got, orc.gemm_f64(X, W)) < TOL


@pytest.mark.parametrize("B", [1, 64, 256])
def test_pipelined_kernel_up_proj_full_size(B):
    """Wup 14336 x 4096 (448 row blocks: one workgroup sums each element of
    y): the decoded weights compared in full, y against the oracle on 48
    sampled output features and against torch's float32 matmul of the same
    BF16 values, and the same bits from a second call."""
    N, K = 14336, 4096
    _say("case gemm pipelined up_proj B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=0, index=5, count=7).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=1)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_PIPE)
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = api.decode_gemm(dt, _x_to_gpu(X), tuning=tune)
    y2 = api.decode_gemm(dt, _x_to_gpu(X), tuning=tune)
    yd = api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg, tuning=tune)
    torch.cuda.synchronize()
    wt = torch.from_numpy(W.view(np.int16)).cuda()
    assert torch.equal(wdbg.view(torch.int16), wt), "decoded weights differ"
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    cols = np.random.default_rng(B + 3).choice(N, size=48, replace=False)
    ref = orc.gemm_f64(X, W[cols])
    yt = (_x_to_gpu(X).float() @ wt.view(torch.bfloat16).float().T)
    for out in (y, yd):
        assert _rel(out.cpu().numpy()[:, cols], ref) < TOL
        assert float((out - yt).norm() / yt.norm()) < TOL


@pytest.mark.parametrize("B", [1, 64])
@pytest.mark.parametrize("kind", ["zero", "sparse95"])
def test_pipelined_kernel_long_segments(kind, B):
    """All-zero and 95%-zero weights: segments of 7,000-8,192 elements, more
    than the units a decoder wave loads ahead, so the rest of each segment
    is merged from bytes loaded during the merge.  Bit-exact weights, y as
    the oracle's (exactly zero for the all-zero weight)."""
    N, K = 64, 4096
    _say("case gemm pipelined long segments %s B=%d" % (kind, B))
    if kind == "zero":
        W = np.zeros((N, K), np.uint16)
    else:
        rng = np.random.default_rng(77)
        W = synth.normal_bf16(N * K, 0.02, seed=78).reshape(N, K)
        W[rng.random((N, K)) < 0.95] = 0
    assert api.encode(W, layout=api.gemm_layout(N, K)).view.max_seg_elems > 7000
    X = synth.activations_bf16(B, K, seed=79)
    y, wd, yd = _run(W, X, tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_PIPE))
    assert np.array_equal(wd, W)
    ref = orc.gemm_f64(X, W)
    for got in (y, yd):
        if kind == "zero":
            assert (got == 0).all()
        else:
            assert _rel(got, ref) < TOL


def test_pipelined_kernel_locate_pass_without_stored_counts():
    """No stored code counts: the decoder waves walk each chunk to count its
    codes first.  Adversarial weights (long codes through the hierarchical
    tables): decoded weights bit-exact, y as the oracle's."""
    N, K, B = 96, 1536, 40
    _say("case gemm pipelined locate pass")
    W = synth.adversarial_bf16(N * K, seed=66).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=67)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    dt.view.counts = None
    dt.view.n_counts = 0
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_PIPE)
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg, tuning=tune)
    torch.cuda.synchronize()
    assert np.array_equal(wdbg.view(torch.int16).cpu().numpy().view(np.uint16), W)
    ref = orc.gemm_f64(X, W)
    got = y.cpu().numpy()
    # output features with no Inf or NaN weight; of those, the ones whose
    # float32 sums stay finite (exponents up to 254 can overflow float32
    # partial sums where the float64 sum is finite)
    fin = np.isfinite(ref).all(axis=0)
    ok = fin & np.isfinite(got).all(axis=0)
    assert 0 < fin.sum() < N and ok.sum() >= fin.sum() - 8
    assert _rel(got[:, ok], ref[:, ok]) < TOL
    assert not np.isfinite(got[:, ~fin]).all(axis=0).any()


# ---- exponent-ring kernel (DF11_GEMM_RING): the pipelined hand-over with
# exponent-only planes, the sign+mantissa bytes merged by the matrix-core waves

@pytest.mark.parametrize("N,K,B,extra", [(256, 4096, 1, dict()), (256, 4096, 8, dict()), (256, 4096, 33, dict()),
                                         (256, 4096, 64, dict(split=3)), (256, 4096, 100, dict(one_writer=1)),
                                         (256, 4096, 128, dict()), (96, 1536, 17, dict()),
                                         (96, 1536, 120, dict(split=1)), (256, 4096, 33, dict(k_slices=1)),
                                         (256, 4096, 5, dict(k_slices=1, split=2)),
                                         (96, 1536, 64, dict(k_slices=2, one_writer=1))])
def test_ring_kernel_matches_oracle(N, K, B, extra):
    """Decoded weights bit-exact through w_debug, y of both calls within the
    oracle's tolerance, and a BF16 y one rounding of the float32 one-writer
    sums."""
    _say("case gemm ring N=%d K=%d B=%d %s" % (N, K, B, extra))
    W = synth.normal_bf16(N * K, 0.02, seed=94).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=95)
    y, wd, yd = _run(W, X, tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_RING, **extra))
    ref = orc.gemm_f64(X, W)
    assert np.array_equal(wd, W)
    assert _rel(y, ref) < TOL and _rel(yd, ref) < TOL
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    y32 = api.decode_gemm(dt, _x_to_gpu(X), tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_RING, one_writer=1))
    y16 = api.decode_gemm(dt, _x_to_gpu(X), out_dtype=torch.bfloat16, tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_RING))
    torch.cuda.synchronize()
    got16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, orc.round_bf16(y32.cpu().numpy()))


@pytest.mark.parametrize("B", [8, 64, 128])
def test_ring_kernel_up_proj_full_size(B):
    """Wup 14336 x 4096: the decoded weights compared in full, y against the
    oracle on 48 sampled output features and against torch's float32 matmul
    of the same BF16 values, and the same bits from a second call."""
    N, K = 14336, 4096
    _say("case gemm ring up_proj B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=0, index=5, count=7).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=1)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_RING)
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = api.decode_gemm(dt, _x_to_gpu(X), tuning=tune)
    y2 = api.decode_gemm(dt, _x_to_gpu(X), tuning=tune)
    yd = api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg, tuning=tune)
    torch.cuda.synchronize()
    wt = torch.from_numpy(W.view(np.int16)).cuda()
    assert torch.equal(wdbg.view(torch.int16), wt), "decoded weights differ"
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    cols = np.random.default_rng(B + 5).choice(N, size=48, replace=False)
    ref = orc.gemm_f64(X, W[cols])
    yt = (_x_to_gpu(X).float() @ wt.view(torch.bfloat16).float().T)
    for out in (y, yd):
        assert _rel(out.cpu().numpy()[:, cols], ref) < TOL
        assert float((out - yt).norm() / yt.norm()) < TOL


@pytest.mark.parametrize("B", [1, 64])
@pytest.mark.parametrize("kind", ["zero", "sparse95"])
def test_ring_kernel_long_segments(kind, B):
    """All-zero and 95%-zero weights (segments of 7,000-8,192 elements):
    bit-exact weights, y as the oracle's (exactly zero for the all-zero
    weight)."""
    N, K = 64, 4096
    _say("case gemm ring long segments %s B=%d" % (kind, B))
    if kind == "zero":
        W = np.zeros((N, K), np.uint16)
    else:
        rng = np.random.default_rng(97)
        W = synth.normal_bf16(N * K, 0.02, seed=98).reshape(N, K)
        W[rng.random((N, K)) < 0.95] = 0
    assert api.encode(W, layout=api.gemm_layout(N, K)).view.max_seg_elems > 7000
    X = synth.activations_bf16(B, K, seed=99)
    y, wd, yd = _run(W, X, tuning=api.gemm_tuning(kernel=_lib.DF11_GEMM_RING))
    assert np.array_equal(wd, W)
    ref = orc.gemm_f64(X, W)
    for got in (y, yd):
        if kind == "zero":
            assert (got == 0).all()
        else:
            assert _rel(got, ref) < TOL


@pytest.mark.parametrize("B", [5, 40])
def test_ring_kernel_locate_pass_and_x_in_place(B):
    """No stored code counts (the decoder waves walk each chunk first) on
    adversarial weights, and x read in place without a workspace: decoded
    weights bit-exact; y as the oracle's on the output features whose
    largest finite weight is below 2^100 (float32 sums of K products with
    |x| < 2^8 cannot overflow there), non-finite where the oracle's is."""
    N, K = 96, 1536
    _say("case gemm ring locate pass B=%d" % B)
    W = synth.adversarial_bf16(N * K, seed=68).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=69)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    dt.view.counts = None
    dt.view.n_counts = 0
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_RING)
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    y = api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg, tuning=tune, workspace=None)
    torch.cuda.synchronize()
    assert np.array_equal(wdbg.view(torch.int16).cpu().numpy().view(np.uint16), W)
    ref = orc.gemm_f64(X, W)
    got = y.cpu().numpy()
    fin = np.isfinite(ref).all(axis=0)
    def as_f32(u):   # BF16 bits -> value (signalling NaN patterns become quiet NaN)
        with np.errstate(invalid="ignore"):
            return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = as_f32(W)
    wmax = np.where(np.isfinite(wf), np.abs(wf), 0.0).max(axis=1)
    safe = fin & (wmax < 2.0 ** 100)
    assert np.abs(as_f32(X)).max() < 2.0 ** 8
    assert 0 < safe.sum() < N
    assert np.isfinite(got[:, safe]).all()
    assert _rel(got[:, safe], ref[:, safe]) < TOL
    assert not np.isfinite(got[:, ~fin]).all(axis=0).any()


@pytest.mark.parametrize("B,extra", [(8, dict(k_slices=2)), (64, dict(k_slices=2, one_writer=1)),
                                     (40, dict(k_slices=1)), (100, dict())])
def test_ring_kernel_many_row_blocks_per_workgroup(B, extra):
    """640 row blocks of one tile each, more than the resident workgroups,
    so each workgroup walks several row blocks and (two k-slices) hands
    partial sums over through the same LDS area again and again: decoded
    weights bit-exact, y against the oracle on 64 sampled output features,
    and every element of a NaN-prefilled y written."""
    N, K = 20480, 512
    _say("case gemm ring many row blocks B=%d %s" % (B, extra))
    W = synth.normal_bf16(N * K, 0.02, seed=101).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=102)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    tune = api.gemm_tuning(kernel=_lib.DF11_GEMM_RING, **extra)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    api.decode_gemm(dt, _x_to_gpu(X), out=y, tuning=tune)
    wdbg = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    yd = api.decode_gemm(dt, _x_to_gpu(X), w_debug=wdbg, tuning=tune)
    torch.cuda.synchronize()
    assert np.array_equal(wdbg.view(torch.int16).cpu().numpy().view(np.uint16), W)
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    cols = np.random.default_rng(B).choice(N, size=64, replace=False)
    ref = orc.gemm_f64(X, W[cols])
    assert _rel(got[:, cols], ref) < TOL and _rel(yd.cpu().numpy()[:, cols], ref) < TOL
