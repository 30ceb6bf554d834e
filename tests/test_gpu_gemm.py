"""GPU parity of df11_decode_gemm (fused decode + bf16 matrix cores) through
the C ABI: the decoded weights are bit-exact against the input (w_debug), and
y matches the oracle's float32 product within 2e-3 relative Frobenius error
(float32 accumulation differs only in summation order; BF16 products are
exact).  Up to 40 rows of x take the segment-parallel kernel (one batch
tile of 32 rows up to 32, two above), which has no w_debug output: its
decode is checked bit-exactly through y with x = rows of the identity.
Above 40 rows (and for w_debug calls above 32) the wide kernel merges each
tile once into a BF16 plane in LDS, one row block per unit up to 112 rows
and two above (DF11_GEMM_RB forces either); up to 32 rows w_debug calls
take the tile-synchronous kernel.  Every case checks y of the call without w_debug
(the product path) as well as of the call with it."""
import ctypes
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import api, synth
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


def _run(W, X, with_debug=True):
    """y of the product call (no w_debug); with_debug: also the decoded
    weights and y of a second call that writes them.  Returns (y, wd, y_dbg)."""
    N, K = W.shape
    enc = api.encode(W, layout=api.gemm_layout(N, K))
    enc.validate()
    dt = enc.to("cuda")
    x = _x_to_gpu(X)
    y = torch.full((X.shape[0], N), float("nan"), dtype=torch.float32, device="cuda")
    api.decode_gemm(dt, x, out=y)
    wd = y_dbg = None
    if with_debug:
        wdbg = torch.full((N, K), 0x5555, dtype=torch.int16, device="cuda")
        yd = torch.full((X.shape[0], N), float("nan"), dtype=torch.float32, device="cuda")
        api.decode_gemm(dt, x, out=yd, w_debug=wdbg.view(torch.bfloat16))
        torch.cuda.synchronize()
        wd = wdbg.cpu().numpy().view(np.uint16)
        y_dbg = yd.cpu().numpy()
    torch.cuda.synchronize()
    return y.cpu().numpy(), wd, y_dbg


def _recover_by_identity(W, rows=32, counts=True):
    """W through y alone: x = rows of the identity placed at columns k0 ..
    k0 + rows - 1, for every k0, gives y[b, n] = W[n, k0 + b] exactly (one
    nonzero product per output).  counts=False drops the stored code counts
    (the kernel then runs the locate pass).  Returns the recovered float32 W."""
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
        y = api.decode_gemm(dt, _x_to_gpu(X))
        got[:, k0:k0 + b] = y.cpu().numpy().T
    return got


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
    ranges; a single tile), through the segment-parallel kernel (5 and 40
    rows of x) and the wide one with 8, 4 and 2 batch tiles (256, 72 and 48
    rows)."""
    _say("case gemm split N=%d K=%d B=%d" % (N, K, B))
    W = synth.normal_bf16(N * K, 0.02, seed=26).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=27)
    y, wd, yd = _run(W, X)
    assert np.array_equal(wd, W), "decoded weights differ"
    assert _rel(y, orc.gemm_f64(X, W)) < TOL
    assert _rel(yd, orc.gemm_f64(X, W)) < TOL


@pytest.mark.parametrize("rb", ["1", "2"])
@pytest.mark.parametrize("B", [64, 100, 256])
def test_wide_kernel_row_block_modes(B, rb, monkeypatch):
    """The wide kernel with one and with two row blocks per unit, each
    forced (DF11_GEMM_RB) on a weight of three row blocks (so the last pair
    has one) and a weight split along K: decoded weights bit-exact, y
    within tolerance."""
    monkeypatch.setenv("DF11_GEMM_RB", rb)
    for N, K, seed in ((96, 1536, 41), (64, 4096, 42)):
        _say("case gemm wide rb=%s B=%d N=%d K=%d" % (rb, B, N, K))
        W = synth.normal_bf16(N * K, 0.02, seed=seed).reshape(N, K)
        X = synth.activations_bf16(B, K, seed=seed + 1)
        y, wd, yd = _run(W, X)
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


@pytest.mark.parametrize("rows", [32, 40, 48, 64])
@pytest.mark.parametrize("N,K,seed", [(96, 1536, 28), (256, 4096, 29)])
def test_identity_x_recovers_weights_segment_parallel(N, K, seed, rows):
    """Every weight through y alone, compared exactly: the segment-parallel
    kernel at 32 and 40 rows of x (one batch tile, then two with the second
    a quarter full: masks at segment edges, rounds, the row block reduction
    per batch tile, the K split of y for the 8-row-block weight) and the
    wide kernel at 48 and 64 rows (the merged BF16 plane, k-slice
    reduction)."""
    _say("case gemm identity segment-parallel N=%d K=%d rows=%d" % (N, K, rows))
    W = synth.normal_bf16(N * K, 0.02, seed=seed).reshape(N, K)
    assert np.array_equal(_recover_by_identity(W, rows=rows), _as_f32(W))


def test_identity_x_recovers_long_code_weights():
    """Adversarial exponent mix (long codes, short segments) without the
    non-finite exponent 255, so that 0 * w stays 0: recovered exactly
    through y of the segment-parallel kernel."""
    N, K = 64, 1024
    _say("case gemm identity adversarial")
    W = synth.adversarial_bf16(N * K, seed=30).reshape(N, K)
    W = np.where((W >> 7) & 0xFF == 0xFF, W & 0x807F, W).astype(np.uint16)
    assert np.array_equal(_recover_by_identity(W), _as_f32(W))
    assert np.array_equal(_recover_by_identity(W, rows=64), _as_f32(W))


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
