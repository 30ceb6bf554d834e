"""GPU checks of df11_decode_rows and of the DF11Linear / DF11Embedding
modules.  Expected values: the input weights themselves (the oracle's
encode/decode round trip is the identity), torch's own products of the same
BF16 values, and the oracle's float64 product."""
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import api, synth
from oracle import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from huffman_decode_df11_amd import nn as dnn   # noqa: E402


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _i16(u):
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).cuda()


@pytest.mark.parametrize("chunk", [16, 8])
@pytest.mark.parametrize("rows,cols", [(1000, 4096), (333, 24), (64, 40000), (4096, 4096)])
def test_decode_rows_matches_input(rows, cols, chunk):
    """Random ids with repeats, the first and last rows; rows spanning one,
    several and a fraction of a segment (one, two and four waves per row),
    and a table of ~5300 segments (three steps of the 64-way segment
    search); 16- and 8-byte chunks."""
    _say("case decode_rows %dx%d chunk %d" % (rows, cols, chunk))
    W = synth.normal_bf16(rows * cols, 0.02, seed=30).reshape(rows, cols)
    dt = api.encode(W, layout=api.make_layout(rows=rows, cols=cols, chunk_bytes=chunk)).to("cuda")
    ids = np.concatenate([[0, rows - 1, rows - 1], np.random.default_rng(31).integers(0, rows, 200)])
    out = api.decode_rows(dt, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), _i16(W[ids]))


@pytest.mark.parametrize("zeros_first", [True, False])
def test_decode_rows_uneven_segments(zeros_first):
    """Half the table all-zero rows (1-bit codes, ~8K elements per segment)
    and half random 16-bit patterns (long codes, ~1K per segment): the
    interpolated segment guess misses by hundreds of segments, below the
    probed window in one order and above it in the other, so the lookup
    falls back to the 64-way search.  Every row is looked up."""
    rows, cols = 2048, 4096
    _say("case decode_rows uneven zeros_first=%s" % zeros_first)
    rnd = synth.adversarial_bf16(rows // 2 * cols, seed=39).reshape(rows // 2, cols)
    zer = np.zeros_like(rnd)
    W = np.ascontiguousarray(np.concatenate([zer, rnd] if zeros_first else [rnd, zer]))
    dt = api.encode(W, layout=api.make_layout(rows=rows, cols=cols)).to("cuda")
    ids = np.concatenate([np.arange(rows), np.random.default_rng(40).integers(0, rows, 300)])
    out = api.decode_rows(dt, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), _i16(W[ids]))


def test_decode_rows_adversarial_and_bad_ids():
    rows, cols = 512, 1024
    _say("case decode_rows adversarial")
    W = synth.adversarial_bf16(rows * cols, seed=32).reshape(rows, cols)
    dt = api.encode(W, layout=api.make_layout(rows=rows, cols=cols)).to("cuda")
    ids = torch.tensor([5, -1, rows, 7, 10 ** 12], dtype=torch.int64, device="cuda")
    out = torch.full((5, cols), 0x5555, dtype=torch.int16, device="cuda")
    api.decode_rows(dt, ids, out=out.view(torch.bfloat16))
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(o[0], W[5]) and np.array_equal(o[3], W[7])
    for k in (1, 2, 4):   # out-of-range ids: rows left as they were
        assert (o[k] == 0x5555).all()


@pytest.mark.parametrize("chunk", [8, 16])
def test_decode_rows_window_and_search_agree(chunk):
    """A few ids take the window mode (every segment of the row's recorded
    window loaded with no search before it); the same view with its window
    field cleared takes the segment search.  Both give the rows bit for bit,
    including the first and last rows of the table."""
    rows, cols = 4096, 4096
    _say("case decode_rows window/search chunk %d" % chunk)
    W = synth.normal_bf16(rows * cols, 0.02, seed=41).reshape(rows, cols)
    dt = api.encode(W, layout=api.make_layout(rows=rows, cols=cols, chunk_bytes=chunk)).to("cuda")
    assert 0 < dt.view.row_win_span <= 16
    ids = torch.from_numpy(np.array([0, rows - 1, 1, 2047, 3000, 17, 17], np.int64)).cuda()
    got_win = api.decode_rows(dt, ids)
    span = dt.view.row_win_span
    dt.view.row_win_span = 0
    try:
        got_search = api.decode_rows(dt, ids)
    finally:
        dt.view.row_win_span = span
    torch.cuda.synchronize()
    want = _i16(W[ids.cpu().numpy()])
    assert torch.equal(got_win.view(torch.int16), want)
    assert torch.equal(got_search.view(torch.int16), want)


def test_decode_rows_rejects_tile_order():
    from huffman_decode_df11_amd import _lib
    W = synth.normal_bf16(64 * 512, 0.02, seed=33).reshape(64, 512)
    dt = api.encode(W, layout=api.gemm_layout(64, 512)).to("cuda")
    with pytest.raises(_lib.DF11Error):
        api.decode_rows(dt, torch.zeros(3, dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("B", [1, 7, 64, 300])
def test_linear_fused_and_decode_modes(B):
    N, K = 256, 1024
    _say("case DF11Linear B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=34).reshape(N, K)
    X = synth.activations_bf16(B, K, seed=35)
    bias = torch.from_numpy(synth.normal_bf16(N, 0.1, seed=36).view(np.int16)).cuda().view(torch.bfloat16)
    x = _i16(X).view(torch.bfloat16).reshape(B, K)
    w = _i16(W).view(torch.bfloat16)
    ref = (x.float() @ w.float().t() + bias.float())
    for mode in ("fused", "decode"):
        lin = dnn.DF11Linear(W, bias=bias, mode=mode)
        y = lin(x)
        torch.cuda.synchronize()
        assert y.dtype == torch.bfloat16 and y.shape == (B, N)
        rel = float((y.float() - ref).norm() / ref.norm())
        assert rel < 8e-3, (mode, rel)          # BF16 output rounding dominates
        assert torch.equal(lin.decoded_weight().view(torch.int16), w.view(torch.int16))
    # without bias, against the oracle's float64 product (float32 output before rounding)
    lin = dnn.DF11Linear(W, mode="fused")
    if B <= 256:
        y32 = api.decode_gemm(lin.weight_df11, x)
        r64 = orc.gemm_f64(X.reshape(B, K), W)
        assert float(np.linalg.norm(y32.cpu().numpy() - r64) / np.linalg.norm(r64)) < 2e-3


@pytest.mark.parametrize("B", [1, 16, 100])
def test_linear_deterministic_mode(B):
    """DF11Linear(deterministic=True) on a q_proj-shaped weight (4096 x 4096,
    whose row blocks are otherwise split): the same output bits on every
    call, equal to torch's product of the same BF16 values within BF16
    output rounding."""
    N = K = 4096
    _say("case DF11Linear deterministic B=%d" % B)
    W = synth.normal_bf16(N * K, 0.02, seed=37).reshape(N, K)
    x = _i16(synth.activations_bf16(B, K, seed=38)).view(torch.bfloat16).reshape(B, K)
    lin = dnn.DF11Linear(W, mode="fused", deterministic=True)
    ys = [lin(x) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    ref = x.float() @ _i16(W).view(torch.bfloat16).float().t()
    assert float((ys[0].float() - ref).norm() / ref.norm()) < 8e-3


@torch.no_grad()
def test_linear_from_torch_and_3d_input():
    lin_t = torch.nn.Linear(512, 96, bias=True).to(torch.bfloat16).cuda()
    lin = dnn.DF11Linear.from_linear(lin_t)
    assert lin.mode == "fused"
    x = torch.randn(2, 5, 512, device="cuda").to(torch.bfloat16)
    y = lin(x)
    yt = lin_t(x)
    assert y.shape == (2, 5, 96)
    assert float((y.float() - yt.float()).norm() / yt.float().norm()) < 8e-3
    odd = dnn.DF11Linear(lin_t.weight[:, :300].contiguous(), mode="auto")   # 300 % 512 != 0
    assert odd.mode == "decode"
    assert torch.equal(odd(x[..., :300]).float(), (x[..., :300] @ lin_t.weight[:, :300].t()).float())


def test_embedding_lookup():
    V, D = 5000, 4096
    _say("case DF11Embedding")
    W = synth.normal_bf16(V * D, 0.02, seed=37).reshape(V, D)
    emb = dnn.DF11Embedding(W)
    ids = torch.from_numpy(np.random.default_rng(38).integers(0, V, (4, 33))).cuda()
    out = emb(ids)
    torch.cuda.synchronize()
    assert out.shape == (4, 33, D) and out.dtype == torch.bfloat16
    ref = torch.nn.functional.embedding(ids, _i16(W).view(torch.bfloat16))
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_llama_mlp_block_decode_mode_is_bit_identical():
    """A Llama-shaped MLP block, down(silu(gate(x)) * up(x)), with the three
    weights held compressed (DF11Linear, decode mode) gives exactly the
    output of the same block on the BF16 weights: the decode is lossless and
    the same matmuls run on the restored weights.  The fused mode (48 rows of
    x: the fused kernel) stays within the float32-accumulation tolerance."""
    torch.manual_seed(0)
    d, f = 1024, 3584
    gate = torch.nn.Linear(d, f, bias=False).cuda().to(torch.bfloat16)
    up = torch.nn.Linear(d, f, bias=False).cuda().to(torch.bfloat16)
    down = torch.nn.Linear(f, d, bias=False).cuda().to(torch.bfloat16)
    for lin in (gate, up, down):
        with torch.no_grad():
            lin.weight.normal_(0, 0.02)
    x = torch.randn(3, 16, d, device="cuda").to(torch.bfloat16)
    _say("case mlp block")

    def block(g, u, dn, x):
        return dn(torch.nn.functional.silu(g(x)) * u(x))

    with torch.no_grad():
        ref = block(gate, up, down, x)
        dec = [dnn.DF11Linear.from_linear(l, mode="decode") for l in (gate, up, down)]
        got = block(*dec, x)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        fused = [dnn.DF11Linear.from_linear(l, mode="fused") for l in (gate, up, down)]
        got_f = block(*fused, x)
        rel = float((got_f.float() - ref.float()).norm() / ref.float().norm())
        assert rel < 1e-2, rel
