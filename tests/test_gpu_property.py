"""GPU property tests (derandomized): the decode kernels restore random
small tensors bit for bit, through df11_decode for every value mix and
aligned-block layout, and through df11_decode_rows for random row shapes
and ids.  The value mixes are those of the host property test; expected
values are the inputs themselves (decode(encode(u)) is the identity)."""
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import api

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from test_property_encode import _values  # noqa: E402

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow])


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@SETTINGS
@given(kind=st.sampled_from(["normal", "specials", "few", "one", "uniform"]),
       n=st.integers(1, 200000), seed=st.integers(0, 2 ** 31 - 1), align=st.sampled_from([0, 512, 16384]),
       chunk=st.sampled_from([16, 8]))
def test_decode_random_tensors(kind, n, seed, align, chunk):
    print("case decode", kind, n, seed, align, chunk, flush=True)
    sys.stdout.flush()
    u = _values(kind, n, seed)
    dt = api.encode(u, layout=api.make_layout(align_elems=align, chunk_bytes=chunk)).to("cuda")
    out = torch.full((n + 8,), 0x5555, dtype=torch.int16, device="cuda")
    api.decode(dt, out=out.view(torch.bfloat16))
    torch.cuda.synchronize()
    got = _bits(out)
    assert np.array_equal(got[:n], u)
    assert (got[n:] == 0x5555).all()


@SETTINGS
@given(kind=st.sampled_from(["normal", "specials", "few", "uniform"]),
       rows=st.integers(1, 300), cols8=st.integers(1, 1200), seed=st.integers(0, 2 ** 31 - 1),
       chunk=st.sampled_from([16, 8]))
def test_decode_rows_random_shapes(kind, rows, cols8, seed, chunk):
    cols = 8 * cols8
    print("case rows", kind, rows, cols, seed, chunk, flush=True)
    sys.stdout.flush()
    u = _values(kind, rows * cols, seed).reshape(rows, cols)
    dt = api.encode(u, layout=api.make_layout(rows=rows, cols=cols, chunk_bytes=chunk)).to("cuda")
    ids = np.random.default_rng(seed).integers(0, rows, 50)
    ids[0], ids[-1] = 0, rows - 1
    out = api.decode_rows(dt, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out).reshape(ids.size, cols), u[ids])


@SETTINGS
@given(kind=st.sampled_from(["normal", "few", "specials"]), nb=st.integers(1, 8), kt=st.integers(1, 4),
       B=st.integers(1, 256), seed=st.integers(0, 2 ** 31 - 1))
def test_decode_gemm_random_shapes(kind, nb, kt, B, seed):
    """Random weights [32 nb, 512 kt] and batches of 1 to 256 rows, through
    whichever fused kernel the size picks (and the K split for few row
    blocks): the decoded weights (w_debug) are bit-exact, and y is within
    the float32-accumulation tolerance of the oracle's float64 product, both
    from the call with w_debug and from the product call."""
    from oracle import oracle as orc
    N, K = 32 * nb, 512 * kt
    print("case gemm", kind, N, K, B, seed, flush=True)
    sys.stdout.flush()
    W = _values(kind, N * K, seed).reshape(N, K)
    # keep |w| < 2^16 so that y stays finite and comparable (exponent 0, and
    # every exponent up to 143, still occur)
    W = np.where((W >> 7) & 0xFF > 0x8F, W & 0x807F | (0x8F << 7), W).astype(np.uint16)
    X = _values("normal", B * K, seed + 1).reshape(B, K)
    X = np.where((X >> 7) & 0xFF >= 0x86, X & 0x807F | 0x3F00, X).astype(np.uint16)   # |x| < 128
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    x = torch.from_numpy(X.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.full((N, K), 0x5555, dtype=torch.int16, device="cuda")
    y_dbg = api.decode_gemm(dt, x, w_debug=wd.view(torch.bfloat16))
    y = api.decode_gemm(dt, x)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(wd).reshape(N, K), W)
    ref = orc.gemm_f64(X, W)
    scale = max(float(np.linalg.norm(ref)), 1e-30)
    for got in (y, y_dbg):
        g = got.cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all()
        assert float(np.linalg.norm(g - ref)) / scale < 2e-3
