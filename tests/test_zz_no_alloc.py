"""df11_decode_gemm_noalloc (the fused product for callers that cannot
allocate: the packed x lives in the library's scratch array) through the C
ABI, against df11_decode_gemm_ex with a caller workspace: two calls in a
row, the second with a smaller weight and fewer rows of x (so it reuses,
and leaves stale, part of what the first wrote); decoded weights bit-exact,
y equal to the workspace call's and within tolerance of the oracle."""
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


def _rel(a, b):
    return float(np.linalg.norm(a.astype(np.float64) - b) / max(np.linalg.norm(b), 1e-30))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _call(fn, dt, x, B, N, K, workspace=None, debug=True):
    """y (and the decoded weights when debug) of one call; debug=False is
    the product path (the ring kernels, x packed above 32 rows), debug=True
    a w_debug call (the wide kernel above 32 rows)."""
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    wd = torch.full((N, K), 0x5555, dtype=torch.int16, device="cuda") if debug else None
    wd_ptr = wd.data_ptr() if debug else None
    L = _lib.lib()
    if fn == "noalloc":
        rc = L.df11_decode_gemm_noalloc(ctypes.byref(dt.view), x.data_ptr(), B, y.data_ptr(), _lib.DF11_Y_F32,
                                        wd_ptr, None, _stream())
    else:
        rc = L.df11_decode_gemm_ex(ctypes.byref(dt.view), x.data_ptr(), B, y.data_ptr(), _lib.DF11_Y_F32,
                                   wd_ptr, None, workspace.data_ptr(), workspace.numel(), _stream())
    assert rc == 0, L.df11_last_error()
    torch.cuda.synchronize()
    return y.cpu().numpy(), (wd.cpu().numpy().view(np.uint16) if debug else None)


def test_noalloc_matches_workspace_entry_point_twice():
    for (N, K, B, seed) in ((512, 8192, 256, 60), (96, 1536, 40, 61)):
        print("case noalloc N=%d K=%d B=%d" % (N, K, B), flush=True)
        sys.stdout.flush()
        W = synth.normal_bf16(N * K, 0.02, seed=seed).reshape(N, K)
        X = synth.activations_bf16(B, K, seed=seed + 1)
        dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
        x = torch.from_numpy(X.view(np.int16)).cuda()
        ws = torch.empty(api.gemm_workspace_bytes(dt, B), dtype=torch.uint8, device="cuda")
        y_ws, wd_ws = _call("ex", dt, x, B, N, K, ws)
        y_na, wd_na = _call("noalloc", dt, x, B, N, K)
        assert np.array_equal(wd_na, W) and np.array_equal(wd_ws, W)
        ref = orc.gemm_f64(X, W)
        assert _rel(y_na, ref) < TOL and _rel(y_ws, ref) < TOL
        assert _rel(y_na, y_ws.astype(np.float64)) < 1e-5
        # the product path: the ring kernels read the packed x from the scratch
        p_ws, _ = _call("ex", dt, x, B, N, K, ws, debug=False)
        p_na, _ = _call("noalloc", dt, x, B, N, K, debug=False)
        assert _rel(p_na, ref) < TOL and _rel(p_ws, ref) < TOL
        assert _rel(p_na, p_ws.astype(np.float64)) < 1e-5


def test_noalloc_refuses_packed_x_beyond_its_scratch():
    N, K, B = 32, 33280, 256     # 2080 k-steps x 8 batch tiles x 1 KiB > 16 MiB
    W = synth.normal_bf16(N * K, 0.02, seed=62).reshape(N, K)
    dt = api.encode(W, layout=api.gemm_layout(N, K)).to("cuda")
    assert api.gemm_workspace_bytes(dt, B) > 16 << 20
    x = torch.zeros((B, K), dtype=torch.int16, device="cuda")
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    L = _lib.lib()
    rc = L.df11_decode_gemm_noalloc(ctypes.byref(dt.view), x.data_ptr(), B, y.data_ptr(), _lib.DF11_Y_F32, None,
                                    None, _stream())
    assert rc == -7 and b"scratch" in L.df11_last_error()
