"""The C ABI on its own on the GPU: the example program built beside the
library copies an encoded weight to the device with plain HIP calls, decodes
it (bit-exact against its input, guard past the end untouched) and runs the
fused product with float32 and BF16 outputs against its own float64 sum."""
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def test_c_api_program_on_device():
    from huffman_decode_df11_amd import build as b
    print("case c-api program", flush=True)
    sys.stdout.flush()
    r = subprocess.run([b.C_API_CHECK], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("c-api ok:"), r.stdout
