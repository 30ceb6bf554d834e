"""GPU check of the compressed CPU offload: groups streamed from pinned host
memory through two device slots and decoded; every decoded matrix is
compared with its input (the oracle's round trip is the identity)."""
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import api, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from huffman_decode_df11_amd.offload import OffloadedModel   # noqa: E402


def test_offload_three_groups_two_passes():
    print("case offload", flush=True)
    sys.stdout.flush()
    groups, inputs = [], {}
    for gi in range(3):
        mats = [(name, synth.normal_bf16(r * c // 16, 0.02, seed=40 + gi, index=i, count=7))
                for i, (name, r, c) in enumerate(synth.LLAMA3_8B_LAYER)]
        if gi == 1:   # one group with every exponent value
            mats[2] = (mats[2][0], synth.adversarial_bf16(mats[2][1].size, seed=44))
        hist = None
        for _, u in mats:
            hist = api.hist_accumulate(u, hist)
        cb = api.build_codebook(hist)
        groups.append(("g%d" % gi, [(name, api.encode(u, codebook=cb)) for name, u in mats]))
        for name, u in mats:
            inputs[("g%d" % gi, name)] = u
    m = OffloadedModel(groups)
    out = torch.empty(m.max_elements, dtype=torch.bfloat16, device="cuda")
    for p in range(2):
        got = {}
        m.decode_pass(out, on_matrix=lambda g, name, o: got.__setitem__((g, name), o.clone()))
        torch.cuda.synchronize()
        assert len(got) == 21
        for key, o in got.items():
            want = torch.from_numpy(inputs[key].view(np.int16)).cuda()
            assert torch.equal(o.view(torch.int16), want), (p, key)
