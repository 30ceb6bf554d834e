"""GPU checks of the whole-model decode driver and of HIP-graph replay.

The expected output of every decode is the generated input itself: the
oracle's encode/decode round trip is the identity (pinned in the oracle
tests), and the HIP path's bit-exactness against the oracle is checked in
test_gpu_decode.py; here every element the driver decodes is compared with
its input on the device."""
import sys

import numpy as np
import pytest

from huffman_decode_df11_amd import api, model, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("encoder", ["device", "host"])
def test_model_pass_two_layers_full_shapes(encoder):
    """Embedding, two full-size decoder layers and the head, encoded on the
    GPU or on host threads: every matrix of the pass decoded into the reused
    buffer and compared in full."""
    _say("case model pass 2 layers, %s encoder" % encoder)
    m = model.synthetic_llama3_8b(seed=3, device="cuda", layers=2, threads=4, encoder=encoder)
    assert len(m.matrices) == 2 * 7 + 2
    assert m.n_elements == 2 * 218103808 + 2 * 128256 * 4096
    assert model.verify_pass(m, seed=3) == m.n_elements
    # per-layer batched launches decode the same bits
    specs = synth.llama3_8b_tensors(2)
    idx = 0
    for gi, (g, mats) in enumerate(m.groups):
        outs = m.decode_group(gi)
        torch.cuda.synchronize()
        for (name, t), o in zip(mats, outs):
            _, _, r, c = specs[idx]
            want = synth.normal_bf16_torch(r, c, 3, idx, "cuda").view(torch.int16).reshape(-1)
            assert torch.equal(o.view(torch.int16), want), (g, name)
            idx += 1


def test_graph_replays_match_eager():
    """Seven per-matrix decodes captured as one graph, each into its own
    buffer: replayed three times with eager work (buffer wipes and an eager
    decode) and a synchronisation between replays; every replay must leave
    every output bit-exact."""
    _say("case graph replay")
    mats = [synth.normal_bf16(r * c // 16, 0.02, seed=9, index=i, count=7)
            for i, (_, r, c) in enumerate(synth.LLAMA3_8B_LAYER)]
    hist = None
    for u in mats:
        hist = api.hist_accumulate(u, hist)
    cb = api.build_codebook(hist)
    dts = [api.encode(u, codebook=cb).to("cuda") for u in mats]
    outs = [torch.empty(u.size, dtype=torch.bfloat16, device="cuda") for u in mats]
    want = [torch.from_numpy(u.view(np.int16)).cuda() for u in mats]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for dt, o in zip(dts, outs):
            api.decode(dt, out=o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for dt, o in zip(dts, outs):
            api.decode(dt, out=o)
    for rep in range(3):
        for o in outs:
            o.view(torch.int16).fill_(0x5555 if rep % 2 else -0x5556)
        api.decode(dts[1], out=outs[0][:dts[1].n])   # unrelated eager work on the same memory
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o.view(torch.int16), w), "replay %d, matrix %d" % (rep, i)
