"""The wide configuration's packed weight copy (include/moe.h, moe_pack_wide):
the copy the library writes equals the header's layout restated in tests/spec.py,
bit for bit; and a layer run with the copy gives the same bits as the same layer
reading row-major weights, in every configuration (only the wide one reads the
copy), at ragged and split-tail loads."""
import numpy as np
import pytest
import torch

import oracle
import synth
from routing_aware_grouped_amd import layer as L
from tests import gpu_helpers as G
from tests import spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("E,H,I", [(3, 256, 384), (2, 384, 128), (5, 128, 640)])
def test_pack_layout(E, H, I):
    G.say(f"pack layout E={E} H={H} I={I}")
    rng = np.random.default_rng([E, H, I])
    w1 = rng.integers(0, 1 << 16, (E, I, H), dtype=np.uint16)
    w3 = rng.integers(0, 1 << 16, (E, I, H), dtype=np.uint16)
    w2 = rng.integers(0, 1 << 16, (E, H, I), dtype=np.uint16)
    p = L.moe_problem(8, H, I, E, 0, E, 2, synth.BF16, synth.BF16, 1)
    dev = [torch.from_numpy(a.view(np.int16)).cuda() for a in (w1, w3, w2)]
    out = torch.full((L.moe_pack_wide_bytes(p),), 0xAB, dtype=torch.uint8, device="cuda")
    L.moe_pack_wide(p, dev[0], dev[1], dev[2], out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, spec.pack_wide(w1, w3, w2))


@pytest.mark.parametrize("shape,B,alpha", [
    ("tiny_bf16", 700, 1.0), ("tiny_bf16", 37, 0.1), ("qwen3", 300, 1.0), ("mixtral", 5, 1.0)])
def test_packed_layer_equals_row_major(shape, B, alpha):
    G.say(f"packed vs row-major {shape} B={B} alpha={alpha}")
    wdev, whost = G.weights(shape)
    layer = synth.make_layer(shape, B, alpha, 0, weights=whost)
    ids, w = oracle.route_topk(layer.logits, layer.shape.top_k)
    for v in range(len(spec.MENU)):
        a = G.fetch(G.run(layer, variant=v, wdev=wdev, pack=True))
        b = G.fetch(G.run(layer, variant=v, wdev=wdev, pack=False))
        np.testing.assert_array_equal(a["Y"].view(np.uint32), b["Y"].view(np.uint32))
    G.check_y(layer, a, ids, w)


def test_packed_split_tail_equals_row_major():
    """The down phase's split tail (pieces and their fix-up) with the packed copy:
    Mixtral B = 2048, alpha = 1 (four pieces per tail tile on a 256-CU GPU)."""
    G.say("packed vs row-major mixtral B=2048 split tail")
    wdev, whost = G.weights("mixtral")
    layer = synth.make_layer("mixtral", 2048, 1.0, 0, weights=whost)
    a = G.fetch(G.run(layer, variant=spec.WIDE, wdev=wdev, pack=True))
    b = G.fetch(G.run(layer, variant=spec.WIDE, wdev=wdev, pack=False))
    np.testing.assert_array_equal(a["Y"].view(np.uint32), b["Y"].view(np.uint32))
    ids, w = oracle.route_topk(layer.logits, 2)
    toks = np.random.default_rng(11).choice(2048, 16, replace=False).astype(np.int32)
    G.check_y(layer, a, ids, w, toks)
