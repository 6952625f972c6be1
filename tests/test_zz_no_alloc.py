"""moe_grouped_ffn_noalloc, the grouped FFN for callers that cannot allocate: it
works in the library's own per-GPU array instead of a caller workspace.  Checked
through the C ABI against moe_grouped_ffn with a caller workspace on the same
inputs, bit for bit (the same kernels run), on two calls in a row with the second
smaller than the first, in every configuration, with bf16 weights, with fp8
weights on the FP8 activation path (codes and scales in the array too), and on a
load whose last round of tiles is split (partial sums in the array)."""
import numpy as np
import pytest
import torch

import synth
from routing_aware_grouped_amd import layer as L
from routing_aware_grouped_amd import moe_grouped_ffn_noalloc
from tests import gpu_helpers as G
from tests import spec

pytestmark = pytest.mark.gpu
V = len(spec.MENU)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _slot_rows(b):
    nb = int(b.num_blocks.item())
    R = nb * spec.MENU[int(b.variant.item())][0]
    return R, b.sorted_slots[:R] >= 0


def _noalloc(b):
    moe_grouped_ffn_noalloc(b.p, b.x, b.w1, b.w3, b.w2, b.s1, b.s3, b.s2, b.sorted_slots,
                            b.block_expert, b.num_blocks, b.variant, b.y_slots)


@pytest.mark.parametrize("shape,sizes", [
    ("qwen3", (300, 37)), ("tiny", (64, 5)), ("small_fp8ah", (130, 9)),
    ("dsv3_share_fp8a", (96, 8)), ("small_sh", (130, 17))])
def test_noalloc_matches_workspace_entry(shape, sizes):
    wdev = G.weights(shape)[0] if shape in ("qwen3", "dsv3_share_fp8a") else None
    for v in range(V):
        for B in sizes:  # two calls in a row, the second smaller
            G.say(f"noalloc {shape} B={B} variant={v}")
            if wdev is not None:
                layer = synth.make_layer(shape, B, 0.3, 1, weights=G.weights(shape)[1])
            else:
                layer = synth.make_layer(shape, B, 0.3, 1)
            b = G.run(layer, variant=v, wdev=wdev)   # moe_grouped_ffn, caller workspace
            R, rows = _slot_rows(b)
            ref_ys = b.y_slots[:R][rows].clone()
            ref_y = b.y.clone()
            b.y_slots.fill_(7.0)
            b.y.fill_(7.0)
            _noalloc(b)
            L.combine(b)
            torch.cuda.synchronize()
            assert torch.equal(b.y_slots[:R][rows].view(torch.int16 if b.y.dtype != torch.float32
                                                       else torch.int32),
                               ref_ys.view(torch.int16 if b.y.dtype != torch.float32
                                           else torch.int32)), (shape, B, v)
            assert torch.equal(b.y, ref_y), (shape, B, v)


def test_noalloc_split_tail_load():
    """Qwen3 B = 130: the last round of tiles is split across the grid in every
    configuration, so the partial sums pass through the library's array."""
    wdev, whost = G.weights("qwen3")
    layer = synth.make_layer("qwen3", 130, 0.3, 5, weights=whost)
    for v in range(V):
        b = G.run(layer, variant=v, wdev=wdev)
        ref = b.y.clone()
        b.y.fill_(3.0)
        _noalloc(b)
        L.combine(b)
        torch.cuda.synchronize()
        assert torch.equal(b.y.view(torch.int16), ref.view(torch.int16)), v
    assert np.isfinite(ref.float().cpu().numpy()).all()
