"""GPU parity of the fused small-batch plan (moe_grouped_ffn_fused +
moe_combine_fused, RaMP appendix A.8 "Fusion") against the CPU oracle: routing,
choice and alignment bit-exact as in the grouped plan, Y within
max|gpu - ref| / max|ref| <= 1e-2 (bf16 weights) or 5e-2 (fp8 weights).  Also:
every configuration's row-block size (several 32-row passes per row-block when a
block holds more rows), agreement with the grouped plan, bitwise determinism,
graph replay, and the device status word."""
import numpy as np
import pytest
import torch

import synth
from routing_aware_grouped_amd import layer as L
from tests import gpu_helpers as G
from tests import spec

pytestmark = pytest.mark.gpu
V = len(spec.MENU)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _run_fused(layer, variant=None, theta=None, wdev=None, pack=None):
    return G.run(layer, variant=variant, theta=theta, wdev=wdev, plan="fused", pack=pack)


def _check_all(layer, b, tokens=None):
    out = G.fetch(b)
    ids, w = G.check_routing(layer, out)
    G.check_align(layer, out, ids)
    err, _ = G.check_y(layer, out, ids, w, tokens=tokens)
    return out, err


@pytest.mark.parametrize("shape,B,alpha,x_std", [
    ("tiny_bf16", 1, 1.0, 0.02), ("tiny_bf16", 5, 1.0, 1.0), ("tiny_bf16", 64, 0.1, 0.02),
    ("small_fp8", 3, 1.0, 0.02), ("small_fp8", 32, 0.1, 1.0),
    ("mixtral", 1, 1.0, 0.02), ("mixtral", 16, 0.1, 0.02),
    ("qwen3", 1, 1.0, 0.02), ("qwen3", 8, 0.05, 0.02),
    ("dsv3_share", 8, 1.0, 0.02), ("dsv3_share", 64, 0.1, 1.0),
    ("kimi_share", 8, 0.05, 0.02), ("kimi_share", 64, 0.05, 0.02)])
def test_fused_plan_matches_oracle(shape, B, alpha, x_std):
    G.say(f"fused plan {shape} B={B} alpha={alpha} x_std={x_std}")
    wdev, whost = G.weights(shape)
    layer = G.layer_with_weights(shape, B, alpha, 0, whost=whost, x_std=x_std)
    b = _run_fused(layer, theta=G.theta_forcing(1), wdev=wdev)  # configuration 1: BLOCK_M 32
    _, err = _check_all(layer, b)
    G.say(f"  rel err {err:.3g}")


@pytest.mark.parametrize("v", range(V))
def test_fused_plan_every_row_block_size(v):
    """B = 64, alpha = 0.1: one expert holds most slots, so the row-blocks of the
    larger BLOCK_M hold more than 32 rows and take several passes."""
    G.say(f"fused plan tiny_bf16 B=64 alpha=0.1 variant={v}")
    layer = synth.make_layer("tiny_bf16", 64, 0.1, 1)
    b = _run_fused(layer, variant=v)
    out, _ = _check_all(layer, b)
    assert out["variant"] == v


def test_fused_plan_agrees_with_grouped_plan_and_is_deterministic():
    for shape, B in (("mixtral", 5), ("dsv3_share", 16)):
        G.say(f"fused vs grouped {shape} B={B}")
        wdev, whost = G.weights(shape)
        layer = G.layer_with_weights(shape, B, 1.0, 2, whost=whost, x_std=1.0)
        bf = _run_fused(layer, theta=G.theta_forcing(0), wdev=wdev)
        bg = G.run(layer, theta=G.theta_forcing(0), wdev=wdev)
        yf = bf.y.float().cpu().numpy()
        yg = bg.y.float().cpu().numpy()
        tol = G.TOL[synth.FP8 if layer.shape.weight_dtype == synth.FP8 else synth.BF16]
        assert G.rel_err(yf, yg.astype(np.float64)) <= tol
        y1 = bf.y.clone()
        L.forward(bf)
        torch.cuda.synchronize()
        assert torch.equal(bf.y, y1)


@pytest.mark.parametrize("shape,B", [("tiny_bf16", 37), ("mixtral", 3), ("qwen3", 16)])
def test_fused_plan_packed_weights_give_the_same_bits(shape, B):
    """bf16 problems read the packed weight copy when the problem names one: the
    same values in the same order, so the same bits as reading W1, W3, W2."""
    G.say(f"fused plan packed vs row-major {shape} B={B}")
    wdev, whost = G.weights(shape)
    layer = G.layer_with_weights(shape, B, 0.3, 3, whost=whost, x_std=1.0)
    bp = _run_fused(layer, theta=G.theta_forcing(1), wdev=wdev, pack=True)
    assert bp.p.packed_weights
    br = _run_fused(layer, theta=G.theta_forcing(1), wdev=wdev, pack=False)
    assert not br.p.packed_weights
    assert torch.equal(bp.y, br.y)


def test_fused_plan_graph_replay_equals_eager():
    layer = synth.make_layer("tiny_bf16", 48, 1.0, 4)
    b = _run_fused(layer, theta=G.theta_forcing(1))
    ref = b.y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        L.forward(b, stream=s)  # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            L.forward(b, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(3):
        b.y.fill_(float(r + 7))
        b.fused_ws.fill_(0xA5)  # poisoned workspace
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.y, ref), r


def _status(b) -> int:
    return int(b.fused_ws[:4].view(torch.int32).item())


def test_fused_plan_status_word_and_zeros_on_a_bad_configuration():
    from routing_aware_grouped_amd import MOE_DEV_BAD_VARIANT, MOE_DEV_OK
    layer = synth.make_layer("tiny_bf16", 32, 1.0, 5)
    b = _run_fused(layer, variant=0)
    torch.cuda.synchronize()
    assert _status(b) == MOE_DEV_OK
    b.variant.fill_(V + 2)
    b.y.fill_(1.0)
    L.ffn_fused(b)
    L.combine_fused(b)
    torch.cuda.synchronize()
    assert _status(b) == MOE_DEV_BAD_VARIANT
    assert torch.all(b.y == 0)
