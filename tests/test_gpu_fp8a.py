"""GPU parity of the FP8 activation path (act_quant = 1): x quantized to E4M3FN per
token and 128-column group, the gate/up GEMM on fp8 x fp8 with the block scales
applied per 128-deep block (RaMP section 3.3 and appendix A.8).

- The codes and scales of moe_quant_act are bit-exact against the oracle's
  quantizer, on full-size activations and on crafted values (midpoints between
  codes, values that round to zero, zero groups, large groups).
- Y matches the oracle of the same method (the FFN on the dequantized x, and with
  act_quant 2 on the dequantized h as well) within max|gpu - ref| / max|ref| <=
  1e-2.  Against the unquantized layer, the quantization error itself is judged
  the way GC-MoE's accuracy suite judges its quantized routed experts (section 6:
  cosine similarity >= 0.97 against the higher-precision reference); the maximum
  relative error is reported next to it (3-5% here, from one or two E4M3
  roundings of every activation)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from routing_aware_grouped_amd import layer as L
from routing_aware_grouped_amd import moe_quant_act
from tests import gpu_helpers as G
from tests import spec

pytestmark = pytest.mark.gpu
V = len(spec.MENU)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _quant_gpu(layer, x_bits: np.ndarray):
    p = L.problem_of(layer)
    B, H = x_bits.shape
    p.tokens = B
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    xq = torch.full((B, H), 0x55, dtype=torch.uint8, device="cuda")
    xs = torch.full((B, H // 128), -1.0, dtype=torch.float32, device="cuda")
    moe_quant_act(p, x, xq, xs)
    torch.cuda.synchronize()
    return xq.cpu().numpy(), xs.cpu().numpy()


def _crafted_rows(H: int) -> np.ndarray:
    """Rows whose groups have the maximum 448 * 2^-12, so that x / s is exact: the
    midpoints between neighbouring codes test round-to-nearest-even, tiny negative
    values the sign of a zero code; plus a zero group and a large group."""
    vals = oracle.decode_fp8(np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    pool = np.concatenate([mids, -mids, vals, -vals, [-2.0 ** -12, -0.0, 2.0 ** -11]])
    rows = []
    rng = np.random.default_rng(17)
    for r in range(4):
        row = rng.choice(pool, H) * 2.0 ** -12
        row[::128] = 448.0 * 2.0 ** -12
        rows.append(row)
    rows[1][128:256] = 0.0                          # a group of zeros
    rows[2][256:384] *= 2.0 ** 20                   # a large group
    rows[3][:128] = -np.abs(rows[3][:128])          # negative maximum
    out = synth.to_bf16_bits(np.asarray(rows, np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(out).astype(np.float64), np.asarray(rows))
    return out


def test_quant_codes_bit_exact():
    wdev, whost = G.weights("dsv3_share_fp8a")
    layer = synth.make_layer("dsv3_share_fp8a", 2048, 1.0, 0, weights=whost)
    x = np.concatenate([layer.x, _crafted_rows(layer.shape.hidden)])
    G.say(f"quant codes B={x.shape[0]} H={x.shape[1]}")
    q, s = _quant_gpu(layer, x)
    q_ref, s_ref = oracle.quant_act_e4m3(x)
    np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(q, q_ref)
    assert (q[-3, 128:256] == 0).all() and (s[-3, 1] == 0)


def _check(layer, out, ids, w, toks):
    ref_q = oracle.layer_tokens(layer, ids, w, toks)
    err_q = G.rel_err(out["Y"][toks], ref_q)
    plain = dataclasses.replace(layer, shape=dataclasses.replace(layer.shape, act_quant=0))
    ref_p = oracle.layer_tokens(plain, ids, w, toks)
    y = out["Y"][toks].astype(np.float64)
    err_p = G.rel_err(y, ref_p)
    cos = float((y * ref_p).sum() / np.sqrt((y * y).sum() * (ref_p * ref_p).sum()))
    assert err_q <= 1e-2, f"vs the FP8-activation oracle: {err_q:.3g}"
    assert cos >= 0.97, f"cosine vs the unquantized oracle: {cos:.5f}"
    return err_q, err_p, cos


@pytest.mark.parametrize("shape,B,alpha,sample", [
    ("small_fp8a", 1, 1.0, None), ("small_fp8a", 37, 0.3, None), ("small_fp8a", 130, 1.0, None),
    ("dsv3_share_fp8a", 8, 1.0, None), ("dsv3_share_fp8a", 96, 0.1, 16),
    ("kimi_share_fp8a", 64, 0.05, 16), ("kimi_share_fp8a", 1000, 0.05, 16),
    ("small_fp8ah", 1, 1.0, None), ("small_fp8ah", 37, 0.3, None), ("small_fp8ah", 130, 1.0, None),
    ("dsv3_share_fp8ah", 8, 1.0, None), ("dsv3_share_fp8ah", 96, 0.1, 16),
    ("kimi_share_fp8ah", 64, 0.05, 16), ("kimi_share_fp8ah", 1000, 0.05, 16)])
def test_fp8a_layer_every_variant(shape, B, alpha, sample):
    G.say(f"fp8a layer {shape} B={B} alpha={alpha}")
    if shape.startswith("small_"):
        wdev, layer = None, synth.make_layer(shape, B, alpha, 0)
    else:
        wdev, whost = G.weights(shape)
        layer = synth.make_layer(shape, B, alpha, 0, weights=whost)
    ids, w = oracle.route_topk(layer.logits, layer.shape.top_k)
    toks = np.arange(B, dtype=np.int32) if sample is None else \
        np.random.default_rng(B).choice(B, sample, replace=False).astype(np.int32)
    first = None
    for v in range(V):
        b = G.run(layer, variant=v, wdev=wdev)
        out = G.fetch(b)
        G.check_routing(layer, out)
        G.check_align(layer, out, ids)
        err_q, err_p, cos = _check(layer, out, ids, w, toks)
        G.say(f"  variant {v}: rel err {err_q:.3g} (method), {err_p:.3g} (unquantized), "
              f"cosine {cos:.5f}")
        if v == 0:
            first = b.y.clone()
            L.ffn(b)            # a second pass on the same workspace: the same bits
            L.combine(b)
            torch.cuda.synchronize()
            assert torch.equal(b.y.view(torch.int16), first.view(torch.int16))
