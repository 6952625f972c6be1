"""Pins of the oracle's FP8 activation quantizer (step Q): per token and 128-column
group, s = amax / 448 and q = the nearest E4M3FN code of x / s (RaMP section 3.3:
FP8 with 128 x 128 block scaling as used by DeepSeek-V3, whose activations carry
one scale per 1 x 128 group).  The pins do not restate the oracle: they use the
E4M3FN value set (round trips, midpoints), torch's float8_e4m3fn cast as an
independent rounding routine, the error bound of round-to-nearest, and a special
case in which quantization is lossless and the FP8 activation layer must equal the
plain layer."""
import dataclasses

import numpy as np
import torch

import synth


def _code_values(oracle_lib):
    return oracle_lib.decode_fp8(np.arange(127, dtype=np.uint8))


def test_round_trip_every_finite_code(oracle_lib):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle_lib.decode_fp8(codes).astype(np.float32)
    q = oracle_lib.e4m3_round(vals)
    np.testing.assert_array_equal(q, codes)


def test_midpoints_round_to_even_code(oracle_lib):
    vals = _code_values(oracle_lib)
    lo, hi = vals[:-1], vals[1:]
    mid = ((lo + hi) / 2).astype(np.float32)  # <= 5 significant bits: exact in fp32
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    q = oracle_lib.e4m3_round(mid)
    c = np.arange(126)
    want = np.where(c % 2 == 0, c, c + 1)
    np.testing.assert_array_equal(q, want.astype(np.uint8))
    # just off the midpoint, the nearer neighbour wins, on both sides
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    np.testing.assert_array_equal(oracle_lib.e4m3_round(up), (c + 1).astype(np.uint8))
    np.testing.assert_array_equal(oracle_lib.e4m3_round(dn), c.astype(np.uint8))
    np.testing.assert_array_equal(oracle_lib.e4m3_round(-mid), (want | 0x80).astype(np.uint8))


def test_rounding_matches_torch_cast(oracle_lib):
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 0.05,          # subnormal range
                        rng.standard_normal(20000) * 1e-4,          # rounds to +-0
                        np.float32([0.0, -0.0, 448.0, -448.0])]).astype(np.float32)
    ours = oracle_lib.e4m3_round(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def _bf16(a):
    return synth.to_bf16_bits(np.asarray(a, np.float32))


def test_quantizer_matches_torch_pipeline_and_error_bound(oracle_lib):
    rng = np.random.default_rng(11)
    B, H = 6, 640
    x = rng.standard_normal((B, H)).astype(np.float32) * 0.02
    x[1, 128:256] = 0.0                       # an all-zero group
    x[2, 256:384] *= 1e4                      # a large group
    x[3, :128] = -np.abs(x[3, :128])          # the group maximum is negative
    bits = _bf16(x)
    q, s = oracle_lib.quant_act_e4m3(bits)
    xf = torch.from_numpy(synth.bf16_bits_to_f32(bits)).reshape(B, H // 128, 128)
    amax = xf.abs().amax(dim=2)
    s_t = amax / 448.0
    v = (xf / torch.where(s_t > 0, s_t, torch.ones_like(s_t))[..., None]).clamp(-448.0, 448.0)
    q_t = v.to(torch.float8_e4m3fn).view(torch.uint8).reshape(B, H).numpy().copy()
    q_t[s_t.repeat_interleave(128, dim=1).numpy() == 0] = 0
    np.testing.assert_array_equal(s, s_t.numpy())
    np.testing.assert_array_equal(q, q_t)
    assert np.all(s[1, 1] == 0) and np.all(q[1, 128:256] == 0)
    # the group maximum maps onto +-448 (code 0x7E / 0xFE)
    xa = np.abs(synth.bf16_bits_to_f32(bits)).reshape(B, H // 128, 128)
    arg = xa.argmax(axis=2)
    top = np.take_along_axis(q.reshape(B, H // 128, 128), arg[..., None], axis=2)[..., 0]
    nz = s > 0
    assert np.all((top[nz] & 0x7F) == 0x7E)
    # round to nearest: |x - q s| <= half a code step of x / s, times s
    xh = oracle_lib.dequant_act(q, s)
    xd = synth.bf16_bits_to_f32(bits).astype(np.float64)
    sv = np.repeat(s.astype(np.float64), 128, axis=1)
    mag = np.abs(xd) / np.where(sv > 0, sv, 1)
    step = np.where(mag >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3),
                    2.0 ** -9)
    bound = sv * (step / 2) * (1 + 2 ** -20) + np.abs(xd) * 2 ** -23
    assert np.all(np.abs(xd - xh) <= bound)


def test_lossless_grid_makes_fp8a_layer_equal_plain_layer(oracle_lib):
    """x already on the E4M3 grid, with every group's maximum equal to 448 * 2^-12:
    s = 2^-12 exactly, q reproduces x, and the FP8 activation layer equals the
    plain bf16-activation layer on the same weights."""
    sh = synth.SHAPES["small_fp8a"]
    lay = synth.make_layer("small_fp8a", 24, 1.0, 0)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 0x7E, (24, sh.hidden)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) * 0x80).astype(np.uint8)
    codes[:, ::128] = 0x7E                       # each group's maximum: 448
    vals = oracle_lib.decode_fp8(codes) * 2.0 ** -12
    bits = _bf16(vals)
    assert np.array_equal(synth.bf16_bits_to_f32(bits).astype(np.float64), vals)
    q, s = oracle_lib.quant_act_e4m3(bits)
    assert np.all(s == np.float32(2.0 ** -12))
    np.testing.assert_array_equal(q, codes)
    lay_q = dataclasses.replace(lay, x=bits)
    plain = dataclasses.replace(lay_q, shape=dataclasses.replace(sh, act_quant=0))
    ids, w = oracle_lib.route_topk(lay.logits, sh.top_k)
    toks = np.arange(24, dtype=np.int32)
    y_q = oracle_lib.layer_tokens(lay_q, ids, w, toks)
    y_p = oracle_lib.layer_tokens(plain, ids, w, toks)
    np.testing.assert_array_equal(y_q, y_p)
    assert np.abs(y_p).max() > 0


def _torch_quant_rows(a: np.ndarray) -> np.ndarray:
    """Q written with torch ops on bf16 rows: per 128-column group s = amax / 448,
    q = float8_e4m3fn(clamp(x / s)); returns q * s in fp64."""
    xf = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).float()
    n, m = xf.shape
    g = xf.reshape(n, m // 128, 128)
    s = g.abs().amax(dim=2) / 448.0
    q = (g / torch.where(s > 0, s, torch.ones_like(s))[..., None]).clamp(-448.0, 448.0)
    q = q.to(torch.float8_e4m3fn).to(torch.float64)
    q[(s == 0)[..., None].expand_as(q)] = 0.0
    return (q * s.double()[..., None]).reshape(n, m).numpy()


def test_one_hot_router_with_fp8_x_and_h_is_quantized_dense_ffn(oracle_lib):
    """All tokens on one expert ("Decoding the Skew" III-C3) with x and h both
    quantized: the dense FFN with torch's quantization of x, h rounded through fp32
    to bf16 and quantized the same way, and fp64 matrix products."""
    rng = np.random.default_rng(21)
    T, E, H, I = 9, 4, 256, 384
    shape = synth.Shape("t", H, I, E, E, 1, synth.BF16, synth.F32, synth.BF16, "normal", 2)
    x = synth.to_bf16_bits((rng.standard_normal((T, H)) * 0.5).astype(np.float32))
    w = {n: (rng.standard_normal((E,) + s) * 0.1).astype(np.float32)
         for n, s in (("w1", (I, H)), ("w3", (I, H)), ("w2", (H, I)))}
    lg = np.full((T, E), -5.0, np.float32)
    lg[:, 1] = 3.0
    lay = synth.Layer(shape, T, None, 0, lg, x, w["w1"], w["w3"], w["w2"])
    out = oracle_lib.full_layer(lay, b=16)
    xq = _torch_quant_rows(synth.bf16_bits_to_f32(x))
    g = xq @ w["w1"][1].astype(np.float64).T
    u = xq @ w["w3"][1].astype(np.float64).T
    hq = _torch_quant_rows((g / (1.0 + np.exp(-g)) * u).astype(np.float32))
    ref = hq @ w["w2"][1].astype(np.float64).T
    np.testing.assert_allclose(out["Y"], ref, rtol=1e-10, atol=1e-12)
    # and h quantization does change the result (the flag reaches the oracle)
    plain = oracle_lib.full_layer(dataclasses.replace(lay, shape=dataclasses.replace(shape, act_quant=1)), b=16)
    assert np.abs(plain["Y"] - out["Y"]).max() > 1e-6 * np.abs(ref).max()
