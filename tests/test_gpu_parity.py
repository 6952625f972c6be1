"""GPU parity: every step of the HIP path against the CPU oracle on the same seeded
inputs.  Integer outputs (ids, counts, chosen configuration, permutation, block
table, inverse map) bit-exact; weights |d| <= 1e-6; Y within
max|gpu - ref| / max|ref| <= 1e-5 (fp32), 1e-2 (bf16), 5e-2 (fp8 weights)."""
import numpy as np
import pytest
import torch

import oracle
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


# ----------------------------------------------------------------- tiny fp32 ---
@pytest.mark.parametrize("v", range(V))
def test_tiny_fp32_every_variant(v):
    G.say(f"tiny fp32 B=64 variant={v}")
    layer = synth.make_layer("tiny", 64, None, 0)
    out = G.fetch(G.run(layer, variant=v))
    ids, w = G.check_routing(layer, out)
    G.check_align(layer, out, ids)
    G.check_y(layer, out, ids, w)


def test_tiny_renormalize_off_and_selection():
    layer = synth.make_layer("tiny", 64, None, 1)
    b = G.run(layer, theta=G.theta_forcing(2), renormalize=0)
    out = G.fetch(b)
    assert out["variant"] == 2
    ids, w = G.check_routing(layer, out, renormalize=0)
    G.check_align(layer, out, ids)
    G.check_y(layer, out, ids, w)


def test_tiny_large_activations_and_ragged_tokens():
    """x ~ N(0, 1) reaches SwiGLU's non-linear range; B = 37 leaves ragged tiles."""
    layer = synth.make_layer("tiny", 37, None, 2, x_std=1.0)
    for v in range(V):
        out = G.fetch(G.run(layer, variant=v))
        ids, w = G.check_routing(layer, out)
        G.check_align(layer, out, ids)
        G.check_y(layer, out, ids, w)


# -------------------------------------------------------------- routing only ---
@pytest.mark.parametrize("shape,B,alpha", [
    ("qwen3", 1, 0.3), ("qwen3", 4096, 0.05), ("qwen3", 1000, 10.0), ("mixtral", 2048, 0.1),
    ("mixtral", 3, 1.0), ("dsv3_share", 2048, 1.0), ("kimi_share", 4096, 0.05),
    ("kimi_share", 65, 0.05),
    # more 64-token blocks than alignment workgroups (64): some take two or three
    ("qwen3", 6000, 1.0), ("mixtral", 8193, 1.0)])
def test_routing_and_permutation_full_batch(shape, B, alpha):
    G.say(f"routing {shape} B={B} alpha={alpha}")
    sh = synth.SHAPES[shape]
    rng = np.random.default_rng([B, 3])
    logits, p = synth.routing_logits(sh, B, alpha, rng)
    e0 = synth.most_loaded_block(p, sh)
    H, I = 256, 256  # the FFN is not exercised here; keep its buffers small
    p_ = L.moe_problem(B, H, I, sh.num_experts, e0, sh.local_experts, sh.top_k, synth.BF16,
                       synth.BF16, 1)
    z = torch.zeros
    w1 = z(sh.local_experts, I, H, dtype=torch.bfloat16)
    w2 = z(sh.local_experts, H, I, dtype=torch.bfloat16)
    for v in range(V):
        b = L.allocate(p_, torch.from_numpy(logits), z(B, H, dtype=torch.bfloat16), w1, w1, w2,
                       theta=G.theta_forcing(v))
        L.route(b)
        L.select(b)
        L.align(b)
        torch.cuda.synchronize()
        out = G.fetch(b)
        assert out["variant"] == v
        lay = synth.Layer(sh, B, alpha, e0, logits, None, None, None, None)
        ids, _ = G.check_routing(lay, out)
        G.check_align(lay, out, ids)


@pytest.mark.parametrize("shape,B,alpha", [
    ("mixtral", 1, 1.0), ("mixtral", 512, 0.1), ("mixtral", 513, 0.1), ("mixtral", 2048, 1.0),
    ("qwen3", 64, 0.3), ("qwen3", 65, 0.3), ("qwen3", 4096, 1.0), ("dsv3_share", 96, 0.1),
    ("kimi_share", 2048, 0.05)])
def test_fused_selection_matches_steps(shape, B, alpha):
    """moe_route_select_align (one launch for a batch one workgroup routes, else
    the routing launches and one select+align launch) writes exactly what
    moe_route_topk, moe_select_config and moe_align_sort write, with a chosen and
    with a given configuration."""
    G.say(f"fused selection {shape} B={B} alpha={alpha}")
    sh = synth.SHAPES[shape]
    logits, p = synth.routing_logits(sh, B, alpha, np.random.default_rng([B, 9]))
    e0 = synth.most_loaded_block(p, sh)
    H, I = 256, 256
    p_ = L.moe_problem(B, H, I, sh.num_experts, e0, sh.local_experts, sh.top_k, synth.BF16,
                       synth.BF16, 1)
    z = torch.zeros
    w1 = z(sh.local_experts, I, H, dtype=torch.bfloat16)
    w2 = z(sh.local_experts, H, I, dtype=torch.bfloat16)
    th = torch.tensor([[50.0 * v, 0.5 * v + 1.0, 0.01, 0.1] for v in range(V)], dtype=torch.float32)
    names = ["topk_ids", "topk_w", "counts", "variant", "t_hat", "num_blocks", "slot_pos"]
    for forced in (False, True):
        bs = []
        for fused in (False, True):
            b = L.allocate(p_, torch.from_numpy(logits), z(B, H, dtype=torch.bfloat16), w1, w1, w2,
                           theta=th)
            b.variant.fill_(V - 1)
            b.t_hat.fill_(-1.0)
            b.sorted_slots.fill_(-7)
            b.block_expert.fill_(-7)
            if fused:
                L.route_select_align(b, forced_variant=forced)
            else:
                L.route(b)
                if not forced:
                    L.select(b)
                L.align(b)
            bs.append(b)
        torch.cuda.synchronize()
        a, f = bs
        for n in names:
            x, y = getattr(a, n), getattr(f, n)
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (n, forced)
        nb = int(a.num_blocks.item())
        R = nb * spec.MENU[int(a.variant.item())][0]
        assert torch.equal(a.sorted_slots[:R], f.sorted_slots[:R]) and torch.equal(
            a.block_expert[:nb], f.block_expert[:nb]), forced
        if forced:
            assert int(f.variant.item()) == V - 1 and torch.all(f.t_hat == -1.0)


def test_routing_ties_and_signed_zeros():
    """Equal logits go to the lower expert index; -0 equals +0."""
    rng = np.random.default_rng(44)
    for E, k in ((8, 2), (128, 8), (384, 8)):
        B = 300
        lg = rng.integers(-3, 4, size=(B, E)).astype(np.float32) * 0.5
        zm = rng.random((B, E)) < 0.2
        lg[zm] = np.where(rng.random(zm.sum()) < 0.5, -0.0, 0.0)
        sh = synth.Shape("t", 128, 128, E, E, k, synth.BF16, synth.BF16, synth.BF16, "normal")
        p_ = L.moe_problem(B, 128, 128, E, 0, E, k, synth.BF16, synth.BF16, 1)
        w = torch.zeros(E, 128, 128, dtype=torch.bfloat16)
        b = L.allocate(p_, torch.from_numpy(lg), torch.zeros(B, 128, dtype=torch.bfloat16), w, w, w)
        L.route(b)
        L.select(b)
        L.align(b)
        torch.cuda.synchronize()
        out = G.fetch(b)
        lay = synth.Layer(sh, B, None, 0, lg, None, None, None, None)
        ids, _ = G.check_routing(lay, out)
        G.check_align(lay, out, ids)


# ------------------------------------------------------------------ selection --
def test_select_config_bit_exact():
    """Chosen index and every fp32 prediction equal the oracle's, on random loads
    and random cost coefficients (including exact ties between configurations)."""
    from routing_aware_grouped_amd import moe_cost_constants, moe_select_config
    rng = np.random.default_rng(5)
    ncu = G.num_cus()
    for trial in range(60):
        El = int(rng.choice([8, 32, 48, 128, 1000]))
        H, I = (2048, 768) if trial % 2 else (7168, 2048)
        p_ = L.moe_problem(64, H, I, El, 0, El, 8, synth.BF16, synth.BF16, 1)
        cc = spec.cost_constants(H, I, ncu)
        assert moe_cost_constants(p_) == cc
        cnt = (rng.integers(0, 600, El) * (rng.random(El) < rng.random())).astype(np.int32)
        th = (rng.random((V, 4)) * np.array([20, 5, 0.05, 0.5])).astype(np.float32)
        if trial % 4 == 0:
            th[V - 1] = th[0]
        d_cnt = torch.from_numpy(cnt).cuda()
        d_th = torch.from_numpy(th).cuda()
        var = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        t_hat = torch.empty(V, dtype=torch.float32, device="cuda")
        moe_select_config(p_, d_cnt, d_th, var, t_hat)
        torch.cuda.synchronize()
        ref_v, ref_t, _ = oracle.select(cnt, cc["b"], cc["q1"], cc["q2"], cc["S1"], cc["S2"], th)
        assert int(var.item()) == ref_v
        np.testing.assert_array_equal(t_hat.cpu().numpy().view(np.uint32), ref_t.view(np.uint32))


# ------------------------------------------------------- bf16 / fp8 layers -----
@pytest.mark.parametrize("shape,B,alpha,sample", [
    ("qwen3", 1, 0.3, None), ("qwen3", 37, 1.0, None), ("qwen3", 130, 0.05, None),
    ("mixtral", 1, 1.0, None), ("mixtral", 5, 0.1, None),
    ("dsv3_share", 8, 1.0, None), ("dsv3_share", 96, 0.1, 24),
    ("kimi_share", 64, 0.05, 24), ("tiny_bf16", 37, 0.1, None), ("tiny_bf16", 700, 1.0, None)])
def test_layer_every_variant(shape, B, alpha, sample):
    G.say(f"layer {shape} B={B} alpha={alpha}")
    wdev, whost = G.weights(shape)
    layer = synth.make_layer(shape, B, alpha, 0, weights=whost)
    ids, w = oracle.route_topk(layer.logits, layer.shape.top_k)
    toks = None
    if sample is not None:
        toks = np.random.default_rng(B).choice(B, sample, replace=False).astype(np.int32)
    ref = None
    for v in range(V):
        out = G.fetch(G.run(layer, variant=v, wdev=wdev))
        G.check_routing(layer, out)
        G.check_align(layer, out, ids)
        err, ref = G.check_y(layer, out, ids, w, toks, ref)
        G.say(f"  variant {v}: rel err {err:.3g}")


def test_one_hot_router_is_dense():
    """All tokens on one expert: the layer equals that expert's dense FFN."""
    wdev, whost = G.weights("qwen3")
    layer = synth.make_layer("qwen3", 200, 1.0, 0, weights=whost)
    layer.logits[:] = -10.0
    layer.logits[:, 77] = 10.0  # expert 77 first for every token, then 0..6 (ties)
    out = G.fetch(G.run(layer, theta=G.theta_forcing(3), wdev=wdev))
    ids, w = G.check_routing(layer, out)
    assert np.all(ids[:, 0] == 77)
    G.check_align(layer, out, ids)
    G.check_y(layer, out, ids, w, tokens=np.arange(0, 200, 7))


def test_empty_rank_gives_zero_output():
    """An expert block that receives no token: no tiles, and Y = 0."""
    wdev, whost = G.weights("dsv3_share")
    layer = synth.make_layer("dsv3_share", 16, 1.0, 0, weights=whost)
    layer.logits[:, layer.expert_begin:layer.expert_begin + 32] = -50.0
    out = G.fetch(G.run(layer, theta=G.theta_forcing(0), wdev=wdev))
    ids, w = G.check_routing(layer, out)
    assert out["num_blocks"] == 0 and np.all(out["counts"] == 0)
    assert np.all(out["slot_pos"] == -1)
    assert np.all(out["Y"] == 0.0)


def _status(b) -> int:
    """The device status word at the start of the grouped-FFN workspace."""
    from routing_aware_grouped_amd import MOE_DEVICE_STATUS_OFFSET
    o = MOE_DEVICE_STATUS_OFFSET
    return int(b.workspace[o:o + 4].view(torch.int32).item())


def test_out_of_range_variant_gives_no_tiles():
    from routing_aware_grouped_amd import MOE_DEV_BAD_VARIANT, MOE_DEV_OK
    layer = synth.make_layer("tiny", 64, None, 3)
    b = G.run(layer, variant=0)
    assert _status(b) == MOE_DEV_OK
    b.variant.fill_(V + 3)
    b.y.fill_(1.0)
    L.align(b)
    L.ffn(b)
    L.combine(b)
    torch.cuda.synchronize()
    assert int(b.num_blocks.item()) == 0
    assert torch.all(b.slot_pos == -1)
    assert torch.all(b.y == 0)
    assert _status(b) == MOE_DEV_BAD_VARIANT
    # a valid configuration again: the next call reports its own inputs
    b.variant.fill_(1)
    L.align(b)
    L.ffn(b)
    torch.cuda.synchronize()
    assert _status(b) == MOE_DEV_OK


def test_block_count_beyond_buffers_is_reported():
    """A row-block count below zero or beyond what rows_max holds (a value the
    alignment step never writes) sets MOE_DEV_BAD_BLOCKS; the kernels compute only
    the row-blocks that fit (here rows past the real ones hold no slot)."""
    from routing_aware_grouped_amd import MOE_DEV_BAD_BLOCKS
    layer = synth.make_layer("tiny", 64, None, 3)
    b = G.run(layer, variant=2)
    nb = int(b.num_blocks.item())
    bm = spec.MENU[2][0]
    ref = b.y_slots[:nb * bm].clone()
    b.sorted_slots[nb * bm:].fill_(-1)
    b.block_expert[nb:].fill_(0)
    for bad in (b.sorted_slots.numel() // bm + 5, -3):
        b.num_blocks.fill_(bad)
        L.ffn(b)
        torch.cuda.synchronize()
        assert _status(b) == MOE_DEV_BAD_BLOCKS, bad
    b.num_blocks.fill_(nb)
    L.ffn(b)
    torch.cuda.synchronize()
    assert torch.equal(b.y_slots[:nb * bm], ref)


def test_out_of_range_variant_on_an_alignment_grid():
    """The same at B = 1000 (16 alignment workgroups, each clearing its share of
    slot_pos)."""
    sh = synth.SHAPES["qwen3"]
    B = 1000
    logits, p = synth.routing_logits(sh, B, 1.0, np.random.default_rng([B, 5]))
    p_ = L.moe_problem(B, 256, 256, sh.num_experts, 0, sh.local_experts, sh.top_k, synth.BF16,
                       synth.BF16, 1)
    z = torch.zeros
    w1 = z(sh.local_experts, 256, 256, dtype=torch.bfloat16)
    b = L.allocate(p_, torch.from_numpy(logits), z(B, 256, dtype=torch.bfloat16), w1, w1, w1,
                   theta=G.theta_forcing(0))
    L.route(b)
    b.variant.fill_(V + 3)
    b.slot_pos.fill_(7)
    b.num_blocks.fill_(9)
    L.align(b)
    torch.cuda.synchronize()
    assert int(b.num_blocks.item()) == 0
    assert torch.all(b.slot_pos == -1)


def test_fp8_decode_every_code():
    """With one-hot tokens, W3 = 1 and W2 = I, each output element is
    silu(s * q) of one fp8 weight code: every code must decode exactly as OCP
    E4M3FN (checked element by element, not in aggregate)."""
    H, I, E, B = 256, 128, 1, 256
    codes = (np.arange(I)[:, None] * 256 + np.arange(H)[None, :]) % 256
    codes[(codes & 0x7F) == 0x7F] = 0  # NaN codes are outside the contract
    w1 = codes.astype(np.uint8)[None]
    w3 = np.full((1, I, H), 0x38, np.uint8)  # 1.0
    w2 = np.zeros((1, H, I), np.uint8)
    w2[0, np.arange(I), np.arange(I)] = 0x38  # identity on the first I outputs
    s1 = np.array([[[1.0, 0.25]]], np.float32)
    s3 = np.ones((1, 1, 2), np.float32)
    s2 = np.ones((1, 2, 1), np.float32)
    x = np.zeros((B, H), np.float32)
    x[np.arange(B), np.arange(B) % H] = 1.0
    sh = synth.Shape("fp8codes", H, I, E, E, 1, synth.BF16, synth.FP8, synth.BF16, "normal")
    layer = synth.Layer(sh, B, None, 0, np.zeros((B, E), np.float32), synth.to_bf16_bits(x),
                        w1, w3, w2, s1, s3, s2)
    out = G.fetch(G.run(layer, variant=0))
    ids, w = oracle.route_topk(layer.logits, 1)
    ref = oracle.layer_tokens(layer, ids, w, np.arange(B, dtype=np.int32))
    gpu = out["Y"].astype(np.float64)
    bad = np.abs(gpu - ref) > 1e-2 * np.abs(ref) + 1e-30
    assert not bad.any(), f"{bad.sum()} elements differ, first at {np.argwhere(bad)[:4]}"


def test_deterministic_repeat():
    wdev, whost = G.weights("qwen3")
    layer = synth.make_layer("qwen3", 300, 0.3, 1, weights=whost)
    for v in range(V):
        a = G.run(layer, variant=v, wdev=wdev).y.clone()
        c = G.run(layer, variant=v, wdev=wdev).y.clone()
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_graph_replay_matches_eager():
    """The five calls captured in one HIP graph replay to the eager result, with
    eager work and synchronisation between replays."""
    wdev, whost = G.weights("qwen3")
    layer = synth.make_layer("qwen3", 64, 1.0, 2, weights=whost)
    th = torch.tensor([[5.0, 0.0, 0.01, 0.1]] * V, dtype=torch.float32)
    th[:, 0] += torch.arange(V, dtype=torch.float32)
    b = L.from_layer(layer, theta=th, weights=G.device_weights(layer, wdev))
    L.forward(b)
    torch.cuda.synchronize()
    eager = b.y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.forward(b, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    b.y.zero_()
    with torch.cuda.graph(g):
        L.forward(b)
    for r in range(4):
        b.y.fill_(float(r + 1))
        b.sorted_slots.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.y.view(torch.int16), eager.view(torch.int16)), r


def test_split_phases_match_ffn():
    """moe_grouped_gate_up then moe_grouped_down give the same y_slots, bit for bit,
    as moe_grouped_ffn (they enqueue the same two launches)."""
    wdev, whost = G.weights("qwen3")
    layer = synth.make_layer("qwen3", 77, 0.3, 4, weights=whost)
    for v in range(V):
        b = G.run(layer, variant=v, wdev=wdev)
        nb = int(b.num_blocks.item())
        R = nb * spec.MENU[v][0]
        rows = b.sorted_slots[:R] >= 0
        ref = b.y_slots[:R][rows].clone()
        b.y_slots.zero_()
        L.gate_up(b)
        L.down(b)
        torch.cuda.synchronize()
        assert torch.equal(b.y_slots[:R][rows].view(torch.int16), ref.view(torch.int16)), v


@pytest.mark.parametrize("B", [130, 1000])
def test_split_tail_tiles(B):
    """Loads whose last round of tiles is split across the grid: every variant
    matches the oracle, and three calls on one workspace agree bit for bit."""
    G.say(f"split tail qwen3 B={B}")
    wdev, whost = G.weights("qwen3")
    layer = synth.make_layer("qwen3", B, 0.3, 5, weights=whost)
    H, I = layer.shape.hidden, layer.shape.inter
    ids, w = oracle.route_topk(layer.logits, layer.shape.top_k)
    toks = np.random.default_rng(B).choice(B, 24, replace=False).astype(np.int32)
    grid = min(G.num_cus() * spec.WG_PER_CU[0], spec.MAX_GRID)
    ref, split = None, set()
    for v in range(V):
        b = G.run(layer, variant=v, wdev=wdev)
        out = G.fetch(b)
        G.check_align(layer, out, ids)
        err, ref = G.check_y(layer, out, ids, w, toks, ref)
        G.say(f"  variant {v}: rel err {err:.3g}")
        for N, BN in ((I, spec.MENU[v][1]), (H, spec.MENU[v][2])):
            tiles = out["num_blocks"] * (N // BN)
            if spec.MENU[v][9] == spec.WG_PER_CU[0] and \
                    spec.splits_tail(tiles % grid, grid, spec.MENU[v][8], tiles // grid):
                split.add(v)
        first = b.y.clone()
        for _ in range(2):
            b.y.fill_(3.0)
            L.align(b)
            L.ffn(b)
            L.combine(b)
            torch.cuda.synchronize()
            assert torch.equal(b.y.view(torch.int16), first.view(torch.int16)), v
    # on a 512-workgroup grid B = 130 splits a tail in every variant, B = 1000 in 0, 2, 3
    assert split, "no variant split a tail: the case tests nothing on this device"
