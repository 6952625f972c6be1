"""The C ABI without a GPU: the library loads, exports every symbol include/moe.h
declares, and its host-side validation returns the documented status codes."""
import ctypes
import os
import re

import pytest

import routing_aware_grouped_amd as moe
from tests import spec

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")


def _declared():
    src = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|int32_t|int64_t|size_t)\s+(moe_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 9
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    for n in ("moe_route_topk", "moe_select_config", "moe_align_sort", "moe_grouped_ffn",
              "moe_combine"):
        assert n in names


def test_binding_mirrors_names():
    for n in _declared():
        assert callable(getattr(moe, n)), n


def test_variant_menu_matches_spec():
    assert moe.moe_abi_version() == 8
    assert moe.moe_num_variants() == len(spec.MENU)
    for v, m in enumerate(spec.MENU):
        assert tuple(moe.moe_variant_info(v)) == m
    for bad in (-1, len(spec.MENU)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_variant_info(bad)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def _p(**kw):
    base = dict(tokens=64, hidden=128, inter=256, num_experts=8, top_k=2, act_dtype=moe.MOE_F32,
                weight_dtype=moe.MOE_F32)
    base.update(kw)
    extra = {k: base.pop(k) for k in ("expert_begin", "local_experts", "renormalize", "act_quant",
                                      "shared_experts") if k in base}
    return moe.problem(base.pop("tokens"), base.pop("hidden"), base.pop("inter"),
                       base.pop("num_experts"), base.pop("top_k"), **base, **extra)


def test_query_sizes():
    s = moe.moe_query_sizes(_p())
    B, k, El, bmax = 64, 2, 8, max(m[0] for m in spec.MENU)
    assert s.rows_max == B * k + min(El, B * k) * (bmax - 1)
    assert s.blocks_max >= s.rows_max // min(m[0] for m in spec.MENU)
    assert s.y_slots_bytes == s.rows_max * 128 * 4
    assert s.workspace_bytes >= s.rows_max * 256 * 4
    s2 = moe.moe_query_sizes(_p(tokens=4096, hidden=2048, inter=768, num_experts=128, top_k=8,
                                act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16))
    assert s2.y_slots_bytes == s2.rows_max * 2048 * 2
    # monotone in the token count
    prev = 0
    for B in (1, 2, 17, 256, 4096):
        r = moe.moe_query_sizes(_p(tokens=B)).rows_max
        assert r >= prev
        prev = r


@pytest.mark.parametrize("kw,status", [
    (dict(tokens=0), moe.MOE_ERR_INVALID_ARG),
    (dict(hidden=100), moe.MOE_ERR_INVALID_ARG),
    (dict(inter=192), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), moe.MOE_ERR_INVALID_ARG),
    (dict(num_experts=64, top_k=33), moe.MOE_ERR_INVALID_ARG),
    (dict(expert_begin=4, local_experts=5), moe.MOE_ERR_INVALID_ARG),
    (dict(local_experts=0), moe.MOE_ERR_INVALID_ARG),
    (dict(renormalize=2), moe.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=moe.MOE_F32, weight_dtype=moe.MOE_BF16), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=moe.MOE_FP8_E4M3, weight_dtype=moe.MOE_FP8_E4M3), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(act_quant=3, act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_FP8_E4M3),
     moe.MOE_ERR_INVALID_ARG),
    (dict(act_quant=2, act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16), moe.MOE_ERR_UNSUPPORTED),
    # the FP8 activation path needs bf16 activations and fp8 weights
    (dict(act_quant=1, act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_quant=1), moe.MOE_ERR_UNSUPPORTED),
    (dict(shared_experts=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(shared_experts=9), moe.MOE_ERR_INVALID_ARG),
    (dict(tokens=1 << 20, num_experts=1024, local_experts=1024, top_k=8), moe.MOE_ERR_UNSUPPORTED),
    # one expert's bf16 weight matrix of 2^31 bytes: beyond the 32-bit buffer offsets
    (dict(hidden=32768, inter=32768, act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16),
     moe.MOE_ERR_UNSUPPORTED),
    # x of 2^31 bytes (B * H bf16)
    (dict(tokens=1 << 18, hidden=4096, num_experts=8, local_experts=8, top_k=1,
          act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_problems(kw, status):
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_query_sizes(_p(**kw))
    assert ei.value.status == status


def test_act_quant_workspace_holds_codes_and_scales():
    """With the FP8 activation path the workspace grows by the x codes (B * H bytes)
    and scales (B * H / 128 floats), each rounded up to 256 bytes."""
    kw = dict(tokens=37, hidden=7168, inter=2048, num_experts=256, top_k=8, expert_begin=32,
              local_experts=32, act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_FP8_E4M3)
    s0 = moe.moe_query_sizes(_p(**kw))
    s1 = moe.moe_query_sizes(_p(act_quant=1, **kw))
    up = lambda n: (n + 255) // 256 * 256  # noqa: E731
    assert s1.workspace_bytes - s0.workspace_bytes == up(37 * 7168) + up(37 * 56 * 4)
    assert (s1.rows_max, s1.y_slots_bytes) == (s0.rows_max, s0.y_slots_bytes)
    # act_quant 2 adds h codes and scales for every slot row
    s2 = moe.moe_query_sizes(_p(act_quant=2, **kw))
    R = s0.rows_max
    assert s2.workspace_bytes - s1.workspace_bytes == up(R * 2048) + up(R * 16 * 4)
    with pytest.raises(moe.MoeError) as ei:  # quantization without the path
        moe.moe_quant_act(_p(**kw), 0x1000, 0x1000, 0x1000, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # x misaligned
        moe.moe_quant_act(_p(act_quant=1, **kw), 0x1008, 0x1000, 0x1000, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_shared_experts_sizes_and_combine_entry_points():
    """Each shared expert adds B rows plus at most BLOCK_M - 1 of padding; the plain
    combine refuses problems with shared experts and the shared combine the others."""
    s0 = moe.moe_query_sizes(_p())
    s2 = moe.moe_query_sizes(_p(shared_experts=2))
    bmax = max(m[0] for m in spec.MENU)
    assert s2.rows_max - s0.rows_max == 2 * (64 + bmax - 1)
    a = 0x10000
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_combine(_p(shared_experts=1), a, a, a, a, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_combine_shared(_p(), a, a, a, a, a, a, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # needs the device block count
        moe.moe_combine_shared(_p(shared_experts=1), a, a, a, None, a, a, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_largest_expert_matrix_is_accepted():
    """An expert matrix one 128-column block below 2^31 bytes is within the limits."""
    s = moe.moe_query_sizes(_p(hidden=32768, inter=32768 - 128, act_dtype=moe.MOE_BF16,
                               weight_dtype=moe.MOE_BF16))
    assert s.rows_max > 0


def test_compute_calls_validate_before_any_gpu_work():
    p = _p()
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_route_topk(p, 0, 0, 0, 0, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_select_config(p, 0, 0, 0, None, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_align_sort(p, 0x1000, 0x1000, 0, 0x1000, 0x1000, 0x1000, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # the fused steps need slot_pos
        moe.moe_route_select_align(p, 0x1000, None, 0x1000, 0x1000, 0x1000, 0x1000, None, 0x1000,
                                   0x1000, 0x1000, 0, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # logits misaligned
        moe.moe_route_select_align(p, 0x1002, None, 0x1000, 0x1000, 0x1000, 0x1000, None, 0x1000,
                                   0x1000, 0x1000, 0x1000, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_combine(p, 0x1000, 0x1000, 0x1000, 0x1004, stream=0)  # y misaligned
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    sz = moe.moe_query_sizes(p)
    a = 0x10000
    with pytest.raises(moe.MoeError) as ei:  # workspace one byte short
        moe.moe_grouped_ffn(p, a, a, a, a, None, None, None, a, a, a, a, a, a,
                            sz.workspace_bytes - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    pf = _p(act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_FP8_E4M3)
    with pytest.raises(moe.MoeError) as ei:  # fp8 weights need their scales
        moe.moe_grouped_ffn(pf, a, a, a, a, None, None, None, a, a, a, a, a, a, 1 << 30, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # the gate/up phase needs x
        moe.moe_grouped_gate_up(p, None, a, a, None, None, a, a, a, a, a, 1 << 30, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # the down phase needs y_slots
        moe.moe_grouped_down(p, a, None, a, a, a, a, None, a, 1 << 30, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # workspace one byte short
        moe.moe_grouped_down(p, a, None, a, a, a, a, a, a, sz.workspace_bytes - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as ei:  # fp8 down needs its scales
        moe.moe_grouped_down(pf, a, None, a, a, a, a, a, a, 1 << 30, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_query_sizes(None)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_noalloc_refuses_problems_beyond_its_array():
    """moe_grouped_ffn_noalloc checks the problem's workspace against its fixed
    per-GPU array on the host, before any HIP call (so this runs without a GPU)."""
    limit = moe.moe_noalloc_workspace_limit()
    assert limit == 256 << 20
    p = _p(tokens=4096, hidden=7168, inter=2048, num_experts=384, top_k=8, local_experts=48,
           expert_begin=0, act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_FP8_E4M3, act_quant=2)
    assert moe.moe_query_sizes(p).workspace_bytes > limit
    d = 1 << 16  # placeholder device address, never dereferenced on the host
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_grouped_ffn_noalloc(p, d, d, d, d, d, d, d, d, d, d, d, d, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE


def test_packed_weights_only_for_bf16_problems():
    """The wide configuration's packed copy: its size follows the header's layout;
    problems that are not bf16, a misaligned copy, and packing a problem that
    already names a copy are rejected before anything runs."""
    p = _p(act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16, hidden=384, inter=256,
           local_experts=5, shared_experts=1)
    assert moe.moe_pack_wide_bytes(p) == spec.pack_wide_bytes(6, 384, 256)
    q = _p()  # fp32
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_wide_bytes(q)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    q.packed_weights = 1 << 20
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_query_sizes(q)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    p.packed_weights = (1 << 20) + 128  # not 256-byte aligned
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_query_sizes(p)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    p.packed_weights = 1 << 20
    moe.moe_query_sizes(p)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_wide(p, 1 << 20, 1 << 21, 1 << 22, 1 << 23, 0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG


def test_pack_layout_restatement_small():
    """spec.pack_wide on a hand-checkable case: element (e, row, k) of W1 lands at
    block (e, row // 128, k // 32), row row % 128, column k % 32."""
    import numpy as np
    E, I, H = 2, 256, 64
    w1 = np.arange(E * I * H, dtype=np.uint16).reshape(E, I, H)
    w3 = (w1 + 7).astype(np.uint16)
    w2 = np.arange(E * H * I, dtype=np.uint16).reshape(E, H, I) ^ 0x5555
    pk = spec.pack_wide(w1, w3, w2)
    assert pk.size * 2 == spec.pack_wide_bytes(E, H, I)
    nst, ncol = H // 32, I // 128
    for (e, r, k) in ((0, 0, 0), (1, 200, 37), (0, 129, 63)):
        blk = (e * ncol + r // 128) * nst + k // 32
        assert pk[blk * 256 * 32 + (r % 128) * 32 + k % 32] == w1[e, r, k]
        assert pk[blk * 256 * 32 + (128 + r % 128) * 32 + k % 32] == w3[e, r, k]
    base = E * ncol * nst * 256 * 32
    for (e, r, k) in ((1, 63, 255), (0, 5, 40)):
        blk = e * 1 * (I // 32) + k // 32  # one down column tile (H = 64 < 256)
        assert pk[base + blk * 256 * 32 + r * 32 + k % 32] == w2[e, r, k]
    # rows 64..255 of each down block are zeros (H = 64)
    assert not pk[base:].reshape(-1, 256, 32)[:, 64:].any()


def test_fused_plan_sizes_and_validation():
    """The fused small-batch plan: its workspace is a 256-byte header plus fp32
    partial rows [I / 32][B k][H] (the header's formula); problems outside it and
    bad arguments are rejected on the host, before anything runs."""
    pb = _p(tokens=3, hidden=384, inter=256, act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16)
    assert moe.moe_fused_workspace_bytes(pb) == 256 + 4 * (256 // 32) * 3 * 2 * 384
    for kw in (dict(),  # fp32
               dict(act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_FP8_E4M3, act_quant=1),
               dict(act_dtype=moe.MOE_BF16, weight_dtype=moe.MOE_BF16, shared_experts=1)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_fused_workspace_bytes(_p(**kw))
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED, kw
    a = 0x10000
    need = moe.moe_fused_workspace_bytes(pb)
    with pytest.raises(moe.MoeError) as ei:  # workspace one byte short
        moe.moe_grouped_ffn_fused(pb, a, a, a, a, None, None, None, a, a, a, a, a, need - 1, stream=0)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as ei:  # workspace not 256-byte aligned
        moe.moe_grouped_ffn_fused(pb, a, a, a, a, None, None, None, a, a, a, a, a + 128, need,
                                  stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    pf = _p(tokens=3, hidden=384, inter=256, act_dtype=moe.MOE_BF16,
            weight_dtype=moe.MOE_FP8_E4M3)
    with pytest.raises(moe.MoeError) as ei:  # fp8 weights need their scales
        moe.moe_grouped_ffn_fused(pf, a, a, a, a, None, None, None, a, a, a, a, a, 1 << 30,
                                  stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # no y
        moe.moe_combine_fused(pb, a, a, a, None, stream=0)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as ei:  # the grouped plan's problems only
        moe.moe_combine_fused(_p(), a, a, a, a, stream=0)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
