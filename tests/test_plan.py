"""The host-side plan rule (layer.choose_plan): the fused small-batch plan for bf16
problems with the packed weight copy whose reachable expert weights, min(E_loc,
B k) experts of 3 H I bf16 values, are at most FUSED_MAX_WEIGHT_BYTES; the
grouped plan otherwise.  No GPU needed."""
import pytest

import routing_aware_grouped_amd as moe
from routing_aware_grouped_amd import layer as L


def _p(tokens, hidden, inter, experts, top_k, wdt=moe.MOE_BF16, packed=True, **kw):
    p = moe.problem(tokens, hidden, inter, experts, top_k, act_dtype=moe.MOE_BF16,
                    weight_dtype=wdt, **kw)
    p.packed_weights = 1 << 20 if packed else None
    return p


def _reach(p):
    return min(p.local_experts, p.tokens * p.top_k) * 3 * p.hidden * p.inter * 2


@pytest.mark.parametrize("tokens,plan", [(1, "fused"), (4, "fused"), (8, "grouped"),
                                         (2048, "grouped")])
def test_qwen3_shaped_batches(tokens, plan):
    p = _p(tokens, 2048, 768, 128, 8)
    assert (_reach(p) <= L.FUSED_MAX_WEIGHT_BYTES) == (plan == "fused")
    assert L.choose_plan(p, "auto") == plan


def test_large_experts_and_unsupported_problems_stay_grouped():
    assert L.choose_plan(_p(1, 4096, 14336, 8, 2), "auto") == "grouped"  # 704 MB reachable
    assert L.choose_plan(_p(1, 2048, 768, 128, 8, packed=False), "auto") == "grouped"
    assert L.choose_plan(_p(1, 7168, 2048, 256, 8, wdt=moe.MOE_FP8_E4M3, packed=False,
                            local_experts=32), "auto") == "grouped"
    assert L.choose_plan(_p(1, 2048, 768, 128, 8, shared_experts=1), "auto") == "grouped"
    assert L.choose_plan(_p(1, 2048, 768, 128, 8, act_quant=0), "fused") == "fused"
    with pytest.raises(ValueError):
        L.choose_plan(_p(1, 2048, 768, 128, 8), "fastest")


def test_fused_support_matches_the_library():
    """fused_supported agrees with what moe_fused_workspace_bytes accepts."""
    cases = [dict(wdt=moe.MOE_BF16), dict(wdt=moe.MOE_FP8_E4M3), dict(shared_experts=1),
             dict(wdt=moe.MOE_FP8_E4M3, act_quant=1)]
    for kw in cases:
        p = _p(3, 384, 256, 8, 2, packed=False, **kw)
        try:
            moe.moe_fused_workspace_bytes(p)
            ok = True
        except moe.MoeError as e:
            assert e.status == moe.MOE_ERR_UNSUPPORTED
            ok = False
        assert L.fused_supported(p) == ok, kw
