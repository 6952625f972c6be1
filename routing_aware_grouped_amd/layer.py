"""Device buffers for one fused-MoE problem and the five library calls in order.

Holds no arithmetic of its own: torch allocates device memory, and `forward`
enqueues moe_route_select_align (routing, configuration choice and alignment
fused) -> moe_grouped_ffn -> moe_combine on one stream, with no host
synchronisation, so a caller may capture it in a HIP graph.  With the fused
plan (small batches) the last two are moe_grouped_ffn_fused -> moe_combine_fused.
The separate step calls (route, select, align) remain for tests and per-step
timing.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, moe_align_sort, moe_combine, moe_combine_fused,
               moe_combine_shared, moe_fused_workspace_bytes, moe_grouped_down,
               moe_grouped_ffn, moe_grouped_ffn_fused, moe_grouped_gate_up, moe_num_variants,
               moe_pack_wide,
               moe_pack_wide_bytes, moe_problem,
               moe_query_sizes, moe_route_select_align, moe_route_topk, moe_select_config)

_TORCH_ACT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


@dataclasses.dataclass
class Buffers:
    p: moe_problem
    logits: torch.Tensor
    x: torch.Tensor
    w1: torch.Tensor
    w3: torch.Tensor
    w2: torch.Tensor
    s1: torch.Tensor | None
    s3: torch.Tensor | None
    s2: torch.Tensor | None
    theta: torch.Tensor
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    variant: torch.Tensor
    t_hat: torch.Tensor
    sorted_slots: torch.Tensor
    block_expert: torch.Tensor
    num_blocks: torch.Tensor
    slot_pos: torch.Tensor
    y_slots: torch.Tensor
    workspace: torch.Tensor
    y: torch.Tensor
    packed: torch.Tensor | None = None  # the wide configuration's packed weights
    fused_ws: torch.Tensor | None = None  # the fused plan's workspace (plan "fused")
    plan: str = "grouped"


# Plan "auto" takes the fused plan for bf16 problems that have the packed weight
# copy when the expert weights the batch can reach, min(E_loc, B k) experts of
# 3 H I bf16 values, are at most this many bytes: there the layer's launches cost
# more than the fused plan's slower weight stream (measured on MI355X: Qwen3-shaped
# layers at B = 1 and 4 are 30% and 17-19% faster fused, B = 16 within 4% either
# way; a Mixtral-shaped layer at B = 1 is 6-9% slower, the fp8-weight shares
# 40-52% slower).
FUSED_MAX_WEIGHT_BYTES = 512 << 20


def fused_supported(p: moe_problem) -> bool:
    """The problems the fused plan covers: bf16 activations with bf16 or fp8
    weights, no FP8 activation path, no shared experts."""
    return (p.act_dtype == MOE_BF16 and p.weight_dtype in (MOE_BF16, MOE_FP8_E4M3)
            and not p.act_quant and not p.shared_experts)


def choose_plan(p: moe_problem, plan: str = "auto") -> str:
    """"grouped", "fused", or "auto" (the rule of FUSED_MAX_WEIGHT_BYTES)."""
    if plan == "auto":
        if not (fused_supported(p) and p.weight_dtype == MOE_BF16 and p.packed_weights):
            return "grouped"
        reach = min(p.local_experts, p.tokens * p.top_k) * 3 * p.hidden * p.inter * 2
        return "fused" if reach <= FUSED_MAX_WEIGHT_BYTES else "grouped"
    if plan not in ("grouped", "fused"):
        raise ValueError(f"unknown plan {plan!r}")
    return plan


def packed_weights(p: moe_problem, w1, w3, w2, stream=None) -> torch.Tensor:
    """The wide configuration's packed copy of bf16 device weights (moe_pack_wide),
    written once per weight set: it is kept on w1 and reused while the problem's
    shapes, the three tensors and their contents (in-place version counters) are
    unchanged."""
    key = (p.local_experts, p.shared_experts, p.hidden, p.inter, w3.data_ptr(), w2.data_ptr(),
           w1._version, w3._version, w2._version)
    cached = getattr(w1, "_moe_wide_pack", None)
    if cached is not None and cached[0] == key:
        return cached[1]
    q = moe_problem.from_buffer_copy(p)
    q.packed_weights = None
    t = torch.empty(moe_pack_wide_bytes(q), dtype=torch.uint8, device=w1.device)
    moe_pack_wide(q, w1, w3, w2, t, stream)
    w1._moe_wide_pack = (key, t)
    return t


def allocate(p: moe_problem, logits, x, w1, w3, w2, s1=None, s3=None, s2=None, theta=None,
             device="cuda", pack=None, plan="grouped") -> Buffers:
    """Output/intermediate buffers sized by moe_query_sizes; inputs are moved to
    the device as given (already dtype-encoded).  pack (default: bf16 problems)
    gives the wide configuration its packed weight copy (packed_weights).  plan:
    see choose_plan; the fused plan also gets its workspace."""
    p = moe_problem.from_buffer_copy(p)
    if pack is None:
        pack = p.act_dtype == MOE_BF16 and p.weight_dtype == MOE_BF16
    sz = moe_query_sizes(p)
    B, k, El = p.tokens, p.top_k, p.local_experts
    V = moe_num_variants()
    dev = torch.device(device)
    act = _TORCH_ACT[p.act_dtype]

    def d(t):
        return None if t is None else t.to(dev).contiguous()

    if theta is None:
        theta = torch.zeros(V, 4, dtype=torch.float32)
    if tuple(theta.shape) != (V, 4):
        # the selection kernels read four coefficients per compiled configuration
        raise ValueError(f"theta must be [{V}][4], got {tuple(theta.shape)}")
    w1, w3, w2 = d(w1), d(w3), d(w2)
    packed = None
    if pack:
        p.packed_weights = None
        packed = packed_weights(p, w1, w3, w2)
        p.packed_weights = packed.data_ptr()
    plan = choose_plan(p, plan)
    return Buffers(
        p=p, logits=d(logits), x=d(x), w1=w1, w3=w3, w2=w2, s1=d(s1), s3=d(s3), s2=d(s2),
        theta=d(theta),
        topk_ids=torch.empty(B, k, dtype=torch.int32, device=dev),
        topk_w=torch.empty(B, k, dtype=torch.float32, device=dev),
        counts=torch.empty(El, dtype=torch.int32, device=dev),
        variant=torch.zeros(1, dtype=torch.int32, device=dev),
        t_hat=torch.empty(V, dtype=torch.float32, device=dev),
        sorted_slots=torch.empty(sz.rows_max, dtype=torch.int32, device=dev),
        block_expert=torch.empty(sz.blocks_max, dtype=torch.int32, device=dev),
        num_blocks=torch.zeros(1, dtype=torch.int32, device=dev),
        slot_pos=torch.empty(B * k, dtype=torch.int32, device=dev),
        y_slots=torch.empty(sz.rows_max, p.hidden, dtype=act, device=dev),
        workspace=torch.empty(sz.workspace_bytes, dtype=torch.uint8, device=dev),
        y=torch.empty(B, p.hidden, dtype=act, device=dev),
        packed=packed,
        fused_ws=(torch.empty(moe_fused_workspace_bytes(p), dtype=torch.uint8, device=dev)
                  if plan == "fused" else None),
        plan=plan,
    )


def use_plan(b: Buffers, plan: str) -> None:
    """Switch existing buffers to another plan (choose_plan), allocating the fused
    plan's workspace on first use."""
    b.plan = choose_plan(b.p, plan)
    if b.plan == "fused" and b.fused_ws is None:
        b.fused_ws = torch.empty(moe_fused_workspace_bytes(b.p), dtype=torch.uint8,
                                 device=b.y.device)


def route(b: Buffers, stream=None):
    moe_route_topk(b.p, b.logits, b.topk_ids, b.topk_w, b.counts, stream)


def select(b: Buffers, stream=None):
    moe_select_config(b.p, b.counts, b.theta, b.variant, b.t_hat, stream)


def align(b: Buffers, stream=None):
    moe_align_sort(b.p, b.topk_ids, b.variant, b.sorted_slots, b.block_expert, b.num_blocks,
                   b.slot_pos, stream)


def route_select_align(b: Buffers, stream=None, forced_variant: bool = False):
    """Steps 1-3 fused; with forced_variant the configuration in b.variant is kept."""
    moe_route_select_align(b.p, b.logits, None if forced_variant else b.theta, b.topk_ids,
                           b.topk_w, b.counts, b.variant, b.t_hat, b.sorted_slots,
                           b.block_expert, b.num_blocks, b.slot_pos, stream)


def ffn(b: Buffers, stream=None):
    moe_grouped_ffn(b.p, b.x, b.w1, b.w3, b.w2, b.s1, b.s3, b.s2, b.sorted_slots, b.block_expert,
                    b.num_blocks, b.variant, b.y_slots, b.workspace, None, stream)


def ffn_fused(b: Buffers, stream=None):
    moe_grouped_ffn_fused(b.p, b.x, b.w1, b.w3, b.w2, b.s1, b.s3, b.s2, b.sorted_slots,
                          b.block_expert, b.num_blocks, b.variant, b.fused_ws, None, stream)


def combine_fused(b: Buffers, stream=None):
    moe_combine_fused(b.p, b.fused_ws, b.slot_pos, b.topk_w, b.y, stream)


def gate_up(b: Buffers, stream=None):
    moe_grouped_gate_up(b.p, b.x, b.w1, b.w3, b.s1, b.s3, b.sorted_slots, b.block_expert,
                        b.num_blocks, b.variant, b.workspace, None, stream)


def down(b: Buffers, stream=None):
    moe_grouped_down(b.p, b.w2, b.s2, b.sorted_slots, b.block_expert, b.num_blocks, b.variant,
                     b.y_slots, b.workspace, None, stream)


def combine(b: Buffers, stream=None):
    if b.p.shared_experts:
        moe_combine_shared(b.p, b.y_slots, b.slot_pos, b.topk_w, b.num_blocks, b.variant, b.y,
                           stream)
    else:
        moe_combine(b.p, b.y_slots, b.slot_pos, b.topk_w, b.y, stream)


def forward(b: Buffers, stream=None, forced_variant: bool = False):
    """The whole layer.  With forced_variant the select step is skipped and the
    value already in b.variant is used (exhaustive timing of every configuration)."""
    route_select_align(b, stream, forced_variant)
    if b.plan == "fused":
        ffn_fused(b, stream)
        combine_fused(b, stream)
        return
    ffn(b, stream)
    combine(b, stream)


def forward_steps(b: Buffers, stream=None, forced_variant: bool = False):
    """The whole layer through the five separate step calls."""
    route(b, stream)
    if not forced_variant:
        select(b, stream)
    align(b, stream)
    ffn(b, stream)
    combine(b, stream)


def weight_tensors(layer):
    """Host numpy (dtype-encoded) -> torch tensors of the library's element types."""
    import numpy as np
    wd = layer.shape.weight_dtype

    def conv(a):
        if wd == MOE_F32:
            return torch.from_numpy(np.ascontiguousarray(a, np.float32))
        if wd == MOE_BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).view(torch.float8_e4m3fn)

    s = [None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32))
         for a in (layer.s1, layer.s3, layer.s2)]
    return conv(layer.w1), conv(layer.w3), conv(layer.w2), s[0], s[1], s[2]


def act_tensor(layer, a):
    import numpy as np
    if layer.shape.act_dtype == MOE_F32:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def problem_of(layer, renormalize: int = 1) -> moe_problem:
    sh = layer.shape
    return moe_problem(layer.tokens, sh.hidden, sh.inter, sh.num_experts, layer.expert_begin,
                       sh.local_experts, sh.top_k, sh.act_dtype, sh.weight_dtype, renormalize,
                       getattr(sh, "act_quant", 0), getattr(sh, "shared", 0), None)


def from_layer(layer, theta=None, device="cuda", weights=None, renormalize: int = 1,
               pack=None, plan="grouped") -> Buffers:
    """Buffers for a synthetic layer (see synth.Layer); `weights` reuses device
    weight tensors (w1, w3, w2, s1, s3, s2) across loads (and their packed copy)."""
    p = problem_of(layer, renormalize)
    if weights is None:
        weights = weight_tensors(layer)
    w1, w3, w2, s1, s3, s2 = weights
    return allocate(p, torch.from_numpy(layer.logits), act_tensor(layer, layer.x), w1, w3, w2, s1,
                    s3, s2, theta=theta, device=device, pack=pack, plan=plan)
