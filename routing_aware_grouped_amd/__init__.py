"""Python binding of libmoe.so, the gfx950 routing-aware fused-MoE layer.

Argument marshalling only: every function here forwards to the C entry point of
the same name in libmoe.so (declared in include/moe.h); all computation runs in
the library's HIP kernels.  Tensors are passed by device pointer (torch is used
for device memory and streams only).  A missing library is an error: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_VARIANT_FIELDS = 11
# the device status word in the grouped-FFN workspace (include/moe.h)
MOE_DEVICE_STATUS_OFFSET = 0
MOE_DEV_OK, MOE_DEV_BAD_VARIANT, MOE_DEV_BAD_BLOCKS = 0, 1, 2
STATUS_NAMES = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
                -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}")
        self.status = status


class moe_problem(ctypes.Structure):  # noqa: N801  (C struct name)
    _fields_ = [("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("expert_begin", ctypes.c_int32),
                ("local_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("act_quant", ctypes.c_int32),
                ("shared_experts", ctypes.c_int32), ("packed_weights", ctypes.c_void_p)]


class moe_sizes(ctypes.Structure):  # noqa: N801
    _fields_ = [("rows_max", ctypes.c_int64), ("blocks_max", ctypes.c_int64),
                ("y_slots_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("align_ws_bytes", ctypes.c_int64)]


def problem(tokens, hidden, inter, num_experts, top_k, *, expert_begin=0, local_experts=None,
            act_dtype=MOE_BF16, weight_dtype=MOE_BF16, renormalize=1, act_quant=0,
            shared_experts=0, packed_weights=None) -> moe_problem:
    return moe_problem(tokens, hidden, inter, num_experts, expert_begin,
                       num_experts if local_experts is None else local_experts, top_k,
                       act_dtype, weight_dtype, renormalize, act_quant, shared_experts,
                       _ptr(packed_weights))


_lib = None
P = ctypes.c_void_p
_SIGS = {
    "moe_abi_version": ([], ctypes.c_int32),
    "moe_query_sizes": ([ctypes.POINTER(moe_problem), ctypes.POINTER(moe_sizes)], ctypes.c_int),
    "moe_num_variants": ([], ctypes.c_int32),
    "moe_variant_info": ([ctypes.c_int32, P], ctypes.c_int),
    "moe_cost_constants": ([ctypes.POINTER(moe_problem), P, P, P, P, P], ctypes.c_int),
    "moe_route_topk": ([ctypes.POINTER(moe_problem), P, P, P, P, P], ctypes.c_int),
    "moe_select_config": ([ctypes.POINTER(moe_problem), P, P, P, P, P], ctypes.c_int),
    "moe_align_sort": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P], ctypes.c_int),
    "moe_route_select_align": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P, P, P, P, P, P],
                               ctypes.c_int),
    "moe_grouped_ffn": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P, P, P, P, P, P, P,
                         ctypes.c_size_t, P], ctypes.c_int),
    "moe_grouped_gate_up": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P, P, P, P,
                             ctypes.c_size_t, P], ctypes.c_int),
    "moe_grouped_down": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P, P, ctypes.c_size_t, P],
                         ctypes.c_int),
    "moe_combine": ([ctypes.POINTER(moe_problem), P, P, P, P, P], ctypes.c_int),
    "moe_quant_act": ([ctypes.POINTER(moe_problem), P, P, P, P], ctypes.c_int),
    "moe_combine_shared": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P], ctypes.c_int),
    "moe_grouped_ffn_noalloc": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P, P, P, P, P, P,
                                 P], ctypes.c_int),
    "moe_noalloc_workspace_limit": ([], ctypes.c_int64),
    "moe_pack_wide_bytes": ([ctypes.POINTER(moe_problem), P], ctypes.c_int),
    "moe_pack_wide": ([ctypes.POINTER(moe_problem), P, P, P, P, P], ctypes.c_int),
    "moe_fused_workspace_bytes": ([ctypes.POINTER(moe_problem), P], ctypes.c_int),
    "moe_grouped_ffn_fused": ([ctypes.POINTER(moe_problem), P, P, P, P, P, P, P, P, P, P, P, P,
                               ctypes.c_size_t, P], ctypes.c_int),
    "moe_combine_fused": ([ctypes.POINTER(moe_problem), P, P, P, P, P], ctypes.c_int),
}


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m routing_aware_grouped_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _pp(p):
    return None if p is None else ctypes.byref(p)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoeError(fn, st)


# ---------------------------------------------------------------- queries ----
def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def moe_query_sizes(p: moe_problem) -> moe_sizes:
    out = moe_sizes()
    _check("moe_query_sizes", lib().moe_query_sizes(_pp(p), ctypes.byref(out)))
    return out


def moe_num_variants() -> int:
    return int(lib().moe_num_variants())


def moe_variant_info(v: int) -> list[int]:
    buf = (ctypes.c_int32 * MOE_VARIANT_FIELDS)()
    _check("moe_variant_info", lib().moe_variant_info(v, ctypes.cast(buf, P)))
    return list(buf)


def moe_cost_constants(p: moe_problem) -> dict:
    V = moe_num_variants()
    arrs = [(ctypes.c_int32 * V)() for _ in range(5)]
    _check("moe_cost_constants", lib().moe_cost_constants(_pp(p), *[ctypes.cast(a, P) for a in arrs]))
    return {k: list(a) for k, a in zip(("b", "q1", "q2", "S1", "S2"), arrs)}


# ------------------------------------------------------------ five steps ----
def moe_route_topk(p, logits, topk_ids, topk_w, counts, stream=None):
    _check("moe_route_topk", lib().moe_route_topk(_pp(p), _ptr(logits), _ptr(topk_ids),
                                                  _ptr(topk_w), _ptr(counts), _stream(stream)))


def moe_select_config(p, counts, theta, variant, t_hat=None, stream=None):
    _check("moe_select_config", lib().moe_select_config(_pp(p), _ptr(counts), _ptr(theta),
                                                        _ptr(variant), _ptr(t_hat), _stream(stream)))


def moe_align_sort(p, topk_ids, variant, sorted_slots, block_expert, num_blocks, slot_pos,
                   stream=None):
    _check("moe_align_sort", lib().moe_align_sort(_pp(p), _ptr(topk_ids), _ptr(variant),
                                                  _ptr(sorted_slots), _ptr(block_expert),
                                                  _ptr(num_blocks), _ptr(slot_pos), _stream(stream)))


def moe_route_select_align(p, logits, theta, topk_ids, topk_w, counts, variant, t_hat,
                           sorted_slots, block_expert, num_blocks, slot_pos, stream=None):
    _check("moe_route_select_align", lib().moe_route_select_align(
        _pp(p), _ptr(logits), _ptr(theta), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
        _ptr(variant), _ptr(t_hat), _ptr(sorted_slots), _ptr(block_expert), _ptr(num_blocks),
        _ptr(slot_pos), _stream(stream)))


def _ws_bytes(workspace, workspace_bytes):
    if workspace_bytes is None:
        return workspace.numel() * workspace.element_size()
    return int(workspace_bytes)


def moe_grouped_ffn(p, x, w1, w3, w2, s1, s3, s2, sorted_slots, block_expert, num_blocks,
                    variant, y_slots, workspace, workspace_bytes=None, stream=None):
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(
        _pp(p), _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(s1), _ptr(s3), _ptr(s2),
        _ptr(sorted_slots), _ptr(block_expert), _ptr(num_blocks), _ptr(variant), _ptr(y_slots),
        _ptr(workspace), _ws_bytes(workspace, workspace_bytes), _stream(stream)))


def moe_grouped_ffn_noalloc(p, x, w1, w3, w2, s1, s3, s2, sorted_slots, block_expert, num_blocks,
                            variant, y_slots, stream=None):
    _check("moe_grouped_ffn_noalloc", lib().moe_grouped_ffn_noalloc(
        _pp(p), _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(s1), _ptr(s3), _ptr(s2),
        _ptr(sorted_slots), _ptr(block_expert), _ptr(num_blocks), _ptr(variant), _ptr(y_slots),
        _stream(stream)))


def moe_noalloc_workspace_limit() -> int:
    return int(lib().moe_noalloc_workspace_limit())


def moe_pack_wide_bytes(p: moe_problem) -> int:
    out = ctypes.c_int64(0)
    _check("moe_pack_wide_bytes", lib().moe_pack_wide_bytes(_pp(p), ctypes.byref(out)))
    return int(out.value)


def moe_pack_wide(p, w1, w3, w2, packed, stream=None):
    _check("moe_pack_wide", lib().moe_pack_wide(_pp(p), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(packed),
                                                _stream(stream)))


def moe_grouped_gate_up(p, x, w1, w3, s1, s3, sorted_slots, block_expert, num_blocks, variant,
                        workspace, workspace_bytes=None, stream=None):
    _check("moe_grouped_gate_up", lib().moe_grouped_gate_up(
        _pp(p), _ptr(x), _ptr(w1), _ptr(w3), _ptr(s1), _ptr(s3), _ptr(sorted_slots),
        _ptr(block_expert), _ptr(num_blocks), _ptr(variant), _ptr(workspace),
        _ws_bytes(workspace, workspace_bytes), _stream(stream)))


def moe_grouped_down(p, w2, s2, sorted_slots, block_expert, num_blocks, variant, y_slots,
                     workspace, workspace_bytes=None, stream=None):
    _check("moe_grouped_down", lib().moe_grouped_down(
        _pp(p), _ptr(w2), _ptr(s2), _ptr(sorted_slots), _ptr(block_expert), _ptr(num_blocks),
        _ptr(variant), _ptr(y_slots), _ptr(workspace), _ws_bytes(workspace, workspace_bytes),
        _stream(stream)))


def moe_quant_act(p, x, xq, xs, stream=None):
    _check("moe_quant_act", lib().moe_quant_act(_pp(p), _ptr(x), _ptr(xq), _ptr(xs),
                                                _stream(stream)))


def moe_combine_shared(p, y_slots, slot_pos, topk_w, num_blocks, variant, y, stream=None):
    _check("moe_combine_shared", lib().moe_combine_shared(
        _pp(p), _ptr(y_slots), _ptr(slot_pos), _ptr(topk_w), _ptr(num_blocks), _ptr(variant),
        _ptr(y), _stream(stream)))


def moe_combine(p, y_slots, slot_pos, topk_w, y, stream=None):
    _check("moe_combine", lib().moe_combine(_pp(p), _ptr(y_slots), _ptr(slot_pos),
                                            _ptr(topk_w), _ptr(y), _stream(stream)))


# ------------------------------------------------- the fused small-batch plan --
def moe_fused_workspace_bytes(p: moe_problem) -> int:
    out = ctypes.c_int64(0)
    _check("moe_fused_workspace_bytes", lib().moe_fused_workspace_bytes(_pp(p), ctypes.byref(out)))
    return int(out.value)


def moe_grouped_ffn_fused(p, x, w1, w3, w2, s1, s3, s2, sorted_slots, block_expert, num_blocks,
                          variant, fused_ws, fused_ws_bytes=None, stream=None):
    _check("moe_grouped_ffn_fused", lib().moe_grouped_ffn_fused(
        _pp(p), _ptr(x), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(s1), _ptr(s3), _ptr(s2),
        _ptr(sorted_slots), _ptr(block_expert), _ptr(num_blocks), _ptr(variant), _ptr(fused_ws),
        _ws_bytes(fused_ws, fused_ws_bytes), _stream(stream)))


def moe_combine_fused(p, fused_ws, slot_pos, topk_w, y, stream=None):
    _check("moe_combine_fused", lib().moe_combine_fused(_pp(p), _ptr(fused_ws), _ptr(slot_pos),
                                                        _ptr(topk_w), _ptr(y), _stream(stream)))


__all__ = [n for n in dir() if n.startswith("moe_") or n.startswith("MOE_")] + [
    "MoeError", "problem", "lib", "LIB_PATH"]
