"""Python binding of libmoe_mi355x.so, the fused-MoE expert computation for
one MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/moe_mi355x.h``.  torch supplies device
memory and the stream.  The functions carry the C names.  Loading fails
loudly when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "ABI_VERSION", "LAYOUT_CONTIGUOUS", "LAYOUT_BATCHED", "W_BF16", "W_MXFP8", "W1_HALVES",
    "W1_INTERLEAVE16", "VARIANT_AUTO", "VARIANT_TILE", "VARIANT_STREAM", "VARIANT_FUSED", "REDUCE_NOOP",
    "REDUCE_CONTIGUOUS", "REDUCE_NAIVE_BATCHED", "MoeError", "MoeProblem", "MoePlan", "MoeWeights",
    "load_library", "library_path", "moe_abi_version", "moe_status_string", "moe_plan_init",
    "moe_plan_reason", "moe_align_permute", "moe_apply_contiguous", "moe_apply_batched",
    "moe_gate_up_act", "moe_down_unpermute",
    "moe_topk_reduce_contiguous", "moe_naive_batched_ws_bytes", "moe_topk_reduce_naive_batched",
    "moe_quantize_mxfp8", "make_problem", "allocate_workspaces", "ws_view",
    "MoeGroupedProblem", "moe_grouped_forward", "moe_grouped_dgrad", "moe_grouped_wgrad",
]

ABI_VERSION = 4
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP = 0, 1, 2, 3
LAYOUT_CONTIGUOUS, LAYOUT_BATCHED = 0, 1
W_BF16, W_MXFP8 = 0, 1
W1_HALVES, W1_INTERLEAVE16 = 0, 1
VARIANT_AUTO, VARIANT_TILE, VARIANT_STREAM, VARIANT_FUSED = -1, 0, 1, 2
REDUCE_NOOP, REDUCE_CONTIGUOUS, REDUCE_NAIVE_BATCHED = 0, 1, 2

_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p


class MoeProblem(ctypes.Structure):
    _fields_ = [("M", _i64), ("K", _i64), ("I", _i64), ("E", _i64), ("topk", _i64),
                ("max_tokens", _i64), ("global_experts", _i64), ("layout", _i32), ("w_dtype", _i32),
                ("w1_order", _i32), ("variant", _i32)]


class MoeGroupedProblem(ctypes.Structure):
    _fields_ = [("R", _i64), ("N", _i64), ("K", _i64), ("E", _i64)]


class MoePlan(ctypes.Structure):
    _fields_ = [("prob", MoeProblem), ("abi_version", _i32), ("variant", _i32), ("block_m", _i32),
                ("reduce_kind", _i32), ("routes", _i64), ("sorted_capacity", _i64),
                ("max_tiles", _i64), ("max_active", _i64), ("align_blocks", _i64),
                ("ws13_bytes", _i64), ("ws2_bytes", _i64), ("out_rows", _i64), ("out_cols", _i64),
                ("off_counts", _i64), ("off_offsets", _i64), ("off_sorted_ids", _i64),
                ("off_block_expert", _i64), ("off_num_post_padded", _i64), ("off_active", _i64),
                ("off_status", _i64), ("off_align_scratch", _i64), ("off_z", _i64),
                ("off_z_scale", _i64), ("off_xq", _i64), ("off_xq_scale", _i64), ("off_sync", _i64),
                ("reason", ctypes.c_char * 192)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w1", _vp), ("w1_scale", _vp), ("w2", _vp), ("w2_scale", _vp), ("expert_map", _vp)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, reason: str = ""):
        self.status = status
        msg = f"{fn}: {_status_name(status)}"
        if reason:
            msg += f" ({reason})"
        super().__init__(msg)


_LIB: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")


def load_library() -> ctypes.CDLL:
    """Load the in-tree library (once).  Raises if it is missing or stale."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run mixture_experts_expert_align_amd/build.py "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    sig = {
        "moe_abi_version": (_i32, []),
        "moe_status_string": (ctypes.c_char_p, [_i32]),
        "moe_struct_sizes": (None, [_vp, _vp, _vp]),
        "moe_plan_init": (_i32, [_vp, _vp]),
        "moe_plan_reason": (ctypes.c_char_p, [_vp]),
        "moe_align_permute": (_i32, [_vp] * 5),
        "moe_apply_contiguous": (_i32, [_vp] * 9),
        "moe_apply_batched": (_i32, [_vp] * 7),
        "moe_gate_up_act": (_i32, [_vp] * 5),
        "moe_down_unpermute": (_i32, [_vp] * 5),
        "moe_topk_reduce_contiguous": (_i32, [_vp] * 7),
        "moe_naive_batched_ws_bytes": (_i64, [_vp, _i64]),
        "moe_topk_reduce_naive_batched": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
        "moe_quantize_mxfp8": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _vp]),
        "moe_grouped_forward": (_i32, [_vp] * 6),
        "moe_grouped_dgrad": (_i32, [_vp] * 6),
        "moe_grouped_wgrad": (_i32, [_vp] * 5 + [_i32, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    v = lib.moe_abi_version()
    if v != ABI_VERSION:
        raise RuntimeError(f"{path}: ABI version {v}, binding expects {ABI_VERSION}; rebuild it")
    sizes = [ctypes.c_int64() for _ in range(3)]
    lib.moe_struct_sizes(*[ctypes.byref(s) for s in sizes])
    want = [ctypes.sizeof(MoeProblem), ctypes.sizeof(MoePlan), ctypes.sizeof(MoeWeights)]
    if [s.value for s in sizes] != want:
        raise RuntimeError(f"struct layout mismatch: library {[s.value for s in sizes]}, binding {want}")
    _LIB = lib
    return lib


def _status_name(status: int) -> str:
    return {0: "ok", 1: "invalid argument", 2: "unsupported problem", 3: "HIP launch error"}.get(
        status, f"status {status}")


def _check(fn: str, status: int, plan: Optional[MoePlan] = None):
    if status != MOE_OK:
        raise MoeError(fn, status, plan.reason.decode() if plan is not None else "")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ calls --

def moe_abi_version() -> int:
    return load_library().moe_abi_version()


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def make_problem(M, K, I, E, topk=0, max_tokens=0, layout=LAYOUT_CONTIGUOUS, w_dtype=W_BF16,
                 w1_order=W1_HALVES, variant=VARIANT_AUTO, global_experts=0) -> MoeProblem:
    return MoeProblem(M, K, I, E, topk, max_tokens, global_experts, layout, w_dtype, w1_order, variant)


def moe_plan_init(prob: MoeProblem) -> MoePlan:
    plan = MoePlan()
    st = load_library().moe_plan_init(ctypes.byref(plan), ctypes.byref(prob))
    _check("moe_plan_init", st, plan)
    return plan


def moe_plan_reason(plan: MoePlan) -> str:
    return load_library().moe_plan_reason(ctypes.byref(plan)).decode()


def allocate_workspaces(plan: MoePlan, device="cuda"):
    """ws13 and ws2 as uint8 device tensors of the sizes the plan states
    (ws13 zero-filled: the single-launch variant keeps its counters there)."""
    ws13 = torch.zeros(max(plan.ws13_bytes, 16), dtype=torch.uint8, device=device)
    ws2 = torch.empty(max(plan.ws2_bytes, 16), dtype=torch.uint8, device=device)
    return ws13, ws2


def ws_view(ws: torch.Tensor, offset: int, count: int, dtype=torch.int32) -> torch.Tensor:
    """A typed view of ``count`` elements at byte ``offset`` of a workspace."""
    nbytes = count * torch.empty((), dtype=dtype).element_size()
    return ws[offset: offset + nbytes].view(dtype)


def moe_align_permute(plan: MoePlan, topk_ids: torch.Tensor, ws13: torch.Tensor, stream=None,
                      expert_map: Optional[torch.Tensor] = None):
    st = load_library().moe_align_permute(ctypes.byref(plan), _ptr(topk_ids), _ptr(expert_map),
                                          _ptr(ws13), _stream(stream))
    _check("moe_align_permute", st)


def _weights(w1, w2, w1_scale=None, w2_scale=None, expert_map=None) -> MoeWeights:
    return MoeWeights(_ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(expert_map))


def moe_apply_contiguous(plan: MoePlan, a, topk_ids, topk_weights, w1, w2, out, ws13, ws2,
                         w1_scale=None, w2_scale=None, stream=None, expert_map=None):
    w = _weights(w1, w2, w1_scale, w2_scale, expert_map)
    st = load_library().moe_apply_contiguous(
        ctypes.byref(plan), _ptr(a), _ptr(topk_ids), _ptr(topk_weights), ctypes.byref(w), _ptr(out),
        _ptr(ws13), _ptr(ws2), _stream(stream))
    _check("moe_apply_contiguous", st)


def moe_gate_up_act(plan: MoePlan, a, w1, w2, ws13, w1_scale=None, w2_scale=None, stream=None):
    w = _weights(w1, w2, w1_scale, w2_scale)
    st = load_library().moe_gate_up_act(ctypes.byref(plan), _ptr(a), ctypes.byref(w), _ptr(ws13),
                                        _stream(stream))
    _check("moe_gate_up_act", st)


def moe_down_unpermute(plan: MoePlan, w1, w2, ws13, ws2, w1_scale=None, w2_scale=None, stream=None):
    w = _weights(w1, w2, w1_scale, w2_scale)
    st = load_library().moe_down_unpermute(ctypes.byref(plan), ctypes.byref(w), _ptr(ws13),
                                           _ptr(ws2), _stream(stream))
    _check("moe_down_unpermute", st)


def moe_apply_batched(plan: MoePlan, a, expert_num_tokens, w1, w2, y, ws13, stream=None):
    w = _weights(w1, w2)
    st = load_library().moe_apply_batched(ctypes.byref(plan), _ptr(a), _ptr(expert_num_tokens),
                                          ctypes.byref(w), _ptr(y), _ptr(ws13), _stream(stream))
    _check("moe_apply_batched", st)


def moe_topk_reduce_contiguous(plan: MoePlan, y, topk_ids, topk_weights, out, stream=None,
                               expert_map: Optional[torch.Tensor] = None):
    st = load_library().moe_topk_reduce_contiguous(ctypes.byref(plan), _ptr(y), _ptr(topk_ids),
                                                   _ptr(topk_weights), _ptr(expert_map), _ptr(out),
                                                   _stream(stream))
    _check("moe_topk_reduce_contiguous", st)


def moe_naive_batched_ws_bytes(plan: MoePlan, n_out: int) -> int:
    v = load_library().moe_naive_batched_ws_bytes(ctypes.byref(plan), n_out)
    if v < 0:
        raise MoeError("moe_naive_batched_ws_bytes", MOE_EINVAL)
    return v


def moe_topk_reduce_naive_batched(plan: MoePlan, y, expert_num_tokens, row_token, row_weight,
                                  n_out: int, out, ws, stream=None):
    st = load_library().moe_topk_reduce_naive_batched(
        ctypes.byref(plan), _ptr(y), _ptr(expert_num_tokens), _ptr(row_token), _ptr(row_weight),
        n_out, _ptr(out), _ptr(ws), _stream(stream))
    _check("moe_topk_reduce_naive_batched", st)


def moe_quantize_mxfp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    rows = x.numel() // x.shape[-1]
    st = load_library().moe_quantize_mxfp8(_ptr(x), 0 if x.dtype == torch.float32 else 1, rows,
                                           x.shape[-1], _ptr(codes), _ptr(scales), _stream(stream))
    _check("moe_quantize_mxfp8", st)


# ------------------------------------------------------------- training ----

def _grouped(R, N, K, E) -> MoeGroupedProblem:
    return MoeGroupedProblem(R=R, N=N, K=K, E=E)


def moe_grouped_forward(x, w, group_offsets, y, stream=None):
    """y[r] = W[e] x[r] over the rows of each group (x [R,K], w [E,N,K], y [R,N] bf16)."""
    p = _grouped(x.shape[0], w.shape[1], w.shape[2], w.shape[0])
    st = load_library().moe_grouped_forward(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(group_offsets),
                                            _ptr(y), _stream(stream))
    _check("moe_grouped_forward", st)


def moe_grouped_dgrad(dy, w, group_offsets, dx, stream=None):
    """dx[r] = W[e]^T dy[r] (dy [R,N], w [E,N,K], dx [R,K] bf16)."""
    p = _grouped(dy.shape[0], w.shape[1], w.shape[2], w.shape[0])
    st = load_library().moe_grouped_dgrad(ctypes.byref(p), _ptr(dy), _ptr(w), _ptr(group_offsets),
                                          _ptr(dx), _stream(stream))
    _check("moe_grouped_dgrad", st)


def moe_grouped_wgrad(dy, x, group_offsets, dw, accumulate: bool = False, stream=None):
    """dW[e] = sum over group e's rows of dy[r] x[r]^T into dw [E,N,K] float32
    (written, or added when ``accumulate``)."""
    p = _grouped(dy.shape[0], dw.shape[1], dw.shape[2], dw.shape[0])
    st = load_library().moe_grouped_wgrad(ctypes.byref(p), _ptr(dy), _ptr(x), _ptr(group_offsets),
                                          _ptr(dw), 1 if accumulate else 0, _stream(stream))
    _check("moe_grouped_wgrad", st)

