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
    "ABI_VERSION", "LAYOUT_CONTIGUOUS", "LAYOUT_BATCHED", "W_BF16", "W_MXFP8", "W_MXFP8_GROUPED", "W1_HALVES",
    "W1_INTERLEAVE16", "VARIANT_AUTO", "VARIANT_TILE", "VARIANT_STREAM", "VARIANT_FUSED", "REDUCE_NOOP",
    "REDUCE_CONTIGUOUS", "REDUCE_NAIVE_BATCHED", "MoeError", "MoeProblem", "MoePlan", "MoeWeights",
    "load_library", "library_path", "moe_abi_version", "moe_status_string", "moe_plan_init",
    "moe_apply_contiguous_static", "STATIC_SCRATCH_BYTES",
    "moe_plan_reason", "moe_align_permute", "moe_apply_contiguous", "moe_apply_batched",
    "moe_gate_up_act", "moe_down_unpermute",
    "moe_topk_reduce_contiguous", "moe_naive_batched_ws_bytes", "moe_topk_reduce_naive_batched",
    "moe_quantize_mxfp8", "moe_pack_mxfp8_scales", "make_problem", "allocate_workspaces", "ws_view", "status_words",
    "check_status",
    "MoeGroupedProblem", "moe_grouped_forward", "moe_grouped_dgrad", "moe_grouped_wgrad",
]

ABI_VERSION = 5
STATIC_SCRATCH_BYTES = 64 << 20     # MOE_STATIC_SCRATCH_BYTES
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP = 0, 1, 2, 3
LAYOUT_CONTIGUOUS, LAYOUT_BATCHED = 0, 1
W_BF16, W_MXFP8, W_MXFP8_GROUPED = 0, 1, 2
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
        "moe_apply_contiguous_static": (_i32, [_vp] * 7),
        "moe_apply_batched": (_i32, [_vp] * 7),
        "moe_gate_up_act": (_i32, [_vp] * 5),
        "moe_down_unpermute": (_i32, [_vp] * 5),
        "moe_topk_reduce_contiguous": (_i32, [_vp] * 7),
        "moe_naive_batched_ws_bytes": (_i64, [_vp, _i64]),
        "moe_topk_reduce_naive_batched": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]),
        "moe_quantize_mxfp8": (_i32, [_vp, _i32, _i64, _i64, _vp, _vp, _vp]),
        "moe_pack_mxfp8_scales": (_i32, [_vp, _vp, _i64, _i64, _i64, _vp]),
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


def _arg(t: Optional[torch.Tensor], name: str, dtypes, numel: int) -> Optional[int]:
    """Device pointer of ``t`` after checking its dtype and that it holds at
    least ``numel`` elements (the kernels read or write that many)."""
    if t is None:
        return None
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the call needs {numel}")
    return _ptr(t)


def _ws(t: torch.Tensor, name: str, nbytes: int) -> int:
    """A workspace: any dtype, at least ``nbytes`` bytes."""
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, the plan needs {nbytes}")
    return _ptr(t)


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


def _ids_arg(plan: MoePlan, topk_ids: torch.Tensor, name="topk_ids") -> int:
    p = plan.prob
    if topk_ids.dtype != torch.int32:
        raise ValueError(f"{name}: dtype {topk_ids.dtype}, expected torch.int32 (e.g. topk ids .int())")
    if topk_ids.numel() != p.M * p.topk:
        raise ValueError(f"{name}: {topk_ids.numel()} elements, expected M*topk = {p.M * p.topk}")
    return _ptr(topk_ids)


def _map_arg(plan: MoePlan, expert_map: Optional[torch.Tensor]) -> Optional[int]:
    return _arg(expert_map, "expert_map", torch.int32, plan.prob.global_experts)


def status_words(plan: MoePlan, ws13: torch.Tensor):
    """(ids outside {-1} U [0,E) seen by the last align, waits of the
    single-launch variant that timed out, summed over calls) from the status
    words in ws13.  Synchronises with the device (a copy to the host)."""
    w = ws_view(ws13, plan.off_status, 2).cpu()
    return int(w[0]), int(w[1])


def check_status(plan: MoePlan, ws13: torch.Tensor):
    """Raise MoeError when a single-launch call on this ws13 gave up a bounded
    wait (its outputs are then undefined).  The count stays until ws13 is
    cleared, so every later check fails too."""
    _, timeouts = status_words(plan, ws13)
    if timeouts:
        raise MoeError("moe_apply_contiguous", MOE_EHIP,
                       f"{timeouts} bounded waits of the single-launch kernel timed out; outputs undefined")


def moe_align_permute(plan: MoePlan, topk_ids: torch.Tensor, ws13: torch.Tensor, stream=None,
                      expert_map: Optional[torch.Tensor] = None):
    st = load_library().moe_align_permute(ctypes.byref(plan), _ids_arg(plan, topk_ids),
                                          _map_arg(plan, expert_map), _ws(ws13, "ws13", plan.ws13_bytes),
                                          _stream(stream))
    _check("moe_align_permute", st)


def _weights(plan: MoePlan, w1, w2, w1_scale=None, w2_scale=None, expert_map=None) -> MoeWeights:
    p = plan.prob
    mx = p.w_dtype in (W_MXFP8, W_MXFP8_GROUPED)
    wt = torch.uint8 if mx else torch.bfloat16
    n1, n2 = p.E * 2 * p.I * p.K, p.E * p.K * p.I
    if mx and (w1_scale is None or w2_scale is None):
        raise ValueError("MXFP8 weights need w1_scale and w2_scale")
    return MoeWeights(_arg(w1, "w1", wt, n1), _arg(w1_scale, "w1_scale", torch.uint8, n1 // 32 if mx else 0),
                      _arg(w2, "w2", wt, n2), _arg(w2_scale, "w2_scale", torch.uint8, n2 // 32 if mx else 0),
                      _map_arg(plan, expert_map))


def moe_apply_contiguous(plan: MoePlan, a, topk_ids, topk_weights, w1, w2, out, ws13, ws2,
                         w1_scale=None, w2_scale=None, stream=None, expert_map=None):
    w = _weights(plan, w1, w2, w1_scale, w2_scale, expert_map)
    p = plan.prob
    st = load_library().moe_apply_contiguous(
        ctypes.byref(plan), _arg(a, "a", torch.bfloat16, p.M * p.K), _ids_arg(plan, topk_ids),
        _arg(topk_weights, "topk_weights", torch.float32, p.M * p.topk), ctypes.byref(w),
        _arg(out, "out", torch.bfloat16, p.M * p.K), _ws(ws13, "ws13", plan.ws13_bytes),
        _ws(ws2, "ws2", plan.ws2_bytes), _stream(stream))
    _check("moe_apply_contiguous", st)


def moe_apply_contiguous_static(plan: MoePlan, a, topk_ids, topk_weights, w1, w2, out, w1_scale=None,
                                w2_scale=None, stream=None, expert_map=None):
    """moe_apply_contiguous with the workspaces inside the library's own
    per-GPU array (no allocation by anyone; calls that overlap on one GPU
    race).  Raises MoeError(MOE_EUNSUPPORTED) when the plan's workspaces do
    not fit in STATIC_SCRATCH_BYTES."""
    w = _weights(plan, w1, w2, w1_scale, w2_scale, expert_map)
    p = plan.prob
    st = load_library().moe_apply_contiguous_static(
        ctypes.byref(plan), _arg(a, "a", torch.bfloat16, p.M * p.K), _ids_arg(plan, topk_ids),
        _arg(topk_weights, "topk_weights", torch.float32, p.M * p.topk), ctypes.byref(w),
        _arg(out, "out", torch.bfloat16, p.M * p.K), _stream(stream))
    _check("moe_apply_contiguous_static", st)


def moe_gate_up_act(plan: MoePlan, a, w1, w2, ws13, w1_scale=None, w2_scale=None, stream=None):
    w = _weights(plan, w1, w2, w1_scale, w2_scale)
    st = load_library().moe_gate_up_act(ctypes.byref(plan), _arg(a, "a", torch.bfloat16, plan.prob.M * plan.prob.K),
                                        ctypes.byref(w), _ws(ws13, "ws13", plan.ws13_bytes), _stream(stream))
    _check("moe_gate_up_act", st)


def moe_down_unpermute(plan: MoePlan, w1, w2, ws13, ws2, w1_scale=None, w2_scale=None, stream=None):
    w = _weights(plan, w1, w2, w1_scale, w2_scale)
    st = load_library().moe_down_unpermute(ctypes.byref(plan), ctypes.byref(w), _ws(ws13, "ws13", plan.ws13_bytes),
                                           _ws(ws2, "ws2", plan.ws2_bytes), _stream(stream))
    _check("moe_down_unpermute", st)


def moe_apply_batched(plan: MoePlan, a, expert_num_tokens, w1, w2, y, ws13, stream=None):
    w = _weights(plan, w1, w2)
    p = plan.prob
    slab = p.E * p.max_tokens * p.K
    st = load_library().moe_apply_batched(ctypes.byref(plan), _arg(a, "a", torch.bfloat16, slab),
                                          _arg(expert_num_tokens, "expert_num_tokens", torch.int32, p.E),
                                          ctypes.byref(w), _arg(y, "y", torch.bfloat16, slab),
                                          _ws(ws13, "ws13", plan.ws13_bytes), _stream(stream))
    _check("moe_apply_batched", st)


def moe_topk_reduce_contiguous(plan: MoePlan, y, topk_ids, topk_weights, out, stream=None,
                               expert_map: Optional[torch.Tensor] = None):
    p = plan.prob
    st = load_library().moe_topk_reduce_contiguous(ctypes.byref(plan), _arg(y, "y", torch.bfloat16, p.M * p.topk * p.K),
                                                   _ids_arg(plan, topk_ids),
                                                   _arg(topk_weights, "topk_weights", torch.float32, p.M * p.topk),
                                                   _map_arg(plan, expert_map),
                                                   _arg(out, "out", torch.bfloat16, p.M * p.K), _stream(stream))
    _check("moe_topk_reduce_contiguous", st)


def moe_naive_batched_ws_bytes(plan: MoePlan, n_out: int) -> int:
    v = load_library().moe_naive_batched_ws_bytes(ctypes.byref(plan), n_out)
    if v < 0:
        raise MoeError("moe_naive_batched_ws_bytes", MOE_EINVAL)
    return v


def moe_topk_reduce_naive_batched(plan: MoePlan, y, expert_num_tokens, row_token, row_weight,
                                  n_out: int, out, ws, stream=None):
    p = plan.prob
    rows = p.E * p.max_tokens
    st = load_library().moe_topk_reduce_naive_batched(
        ctypes.byref(plan), _arg(y, "y", torch.bfloat16, rows * p.K),
        _arg(expert_num_tokens, "expert_num_tokens", torch.int32, p.E),
        _arg(row_token, "row_token", torch.int32, rows), _arg(row_weight, "row_weight", torch.float32, rows),
        n_out, _arg(out, "out", torch.bfloat16, n_out * p.K),
        _ws(ws, "ws", moe_naive_batched_ws_bytes(plan, n_out)), _stream(stream))
    _check("moe_topk_reduce_naive_batched", st)


def moe_quantize_mxfp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None):
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    rows = x.numel() // x.shape[-1]
    st = load_library().moe_quantize_mxfp8(_ptr(x), 0 if x.dtype == torch.float32 else 1, rows,
                                           x.shape[-1], _arg(codes, "codes", torch.uint8, x.numel()),
                                           _arg(scales, "scales", torch.uint8, x.numel() // 32),
                                           _stream(stream))
    _check("moe_quantize_mxfp8", st)


def moe_pack_mxfp8_scales(scales: torch.Tensor, packed: torch.Tensor, stream=None):
    """Row-major MXFP8 scale arrays ``[..., rows, cols/32]`` (as
    moe_quantize_mxfp8 writes them) into ``packed`` (same size) in the layout
    of W_MXFP8_GROUPED: each matrix of the last two dimensions in groups of
    16 bytes a row."""
    if scales.dim() < 2:
        raise ValueError("scales: expected [..., rows, cols/32]")
    rows, ncols = scales.shape[-2], scales.shape[-1] * 32
    mats = scales.numel() // max(rows * scales.shape[-1], 1)
    st = load_library().moe_pack_mxfp8_scales(_arg(scales, "scales", torch.uint8, scales.numel()),
                                              _arg(packed, "packed", torch.uint8, scales.numel()),
                                              mats, rows, ncols, _stream(stream))
    _check("moe_pack_mxfp8_scales", st)


# ------------------------------------------------------------- training ----

def _grouped(R, N, K, E) -> MoeGroupedProblem:
    return MoeGroupedProblem(R=R, N=N, K=K, E=E)


def moe_grouped_forward(x, w, group_offsets, y, stream=None):
    """y[r] = W[e] x[r] over the rows of each group (x [R,K], w [E,N,K], y [R,N] bf16)."""
    p = _grouped(x.shape[0], w.shape[1], w.shape[2], w.shape[0])
    st = load_library().moe_grouped_forward(ctypes.byref(p), _arg(x, "x", torch.bfloat16, p.R * p.K),
                                            _arg(w, "w", torch.bfloat16, p.E * p.N * p.K),
                                            _arg(group_offsets, "group_offsets", torch.int32, p.E + 1),
                                            _arg(y, "y", torch.bfloat16, p.R * p.N), _stream(stream))
    _check("moe_grouped_forward", st)


def moe_grouped_dgrad(dy, w, group_offsets, dx, stream=None):
    """dx[r] = W[e]^T dy[r] (dy [R,N], w [E,N,K], dx [R,K] bf16)."""
    p = _grouped(dy.shape[0], w.shape[1], w.shape[2], w.shape[0])
    st = load_library().moe_grouped_dgrad(ctypes.byref(p), _arg(dy, "dy", torch.bfloat16, p.R * p.N),
                                          _arg(w, "w", torch.bfloat16, p.E * p.N * p.K),
                                          _arg(group_offsets, "group_offsets", torch.int32, p.E + 1),
                                          _arg(dx, "dx", torch.bfloat16, p.R * p.K), _stream(stream))
    _check("moe_grouped_dgrad", st)


def moe_grouped_wgrad(dy, x, group_offsets, dw, accumulate: bool = False, stream=None):
    """dW[e] = sum over group e's rows of dy[r] x[r]^T into dw [E,N,K] float32
    (written, or added when ``accumulate``)."""
    p = _grouped(dy.shape[0], dw.shape[1], dw.shape[2], dw.shape[0])
    st = load_library().moe_grouped_wgrad(ctypes.byref(p), _arg(dy, "dy", torch.bfloat16, p.R * p.N),
                                          _arg(x, "x", torch.bfloat16, p.R * p.K),
                                          _arg(group_offsets, "group_offsets", torch.int32, p.E + 1),
                                          _arg(dw, "dw", torch.float32, p.E * p.N * p.K),
                                          1 if accumulate else 0, _stream(stream))
    _check("moe_grouped_wgrad", st)

