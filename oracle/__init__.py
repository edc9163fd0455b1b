"""CPU oracle for the fused-MoE expert computation.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (the HIP library and its Python binding) never does, and shares
no code with this module.

Plain, slow and meant to be checked by eye: numpy, float64 for every floating
point step (bf16 and E4M3 inputs decode exactly into float64), library matmuls
as the only building block beyond elementwise numpy.  Each function names the
passage of the pages it restates:

* [MK]   "Fused MoE Modular Kernel" (vLLM design doc): introduction (contiguous
         and batched activation formats), "TopKWeightAndReduce",
         "FusedMoEExpertsModular / apply()".
* [CAKE] "FlashInfer: Cake MegaMoE EP16 backend for BF16 activations and MXFP8
         weights" (PR 5148 analysis): section 1 (routing), section 2 (gate/up
         interleave by 16, the block-32 MXFP8 scale rule), section 3 (FC2 results
         written per (token, top-k slot); ordered Top-K reduce).
* [MEGA] "DeepGEMM Mega MoE as an EP implementation" (transformers PR 49606
         analysis), section 2: padded slots carry expert id -1 and weight 0.
* [DET]  "Cake deterministic MoE grouped GEMM" (FlashInfer PR 9132 analysis):
         introduction (a ragged bf16 grouped GEMM for training: forward, dgrad,
         wgrad; the fp32 weight-gradient accumulate into main_grad), section 1
         (the fused accumulate equals out.add_(dW)), section 2 (an empty sum is
         +0.0, so an empty group turns -0.0 into +0.0).

Readings where the pages are silent (each also listed in the design notes):
* W1 rows [0, I) are the gate projection and [I, 2I) the up projection
  ("halves"), unless the interleave-16 layout is named.
* silu(v) = v / (1 + exp(-v)); the activation is silu(gate) * up.
* Top-k weights multiply the W2 output (weight application follows Unpermute in
  the apply() step list).
* The MXFP8 scale exponent is the exact ceil(log2(blockmax / 448)), i.e. the
  smallest integer e with 448 * 2^e >= blockmax; the page's expression evaluated
  in float32 can be one too small just above a power of two.
* The align step pads each expert's run of routes to a multiple of the tile
  size B with the sentinel M*topk; routes keep ascending flat (t*topk + j) order
  within an expert; ids outside {-1} U [0, E) are skipped and counted.
* With global expert ids, the map is applied first (``map_expert_ids``) and the
  steps then run on local ids; a slot whose expert another GPU holds is
  skipped without being counted as invalid.
* Training grouped GEMMs: rows are grouped by expert, group e being rows
  [offsets[e], offsets[e+1]) of the row-major operands; the weight of expert e
  is W[e] [N, K] and the forward is y = x W[e]^T, so dgrad is dy W[e] and wgrad
  sums dy^T x over the group's rows.  The accumulate adds that sum to the fp32
  buffer once.

parity pins: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, library special cases, brute force, invariants); none is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Iterable, Optional

import numpy as np

__all__ = [
    "bf16_to_f64", "e4m3fn_table", "e4m3fn_encode", "mx_scale_exponent", "mx_scale_code",
    "mxfp8_quantize", "mxfp8_dequantize", "split_gate_up", "silu", "expert_ffn",
    "align_permute", "moe_contiguous", "moe_routes", "topk_reduce_contiguous",
    "moe_batched_rows", "naive_batched_reduce", "grouped_forward", "grouped_dgrad",
    "grouped_wgrad", "grouped_wgrad_accumulate",
]

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of
    an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (OCP FP8: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN,
    exponent field 0 encodes subnormals m/8 * 2^-6).  Largest finite is 448."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        ef = (c >> 3) & 0xF
        m = c & 0x7
        if ef == 0xF and m == 0x7:
            vals[c] = np.nan
        elif ef == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (ef - 7)
    return vals


_E4M3 = e4m3fn_table()


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Round float64 values with |v| <= 448 to the nearest E4M3FN code, ties to
    the even code (even mantissa), keeping the sign bit of v (so -0.0 and
    negative values that round to zero give 0x80).

    The finite E4M3FN magnitudes are a uniform grid: step 2^-9 on [0, 2^-6]
    (subnormals, then the first normal binade has the same step) and step
    2^(E-3) on each binade [2^E, 2^(E+1)), E = -6..8.  |v|'s neighbours on its
    grid are k*step and (k+1)*step with k = floor(|v|/step); the nearer one
    wins, a tie goes to even k.  Code = 8*(E+7) + k - 8 (k = 16 is the first
    value of the next binade, which the same formula encodes)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("e4m3fn_encode: value outside the finite E4M3FN range")
    _, p = np.frexp(a)                                   # a = f * 2^p, f in [0.5, 1)
    E = np.where(a < 2.0 ** -6, -6, p - 1).astype(np.int32)
    q = a / np.ldexp(1.0, E - 3)                         # |v| in grid steps; exact
    k = np.floor(q)
    r = q - k                                            # distance past the lower neighbour
    ki = k.astype(np.int64)
    ki += (r > 0.5) | ((r == 0.5) & ((ki & 1) == 1))
    code = (8 * (E.astype(np.int64) + 7) + ki - 8).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def mx_scale_exponent(blockmax: np.ndarray) -> np.ndarray:
    """Smallest integer e with 448 * 2^e >= blockmax (blockmax > 0), computed
    exactly: frexp gives a first guess, exact power-of-two comparisons fix it.
    [CAKE] section 2, the new scale rule ceil(log2(blockmax / 448))."""
    bm = np.asarray(blockmax, dtype=np.float64)
    _, p = np.frexp(bm)                       # bm = f * 2^p, f in [0.5, 1)
    e = p.astype(np.int64) - 9                # 448*2^(p-9) = 0.875*2^p: may be < bm
    for _ in range(3):
        e = np.where(np.ldexp(E4M3_MAX, e) < bm, e + 1, e)
    for _ in range(3):
        e = np.where(np.ldexp(E4M3_MAX, e - 1) >= bm, e - 1, e)
    return e


def mx_scale_code(blockmax: np.ndarray) -> np.ndarray:
    """UE8M0 scale code of a block: clamp(e + 127, 0, 254) with e from
    ``mx_scale_exponent``; 0 for an all-zero block.  [CAKE] section 2."""
    bm = np.asarray(blockmax, dtype=np.float64)
    safe = np.where(bm > 0, bm, 1.0)
    code = np.clip(mx_scale_exponent(safe) + 127, 0, 254)
    return np.where(bm > 0, code, 0).astype(np.uint8)


def mxfp8_quantize(x: np.ndarray):
    """MXFP8 encoding along the last axis in blocks of 32 [CAKE] section 2.

    x: float array [..., n] with n % 32 == 0 (float32 or bf16-decoded values).
    Returns (codes uint8 [..., n], scales uint8 [..., n/32]) with
    decoded value = E4M3(code) * 2^(scale - 127).  Blocks are independent;
    rows are taken a slab at a time only to keep temporaries small."""
    x = np.asarray(x)
    n = x.shape[-1]
    if n % 32:
        raise ValueError("mxfp8_quantize: last dimension must be a multiple of 32")
    flat = x.reshape(-1, n)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty((flat.shape[0], n // 32), dtype=np.uint8)
    step = max(1, (1 << 19) // n)
    for r0 in range(0, flat.shape[0], step):
        blocks = flat[r0:r0 + step].astype(np.float64).reshape(-1, n // 32, 32)
        bm = np.abs(blocks).max(axis=-1)
        sc = mx_scale_code(bm)
        s = np.ldexp(1.0, sc.astype(np.int32) - 127)
        codes[r0:r0 + step] = e4m3fn_encode(blocks / s[..., None]).reshape(-1, n)  # exact division
        scales[r0:r0 + step] = sc
    return codes.reshape(x.shape), scales.reshape(*x.shape[:-1], n // 32)


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    v = _E4M3[codes].reshape(*codes.shape[:-1], n // 32, 32)
    s = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (v * s[..., None]).reshape(codes.shape)


# --------------------------------------------------------------------------
# The expert FFN
# --------------------------------------------------------------------------

def split_gate_up(w1: np.ndarray, order: str):
    """Gate and up projections (each [I, K]) of one expert's W1 [2I, K].

    "halves": rows [0, I) gate, [I, 2I) up.
    "interleave16": rows are in blocks of 32; in block b the first 16 rows are
    gate rows 16b..16b+15 and the next 16 the matching up rows
    ([CAKE] section 2, the 16-row gate/up interleave)."""
    two_i, k = w1.shape
    i = two_i // 2
    if order == "halves":
        return w1[:i], w1[i:]
    if order == "interleave16":
        if i % 16:
            raise ValueError("interleave16 needs I % 16 == 0")
        gate = np.empty((i, k), dtype=w1.dtype)
        up = np.empty((i, k), dtype=w1.dtype)
        for b in range(i // 16):
            gate[16 * b:16 * b + 16] = w1[32 * b:32 * b + 16]
            up[16 * b:16 * b + 16] = w1[32 * b + 16:32 * b + 32]
        return gate, up
    raise ValueError(order)


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def expert_ffn(x: np.ndarray, w1: np.ndarray, w2: np.ndarray, order: str = "halves") -> np.ndarray:
    """One expert on rows x [n, K]: W2 (silu(W1_gate x) * (W1_up x)), float64.
    [MK] apply(): matmul with W1, act + mul, matmul with W2."""
    gate, up = split_gate_up(np.asarray(w1, dtype=np.float64), order)
    x = np.asarray(x, dtype=np.float64)
    g = x @ gate.T
    u = x @ up.T
    z = silu(g) * u
    return z @ np.asarray(w2, dtype=np.float64).T


# --------------------------------------------------------------------------
# Global expert ids (expert parallelism)
# --------------------------------------------------------------------------

def map_expert_ids(topk_ids: np.ndarray, expert_map: np.ndarray) -> np.ndarray:
    """Global expert ids -> this GPU's local ids through an expert map.

    [MK] "How To Add a FusedMoEExpertsModular Type", supports_expert_map():
    an implementation may take global ids with a map; [MEGA] introduction:
    the expert kernel receives global (not rank-remapped) ids and unmasked
    weights.  expert_map[g] is the local id of global expert g, or -1 when
    another GPU holds it.  Result: -1 stays -1 (skipped slot); g in [0, G)
    becomes expert_map[g] (-1: held elsewhere, skipped); any other id becomes
    -2 (skipped and counted as invalid by the steps below, like a local id
    outside [0, E); so is a map entry outside {-1} U [0, E))."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    emap = np.asarray(expert_map, dtype=np.int64)
    out = np.full(ids.shape, -2, dtype=np.int64)
    out[ids == -1] = -1
    inside = (ids >= 0) & (ids < emap.size)
    out[inside] = emap[ids[inside]]
    return out.astype(np.int32)


# --------------------------------------------------------------------------
# Permute (align)
# --------------------------------------------------------------------------

def align_permute(topk_ids: np.ndarray, E: int, block: int) -> Dict[str, np.ndarray]:
    """Group the (token, slot) routes by expert, padded to the tile size.

    [MK] apply(), the Permute step; the contiguous format of the introduction
    (ids (M, topk), -1 = skipped slot, [MEGA] section 2).

    Steps: per-expert histogram of the flat ids; pad each count up to a
    multiple of ``block``; exclusive scan of the padded counts gives each
    expert's offset; walk the flat routes in ascending order and place flat
    index t*topk + j at the next free position of its expert.  Unused
    positions hold the sentinel R = M*topk.  Tile b (positions
    [b*block, (b+1)*block)) belongs to the expert whose run contains it, or -1
    past the last padded run.  Buffers are sized for the worst case over all
    routings with R routes."""
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    R = flat.size
    valid = (flat >= 0) & (flat < E)
    n_invalid = int(np.count_nonzero((flat != -1) & ~valid))
    counts = np.zeros(E, dtype=np.int64)
    for v in flat[valid]:
        counts[v] += 1
    padded = (counts + block - 1) // block * block
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    max_tiles = (R + min(E, R) * (block - 1)) // block
    capacity = max_tiles * block
    sorted_ids = np.full(capacity, R, dtype=np.int64)
    cursor = offsets[:-1].copy()
    for i in range(R):
        e = flat[i]
        if 0 <= e < E:
            sorted_ids[cursor[e]] = i
            cursor[e] += 1
    block_expert = np.full(max_tiles, -1, dtype=np.int64)
    for e in range(E):
        for b in range(offsets[e] // block, offsets[e + 1] // block):
            block_expert[b] = e
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_ids": sorted_ids.astype(np.int32),
        "block_expert": block_expert.astype(np.int32),
        "num_post_padded": np.int32(offsets[E]),
        "n_invalid": n_invalid,
        "capacity": capacity,
        "max_tiles": max_tiles,
    }


# --------------------------------------------------------------------------
# Whole computation, contiguous format
# --------------------------------------------------------------------------

WeightFn = Callable[[int], np.ndarray]


def moe_routes(x_rows: np.ndarray, tokens: np.ndarray, topk_ids: np.ndarray, E: int,
               w1_of: WeightFn, w2_of: WeightFn, order: str = "halves") -> Dict[tuple, np.ndarray]:
    """FFN_e(x_t) for every valid slot (t, j) of the listed tokens, float64.

    ``x_rows[i]`` is token ``tokens[i]``'s activation row; ``w1_of(e)`` /
    ``w2_of(e)`` return expert e's weights as float64 (W1 [2I,K], W2 [K,I]).
    Returns {(t, j): y [K]}.  This is the per-(token, top-k slot) buffer the
    FC2 results are written to ([CAKE] section 3)."""
    tokens = np.asarray(tokens)
    sel = np.asarray(topk_ids)[tokens]
    out = {}
    experts = sorted({int(e) for e in sel.reshape(-1) if 0 <= e < E})
    for e in experts:
        pairs = [(i, j) for i in range(len(tokens)) for j in range(sel.shape[1]) if sel[i, j] == e]
        rows = np.asarray([i for i, _ in pairs])
        y = expert_ffn(x_rows[rows], w1_of(e), w2_of(e), order)
        for r, (i, j) in enumerate(pairs):
            out[(int(tokens[i]), j)] = y[r]
    return out


def moe_contiguous(x_rows: np.ndarray, tokens: np.ndarray, topk_ids: np.ndarray,
                   topk_weights: np.ndarray, E: int, w1_of: WeightFn, w2_of: WeightFn,
                   order: str = "halves") -> np.ndarray:
    """out[t] = sum over slots j with a valid id e = ids[t, j] of
    w[t, j] * W2_e (silu(W1gate_e x_t) * (W1up_e x_t)), for the listed tokens.

    [MK] apply() steps in order, with the TopK weight application + reduction
    after Unpermute; slots with id -1 (or out of range) contribute nothing
    ([MEGA] section 2); a token with no valid slot gets +0.0 ([DET] section 2).
    Returns float64 [len(tokens), K]."""
    tokens = np.asarray(tokens)
    ys = moe_routes(x_rows, tokens, topk_ids, E, w1_of, w2_of, order)
    K = x_rows.shape[1]
    out = np.zeros((len(tokens), K), dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64)
    for i, t in enumerate(tokens):
        for j in range(topk_ids.shape[1]):
            if (int(t), j) in ys:
                out[i] += w[t, j] * ys[(int(t), j)]
    return out + 0.0


def topk_reduce_contiguous(y: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
                           E: int) -> np.ndarray:
    """TopKWeightAndReduceContiguous ([MK] "TopKWeightAndReduce"):
    out[t] = sum_j w[t, j] * y[t*topk + j] over slots with a valid id.
    y: [M*topk, K] rows ordered (token, slot).  Empty rows are +0.0."""
    ids = np.asarray(topk_ids)
    M, topk = ids.shape
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros((M, y.shape[1]), dtype=np.float64)
    w = np.asarray(topk_weights, dtype=np.float64)
    for t in range(M):
        for j in range(topk):
            if 0 <= ids[t, j] < E:
                out[t] += w[t, j] * y[t * topk + j]
    return out + 0.0


# --------------------------------------------------------------------------
# Batched format
# --------------------------------------------------------------------------

def moe_batched_rows(a_rows_of: Callable[[int, np.ndarray], np.ndarray], counts: np.ndarray,
                     w1_of: WeightFn, w2_of: WeightFn, order: str = "halves",
                     rows_of: Optional[Callable[[int], Iterable[int]]] = None) -> Dict[int, np.ndarray]:
    """Batched format ([MK] introduction): expert e's valid rows are
    r < counts[e] of its (max_tokens, K) slab; the rest are never read.
    ``a_rows_of(e, rows)`` returns those rows as float64; ``rows_of(e)``
    optionally restricts which valid rows are evaluated.
    Returns {e: (rows, Y [len(rows), K])}."""
    out = {}
    for e in range(len(counts)):
        rows = np.arange(int(counts[e])) if rows_of is None else np.asarray(list(rows_of(e)), dtype=np.int64)
        rows = rows[rows < counts[e]]
        if rows.size == 0:
            continue
        out[e] = (rows, expert_ffn(a_rows_of(e, rows), w1_of(e), w2_of(e), order))
    return out


def naive_batched_reduce(y_of: Callable[[int, int], np.ndarray], counts: np.ndarray,
                         row_token: np.ndarray, row_weight: np.ndarray, n_out: int,
                         K: int, tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """TopKWeightAndReduceNaiveBatched ([MK] "TopKWeightAndReduce"):
    out[tok] = sum over valid rows (e, r) (r < counts[e]) with
    row_token[e, r] == tok of row_weight[e, r] * Y[e, r].  Tokens no row maps
    to are +0.0.  ``y_of(e, r)`` returns Y[e, r] as float64.
    ``tokens`` restricts the output to those token ids (default: all)."""
    tokens = np.arange(n_out) if tokens is None else np.asarray(tokens)
    pos = {int(t): i for i, t in enumerate(tokens)}
    out = np.zeros((len(tokens), K), dtype=np.float64)
    for e in range(len(counts)):
        for r in range(int(counts[e])):
            t = int(row_token[e, r])
            if t in pos:
                out[pos[t]] += float(row_weight[e, r]) * y_of(e, r)
    return out + 0.0


# ------------------------------------------------------------ training ----
# [DET] introduction: the ragged grouped GEMM of a MoE layer's training step.
# Group e holds rows [offsets[e], offsets[e+1]); W[e] is [N, K].

def _groups(offsets: np.ndarray):
    offsets = np.asarray(offsets, dtype=np.int64)
    assert offsets[0] == 0 and np.all(np.diff(offsets) >= 0)
    return [(e, int(offsets[e]), int(offsets[e + 1])) for e in range(len(offsets) - 1)]


def grouped_forward(x: np.ndarray, w: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """y[r] = W[e] x[r] for the rows r of group e (x [R, K], w [E, N, K];
    returns [R, N] float64)."""
    y = np.zeros((x.shape[0], w.shape[1]), dtype=np.float64)
    for e, a, b in _groups(offsets):
        y[a:b] = x[a:b].astype(np.float64) @ w[e].astype(np.float64).T
    return y


def grouped_dgrad(dy: np.ndarray, w: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """The input gradient of grouped_forward: dx[r] = W[e]^T dy[r] (dy [R, N];
    returns [R, K] float64)."""
    dx = np.zeros((dy.shape[0], w.shape[2]), dtype=np.float64)
    for e, a, b in _groups(offsets):
        dx[a:b] = dy[a:b].astype(np.float64) @ w[e].astype(np.float64)
    return dx


def grouped_wgrad(dy: np.ndarray, x: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """The weight gradient of grouped_forward: dW[e] = sum over the rows r of
    group e of dy[r] x[r]^T ([E, N, K] float64).  A group without rows gives
    +0.0 everywhere ([DET] section 2)."""
    groups = _groups(offsets)
    dw = np.zeros((len(groups), dy.shape[1], x.shape[1]), dtype=np.float64)
    for e, a, b in groups:
        if b > a:
            dw[e] = dy[a:b].astype(np.float64).T @ x[a:b].astype(np.float64)
    return dw + 0.0   # +0.0, never -0.0


def grouped_wgrad_accumulate(out: np.ndarray, dy: np.ndarray, x: np.ndarray,
                             offsets: np.ndarray) -> np.ndarray:
    """main_grad after the accumulate: out + dW ([DET] section 1: the same as
    out.add_(dW)); float64 of the fp32 buffer plus the float64 gradient."""
    return np.asarray(out, dtype=np.float64) + grouped_wgrad(dy, x, offsets)

