"""Planted mistakes in the oracle must each fail at least one pin.

Each mutation below replaces one oracle function (on the CPU, via
monkeypatch) with a plausible wrong version: a swapped operand, a dropped
term, a wrong sign, an off-by-one, an unstable order.  The test runs every pin
of the codec, align and FFN pin sets and requires that one of them fails.
"""
import numpy as np
import pytest

import oracle
import test_oracle_align as A
import test_oracle_codec as C
import test_oracle_ffn as FF
import test_oracle_train as T

ALL_PINS = C.PINS + A.PINS + FF.PINS + T.PINS

_orig = {n: getattr(oracle, n) for n in ("split_gate_up", "silu", "expert_ffn", "align_permute",
                                         "mx_scale_exponent", "e4m3fn_encode",
                                         "topk_reduce_contiguous", "moe_contiguous",
                                         "map_expert_ids", "grouped_forward", "grouped_dgrad",
                                         "naive_batched_reduce", "moe_batched_rows",
                                         "grouped_wgrad", "grouped_wgrad_accumulate",
                                         "mx_scale_code", "mxfp8_quantize", "mxfp8_dequantize")}


def m_swap_gate_up(w1, order):
    g, u = _orig["split_gate_up"](w1, order)
    return u, g


def m_interleave_up_first(w1, order):
    if order != "interleave16":
        return _orig["split_gate_up"](w1, order)
    g, u = _orig["split_gate_up"](w1, order)
    return u, g


def m_silu_sign(v):
    return v / (1.0 + np.exp(v))


def m_ffn_no_act(x, w1, w2, order="halves"):
    g, u = oracle.split_gate_up(np.asarray(w1, np.float64), order)
    return ((x @ g.T) * (x @ u.T)) @ np.asarray(w2, np.float64).T


def m_ffn_w2_transposed(x, w1, w2, order="halves"):
    g, u = oracle.split_gate_up(np.asarray(w1, np.float64), order)
    z = oracle.silu(x @ g.T) * (x @ u.T)
    w2 = np.asarray(w2, np.float64)
    if w2.shape[0] == w2.shape[1]:
        return z @ w2
    # a transposed read of a non-square W2: same element count, wrong layout
    return z @ w2.reshape(w2.shape[1], w2.shape[0])


def m_align_descending(ids, E, B):
    got = _orig["align_permute"](ids, E, B)
    s = got["sorted_ids"].copy()
    for e in range(E):
        lo, n = got["offsets"][e], got["counts"][e]
        s[lo:lo + n] = s[lo:lo + n][::-1]
    got["sorted_ids"] = s
    return got


def m_align_no_padding(ids, E, B):
    return _orig["align_permute"](ids, E, 1)


def m_scale_floor(bm):
    return _orig["mx_scale_exponent"](bm) - 1


def m_encode_ties_away(v):
    v = np.asarray(v, np.float64)
    c = _orig["e4m3fn_encode"](v)
    tab = oracle.e4m3fn_table()
    a = np.abs(v)
    up = np.minimum((c & 0x7F).astype(np.int64) + 1, 126)
    mid = (tab[c & 0x7F] + tab[up]) / 2
    bump = (a == mid) & (up != (c & 0x7F))
    return np.where(bump, (c & 0x80) | up.astype(np.uint8), c).astype(np.uint8)


def m_scale_code_zero_block_biased(bm):
    bm = np.asarray(bm, np.float64)
    return np.where(bm > 0, _orig["mx_scale_code"](bm), 127).astype(np.uint8)   # zero block: 2^0


def m_quantize_half_block_max(x):
    # the block maximum taken over the first 16 values of each block only
    x = np.asarray(x, np.float64)
    n = x.shape[-1]
    b = x.reshape(-1, n // 32, 32)
    sc = oracle.mx_scale_code(np.abs(b[..., :16]).max(axis=-1))
    s = np.ldexp(1.0, sc.astype(np.int32) - 127)
    codes = oracle.e4m3fn_encode(np.clip(b / s[..., None], -448.0, 448.0)).reshape(x.shape)
    return codes, sc.reshape(*x.shape[:-1], n // 32)


def m_dequantize_bias_128(codes, scales):
    return _orig["mxfp8_dequantize"](codes, np.asarray(scales, np.int64) - 1)


def m_reduce_reads_skipped(y, ids, w, E):
    ids2 = np.where(np.asarray(ids) < 0, 0, ids)
    return _orig["topk_reduce_contiguous"](y, ids2, w, E)


def m_moe_ignores_weights(x_rows, tokens, ids, w, E, w1_of, w2_of, order="halves"):
    return _orig["moe_contiguous"](x_rows, tokens, ids, np.ones_like(w), E, w1_of, w2_of, order)


def m_map_ignored(ids, emap):
    return np.asarray(ids, np.int32)                     # global ids used as local ones


def m_map_remote_invalid(ids, emap):
    out = _orig["map_expert_ids"](ids, emap)
    return np.where((out == -1) & (np.asarray(ids) != -1), -2, out).astype(np.int32)


def m_map_out_of_range_kept(ids, emap):
    ids = np.asarray(ids, np.int64)
    out = _orig["map_expert_ids"](np.where(ids >= len(emap), -1, ids), emap)
    return out                                           # ids past G silently skipped


def m_forward_w_layout(x, w, off):
    # W[e] read as [K, N] row-major instead of [N, K]
    w = np.asarray(w)
    return _orig["grouped_forward"](x, w.reshape(w.shape[0], w.shape[2], w.shape[1]).transpose(0, 2, 1), off)


def m_dgrad_wrong_expert(dy, w, off):
    return _orig["grouped_dgrad"](dy, np.roll(np.asarray(w), 1, axis=0), off)


def m_dgrad_w_layout(dy, w, off):
    w = np.asarray(w)
    return _orig["grouped_dgrad"](dy, w.reshape(w.shape[0], w.shape[2], w.shape[1]).transpose(0, 2, 1), off)


def m_wgrad_drops_last_row(dy, x, off):
    off = np.asarray(off, np.int64)
    dw = np.zeros((len(off) - 1, dy.shape[1], x.shape[1]))
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1]) - 1
        if b > a:
            dw[e] = dy[a:b].T @ x[a:b]
    return dw


def m_wgrad_minus_zero(dy, x, off):
    dw = _orig["grouped_wgrad"](dy, x, off)
    empty = np.diff(np.asarray(off)) == 0
    dw[empty] = -0.0
    return dw


def m_accumulate_ignores_out(out, dy, x, off):
    return _orig["grouped_wgrad"](dy, x, off)


def m_batched_reduce_ignores_counts(y_of, counts, row_token, row_weight, n_out, K, tokens=None):
    full = np.full_like(np.asarray(counts), row_token.shape[1])
    return _orig["naive_batched_reduce"](y_of, full, row_token, row_weight, n_out, K, tokens)


def m_batched_reduce_transposed_map(y_of, counts, row_token, row_weight, n_out, K, tokens=None):
    tokens = np.arange(n_out) if tokens is None else np.asarray(tokens)
    pos = {int(t): i for i, t in enumerate(tokens)}
    out = np.zeros((len(tokens), K))
    for e in range(len(counts)):
        for r in range(int(counts[e])):
            t = int(row_token[r, e])                 # indices swapped
            if t in pos:
                out[pos[t]] += float(row_weight[e, r]) * y_of(e, r)
    return out


def m_batched_reduce_unweighted(y_of, counts, row_token, row_weight, n_out, K, tokens=None):
    return _orig["naive_batched_reduce"](y_of, counts, row_token, np.ones_like(row_weight), n_out, K, tokens)


def m_batched_rows_one_past(a_rows_of, counts, w1_of, w2_of, order="halves", rows_of=None):
    cap = lambda e: range(int(counts[e]) + 1)
    return _orig["moe_batched_rows"](a_rows_of, np.asarray(counts) + 1, w1_of, w2_of, order,
                                     rows_of or cap)


def m_batched_rows_wrong_expert(a_rows_of, counts, w1_of, w2_of, order="halves", rows_of=None):
    n = len(counts)
    return _orig["moe_batched_rows"](a_rows_of, counts, lambda e: w1_of((e + 1) % n),
                                     lambda e: w2_of((e + 1) % n), order, rows_of)


MUTATIONS = [
    ("grouped_forward", m_forward_w_layout), ("grouped_dgrad", m_dgrad_wrong_expert),
    ("grouped_dgrad", m_dgrad_w_layout), ("grouped_wgrad", m_wgrad_drops_last_row),
    ("grouped_wgrad", m_wgrad_minus_zero), ("grouped_wgrad_accumulate", m_accumulate_ignores_out),
    ("split_gate_up", m_swap_gate_up), ("split_gate_up", m_interleave_up_first),
    ("silu", m_silu_sign), ("expert_ffn", m_ffn_no_act), ("expert_ffn", m_ffn_w2_transposed),
    ("align_permute", m_align_descending), ("align_permute", m_align_no_padding),
    ("mx_scale_exponent", m_scale_floor), ("e4m3fn_encode", m_encode_ties_away),
    ("topk_reduce_contiguous", m_reduce_reads_skipped), ("moe_contiguous", m_moe_ignores_weights),
    ("map_expert_ids", m_map_ignored), ("map_expert_ids", m_map_remote_invalid),
    ("map_expert_ids", m_map_out_of_range_kept),
    ("naive_batched_reduce", m_batched_reduce_ignores_counts),
    ("naive_batched_reduce", m_batched_reduce_transposed_map),
    ("naive_batched_reduce", m_batched_reduce_unweighted),
    ("moe_batched_rows", m_batched_rows_one_past), ("moe_batched_rows", m_batched_rows_wrong_expert),
    ("mx_scale_code", m_scale_code_zero_block_biased), ("mxfp8_quantize", m_quantize_half_block_max),
    ("mxfp8_dequantize", m_dequantize_bias_128),
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(oracle, name, fn)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {fn.__name__}"
