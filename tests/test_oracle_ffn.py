"""Pins for the oracle's expert FFN, contiguous MoE, reduces and batched format.

What the method computes is fixed by the modular kernel's apply() step list
(permute, W1, act+mul, W2, unpermute, TopK weight + reduce) on the contiguous
and batched formats of that page's introduction.  The pins, none of which
re-runs the oracle's own code path:
* closed forms: gate/up/W2 built from scaled selection matrices, so each
  output element is c * silu(a * x_p) * (b * x_q) with known p, q (catches a
  swapped gate/up, a transposed operand, a wrong interleave, a dropped silu);
* library special cases: E=1 top-1 equals a dense SwiGLU written with
  torch.nn.functional in float64; torch's silu;
* a different algorithm: every expert on every token, mixed by a dense
  (token, expert) gate matrix;
* invariants: token-shuffle equivariance, nullity of weight-0 / id -1 slots,
  exact linearity in the top-k weights, +0.0 for tokens with no valid slot;
* layout: the 16-row gate/up interleave of the Cake MegaMoE EP16 page
  (section 2) built with a reshape as that page describes it.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def torch_swiglu(x, gate, up, w2):
    x, gate, up, w2 = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (x, gate, up, w2))
    return F.linear(F.silu(F.linear(x, gate)) * F.linear(x, up), w2).numpy()


def random_problem(rng, M=13, K=24, I=16, E=5, topk=3, order="halves"):
    x = rng.standard_normal((M, K))
    w1 = rng.standard_normal((E, 2 * I, K)) / math.sqrt(K)
    w2 = rng.standard_normal((E, K, I)) / math.sqrt(I)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(M)]).astype(np.int32)
    w = rng.random((M, topk)).astype(np.float32)
    return x, w1, w2, ids, w


def run_oracle(x, w1, w2, ids, w, order="halves", tokens=None):
    tokens = np.arange(x.shape[0]) if tokens is None else tokens
    return oracle.moe_contiguous(x[tokens], tokens, ids, w, w1.shape[0], lambda e: w1[e],
                                 lambda e: w2[e], order)


# ---------------------------------------------------------------- pins ----

def pin_silu_library():
    v = np.concatenate([np.linspace(-40, 40, 2001), [0.0, 1.0, -1.0, 700.0, -700.0]])
    assert np.allclose(oracle.silu(v), F.silu(torch.from_numpy(v)).numpy(), rtol=1e-15, atol=1e-300)
    assert oracle.silu(np.array([1.0]))[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)


def selection_expert(rng, K, I, order):
    """W1/W2 made of scaled one-hot rows; returns them plus p, q, a, b, r, c."""
    p, q = rng.integers(0, K, I), rng.integers(0, K, I)
    a, b = rng.uniform(0.5, 2, I) * rng.choice([-1, 1], I), rng.uniform(0.5, 2, I)
    gate = np.zeros((I, K)); up = np.zeros((I, K))
    gate[np.arange(I), p] = a
    up[np.arange(I), q] = b
    if order == "halves":
        w1 = np.concatenate([gate, up])
    else:
        w1 = np.empty((2 * I, K))
        for blk in range(I // 16):
            w1[32 * blk: 32 * blk + 16] = gate[16 * blk: 16 * blk + 16]
            w1[32 * blk + 16: 32 * blk + 32] = up[16 * blk: 16 * blk + 16]
    r = rng.integers(0, I, K)
    c = rng.uniform(0.5, 2, K) * rng.choice([-1, 1], K)
    w2 = np.zeros((K, I))
    w2[np.arange(K), r] = c
    return w1, w2, (p, q, a, b, r, c)


def pin_closed_form_selection():
    rng = np.random.default_rng(11)
    for order in ("halves", "interleave16"):
        K, I, M = 40, 32, 6
        w1, w2, (p, q, a, b, r, c) = selection_expert(rng, K, I, order)
        x = rng.standard_normal((M, K))
        y = oracle.expert_ffn(x, w1, w2, order)
        for t in range(M):
            for k in range(K):
                i = r[k]
                g = a[i] * x[t, p[i]]
                want = c[k] * (g / (1 + math.exp(-g))) * (b[i] * x[t, q[i]])
                assert y[t, k] == pytest.approx(want, rel=1e-13, abs=1e-14), (order, t, k)
        # the same expert through the full MoE with topk=1, weight 1
        ids = np.zeros((M, 1), dtype=np.int32)
        w = np.ones((M, 1), dtype=np.float32)
        out = oracle.moe_contiguous(x, np.arange(M), ids, w, 1, lambda e: w1, lambda e: w2, order)
        assert np.allclose(out, y, rtol=1e-14, atol=1e-14)


def pin_dense_swiglu_library():
    rng = np.random.default_rng(12)
    M, K, I = 9, 48, 40
    x = rng.standard_normal((M, K))
    w1 = rng.standard_normal((2 * I, K)) / math.sqrt(K)
    w2 = rng.standard_normal((K, I)) / math.sqrt(I)
    out = oracle.moe_contiguous(x, np.arange(M), np.zeros((M, 1), np.int32),
                                np.ones((M, 1), np.float32), 1, lambda e: w1, lambda e: w2)
    ref = torch_swiglu(x, w1[:I], w1[I:], w2)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def dense_mixing(x, w1, w2, ids, w, E, order="halves"):
    """Every expert on every token (torch float64), mixed by G[t, e] = sum of
    the weights of t's slots routed to e."""
    M = x.shape[0]
    G = np.zeros((M, E))
    for t in range(M):
        for j in range(ids.shape[1]):
            if 0 <= ids[t, j] < E:
                G[t, ids[t, j]] += float(w[t, j])
    I = w1.shape[1] // 2
    out = np.zeros((M, x.shape[1]))
    for e in range(E):
        if order == "halves":
            gate, up = w1[e][:I], w1[e][I:]
        else:
            v = w1[e].reshape(I // 16, 2, 16, -1)
            gate, up = v[:, 0].reshape(I, -1), v[:, 1].reshape(I, -1)
        out += G[:, e:e + 1] * torch_swiglu(x, gate, up, w2[e])
    return out


def pin_dense_mixing_bruteforce():
    rng = np.random.default_rng(13)
    for order in ("halves", "interleave16"):
        x, w1, w2, ids, w = random_problem(rng, M=17, K=24, I=32, E=6, topk=3)
        ids[2, 1] = -1                  # a skipped slot
        ids[5, :] = -1                  # a token with no valid slot
        ids[7, 2] = ids[7, 0]           # the same expert twice in one token
        ids[9, 0] = 99                  # out of range: skipped
        out = run_oracle(x, w1, w2, ids, w, order)
        ref = dense_mixing(x, w1, w2, ids, w, 6, order)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
        assert np.all(out[5] == 0) and not np.any(np.signbit(out[5]))


def pin_equivariance():
    rng = np.random.default_rng(14)
    x, w1, w2, ids, w = random_problem(rng)
    perm = rng.permutation(x.shape[0])
    a = run_oracle(x, w1, w2, ids, w)
    b = run_oracle(x[perm], w1, w2, ids[perm], w[perm])
    assert np.allclose(b, a[perm], rtol=1e-13, atol=1e-15)


def pin_nullity_linearity():
    rng = np.random.default_rng(15)
    x, w1, w2, ids, w = random_problem(rng)
    base = run_oracle(x, w1, w2, ids, w)
    w0 = w.copy(); w0[3, 1] = 0.0
    ids_m = ids.copy(); ids_m[3, 1] = -1
    a = run_oracle(x, w1, w2, ids, w0)
    b = run_oracle(x, w1, w2, ids_m, w)        # same as dropping the slot
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    assert not np.allclose(a[3], base[3])
    assert np.allclose(np.delete(a, 3, 0), np.delete(base, 3, 0), rtol=1e-13, atol=1e-15)
    doubled = run_oracle(x, w1, w2, ids, (2 * w).astype(np.float32))
    assert np.array_equal(doubled, 2 * base)


def pin_reduce_contiguous():
    rng = np.random.default_rng(16)
    M, topk, K, E = 7, 3, 10, 4
    ids = rng.integers(0, E, (M, topk)).astype(np.int32)
    ids[2] = -1
    ids[4, 1] = -1
    w = rng.random((M, topk)).astype(np.float32)
    y = rng.standard_normal((M * topk, K))
    y[4 * topk + 1] = np.nan                   # a skipped slot's row is never read
    out = oracle.topk_reduce_contiguous(y, ids, w, E)
    for t in range(M):
        want = sum((float(w[t, j]) * y[t * topk + j] for j in range(topk) if ids[t, j] >= 0),
                   np.zeros(K))
        assert np.allclose(out[t], want, rtol=1e-15, atol=0)
    assert np.all(out[2] == 0) and not np.any(np.signbit(out[2]))


def pin_interleave_layout():
    rng = np.random.default_rng(17)
    E, I, K = 3, 64, 8
    gate = rng.standard_normal((E, I, K)); up = rng.standard_normal((E, I, K))
    w1 = np.empty((E, 2 * I, K))
    blocks = w1.reshape(E, I // 16, 2, 16, K)          # the page's view of W1
    blocks[:, :, 0] = gate.reshape(E, I // 16, 16, K)
    blocks[:, :, 1] = up.reshape(E, I // 16, 16, K)
    for e in range(E):
        g, u = oracle.split_gate_up(w1[e], "interleave16")
        assert np.array_equal(g, gate[e]) and np.array_equal(u, up[e])
        g, u = oracle.split_gate_up(np.concatenate([gate[e], up[e]]), "halves")
        assert np.array_equal(g, gate[e]) and np.array_equal(u, up[e])


def pin_batched():
    rng = np.random.default_rng(18)
    E, T, K, I, n_out = 4, 6, 16, 16, 5
    a = rng.standard_normal((E, T, K))
    w1 = rng.standard_normal((E, 2 * I, K)) / 4
    w2 = rng.standard_normal((E, K, I)) / 4
    counts = np.array([6, 0, 2, 3], np.int32)
    tok = rng.integers(0, n_out - 1, (E, T)).astype(np.int32)     # token n_out-1 gets nothing
    wt = rng.random((E, T)).astype(np.float32)
    ys = oracle.moe_batched_rows(lambda e, r: a[e][r], counts, lambda e: w1[e], lambda e: w2[e])
    assert set(ys) == {0, 2, 3}
    out = oracle.naive_batched_reduce(lambda e, r: ys[e][1][list(ys[e][0]).index(r)], counts,
                                      tok, wt, n_out, K)
    ref = np.zeros((n_out, K))
    for e in range(E):
        for r in range(counts[e]):
            ref[tok[e, r]] += float(wt[e, r]) * torch_swiglu(a[e][r:r + 1], w1[e][:I], w1[e][I:],
                                                             w2[e])[0]
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    assert np.all(out[n_out - 1] == 0) and not np.any(np.signbit(out[n_out - 1]))
    # junk rows (r >= count) are never read: poison them
    a[0, :] += 0; a[2, 2:] = np.nan; a[3, 3:] = np.nan
    ys2 = oracle.moe_batched_rows(lambda e, r: a[e][r], counts, lambda e: w1[e], lambda e: w2[e])
    assert all(np.array_equal(ys[e][1], ys2[e][1]) for e in ys)


def pin_batched_reduce_worked_example():
    """TopKWeightAndReduceNaiveBatched ("Fused MoE Modular Kernel",
    TopKWeightAndReduce) by hand: E=2 slabs of 3 rows, K=2, 3 output tokens.
    Expert 0 has 2 valid rows, expert 1 has 1; the junk rows carry a valid
    looking token id and a large weight, so reading them changes the result.
      Y[0,0] = [1, 2]  -> token 1, weight 0.5
      Y[0,1] = [3, 4]  -> token 0, weight 2
      Y[0,2] = [5, 5]  (junk: token 2, weight 99)
      Y[1,0] = [8, -4] -> token 1, weight 0.25
      Y[1,1], Y[1,2]   (junk: token 0 / 2, weight 7)
    out[0] = 2*[3,4] = [6, 8]; out[1] = 0.5*[1,2] + 0.25*[8,-4] = [2.5, 0];
    out[2] = [+0, +0] (no valid row maps to token 2)."""
    Y = np.array([[[1, 2], [3, 4], [5, 5]], [[8, -4], [9, 9], [6, 6]]], np.float64)
    counts = np.array([2, 1], np.int32)
    tok = np.array([[1, 0, 2], [1, 0, 2]], np.int32)
    wt = np.array([[0.5, 2.0, 99.0], [0.25, 7.0, 7.0]], np.float32)
    out = oracle.naive_batched_reduce(lambda e, r: Y[e, r], counts, tok, wt, 3, 2)
    assert np.array_equal(out, np.array([[6, 8], [2.5, 0], [0, 0]], np.float64))
    assert not np.any(np.signbit(out))
    part = oracle.naive_batched_reduce(lambda e, r: Y[e, r], counts, tok, wt, 3, 2, tokens=np.array([1]))
    assert np.array_equal(part, np.array([[2.5, 0]]))


def pin_batched_equals_contiguous():
    """The two activation formats ("Fused MoE Modular Kernel", introduction)
    differ only in how routes are laid out: dispatching a contiguous problem
    into per-expert slabs (row r of expert e = a copy of its token's x, the
    map holding the token and its top-k weight) and running the batched
    format's rows + naive-batched reduce gives the contiguous result.  Slots
    with id -1 are not dispatched; a token may hit one expert twice."""
    rng = np.random.default_rng(29)
    M, K, I, E, topk = 9, 16, 8, 4, 3
    x = rng.standard_normal((M, K))
    w1 = rng.standard_normal((E, 2 * I, K)) / 4
    w2 = rng.standard_normal((E, K, I)) / 4
    ids = rng.integers(0, E, (M, topk)).astype(np.int32)
    ids[2, 1] = -1
    ids[4] = -1                                   # token 4: no valid slot
    ids[6] = [3, 3, 1]                            # expert 3 twice
    wts = rng.random((M, topk)).astype(np.float32)
    ref = oracle.moe_contiguous(x, np.arange(M), ids, wts, E, lambda e: w1[e], lambda e: w2[e])
    T = M * topk
    a = np.full((E, T, K), np.nan)                # rows past the counts stay NaN: never read
    tok = np.full((E, T), -1, np.int32)
    wt = np.zeros((E, T), np.float32)
    counts = np.zeros(E, np.int32)
    for t in range(M):
        for j in range(topk):
            e = ids[t, j]
            if e < 0:
                continue
            r = counts[e]
            a[e, r], tok[e, r], wt[e, r] = x[t], t, wts[t, j]
            counts[e] += 1
    ys = oracle.moe_batched_rows(lambda e, r: a[e][r], counts, lambda e: w1[e], lambda e: w2[e])
    pos = {e: {int(r): i for i, r in enumerate(ys[e][0])} for e in ys}
    out = oracle.naive_batched_reduce(lambda e, r: ys[e][1][pos[e][r]], counts, tok, wt, M, K)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    assert np.all(out[4] == 0) and not np.any(np.signbit(out[4]))


def pin_mxfp8_weights_layer():
    # A layer whose weights went through the codec stays within the format's
    # relative error of the unquantised layer (sanity of the dequantised path).
    rng = np.random.default_rng(19)
    x, w1, w2, ids, w = random_problem(rng, M=8, K=64, I=32, E=3, topk=2)
    q1 = [oracle.mxfp8_dequantize(*oracle.mxfp8_quantize(w1[e].astype(np.float32))) for e in range(3)]
    q2 = [oracle.mxfp8_dequantize(*oracle.mxfp8_quantize(w2[e].astype(np.float32))) for e in range(3)]
    ref = run_oracle(x, w1, w2, ids, w)
    got = oracle.moe_contiguous(x, np.arange(8), ids, w, 3, lambda e: q1[e], lambda e: q2[e])
    assert np.abs(got - ref).max() <= 0.1 * np.abs(ref).max()
    assert not np.array_equal(got, ref)


def pin_expert_map_partition():
    # Expert parallelism with global ids: P ranks each hold a disjoint set of
    # the G global experts (in a scrambled local order) and see the same
    # global ids and unmasked weights; the sum of their outputs is the
    # single-GPU result with every expert local (identity ids).
    rng = np.random.default_rng(20)
    G, P = 6, 3
    x, w1, w2, ids, w = random_problem(rng, M=11, K=16, I=8, E=G, topk=3)
    ids[2, 1] = -1
    full = run_oracle(x, w1, w2, ids, w)
    owner = rng.permutation(G) % P                       # rank of each global expert
    total = np.zeros_like(full)
    for r in range(P):
        held = [int(g) for g in rng.permutation(np.flatnonzero(owner == r))]   # local order
        emap = np.full(G, -1, np.int32)
        emap[held] = np.arange(len(held))
        local = oracle.map_expert_ids(ids, emap)
        assert np.all((local == -1) | ((local >= 0) & (local < len(held))))
        total += oracle.moe_contiguous(x, np.arange(11), local, w, len(held),
                                       lambda e: w1[held[e]], lambda e: w2[held[e]])
    assert np.allclose(total, full, rtol=1e-12, atol=1e-13)


def pin_expert_map_worked_example():
    # G = 8 global experts, this GPU holds global 5 (local 0) and 0 (local 1);
    # global 7 maps to 9, outside [0, E=2).  By hand, slot by slot:
    #   -1 -> skipped;  0 -> local 1;  5 -> local 0;  1 -> held elsewhere
    #   (skipped, not invalid);  7 -> 9 (invalid);  8 -> outside [0, G)
    #   (invalid);  -3 -> invalid;  5 -> local 0.
    emap = np.array([1, -1, -1, -1, -1, 0, -1, 9], np.int32)
    ids = np.array([[-1, 0, 5, 1], [7, 8, -3, 5]], np.int32)
    local = oracle.map_expert_ids(ids, emap)
    got = oracle.align_permute(local, 2, 1)
    assert got["n_invalid"] == 3
    assert list(got["counts"]) == [2, 1]                 # local 0: flat 2 and 7; local 1: flat 1
    assert list(got["sorted_ids"][:3]) == [2, 7, 1]
    y = np.arange(8, dtype=np.float64)[:, None] + 1.0     # y row of slot (t, j) = t*4 + j + 1
    wts = np.full((2, 4), 0.5, np.float32)
    out = oracle.topk_reduce_contiguous(y, local, wts, 2)
    assert out[0, 0] == 0.5 * (2 + 3) and out[1, 0] == 0.5 * 8


PINS = [pin_silu_library, pin_closed_form_selection, pin_dense_swiglu_library,
        pin_dense_mixing_bruteforce, pin_equivariance, pin_nullity_linearity, pin_reduce_contiguous,
        pin_interleave_layout, pin_batched, pin_batched_reduce_worked_example,
        pin_batched_equals_contiguous, pin_mxfp8_weights_layer, pin_expert_map_partition,
        pin_expert_map_worked_example]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_ffn_pin(pin):
    pin()
