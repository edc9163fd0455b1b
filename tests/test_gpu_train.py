"""The training grouped GEMMs on the GPU (through the C ABI) against the
oracle ([DET]: forward, dgrad and wgrad of a ragged bf16 grouped GEMM; the
fp32 accumulate; +0.0 for an empty group).

Tolerances: bf16 outputs (y, dx) |gpu - ref| <= 2e-2 * max|ref| + 1e-3; fp32
dW per element |gpu - ref| <= (m + 1) * 2^-24 * sum_r |dy[r,n]| |x[r,k]| + 1e-30
with m the group's rows (the worst-case bound of an m-term fp32 sum in any
order).  Bitwise: run-to-run equality of every output, and the accumulate
equal to main_grad + overwrite in fp32 (numpy), -0.0 turned into +0.0.
"""
import gc

import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_expert_align_amd as moe
import oracle
from moe_cases import BF16_ABS, BF16_REL, check_close, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def free():
    gc.collect()
    torch.cuda.empty_cache()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.detach().cpu().numpy()


def run(ti):
    """forward, dgrad, wgrad (overwrite) and wgrad (accumulate onto a copy of
    main_grad), twice each; returns the first results and checks the second
    are the same bits."""
    c = ti.cfg
    off = torch.from_numpy(ti.offsets).cuda()
    R = int(ti.offsets[-1])
    outs = []
    for _ in range(2):
        y = torch.empty((R, c.N), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty((R, c.K), dtype=torch.bfloat16, device="cuda")
        dw = torch.full((c.E, c.N, c.K), float("nan"), dtype=torch.float32, device="cuda")
        acc = ti.main_grad.clone()
        moe.moe_grouped_forward(ti.x, ti.w, off, y)
        moe.moe_grouped_dgrad(ti.dy, ti.w, off, dx)
        moe.moe_grouped_wgrad(ti.dy, ti.x, off, dw, accumulate=False)
        moe.moe_grouped_wgrad(ti.dy, ti.x, off, acc, accumulate=True)
        torch.cuda.synchronize()
        outs.append((y, dx, dw, acc))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
            "run-to-run bits differ"
    return outs[0]


def check_accumulate_bits(ti, dw, acc):
    """acc == main_grad + dw in fp32, element by element (numpy's IEEE add)."""
    want = (ti.main_grad.cpu().numpy() + dw.cpu().numpy()).astype(np.float32)
    got = acc.cpu().numpy()
    assert np.array_equal(want.view(np.int32), got.view(np.int32)), "accumulate != main_grad + overwrite"
    sizes = np.diff(ti.offsets)
    for e in np.flatnonzero(sizes == 0):
        assert np.all(got[e] == 0) and not np.any(np.signbit(got[e])), f"group {e}: -0.0 kept"


def wgrad_bound(dy, x, off):
    """(m + 1) 2^-24 sum_r |dy| |x| per element, m the group's rows."""
    s = oracle.grouped_wgrad(np.abs(dy), np.abs(x), off)
    m = np.diff(np.asarray(off, np.int64)).astype(np.float64)
    return (m[:, None, None] + 1) * U * s + 1e-30


def test_train_small_every_element():
    cfg = mi.train_config("train_small")
    ti = mi.make_train_inputs(cfg, device="cuda")
    say(f"[train] {cfg.name}: group sizes {np.diff(ti.offsets).tolist()}")
    y, dx, dw, acc = run(ti)
    x, dy, w = host(ti.x), host(ti.dy), host(ti.w)
    off = ti.offsets
    check_close(y, oracle.grouped_forward(x, w, off), BF16_REL, BF16_ABS, "forward")
    check_close(dx, oracle.grouped_dgrad(dy, w, off), BF16_REL, BF16_ABS, "dgrad")
    ref = oracle.grouped_wgrad(dy, x, off)
    err = np.abs(dw.cpu().numpy().astype(np.float64) - ref)
    bound = wgrad_bound(dy, x, off)
    say(f"[parity] wgrad: max err/bound {np.max(err / bound):.3e}")
    assert np.all(err <= bound)
    assert not np.any(np.signbit(dw.cpu().numpy()[np.diff(off) == 0]))
    ref_acc = oracle.grouped_wgrad_accumulate(ti.main_grad.cpu().numpy(), dy, x, off)
    err = np.abs(acc.cpu().numpy().astype(np.float64) - ref_acc)
    assert np.all(err <= bound + U * np.abs(ref_acc))
    check_accumulate_bits(ti, dw, acc)
    del ti; free()


@pytest.mark.parametrize("sizes", [(0, 0, 0, 0), (1, 0, 31, 33, 0, 127, 129, 1), (300, 0, 0, 2)])
def test_train_ragged_edges(sizes):
    """Empty input, single rows, groups around one slice (32) and one tile
    (128), and a tile shared by several groups."""
    E = len(sizes)
    cfg = mi.TrainConfig("train_edges", 23, E=E, N=256, K=128, rows=int(sum(sizes)))
    ti = mi.make_train_inputs(cfg.scaled(balance="balanced", rows=max(1, int(sum(sizes)))), device="cuda")
    # regroup the same rows into the requested sizes
    R = int(sum(sizes))
    ti.offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    ti.x, ti.dy = ti.x[:R].contiguous(), ti.dy[:R].contiguous()
    for e in range(E):
        if sizes[e] == 0:
            ti.main_grad[e] = -0.0
    y, dx, dw, acc = run(ti)
    x, dy, w = host(ti.x), host(ti.dy), host(ti.w)
    off = ti.offsets
    if R:
        check_close(y, oracle.grouped_forward(x, w, off), BF16_REL, BF16_ABS, f"forward {sizes}")
        check_close(dx, oracle.grouped_dgrad(dy, w, off), BF16_REL, BF16_ABS, f"dgrad {sizes}")
    ref = oracle.grouped_wgrad(dy, x, off)
    err = np.abs(dw.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= wgrad_bound(dy, x, off))
    check_accumulate_bits(ti, dw, acc)


@pytest.mark.parametrize("E,N,K,rows", [(16, 512, 1024, 5000), (9, 768, 256, 2600)])
def test_train_zipf_every_element(E, N, K, rows):
    """Zipf-sized groups (two of them empty) that start and end inside the
    256-row tiles of the forward, several groups sharing a tile: every
    element of y, dx and dW against the oracle."""
    cfg = mi.TrainConfig(f"train_zipf_e{E}_n{N}_k{K}_r{rows}", 24, E=E, N=N, K=K, rows=rows, balance="zipf")
    ti = mi.make_train_inputs(cfg, device="cuda")
    sizes = np.diff(ti.offsets)
    say(f"[train] {cfg.name}: group sizes {sizes.tolist()}")
    y, dx, dw, acc = run(ti)
    x, dy, w = host(ti.x), host(ti.dy), host(ti.w)
    off = ti.offsets
    check_close(y, oracle.grouped_forward(x, w, off), BF16_REL, BF16_ABS, "forward")
    check_close(dx, oracle.grouped_dgrad(dy, w, off), BF16_REL, BF16_ABS, "dgrad")
    ref = oracle.grouped_wgrad(dy, x, off)
    err = np.abs(dw.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= wgrad_bound(dy, x, off))
    check_accumulate_bits(ti, dw, acc)
    del ti; free()


def test_train_gu_full_size_sampled():
    """The gate/up shape at full size (E=32, N=4096, K=6144, 1024 rows per
    group), in the launch configuration bench.py times: sampled y and dx rows
    and dW elements against the oracle, every element's accumulate bits, and
    run-to-run equality of every output."""
    cfg = mi.train_config("train_gu")
    ti = mi.make_train_inputs(cfg, device="cuda")
    off = torch.from_numpy(ti.offsets).cuda()
    R = int(ti.offsets[-1])
    outs = []
    for _ in range(2):
        y = torch.empty((R, cfg.N), dtype=torch.bfloat16, device="cuda")
        dx = torch.empty((R, cfg.K), dtype=torch.bfloat16, device="cuda")
        dw = torch.empty((cfg.E, cfg.N, cfg.K), dtype=torch.float32, device="cuda")
        moe.moe_grouped_forward(ti.x, ti.w, off, y)
        moe.moe_grouped_dgrad(ti.dy, ti.w, off, dx)
        moe.moe_grouped_wgrad(ti.dy, ti.x, off, dw)
        torch.cuda.synchronize()
        outs.append((y, dx, dw))
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
    assert torch.equal(outs[0][2].view(torch.int32), outs[1][2].view(torch.int32))
    y, dx, dw = outs[0]
    del outs
    acc = ti.main_grad.clone()
    moe.moe_grouped_wgrad(ti.dy, ti.x, off, acc, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal((ti.main_grad + dw).view(torch.int32), acc.view(torch.int32))
    del acc
    rng = np.random.default_rng(0)
    for e in rng.choice(cfg.E, size=3, replace=False):
        a, b = int(ti.offsets[e]), int(ti.offsets[e + 1])
        rows = np.sort(rng.choice(np.arange(a, b), size=8, replace=False))
        we = host(ti.w[e])
        ref = host(ti.x[torch.from_numpy(rows).cuda()]) @ we.T
        check_close(y[torch.from_numpy(rows).cuda()], ref, BF16_REL, BF16_ABS, f"forward e={e}")
        ref = host(ti.dy[torch.from_numpy(rows).cuda()]) @ we
        check_close(dx[torch.from_numpy(rows).cuda()], ref, BF16_REL, BF16_ABS, f"dgrad e={e}")
        n = rng.integers(0, cfg.N, size=64)
        k = rng.integers(0, cfg.K, size=64)
        dye = host(ti.dy[a:b])
        xe = host(ti.x[a:b])
        ref = np.einsum("rs,rs->s", dye[:, n], xe[:, k])
        bound = (b - a + 1) * U * np.einsum("rs,rs->s", np.abs(dye[:, n]), np.abs(xe[:, k])) + 1e-30
        got = dw[e].cpu().numpy()[n, k].astype(np.float64)
        say(f"[parity] wgrad e={e}: max err/bound {np.max(np.abs(got - ref) / bound):.3e}")
        assert np.all(np.abs(got - ref) <= bound)
    del ti, y, dx, dw; free()
