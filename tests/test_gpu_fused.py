"""The single-launch variant (MOE_VARIANT_FUSED) on the GPU through the C ABI.

Every case checks, on the same seeded inputs: every output element against
the oracle (bf16 weights: |gpu - ref| <= 2e-2 * max|ref| + 1e-3), bitwise
equality with the two-launch streaming variant (same strips, same summation
order), bitwise equality over repeated calls on one workspace (the work-queue
counters must come back to zero after each call), the counters themselves
(all zero after a call) and the time-out count (zero)."""
import gc

import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_expert_align_amd as moe
import oracle
from moe_cases import (BF16_ABS, BF16_REL, check_close, make_case, oracle_contiguous, problem,
                       run_contiguous, say)

pytestmark = pytest.mark.gpu


def free():
    gc.collect()
    torch.cuda.empty_cache()


def sync_words(plan, ws13):
    """The work-queue counters: one per 128-byte line (ticket, align flag,
    one per slot); the per-slot records after them are not counters."""
    lines = 2 + plan.max_active
    return moe.ws_view(ws13, plan.off_sync, 32 * lines).cpu().numpy()[::32]


def status(plan, ws13):
    return moe.ws_view(ws13, plan.off_status, 2).cpu().numpy()


def fused_calls(c, n, ids=None, wts=None, expert_map=None):
    """n calls of the fused variant on one workspace; the outputs and plan."""
    G = 0 if expert_map is None else len(expert_map)
    plan = moe.moe_plan_init(problem(c.cfg, moe.VARIANT_FUSED, global_experts=G))
    assert plan.variant == moe.VARIANT_FUSED, plan.reason
    ws13, ws2 = moe.allocate_workspaces(plan)
    emap = None if expert_map is None else torch.from_numpy(np.asarray(expert_map, np.int32)).cuda()
    outs = []
    for _ in range(n):
        out = torch.empty((c.cfg.M, c.cfg.K), dtype=torch.bfloat16, device="cuda")
        moe.moe_apply_contiguous(plan, c.inp.x, c.ids if ids is None else ids,
                                 c.wts if wts is None else wts, c.w1, c.w2, out, ws13, ws2,
                                 expert_map=emap)
        torch.cuda.synchronize()
        assert not sync_words(plan, ws13).any(), "work-queue counters not reset"
        outs.append(out)
    return outs, plan, ws13


CASES = [
    ("tiny", mi.config(0)),                                               # K=256: 2-wave W1 strips
    ("decode_m4", mi.config(1).scaled(K=512, I=1024)),
    ("decode_m13", mi.config(1).scaled(M=13, K=512, I=1024)),
    ("decode_m16_k384", mi.config(1).scaled(M=16, K=384, I=640)),          # 3 steps: 1-wave W1 strips
    ("prefill_m100", mi.config(2).scaled(M=100, K=256, I=256, E=16)),
    ("prefill_m1000_e64", mi.config(2).scaled(M=1000, K=256, I=128, E=64)),  # R = 8000
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[s[0] for s in CASES])
def test_fused_scaled(name, cfg):
    c = make_case(cfg)
    outs, plan, ws13 = fused_calls(c, 3)
    say(f"[fused] {name}: {plan.reason.decode()}")
    ref = oracle_contiguous(c, np.arange(cfg.M))
    check_close(outs[0], ref, BF16_REL, BF16_ABS, f"fused {name}")
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16)), "repeated calls differ"
    st = status(plan, ws13)
    assert st[0] == 0 and st[1] == 0, st
    two, *_ = run_contiguous(c, moe.VARIANT_STREAM)
    assert torch.equal(outs[0].view(torch.int16), two.view(torch.int16)), "fused != two-launch stream"
    del c; free()


def test_fused_expert_map():
    """Global ids through an expert map (rank 1 of 3, experts 16..31 local);
    one id outside [0, G) is counted as invalid and skipped."""
    cfg = mi.config(2).scaled(M=200, K=256, I=256, E=16)
    c = make_case(cfg)
    rng = np.random.default_rng(21)
    ids = c.inp.topk_ids
    gid = (ids + 16 * rng.integers(0, 3, ids.shape)).astype(np.int32)
    gid[ids < 0] = -1
    gid[5, 0] = 48
    emap = mi.ep_expert_map(48, 16, rank=1)
    outs, plan, ws13 = fused_calls(c, 2, ids=torch.from_numpy(gid).cuda(), expert_map=emap)
    local = oracle.map_expert_ids(gid, emap)
    ref = oracle_contiguous(c, np.arange(cfg.M), ids=local)
    check_close(outs[0], ref, BF16_REL, BF16_ABS, "fused expert_map")
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    st = status(plan, ws13)
    assert st[0] == 1 and st[1] == 0, st     # the invalid id (each call rewrites the count)
    two, *_ = run_contiguous(c, moe.VARIANT_STREAM, ids=torch.from_numpy(gid).cuda(), expert_map=emap)
    assert torch.equal(outs[0].view(torch.int16), two.view(torch.int16))
    del c; free()


def test_fused_all_slots_skipped():
    cfg = mi.config(0)
    c = make_case(cfg)
    ids = torch.full((cfg.M, cfg.topk), -1, dtype=torch.int32, device="cuda")
    outs, plan, ws13 = fused_calls(c, 2, ids=ids)
    for o in outs:
        assert np.all(o.view(torch.int16).cpu().numpy() == 0)
    assert status(plan, ws13)[1] == 0


def test_fused_full_decode():
    """The decode workload at full size in the launch configuration bench.py
    times with --variant fused: every output element against the oracle and
    bitwise against the two-launch streaming variant."""
    cfg = mi.config(1)
    c = make_case(cfg)
    outs, plan, ws13 = fused_calls(c, 2)
    ref = oracle_contiguous(c, np.arange(cfg.M))
    check_close(outs[0], ref, BF16_REL, BF16_ABS, f"fused {cfg.name}")
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    two, *_ = run_contiguous(c, moe.VARIANT_STREAM)
    assert torch.equal(outs[0].view(torch.int16), two.view(torch.int16))
    assert status(plan, ws13)[1] == 0
    del c; free()
