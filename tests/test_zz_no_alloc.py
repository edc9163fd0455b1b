"""moe_apply_contiguous_static, the entry point for callers that cannot
allocate, through the C ABI: its output equals moe_apply_contiguous's (own
workspaces) bit for bit, on two calls in a row whose second is smaller
(the library's array keeps the first call's contents), for the streaming,
single-launch and tile plans that fit; a plan whose workspaces do not fit
is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_expert_align_amd as moe
from moe_cases import (BF16_ABS, BF16_REL, MX_REL, check_close, grouped_scales, make_case, oracle_contiguous,
                       problem, say)

pytestmark = pytest.mark.gpu


def static_vs_allocating(c, variant=moe.VARIANT_AUTO, w_dtype=None):
    plan = moe.moe_plan_init(problem(c.cfg, variant, w_dtype=w_dtype))
    need = -(-plan.ws13_bytes // 256) * 256 + plan.ws2_bytes
    say(f"[no_alloc] {c.cfg.name} variant {plan.variant}: workspaces {need} of {moe.STATIC_SCRATCH_BYTES} bytes")
    assert need <= moe.STATIC_SCRATCH_BYTES
    ws13, ws2 = moe.allocate_workspaces(plan)
    ref = torch.empty((c.cfg.M, c.cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.moe_apply_contiguous(plan, c.inp.x, c.ids, c.wts, c.w1, c.w2, ref, ws13, ws2, c.w1_scale, c.w2_scale)
    out = torch.full((c.cfg.M, c.cfg.K), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_apply_contiguous_static(plan, c.inp.x, c.ids, c.wts, c.w1, c.w2, out, c.w1_scale, c.w2_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{c.cfg.name}: static call differs"
    return out


@pytest.mark.parametrize("first,second", [
    # full decode batch (streaming), then the tiny batch (single launch):
    # the second call's counters sit where the first call left z rows
    ((1, None, moe.VARIANT_AUTO), (0, None, moe.VARIANT_AUTO)),
    # a scaled prefill batch (tiles), then a smaller streaming one
    ((2, dict(M=300, K=256, I=256, E=16), moe.VARIANT_AUTO),
     (1, dict(M=13, K=512, I=1024), moe.VARIANT_STREAM)),
    # single launch twice: a larger then a smaller batch of the same layer
    ((0, dict(M=200), moe.VARIANT_FUSED), (0, None, moe.VARIANT_FUSED)),
    # MXFP8 tiles: scale words in groups of four steps (K, I multiples of
    # 512), then a smaller layer whose W2 loads them step by step
    ((3, dict(M=700, K=1024, I=512), moe.VARIANT_AUTO), (3, dict(M=300, K=512, I=256), moe.VARIANT_AUTO)),
    # MXFP8 tiles on grouped scale arrays, twice: the second call's scale
    # groups are shorter (fewer sorted rows) than the first call left them
    ((3, dict(M=700, K=1024, I=512), "grouped"), (3, dict(M=300, K=512, I=512), "grouped")),
])
def test_static_matches_allocating_two_calls(first, second):
    outs = []
    for idx, kw, variant in (first, second):
        cfg = mi.config(idx) if kw is None else mi.config(idx).scaled(**kw)
        c = make_case(cfg)
        if variant == "grouped":                           # W_MXFP8_GROUPED, the tile kernels
            c = grouped_scales(c)
            outs.append((c, static_vs_allocating(c, moe.VARIANT_TILE, moe.W_MXFP8_GROUPED)))
        else:
            outs.append((c, static_vs_allocating(c, variant)))
    # the second call against the oracle as well
    c, out = outs[-1]
    rel, ab = (MX_REL, 0.0) if c.cfg.w_dtype == "mxfp8" else (BF16_REL, BF16_ABS)
    check_close(out, oracle_contiguous(c, np.arange(c.cfg.M)), rel, ab, f"static {c.cfg.name}")


def test_static_refuses_plans_that_do_not_fit():
    cfg = mi.config(2)                                     # full prefill: ~1 GB of workspaces
    plan = moe.moe_plan_init(problem(cfg))
    assert plan.ws13_bytes + plan.ws2_bytes > moe.STATIC_SCRATCH_BYTES
    x = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((cfg.M, cfg.topk), dtype=torch.int32, device="cuda")
    wts = torch.zeros((cfg.M, cfg.topk), dtype=torch.float32, device="cuda")
    w1 = torch.empty((cfg.E, 2 * cfg.I, cfg.K), dtype=torch.bfloat16, device="cuda")
    w2 = torch.empty((cfg.E, cfg.K, cfg.I), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_apply_contiguous_static(plan, x, ids, wts, w1, w2, out)
    assert ei.value.status == moe.MOE_EUNSUPPORTED
