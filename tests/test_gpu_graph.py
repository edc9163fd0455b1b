"""HIP graph capture of the library's calls, and calls on two streams at once.

The boundary documents that a call only enqueues kernels on the caller's
stream (no host synchronisation, no allocation, grid sizes from the plan
alone), so it can be captured once and replayed.  Each case warms the call up
eagerly, captures it in a graph, and replays the graph several times with
eager work in between (another eager call, and the output poisoned with NaN
before each replay); every replay must give the eager call's output bit for
bit (the computation is deterministic)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_expert_align_amd as moe
from moe_cases import grouped_scales, make_case, problem, say

pytestmark = pytest.mark.gpu

REPLAYS = 4

CONTIGUOUS = [
    ("tiny_single_launch", mi.config(0), moe.VARIANT_FUSED),
    ("tiny_tile", mi.config(0), moe.VARIANT_TILE),
    ("decode_stream", mi.config(1).scaled(K=512, I=1024), moe.VARIANT_STREAM),
    ("prefill_tile", mi.config(2).scaled(M=700, K=512, I=384, E=24), moe.VARIANT_AUTO),
    ("mxfp8_tile", mi.config(3).scaled(M=512, K=512, I=256), moe.VARIANT_AUTO),
    ("mxfp8_stream", mi.config(3).scaled(M=512, K=512, I=256), moe.VARIANT_STREAM),
    ("mxfp8_tile_scale_groups", mi.config(3).scaled(M=700, K=1024, I=512), moe.VARIANT_AUTO),
    ("mxfp8_tile_grouped_arrays", mi.config(3).scaled(M=700, K=1024, I=512), "grouped scale arrays"),
]


def capture(fn):
    """Warm ``fn`` up on a side stream, then capture it; returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16).clone()


@pytest.mark.parametrize("name,cfg,variant", CONTIGUOUS, ids=[c[0] for c in CONTIGUOUS])
def test_graph_contiguous(name, cfg, variant):
    c = make_case(cfg)
    if variant == "grouped scale arrays":   # the tiles, W_MXFP8_GROUPED
        c = grouped_scales(c)
        plan = moe.moe_plan_init(problem(cfg, moe.VARIANT_TILE, w_dtype=moe.W_MXFP8_GROUPED))
    else:
        plan = moe.moe_plan_init(problem(cfg, variant))
    say(f"[graph] {name}: variant {plan.variant} ({plan.reason.decode()})")

    def call(out, ws13, ws2):
        moe.moe_apply_contiguous(plan, c.inp.x, c.ids, c.wts, c.w1, c.w2, out, ws13, ws2,
                                 c.w1_scale, c.w2_scale)

    # eager reference, on buffers of its own
    ref_out = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device="cuda")
    ref_ws13, ref_ws2 = moe.allocate_workspaces(plan)
    call(ref_out, ref_ws13, ref_ws2)
    torch.cuda.synchronize()
    ref = bits(ref_out)

    out = torch.empty_like(ref_out)
    ws13, ws2 = moe.allocate_workspaces(plan)
    g = capture(lambda: call(out, ws13, ws2))
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        call(ref_out, ref_ws13, ref_ws2)          # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), ref), f"{name}: replay {i} differs from the eager call"
        assert torch.equal(bits(ref_out), ref), f"{name}: eager call {i} differs"
    assert int(moe.ws_view(ws13, plan.off_status, 1).cpu()[0]) == 0


def test_graph_batched():
    cfg = mi.config(4).scaled(E=8, max_tokens=100, K=256, I=128, M=64, slot_pool=400)
    c = make_case(cfg)
    plan = moe.moe_plan_init(problem(cfg))
    rws = moe.moe_naive_batched_ws_bytes(plan, cfg.M)

    def buffers():
        ws13, _ = moe.allocate_workspaces(plan)
        y = torch.empty((cfg.E, cfg.max_tokens, cfg.K), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(rws, dtype=torch.uint8, device="cuda")
        out = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device="cuda")
        return ws13, y, ws, out

    def call(ws13, y, ws, out):
        moe.moe_apply_batched(plan, c.inp.a, c.counts, c.w1, c.w2, y, ws13)
        moe.moe_topk_reduce_naive_batched(plan, y, c.counts, c.row_token, c.row_weight, cfg.M, out, ws)

    rb = buffers()
    call(*rb)
    torch.cuda.synchronize()
    ref = bits(rb[3])

    gb = buffers()
    g = capture(lambda: call(*gb))
    for i in range(REPLAYS):
        gb[3].fill_(float("nan"))
        call(*rb)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(gb[3]), ref), f"batched: replay {i} differs from the eager call"


def test_two_streams():
    """Reentrancy: two problems with workspaces of their own, issued
    interleaved on two streams, give their single-stream outputs bit for bit."""
    cases = [(mi.config(2).scaled(M=700, K=512, I=384, E=24), moe.VARIANT_AUTO),
             (mi.config(1).scaled(K=512, I=1024), moe.VARIANT_STREAM)]
    runs = []
    for cfg, variant in cases:
        c = make_case(cfg)
        plan = moe.moe_plan_init(problem(cfg, variant))
        ws13, ws2 = moe.allocate_workspaces(plan)
        out = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device="cuda")
        moe.moe_apply_contiguous(plan, c.inp.x, c.ids, c.wts, c.w1, c.w2, out, ws13, ws2)
        torch.cuda.synchronize()
        runs.append((c, plan, ws13, ws2, out, bits(out)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for i in range(REPLAYS):
        for (c, plan, ws13, ws2, out, _), s in zip(runs, streams):
            with torch.cuda.stream(s):
                out.fill_(float("nan"))
                moe.moe_apply_contiguous(plan, c.inp.x, c.ids, c.wts, c.w1, c.w2, out, ws13, ws2)
    torch.cuda.synchronize()
    for (c, plan, _, _, out, ref) in runs:
        assert torch.equal(bits(out), ref), f"{c.cfg.name}: two-stream output differs"


@pytest.mark.parametrize("E,N,K,rows", [(9, 768, 256, 2600), (8, 256, 384, 1000)],
                         ids=["tiles", "older_kernels"])
def test_graph_training(E, N, K, rows):
    """The training grouped GEMMs (forward, dgrad, wgrad with the fp32
    accumulate) captured in one graph and replayed: every replay equals the
    eager calls bit for bit, the accumulate included (main_grad is restored
    by a device copy inside the graph before each accumulate).  N, K
    multiples of 256 take the split-ring tiles; K = 384 the older kernels."""
    cfg = mi.TrainConfig(f"train_graph_e{E}", 25, E=E, N=N, K=K, rows=rows, balance="zipf")
    ti = mi.make_train_inputs(cfg, device="cuda")
    off = torch.from_numpy(ti.offsets).cuda()
    R = int(ti.offsets[-1])

    def buffers():
        return (torch.empty((R, N), dtype=torch.bfloat16, device="cuda"),
                torch.empty((R, K), dtype=torch.bfloat16, device="cuda"),
                torch.empty((E, N, K), dtype=torch.float32, device="cuda"))

    def call(y, dx, acc):
        acc.copy_(ti.main_grad)
        moe.moe_grouped_forward(ti.x, ti.w, off, y)
        moe.moe_grouped_dgrad(ti.dy, ti.w, off, dx)
        moe.moe_grouped_wgrad(ti.dy, ti.x, off, acc, accumulate=True)

    rb = buffers()
    call(*rb)
    torch.cuda.synchronize()
    ref = [rb[0].view(torch.int16).clone(), rb[1].view(torch.int16).clone(), rb[2].view(torch.int32).clone()]
    gb = buffers()
    g = capture(lambda: call(*gb))
    for i in range(REPLAYS):
        for t in gb:
            t.fill_(float("nan"))
        call(*rb)                      # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        got = [gb[0].view(torch.int16), gb[1].view(torch.int16), gb[2].view(torch.int32)]
        for name, a, b in zip(("y", "dx", "main_grad"), got, ref):
            assert torch.equal(a, b), f"training {name}: replay {i} differs from the eager calls"
