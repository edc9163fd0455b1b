"""The two TopKWeightAndReduce kernels on the GPU against the oracle.

Inputs (y rows, ids, weights, the batched row map) come from the generator,
never from another GPU kernel.  Each output element is one float32 sum of at
most a few bf16 * float32 products, rounded once to bf16, so the bar is
one bf16 rounding of the reference plus float32 accumulation error.  Runs
must agree bit for bit, tokens with nothing to sum are +0.0, and rows the
format marks invalid are never read (they hold NaN here)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_expert_align_amd as moe
import oracle
from moe_cases import say

pytestmark = pytest.mark.gpu


def bf16_bound(ref: np.ndarray, absum: np.ndarray) -> np.ndarray:
    return 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * absum + 1e-30


def test_reduce_contiguous():
    rng = np.random.default_rng(4)
    M, topk, K, E = 777, 8, 512, 16
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(M)]).astype(np.int32)
    ids[rng.random((M, topk)) < 0.15] = -1
    ids[5] = -1                                    # a token with no valid slot
    ids[9, 2] = E + 3                              # out of range: skipped
    w = rng.random((M, topk)).astype(np.float32)
    y = mi.ih4_normal(M * topk * K, 1.0, 99, 9, 0, device="cuda").view(M * topk, K)
    skipped = torch.from_numpy((ids.reshape(-1) < 0) | (ids.reshape(-1) >= E)).cuda()
    y[skipped] = float("nan")                      # rows of skipped slots must not be read
    plan = moe.moe_plan_init(moe.make_problem(M, K, 512, E, topk=topk))
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    ids_d, w_d = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    moe.moe_topk_reduce_contiguous(plan, y, ids_d, w_d, out)
    out2 = torch.empty_like(out)
    moe.moe_topk_reduce_contiguous(plan, y, ids_d, w_d, out2)
    torch.cuda.synchronize()
    yh = np.nan_to_num(oracle.bf16_to_f64(mi.bf16_bits(y)))
    ref = oracle.topk_reduce_contiguous(yh, ids, w, E)
    absum = oracle.topk_reduce_contiguous(np.abs(yh), ids, np.abs(w), E)
    g = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    say(f"[reduce] contiguous max err {err.max():.3e}")
    assert np.all(err <= bf16_bound(ref, absum))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert np.all(out[5].view(torch.int16).cpu().numpy() == 0)          # +0.0


def test_reduce_contiguous_expert_map():
    """Global ids mapped through an expert map: slots of experts held
    elsewhere (map -1) are skipped like id -1; their y rows are never read."""
    rng = np.random.default_rng(6)
    M, topk, K, E, G = 300, 4, 256, 6, 20
    gid = rng.integers(0, G, (M, topk)).astype(np.int32)
    gid[rng.random((M, topk)) < 0.1] = -1
    emap = np.full(G, -1, np.int32)
    emap[rng.choice(G, E, replace=False)] = rng.permutation(E)
    local = oracle.map_expert_ids(gid, emap)
    w = rng.random((M, topk)).astype(np.float32)
    y = mi.ih4_normal(M * topk * K, 1.0, 98, 9, 2, device="cuda").view(M * topk, K)
    y[torch.from_numpy((local.reshape(-1) < 0)).cuda()] = float("nan")     # never read
    plan = moe.moe_plan_init(moe.make_problem(M, K, 512, E, topk=topk, global_experts=G))
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    moe.moe_topk_reduce_contiguous(plan, y, torch.from_numpy(gid).cuda(), torch.from_numpy(w).cuda(),
                                   out, expert_map=torch.from_numpy(emap).cuda())
    torch.cuda.synchronize()
    yh = np.nan_to_num(oracle.bf16_to_f64(mi.bf16_bits(y)))
    ref = oracle.topk_reduce_contiguous(yh, local, w, E)
    absum = oracle.topk_reduce_contiguous(np.abs(yh), local, np.abs(w), E)
    g = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g - ref) <= bf16_bound(ref, absum))


# (M, topk, K, E, G): a sparse share; an MXFP8-like share; a dense map (most
# slots local, more per token than one load batch) with M not a multiple of
# the tokens a workgroup takes; K / 8 > 1024 and topk > 64 (the other kernel)
MAP_SHAPES = [(300, 4, 256, 6, 20), (1001, 8, 6144, 32, 512), (77, 16, 512, 40, 48),
              (130, 8, 8448, 8, 16), (50, 70, 256, 70, 100)]


@pytest.mark.parametrize("M,topk,K,E,G", MAP_SHAPES, ids=[f"m{m}_k{k}_t{t}_e{e}_g{g}" for m, t, k, e, g in MAP_SHAPES])
def test_reduce_expert_map_matches_host_masked(M, topk, K, E, G):
    """The reduce with global ids and an expert map gives the same bits as
    the reduce with the ids masked on the host, and is within the bf16 bound
    of the oracle; rows of slots held elsewhere (or invalid) hold NaN."""
    rng = np.random.default_rng(M + K)
    gid = rng.integers(0, G, (M, topk)).astype(np.int32)
    gid[rng.random((M, topk)) < 0.05] = -1
    gid[rng.random((M, topk)) < 0.02] = G + 5                      # out of range: skipped
    emap = np.full(G, -1, np.int32)
    emap[rng.choice(G, E, replace=False)] = rng.permutation(E)
    local = oracle.map_expert_ids(gid, emap)
    host = np.where((local >= 0) & (local < E), local, -1).astype(np.int32)
    w = rng.random((M, topk)).astype(np.float32)
    y = mi.ih4_normal(M * topk * K, 1.0, 97, 9, 3, device="cuda").view(M * topk, K)
    y[torch.from_numpy(host.reshape(-1) < 0).cuda()] = float("nan")     # never read
    plan = moe.moe_plan_init(moe.make_problem(M, K, 512, E, topk=topk, global_experts=G))
    plan_h = moe.moe_plan_init(moe.make_problem(M, K, 512, E, topk=topk))
    w_d = torch.from_numpy(w).cuda()
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    out_h = torch.empty_like(out)
    moe.moe_topk_reduce_contiguous(plan, y, torch.from_numpy(gid).cuda(), w_d, out,
                                   expert_map=torch.from_numpy(emap).cuda())
    moe.moe_topk_reduce_contiguous(plan_h, y, torch.from_numpy(host).cuda(), w_d, out_h)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_h.view(torch.int16))
    yh = np.nan_to_num(oracle.bf16_to_f64(mi.bf16_bits(y)))
    ref = oracle.topk_reduce_contiguous(yh, host, w, E)
    absum = oracle.topk_reduce_contiguous(np.abs(yh), host, np.abs(w), E)
    g = out.float().cpu().numpy().astype(np.float64)
    say(f"[reduce] map M={M} topk={topk} K={K}: local slots per token {np.mean((host >= 0).sum(1)):.2f}")
    assert np.all(np.abs(g - ref) <= bf16_bound(ref, absum))


def run_naive_batched(E, T, K, n_out, counts, tok, w, seed):
    y = mi.ih4_normal(E * T * K, 1.0, seed, 9, 1, device="cuda").view(E, T, K)
    invalid = torch.arange(T, device="cuda")[None, :] >= torch.from_numpy(counts).cuda()[:, None]
    y[invalid] = float("nan")                      # junk rows: never read
    tok = tok.copy(); w = w.copy()
    tok[np.arange(T)[None, :] >= counts[:, None]] = 1 << 30   # junk map entries: never read
    plan = moe.moe_plan_init(moe.make_problem(n_out, K, 128, E, max_tokens=T, layout=moe.LAYOUT_BATCHED))
    ws = torch.empty(moe.moe_naive_batched_ws_bytes(plan, n_out), dtype=torch.uint8, device="cuda")
    out = torch.empty((n_out, K), dtype=torch.bfloat16, device="cuda")
    args = (torch.from_numpy(counts).cuda(), torch.from_numpy(tok).cuda(), torch.from_numpy(w).cuda())
    moe.moe_topk_reduce_naive_batched(plan, y, *args, n_out, out, ws)
    out2 = torch.empty_like(out)
    moe.moe_topk_reduce_naive_batched(plan, y, *args, n_out, out2, ws)
    torch.cuda.synchronize()
    status = int(moe.ws_view(ws, 0, 1).cpu()[0])
    return y, out, out2, status


@pytest.mark.parametrize("which", ["scaled", "full"])
def test_reduce_naive_batched(which):
    if which == "full":
        cfg = mi.config(4)
    else:
        cfg = mi.config(4).scaled(E=8, max_tokens=100, K=256, M=64, slot_pool=400)
    counts, tok, w = mi.batched_zipf_rows(cfg.E, cfg.max_tokens, cfg.M, cfg.slot_pool, cfg.seed)
    y, out, out2, status = run_naive_batched(cfg.E, cfg.max_tokens, cfg.K, cfg.M, counts, tok, w, 5)
    yh = y.cpu()                                                  # generator output, bf16
    sample = np.arange(cfg.M) if which == "scaled" else np.sort(
        np.random.default_rng(0).choice(cfg.M, 48, replace=False))

    def y_of(e, r):
        return oracle.bf16_to_f64(mi.bf16_bits(yh[e, r]))

    ref = oracle.naive_batched_reduce(y_of, counts, tok, w, cfg.M, cfg.K, tokens=sample)
    absum = oracle.naive_batched_reduce(lambda e, r: np.abs(y_of(e, r)), counts, tok, np.abs(w),
                                        cfg.M, cfg.K, tokens=sample)
    g = out[torch.from_numpy(sample).cuda()].float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    say(f"[reduce] naive batched {which}: V={counts.sum()} max err {err.max():.3e}")
    assert np.all(err <= bf16_bound(ref, absum))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert status == 0
    hit = np.zeros(cfg.M, bool)
    for e in range(cfg.E):
        hit[tok[e, :counts[e]]] = True
    if (~hit).any():
        assert np.all(out[torch.from_numpy(np.flatnonzero(~hit)).cuda()].view(torch.int16).cpu().numpy() == 0)


@pytest.mark.parametrize("K", [128, 8448], ids=["one_launch", "wide_rows_list_path"])
def test_reduce_naive_batched_out_of_range_rows_skipped(K):
    """Valid rows whose token is outside [0, n_out) are skipped and counted
    (id -1 is a skipped row, not counted).  K = 8448 takes the path that
    builds the per-token row lists with the align kernels (rows wider than
    8192 columns); K = 128 the one-launch reduce."""
    E, T, n_out = 4, 40, 16
    counts = np.array([40, 3, 0, 17], np.int32)
    rng = np.random.default_rng(2)
    tok = rng.integers(0, n_out, (E, T)).astype(np.int32)
    tok[0, 5] = n_out + 2                           # valid row, token out of range: skipped
    tok[3, 1] = -1
    w = rng.random((E, T)).astype(np.float32)
    y, out, _, status = run_naive_batched(E, T, K, n_out, counts, tok, w, 6)
    assert status == 1
    yh = y.cpu()
    ref = oracle.naive_batched_reduce(lambda e, r: oracle.bf16_to_f64(mi.bf16_bits(yh[e, r])),
                                      counts, tok, w, n_out, K)
    g = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3)
