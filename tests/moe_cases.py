"""Shared machinery of the GPU parity tests: device inputs for a workload,
one call of the HIP path through the C ABI, and the oracle's reference for
(a sample of) the same outputs.

Inputs come from moe_inputs (generated on the device; the oracle gets host
copies of the same generator output).  Nothing the HIP path computes is
ever fed to the oracle.
"""
from __future__ import annotations

import dataclasses
import math
import sys
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

import moe_inputs as mi
import mixture_experts_expert_align_amd as moe
import oracle

BF16_REL, BF16_ABS = 2e-2, 1e-3      # |gpu - ref| <= 2e-2 * max|ref| + 1e-3  (bf16 weights)
MX_REL = 6e-2                        # |gpu - ref| <= 6e-2 * max|ref|          (MXFP8 weights)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class DeviceCase:
    cfg: mi.MoEConfig
    inp: mi.Inputs
    ids: Optional[torch.Tensor] = None          # int32 [M,topk] on the device
    wts: Optional[torch.Tensor] = None          # float32 [M,topk]
    counts: Optional[torch.Tensor] = None       # batched: int32 [E]
    row_token: Optional[torch.Tensor] = None
    row_weight: Optional[torch.Tensor] = None
    w1: Optional[torch.Tensor] = None           # what the kernels read (bf16 or E4M3 codes)
    w2: Optional[torch.Tensor] = None
    w1_scale: Optional[torch.Tensor] = None
    w2_scale: Optional[torch.Tensor] = None
    cache: dict = field(default_factory=dict)


def problem(cfg: mi.MoEConfig, variant=moe.VARIANT_AUTO, global_experts=0, w_dtype=None):
    """The problem of a workload; ``w_dtype`` overrides the weight type (e.g.
    W_MXFP8_GROUPED for grouped scale arrays)."""
    if w_dtype is None:
        w_dtype = moe.W_BF16 if cfg.w_dtype == "bf16" else moe.W_MXFP8
    return moe.make_problem(cfg.M, cfg.K, cfg.I, cfg.E, topk=cfg.topk, max_tokens=cfg.max_tokens,
                            layout=moe.LAYOUT_CONTIGUOUS if cfg.layout == "contiguous" else moe.LAYOUT_BATCHED,
                            w_dtype=w_dtype,
                            w1_order=moe.W1_HALVES if cfg.w1_order == "halves" else moe.W1_INTERLEAVE16,
                            variant=variant, global_experts=global_experts)


def quantize_on_device(w: torch.Tensor):
    """MXFP8 codes/scales of a float32 [..., n] device tensor through the
    library's own codec (moe_quantize_mxfp8)."""
    codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scales = torch.empty((*w.shape[:-1], w.shape[-1] // 32), dtype=torch.uint8, device=w.device)
    moe.moe_quantize_mxfp8(w.contiguous(), codes, scales)
    return codes, scales


def grouped_scales(c: DeviceCase) -> DeviceCase:
    """The case with its MXFP8 scale arrays grouped by moe_pack_mxfp8_scales
    (for W_MXFP8_GROUPED)."""
    p1, p2 = torch.empty_like(c.w1_scale), torch.empty_like(c.w2_scale)
    moe.moe_pack_mxfp8_scales(c.w1_scale, p1)
    moe.moe_pack_mxfp8_scales(c.w2_scale, p2)
    torch.cuda.synchronize()
    return dataclasses.replace(c, w1_scale=p1, w2_scale=p2)


def make_case(cfg: mi.MoEConfig, device="cuda") -> DeviceCase:
    say(f"[case] generating {cfg.name} M={cfg.M} K={cfg.K} I={cfg.I} E={cfg.E}")
    inp = mi.make_inputs(cfg, device=device, weights=True)
    c = DeviceCase(cfg=cfg, inp=inp)
    if cfg.layout == "contiguous":
        c.ids = torch.from_numpy(inp.topk_ids).to(device)
        c.wts = torch.from_numpy(inp.topk_weights).to(device)
    else:
        c.counts = torch.from_numpy(inp.expert_num_tokens).to(device)
        c.row_token = torch.from_numpy(inp.row_token).to(device)
        c.row_weight = torch.from_numpy(inp.row_weight).to(device)
    if cfg.w_dtype == "mxfp8":
        c.w1, c.w1_scale = quantize_on_device(inp.w1)
        c.w2, c.w2_scale = quantize_on_device(inp.w2)
    else:
        c.w1, c.w2 = inp.w1, inp.w2
    torch.cuda.synchronize()
    return c


def poison_workspaces(plan, ws13: torch.Tensor, ws2: torch.Tensor):
    """Fill z (in ws13) and the per-(token, slot) rows y (ws2) with 0xFF bytes
    (bf16 NaN, E4M3 NaN): a row the kernels should have written but did not
    then turns the output it feeds into NaN instead of a stale zero."""
    end = plan.off_xq if plan.off_xq > 0 else plan.ws13_bytes
    if plan.off_sync > 0:
        end = min(end, plan.off_sync)
    ws13[plan.off_z:end].fill_(0xFF)
    ws2.fill_(0xFF)


def run_contiguous(c: DeviceCase, variant=moe.VARIANT_AUTO, ids=None, wts=None, x=None,
                   expert_map: Optional[np.ndarray] = None, poison: bool = False, w_dtype=None):
    """One moe_apply_contiguous call; with ``expert_map`` (host int32 [G]) the
    ids are global and the plan's global_experts is G.  ``poison``: the
    intermediate buffers start as NaN patterns (see poison_workspaces).
    ``w_dtype``: as in problem()."""
    G = 0 if expert_map is None else len(expert_map)
    plan = moe.moe_plan_init(problem(c.cfg, variant, global_experts=G, w_dtype=w_dtype))
    ws13, ws2 = moe.allocate_workspaces(plan)
    if poison:
        poison_workspaces(plan, ws13, ws2)
    out = torch.empty((c.cfg.M, c.cfg.K), dtype=torch.bfloat16, device="cuda")
    emap = None if expert_map is None else torch.from_numpy(np.asarray(expert_map, np.int32)).cuda()
    moe.moe_apply_contiguous(plan, c.inp.x if x is None else x, c.ids if ids is None else ids,
                             c.wts if wts is None else wts, c.w1, c.w2, out, ws13, ws2,
                             c.w1_scale, c.w2_scale, expert_map=emap)
    torch.cuda.synchronize()
    return out, plan, ws13, ws2


def run_batched(c: DeviceCase):
    plan = moe.moe_plan_init(problem(c.cfg))
    ws13, _ = moe.allocate_workspaces(plan)
    cfg = c.cfg
    y = torch.empty((cfg.E, cfg.max_tokens, cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.moe_apply_batched(plan, c.inp.a, c.counts, c.w1, c.w2, y, ws13)
    ws = torch.empty(moe.moe_naive_batched_ws_bytes(plan, cfg.M), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.M, cfg.K), dtype=torch.bfloat16, device="cuda")
    moe.moe_topk_reduce_naive_batched(plan, y, c.counts, c.row_token, c.row_weight, cfg.M, out, ws)
    torch.cuda.synchronize()
    return y, out, plan


# ------------------------------------------------------------ oracle side --

def _host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return oracle.bf16_to_f64(mi.bf16_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def oracle_weights(c: DeviceCase):
    """w1_of(e), w2_of(e) as float64 for the oracle: bf16 decoded exactly, or
    the oracle's own MXFP8 codec applied to the float32 generator output.
    Small experts are cached; large ones are decoded on each request."""
    def get(name, e):
        key = (name, e)
        if key in c.cache:
            return c.cache[key]
        w = (c.inp.w1 if name == "w1" else c.inp.w2)[e]
        if c.cfg.w_dtype == "mxfp8":
            v = oracle.mxfp8_dequantize(*oracle.mxfp8_quantize(w.cpu().numpy()))
        else:
            v = _host_f64(w)
        if w.numel() <= (1 << 22):
            c.cache[key] = v
        return v

    return (lambda e: get("w1", e)), (lambda e: get("w2", e))


def oracle_contiguous(c: DeviceCase, tokens: np.ndarray, ids=None, wts=None) -> np.ndarray:
    cfg = c.cfg
    ids = c.inp.topk_ids if ids is None else ids
    wts = c.inp.topk_weights if wts is None else wts
    x = _host_f64(c.inp.x[torch.from_numpy(np.asarray(tokens)).to(c.inp.x.device)])
    w1_of, w2_of = oracle_weights(c)
    return oracle.moe_contiguous(x, tokens, ids, wts, cfg.E, w1_of, w2_of, cfg.w1_order)


def check_close(gpu: torch.Tensor, ref: np.ndarray, rel: float, abs_: float, what: str):
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    bound = rel * np.abs(ref).max() + abs_
    err = np.abs(g - ref)
    i = np.unravel_index(np.argmax(err), err.shape)
    say(f"[parity] {what}: max|err| {err.max():.3e} bound {bound:.3e} max|ref| {np.abs(ref).max():.3e}")
    assert err.max() <= bound, f"{what}: max err {err.max()} at {i} > {bound} (gpu {g[i]}, ref {ref[i]})"


def tokens_covering_experts(ids: np.ndarray, E: int, experts=None, per_expert: int = 2) -> np.ndarray:
    """Tokens that together reach every listed expert (default: all E): for
    each expert its first and last routed token in flat order (and, with
    per_expert > 2, evenly spaced ones between), so each expert's run is
    checked at its start and its end."""
    flat_tok = np.repeat(np.arange(ids.shape[0]), ids.shape[1])
    flat = ids.reshape(-1)
    pick = set()
    for e in (range(E) if experts is None else experts):
        toks = flat_tok[flat == e]
        if toks.size == 0:
            continue
        idx = np.unique(np.linspace(0, toks.size - 1, per_expert).round().astype(int))
        pick.update(int(t) for t in toks[idx])
    return np.array(sorted(pick), dtype=np.int64)


def heavy_tail_rows(x: torch.Tensor, seed: int, every: int = 3):
    """Put large values into the activations, in place: in every ``every``-th
    row, one element of each 32-column block becomes +-(4 .. 8) (4 to 8 sigma
    of the N(0,1) rows; the seeded generator's own values stay within 3.46
    sigma), and one block of row 0 holds a single 64.  The block maximum then
    sets the MXFP8 scale, so the other elements of the block lose precision
    the way normal tails make them."""
    M, K = x.shape
    rng = np.random.default_rng(seed)
    rows = np.arange(0, M, every)
    nb = K // 32
    col = (np.arange(nb)[None, :] * 32 + rng.integers(0, 32, (rows.size, nb))).reshape(-1)
    row = np.repeat(rows, nb)
    val = rng.uniform(4.0, 8.0, row.size) * np.where(rng.random(row.size) < 0.5, -1.0, 1.0)
    xr = torch.from_numpy(row).to(x.device)
    xc = torch.from_numpy(col).to(x.device)
    x[xr, xc] = torch.from_numpy(val).to(x.device, torch.float32).to(x.dtype)
    x[0, 5] = 64.0


def sample_tokens(M: int, n: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(M, size=min(n, M), replace=False))
