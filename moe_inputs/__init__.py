"""Seeded synthetic inputs for the fused-MoE expert computation.

This module draws every input the expert computation consumes and nothing
else: activations, router outputs (top-k ids and weights; routing happens
before the experts, so it is input generation here), expert weight tensors,
and the batched layout's per-expert row counts and row -> token map.  It holds
none of the method's own arithmetic (no align, no GEMM, no activation, no
quantisation, no reduce).  Both the CPU oracle and the HIP path consume what
it produces; neither imports the other.

Five workloads are defined (``CONFIGS``), each with a seed equal to its index:

* ``tiny``      M=64   K=256  I=512  E=8   topk=2   bf16, softmax top-2 routing
* ``decode``    M=4    K=4096 I=8192 E=64  topk=8   bf16, softmax top-8 routing
* ``prefill``   M=8192 K=4096 I=1536 E=128 topk=8   bf16, softmax(logits+bias)
* ``mxfp8``     M=4096 K=6144 I=2048 E=32 (local share of 512) topk=8, the
                affine route map ((8t+j)*73+19) mod 512, fp32 weights that each
                side quantises to MXFP8 itself, gate/up rows interleaved by 16
* ``batched``   E=32 max_tokens=512 K=7168 I=2048, Zipf(1.2) row counts capped
                at 512, 512 output tokens

and the training grouped GEMMs' workloads (``TRAIN_CONFIGS``): ragged rows
grouped by expert (balanced, or Zipf-sized with two empty groups), x [R, K],
dy [R, N], W [E, N, K] and an fp32 main_grad [E, N, K], the shapes of one
rank's gate/up (N = 2I = 4096, K = 6144) and down (N = 6144, K = 2048)
projections with 32 local experts.

Large tensors come from a counter-based generator defined with integer
operations only (``ih4_normal``), so that the same values come out bit for bit
on the CPU and on the GPU: each element is the centred sum of four 16-bit
uniforms (an Irwin-Hall(4) variate) times a constant chosen so the variance is
sigma^2.  It has the mean and variance of N(0, sigma^2) and support +-3.46
sigma.  Router logits and biases are small and come from numpy's PCG64 normal.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = [
    "MoEConfig", "CONFIGS", "config", "ih4_normal", "Inputs", "make_inputs",
    "routing_softmax_topk", "routing_affine_ep_share", "batched_zipf_rows",
    "bf16_bits", "TrainConfig", "TRAIN_CONFIGS", "train_config", "train_group_sizes",
    "TrainInputs", "make_train_inputs",
]

MASK32 = 0xFFFFFFFF

# Stream tags: one per kind of tensor, so streams never share a key.
TAG_X, TAG_W1, TAG_W2, TAG_A = 1, 2, 3, 4
TAG_TX, TAG_TDY, TAG_TW, TAG_TG = 5, 6, 7, 8   # training grouped GEMMs


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    seed: int
    layout: str              # "contiguous" | "batched"
    M: int                   # tokens (contiguous) / output tokens (batched)
    K: int                   # hidden size
    I: int                   # intermediate size
    E: int                   # experts held on this GPU
    topk: int = 0            # contiguous only
    max_tokens: int = 0      # batched only
    w_dtype: str = "bf16"    # "bf16" | "mxfp8"
    w1_order: str = "halves"  # "halves" | "interleave16"
    routing: str = "softmax_topk"  # see make_inputs
    global_experts: int = 0  # affine routing: size of the global expert space
    slot_pool: int = 0       # batched: token-slots the Zipf counts are drawn from

    def scaled(self, **kw) -> "MoEConfig":
        """Same recipe at other sizes (parity cases the oracle finishes fast)."""
        return dataclasses.replace(self, **kw)

    @property
    def routes_capacity(self) -> int:
        return self.M * self.topk if self.layout == "contiguous" else self.E * self.max_tokens


CONFIGS = [
    MoEConfig("tiny_m64_k256_i512_e8_top2", 0, "contiguous", M=64, K=256, I=512, E=8, topk=2),
    MoEConfig("decode_m4_k4096_i8192_e64_top8", 1, "contiguous", M=4, K=4096, I=8192, E=64, topk=8),
    MoEConfig("prefill_m8192_k4096_i1536_e128_top8", 2, "contiguous", M=8192, K=4096, I=1536,
              E=128, topk=8, routing="softmax_topk_bias"),
    MoEConfig("mxfp8_share_m4096_k6144_i2048_e32of512_top8", 3, "contiguous", M=4096, K=6144,
              I=2048, E=32, topk=8, w_dtype="mxfp8", w1_order="interleave16",
              routing="affine_ep_share", global_experts=512),
    MoEConfig("batched_e32_t512_k7168_i2048", 4, "batched", M=512, K=7168, I=2048, E=32,
              max_tokens=512, routing="batched_zipf", slot_pool=4096),
]


def config(name_or_index) -> MoEConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    for c in CONFIGS:
        if c.name == name_or_index or c.name.split("_")[0] == name_or_index:
            return c
    raise KeyError(name_or_index)


# --------------------------------------------------------------------------
# Counter-based integer generator (bit-identical on any torch device)
# --------------------------------------------------------------------------

def _hash32(x: torch.Tensor) -> torch.Tensor:
    """A 32-bit avalanche bijection on int64 tensors holding values < 2**32.

    Two xor-shift-multiply rounds with odd multipliers (the "lowbias32"
    constants published by C. Wellons).  Products may wrap past 2**63; only
    their low 32 bits are kept, which wrapping does not change.
    """
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & MASK32
    x = x ^ (x >> 15)
    x = (x * 0x846CA68B) & MASK32
    x = x ^ (x >> 16)
    return x


def _hash32_int(v: int) -> int:
    return int(_hash32(torch.tensor([v & MASK32], dtype=torch.int64))[0])


def stream_keys(seed: int, tag: int, sub: int) -> tuple[int, int]:
    k1 = _hash32_int(seed * 0x9E3779B1 + tag * 0x85EBCA77 + sub * 0xC2B2AE3D)
    k2 = _hash32_int(k1 ^ 0x27D4EB2F)
    return k1, k2


IH4_MEAN = 2 * 65535            # mean of a sum of four U{0..65535}
IH4_STD = math.sqrt(4 * (65536.0 ** 2 - 1) / 12.0)


def ih4_normal(n: int, sigma: float, seed: int, tag: int, sub: int, *,
               start: int = 0, device="cpu", out_dtype=torch.bfloat16) -> torch.Tensor:
    """Elements [start, start+n) of stream (seed, tag, sub), as ``out_dtype``.

    Element j: u = H(H(2j ^ k1) ^ k2), v = H(H(2j+1 ^ k1) ^ k2) with H the
    32-bit hash above; s = sum of the four 16-bit halves of u and v;
    value = float32(s - 131070) * float32(sigma / IH4_STD), rounded to
    ``out_dtype`` (round-to-nearest-even for bf16).
    """
    assert start + n <= 1 << 31
    k1, k2 = stream_keys(seed, tag, sub)
    j = torch.arange(start, start + n, dtype=torch.int64, device=device)
    u = _hash32(_hash32((2 * j) ^ k1) ^ k2)
    v = _hash32(_hash32((2 * j + 1) ^ k1) ^ k2)
    del j
    s = (u & 0xFFFF) + (u >> 16) + (v & 0xFFFF) + (v >> 16) - IH4_MEAN
    del u, v
    c = torch.tensor(sigma / IH4_STD, dtype=torch.float32, device=device)
    z = s.to(torch.float32) * c
    del s
    return z if out_dtype == torch.float32 else z.to(out_dtype)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a bf16 torch tensor, as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# Routing (input generation: it precedes the expert computation)
# --------------------------------------------------------------------------

def routing_softmax_topk(logits: np.ndarray, topk: int, bias: Optional[np.ndarray] = None):
    """softmax over experts (after adding the per-expert bias), keep the top-k
    probabilities (ties to the lower expert id), renormalise them to sum 1.

    Returns ids int32 [M,topk] in descending-probability order and weights
    float32 [M,topk]."""
    z = logits.astype(np.float64)
    if bias is not None:
        z = z + bias.astype(np.float64)[None, :]
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    pk = np.take_along_axis(p, order, axis=1)
    w = pk / pk.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def routing_affine_ep_share(M: int, topk: int, global_experts: int, local_experts: int):
    """The affine route map of the MegaMoE EP16 example: global id of slot
    (t, j) is ((t*topk + j)*73 + 19) mod global_experts, every slot weighted
    1/topk.  This GPU holds the experts [0, local_experts).  Returns the
    host-masked local form (other ids -1 with weight 0) and the global form
    (global ids, unmasked weights) that goes with ``ep_expert_map``."""
    t = np.arange(M, dtype=np.int64)[:, None]
    j = np.arange(topk, dtype=np.int64)[None, :]
    gid = ((t * topk + j) * 73 + 19) % global_experts
    local = gid < local_experts
    ids = np.where(local, gid, -1).astype(np.int32)
    w = np.where(local, np.float32(1.0 / topk), np.float32(0.0)).astype(np.float32)
    gw = np.full(gid.shape, np.float32(1.0 / topk), dtype=np.float32)
    return ids, w, gid.astype(np.int32), gw


def ep_expert_map(global_experts: int, local_experts: int, rank: int = 0) -> np.ndarray:
    """int32 [global_experts]: rank ``rank`` of an expert-parallel group holds
    the global experts [rank*local_experts, (rank+1)*local_experts) as local
    ids 0.., every other entry is -1."""
    g = np.arange(global_experts, dtype=np.int64)
    lo = rank * local_experts
    return np.where((g >= lo) & (g < lo + local_experts), g - lo, -1).astype(np.int32)


def batched_zipf_rows(E: int, max_tokens: int, n_out: int, slot_pool: int, seed: int,
                      alpha: float = 1.2):
    """Per-expert valid row counts min(max_tokens, Multinomial(slot_pool, p))
    with p_e proportional to (e+1)^-alpha, and for each valid row an output
    token id ~ U{0..n_out-1} and a weight ~ U(0,1) (float32).  Entries of
    invalid rows are -1 / 0 and must never be read."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77])))
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-alpha)
    p /= p.sum()
    counts = np.minimum(rng.multinomial(slot_pool, p), max_tokens).astype(np.int32)
    tok = rng.integers(0, n_out, size=(E, max_tokens), dtype=np.int64).astype(np.int32)
    w = rng.random((E, max_tokens), dtype=np.float32)
    valid = np.arange(max_tokens)[None, :] < counts[:, None]
    tok = np.where(valid, tok, -1).astype(np.int32)
    w = np.where(valid, w, np.float32(0)).astype(np.float32)
    return counts, tok, w


# --------------------------------------------------------------------------
# Whole input sets
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    cfg: MoEConfig
    device: str
    # contiguous
    x: Optional[torch.Tensor] = None            # bf16 [M,K]
    topk_ids: Optional[np.ndarray] = None       # int32 [M,topk]
    topk_weights: Optional[np.ndarray] = None   # float32 [M,topk]
    global_ids: Optional[np.ndarray] = None     # int32 [M,topk] (affine routing only)
    global_weights: Optional[np.ndarray] = None # float32 [M,topk], unmasked (affine routing only)
    # batched
    a: Optional[torch.Tensor] = None            # bf16 [E,max_tokens,K]
    expert_num_tokens: Optional[np.ndarray] = None  # int32 [E]
    row_token: Optional[np.ndarray] = None      # int32 [E,max_tokens]
    row_weight: Optional[np.ndarray] = None     # float32 [E,max_tokens]
    # weights: bf16 for bf16 configs, float32 for mxfp8 configs (each side
    # quantises them itself)
    w1: Optional[torch.Tensor] = None           # [E,2I,K]
    w2: Optional[torch.Tensor] = None           # [E,K,I]


def expert_w1(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    dt = torch.float32 if cfg.w_dtype == "mxfp8" else torch.bfloat16
    return ih4_normal(2 * cfg.I * cfg.K, 1.0 / math.sqrt(cfg.K), cfg.seed, TAG_W1, e,
                      device=device, out_dtype=dt).view(2 * cfg.I, cfg.K)


def expert_w2(cfg: MoEConfig, e: int, device="cpu") -> torch.Tensor:
    dt = torch.float32 if cfg.w_dtype == "mxfp8" else torch.bfloat16
    return ih4_normal(cfg.K * cfg.I, 1.0 / math.sqrt(cfg.I), cfg.seed, TAG_W2, e,
                      device=device, out_dtype=dt).view(cfg.K, cfg.I)


def activations(cfg: MoEConfig, device="cpu", rows: Optional[np.ndarray] = None) -> torch.Tensor:
    """x [M,K] (contiguous) or A [E*max_tokens,K] flattened (batched), bf16.
    ``rows`` selects a subset of rows (regenerated from the counter)."""
    tag = TAG_X if cfg.layout == "contiguous" else TAG_A
    nrows = cfg.M if cfg.layout == "contiguous" else cfg.E * cfg.max_tokens
    if rows is None:
        out = torch.empty((nrows, cfg.K), dtype=torch.bfloat16, device=device)
        step = max(1, (1 << 26) // cfg.K)
        for r0 in range(0, nrows, step):
            r1 = min(nrows, r0 + step)
            out[r0:r1] = ih4_normal((r1 - r0) * cfg.K, 1.0, cfg.seed, tag, 0, start=r0 * cfg.K,
                                    device=device).view(r1 - r0, cfg.K)
        return out
    return torch.stack([ih4_normal(cfg.K, 1.0, cfg.seed, tag, 0, start=int(r) * cfg.K, device=device)
                        for r in rows]) if len(rows) else torch.empty((0, cfg.K), dtype=torch.bfloat16)


def make_routing(cfg: MoEConfig):
    """Top-k ids/weights (contiguous) or counts/map (batched), on the host."""
    if cfg.layout == "batched":
        return batched_zipf_rows(cfg.E, cfg.max_tokens, cfg.M, cfg.slot_pool, cfg.seed)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 11])))
    if cfg.routing == "softmax_topk":
        logits = rng.standard_normal((cfg.M, cfg.E))
        return routing_softmax_topk(logits, cfg.topk)
    if cfg.routing == "softmax_topk_bias":
        logits = rng.standard_normal((cfg.M, cfg.E))
        bias = rng.normal(0.0, 0.5, size=cfg.E)
        return routing_softmax_topk(logits, cfg.topk, bias)
    if cfg.routing == "affine_ep_share":
        return routing_affine_ep_share(cfg.M, cfg.topk, cfg.global_experts, cfg.E)
    raise ValueError(cfg.routing)


def make_inputs(cfg: MoEConfig, device="cpu", weights: bool = True) -> Inputs:
    inp = Inputs(cfg=cfg, device=str(device))
    if cfg.layout == "contiguous":
        r = make_routing(cfg)
        inp.topk_ids, inp.topk_weights = r[0], r[1]
        if len(r) > 2:
            inp.global_ids, inp.global_weights = r[2], r[3]
        inp.x = activations(cfg, device)
    else:
        inp.expert_num_tokens, inp.row_token, inp.row_weight = make_routing(cfg)
        inp.a = activations(cfg, device).view(cfg.E, cfg.max_tokens, cfg.K)
    if weights:
        dt = torch.float32 if cfg.w_dtype == "mxfp8" else torch.bfloat16
        inp.w1 = torch.empty((cfg.E, 2 * cfg.I, cfg.K), dtype=dt, device=device)
        inp.w2 = torch.empty((cfg.E, cfg.K, cfg.I), dtype=dt, device=device)
        for e in range(cfg.E):
            inp.w1[e] = expert_w1(cfg, e, device)
            inp.w2[e] = expert_w2(cfg, e, device)
    return inp


# --------------------------------------------------------------------------
# Training grouped GEMMs
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class TrainConfig:
    name: str
    seed: int
    E: int                   # groups (experts)
    N: int                   # output features of the forward (W[e] is [N, K])
    K: int                   # contraction of the forward
    rows: int                # R: rows over all groups
    balance: str = "balanced"  # "balanced" | "zipf" (Zipf(1.2) sizes, two empty groups)

    def scaled(self, **kw) -> "TrainConfig":
        return dataclasses.replace(self, **kw)


TRAIN_CONFIGS = [
    TrainConfig("train_small_e8_n256_k384_r1000", 20, E=8, N=256, K=384, rows=1000, balance="zipf"),
    TrainConfig("train_gu_e32_n4096_k6144_r32768", 21, E=32, N=4096, K=6144, rows=32768),
    TrainConfig("train_dn_e32_n6144_k2048_r32768", 22, E=32, N=6144, K=2048, rows=32768),
]


def train_config(name: str) -> TrainConfig:
    for c in TRAIN_CONFIGS:
        if c.name == name or c.name.split("_")[1] == name or "_".join(c.name.split("_")[:2]) == name:
            return c
    raise KeyError(name)


def train_group_sizes(cfg: TrainConfig) -> np.ndarray:
    """Rows per group: R/E each (the remainder to the first groups), or
    Zipf(1.2)-distributed over all but groups 2 and E-1, which stay empty."""
    if cfg.balance == "balanced":
        sizes = np.full(cfg.E, cfg.rows // cfg.E, dtype=np.int64)
        sizes[: cfg.rows % cfg.E] += 1
        return sizes
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, 31])))
    live = [e for e in range(cfg.E) if e not in (2, cfg.E - 1)]
    p = np.arange(1, len(live) + 1, dtype=np.float64) ** -1.2
    sizes = np.zeros(cfg.E, dtype=np.int64)
    sizes[live] = rng.multinomial(cfg.rows, p / p.sum())
    return sizes


@dataclasses.dataclass
class TrainInputs:
    cfg: TrainConfig
    offsets: np.ndarray          # int32 [E+1]
    x: torch.Tensor              # bf16 [R, K]
    dy: torch.Tensor             # bf16 [R, N]
    w: torch.Tensor              # bf16 [E, N, K]
    main_grad: torch.Tensor      # float32 [E, N, K]; groups without rows hold -0.0


def make_train_inputs(cfg: TrainConfig, device="cpu") -> TrainInputs:
    sizes = train_group_sizes(cfg)
    off = np.zeros(cfg.E + 1, dtype=np.int32)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1])

    def big(n_rows, n_cols, sigma, tag):
        out = torch.empty((n_rows, n_cols), dtype=torch.bfloat16, device=device)
        step = max(1, (1 << 26) // n_cols)
        for r0 in range(0, n_rows, step):
            r1 = min(n_rows, r0 + step)
            out[r0:r1] = ih4_normal((r1 - r0) * n_cols, sigma, cfg.seed, tag, 0, start=r0 * n_cols,
                                    device=device).view(r1 - r0, n_cols)
        return out

    x = big(R, cfg.K, 1.0, TAG_TX)
    dy = big(R, cfg.N, 1.0, TAG_TDY)
    w = torch.empty((cfg.E, cfg.N, cfg.K), dtype=torch.bfloat16, device=device)
    g = torch.empty((cfg.E, cfg.N, cfg.K), dtype=torch.float32, device=device)
    for e in range(cfg.E):
        w[e] = ih4_normal(cfg.N * cfg.K, 1.0 / math.sqrt(cfg.K), cfg.seed, TAG_TW, e,
                          device=device).view(cfg.N, cfg.K)
        g[e] = ih4_normal(cfg.N * cfg.K, 1.0, cfg.seed, TAG_TG, e, device=device,
                          out_dtype=torch.float32).view(cfg.N, cfg.K)
        if sizes[e] == 0:
            g[e] = -0.0
    return TrainInputs(cfg=cfg, offsets=off, x=x, dy=dy, w=w, main_grad=g)

