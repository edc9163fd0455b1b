"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/moe_mi355x.h declares, agrees with the binding on struct
layouts, and validates problems / lays out workspaces as documented."""
import os
import re

import pytest

import moe_inputs as mi
import mixture_experts_expert_align_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(moe_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_function():
    lib = moe.load_library()
    names = header_functions()
    assert {"moe_plan_init", "moe_apply_contiguous", "moe_apply_batched", "moe_align_permute",
            "moe_topk_reduce_contiguous", "moe_topk_reduce_naive_batched",
            "moe_quantize_mxfp8"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strings():
    assert moe.moe_abi_version() == moe.ABI_VERSION
    assert moe.moe_status_string(0) == "ok"
    assert moe.moe_status_string(2) == "unsupported problem"


def plan_for(cfg, **kw):
    prob = moe.make_problem(cfg.M, cfg.K, cfg.I, cfg.E, topk=cfg.topk, max_tokens=cfg.max_tokens,
                            layout=0 if cfg.layout == "contiguous" else 1,
                            w_dtype=0 if cfg.w_dtype == "bf16" else 1,
                            w1_order=0 if cfg.w1_order == "halves" else 1, **kw)
    return moe.moe_plan_init(prob)


@pytest.mark.parametrize("idx", range(5))
def test_plans_of_the_five_workloads(idx):
    cfg = mi.config(idx)
    p = plan_for(cfg)
    if cfg.layout == "contiguous":
        R = cfg.M * cfg.topk
        assert p.routes == R and p.reduce_kind == moe.REDUCE_NOOP
        B = p.block_m
        assert p.max_active == min(cfg.E, R)
        assert p.max_tiles == (R + p.max_active * (B - 1)) // B
        assert p.sorted_capacity == p.max_tiles * B
        assert p.ws2_bytes >= R * cfg.K * 2
        assert p.out_rows == cfg.M and p.out_cols == cfg.K
    else:
        assert p.reduce_kind == moe.REDUCE_NAIVE_BATCHED and p.variant == moe.VARIANT_TILE
    expected_variant = {0: moe.VARIANT_FUSED, 1: moe.VARIANT_STREAM, 2: moe.VARIANT_TILE,
                        3: moe.VARIANT_TILE, 4: moe.VARIANT_TILE}[idx]
    assert p.variant == expected_variant, p.reason
    # sub-buffers are in order, 256-byte aligned, and inside ws13
    offs = [p.off_counts, p.off_offsets, p.off_sorted_ids, p.off_block_expert,
            p.off_num_post_padded, p.off_active, p.off_status, p.off_align_scratch, p.off_z]
    if cfg.w_dtype == "mxfp8":
        offs += [p.off_z_scale, p.off_xq, p.off_xq_scale]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert offs[-1] < p.ws13_bytes
    if idx == 2:
        assert p.sorted_capacity == 98048            # floor((65536 + 128 * 255) / 256) * 256
    if idx == 3:
        assert p.block_m == 64                       # MXFP8 tiles: 64 routes
    if idx == 4:
        assert moe.moe_naive_batched_ws_bytes(p, 512) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), moe.MOE_EINVAL), (dict(K=-1), moe.MOE_EINVAL), (dict(topk=9), moe.MOE_EINVAL),
    (dict(layout=7), moe.MOE_EINVAL), (dict(w_dtype=3), moe.MOE_EINVAL),
    (dict(variant=5), moe.MOE_EINVAL), (dict(K=4000), moe.MOE_EUNSUPPORTED),
    (dict(I=100), moe.MOE_EUNSUPPORTED), (dict(M=1 << 30), moe.MOE_EINVAL), (dict(M=1 << 28), moe.MOE_EUNSUPPORTED),
    (dict(layout=1, max_tokens=0), moe.MOE_EINVAL),
    (dict(layout=1, max_tokens=64, variant=moe.VARIANT_STREAM), moe.MOE_EUNSUPPORTED),
    (dict(layout=1, max_tokens=64, w_dtype=moe.W_MXFP8), moe.MOE_EUNSUPPORTED),
    (dict(K=128, variant=moe.VARIANT_TILE), moe.MOE_EUNSUPPORTED),   # contiguous tiles need K % 256
    (dict(global_experts=4), moe.MOE_EINVAL),             # fewer global than local experts
    (dict(global_experts=1 << 31), moe.MOE_EINVAL),
    (dict(layout=1, max_tokens=64, global_experts=16), moe.MOE_EINVAL),
    (dict(K=128, I=96, layout=1, max_tokens=64), moe.MOE_EUNSUPPORTED),
    (dict(w1_order=moe.W1_INTERLEAVE16, I=72), moe.MOE_EINVAL),
    (dict(variant=moe.VARIANT_FUSED, w_dtype=moe.W_MXFP8), moe.MOE_EUNSUPPORTED),
    (dict(variant=moe.VARIANT_FUSED, layout=1, max_tokens=64), moe.MOE_EUNSUPPORTED),
    (dict(variant=moe.VARIANT_FUSED, M=4097), moe.MOE_EUNSUPPORTED),      # M*topk > 8192
    (dict(variant=moe.VARIANT_FUSED, E=2049), moe.MOE_EUNSUPPORTED),
    (dict(variant=moe.VARIANT_FUSED, K=200), moe.MOE_EUNSUPPORTED),
    # grouped MXFP8 scales: K and I multiples of 512, tile kernels, contiguous
    (dict(K=512, I=384, w_dtype=moe.W_MXFP8_GROUPED), moe.MOE_EUNSUPPORTED),
    (dict(K=384, I=512, w_dtype=moe.W_MXFP8_GROUPED), moe.MOE_EUNSUPPORTED),
    (dict(K=512, I=512, w_dtype=moe.W_MXFP8_GROUPED, variant=moe.VARIANT_STREAM), moe.MOE_EUNSUPPORTED),
    (dict(K=512, I=512, w_dtype=moe.W_MXFP8_GROUPED, layout=1, max_tokens=64), moe.MOE_EUNSUPPORTED),
])
def test_plan_validation(kw, code):
    base = dict(M=64, K=256, I=512, E=8, topk=2)
    base.update(kw)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_plan_init(moe.make_problem(**base))
    assert ei.value.status == code
    assert str(ei.value)


def test_global_experts_topk_range():
    """With global ids, topk is bounded by the global id space, not by E."""
    p = moe.moe_plan_init(moe.make_problem(64, 256, 512, 2, topk=8, global_experts=512))
    assert p.prob.global_experts == 512
    with pytest.raises(moe.MoeError):
        moe.moe_plan_init(moe.make_problem(64, 256, 512, 2, topk=8))


def test_mxfp8_grouped_plan():
    """Grouped MXFP8 scale arrays plan like row-major ones (the tiles, the
    same workspace layout and sizes: only the scale bytes' order differs)."""
    a = moe.moe_plan_init(moe.make_problem(512, 6144, 2048, 32, topk=8, w_dtype=moe.W_MXFP8))
    b = moe.moe_plan_init(moe.make_problem(512, 6144, 2048, 32, topk=8, w_dtype=moe.W_MXFP8_GROUPED))
    assert b.variant == moe.VARIANT_TILE and b.block_m == 64
    for f in ("ws13_bytes", "ws2_bytes", "sorted_capacity", "off_z", "off_z_scale", "off_xq", "off_xq_scale"):
        assert getattr(a, f) == getattr(b, f), f


def test_mxfp8_tile_shapes():
    """The MXFP8 tiles (128 weight rows: 64 W1 features, 128 W2 rows) take
    every shape the MXFP8 kernels take (K and I multiples of 128); the
    streaming kernels only when asked for."""
    for K, I in [(128, 128), (384, 256), (6144, 2048)]:
        p = moe.moe_plan_init(moe.make_problem(512, K, I, 32, topk=8, w_dtype=moe.W_MXFP8))
        assert p.variant == moe.VARIANT_TILE and p.block_m == 64
    p = moe.moe_plan_init(moe.make_problem(512, 384, 256, 32, topk=8, w_dtype=moe.W_MXFP8,
                                           variant=moe.VARIANT_STREAM))
    assert p.variant == moe.VARIANT_STREAM and p.block_m == 16


def test_batched_tile_shapes():
    """The batched tiles (128 weight rows) need only K % 128 and I % 64."""
    p = moe.moe_plan_init(moe.make_problem(64, 128, 64, 8, max_tokens=64, layout=moe.LAYOUT_BATCHED))
    assert p.variant == moe.VARIANT_TILE


def test_variant_choice_and_override():
    p = moe.moe_plan_init(moe.make_problem(64, 256, 512, 8, topk=2))          # small layer
    assert p.variant == moe.VARIANT_FUSED
    p = moe.moe_plan_init(moe.make_problem(300, 256, 512, 8, topk=2))         # 75 rows per expert
    assert p.variant == moe.VARIANT_TILE and p.block_m == 256
    p = moe.moe_plan_init(moe.make_problem(16, 4096, 8192, 64, topk=8))       # weights past 1 GiB
    assert p.variant == moe.VARIANT_STREAM
    p = moe.moe_plan_init(moe.make_problem(17, 4096, 8192, 64, topk=8))
    assert p.variant == moe.VARIANT_TILE and p.block_m == 256
    p = moe.moe_plan_init(moe.make_problem(17, 256, 512, 8, topk=2, variant=moe.VARIANT_STREAM))
    assert p.variant == moe.VARIANT_STREAM and p.block_m == 16
    assert "stream" in moe.moe_plan_reason(p)


def test_align_path_choice():
    small = moe.moe_plan_init(moe.make_problem(1024, 256, 512, 8, topk=8))     # R = 8192
    big = moe.moe_plan_init(moe.make_problem(1025, 256, 512, 8, topk=8))       # R = 8200
    assert small.align_blocks == 0
    assert big.align_blocks == 9                                                # chunks of 1024
    huge = moe.moe_plan_init(moe.make_problem(131073, 256, 512, 8, topk=8))    # R = 1048584
    assert huge.align_blocks == 1024                                            # at most 1024 chunks


def test_fused_plan():
    """The single-launch variant: streaming strips (block_m 16), the one-
    workgroup align, and a zero-initialised sync area after the other buffers."""
    p = moe.moe_plan_init(moe.make_problem(4096, 256, 512, 2048, topk=2, variant=moe.VARIANT_FUSED))
    assert p.variant == moe.VARIANT_FUSED and p.block_m == 16 and p.align_blocks == 0
    assert "fused" in moe.moe_plan_reason(p)
    assert p.off_sync >= p.off_z + p.sorted_capacity * 512 * 2
    assert p.ws13_bytes >= p.off_sync + 4 * (32 * (2 + p.max_active) + 4 * p.max_active)
    q = moe.moe_plan_init(moe.make_problem(4, 256, 512, 8, topk=2, variant=moe.VARIANT_STREAM))
    assert q.off_sync == -1


# every case fails validation before any launch, so the fake (aligned,
# non-null) pointers are never dereferenced
@pytest.mark.parametrize("R,N,K,E,acc,misalign,code", [
    (1000, 256, 384, 0, 0, 0, moe.MOE_EINVAL), (1000, 256, 384, 65536, 0, 0, moe.MOE_EINVAL),
    (-1, 256, 384, 8, 0, 0, moe.MOE_EINVAL), (1 << 31, 256, 384, 8, 0, 0, moe.MOE_EINVAL),
    (1000, 0, 384, 8, 0, 0, moe.MOE_EINVAL), (1000, 200, 384, 8, 0, 0, moe.MOE_EUNSUPPORTED),
    (1000, 256, 100, 8, 0, 0, moe.MOE_EUNSUPPORTED), (1 << 20, 2048, 128, 8, 0, 0, moe.MOE_EUNSUPPORTED),
    (1000, 256, 384, 8, 2, 0, moe.MOE_EINVAL), (1000, 256, 384, 8, 0, 8, moe.MOE_EINVAL),
])
def test_grouped_validation(R, N, K, E, acc, misalign, code):
    import ctypes
    lib = moe.load_library()
    p = moe.MoeGroupedProblem(R=R, N=N, K=K, E=E)
    fake = ctypes.c_void_p(1 << 20)
    out = ctypes.c_void_p((1 << 20) + misalign)
    assert lib.moe_grouped_wgrad(ctypes.byref(p), fake, fake, fake, out, acc, None) == code
    if acc == 0:
        assert lib.moe_grouped_dgrad(ctypes.byref(p), fake, fake, fake, out, None) == code
        assert lib.moe_grouped_forward(ctypes.byref(p), fake, fake, fake, out, None) == code


@pytest.mark.parametrize("kw", [
    # MXFP8: gathered activation codes sorted_capacity * K = 2.2 GB
    dict(M=45000, K=6144, I=2048, E=32, topk=8, w_dtype=moe.W_MXFP8, w1_order=moe.W1_INTERLEAVE16),
    # forced streaming bf16: z = sorted_capacity * I * 2 = 2.15 GB
    dict(M=65536, K=4096, I=2048, E=64, topk=8, variant=moe.VARIANT_STREAM),
    # MXFP8 z = sorted_capacity * I bytes past 2^31 with a small K
    dict(M=40000, K=128, I=8192, E=8, topk=8, w_dtype=moe.W_MXFP8),
])
def test_plan_refuses_32bit_offset_overflow(kw):
    """The streaming and MXFP8 kernels address z and the gathered activation
    codes through one buffer each with 32-bit offsets: plans whose buffers
    reach 2^31 bytes are refused instead of reading zeros past that point."""
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_plan_init(moe.make_problem(**kw))
    assert ei.value.status == moe.MOE_EUNSUPPORTED
    assert "32-bit" in str(ei.value)


def test_plan_accepts_largest_streaming_buffers_below_2g():
    """Just below the limit the same shapes plan (MXFP8 share, 30000 tokens:
    sorted_capacity * K = 1.48 GB)."""
    p = moe.moe_plan_init(moe.make_problem(30000, 6144, 2048, 32, topk=8, w_dtype=moe.W_MXFP8,
                                           w1_order=moe.W1_INTERLEAVE16))
    assert p.sorted_capacity * 6144 < (1 << 31) - 1


def test_binding_checks_dtypes_and_sizes(monkeypatch):
    """The wrappers refuse tensors of the wrong dtype or size before any call:
    int64 ids (torch.topk's dtype) would be read as int32 pairs, a bf16 dw
    would be written past its end as fp32, a short workspace overrun.  (Host
    tensors stand in for device ones: the device check is switched off, and
    every case fails a check before the library is called.)"""
    import torch
    monkeypatch.setattr(moe, "_ptr", lambda t: None if t is None else t.data_ptr())
    cfg = mi.config(0)
    plan = plan_for(cfg)
    ids64 = torch.zeros((cfg.M, cfg.topk), dtype=torch.int64)
    with pytest.raises(ValueError, match="int32"):
        moe.moe_align_permute(plan, ids64, torch.zeros(plan.ws13_bytes, dtype=torch.uint8))
    ids = torch.zeros((cfg.M, cfg.topk + 1), dtype=torch.int32)
    with pytest.raises(ValueError, match="M\\*topk"):
        moe.moe_align_permute(plan, ids, torch.zeros(plan.ws13_bytes, dtype=torch.uint8))
    ids = torch.zeros((cfg.M, cfg.topk), dtype=torch.int32)
    with pytest.raises(ValueError, match="ws13"):
        moe.moe_align_permute(plan, ids, torch.zeros(plan.ws13_bytes - 1, dtype=torch.uint8))
    x = torch.zeros((cfg.M, cfg.K), dtype=torch.float32)
    w1 = torch.zeros((cfg.E, 2 * cfg.I, cfg.K), dtype=torch.bfloat16)
    w2 = torch.zeros((cfg.E, cfg.K, cfg.I), dtype=torch.bfloat16)
    out = torch.zeros((cfg.M, cfg.K), dtype=torch.bfloat16)
    wts = torch.zeros((cfg.M, cfg.topk), dtype=torch.float32)
    ws13 = torch.zeros(plan.ws13_bytes, dtype=torch.uint8)
    ws2 = torch.zeros(plan.ws2_bytes, dtype=torch.uint8)
    with pytest.raises(ValueError, match="a: dtype"):
        moe.moe_apply_contiguous(plan, x, ids, wts, w1, w2, out, ws13, ws2)
    with pytest.raises(ValueError, match="w2"):
        moe.moe_apply_contiguous(plan, x.bfloat16(), ids, wts, w1, w2[:1], out, ws13, ws2)
    dy = torch.zeros((256, 128), dtype=torch.bfloat16)
    xx = torch.zeros((256, 128), dtype=torch.bfloat16)
    off = torch.tensor([0, 256], dtype=torch.int32)
    with pytest.raises(ValueError, match="dw"):
        moe.moe_grouped_wgrad(dy, xx, off, torch.zeros((1, 128, 128), dtype=torch.bfloat16))
