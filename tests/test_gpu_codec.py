"""moe_quantize_mxfp8 on the GPU against the oracle's codec, bit for bit
(E4M3 codes and UE8M0 scales), from float32 and from bf16, including the
cases where a rule is easiest to get wrong: block maxima at and one float32
step above 448 * 2^k, exact ties between E4M3 neighbours, subnormal
results, all-zero blocks, negative zeros and blocks at the clamps."""
import numpy as np
import pytest
import torch

import mixture_experts_expert_align_amd as moe
import oracle
from moe_cases import say

pytestmark = pytest.mark.gpu


def gpu_quantize(x: np.ndarray):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((*x.shape[:-1], x.shape[-1] // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(t, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def special_blocks() -> np.ndarray:
    rng = np.random.default_rng(7)
    rows = []
    tab = oracle.e4m3fn_table()[:127]
    mids = (tab[1:] + tab[:-1]) / 2
    for k in range(-20, 20):
        p = np.float32(448.0 * 2.0 ** k)
        for bm in (p, np.nextafter(p, np.float32(np.inf)), np.nextafter(p, np.float32(0))):
            blk = rng.standard_normal(32).astype(np.float32) * np.float32(bm / 4)
            blk[rng.integers(32)] = bm
            rows.append(np.clip(blk, -bm, bm))
        # the block max pins the scale to 2^k, the rest sit on exact ties
        blk = (rng.choice(mids, 32) * rng.choice([-1, 1], 32) * 2.0 ** k).astype(np.float32)
        blk[0] = np.float32(448.0 * 2.0 ** k)
        rows.append(blk)
    rows.append(np.zeros(32, np.float32))
    z = np.zeros(32, np.float32); z[3] = -0.0; z[5] = np.float32(-1e-30); z[6] = np.float32(1.0)
    rows.append(z)
    rows.append(np.full(32, np.float32(1e-40)))                    # float32 subnormals: scale 0
    rows.append(np.full(32, np.float32(3.0e38)) * rng.choice([-1, 1], 32).astype(np.float32))
    blk = rng.standard_normal(32).astype(np.float32); blk[:8] *= np.float32(1e-4)
    rows.append(blk)                                              # E4M3 subnormal results
    return np.stack(rows)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_codec_bit_exact(dtype):
    rng = np.random.default_rng(1)
    rand = (rng.standard_normal((333, 256)) * 2.0 ** rng.integers(-30, 30, (333, 1))).astype(np.float32)
    blocks = special_blocks()
    pad = (-blocks.shape[0]) % 8
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.float32)]).reshape(-1, 256)
    x = np.concatenate([rand, blocks])
    if dtype == "bfloat16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        ref_in = xt.float().numpy()                       # exact decode of the bf16 values
        codes, scales = gpu_quantize_bf16(xt)
    else:
        ref_in = x
        codes, scales = gpu_quantize(x)
    rc, rs = oracle.mxfp8_quantize(ref_in)
    say(f"[codec] {dtype}: {x.shape} mismatching codes {(codes != rc).sum()} scales {(scales != rs).sum()}")
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


def gpu_quantize_bf16(xt: torch.Tensor):
    t = xt.contiguous().cuda()
    codes = torch.empty(t.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((*t.shape[:-1], t.shape[-1] // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(t, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_codec_expert_weights_full_size():
    """One expert of the MXFP8 workload's W1 (4096 x 6144 float32)."""
    import moe_inputs as mi
    cfg = mi.config(3)
    w = mi.expert_w1(cfg, 5, device="cuda")
    codes = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((w.shape[0], w.shape[1] // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(w, codes, scales)
    torch.cuda.synchronize()
    rc, rs = oracle.mxfp8_quantize(w.cpu().numpy())
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_codec_every_bf16_magnitude():
    """Every bf16 value of magnitude <= 448 (both signs, subnormals, +-0),
    31 to a block next to a 448: the block scale is 2^0, so the E4M3 rounding
    sees each value unscaled.  Through the float32 and the bf16 entry."""
    bits = np.arange(0, 0x43E1, dtype=np.uint32)
    vals = np.concatenate([bits, bits | 0x8000]).astype(np.uint32) << 16
    vals = vals.view(np.float32)
    nblk = -(-vals.size // 31)
    blocks = np.zeros((nblk, 32), np.float32)
    blocks[:, 0] = 448.0
    blocks[:, 1:].flat[:vals.size] = vals
    pad = (-nblk) % 8
    x = np.concatenate([blocks, np.zeros((pad, 32), np.float32)]).reshape(-1, 256)
    rc, rs = oracle.mxfp8_quantize(x)
    assert np.all(rs[: nblk // 8] == 127)
    codes, scales = gpu_quantize(x)
    assert np.array_equal(scales, rs) and np.array_equal(codes, rc)
    codes, scales = gpu_quantize_bf16(torch.from_numpy(x).to(torch.bfloat16))
    say(f"[codec] every bf16 magnitude <= 448: {vals.size} values, mismatching codes {(codes != rc).sum()}")
    assert np.array_equal(scales, rs) and np.array_equal(codes, rc)
