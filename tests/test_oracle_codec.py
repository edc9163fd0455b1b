"""Pins for the oracle's MXFP8 codec (E4M3FN elements, UE8M0 block-32 scales).

The rule being pinned is the new scale rule of the Cake MegaMoE EP16 page,
section 2: per block of 32, scale exponent ceil(log2(blockmax/448)) clamped to
[0, 254] after the +127 bias, 0 for an all-zero block, decoded scale
2^(code-127).  What pins it here, other than the oracle itself:
* torch's float8_e4m3fn dtype (a library routine) for the element format;
* the page's older scale rule (exponent field of the float32 quotient plus
  one when its mantissa is non-zero), an independent formula that agrees with
  the exact rule except where the float32 quotient rounds across a power of
  two or the clamp/zero-block conventions differ;
* closed forms at powers of two and their float32 neighbours;
* round trips of exactly representable values and the format's error bound.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3_encode(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_decode_table() -> np.ndarray:
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


# ---------------------------------------------------------------- pins ----

def pin_e4m3_table():
    ours = oracle.e4m3fn_table()
    ref = torch_e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x38] == 1.0 and ours[0x01] == 2.0 ** -9


def pin_e4m3_encode_vs_torch():
    tab = torch_e4m3_decode_table()[:127]
    mids = (tab[1:] + tab[:-1]) / 2            # every tie between neighbours
    rng = np.random.default_rng(5)
    rnd = rng.uniform(-448, 448, 20000)
    small = rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 3, 20000)
    vals = np.concatenate([tab, -tab, mids, -mids, rnd, np.clip(small, -448, 448),
                           [0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 2.0 ** -11, 448.0]])
    vals = vals.astype(np.float32)             # every value here is exact in float32
    assert np.array_equal(oracle.e4m3fn_encode(vals.astype(np.float64)), torch_e4m3_encode(vals))


def pin_scale_closed_form():
    for k in range(-40, 40):
        p = np.float32(448.0 * 2.0 ** k)
        up = np.nextafter(p, np.float32(np.inf))
        dn = np.nextafter(p, np.float32(0))
        e = oracle.mx_scale_exponent(np.array([p, up, dn], dtype=np.float64))
        assert list(e) == [k, k + 1, k], (k, e)
    # codes: bias 127, clamped to [0, 254]; all-zero block -> 0
    bm = np.array([0.0, 448.0, 1.0, 448.0 * 2.0 ** -140, 1e-45, 3.0e38])
    assert list(oracle.mx_scale_code(bm)) == [0, 127, 127 - 8, 0, 0, 127 + 120]


def older_rule_codes(bm: np.ndarray) -> np.ndarray:
    """The page's older rule: float32 quotient max(bm, 1e-7) / 448, then the
    biased exponent field plus one if any mantissa bit is set, clamped to
    [1, 254]."""
    q = (np.maximum(bm.astype(np.float32), np.float32(1e-7)) / np.float32(448.0)).astype(np.float32)
    bits = q.view(np.uint32).astype(np.int64)
    code = ((bits >> 23) & 255) + ((bits & 0x7FFFFF) != 0)
    return np.clip(code, 1, 254)


def pin_scale_vs_older_rule():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((4000, 32)) * 2.0 ** rng.integers(-20, 20, (4000, 1))).astype(np.float32)
    bm = np.abs(x).max(axis=1)
    ours = oracle.mx_scale_code(bm.astype(np.float64)).astype(np.int64)
    old = older_rule_codes(bm)
    q = bm.astype(np.float64) / 448.0
    # exclude quotients within one float32 ulp of a power of two, where the
    # float32 division may round across it
    _, p = np.frexp(q)
    near = np.abs(q - np.ldexp(0.5, p)) <= q * 2.0 ** -23
    assert np.array_equal(ours[~near], old[~near])
    assert (~near).sum() > 3900


def pin_quantize_block_properties():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((512, 256)) * 2.0 ** rng.integers(-12, 12, (512, 1))).astype(np.float32)
    x[7, 32:64] = 0.0                                     # an all-zero block
    codes, scales = oracle.mxfp8_quantize(x)
    assert codes.shape == x.shape and scales.shape == (512, 8)
    assert scales[7, 1] == 0 and not codes[7, 32:64].any()
    deq = oracle.mxfp8_dequantize(codes, scales)
    xb = x.astype(np.float64).reshape(512, 8, 32)
    s = np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    rel = np.abs(deq.reshape(512, 8, 32) - xb)
    normal = np.abs(xb) / s >= 2.0 ** -6
    assert np.all(rel[normal] <= np.abs(xb[normal]) * 2.0 ** -4)
    assert np.all(rel[~normal] <= s.repeat(32, -1)[~normal] * 2.0 ** -10)
    bm = np.abs(xb).max(-1)
    nz = bm > 0
    ratio = bm[nz] / s[..., 0][nz]
    assert np.all(ratio <= 448.0) and np.all(ratio > 224.0)


def pin_roundtrip_exact():
    rng = np.random.default_rng(4)
    tab = oracle.e4m3fn_table()
    finite = np.array([c for c in range(256) if not np.isnan(tab[c])])
    codes = rng.choice(finite, size=(64, 64)).astype(np.uint8)
    codes[:, ::32] = 0x7E                                   # each block holds 448 -> scale fixed
    sc = rng.integers(100, 150, size=(64, 2)).astype(np.uint8)
    v = oracle.mxfp8_dequantize(codes, sc).astype(np.float32)
    c2, s2 = oracle.mxfp8_quantize(v)
    assert np.array_equal(s2, sc)
    # +0 and -0 both decode to zero; compare values, then codes away from zero
    assert np.array_equal(oracle.mxfp8_dequantize(c2, s2), oracle.mxfp8_dequantize(codes, sc))
    nz = tab[codes] != 0
    assert np.array_equal(c2[nz], codes[nz])


PINS = [pin_e4m3_table, pin_e4m3_encode_vs_torch, pin_scale_closed_form, pin_scale_vs_older_rule,
        pin_quantize_block_properties, pin_roundtrip_exact]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_codec_pin(pin):
    pin()


def test_bf16_decode_exact():
    vals = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 1e-38, 65280.0], dtype=np.float32)
    t = torch.from_numpy(vals).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(bits), t.to(torch.float64).numpy())
