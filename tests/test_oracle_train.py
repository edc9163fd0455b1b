"""Pins of the oracle's training grouped GEMMs ([DET] introduction: forward,
dgrad and wgrad of a ragged bf16 grouped GEMM; section 1: the fp32
accumulate; section 2: an empty sum is +0.0).

The pins do not restate the definitions: dgrad and wgrad are checked as the
gradients of the forward (central differences of a bilinear loss are exact
up to rounding, so a transposed operand, a wrong group or a dropped row
fails), the forward against closed forms (scalar-identity weights, one row
per group), and the sign rules of the page.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def ragged(E, sizes):
    off = np.zeros(E + 1, dtype=np.int64)
    off[1:] = np.cumsum(sizes)
    return off


def case(seed=0, E=5, N=6, K=7, sizes=(3, 0, 1, 4, 2)):
    rng = np.random.default_rng(seed)
    off = ragged(E, sizes)
    R = int(off[-1])
    return (rng.standard_normal((R, K)), rng.standard_normal((E, N, K)), rng.standard_normal((R, N)),
            off)


def loss(g, x, w, off):
    """L = <g, forward(x, W)>: bilinear in (x, W)."""
    return float(np.sum(g * oracle.grouped_forward(x, w, off)))


def pin_dgrad_is_the_input_gradient():
    for seed in (0, 1, 2):
        x, w, g, off = case(seed)
        d = np.random.default_rng(100 + seed).standard_normal(x.shape)
        h = 0.5
        fd = (loss(g, x + h * d, w, off) - loss(g, x - h * d, w, off)) / (2 * h)
        an = float(np.sum(oracle.grouped_dgrad(g, w, off) * d))
        assert abs(fd - an) <= 1e-10 * (1 + abs(an))


def pin_wgrad_is_the_weight_gradient():
    for seed in (0, 1, 2):
        x, w, g, off = case(seed)
        d = np.random.default_rng(200 + seed).standard_normal(w.shape)
        h = 0.5
        fd = (loss(g, x, w + h * d, off) - loss(g, x, w - h * d, off)) / (2 * h)
        an = float(np.sum(oracle.grouped_wgrad(g, x, off) * d))
        assert abs(fd - an) <= 1e-10 * (1 + abs(an))


def pin_forward_scalar_identity_weights():
    """W[e] = c_e I: y[r] = c_e x[r] with the scale of the row's own group."""
    E, K = 4, 5
    sizes = (2, 3, 0, 1)
    off = ragged(E, sizes)
    c = np.array([2.0, -3.0, 5.0, 0.5])
    w = c[:, None, None] * np.eye(K)[None]
    x = np.random.default_rng(5).standard_normal((int(off[-1]), K))
    grp = np.repeat(np.arange(E), sizes)
    np.testing.assert_array_equal(oracle.grouped_forward(x, w, off), c[grp][:, None] * x)
    # and the input gradient of the same map scales by the same c_e
    np.testing.assert_array_equal(oracle.grouped_dgrad(x, w, off), c[grp][:, None] * x)


def pin_wgrad_single_row_groups_are_outer_products():
    E, N, K = 3, 4, 6
    off = ragged(E, (1, 1, 1))
    rng = np.random.default_rng(9)
    dy, x = rng.standard_normal((3, N)), rng.standard_normal((3, K))
    dw = oracle.grouped_wgrad(dy, x, off)
    for e in range(E):
        np.testing.assert_allclose(dw[e], np.outer(dy[e], x[e]), rtol=0, atol=1e-15)


def pin_wgrad_empty_group_is_plus_zero():
    x, w, g, off = case(3, sizes=(3, 0, 1, 4, 0))
    dw = oracle.grouped_wgrad(g, x, off)
    for e in (1, 4):
        assert np.all(dw[e] == 0) and not np.any(np.signbit(dw[e]))


def pin_accumulate_turns_minus_zero_into_plus_zero():
    """[DET] section 2: with an empty group, -0.0 in main_grad becomes +0.0
    (out + (+0.0)); other groups add their gradient once."""
    x, w, g, off = case(4, sizes=(2, 0, 3, 1, 1))
    out = np.random.default_rng(6).standard_normal(w.shape).astype(np.float32)
    out[1] = -0.0
    acc = oracle.grouped_wgrad_accumulate(out, g, x, off)
    assert np.all(acc[1] == 0) and not np.any(np.signbit(acc[1]))
    np.testing.assert_allclose(acc[0] - out[0].astype(np.float64), g[:2].T @ x[:2], rtol=0, atol=1e-12)


def pin_group_boundaries():
    """Moving one row from group 0 to group 1 changes exactly those two
    groups' gradients, by that row's outer product."""
    x, w, g, off = case(7, sizes=(3, 2, 1, 1, 1))
    moved = off.copy()
    moved[1] -= 1                                   # row 2 now belongs to group 1
    a = oracle.grouped_wgrad(g, x, off)
    b = oracle.grouped_wgrad(g, x, moved)
    r = int(off[1]) - 1
    np.testing.assert_allclose(a[0] - b[0], np.outer(g[r], x[r]), atol=1e-12)
    np.testing.assert_allclose(b[1] - a[1], np.outer(g[r], x[r]), atol=1e-12)
    np.testing.assert_array_equal(a[2:], b[2:])


PINS = [pin_dgrad_is_the_input_gradient, pin_wgrad_is_the_weight_gradient,
        pin_forward_scalar_identity_weights, pin_wgrad_single_row_groups_are_outer_products,
        pin_wgrad_empty_group_is_plus_zero, pin_accumulate_turns_minus_zero_into_plus_zero,
        pin_group_boundaries]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_train_pin(pin):
    pin()

