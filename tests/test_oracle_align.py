"""Pins for the oracle's align (Permute) step.

The Permute step of the modular kernel's apply() groups the (token, slot)
routes by expert; the contiguous format marks skipped slots with id -1.
Pinned here by: a brute force built differently (a lexicographic sort of
(expert, flat index) pairs), a hand-worked example, invariants on random
routings, and two closed forms that follow from the affine route map of the
Cake MegaMoE EP16 page (section 1): with global ids ((8t+j)*73+19) mod 512
every expert gets the same load at the page's token counts (its comment says
so), and a 32-expert local share of 4096 tokens gets exactly 64 routes per
expert.
"""
import os
from collections import Counter

import numpy as np
import pytest

import moe_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_force_align(ids: np.ndarray, E: int, B: int):
    flat = ids.reshape(-1)
    pairs = sorted((int(e), i) for i, e in enumerate(flat) if 0 <= e < E)
    by_e = {e: [i for (ee, i) in pairs if ee == e] for e in range(E)}
    seq, owners = [], []
    for e in range(E):
        run = by_e[e]
        padded = -(-len(run) // B) * B
        seq += run + [flat.size] * (padded - len(run))
        owners += [e] * (padded // B)
    return by_e, seq, owners


def check_against_brute(ids, E, B):
    got = oracle.align_permute(ids, E, B)
    by_e, seq, owners = brute_force_align(ids, E, B)
    R = ids.size
    n = len(seq)
    assert got["num_post_padded"] == n
    assert list(got["sorted_ids"][:n]) == seq
    assert np.all(got["sorted_ids"][n:] == R)
    assert list(got["block_expert"][:len(owners)]) == owners
    assert np.all(got["block_expert"][len(owners):] == -1)
    assert list(got["counts"]) == [len(by_e[e]) for e in range(E)]
    assert got["capacity"] >= n and got["capacity"] % B == 0
    return got


# ---------------------------------------------------------------- pins ----

def pin_worked_example():
    # flat slots: 0:e1 1:e0 2:e1 3:skip 4:e0 5:e1 ; E=2, B=2
    ids = np.array([[1, 0], [1, -1], [0, 1]], dtype=np.int32)
    got = oracle.align_permute(ids, 2, 2)
    assert list(got["counts"]) == [2, 3]
    assert list(got["offsets"]) == [0, 2, 6]
    assert got["num_post_padded"] == 6
    # worst case over routings of 6 routes on 2 experts: (6 + 2*1)//2 = 4 tiles
    assert list(got["sorted_ids"]) == [1, 4, 0, 2, 5, 6, 6, 6]
    assert list(got["block_expert"]) == [0, 1, 1, -1]
    assert got["n_invalid"] == 0


def pin_brute_force_random():
    rng = np.random.default_rng(1)
    for trial in range(60):
        M = int(rng.integers(1, 40))
        topk = int(rng.integers(1, 5))
        E = int(rng.integers(1, 9))
        B = int(rng.choice([1, 2, 3, 4, 16]))
        ids = rng.integers(-1, E, size=(M, topk)).astype(np.int32)
        if trial % 5 == 0:
            ids[rng.random((M, topk)) < 0.1] = E + 3          # out-of-range ids are skipped
        got = check_against_brute(ids, E, B)
        assert got["n_invalid"] == int(np.count_nonzero(ids >= E))


def pin_invariants():
    rng = np.random.default_rng(2)
    M, topk, E, B = 300, 8, 16, 16
    ids = rng.integers(-1, E, size=(M, topk)).astype(np.int32)
    got = oracle.align_permute(ids, E, B)
    valid = ids[ids >= 0]
    assert got["counts"].sum() == valid.size                  # counts sum to the valid slots
    assert np.all(got["offsets"] % B == 0)
    s = got["sorted_ids"][: got["num_post_padded"]]
    real = s[s < ids.size]
    assert sorted(real.tolist()) == sorted(np.flatnonzero(ids.reshape(-1) >= 0).tolist())
    for e in range(E):
        run = got["sorted_ids"][got["offsets"][e]: got["offsets"][e] + got["counts"][e]]
        assert np.all(np.diff(run) > 0)                        # stable: ascending flat order
        assert np.all(ids.reshape(-1)[run] == e)


def pin_affine_equal_load():
    # tests/golden/cake_affine_route_map.txt: the page's token counts and loads
    rows = [l.split() for l in open(os.path.join(GOLDEN, "cake_affine_route_map.txt"))
            if l.strip() and not l.startswith("#")]
    for tokens, topk, n_exp, load in [tuple(int(v) for v in r) for r in rows]:
        _, _, gid, _ = moe_inputs.routing_affine_ep_share(tokens, topk, n_exp, n_exp)
        got = oracle.align_permute(gid, n_exp, 1)
        assert np.all(got["counts"] == load), (tokens, load)


def pin_mxfp8_share_closed_form():
    cfg = moe_inputs.config(3)
    ids, w, _, _ = moe_inputs.routing_affine_ep_share(cfg.M, cfg.topk, cfg.global_experts, cfg.E)
    got = oracle.align_permute(ids, cfg.E, 16)
    assert np.all(got["counts"] == 64) and got["counts"].sum() == 2048
    per_token = (ids >= 0).sum(axis=1)
    c = Counter(per_token.tolist())
    assert c == {0: 2304, 1: 1536, 2: 256}
    two = np.flatnonzero(per_token == 2)
    assert np.all(ids[two, 0] >= 0) and np.all(ids[two, 7] >= 0)   # slots j=0 and j=7
    assert np.all(w[ids < 0] == 0) and np.all(w[ids >= 0] == np.float32(0.125))


PINS = [pin_worked_example, pin_brute_force_random, pin_invariants, pin_affine_equal_load,
        pin_mxfp8_share_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_align_pin(pin):
    pin()
