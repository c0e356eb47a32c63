"""Pins for the oracle's threshold form of confidence unmasking and its
adaptive-step loop (CPU only): hand-worked cases, and the two limits in which
the rule coincides with the separately pinned count form (gamma at or above 1:
top-1; gamma below 0: every masked position)."""
import math

import numpy as np
import pytest

import oracle
from golden_util import load

G = load("unmask_threshold_hand_cases.json")


def _val(v):
    if v == "ln9":
        return math.log(9.0)
    if v == "ln99":
        return math.log(99.0)
    return float(v)


def _rows(rows):
    return np.array([[_val(v) for v in r] for r in rows], dtype=np.float32)


def test_hand_sequence_by_gamma():
    c = G["sequence"]
    lg, mask = _rows(c["logits"]), np.array([c["mask"]], np.uint8)
    for gamma, want in c["by_gamma"]:
        ids, commit, conf, ns = oracle.unmask_threshold(lg, mask, gamma)
        assert commit[0].tolist() == want, gamma
        assert ns.tolist() == [1]
        assert ids[0].tolist() == [0] * 6


def test_hand_fallback_tie():
    c = G["fallback_tie"]
    _, commit, conf, _ = oracle.unmask_threshold(_rows(c["logits"]), np.array([c["mask"]], np.uint8),
                                                 c["gamma"])
    assert conf[0, 1] == conf[0, 2] == 0.5
    assert commit[0].tolist() == c["commit"]


def test_hand_empty_mask():
    c = G["empty_mask"]
    _, commit, _, ns = oracle.unmask_threshold(_rows(c["logits"]), np.array([c["mask"]], np.uint8),
                                               c["gamma"], np.array([c["nsteps_in"]], np.int32))
    assert commit[0].tolist() == c["commit"]
    assert ns.tolist() == [c["nsteps_out"]]


def test_hand_adaptive_loop():
    c = G["loop"]
    steps = [np.stack([_rows(seq) for seq in step]).reshape(2 * 4, 4) for step in c["logits"]]
    res = oracle.adaptive_unmask_loop(steps, 2, 4, c["gamma"], c["max_steps"])
    assert res["steps"] == c["steps"]
    assert [cm.tolist() for cm in res["commit"]] == c["commit"]
    assert res["nsteps"].tolist() == c["nsteps"]
    assert not res["mask"][-1].any()


def _random_block(rng, B, S, V):
    """Logits with repeated rows (exact confidence ties) and a random mask."""
    pool = (rng.standard_normal((4, V)) * rng.uniform(0.5, 4.0, size=(4, 1))).astype(np.float32)
    lg = pool[rng.integers(0, 4, size=B * S)]
    mask = (rng.random((B, S)) < 0.7).astype(np.uint8)
    return lg, mask


@pytest.mark.parametrize("seed", range(6))
def test_gamma_one_is_top1(seed):
    """No confidence exceeds 1, so every step falls back to the single most
    confident masked position: the count form with k = 1."""
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    lg, mask = _random_block(rng, 3, 8, 6)
    _, ct, _, _ = oracle.unmask_threshold(lg, mask, 1.0)
    _, ck, _ = oracle.unmask(lg, mask, np.ones(3, np.int32))
    assert np.array_equal(ct, ck)


@pytest.mark.parametrize("seed", range(6))
def test_negative_gamma_commits_every_masked(seed):
    """Every confidence is positive, so gamma < 0 commits the whole mask: the
    count form with k = #masked."""
    rng = np.random.Generator(np.random.PCG64(200 + seed))
    lg, mask = _random_block(rng, 3, 8, 6)
    _, ct, _, _ = oracle.unmask_threshold(lg, mask, -0.5)
    _, ck, _ = oracle.unmask(lg, mask, mask.sum(axis=1).astype(np.int32))
    assert np.array_equal(ct, ck)
    assert np.array_equal(ct, mask)


@pytest.mark.parametrize("seed", range(6))
def test_rule_properties(seed):
    """Commits are masked positions only; every masked position above gamma is
    committed and nothing at or below it, unless none is above, in which case
    exactly one position is committed."""
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    lg, mask = _random_block(rng, 4, 8, 6)
    gamma = float(rng.uniform(0.2, 0.9))
    _, commit, conf, ns = oracle.unmask_threshold(lg, mask, gamma)
    assert not (commit & (1 - mask)).any()
    for b in range(4):
        above = (mask[b] == 1) & (conf[b] > gamma)
        if above.any():
            assert np.array_equal(commit[b] == 1, above)
        elif mask[b].any():
            assert commit[b].sum() == 1
        else:
            assert commit[b].sum() == 0
        assert ns[b] == (1 if mask[b].any() else 0)


def test_loop_budget_stops_unresolved_blocks():
    """With gamma above every confidence each step commits one position, so an
    S-slot block needs S steps; a smaller budget leaves the rest masked."""
    rng = np.random.Generator(np.random.PCG64(5))
    lg = rng.standard_normal((2 * 8, 16)).astype(np.float32)
    res = oracle.adaptive_unmask_loop([lg], 2, 8, 1.0, 5)
    assert res["steps"] == 5
    assert res["nsteps"].tolist() == [5, 5]
    assert res["mask"][-1].sum(axis=1).tolist() == [3, 3]
    full = oracle.adaptive_unmask_loop([lg], 2, 8, 1.0, 16)
    assert full["steps"] == 8 and not full["mask"][-1].any()
