"""Pins for the oracle's confidence unmask (CPU only): hand-worked cases,
library routines (numpy argmax, scipy logsumexp), and brute-force enumeration
of commit sets on tiny blocks."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from golden_util import load

G = load("unmask_hand_cases.json")


def _row(vals):
    return np.array([float(v) for v in vals], dtype=np.float32)


@pytest.mark.parametrize("row", G["rows"], ids=lambda r: str(r["logits"]))
def test_hand_rows(row):
    lg = _row(row["logits"])[None, :]
    ids, commit, conf = oracle.unmask(lg, np.ones((1, 1), np.uint8), np.array([1], np.int32))
    assert ids[0, 0] == row["id"]
    assert commit[0, 0] == 1
    assert conf[0, 0] == pytest.approx(row["conf"], rel=1e-15, abs=0)


def _commit_inputs():
    cc = G["commit_cases"]
    lg = np.stack([_row(r) for r in cc["logits"]])          # [S, 2]
    mask = np.array(cc["mask"], dtype=np.uint8)[None, :]
    return cc, lg, mask


def test_hand_commit_by_k():
    cc, lg, mask = _commit_inputs()
    for k, want in cc["by_k"]:
        ids, commit, conf = oracle.unmask(lg, mask, np.array([k], np.int32))
        assert commit[0].tolist() == want, (k, commit)
        assert ids[0].tolist() == [0, 0, 0, 0]


def test_hand_commit_by_remaining_steps():
    cc, lg, mask = _commit_inputs()
    for rem, want in cc["by_remaining"]:
        _, commit, _ = oracle.unmask(lg, mask, None, rem)
        assert commit[0].tolist() == want, (rem, commit)


def test_conf_and_ids_against_library():
    rng = np.random.Generator(np.random.PCG64(21))
    B, S, V = 3, 16, 1000
    lg = (3 * rng.standard_normal((B * S, V))).astype(np.float32)
    lg[5, 17] = -np.inf
    lg[7, :] = np.float32(1.5)                               # all equal -> id 0, conf 1/V
    lg[9, 400] = lg[9, 100] = lg[9].max() + 1               # tie -> 100
    ids, _, conf = oracle.unmask(lg, np.ones((B, S), np.uint8), np.full(B, 3, np.int32))
    lg64 = lg.astype(np.float64)
    assert np.array_equal(ids.reshape(-1), np.argmax(lg, axis=1))
    want = np.exp(lg64.max(axis=1) - logsumexp(lg64, axis=1))
    np.testing.assert_allclose(conf.reshape(-1), want, rtol=1e-12)
    assert ids.reshape(-1)[9] == 100 and ids.reshape(-1)[7] == 0
    assert conf.reshape(-1)[7] == pytest.approx(1.0 / V, rel=1e-14)


def _brute_force(conf, mask, k):
    """Among all k-subsets of masked positions, the one whose confidences,
    sorted descending, are lexicographically largest; ties between subsets go
    to the lexicographically smallest sorted position set."""
    cand = [t for t in range(len(mask)) if mask[t]]
    k = max(0, min(k, len(cand)))
    best = None
    for sub in itertools.combinations(cand, k):
        key = (tuple(sorted((conf[t] for t in sub), reverse=True)), tuple(-t for t in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    out = np.zeros(len(mask), np.uint8)
    out[list(best[1])] = 1
    return out


@pytest.mark.parametrize("seed", range(12))
def test_commit_brute_force(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    B, S, V = 4, 8, 6
    # few distinct logit rows so that equal confidences (ties) are common
    pool = (2 * rng.standard_normal((3, V))).astype(np.float32)
    lg = pool[rng.integers(0, 3, size=B * S)]
    mask = (rng.random((B, S)) < 0.6).astype(np.uint8)
    mask[0] = 1
    mask[1] = 0
    k = rng.integers(-1, S + 2, size=B).astype(np.int32)
    ids, commit, conf = oracle.unmask(lg, mask, k)
    for b in range(B):
        want = _brute_force(conf[b], mask[b], int(k[b]))
        assert np.array_equal(commit[b], want), (b, conf[b], mask[b], k[b])
        assert commit[b].sum() == max(0, min(int(k[b]), int(mask[b].sum())))
        assert not np.any(commit[b] & (1 - mask[b]))


def test_remaining_steps_counts():
    rng = np.random.Generator(np.random.PCG64(9))
    B, S, V = 5, 16, 32
    lg = rng.standard_normal((B * S, V)).astype(np.float32)
    mask = np.ones((B, S), np.uint8)
    mask[1, :5] = 0
    mask[2] = 0
    for rem in (1, 2, 3, 4, 16, 40):
        _, commit, _ = oracle.unmask(lg, mask, None, rem)
        for b in range(B):
            n = int(mask[b].sum())
            assert commit[b].sum() == math.ceil(n / rem)


def test_single_vocab_entry():
    lg = np.array([[3.0], [-1.0]], dtype=np.float32)
    ids, commit, conf = oracle.unmask(lg, np.array([[1, 1]], np.uint8), np.array([1], np.int32))
    assert ids.tolist() == [[0, 0]]
    assert conf.tolist() == [[1.0, 1.0]]
    assert commit.tolist() == [[1, 0]]     # equal confidences -> lower position
