"""Pins for the oracle's LM head + unmask (CPU only): a hand-worked case, the
identity and permutation heads (which reduce it to the separately pinned
unmask), brute force on tiny inputs, exact scaling, and row selection."""
import math

import numpy as np
import pytest

import oracle
import workloads
from golden_util import load

G = load("lmhead_hand_cases.json")
ONE = 0x3F80  # bf16 bits of 1.0


def _bits(a):
    return workloads.bf16_bits(np.asarray(a, dtype=np.float32))


def test_hand_case():
    h, w = _bits(G["hidden"]), _bits(G["weight"])
    logits = oracle.lmhead_logits(h, w)
    assert np.array_equal(logits, np.array(G["logits"], dtype=np.float64))
    mask = np.ones((1, 3), np.uint8)
    want_conf = [eval(e, {"exp": math.exp}) for e in G["conf"]]
    for k, want_commit in G["commit_by_k"]:
        ids, commit, conf = oracle.lmhead_unmask(h, w, mask, np.array([k], np.int32))
        assert ids[0].tolist() == G["ids"]
        np.testing.assert_allclose(conf[0], want_conf, rtol=1e-15, atol=0)
        assert commit[0].tolist() == want_commit, k


def _random_hidden(rng, R, H):
    return _bits(rng.standard_normal((R, H)) * rng.uniform(0.5, 3.0, size=(R, 1)))


@pytest.mark.parametrize("seed", range(4))
def test_identity_head_is_unmask(seed):
    """W = I: the logits are the hidden state itself, so the result must be the
    pinned unmask of that state, bit for bit."""
    rng = np.random.Generator(np.random.PCG64(10 + seed))
    B, S, H = 3, 4, 16
    h = _random_hidden(rng, B * S, H)
    w = np.zeros((H, H), np.uint16)
    w[np.arange(H), np.arange(H)] = ONE
    mask = (rng.random((B, S)) < 0.7).astype(np.uint8)
    k = rng.integers(0, S + 1, size=B).astype(np.int32)
    got = oracle.lmhead_unmask(h, w, mask, k)
    ref = oracle.unmask(workloads.bits_to_f32(h), mask, k)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("seed", range(3))
def test_permuted_head(seed):
    """W row v = unit vector e_pi(v): logit v is hidden[pi(v)], so the greedy id
    is pi^-1 of the hidden argmax and the confidence is unchanged."""
    rng = np.random.Generator(np.random.PCG64(20 + seed))
    B, S, H = 2, 5, 12
    h = _random_hidden(rng, B * S, H)
    pi = rng.permutation(H)
    w = np.zeros((H, H), np.uint16)
    w[np.arange(H), pi] = ONE
    mask = np.ones((B, S), np.uint8)
    ids, _, conf = oracle.lmhead_unmask(h, w, mask, np.full(B, 2, np.int32))
    ids0, _, conf0 = oracle.unmask(workloads.bits_to_f32(h), mask, np.full(B, 2, np.int32))
    inv = np.argsort(pi)
    assert np.array_equal(ids.ravel(), inv[ids0.ravel()])
    np.testing.assert_allclose(conf, conf0, rtol=1e-15)


def test_brute_force_tiny():
    rng = np.random.Generator(np.random.PCG64(30))
    R, H, V = 3, 5, 7
    h, w = _random_hidden(rng, R, H), _random_hidden(rng, V, H)
    hf, wf = workloads.bits_to_f32(h), workloads.bits_to_f32(w)
    want = [[sum(float(hf[r, j]) * float(wf[v, j]) for j in range(H)) for v in range(V)]
            for r in range(R)]
    np.testing.assert_allclose(oracle.lmhead_logits(h, w), want, rtol=1e-14, atol=1e-14)


def test_doubled_weight_doubles_logits():
    rng = np.random.Generator(np.random.PCG64(31))
    h, w = _random_hidden(rng, 6, 20), _random_hidden(rng, 9, 20)
    w2 = _bits(2.0 * workloads.bits_to_f32(w))  # exact in bf16
    assert np.array_equal(oracle.lmhead_logits(h, w2), 2.0 * oracle.lmhead_logits(h, w))


def test_sequence_selection():
    rng = np.random.Generator(np.random.PCG64(32))
    B, S, H, V = 4, 3, 8, 11
    h, w = _random_hidden(rng, B * S, H), _random_hidden(rng, V, H)
    mask = (rng.random((B, S)) < 0.8).astype(np.uint8)
    full = oracle.lmhead_unmask(h, w, mask, None, 2, with_logits=True)
    part = oracle.lmhead_unmask(h, w, mask, None, 2, seqs=[3, 1], with_logits=True)
    for f, p in zip(full[:3], part[:3]):
        assert np.array_equal(p, f[[3, 1]])
    assert np.array_equal(part[3], full[3].reshape(B, S, V)[[3, 1]].reshape(2 * S, V))
