"""GPU parity of tt_unmask_threshold (threshold form of the commit rule) and
of the adaptive-step loop driven through it, against the oracle."""
import math

import numpy as np
import pytest

import oracle
import workloads
from golden_util import load
from gpu_util import assert_threshold_commit_ok, dev_tensor, torch_mod

pytestmark = pytest.mark.gpu

G = load("unmask_threshold_hand_cases.json")


def _val(v):
    return {"ln9": math.log(9.0), "ln99": math.log(99.0)}.get(v, v)


def _rows(rows):
    return np.array([[float(_val(v)) for v in r] for r in rows], dtype=np.float32)


def run_threshold(logits, mask, gamma, nsteps=None, update=False):
    """One tt_unmask_threshold call; returns (ids, commit, conf, nsteps, mask after)."""
    import two_tower_attention_amd as tt
    torch = torch_mod()
    B, S = mask.shape
    V = logits.shape[-1]
    lg = dev_tensor(np.ascontiguousarray(logits, np.float32).reshape(B * S, V), "f32")
    mk = dev_tensor(np.ascontiguousarray(mask, np.uint8), "u8")
    ids = torch.empty((B, S), dtype=torch.int32, device="cuda")
    com = torch.empty((B, S), dtype=torch.uint8, device="cuda")
    conf = torch.empty((B, S), dtype=torch.float32, device="cuda")
    ns = dev_tensor(np.zeros(B, np.int32) if nsteps is None else np.asarray(nsteps, np.int32), "i32")
    ws = torch.empty(max(tt.tt_unmask_workspace_bytes(B, S, V), 16), dtype=torch.uint8, device="cuda")
    tt.tt_unmask_threshold(lg, mk, gamma, ids, com, conf, ns,
                           tt.TT_UNMASK_UPDATE_MASK if update else 0, ws)
    torch.cuda.synchronize()
    return (ids.cpu().numpy(), com.cpu().numpy(), conf.cpu().numpy(), ns.cpu().numpy(),
            mk.cpu().numpy())


def test_hand_sequence_by_gamma():
    c = G["sequence"]
    lg, mask = _rows(c["logits"]), np.array([c["mask"]], np.uint8)
    for gamma, want in c["by_gamma"]:
        ids, commit, conf, ns, _ = run_threshold(lg, mask, gamma)
        assert commit[0].tolist() == want, gamma
        assert ns.tolist() == [1] and ids[0].tolist() == [0] * 6


def test_hand_fallback_tie_and_empty_mask():
    c = G["fallback_tie"]
    _, commit, _, _, _ = run_threshold(_rows(c["logits"]), np.array([c["mask"]], np.uint8), c["gamma"])
    assert commit[0].tolist() == c["commit"]
    c = G["empty_mask"]
    _, commit, _, ns, _ = run_threshold(_rows(c["logits"]), np.array([c["mask"]], np.uint8), c["gamma"],
                                        nsteps=[c["nsteps_in"]])
    assert commit[0].tolist() == c["commit"] and ns.tolist() == [c["nsteps_out"]]


def test_hand_adaptive_loop_on_device():
    c = G["loop"]
    mask = np.ones((2, 4), np.uint8)
    ns = np.zeros(2, np.int32)
    steps = 0
    while mask.any() and steps < c["max_steps"]:
        lg = np.stack([_rows(seq) for seq in c["logits"][steps]]).reshape(8, 4)
        _, commit, _, ns, mask_after = run_threshold(lg, mask, c["gamma"], ns, update=True)
        assert commit.tolist() == c["commit"][steps]
        assert np.array_equal(mask_after, mask & (1 - commit))
        mask = mask_after
        steps += 1
    assert steps == c["steps"] and ns.tolist() == c["nsteps"]


@pytest.mark.parametrize("gamma", [0.8, 0.5, 0.95, 1.0])
@pytest.mark.parametrize("V", [4096, 131072])
def test_peaked_parity(V, gamma):
    B = 32 if V == 4096 else 8
    rng = np.random.Generator(np.random.PCG64(V + int(gamma * 100)))
    blk = workloads.make_peaked_block(rng, B, 16, V)
    lg = workloads.peaked_logits(rng, blk, 0)
    mask = (rng.random((B, 16)) < 0.8).astype(np.uint8)
    mask[0] = 0                                            # one sequence already resolved
    ids, commit, conf, ns, _ = run_threshold(lg, mask, gamma, nsteps=np.full(B, 2, np.int32))
    rids, rcommit, rconf, rns = oracle.unmask_threshold(lg, mask, gamma, np.full(B, 2, np.int32))
    assert np.array_equal(ids, rids)
    assert np.allclose(conf, rconf, rtol=1e-5, atol=1e-7)
    assert np.array_equal(ns, rns)
    assert_threshold_commit_ok(commit, rconf, mask, gamma)
    if gamma < 1.0:
        assert (commit == rcommit).mean() > 0.99


def test_adaptive_loop_parity():
    """The sampler loop with the mask kept on the device: every step's ids are
    exact, commits follow the rule (within the confidence band), and the step
    counts match the oracle run on the same trajectory."""
    B, S, V = 32, 16, 4096
    rng = np.random.Generator(np.random.PCG64(16))
    blk = workloads.make_peaked_block(rng, B, S, V)
    steps_lg = [workloads.peaked_logits(rng, blk, s) for s in range(6)]
    mask = np.ones((B, S), np.uint8)
    ns = np.zeros(B, np.int32)
    rns = np.zeros(B, np.int32)
    s = 0
    while mask.any() and s < 16:
        lg = steps_lg[s % len(steps_lg)]
        ids, commit, conf, ns, mask_after = run_threshold(lg, mask, 0.8, ns, update=True)
        rids, _, rconf, rns = oracle.unmask_threshold(lg, mask, 0.8, rns)
        assert np.array_equal(ids, rids), s
        assert_threshold_commit_ok(commit, rconf, mask, 0.8)
        assert np.array_equal(mask_after, mask & (1 - commit))
        assert np.array_equal(ns, rns)
        mask = mask_after
        s += 1
    assert not mask.any() and 2 <= s <= 8
