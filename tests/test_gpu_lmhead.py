"""GPU parity of tt_lmhead_unmask / tt_lmhead_unmask_threshold (LM head fused
with the confidence unmask) against the oracle's exact fp64 head + unmask.

Tolerance.  bf16 x bf16 products are exact in fp32; the GPU sums H of them in
fp32 (in its own order), so a logit carries an absolute error of roughly
sqrt(H) * 2^-24 * (partial-sum size), below 1e-4 for H <= 4096 and
|logits| <= 20, growing like sqrt(H) beyond.  The confidence 1/Z moves by at
most about twice the largest logit error, relatively.  Hence conf_tol(H) =
2.5e-4 * max(1, sqrt(H / 4096)), a relative bound: GPU confidences lie within
it of the oracle's, and commits may differ from the oracle's only among slots
whose oracle confidences lie within it (relative) of the deciding confidence
(the k-th largest, or gamma).  The GPU's id must attain the oracle's maximum
logit within LOGIT_TIE (a near-tie may go either way).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_commit_ok, assert_threshold_commit_ok, torch_mod

pytestmark = pytest.mark.gpu

LOGIT_TIE = 1e-3


def conf_tol(H):
    """Relative bound on the confidence error for hidden size H (see above)."""
    return 2.5e-4 * max(1.0, float(np.sqrt(H / 4096.0)))


class Run:
    def __init__(self, case):
        torch = torch_mod()
        self.torch = torch
        self.c = case
        dev = torch.device("cuda:0")
        bf = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)
        self.hidden = bf(case.hidden)
        self.weight = bf(case.weight)
        B, S = case.B, case.S
        self.ids = torch.empty((B, S), dtype=torch.int32, device=dev)
        self.commit = torch.empty((B, S), dtype=torch.uint8, device=dev)
        self.conf = torch.empty((B, S), dtype=torch.float32, device=dev)
        import two_tower_attention_amd as tt
        self.tt = tt
        n = tt.tt_lmhead_unmask_workspace_bytes(B, S, case.V, case.H)
        self.ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)

    def count(self, mask, k_commit=None, remaining=1, flags=0):
        torch = self.torch
        m = torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
        kc = None if k_commit is None else torch.from_numpy(np.asarray(k_commit, np.int32)).cuda()
        self.tt.tt_lmhead_unmask(self.hidden, self.weight, m, kc, remaining, self.ids, self.commit,
                                 self.conf, flags, self.ws)
        torch.cuda.synchronize()
        return self.ids.cpu().numpy(), self.commit.cpu().numpy(), self.conf.cpu().numpy(), m.cpu().numpy()

    def threshold(self, mask, gamma, nsteps=None, flags=0):
        torch = self.torch
        m = torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
        ns = None if nsteps is None else torch.from_numpy(np.asarray(nsteps, np.int32)).cuda()
        self.tt.tt_lmhead_unmask_threshold(self.hidden, self.weight, m, gamma, self.ids, self.commit,
                                           self.conf, ns, flags, self.ws)
        torch.cuda.synchronize()
        return (self.ids.cpu().numpy(), self.commit.cpu().numpy(), self.conf.cpu().numpy(),
                m.cpu().numpy(), None if ns is None else ns.cpu().numpy())


def check_rows(ids, conf, ref_ids, ref_conf, logits, what, H):
    """ids/conf of the GPU against the oracle's (rows flattened)."""
    ids, conf = ids.reshape(-1), conf.reshape(-1)
    ref_ids, ref_conf = ref_ids.reshape(-1), ref_conf.reshape(-1)
    for r in np.nonzero(ids != ref_ids)[0]:
        assert 0 <= ids[r] < logits.shape[1], (what, r, ids[r])
        assert logits[r, ids[r]] >= logits[r].max() - LOGIT_TIE, \
            (what, "row %d: id %d is not a near-maximum" % (r, ids[r]), logits[r, ids[r]], logits[r].max())
    np.testing.assert_allclose(conf, ref_conf, rtol=conf_tol(H), atol=0, err_msg=what)


CASES = [
    # name, B, S, H, V
    ("h32_one_stage", 2, 16, 32, 300),
    ("h64_two_stages", 1, 8, 64, 128),
    ("h96_three_stages", 3, 5, 96, 1000),
    ("ragged_vocab", 2, 16, 256, 2048 + 77),
    ("vocab_below_one_chunk", 2, 4, 64, 100),
    ("rows_over_one_tile", 20, 16, 128, 1024),  # 320 rows: two row tiles, the second ragged
    ("one_row", 1, 1, 128, 513),
    ("h512", 2, 16, 512, 4096),
    ("hidden_max", 1, 16, 65536, 512),           # 1024 stages per tile
    ("hidden_odd_stages", 2, 3, 4064, 700),      # 63.5 stages: a half last stage, padded to an even count
]


@pytest.mark.parametrize("name,B,S,H,V", CASES, ids=[c[0] for c in CASES])
def test_count_form_against_oracle(name, B, S, H, V):
    rng = np.random.Generator(np.random.PCG64(B * 1000 + S * 10 + H + V))
    case = workloads.make_lmhead_case(rng, B, S, H, V)
    mask = (rng.random((B, S)) < 0.75).astype(np.uint8)
    k = rng.integers(0, S + 1, size=B).astype(np.int32)
    run = Run(case)
    ids, commit, conf, _ = run.count(mask, k)
    ref_ids, ref_commit, ref_conf, logits = oracle.lmhead_unmask(case.hidden, case.weight, mask, k,
                                                                 with_logits=True)
    check_rows(ids, conf, ref_ids, ref_conf, logits, name, H)
    k_eff = np.minimum(k, mask.sum(axis=1))
    assert_commit_ok(commit, ref_commit, ref_conf, mask, k_eff, tie=conf_tol(H), rel=True)


def test_remaining_steps_and_mask_update():
    rng = np.random.Generator(np.random.PCG64(7))
    B, S, H, V = 4, 16, 128, 2000
    case = workloads.make_lmhead_case(rng, B, S, H, V)
    mask = np.ones((B, S), np.uint8)
    mask[1, :5] = 0
    run = Run(case)
    ids, commit, conf, mask_after = run.count(mask, None, 3, flags=1)
    ref_ids, ref_commit, ref_conf, logits = oracle.lmhead_unmask(case.hidden, case.weight, mask,
                                                                 None, 3, with_logits=True)
    check_rows(ids, conf, ref_ids, ref_conf, logits, "remaining", H)
    k_eff = -(-mask.sum(axis=1).astype(np.int64) // 3)
    assert_commit_ok(commit, ref_commit, ref_conf, mask, k_eff, tie=conf_tol(H), rel=True)
    assert np.array_equal(mask_after, mask * (1 - commit))


def test_threshold_form_and_nsteps():
    """Rows of mixed scale give confidences on both sides of gamma = 0.8."""
    rng = np.random.Generator(np.random.PCG64(8))
    B, S, H, V = 6, 16, 256, 3000
    scale = rng.choice([0.5, 1.0, 3.0, 6.0], size=B * S)
    case = workloads.make_lmhead_case(rng, B, S, H, V, row_scale=scale)
    mask = (rng.random((B, S)) < 0.8).astype(np.uint8)
    mask[2] = 0  # a sequence with nothing masked
    run = Run(case)
    ids, commit, conf, mask_after, ns = run.threshold(mask, 0.8, nsteps=np.zeros(B, np.int32), flags=1)
    logits = oracle.lmhead_logits(case.hidden, case.weight)
    ref_ids, _, ref_conf = oracle.unmask_f64(logits, mask, np.zeros(B, np.int32))
    check_rows(ids, conf, ref_ids, ref_conf, logits, "threshold", H)
    assert_threshold_commit_ok(commit, ref_conf, mask, 0.8, tie=conf_tol(H), rel=True)
    assert np.array_equal(mask_after, mask * (1 - commit))
    assert ns.tolist() == [int(mask[b].any()) for b in range(B)]
    assert (ref_conf[mask == 1] > 0.8).any() and (ref_conf[mask == 1] < 0.8).any()


def test_equal_weight_rows_take_the_lowest_id():
    """Duplicated head rows give exactly equal logits: the lowest id wins, also
    across 128-entry chunks and work-group tiles."""
    rng = np.random.Generator(np.random.PCG64(9))
    B, S, H, V = 2, 8, 64, 1200
    case = workloads.make_lmhead_case(rng, B, S, H, V)
    # make row 5 dominant for every hidden row by aligning it with the mean
    # direction, then copy it to ids 700 and 1100 (other chunks / tiles)
    hid = workloads.bits_to_f32(case.hidden)
    direction = np.sign(hid.sum(axis=0)).astype(np.float32)
    row = workloads.bf16_bits(direction * 0.5)
    case.weight[5] = row
    case.weight[700] = row
    case.weight[1100] = row
    case.hidden = workloads.bf16_bits(np.abs(hid) * direction)  # every row aligned with it
    run = Run(case)
    ids, _, conf, _ = run.count(np.ones((B, S), np.uint8), np.ones(B, np.int32))
    ref_ids, _, ref_conf, logits = oracle.lmhead_unmask(case.hidden, case.weight,
                                                        np.ones((B, S), np.uint8),
                                                        np.ones(B, np.int32), with_logits=True)
    assert np.all(ref_ids == 5)
    assert np.all(ids == 5)
    np.testing.assert_allclose(conf, ref_conf, rtol=conf_tol(H))


def test_full_size_sampled_sequences():
    """The unmask workload's shape with a 4096-wide head (B=32, S=16, H=4096,
    V=131072): every row on the GPU, eight whole sequences spread over the
    batch (so over both 256-row tiles) checked against the oracle (the commit
    ranks within a sequence)."""
    rng = np.random.Generator(np.random.PCG64(55))
    B, S, H, V = 32, 16, 4096, 131072
    case = workloads.make_lmhead_case(rng, B, S, H, V, seed=55)
    mask = (rng.random((B, S)) < 0.9).astype(np.uint8)
    run = Run(case)
    ids, commit, conf, _ = run.count(mask, None, 4)
    seqs = [0, 3, 9, 14, 17, 22, 27, 31]
    ref_ids, ref_commit, ref_conf, logits = oracle.lmhead_unmask(case.hidden, case.weight, mask,
                                                                 None, 4, seqs=seqs, with_logits=True)
    check_rows(ids[seqs], conf[seqs], ref_ids, ref_conf, logits, "full size", H)
    k_eff = -(-mask[seqs].sum(axis=1).astype(np.int64) // 4)
    assert_commit_ok(commit[seqs], ref_commit, ref_conf, mask[seqs], k_eff, tie=conf_tol(H),
                     rel=True)
    # every row produced a valid id and a probability
    assert ids.min() >= 0 and ids.max() < V
    assert np.all((conf > 0) & (conf <= 1))


def test_agrees_with_unfused_path():
    """Same inputs through torch's fp32 product and tt_unmask (logits in HBM)."""
    torch = torch_mod()
    rng = np.random.Generator(np.random.PCG64(10))
    B, S, H, V = 4, 16, 512, 8192
    case = workloads.make_lmhead_case(rng, B, S, H, V)
    run = Run(case)
    mask = np.ones((B, S), np.uint8)
    ids, commit, conf, _ = run.count(mask, np.full(B, 4, np.int32))
    logits = run.hidden.float() @ run.weight.float().t().contiguous()
    import two_tower_attention_amd as tt
    uws = torch.empty(max(tt.tt_unmask_workspace_bytes(B, S, V), 16), dtype=torch.uint8, device="cuda")
    ids2 = torch.empty_like(run.ids)
    com2 = torch.empty_like(run.commit)
    conf2 = torch.empty_like(run.conf)
    tt.tt_unmask(logits.contiguous(), torch.from_numpy(mask).cuda(),
                 torch.from_numpy(np.full(B, 4, np.int32)).cuda(), 1, ids2, com2, conf2, 0, uws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(conf, conf2.cpu().numpy(), rtol=2 * conf_tol(H))
    lg = logits.cpu().numpy().astype(np.float64)
    check_rows(ids, conf, ids2.cpu().numpy(), conf2.cpu().numpy(), lg, "unfused", H)
