"""GPU parity of tt_unmask against the oracle: argmax ids bit-exact, confidence
within fp32 rounding, commit sets exact up to near-ties of the k-th confidence."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_commit_ok, dev_tensor, torch_mod

pytestmark = pytest.mark.gpu


def run_unmask(logits, mask, k=None, remaining=1, flags=0, misalign=False):
    import two_tower_attention_amd as tt
    torch = torch_mod()
    B, S = mask.shape
    V = logits.shape[-1]
    if misalign:   # rows start off a 16-byte boundary -> scalar path
        buf = torch.empty(B * S * V + 1, dtype=torch.float32, device="cuda")
        lg = buf[1:].view(B * S, V)
        lg.copy_(torch.from_numpy(logits.reshape(B * S, V)))
    else:
        lg = dev_tensor(logits.reshape(B * S, V), "f32")
    m = dev_tensor(mask.astype(np.uint8), "u8")
    kk = None if k is None else dev_tensor(np.asarray(k, np.int32), "i32")
    ids = torch.full((B, S), -7, dtype=torch.int32, device="cuda")
    com = torch.full((B, S), 9, dtype=torch.uint8, device="cuda")
    conf = torch.full((B, S), float("nan"), dtype=torch.float32, device="cuda")
    nb = tt.tt_unmask_workspace_bytes(B, S, V)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    tt.tt_unmask(lg, m, kk, remaining, ids, com, conf, flags, ws)
    return ids.cpu().numpy(), com.cpu().numpy(), conf.cpu().numpy(), m.cpu().numpy()


def check(logits, mask, k=None, remaining=1, **kw):
    ids, com, conf, _ = run_unmask(logits, mask, k, remaining, **kw)
    rids, rcom, rconf = oracle.unmask(logits, mask, k, remaining)
    assert np.array_equal(ids, rids), np.argwhere(ids != rids)[:5]
    np.testing.assert_allclose(conf, rconf, rtol=1e-5, atol=1e-7)
    n = mask.astype(bool).sum(axis=1)
    kb = np.asarray(k) if k is not None else -(-n // remaining)
    k_eff = np.clip(kb, 0, n)
    assert_commit_ok(com, rcom, rconf, mask, k_eff)
    return ids, com, conf


def test_config1_unmask():
    _, logits, mask, k = workloads.config1()
    check(logits, mask, k)


def test_config5_unmask_full_size():
    rng = np.random.Generator(np.random.PCG64(5))
    B, S, V = 32, 16, 131072
    logits = workloads.make_logits(rng, B * S, V)
    mask = (rng.random((B, S)) < 0.75).astype(np.uint8)
    for rem in (4, 3, 1):
        check(logits, mask, None, rem)


@pytest.mark.parametrize("B,S", [(4095, 16), (65535, 1)])
def test_maximum_rows(B, S):
    """The most rows the ABI accepts (batch * block <= 65535; one row per
    work-group column), an odd vocabulary, a random mask and k from
    remaining_steps."""
    rng = np.random.Generator(np.random.PCG64(B + S))
    V = 257
    logits = workloads.make_logits(rng, B * S, V)
    mask = (rng.random((B, S)) < 0.6).astype(np.uint8)
    check(logits, mask, None, 2)


@pytest.mark.parametrize("V", [1, 3, 1000, 1023, 4097, 40000])
def test_odd_vocab_sizes(V):
    rng = np.random.Generator(np.random.PCG64(V))
    B, S = 3, 16
    logits = (3 * rng.standard_normal((B * S, V))).astype(np.float32)
    mask = (rng.random((B, S)) < 0.6).astype(np.uint8)
    check(logits, mask, np.array([0, 3, 20], np.int32))


def test_scalar_path_misaligned_rows():
    rng = np.random.Generator(np.random.PCG64(3))
    logits = (3 * rng.standard_normal((2 * 16, 4096))).astype(np.float32)
    mask = np.ones((2, 16), np.uint8)
    check(logits, mask, np.array([4, 16], np.int32), misalign=True)


def test_ties_across_chunks_and_neg_inf():
    B, S, V = 2, 16, 131072
    rng = np.random.Generator(np.random.PCG64(11))
    logits = (3 * rng.standard_normal((B * S, V))).astype(np.float32)
    top = np.float32(40.0)
    logits[0, [70000, 5, 131071]] = top          # tie across chunks -> 5
    logits[1, [131071, 100000]] = top             # -> 100000
    logits[2, :] = -np.inf
    logits[2, 12345] = 0.0                        # single finite entry -> conf 1
    logits[3, :V // 2] = -np.inf
    logits[4, 0] = top
    logits[4, 1] = np.float32(-0.0) + top         # equal -> 0
    logits[5, 7] = np.float32(0.0)
    logits[5] = np.where(np.arange(V) == 7, np.float32(0.0), np.float32(-0.0))  # all zero: id 0
    logits[16:] = logits[:16]                     # duplicate rows -> equal confidences
    mask = np.ones((B, S), np.uint8)
    ids, _, conf = check(logits, mask, np.array([5, 7], np.int32))
    assert ids[0, 0] == 5 and ids[0, 1] == 100000 and ids[0, 2] == 12345 and ids[0, 5] == 0
    assert conf[0, 2] == 1.0


def test_commit_edge_counts():
    rng = np.random.Generator(np.random.PCG64(8))
    B, S, V = 6, 16, 512
    logits = (2 * rng.standard_normal((B * S, V))).astype(np.float32)
    mask = np.ones((B, S), np.uint8)
    mask[1] = 0                  # nothing masked
    mask[2, ::2] = 0
    mask[3, :15] = 0             # one masked
    check(logits, mask, np.array([0, 4, 100, 1, -5, 16], np.int32))
    for rem in (1, 2, 5, 16, 1000):
        check(logits, mask, None, rem)
    # ceil(#masked / remaining_steps) must not overflow near INT_MAX: one slot each
    ids, com, _ = check(logits, mask, None, 2**31 - 1)
    assert com.sum(axis=1).tolist() == [1, 0, 1, 1, 1, 1]


def test_small_blocks():
    rng = np.random.Generator(np.random.PCG64(4))
    for S in (1, 2, 7, 64):
        B, V = 3, 300
        logits = rng.standard_normal((B * S, V)).astype(np.float32)
        mask = (rng.random((B, S)) < 0.7).astype(np.uint8)
        check(logits, mask, None, 2)


def test_update_mask_flag():
    import two_tower_attention_amd as tt
    rng = np.random.Generator(np.random.PCG64(12))
    B, S, V = 4, 16, 2048
    logits = (3 * rng.standard_normal((B * S, V))).astype(np.float32)
    mask = (rng.random((B, S)) < 0.8).astype(np.uint8)
    ids, com, conf, new_mask = run_unmask(logits, mask, None, 2, flags=tt.TT_UNMASK_UPDATE_MASK)
    assert np.array_equal(new_mask, mask & (1 - com))
    _, _, _, same = run_unmask(logits, mask, None, 2, flags=0)
    assert np.array_equal(same, mask)
