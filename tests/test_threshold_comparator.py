"""The GPU tests' threshold-commit comparator accepts the oracle's own commit
sets and rejects plausible wrong ones (CPU only)."""
import numpy as np
import pytest

import oracle
from gpu_util import COMMIT_TIE, assert_threshold_commit_ok


def _case(seed, gamma):
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = (rng.standard_normal((5, 8)) * rng.uniform(0.5, 5.0, size=(5, 1))).astype(np.float32)
    lg = pool[rng.integers(0, 5, size=4 * 8)]
    mask = (rng.random((4, 8)) < 0.7).astype(np.uint8)
    _, commit, conf, _ = oracle.unmask_threshold(lg, mask, gamma)
    return commit, conf, mask


@pytest.mark.parametrize("seed", range(8))
def test_accepts_oracle_and_rejects_mistakes(seed):
    gamma = 0.3 + 0.08 * seed
    commit, conf, mask = _case(seed, gamma)
    assert_threshold_commit_ok(commit, conf, mask, gamma)
    for b in range(4):
        if not mask[b].any():
            continue
        wrong = [commit.copy() for _ in range(3)]
        unmasked = np.nonzero(mask[b] == 0)[0]
        if unmasked.size:
            wrong[0][b, unmasked[0]] = 1                      # commits an unmasked slot
        else:
            wrong[0][b] = 0                                   # no progress
        off = np.nonzero((mask[b] == 1) & (commit[b] == 0))[0]
        if off.size:
            wrong[1][b, off[0]] = 1                           # extra slot below gamma / second fallback
        else:
            wrong[1][b] = 0
        on = np.nonzero(commit[b] == 1)[0]
        wrong[2][b, on[0]] = 0                                # drops a committed slot
        for w in wrong:
            if np.array_equal(w, commit):
                continue
            near = np.abs(conf[b] - gamma) <= COMMIT_TIE
            if near.any():
                continue
            with pytest.raises(AssertionError):
                assert_threshold_commit_ok(w, conf, mask, gamma)
