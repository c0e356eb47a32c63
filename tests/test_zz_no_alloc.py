"""tt_unmask_noalloc, the unmask for callers that cannot allocate (its row
partials live in the library's static device array), against tt_unmask with
a caller workspace on the same inputs: two calls in a row, the second on a
smaller batch and vocabulary, so the second reads none of the first call's
partials.  Both run the same kernels, so every output is bit-identical."""
import numpy as np
import pytest

import workloads
from gpu_util import dev_tensor, torch_mod

pytestmark = pytest.mark.gpu


def _outputs(B, S, dev):
    torch = torch_mod()
    return (torch.full((B, S), -7, dtype=torch.int32, device=dev),
            torch.full((B, S), 0xAA, dtype=torch.uint8, device=dev),
            torch.full((B, S), float("nan"), dtype=torch.float32, device=dev))


def test_noalloc_matches_workspace_call_twice():
    import two_tower_attention_amd as tt
    torch = torch_mod()
    rng = np.random.Generator(np.random.PCG64(77))
    # (B, S, V, k_commit given?): the denoise-loop shape, then a smaller one
    # with an odd vocabulary and explicit per-sequence counts
    for B, S, V, with_k in ((32, 16, 131072, False), (3, 16, 5001, True)):
        logits = dev_tensor(workloads.make_logits(rng, B * S, V), "f32")
        mask_np = (rng.random((B, S)) < 0.8).astype(np.uint8)
        k_np = rng.integers(0, S + 2, size=B).astype(np.int32)
        k = dev_tensor(k_np, "i32") if with_k else None
        m_ws = dev_tensor(mask_np, "u8")
        m_na = dev_tensor(mask_np, "u8")
        nb = tt.tt_unmask_workspace_bytes(B, S, V)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda").fill_(0xFF)
        ids_a, com_a, conf_a = _outputs(B, S, "cuda")
        ids_b, com_b, conf_b = _outputs(B, S, "cuda")
        tt.tt_unmask(logits, m_ws, k, 3, ids_a, com_a, conf_a, tt.TT_UNMASK_UPDATE_MASK, ws)
        tt.tt_unmask_noalloc(logits, m_na, k, 3, ids_b, com_b, conf_b, tt.TT_UNMASK_UPDATE_MASK)
        torch.cuda.synchronize()
        print("tt_unmask_noalloc B=%d S=%d V=%d k_commit=%s" % (B, S, V, with_k), flush=True)
        assert torch.equal(ids_a, ids_b)
        assert torch.equal(com_a, com_b)
        assert torch.equal(conf_a.view(torch.int32), conf_b.view(torch.int32))
        assert torch.equal(m_ws, m_na)
        # and the results are the unmask's: ids in range, commits only on
        # masked slots, the committed count per sequence as the rule fixes
        ids, com = ids_b.cpu().numpy(), com_b.cpu().numpy().astype(bool)
        assert ids.min() >= 0 and ids.max() < V
        assert not np.any(com & (mask_np == 0))
        n = mask_np.sum(axis=1).astype(np.int64)
        want = np.clip(k_np, 0, n) if with_k else -(-n // 3)
        assert np.array_equal(com.sum(axis=1), want)
