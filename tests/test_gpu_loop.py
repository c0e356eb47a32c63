"""GPU parity of tt_kv_append (bit-exact) and of the denoise loop (attention per
layer and step, unmask with the mask updated on the device, then the block
commit) against the oracle loop."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (DevCase, assert_attn_close, assert_attn_units, assert_commit_ok, dev_tensor,
                      to_f64, torch_mod)

pytestmark = pytest.mark.gpu


def _bits(t, dtype):
    torch = torch_mod()
    if dtype == "bf16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("dtype,ps,lens", [("bf16", 256, [0, 250, 256, 1000, 17]),
                                           ("bf16", 16, [5, 16, 31]),
                                           ("f32", 32, [0, 40, 63])])
def test_kv_append_bit_exact(dtype, ps, lens):
    import two_tower_attention_amd as tt
    rng = np.random.Generator(np.random.PCG64(ps + len(lens)))
    c = workloads.make_attn_case(rng, B=len(lens), S=16, Hq=8, Hkv=2, D=64, ctx_lens=lens,
                                 page_size=ps, dtype=dtype, extra_tokens=16)
    dc = DevCase(c)
    tt.tt_kv_append(dc.desc, dc.k_blk, dc.v_blk, dc.k_pages, dc.v_pages, dc.page_table, dc.ctx_lens)
    kp, vp, nl = oracle.kv_append(c.k_pages, c.v_pages, c.page_table, c.ctx_lens, c.k_blk, c.v_blk)
    assert np.array_equal(dc.ctx_lens.cpu().numpy(), nl)
    assert np.array_equal(_bits(dc.k_pages, dtype).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(_bits(dc.v_pages, dtype).view(np.uint8), vp.view(np.uint8))


@pytest.mark.parametrize("dtype,S,Hkv,D,lens", [
    ("bf16", 64, 3, 128, [0, 200, 300]),   # one head is 16 KiB: passes of 2 heads, then 1
    ("bf16", 20, 2, 64, [0, 8, 13, 232]),  # runs of 8 tokens and a 4-token tail; one unaligned start
    ("f32", 23, 2, 64, [4, 12, 6]),        # runs of 4 tokens and a 3-token tail
    ("f32", 64, 3, 128, [64, 5, 511]),     # one head is 32 KiB: one head per pass
    ("bf16", 1, 5, 64, [0, 255, 256]),     # a one-token block, all 5 heads in one pass
])
def test_kv_append_head_passes(dtype, S, Hkv, D, lens):
    """Bit-exact append when the heads' values do not fit one LDS pass."""
    import two_tower_attention_amd as tt
    rng = np.random.Generator(np.random.PCG64(S * 100 + Hkv * 10 + D))
    c = workloads.make_attn_case(rng, B=len(lens), S=S, Hq=Hkv, Hkv=Hkv, D=D, ctx_lens=lens,
                                 page_size=256, dtype=dtype, extra_tokens=S)
    dc = DevCase(c)
    tt.tt_kv_append(dc.desc, dc.k_blk, dc.v_blk, dc.k_pages, dc.v_pages, dc.page_table, dc.ctx_lens)
    kp, vp, nl = oracle.kv_append(c.k_pages, c.v_pages, c.page_table, c.ctx_lens, c.k_blk, c.v_blk)
    assert np.array_equal(dc.ctx_lens.cpu().numpy(), nl)
    assert np.array_equal(_bits(dc.k_pages, dtype).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(_bits(dc.v_pages, dtype).view(np.uint8), vp.view(np.uint8))


@pytest.mark.parametrize("which", ["k", "v"])
def test_kv_append_unaligned_block(which):
    """Block keys or values that start off a 16-byte boundary take the element-wise path."""
    import two_tower_attention_amd as tt
    torch = torch_mod()
    rng = np.random.Generator(np.random.PCG64(21))
    c = workloads.make_attn_case(rng, B=2, S=16, Hq=4, Hkv=2, D=64, ctx_lens=[7, 300],
                                 page_size=256, extra_tokens=16)
    dc = DevCase(c)
    src = dc.k_blk if which == "k" else dc.v_blk
    buf = torch.empty(src.numel() + 1, dtype=src.dtype, device=src.device)
    off = buf[1:].view(src.shape)   # 2 bytes past a 16-byte boundary
    off.copy_(src)
    assert off.data_ptr() % 16 != 0
    k_arg, v_arg = (off, dc.v_blk) if which == "k" else (dc.k_blk, off)
    tt.tt_kv_append(dc.desc, k_arg, v_arg, dc.k_pages, dc.v_pages, dc.page_table, dc.ctx_lens)
    kp, vp, nl = oracle.kv_append(c.k_pages, c.v_pages, c.page_table, c.ctx_lens, c.k_blk, c.v_blk)
    assert np.array_equal(dc.ctx_lens.cpu().numpy(), nl)
    assert np.array_equal(_bits(dc.k_pages, "bf16").view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(_bits(dc.v_pages, "bf16").view(np.uint8), vp.view(np.uint8))


def test_kv_append_maximum_batch():
    """Bit-exact append for the largest batch the ABI accepts (2048 sequences,
    one work-group each), lengths 0..299 with 16-token pages."""
    import two_tower_attention_amd as tt
    rng = np.random.Generator(np.random.PCG64(2049))
    lens = [int(x) for x in rng.integers(0, 300, 2048)]
    c = workloads.make_attn_case(rng, B=2048, S=4, Hq=2, Hkv=2, D=64, ctx_lens=lens,
                                 page_size=16, extra_tokens=4)
    dc = DevCase(c)
    tt.tt_kv_append(dc.desc, dc.k_blk, dc.v_blk, dc.k_pages, dc.v_pages, dc.page_table, dc.ctx_lens)
    kp, vp, nl = oracle.kv_append(c.k_pages, c.v_pages, c.page_table, c.ctx_lens, c.k_blk, c.v_blk)
    assert np.array_equal(dc.ctx_lens.cpu().numpy(), nl)
    assert np.array_equal(_bits(dc.k_pages, "bf16").view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(_bits(dc.v_pages, "bf16").view(np.uint8), vp.view(np.uint8))


def test_kv_append_skips_sequence_without_pages():
    import two_tower_attention_amd as tt
    rng = np.random.Generator(np.random.PCG64(3))
    c = workloads.make_attn_case(rng, B=3, S=16, Hq=8, Hkv=2, D=64, ctx_lens=[10, 250, 20],
                                 page_size=256, extra_tokens=0)
    c.page_table[2, 0] = 10**6               # invalid page id for sequence 2
    dc = DevCase(c)
    before_k = _bits(dc.k_pages, "bf16").copy()
    tt.tt_kv_append(dc.desc, dc.k_blk, dc.v_blk, dc.k_pages, dc.v_pages, dc.page_table, dc.ctx_lens)
    lens = dc.ctx_lens.cpu().numpy()
    # 0 fits in its page; 1 would run past its only page (250+16 > 256); 2 has a bad page id
    assert lens.tolist() == [26, 250, 20]
    kp, _, _ = oracle.kv_append(c.k_pages, c.v_pages, c.page_table[:1], c.ctx_lens[:1],
                                c.k_blk[:1], c.v_blk[:1])
    assert np.array_equal(_bits(dc.k_pages, "bf16").view(np.uint8), kp.view(np.uint8))
    assert not np.array_equal(before_k.view(np.uint8), kp.view(np.uint8))


def run_loop_gpu(lp):
    """The denoise loop driven through the C ABI with device-side mask state."""
    import two_tower_attention_amd as tt
    torch = torch_mod()
    B, S, T = lp.B, lp.S, lp.steps
    devs = [DevCase(p) for p in lp.pools]
    # all layers share one ctx_lens vector (one per layer here, kept in sync)
    q = [[dev_tensor(lp.q[s][i], "bf16") for i in range(lp.layers)] for s in range(T)]
    kb = [[dev_tensor(lp.k_blk[s][i], "bf16") for i in range(lp.layers)] for s in range(T)]
    vb = [[dev_tensor(lp.v_blk[s][i], "bf16") for i in range(lp.layers)] for s in range(T)]
    logits = [dev_tensor(l, "f32") for l in lp.logits]
    mask = torch.ones((B, S), dtype=torch.uint8, device="cuda")
    nb = tt.tt_unmask_workspace_bytes(B, S, lp.vocab)
    uws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    res = {"attn": [], "ids": [], "commit": [], "mask": []}
    for s in range(T):
        outs = []
        for i, d in enumerate(devs):
            outs.append(d.attn(q=q[s][i], k_blk=kb[s][i], v_blk=vb[s][i]))
        ids = torch.empty((B, S), dtype=torch.int32, device="cuda")
        com = torch.empty((B, S), dtype=torch.uint8, device="cuda")
        tt.tt_unmask(logits[s], mask, None, T - s, ids, com, None, tt.TT_UNMASK_UPDATE_MASK, uws)
        res["attn"].append([to_f64(o, "bf16") for o in outs])
        res["ids"].append(ids.cpu().numpy())
        res["commit"].append(com.cpu().numpy())
        res["mask"].append(mask.cpu().numpy())
    for i, d in enumerate(devs):
        tt.tt_kv_append(d.desc, kb[T - 1][i], vb[T - 1][i], d.k_pages, d.v_pages, d.page_table,
                        d.ctx_lens)
    torch.cuda.synchronize()
    res["pools"] = [(_bits(d.k_pages, "bf16"), _bits(d.v_pages, "bf16"),
                     d.ctx_lens.cpu().numpy()) for d in devs]
    return res


def test_reduced_denoise_loop():
    lp = workloads.config5(seed=5, B=4, layers=2, vocab=4096, lo=256, hi=1024)
    got = run_loop_gpu(lp)
    ref = oracle.denoise_loop(lp)
    mask = np.ones((lp.B, lp.S), np.uint8)
    for s in range(lp.steps):
        for i in range(lp.layers):
            assert_attn_close(got["attn"][s][i], ref["attn"][s][i], "bf16", "step %d layer %d" % (s, i))
        assert np.array_equal(got["ids"][s], ref["ids"][s])
        n = mask.sum(axis=1).astype(np.int64)
        k_eff = -(-n // (lp.steps - s))
        assert_commit_ok(got["commit"][s], ref["commit"][s], ref["conf"][s], mask, k_eff)
        mask = mask & (1 - got["commit"][s])
        assert np.array_equal(got["mask"][s], mask)
    assert not mask.any()
    for (gk, gv, gl), (rk, rv, rl) in zip(got["pools"], ref["pools"]):
        assert np.array_equal(gl, rl)
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


@pytest.mark.timeout(900)
def test_full_size_denoise_loop():
    """config5 at full size: B=32, 6 layers, T=4, V=131072.  Unmask ids exact
    every step; every layer's attention at every step compared element by
    element with the oracle, and per (b, h_kv) unit; appended slots
    bit-exact."""
    lp = workloads.config5()
    got = run_loop_gpu_full(lp)
    assert got is None


def run_loop_gpu_full(lp):
    import two_tower_attention_amd as tt
    torch = torch_mod()
    B, S, T = lp.B, lp.S, lp.steps
    devs = [DevCase(p) for p in lp.pools]
    mask_h = np.ones((B, S), np.uint8)
    mask = torch.ones((B, S), dtype=torch.uint8, device="cuda")
    nb = tt.tt_unmask_workspace_bytes(B, S, lp.vocab)
    uws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    for s in range(T):
        for i, d in enumerate(devs):
            q = dev_tensor(lp.q[s][i], "bf16")
            kb = dev_tensor(lp.k_blk[s][i], "bf16")
            vb = dev_tensor(lp.v_blk[s][i], "bf16")
            out = to_f64(d.attn(q=q, k_blk=kb, v_blk=vb), "bf16")
            ref = oracle.block_attn(lp.pools[i], q=lp.q[s][i], k_blk=lp.k_blk[s][i],
                                    v_blk=lp.v_blk[s][i])
            assert_attn_units(out, ref, lp.pools[i].Hkv, "bf16",
                              "full loop step %d layer %d" % (s, i))
        lg = dev_tensor(lp.logits[s], "f32")
        ids = torch.empty((B, S), dtype=torch.int32, device="cuda")
        com = torch.empty((B, S), dtype=torch.uint8, device="cuda")
        tt.tt_unmask(lg, mask, None, T - s, ids, com, None, tt.TT_UNMASK_UPDATE_MASK, uws)
        rids, rcom, rconf = oracle.unmask(lp.logits[s], mask_h, None, T - s)
        assert np.array_equal(ids.cpu().numpy(), rids)
        n = mask_h.sum(axis=1).astype(np.int64)
        assert_commit_ok(com.cpu().numpy(), rcom, rconf, mask_h, -(-n // (T - s)))
        mask_h = mask_h & (1 - com.cpu().numpy())
        assert np.array_equal(mask.cpu().numpy(), mask_h)
        del lg
    assert not mask_h.any()
    for i, d in enumerate(devs):
        kb = dev_tensor(lp.k_blk[T - 1][i], "bf16")
        vb = dev_tensor(lp.v_blk[T - 1][i], "bf16")
        tt.tt_kv_append(d.desc, kb, vb, d.k_pages, d.v_pages, d.page_table, d.ctx_lens)
        p = lp.pools[i]
        lens = d.ctx_lens.cpu().numpy()
        assert np.array_equal(lens, p.ctx_lens + S)
        gk, gv = _bits(d.k_pages, "bf16"), _bits(d.v_pages, "bf16")
        for b in range(B):
            L = int(p.ctx_lens[b])
            for t in range(S):
                pg, o = p.page_table[b, (L + t) // p.page_size], (L + t) % p.page_size
                assert np.array_equal(gk[pg, :, o, :], lp.k_blk[T - 1][i][b, t])
                assert np.array_equal(gv[pg, :, :, o], lp.v_blk[T - 1][i][b, t])
    return None
