"""Pins for the oracle's block attention (CPU only).

The oracle is checked against things other than itself: hand-worked closed
forms (tests/golden/attn_hand_cases.json), torch's scaled_dot_product_attention
in float64 on a concatenation the test gathers with its own code, and
invariants that the definition implies (weights sum to one, equivariance under
block permutation, invariance under physical page order and page size).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from golden_util import attn_case, expected, load


def _f64(a, dtype):
    if dtype == "bf16":
        return workloads.bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def logical_kv(c):
    """Test-side gather of the committed context, per the documented layouts:
    k_pages [P,Hkv,page,D] token-major, v_pages [P,Hkv,D,page] feature-major."""
    ks, vs = [], []
    kp, vp = _f64(c.k_pages, c.dtype), _f64(c.v_pages, c.dtype)
    for b in range(c.B):
        L = int(c.ctx_lens[b])
        pos = np.arange(L)
        pages = c.page_table[b, pos // c.page_size]
        off = pos % c.page_size
        ks.append(kp[pages, :, off, :])                       # [L, Hkv, D]
        vs.append(vp[pages, :, :, off])                      # [L, Hkv, D]
    return ks, vs


def sdpa_reference(c):
    """torch float64 SDPA over [context ; block] with GQA by repeat_interleave."""
    ks, vs = logical_kv(c)
    q = _f64(c.q, c.dtype)
    kb, vb = _f64(c.k_blk, c.dtype), _f64(c.v_blk, c.dtype)
    g = c.Hq // c.Hkv
    out = np.zeros((c.B, c.S, c.Hq, c.D))
    for b in range(c.B):
        K = np.concatenate([ks[b], kb[b]], axis=0)             # [N, Hkv, D]
        V = np.concatenate([vs[b], vb[b]], axis=0)
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0)
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0)
        Qt = torch.from_numpy(q[b]).permute(1, 0, 2)            # [Hq, S, D]
        o = torch.nn.functional.scaled_dot_product_attention(
            Qt.unsqueeze(0), Kt.contiguous().unsqueeze(0), Vt.contiguous().unsqueeze(0),
            scale=c.scale)
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


# ----------------------------------------------------------------- goldens

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", load("attn_hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_cases(case, dtype):
    c = attn_case(case, dtype)
    out = oracle.block_attn(c)
    exp = expected(case)
    fixed = ~np.isnan(exp)
    assert fixed.any()
    np.testing.assert_allclose(out[fixed], exp[fixed], rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------- library reductions

SHAPES = [
    # B, S, Hq, Hkv, D, lens, page_size
    (1, 16, 4, 1, 64, [48], 16),
    (2, 1, 8, 2, 64, [0, 300], 32),        # S=1: decode attention over L+1 keys
    (3, 2, 16, 1, 32, [1, 17, 48], 16),
    (2, 16, 16, 1, 128, [0, 0], 16),        # L=0: plain bidirectional attention
    (2, 16, 32, 2, 128, [300, 65], 256),    # g=16, ragged, partial last page
    (1, 5, 3, 3, 16, [33], 16),             # MHA, odd sizes
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_against_torch_sdpa(shape, dtype):
    B, S, Hq, Hkv, D, lens, ps = shape
    rng = np.random.Generator(np.random.PCG64(hash((shape[0], S, Hq, D, ps)) % 2**32))
    c = workloads.make_attn_case(rng, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=lens,
                                 page_size=ps, dtype=dtype)
    out, ws = oracle.block_attn(c, with_wsum=True)
    ref = sdpa_reference(c)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ws, 1.0, rtol=0, atol=1e-12)
    assert np.isfinite(out).all()          # the NaN poison past each length is never read


def test_rows_subset_matches_full():
    rng = np.random.Generator(np.random.PCG64(7))
    c = workloads.make_attn_case(rng, B=3, S=4, Hq=8, Hkv=2, D=32, ctx_lens=[5, 0, 70],
                                 page_size=16, dtype="bf16")
    full = oracle.block_attn(c)
    rows = [(2, 3, 7), (0, 0, 0), (1, 2, 5), (2, 0, 1)]
    sub = oracle.block_attn(c, rows=rows)
    for i, (b, t, h) in enumerate(rows):
        assert np.array_equal(sub[i], full[b, t, h])


# ----------------------------------------------------------------- invariants

def _case(seed=11, dtype="bf16", lens=(37, 100), ps=16, S=8, Hq=8, Hkv=2, D=32):
    rng = np.random.Generator(np.random.PCG64(seed))
    return workloads.make_attn_case(rng, B=len(lens), S=S, Hq=Hq, Hkv=Hkv, D=D,
                                    ctx_lens=list(lens), page_size=ps, dtype=dtype)


def test_block_permutation_equivariance():
    c = _case()
    out = oracle.block_attn(c)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(c.S)
    c.q, c.k_blk, c.v_blk = c.q[:, perm], c.k_blk[:, perm], c.v_blk[:, perm]
    out2 = oracle.block_attn(c)
    np.testing.assert_allclose(out2, out[:, perm], rtol=1e-12, atol=1e-14)


def test_physical_page_order_invariance():
    c = _case()
    out = oracle.block_attn(c)
    P = c.k_pages.shape[0]
    new_of_old = np.random.Generator(np.random.PCG64(5)).permutation(P)
    kp = np.empty_like(c.k_pages); vp = np.empty_like(c.v_pages)
    kp[new_of_old] = c.k_pages
    vp[new_of_old] = c.v_pages
    pt = np.where(c.page_table >= 0, new_of_old[np.maximum(c.page_table, 0)], -1).astype(np.int32)
    out2 = oracle.block_attn(c, k_pages=kp, v_pages=vp, page_table=pt)
    assert np.array_equal(out, out2)


def test_page_size_invariance():
    c = _case(ps=16)
    out = oracle.block_attn(c)
    ks, vs = logical_kv(c)
    # repack the same logical context into pages of 48 tokens, identity order
    ps2 = 48
    caps = [max(1, math.ceil(int(L) / ps2)) for L in c.ctx_lens]
    P2 = sum(caps)
    el = c.k_pages.dtype
    kp = np.zeros((P2, c.Hkv, ps2, c.D), dtype=el)
    vp = np.zeros((P2, c.Hkv, c.D, ps2), dtype=el)
    pt = np.full((c.B, max(caps)), -1, dtype=np.int32)
    base = 0
    for b in range(c.B):
        L = int(c.ctx_lens[b])
        for j in range(caps[b]):
            pt[b, j] = base + j
        for pos in range(L):
            src_page = c.page_table[b, pos // c.page_size]
            kp[base + pos // ps2, :, pos % ps2, :] = c.k_pages[src_page, :, pos % c.page_size, :]
            vp[base + pos // ps2, :, :, pos % ps2] = c.v_pages[src_page, :, :, pos % c.page_size]
        base += caps[b]
    c.page_size = ps2
    out2 = oracle.block_attn(c, k_pages=kp, v_pages=vp, page_table=pt)
    assert np.array_equal(out, out2)


def test_constant_values_closed_form():
    c = _case(dtype="f32")
    c.v_blk[...] = 0.75
    c.v_pages[...] = 0.75
    out = oracle.block_attn(c)
    np.testing.assert_allclose(out, 0.75, rtol=0, atol=1e-12)


def test_zero_queries_give_value_mean():
    c = _case(dtype="f32")
    c.q[...] = 0.0
    out = oracle.block_attn(c)
    ks, vs = logical_kv(c)
    g = c.Hq // c.Hkv
    for b in range(c.B):
        allv = np.concatenate([vs[b], c.v_blk[b].astype(np.float64)], axis=0)   # [N, Hkv, D]
        mean = allv.mean(axis=0)
        for h in range(c.Hq):
            np.testing.assert_allclose(out[b, :, h, :], np.broadcast_to(mean[h // g], (c.S, c.D)),
                                       rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value():
    # L=0, S=1: the only key gets weight one
    c = _case(dtype="f32", lens=(0, 0), S=1)
    out = oracle.block_attn(c)
    g = c.Hq // c.Hkv
    for h in range(c.Hq):
        np.testing.assert_array_equal(out[:, 0, h, :], c.v_blk[:, 0, h // g, :].astype(np.float64))
