"""Pins for the oracle's causal chunk ingest (CPU only): hand-worked closed
forms, torch float64 scaled_dot_product_attention with an explicit mask the
test builds over a concatenation it gathers itself, and the invariants that
causality implies."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from golden_util import attn_case, expected, load
from test_oracle_attn import _f64, logical_kv

G = load("chunk_hand_cases.json")


@pytest.mark.parametrize("case", G["cases"], ids=[c["name"] for c in G["cases"]])
def test_hand_cases(case):
    c = attn_case(case, "f32")
    exp = expected(case)
    out = oracle.block_attn(c, causal=True)
    fixed = ~np.isnan(exp)
    assert np.allclose(out[fixed], exp[fixed], rtol=1e-12, atol=1e-12)


def causal_sdpa_reference(c):
    """torch float64 SDPA over [context ; chunk] with a boolean mask: chunk
    position t sees the whole context and chunk tokens 0..t."""
    ks, vs = logical_kv(c)
    q = _f64(c.q, c.dtype)
    kb, vb = _f64(c.k_blk, c.dtype), _f64(c.v_blk, c.dtype)
    g = c.Hq // c.Hkv
    out = np.zeros((c.B, c.S, c.Hq, c.D))
    for b in range(c.B):
        L = ks[b].shape[0]
        K = np.concatenate([ks[b], kb[b]], axis=0)
        V = np.concatenate([vs[b], vb[b]], axis=0)
        allowed = np.zeros((c.S, L + c.S), dtype=bool)
        for t in range(c.S):
            allowed[t, :L + t + 1] = True
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0)
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0)
        Qt = torch.from_numpy(q[b]).permute(1, 0, 2)
        o = torch.nn.functional.scaled_dot_product_attention(
            Qt.unsqueeze(0), Kt.contiguous().unsqueeze(0), Vt.contiguous().unsqueeze(0),
            attn_mask=torch.from_numpy(allowed), scale=c.scale)
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("lens,S,Hq,Hkv,ps", [([21, 0, 40], 4, 8, 2, 16), ([0], 16, 4, 1, 16),
                                             ([300, 17], 16, 32, 2, 256), ([5], 1, 4, 4, 16)])
def test_against_masked_sdpa(lens, S, Hq, Hkv, ps):
    rng = np.random.Generator(np.random.PCG64(len(lens) * 100 + S))
    c = workloads.make_attn_case(rng, B=len(lens), S=S, Hq=Hq, Hkv=Hkv, D=32, ctx_lens=lens,
                                 page_size=ps, dtype="f32")
    assert np.allclose(oracle.block_attn(c, causal=True), causal_sdpa_reference(c),
                       rtol=1e-10, atol=1e-12)


def test_empty_context_is_torch_causal():
    rng = np.random.Generator(np.random.PCG64(9))
    c = workloads.make_attn_case(rng, B=2, S=16, Hq=4, Hkv=2, D=16, ctx_lens=[0, 0],
                                 page_size=16, dtype="f32")
    q = torch.from_numpy(_f64(c.q, "f32")).permute(0, 2, 1, 3)
    k = torch.from_numpy(_f64(c.k_blk, "f32")).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    v = torch.from_numpy(_f64(c.v_blk, "f32")).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k.contiguous(), v.contiguous(),
                                                           is_causal=True, scale=c.scale)
    assert np.allclose(oracle.block_attn(c, causal=True), ref.permute(0, 2, 1, 3).numpy(),
                       rtol=1e-10, atol=1e-12)


def test_future_chunk_tokens_do_not_matter():
    """Output at chunk position t is unchanged, bit for bit, when the keys and
    values of later chunk tokens change; the last position equals the
    bidirectional block attention."""
    rng = np.random.Generator(np.random.PCG64(11))
    c = workloads.make_attn_case(rng, B=2, S=8, Hq=4, Hkv=2, D=16, ctx_lens=[13, 30],
                                 page_size=16, dtype="f32")
    base = oracle.block_attn(c, causal=True)
    for t in range(c.S - 1):
        kb, vb = c.k_blk.copy(), c.v_blk.copy()
        kb[:, t + 1:] = rng.standard_normal(kb[:, t + 1:].shape).astype(np.float32)
        vb[:, t + 1:] = rng.standard_normal(vb[:, t + 1:].shape).astype(np.float32)
        out = oracle.block_attn(c, causal=True, k_blk=kb, v_blk=vb)
        assert np.array_equal(out[:, :t + 1], base[:, :t + 1])
        assert not np.allclose(out[:, t + 1:], base[:, t + 1:])
    assert np.array_equal(base[:, -1], oracle.block_attn(c)[:, -1])
