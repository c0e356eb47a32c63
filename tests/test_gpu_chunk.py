"""GPU parity of tt_chunk_attn (the context tower's causal chunk ingest)
against the oracle, on the bf16 MFMA path and the fp32 path."""
import numpy as np
import pytest

import oracle
import workloads
from golden_util import attn_case, expected, load
from gpu_util import DevCase, assert_attn_close, assert_attn_units, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", load("chunk_hand_cases.json")["cases"], ids=lambda c: c["name"])
def test_hand_cases(case, dtype):
    c = attn_case(case, dtype)
    got = to_f64(DevCase(c).attn(causal=True), dtype)
    exp = expected(case)
    fixed = ~np.isnan(exp)
    tol = 1e-2 if dtype == "bf16" else 1e-6
    np.testing.assert_allclose(got[fixed], exp[fixed], rtol=tol, atol=tol)


CASES = [
    # name, B, S, Hq, Hkv, D, lens, page_size, dtype
    ("ragged_256", 3, 16, 32, 2, 128, [0, 700, 64], 256, "bf16"),
    ("small_pages", 3, 16, 32, 2, 128, [5, 200, 64], 16, "bf16"),
    ("d64", 2, 16, 16, 2, 64, [130, 1], 256, "bf16"),
    ("s32_two_query_chunks", 2, 32, 32, 2, 128, [90, 1000], 256, "bf16"),
    ("s64_four_query_chunks", 1, 64, 32, 2, 128, [333], 256, "bf16"),
    ("mha_s8", 2, 8, 4, 4, 128, [64, 0], 256, "bf16"),
    ("fp32", 2, 16, 4, 1, 64, [48, 3], 16, "f32"),
]


@pytest.mark.parametrize("name,B,S,Hq,Hkv,D,lens,ps,dtype", CASES, ids=[c[0] for c in CASES])
def test_against_oracle(name, B, S, Hq, Hkv, D, lens, ps, dtype):
    rng = np.random.Generator(np.random.PCG64(sum(lens) + S))
    c = workloads.make_attn_case(rng, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=lens, page_size=ps,
                                 dtype=dtype)
    got = to_f64(DevCase(c).attn(causal=True), dtype)
    assert_attn_close(got, oracle.block_attn(c, causal=True), dtype, name)


def test_last_position_equals_block_attention_and_future_keys_ignored():
    """On the GPU too: the last chunk position sees the whole chunk, so it is
    bit-identical to tt_block_attn there; changing chunk keys/values past a
    position leaves that position's output bit-identical."""
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(21))
    c = workloads.make_attn_case(rng, B=2, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[300, 70],
                                 page_size=256)
    dc = DevCase(c)
    causal = dc.attn(causal=True).clone()
    full = dc.attn()
    assert torch.equal(causal[:, -1], full[:, -1])
    t = 5
    kb, vb = dc.k_blk.clone(), dc.v_blk.clone()
    kb[:, t + 1:] = kb[:, t + 1:].flip(1)
    vb[:, t + 1:] = -vb[:, t + 1:]
    again = dc.attn(k_blk=kb, v_blk=vb, causal=True)
    assert torch.equal(again[:, :t + 1], causal[:, :t + 1])


@pytest.mark.timeout(300)
def test_config5_layer_whole_tensor():
    """One layer of the denoise-loop workload (B=32, ragged 2K-8K contexts)
    ingested causally: every element, and every (b, h_kv) unit on its own."""
    lp_rng = np.random.Generator(np.random.PCG64(55))
    lens = (16 * lp_rng.integers(128, 513, size=32)).astype(np.int32)
    c = workloads.make_attn_case(lp_rng, B=32, S=16, Hq=32, Hkv=2, D=128, ctx_lens=lens,
                                 page_size=256, seed=55)
    got = to_f64(DevCase(c).attn(causal=True), "bf16")
    ref = oracle.block_attn(c, causal=True)
    assert_attn_units(got, ref, c.Hkv, "bf16", "config5 layer causal")
