"""GPU parity of tt_block_attn against the fp64 oracle (through the C ABI).

Every case compares every output element; the full-size workloads also hold
each (b, h_kv) unit to the rel-L2 bound on its own.  Outputs are pre-filled with
NaN and the workspace with NaN bit patterns, so an element the kernels never
write, or a partial read before it is written, fails.
"""
import numpy as np
import pytest

import oracle
import workloads
from golden_util import attn_case, expected, load
from gpu_util import DevCase, assert_attn_close, assert_attn_units, to_f64

pytestmark = pytest.mark.gpu


def _run_full(c, what=""):
    dc = DevCase(c)
    got = to_f64(dc.attn(), c.dtype)
    ref = oracle.block_attn(c)
    return assert_attn_units(got, ref, c.Hkv, c.dtype, what)


def _case(seed, B, S, Hq, Hkv, D, lens, ps, dtype="bf16", **kw):
    rng = np.random.Generator(np.random.PCG64(seed))
    return workloads.make_attn_case(rng, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=lens,
                                    page_size=ps, dtype=dtype, **kw)


# ------------------------------------------------------------ hand cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [c for c in load("attn_hand_cases.json")["cases"]
                                  if c["page_size"] >= 16], ids=lambda c: c["name"])
def test_hand_cases(case, dtype):
    c = attn_case(case, dtype)
    dc = DevCase(c)
    got = to_f64(dc.attn(), dtype)
    exp = expected(case)
    fixed = ~np.isnan(exp)
    tol = 1e-2 if dtype == "bf16" else 1e-6
    np.testing.assert_allclose(got[fixed], exp[fixed], rtol=tol, atol=tol)


# ------------------------------------------------------------ the small workload (fp32)

@pytest.mark.parametrize("page_size", [16, 256])
def test_config1_fp32(page_size):
    c, _, _, _ = workloads.config1(page_size=page_size)
    _run_full(c, "config1 fp32 page %d" % page_size)


def test_config1_shape_in_bf16():
    rng = np.random.Generator(np.random.PCG64(1))
    for ps in (16, 64, 256):
        c = workloads.make_attn_case(rng, B=1, S=16, Hq=4, Hkv=1, D=64, ctx_lens=[48],
                                     page_size=ps, dtype="bf16")
        _run_full(c, "config1 shape bf16 page %d" % ps)


# ------------------------------------------------------------ edge cases, full compare

EDGE = [
    # name, B, S, Hq, Hkv, D, lens, page_size
    ("empty_context", 2, 16, 32, 2, 128, [0, 0], 256),
    ("decode_S1", 3, 1, 32, 2, 128, [1, 300, 4100], 256),
    ("tile_edges", 7, 16, 32, 2, 128, [1, 63, 64, 65, 255, 256, 257], 256),
    ("small_pages", 5, 16, 32, 2, 128, [16, 48, 70, 129, 200], 16),
    ("pages32", 3, 16, 32, 2, 128, [31, 32, 500], 32),
    ("head64_g4", 3, 16, 8, 2, 64, [48, 0, 333], 64),
    ("mha_g1", 2, 16, 4, 4, 128, [100, 7], 256),
    ("block8", 3, 8, 32, 2, 128, [0, 90, 1000], 256),
    ("two_query_chunks", 2, 32, 32, 2, 128, [80, 700], 256),
    ("block64_d128", 2, 64, 32, 2, 128, [64, 777], 256),
    ("four_query_chunks", 1, 64, 32, 2, 64, [129], 128),
    ("odd_block", 3, 5, 6, 3, 64, [17, 0, 90], 16),
    ("many_units", 100, 16, 32, 2, 128, list(range(0, 1000, 10)), 256),
    ("long_split", 1, 16, 32, 2, 128, [20000], 256),
    # S*g = 160: waves 0-4 hold rows (lag wave 4 among them), waves 5-7 are idle
    ("lag_partly_idle", 2, 10, 32, 2, 128, [100, 3000], 256),
    # S*g = 384: the second query chunk holds 128 rows, its waves 4-7 are idle
    ("second_chunk_half_full", 2, 24, 32, 2, 128, [90, 2000], 256),
    # S*g = 768: teams of 3 work-groups (the work-group count is a multiple of
    # 3, not of 8), ranges long enough that teams cut pairs
    ("three_chunk_teams", 3, 48, 32, 2, 128, [1500, 6000, 300], 256),
    # S*g = 4096: teams of 16 larger than the range count a tiny context
    # needs, so one team covers every tile
    ("one_team_16_chunks", 1, 64, 64, 1, 64, [100], 64),
    # S*g = 16384: teams of 64 chunks over a longer context
    ("teams_of_64_chunks", 1, 64, 256, 1, 128, [2000], 256),
    # two chunks per pair with 16-token pages (per-lane page lookups)
    ("two_chunks_small_pages", 2, 32, 32, 2, 128, [100, 900], 16),
    # the largest page size: a tile's keys and values inside one 4096-token page
    ("pages_4096", 2, 16, 32, 2, 128, [5000, 100], 4096),
    # the most heads: 4096 one-row units (S*g = 1), seven of eight waves idle
    ("max_heads_mha", 1, 1, 4096, 4096, 64, [10], 16),
]


@pytest.mark.parametrize("name,B,S,Hq,Hkv,D,lens,ps", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, B, S, Hq, Hkv, D, lens, ps):
    c = _case(sum(map(ord, name)), B, S, Hq, Hkv, D, lens, ps)
    _run_full(c, name)


def test_maximum_batch():
    """The largest batch the ABI accepts (2048 sequences): the device prefix
    scans 32 groups of 64 lengths, and each work-group's range spans many short
    units (lengths 0..299, some empty), compared whole-tensor and per unit."""
    lens = [int(x) for x in np.random.Generator(np.random.PCG64(2048)).integers(0, 300, 2048)]
    lens[:3] = [0, 0, 299]
    c = _case(2048, 2048, 1, 4, 2, 64, lens, 16)
    _run_full(c, "maximum batch")


def test_fp32_edge_cases():
    for seed, (B, S, Hq, Hkv, D, lens, ps) in enumerate([
            (2, 16, 4, 1, 64, [0, 48], 16), (2, 1, 8, 2, 128, [300, 1], 32),
            (1, 3, 3, 3, 200, [77], 64)]):
        c = _case(50 + seed, B, S, Hq, Hkv, D, lens, ps, dtype="f32")
        _run_full(c, "fp32 edge %d" % seed)


def test_max_ctx_len_above_actual_lengths():
    """A loose host bound only changes the launch plan, not the result."""
    c = _case(7, 4, 16, 32, 2, 128, [100, 2000, 0, 513], 256, extra_tokens=5000)
    dc = DevCase(c, max_ctx_len=c.page_table.shape[1] * 256)
    got = to_f64(dc.attn(), "bf16")
    assert_attn_close(got, oracle.block_attn(c), "bf16", "loose max_ctx_len")


# ------------------------------------------------------------ self-consistency

def test_page_permutation_bit_exact_and_deterministic():
    c = _case(31, 4, 16, 32, 2, 128, [1000, 3000, 17, 4096], 256)
    import torch
    a = DevCase(c).attn().cpu().view(torch.int16)
    b = DevCase(c).attn().cpu().view(torch.int16)
    assert a.equal(b), "rerun differs"
    P = c.k_pages.shape[0]
    perm = np.random.Generator(np.random.PCG64(9)).permutation(P)
    kp = np.empty_like(c.k_pages); vp = np.empty_like(c.v_pages)
    kp[perm] = c.k_pages
    vp[perm] = c.v_pages
    c.page_table = np.where(c.page_table >= 0, perm[np.maximum(c.page_table, 0)], -1).astype(np.int32)
    c.k_pages, c.v_pages = kp, vp
    d = DevCase(c).attn().cpu().view(torch.int16)
    assert a.equal(d), "output changed under a physical page permutation"


def test_gqa_equals_mha_with_repeated_kv():
    c = _case(41, 2, 16, 8, 2, 128, [300, 129], 64)
    gq = to_f64(DevCase(c).attn(), "bf16")
    g = c.Hq // c.Hkv
    m = workloads.AttnCase(**{**c.__dict__})
    m.Hkv = c.Hq
    m.k_blk = np.repeat(c.k_blk, g, axis=2)
    m.v_blk = np.repeat(c.v_blk, g, axis=2)
    m.k_pages = np.repeat(c.k_pages, g, axis=1)
    m.v_pages = np.repeat(c.v_pages, g, axis=1)
    mh = to_f64(DevCase(m).attn(), "bf16")
    np.testing.assert_allclose(gq, mh, rtol=0, atol=1e-2)


# ------------------------------------------------------------ full-size workloads, whole tensor

def _whole_parity(c, name):
    """Every output element against the oracle (run on all host threads),
    with the rel-L2 bound applied per (b, h_kv) unit as well."""
    dc = DevCase(c)
    out = to_f64(dc.attn(), "bf16")
    ref = oracle.block_attn(c)
    assert_attn_units(out, ref, c.Hkv, "bf16", name)


@pytest.mark.timeout(300)
def test_config2_full_size():
    _whole_parity(workloads.config2(), "config2 B=8 L=4096")


@pytest.mark.timeout(600)
def test_config3_full_size():
    _whole_parity(workloads.config3(), "config3 B=64 ragged 1K..16K")


@pytest.mark.timeout(600)
def test_config4_full_size():
    _whole_parity(workloads.config4(), "config4 B=4 L=65536")


@pytest.mark.timeout(900)
def test_ranges_spanning_several_page_cache_fills():
    """With 16-token pages a work-group caches the page ids of at most 255
    tiles at a time, so a longer range is processed in several sub-ranges,
    each refilling the cache from a different page base (pages of at least
    256 tokens would need over a million tiles per launch for that).  B=1
    with 16 KV heads of 256K tokens gives 65,616 flat tiles, more than
    255 per work-group at up to 256 work-groups: every range crosses a
    sub-range boundary, mostly in the middle of a page-table row."""
    c = _case(77, 1, 16, 16, 16, 64, [262144], 16)
    _run_full(c, "256K tokens, 16-token pages")

