"""Host-side checks of libtt.so that need no GPU: it loads, exports every
function include/tt.h declares, and its argument validation returns the
documented status before touching a device."""
import ctypes
import os
import re

import pytest

import two_tower_attention_amd as tt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tt.h")

FAKE = ctypes.c_void_p(1 << 20)     # aligned, never dereferenced on the host


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tt.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return tt.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(tt.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.tt_abi_version() == 1
    for code in range(0, -8, -1):
        s = tt.tt_status_str(code)
        assert s.startswith("TT_"), s
    assert "unknown" in tt.tt_status_str(-99)


def good_desc(**kw):
    d = dict(B=2, S=16, Hq=32, Hkv=2, D=128, page_size=256, max_pages=4, num_pages=8,
             max_ctx_len=1000, scale=0.0, dtype="bf16")
    d.update(kw)
    return tt.make_desc(**d)


BAD = [
    ("dtype", dict(dtype="bf16"), {"dtype": 7}, -3),
    ("batch", {}, {"batch": -1}, -2),
    ("batch_big", {}, {"batch": 5000}, -2),
    ("block0", {}, {"block": 0}, -2),
    ("block65", {}, {"block": 65}, -2),
    ("gqa", {}, {"heads_q": 30, "heads_kv": 4}, -2),
    ("page_not_pow2", {}, {"page_size": 48}, -2),
    ("page_small", {}, {"page_size": 8}, -2),
    ("no_pages", {}, {"num_pages": 0}, -2),
    ("ctx_over_capacity", {}, {"max_ctx_len": 4 * 256 + 1}, -2),
    ("head_dim_bf16", {}, {"head_dim": 96}, -4),
    ("head_dim_f32", dict(dtype="f32"), {"head_dim": 300}, -4),
]


@pytest.mark.parametrize("name,base,patch,code", BAD, ids=[b[0] for b in BAD])
def test_desc_validation(lib, name, base, patch, code):
    d = good_desc(**base)
    for k, v in patch.items():
        setattr(d, k, v)
    n = ctypes.c_size_t(0)
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == code
    assert tt.tt_last_error() != ""
    st = lib.tt_block_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           FAKE, ctypes.c_size_t(1 << 30), None)
    assert st == code
    st = lib.tt_kv_append(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == code


def test_null_pointers(lib):
    d = good_desc()
    args = [FAKE] * 8
    for i in (0, 1, 2, 6, 7):       # q, k_blk, v_blk, ctx_lens, out
        a = list(args)
        a[i] = None
        assert lib.tt_block_attn(ctypes.byref(d), *a, FAKE, ctypes.c_size_t(1 << 30), None) == -1
    a = list(args)
    a[3] = None                     # k_pages with a context
    assert lib.tt_block_attn(ctypes.byref(d), *a, FAKE, ctypes.c_size_t(1 << 30), None) == -1
    d0 = good_desc(max_ctx_len=0)   # without context the pool may be NULL
    a[4] = a[5] = None
    st = lib.tt_block_attn(ctypes.byref(d0), *a, FAKE, ctypes.c_size_t(1 << 30), None)
    assert st in (0, -6)            # OK on a GPU machine, no device here
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(d), None) == -1


def test_misaligned_pointer(lib):
    d = good_desc()
    bad = ctypes.c_void_p((1 << 20) + 2)
    st = lib.tt_block_attn(ctypes.byref(d), bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           ctypes.c_size_t(1 << 30), None)
    assert st == -4


def test_batch_zero_is_noop(lib):
    d = good_desc(B=0)
    assert lib.tt_block_attn(ctypes.byref(d), None, None, None, None, None, None, None, None,
                             None, 0, None) == 0
    n = ctypes.c_size_t(7)
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0 and n.value == 0


def test_workspace_sizes(lib):
    n = ctypes.c_size_t(0)
    d = good_desc()
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value > 0 and n.value % 16 == 0
    d32 = good_desc(dtype="f32", D=64)
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(d32), ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.tt_unmask_workspace_bytes(32, 16, 131072, ctypes.byref(n)) == 0
    assert n.value >= 32 * 16 * 16


@pytest.mark.parametrize("B,S,Hq,Hkv,max_ctx,chunks", [
    (32, 16, 32, 2, 8192, 1), (32, 32, 32, 2, 8192, 2), (32, 48, 32, 2, 8192, 3),
    (32, 64, 32, 2, 8192, 4),
    (1, 64, 64, 1, 100, 16),  # a short context: 28 work-groups round down to one team of 16
])
def test_plan_uses_whole_query_chunk_teams(lib, B, S, Hq, Hkv, max_ctx, chunks):
    """The bf16 plan forms teams of one work-group per 256-row query chunk of a
    (sequence, KV head) pair, so its work-group count G is a whole number of
    teams (at least one), at most the 256 CUs planned for without a device.
    G is read back from the workspace size: the published prefix, then two
    partial slots per work-group (bf16 O of 256 rows x D, fp32 max and sum)."""
    D = 128
    d = good_desc(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, max_ctx_len=max_ctx, page_size=256,
                  max_pages=(max_ctx + 255) // 256, num_pages=B * ((max_ctx + 255) // 256))
    n = ctypes.c_size_t(0)
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    pre = ((B + 1) * 4 + 255) // 256 * 256
    slot = D * 256 * 2 + 256 * 2 * 4
    assert (n.value - pre) % (2 * slot) == 0
    G = (n.value - pre) // (2 * slot)
    assert G % chunks == 0 and chunks <= G <= max(256, chunks)
    if B == 1:
        assert G == chunks


def test_tile_count_beyond_device_index(lib):
    """The device plans with int tile indices: a shape whose flat tile list
    could exceed that range is rejected on the host (TT_ERR_SHAPE) by both the
    workspace query and the call, before any device work."""
    d = good_desc(B=2048, S=1, Hq=4096, Hkv=4096, D=64, page_size=4096, max_pages=256,
                  num_pages=1 << 20, max_ctx_len=1 << 20)
    n = ctypes.c_size_t(0)
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == -2
    assert "tiles" in tt.tt_last_error()
    st = lib.tt_block_attn(ctypes.byref(d), *([FAKE] * 8), FAKE, ctypes.c_size_t(1 << 40), None)
    assert st in (-2, -6)           # no device here: the device query may come first
    # just inside the bound: 2048 sequences x 16 KV heads x 16389 tiles < 2^31
    ok = good_desc(B=2048, S=1, Hq=16, Hkv=16, D=64, page_size=4096, max_pages=256,
                   num_pages=1 << 20, max_ctx_len=1 << 20)
    assert lib.tt_block_attn_workspace_bytes(ctypes.byref(ok), ctypes.byref(n)) == 0


def test_workspace_too_small(lib):
    d = good_desc()
    st = lib.tt_block_attn(ctypes.byref(d), *([FAKE] * 8), FAKE, ctypes.c_size_t(16), None)
    assert st in (-5, -6)           # size is checked after the device query


UNMASK_BAD = [
    ("block0", dict(S=0), -2),
    ("block65", dict(S=65), -2),
    ("vocab0", dict(V=0), -2),
    ("rows", dict(B=5000, S=16), -2),
    ("remaining0", dict(rem=0, k=None), -2),
    ("flags", dict(flags=2), -4),
]


@pytest.mark.parametrize("name,kw,code", UNMASK_BAD, ids=[u[0] for u in UNMASK_BAD])
def test_unmask_validation(lib, name, kw, code):
    a = dict(B=2, S=16, V=1024, rem=1, k=FAKE, flags=0)
    a.update(kw)
    st = lib.tt_unmask(FAKE, FAKE, a["k"], a["rem"], a["B"], a["S"], a["V"], FAKE, FAKE, None,
                       a["flags"], FAKE, ctypes.c_size_t(1 << 30), None)
    assert st == code


def test_unmask_nulls(lib):
    st = lib.tt_unmask(None, FAKE, FAKE, 1, 2, 16, 1024, FAKE, FAKE, None, 0, FAKE,
                       ctypes.c_size_t(1 << 30), None)
    assert st == -1


@pytest.mark.parametrize("name,kw,code", UNMASK_BAD, ids=[u[0] for u in UNMASK_BAD])
def test_unmask_noalloc_validation(lib, name, kw, code):
    """The no-workspace variant checks its arguments as tt_unmask does."""
    a = dict(B=2, S=16, V=1024, rem=1, k=FAKE, flags=0)
    a.update(kw)
    st = lib.tt_unmask_noalloc(FAKE, FAKE, a["k"], a["rem"], a["B"], a["S"], a["V"], FAKE, FAKE,
                               None, a["flags"], None)
    assert st == code
    assert lib.tt_unmask_noalloc(None, FAKE, FAKE, 1, 2, 16, 1024, FAKE, FAKE, None, 0, None) == -1
    assert lib.tt_unmask_noalloc(FAKE, FAKE, FAKE, 1, 0, 16, 1024, FAKE, FAKE, None, 0, None) == 0


def test_unmask_noalloc_static_scratch_holds_every_shape(lib):
    """The static array (1 MiB) holds the row partials of every shape the
    unmask accepts: the planner's need peaks at 16 B x max(B*S, 1023)."""
    limit = 1 << 20
    worst = 0
    for rows in list(range(1, 1100)) + [4095, 4096, 20000, 65535]:
        for S in (1, 16, 64):
            if rows % S:
                continue
            for V in (1, 7, 1024, 131072, 2 ** 31 - 1):
                n = ctypes.c_size_t(0)
                assert lib.tt_unmask_workspace_bytes(rows // S, S, V, ctypes.byref(n)) == 0
                worst = max(worst, n.value)
                assert n.value <= 16 * max(rows, 1023) <= limit, (rows, S, V, n.value)
    assert worst == 16 * 65535


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(tt.LibraryMissing):
        tt.load_library(str(tmp_path / "nope.so"))


THRESH_BAD = [
    ("block0", dict(S=0), -2),
    ("vocab0", dict(V=0), -2),
    ("gamma_nan", dict(gamma=float("nan")), -2),
    ("gamma_inf", dict(gamma=float("inf")), -2),
    ("flags", dict(flags=2), -4),
]


@pytest.mark.parametrize("name,kw,code", THRESH_BAD, ids=[u[0] for u in THRESH_BAD])
def test_unmask_threshold_validation(lib, name, kw, code):
    a = dict(B=2, S=16, V=1024, gamma=0.8, flags=0)
    a.update(kw)
    st = lib.tt_unmask_threshold(FAKE, FAKE, a["gamma"], a["B"], a["S"], a["V"], FAKE, FAKE, None,
                                 None, a["flags"], FAKE, ctypes.c_size_t(1 << 30), None)
    assert st == code


def test_unmask_threshold_nulls_and_workspace(lib):
    st = lib.tt_unmask_threshold(FAKE, None, 0.8, 2, 16, 1024, FAKE, FAKE, None, None, 0, FAKE,
                                 ctypes.c_size_t(1 << 30), None)
    assert st == -1
    st = lib.tt_unmask_threshold(FAKE, FAKE, 0.8, 2, 16, 131072, FAKE, FAKE, None, None, 0, FAKE,
                                 ctypes.c_size_t(16), None)
    assert st == tt.load_library().tt_unmask(FAKE, FAKE, None, 1, 2, 16, 131072, FAKE, FAKE, None,
                                             0, FAKE, ctypes.c_size_t(16), None)
    assert st == -5


LMHEAD_BAD = [
    ("hidden31", dict(H=31), -2),
    ("hidden0", dict(H=0), -2),
    ("hidden_too_big", dict(H=65536 + 32), -2),
    ("block0", dict(S=0), -2),
    ("vocab0", dict(V=0), -2),
    ("remaining0", dict(rem=0, k=None), -2),
    ("flags", dict(flags=2), -4),
    # 256 row tiles x 2^23 vocabulary tiles: 2^31 work-groups, one too many
    ("grid_too_large", dict(B=4095, S=16, V=2**31 - 1), -2),
]


@pytest.mark.parametrize("name,kw,code", LMHEAD_BAD, ids=[u[0] for u in LMHEAD_BAD])
def test_lmhead_validation(lib, name, kw, code):
    a = dict(B=2, S=16, V=1000, H=256, rem=1, k=FAKE, flags=0)
    a.update(kw)
    st = lib.tt_lmhead_unmask(FAKE, FAKE, FAKE, a["k"], a["rem"], a["B"], a["S"], a["V"], a["H"],
                              FAKE, FAKE, None, a["flags"], FAKE, ctypes.c_size_t(1 << 30), None)
    assert st == code
    if name != "remaining0":
        st = lib.tt_lmhead_unmask_threshold(FAKE, FAKE, FAKE, 0.8, a["B"], a["S"], a["V"], a["H"],
                                            FAKE, FAKE, None, None, a["flags"], FAKE,
                                            ctypes.c_size_t(1 << 30), None)
        assert st == code


def test_lmhead_nulls_alignment_workspace(lib):
    args = lambda hid, w, ws, n: (hid, w, FAKE, None, 1, 2, 16, 1000, 256, FAKE, FAKE, None, 0, ws,
                                  ctypes.c_size_t(n), None)
    assert lib.tt_lmhead_unmask(*args(None, FAKE, FAKE, 1 << 30)) == -1
    assert lib.tt_lmhead_unmask(*args(FAKE, None, FAKE, 1 << 30)) == -1
    odd = ctypes.c_void_p((1 << 20) + 8)  # 8-byte aligned only
    assert lib.tt_lmhead_unmask(*args(odd, FAKE, FAKE, 1 << 30)) == -4
    assert lib.tt_lmhead_unmask(*args(FAKE, odd, FAKE, 1 << 30)) == -4
    need = ctypes.c_size_t(0)
    assert lib.tt_lmhead_unmask_workspace_bytes(2, 16, 1000, 256, ctypes.byref(need)) == 0
    # per (row, 128-entry chunk) partials plus one merged partial per row, 16 bytes each
    assert need.value >= 32 * (8 + 1) * 16
    assert lib.tt_lmhead_unmask(*args(FAKE, FAKE, FAKE, need.value - 1)) == -5
    assert lib.tt_lmhead_unmask(*args(FAKE, FAKE, None, 1 << 30)) == -5
    zero = ctypes.c_size_t(7)
    assert lib.tt_lmhead_unmask_workspace_bytes(0, 16, 1000, 256, ctypes.byref(zero)) == 0
    assert zero.value == 0
    assert lib.tt_lmhead_unmask(FAKE, FAKE, FAKE, None, 1, 0, 16, 1000, 256, FAKE, FAKE, None, 0,
                                None, ctypes.c_size_t(0), None) == 0
