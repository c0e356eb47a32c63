"""Helpers for the GPU parity tests: move a workloads case to the device, run
the library through its C ABI (the Python binding), and compare with the
oracle under the stated tolerances."""
import numpy as np

import workloads

# bf16 attention output vs the fp64 oracle (whole tensor): the stated contract
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 1e-2
# fp32 path
F32_MAX_ABS = 1e-4
F32_REL_L2 = 1e-5
# commit sets may differ only where the oracle's confidence is this close to
# the k-th largest masked confidence
COMMIT_TIE = 1e-6


def torch_mod():
    import torch
    return torch


def dev_tensor(a: np.ndarray, dtype: str):
    """numpy (bf16 bits as uint16, or float32/int32/uint8) -> GPU tensor."""
    torch = torch_mod()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def to_f64(t, dtype: str) -> np.ndarray:
    torch = torch_mod()
    if dtype == "bf16":
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        return workloads.bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


class DevCase:
    """Device copies of an AttnCase plus its descriptor and workspace."""

    def __init__(self, c, max_ctx_len=None):
        import two_tower_attention_amd as tt
        torch = torch_mod()
        self.c = c
        self.q = dev_tensor(c.q, c.dtype)
        self.k_blk = dev_tensor(c.k_blk, c.dtype)
        self.v_blk = dev_tensor(c.v_blk, c.dtype)
        self.k_pages = dev_tensor(c.k_pages, c.dtype)
        self.v_pages = dev_tensor(c.v_pages, c.dtype)
        self.page_table = dev_tensor(c.page_table, "i32")
        self.ctx_lens = dev_tensor(c.ctx_lens, "i32")
        mcl = int(c.ctx_lens.max()) if max_ctx_len is None else int(max_ctx_len)
        self.desc = tt.make_desc(c.B, c.S, c.Hq, c.Hkv, c.D, c.page_size, c.page_table.shape[1],
                                 c.k_pages.shape[0], mcl, c.scale, c.dtype)
        nbytes = tt.tt_block_attn_workspace_bytes(self.desc)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        el = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.el = el

    def new_out(self):
        torch = torch_mod()
        c = self.c
        return torch.full((c.B, c.S, c.Hq, c.D), float("nan"), dtype=self.el, device="cuda")

    def attn(self, out=None, q=None, k_blk=None, v_blk=None, causal=False):
        import two_tower_attention_amd as tt
        out = self.new_out() if out is None else out
        self.ws.fill_(0xFF)   # NaN-poison the workspace: partials must be written before use
        fn = tt.tt_chunk_attn if causal else tt.tt_block_attn
        fn(self.desc, self.q if q is None else q,
                         self.k_blk if k_blk is None else k_blk,
                         self.v_blk if v_blk is None else v_blk, self.k_pages, self.v_pages,
                         self.page_table, self.ctx_lens, out, self.ws)
        return out


def attn_errors(got: np.ndarray, ref: np.ndarray):
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


def assert_attn_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite output (unwritten or poisoned) " + what
    max_abs, rel = attn_errors(got, ref)
    lim_abs, lim_rel = (ATTN_MAX_ABS, ATTN_REL_L2) if dtype == "bf16" else (F32_MAX_ABS, F32_REL_L2)
    assert max_abs <= lim_abs and rel <= lim_rel, \
        "%s max_abs=%.3g (<= %.3g) rel_l2=%.3g (<= %.3g)" % (what, max_abs, lim_abs, rel, lim_rel)
    return max_abs, rel


def assert_attn_units(got: np.ndarray, ref: np.ndarray, Hkv: int, dtype: str, what: str = ""):
    """Whole-tensor bound, then the rel-L2 bound again on every (b, h_kv) unit
    (its S x g query rows), so an error confined to one unit (a dropped or
    doubled tile of one sequence) cannot hide in the aggregate.  Outputs are
    [B, S, Hq, D] with query head h reading key/value head h // g."""
    assert_attn_close(got, ref, dtype, what)
    B, S, Hq, D = ref.shape
    g = Hq // Hkv
    lim_rel = ATTN_REL_L2 if dtype == "bf16" else F32_REL_L2
    gu = got.reshape(B, S, Hkv, g, D)
    ru = ref.reshape(B, S, Hkv, g, D)
    num = np.sqrt(((gu - ru) ** 2).sum(axis=(1, 3, 4)))
    den = np.maximum(np.sqrt((ru ** 2).sum(axis=(1, 3, 4))), 1e-300)
    rel = num / den
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape)
    assert rel.max() <= lim_rel, "%s unit (b=%d, h_kv=%d) rel_l2=%.3g (<= %.3g)" % (
        what, worst[0], worst[1], rel.max(), lim_rel)
    return float(rel.max())


def assert_commit_ok(commit_gpu, commit_ref, conf_ref, mask, k_eff, tie=COMMIT_TIE, rel=False):
    """Commit comparator: exact count, only masked slots, and any difference
    from the oracle's set only among near-ties of the k-th confidence c*:
    |conf - c*| <= tie, or <= tie * c* with ``rel`` (for confidences computed
    from logits that carry a rounding error, whose effect on 1/Z is relative)."""
    B, S = mask.shape
    for b in range(B):
        cg, cr = commit_gpu[b].astype(bool), commit_ref[b].astype(bool)
        m = mask[b].astype(bool)
        assert cg.sum() == k_eff[b], (b, cg.sum(), k_eff[b])
        assert not np.any(cg & ~m), "committed an unmasked slot in sequence %d" % b
        diff = np.nonzero(cg ^ cr)[0]
        if diff.size:
            masked_conf = np.sort(conf_ref[b][m])[::-1]
            cstar = masked_conf[k_eff[b] - 1]
            band = tie * cstar if rel else tie
            assert np.all(np.abs(conf_ref[b][diff] - cstar) <= band), \
                (b, diff, conf_ref[b][diff], cstar, band)


def assert_threshold_commit_ok(commit_gpu, conf_ref, mask, gamma, tie=COMMIT_TIE, rel=False):
    """Threshold-rule comparator.  The GPU decides conf > gamma on its fp32
    confidence, the oracle's confidence is fp64, so a slot whose oracle
    confidence lies within COMMIT_TIE of gamma may go either way; the same band
    applies to ties of the fallback's maximum.  Everything else is fixed:
    only masked slots commit; slots surely above gamma commit, slots surely
    below it do not (unless a fallback); a fallback commits exactly one slot
    among the most confident.  With ``rel`` the band is ``tie`` times the
    confidence it is taken around (gamma, or the fallback's maximum)."""
    B, S = mask.shape
    for b in range(B):
        cg = commit_gpu[b].astype(bool)
        m = mask[b].astype(bool)
        c = conf_ref[b]
        assert not np.any(cg & ~m), "committed an unmasked slot in sequence %d" % b
        if not m.any():
            assert not cg.any()
            continue
        gband = tie * abs(gamma) if rel else tie
        sure = m & (c > gamma + gband)
        near = m & (np.abs(c - gamma) <= gband)
        if sure.any():
            assert np.all(cg[sure]), (b, "a slot surely above gamma was not committed")
            assert not np.any(cg & m & ~sure & ~near), (b, "a slot surely below gamma committed")
            continue
        # nothing surely above: either the GPU judged some near-gamma slots
        # above gamma (then exactly those commit), or none (then the fallback
        # commits one slot whose confidence is within the band of the maximum)
        assert cg.any(), (b, "no progress")
        judged_above = np.all(near[cg])
        mband = tie * c[m].max() if rel else tie
        fallback = cg.sum() == 1 and abs(c[cg][0] - c[m].max()) <= mband
        assert judged_above or fallback, (b, np.nonzero(cg)[0], c[cg], c[m].max())
