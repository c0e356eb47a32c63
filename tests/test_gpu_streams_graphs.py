"""GPU: the entry points on a caller's non-default stream and under HIP graph
capture, against the same calls launched eagerly on the default stream.

The kernels are deterministic (fixed reduction orders, no atomics on data),
so every comparison here is bitwise.  The graph is replayed several times
with eager library work and poisoned outputs in between, and every replay is
checked."""
import numpy as np
import pytest

import workloads
from gpu_util import DevCase, torch_mod

pytestmark = pytest.mark.gpu


class Inputs:
    """One attention layer, one unmask and one LM-head call, with output and
    workspace buffers of their own."""

    def __init__(self, seed=31):
        import two_tower_attention_amd as tt
        torch = torch_mod()
        self.tt = tt
        rng = np.random.Generator(np.random.PCG64(seed))
        case = workloads.make_attn_case(rng, B=4, S=16, Hq=32, Hkv=2, D=128,
                                        ctx_lens=[100, 1000, 2047, 3000], page_size=256, seed=seed)
        self.dc = DevCase(case)
        B, S, V = 4, 16, 3000
        self.logits = torch.from_numpy(workloads.make_logits(rng, B * S, V)).cuda()
        self.mask = torch.from_numpy((rng.random((B, S)) < 0.7).astype(np.uint8)).cuda()
        self.uws = torch.empty(max(tt.tt_unmask_workspace_bytes(B, S, V), 16), dtype=torch.uint8, device="cuda")
        lm = workloads.make_lmhead_case(rng, B, S, 512, 4096)
        bf = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()
        self.hidden, self.weight = bf(lm.hidden), bf(lm.weight)
        self.lws = torch.empty(max(tt.tt_lmhead_unmask_workspace_bytes(B, S, 4096, 512), 16),
                               dtype=torch.uint8, device="cuda")
        self.B, self.S = B, S

    def outputs(self):
        torch = torch_mod()
        B, S = self.B, self.S
        o = {"attn": self.dc.new_out()}
        for k in ("u", "lm"):
            o[k + "_ids"] = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
            o[k + "_commit"] = torch.full((B, S), 7, dtype=torch.uint8, device="cuda")
            o[k + "_conf"] = torch.full((B, S), float("nan"), dtype=torch.float32, device="cuda")
        return o

    def run(self, o, stream=None):
        """Attention, unmask and LM head (flags 0: the mask is read only)."""
        tt, d = self.tt, self.dc
        tt.tt_block_attn(d.desc, d.q, d.k_blk, d.v_blk, d.k_pages, d.v_pages, d.page_table, d.ctx_lens,
                         o["attn"], d.ws, stream)
        tt.tt_unmask(self.logits, self.mask, None, 4, o["u_ids"], o["u_commit"], o["u_conf"], 0,
                     self.uws, stream)
        tt.tt_lmhead_unmask(self.hidden, self.weight, self.mask, None, 4, o["lm_ids"], o["lm_commit"],
                            o["lm_conf"], 0, self.lws, stream)

    @staticmethod
    def poison(o):
        o["attn"].fill_(float("nan"))
        for k in ("u", "lm"):
            o[k + "_ids"].fill_(-1)
            o[k + "_commit"].fill_(7)
            o[k + "_conf"].fill_(float("nan"))


def assert_same(got, ref, what):
    torch = torch_mod()
    for k in ref:
        assert torch.equal(got[k], ref[k]), "%s: %s differs" % (what, k)


def test_side_stream_matches_default_stream():
    torch = torch_mod()
    x = Inputs()
    ref = x.outputs()
    x.run(ref)
    torch.cuda.synchronize()
    assert not torch.isnan(ref["attn"].float()).any()
    side = torch.cuda.Stream()
    got = x.outputs()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        x.run(got, side)
    side.synchronize()
    assert_same(got, ref, "side stream")
    # and once more on the default stream: run-to-run determinism
    again = x.outputs()
    x.run(again)
    torch.cuda.synchronize()
    assert_same(again, ref, "second default-stream run")


def test_graph_capture_replays():
    torch = torch_mod()
    x = Inputs(seed=32)
    ref = x.outputs()
    x.run(ref)
    torch.cuda.synchronize()
    got = x.outputs()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            x.run(got)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    scratch = x.outputs()
    for replay in range(3):
        Inputs.poison(got)
        x.run(scratch)            # eager library work between replays, same workspaces
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_same(got, ref, "graph replay %d" % replay)
        assert_same(scratch, ref, "eager run between replays %d" % replay)
