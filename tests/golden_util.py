"""Decode the sparse tensor fixtures under tests/golden/ into numpy arrays."""
import json
import os
import types

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _val(v):
    if isinstance(v, str):
        return float(v)          # "nan", "-inf", "-0.0" ...
    return float(v)


def _idx(i):
    if isinstance(i, str):
        if i == ":":
            return slice(None)
        a, b = i.split(":")
        return slice(int(a) if a else None, int(b) if b else None)
    return int(i)


def tensor(spec, dtype=np.float32):
    a = np.full(spec["shape"], _val(spec["fill"]), dtype=dtype)
    for entry in spec["set"]:
        a[tuple(_idx(i) for i in entry[:-1])] = _val(entry[-1])
    return a


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def attn_case(c, dtype="f32"):
    """A workloads.AttnCase-like namespace for a hand case (fp32 arrays, or bf16 bits)."""
    arrs = {k: tensor(c[k]) for k in ("q", "k_blk", "v_blk", "k_pages", "v_pages")}
    if dtype == "bf16":
        from workloads import bf16_bits
        arrs = {k: bf16_bits(v) for k, v in arrs.items()}
    pt = np.asarray(c["page_table"], dtype=np.int32)
    return types.SimpleNamespace(
        B=c["B"], S=c["S"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], page_size=c["page_size"],
        max_pages=pt.shape[1], num_pages=arrs["k_pages"].shape[0], dtype=dtype,
        scale=c["scale"], ctx_lens=np.asarray(c["ctx_lens"], dtype=np.int32), page_table=pt,
        **arrs)


def expected(c):
    """Full expected output [B,S,Hq,D] (NaN where the case does not fix a value)."""
    out = np.full((c["B"], c["S"], c["Hq"], c["D"]), np.nan)
    e = c["expect"]
    if "all" in e:
        out[...] = e["all"]
    for b, t, h, v in e.get("rows", []):
        out[b, t, h, :] = v
    return out
