"""Seeded synthetic inputs for the denoiser block-attention / unmask path.

This module only draws random numbers and lays them out in the memory layout
that ``include/tt.h`` documents; it holds none of the method's arithmetic.
Both the CPU oracle (``oracle/``) and the GPU library are fed from here, and
neither side imports the other.

Layouts (row-major, last index fastest):

* ``q``                 ``[B, S, H_q, D]``
* ``k_blk`` / ``v_blk`` ``[B, S, H_kv, D]``   the block's own keys / values
* ``k_pages``           ``[P, H_kv, page_size, D]``   context keys, token-major
* ``v_pages``           ``[P, H_kv, D, page_size]``   context values, stored
  transposed inside each page (feature-major)
* ``page_table``        ``int32 [B, max_pages]``; entry j of row b holds the
  physical page of tokens ``[j*page_size, (j+1)*page_size)``; unused = -1
* ``ctx_lens``          ``int32 [B]``

bf16 tensors are carried as ``uint16`` bit patterns (numpy has no bf16); the
fp32 draws are rounded to bf16 round-to-nearest-even by torch's CPU cast.

Draw order for one attention case: page permutation -> Q -> K_blk -> V_blk ->
K pool -> V pool.  Lengths are drawn first by the config builders.  Slots of
an allocated page that lie beyond a sequence's length are filled with a
poison value (bf16/fp32 NaN) so that any read past the committed context is
visible in the outputs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

__all__ = [
    "AttnCase", "make_attn_case", "bf16_bits", "bits_to_f32",
    "config1", "config2", "config3", "config4", "config5",
    "Loop", "make_logits", "NAN_BF16", "LmHeadCase", "make_lmhead_case",
]

NAN_BF16 = np.uint16(0x7FC0)
NAN_F32 = np.float32("nan")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE, via torch's CPU cast); return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class AttnCase:
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    page_size: int
    max_pages: int
    num_pages: int
    dtype: str                 # "bf16" or "f32"
    scale: float
    ctx_lens: np.ndarray       # int32 [B]
    page_table: np.ndarray     # int32 [B, max_pages]
    q: np.ndarray
    k_blk: np.ndarray
    v_blk: np.ndarray
    k_pages: np.ndarray
    v_pages: np.ndarray
    seed: int = 0

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_lens.max()) if self.B else 0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _draw(rng: np.random.Generator, shape, dtype: str, sigma: float = 1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return bf16_bits(x) if dtype == "bf16" else x


def block_inputs(rng: np.random.Generator, B: int, S: int, Hq: int, Hkv: int, D: int,
                 dtype: str = "bf16"):
    """Queries and the block's own keys/values, N(0, 1): q [B,S,Hq,D],
    k_blk and v_blk [B,S,Hkv,D] (bf16 bits or fp32)."""
    return (_draw(rng, (B, S, Hq, D), dtype), _draw(rng, (B, S, Hkv, D), dtype),
            _draw(rng, (B, S, Hkv, D), dtype))


def make_attn_case(rng: np.random.Generator, *, B: int, S: int, Hq: int, Hkv: int,
                   D: int, ctx_lens, page_size: int, dtype: str = "bf16",
                   extra_tokens: int = 0, shuffle_pages: bool = True,
                   poison_tail: bool = True, scale: Optional[float] = None,
                   seed: int = 0) -> AttnCase:
    """Draw one block-attention case.

    Every sequence b gets ``ceil((ctx_lens[b] + extra_tokens) / page_size)``
    pages (at least one), placed at physical ids from a random permutation of
    the whole pool when ``shuffle_pages``.
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32).reshape(B)
    caps = [max(1, math.ceil((int(L) + extra_tokens) / page_size)) for L in ctx_lens]
    P = int(sum(caps))
    max_pages = max(caps) if caps else 1
    perm = rng.permutation(P).astype(np.int32) if shuffle_pages else np.arange(P, dtype=np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b, c in enumerate(caps):
        page_table[b, :c] = perm[off:off + c]
        off += c
    q = _draw(rng, (B, S, Hq, D), dtype)
    k_blk = _draw(rng, (B, S, Hkv, D), dtype)
    v_blk = _draw(rng, (B, S, Hkv, D), dtype)
    k_pages = _draw(rng, (P, Hkv, page_size, D), dtype)
    v_pages = _draw(rng, (P, Hkv, D, page_size), dtype)
    if poison_tail:
        poison = NAN_BF16 if dtype == "bf16" else NAN_F32
        for b in range(B):
            L = int(ctx_lens[b])
            for pos in range(L, caps[b] * page_size):
                pg = page_table[b, pos // page_size]
                o = pos % page_size
                k_pages[pg, :, o, :] = poison
                v_pages[pg, :, :, o] = poison
    return AttnCase(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, page_size=page_size,
                    max_pages=max_pages, num_pages=P, dtype=dtype,
                    scale=(1.0 / math.sqrt(D)) if scale is None else float(scale),
                    ctx_lens=ctx_lens, page_table=page_table, q=q, k_blk=k_blk,
                    v_blk=v_blk, k_pages=k_pages, v_pages=v_pages, seed=seed)


def make_logits(rng: np.random.Generator, rows: int, vocab: int, sigma: float = 3.0) -> np.ndarray:
    """fp32 logits ``[rows, vocab]`` ~ N(0, sigma^2)."""
    return _draw(rng, (rows, vocab), "f32", sigma)


# ---------------------------------------------------------------------------
# The five measured workloads.  Seeds 1..5 by default.
# ---------------------------------------------------------------------------

def config1(seed: int = 1, page_size: int = 16):
    """Tiny fp32 case: B=1, H_q=4, H_kv=1, D=64, S=16, L=48; unmask on
    [16, 1024] logits ~ N(0, 3^2), all 16 masked, k=4."""
    rng = np.random.Generator(np.random.PCG64(seed))
    case = make_attn_case(rng, B=1, S=16, Hq=4, Hkv=1, D=64, ctx_lens=[48],
                          page_size=page_size, dtype="f32", seed=seed)
    logits = make_logits(rng, 16, 1024)
    mask = np.ones((1, 16), dtype=np.uint8)
    k = np.array([4], dtype=np.int32)
    return case, logits, mask, k


def config2(seed: int = 2):
    """B=8, H_q=32, H_kv=2, D=128, S=16, every L=4096, 256-token pages."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return make_attn_case(rng, B=8, S=16, Hq=32, Hkv=2, D=128,
                          ctx_lens=[4096] * 8, page_size=256, seed=seed)


def config3_lens(rng: np.random.Generator, B: int = 64) -> np.ndarray:
    return (16 * rng.integers(64, 1025, size=B)).astype(np.int32)


def config3(seed: int = 3, B: int = 64):
    """Ragged decode-serving batch: B=64, L uniform over multiples of 16 in [1024, 16384]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = config3_lens(rng, B)
    return make_attn_case(rng, B=B, S=16, Hq=32, Hkv=2, D=128, ctx_lens=lens,
                          page_size=256, seed=seed)


def config4(seed: int = 4, B: int = 4, L: int = 65536):
    """Long context: B=4, L=65536 per sequence."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return make_attn_case(rng, B=B, S=16, Hq=32, Hkv=2, D=128, ctx_lens=[L] * B,
                          page_size=256, seed=seed)


@dataclasses.dataclass
class Loop:
    """Inputs of the block denoise loop: per-layer context pools (sharing one
    length vector and one page table shape), per (step, layer) block
    tensors, and per-step logits."""
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    layers: int
    steps: int
    vocab: int
    page_size: int
    pools: List[AttnCase]            # one per layer; q/k_blk/v_blk of step 0
    q: list                          # [steps][layers] arrays [B,S,Hq,D]
    k_blk: list
    v_blk: list
    logits: list                     # [steps] fp32 [B*S, vocab]
    seed: int = 5


def config5(seed: int = 5, B: int = 32, layers: int = 6, steps: int = 4,
            vocab: int = 131072, lo: int = 2048, hi: int = 8192,
            extra_blocks: int = 1, Hq: int = 32, Hkv: int = 2, D: int = 128,
            page_size: int = 256) -> Loop:
    """Full denoise loop for one block: B=32, 6 attention layers with
    independent context pools, L uniform over multiples of 16 in [2048, 8192],
    T=4 steps, logits [B*16, 131072] ~ N(0, 3^2) per step.  ``extra_blocks``
    sizes the pools for that many appended 16-token blocks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    S = 16
    lens = (16 * rng.integers(lo // 16, hi // 16 + 1, size=B)).astype(np.int32)
    pools = [make_attn_case(rng, B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, ctx_lens=lens,
                            page_size=page_size, extra_tokens=S * extra_blocks,
                            seed=seed) for _ in range(layers)]
    q, kb, vb = [], [], []
    for s in range(steps):
        q.append([]); kb.append([]); vb.append([])
        for _ in range(layers):
            q[s].append(_draw(rng, (B, S, Hq, D), "bf16"))
            kb[s].append(_draw(rng, (B, S, Hkv, D), "bf16"))
            vb[s].append(_draw(rng, (B, S, Hkv, D), "bf16"))
    logits = [make_logits(rng, B * S, vocab) for _ in range(steps)]
    return Loop(B=B, S=S, Hq=Hq, Hkv=Hkv, D=D, layers=layers, steps=steps,
                vocab=vocab, page_size=page_size, pools=pools, q=q, k_blk=kb,
                v_blk=vb, logits=logits, seed=seed)


# ---------------------------------------------------------------------------
# Peaked logits for the threshold (adaptive-step) sampler.  N(0, 3^2) logits
# over a large vocabulary never give a greedy probability near 0.8, so each
# row gets one spiked entry whose height sets its confidence.  The shape of
# the schedule follows what the pages report about the sampler: most slots
# resolve at the first step, the rest over a short tail, earlier slots more
# readily than later ones.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class PeakedBlock:
    B: int
    S: int
    vocab: int
    difficulty: np.ndarray      # [B*S] in [0, 1)
    spike_ids: np.ndarray       # [B*S] int64, the entry that is spiked in every step
    seed: int


def make_peaked_block(rng: np.random.Generator, B: int, S: int, vocab: int,
                      seed: int = 0) -> PeakedBlock:
    return PeakedBlock(B=B, S=S, vocab=vocab, difficulty=rng.random(B * S),
                       spike_ids=rng.integers(0, vocab, size=B * S), seed=seed)


def peaked_logits(rng: np.random.Generator, blk: PeakedBlock, step: int,
                  sigma: float = 3.0) -> np.ndarray:
    """fp32 logits [B*S, vocab] for one sampler step: N(0, sigma^2) plus, per
    row, a spike of height ln(vocab) + sigma^2/2 + margin at spike_ids, where
    margin = 4 - 4*difficulty - 0.15*slot + step + 0.3*N(0, 1).  A margin of
    about ln 4 puts the greedy probability near 0.8."""
    rows = blk.B * blk.S
    x = _draw(rng, (rows, blk.vocab), "f32", sigma)
    slot = np.tile(np.arange(blk.S), blk.B)
    margin = 4.0 - 4.0 * blk.difficulty - 0.15 * slot + step + 0.3 * rng.standard_normal(rows)
    height = np.log(blk.vocab) + 0.5 * sigma * sigma + margin
    x[np.arange(rows), blk.spike_ids] = height.astype(np.float32)
    return x


# ---------------------------------------------------------------------------
# LM head ahead of the unmask.  The pages give no head shape; the hidden size
# is H_q * D of the attention configs (4096) and the vocabulary that of the
# unmask workload (131072).  Weights are scaled so that the logits are
# ~ N(0, sigma^2), the distribution of the unmask workload's logits.
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class LmHeadCase:
    B: int
    S: int
    H: int
    V: int
    hidden: np.ndarray   # uint16 bf16 bits [B*S, H]
    weight: np.ndarray   # uint16 bf16 bits [V, H]
    seed: int


def make_lmhead_case(rng: np.random.Generator, B: int, S: int, H: int, V: int,
                     sigma: float = 3.0, row_scale: Optional[np.ndarray] = None,
                     seed: int = 0) -> LmHeadCase:
    """Hidden state ~ N(0, 1) (times ``row_scale[r]`` per row when given: larger
    scales give more confident rows) and head weights ~ N(0, sigma^2 / H),
    drawn hidden first, then the weight in blocks of vocabulary rows."""
    hidden = rng.standard_normal((B * S, H), dtype=np.float32)
    if row_scale is not None:
        hidden *= np.asarray(row_scale, dtype=np.float32).reshape(-1, 1)
    hidden_bits = bf16_bits(hidden)
    weight = np.empty((V, H), dtype=np.uint16)
    step = max(1, (1 << 24) // H)
    for v0 in range(0, V, step):
        n = min(step, V - v0)
        w = rng.standard_normal((n, H), dtype=np.float32)
        w *= np.float32(sigma / math.sqrt(H))
        weight[v0:v0 + n] = bf16_bits(w)
    return LmHeadCase(B=B, S=S, H=H, V=V, hidden=hidden_bits, weight=weight, seed=seed)
