"""CPU oracle for the TwoTower denoiser block-attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library in ``two_tower_attention_amd/`` and never imports it.

The arithmetic lives in ``tt_oracle.c`` (plain fp64 loops, OpenMP over rows);
this module builds it with gcc, marshals numpy arrays, and composes the
block-commit append and the denoise loop, which are pure data movement and
control flow.

Sources (page title and section):

* "Nemotron-Labs-TwoTower: Diffusion Language Modeling with Pretrained
  Autoregressive Context" (paperfeed.app review) -- "The idea: freeze the
  reader, train the writer" (block attention over [context cache ; block KV],
  block commit and cache ingest), "Training and sampling" (confidence
  unmasking).
* "NVIDIA's Dual-Tower Diffusion Language Model Explained" (kongchang.com) --
  "Generating Text in Parallel Like Solving a Sudoku" (16-slot block, predict
  all, commit confident ones, committed tokens stay fixed).
* "NVIDIA Bolted a Diffusion Model Onto a Frozen LLM ..." (aibacon.net) --
  "Why a builder should care" (16-token blocks, a budget of 16 steps).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtt_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile tt_oracle.c with gcc -O2 -fopenmp into oracle/libtt_oracle.so."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.tto_block_attn.argtypes = [I, I, I, I, I, I, I, I, ctypes.c_double, I,
                                       P, P, P, P, P, P, P, I, P, P, P]
        lib.tto_block_attn.restype = I
        lib.tto_chunk_attn.argtypes = lib.tto_block_attn.argtypes
        lib.tto_chunk_attn.restype = I
        lib.tto_unmask.argtypes = [I, I, I, P, P, P, I, P, P, P]
        lib.tto_unmask.restype = I
        lib.tto_unmask_threshold.argtypes = [I, I, I, P, P, ctypes.c_double, P, P, P, P]
        lib.tto_unmask_threshold.restype = I
        lib.tto_lmhead_logits.argtypes = [I, I, I, P, P, P, I, P]
        lib.tto_lmhead_logits.restype = I
        lib.tto_unmask_f64.argtypes = [I, I, I, P, P, P, I, P, P, P]
        lib.tto_unmask_f64.restype = I
        lib.tto_num_threads.argtypes = []
        lib.tto_num_threads.restype = I
        lib.tto_set_num_threads.argtypes = [I]
        lib.tto_set_num_threads.restype = None
        _lib = lib
    return _lib


class library:
    """Context manager that points the wrappers at another build of the oracle
    (used by the test that plants mistakes in a copy of tt_oracle.c)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib, _LIB_PATH
        self._saved = (_lib, _LIB_PATH)
        _lib, _LIB_PATH = None, self.path
        return self

    def __exit__(self, *exc):
        global _lib, _LIB_PATH
        _lib, _LIB_PATH = self._saved
        return False


def num_threads() -> int:
    return int(_load().tto_num_threads())


class threads:
    """Context manager: run the oracle on n OpenMP threads inside the block."""

    def __init__(self, n: int):
        self.n = int(n)

    def __enter__(self):
        self._saved = num_threads()
        _load().tto_set_num_threads(self.n)
        return self

    def __exit__(self, *exc):
        _load().tto_set_num_threads(self._saved)
        return False


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a, dtype=dtype)


def block_attn(c, rows: Optional[Sequence[Sequence[int]]] = None, with_wsum: bool = False,
               q=None, k_blk=None, v_blk=None, k_pages=None, v_pages=None,
               ctx_lens=None, page_table=None, causal: bool = False):
    """fp64 block attention (``causal``: the context tower's chunk ingest, where
    chunk position t sees chunk tokens 0..t only).

    ``c`` carries the shapes and arrays (any object with the attribute names
    used by ``workloads.AttnCase``); keyword arrays override its fields.
    Returns ``out`` as float64 ``[B, S, Hq, D]`` (rows None) or
    ``[len(rows), D]`` for the requested (b, t, h) rows; with ``with_wsum`` also
    the per-row sum of the normalised softmax weights.
    """
    is_bf16 = 1 if c.dtype == "bf16" else 0
    el = np.uint16 if is_bf16 else np.float32
    q = _c(c.q if q is None else q, el)
    k_blk = _c(c.k_blk if k_blk is None else k_blk, el)
    v_blk = _c(c.v_blk if v_blk is None else v_blk, el)
    k_pages = _c(c.k_pages if k_pages is None else k_pages, el)
    v_pages = _c(c.v_pages if v_pages is None else v_pages, el)
    ctx_lens = _c(c.ctx_lens if ctx_lens is None else ctx_lens, np.int32)
    page_table = _c(c.page_table if page_table is None else page_table, np.int32)
    B, S, Hq, D = c.B, c.S, c.Hq, c.D
    if rows is None:
        out = np.zeros((B, S, Hq, D), dtype=np.float64)
        ws = np.zeros((B, S, Hq), dtype=np.float64) if with_wsum else None
        rows_arr, n = None, 0
    else:
        rows_arr = _c(np.asarray(rows, dtype=np.int32).reshape(-1, 3), np.int32)
        n = rows_arr.shape[0]
        out = np.zeros((n, D), dtype=np.float64)
        ws = np.zeros((n,), dtype=np.float64) if with_wsum else None
    fn = _load().tto_chunk_attn if causal else _load().tto_block_attn
    err = fn(B, S, Hq, c.Hkv, D, c.page_size, page_table.shape[1],
             k_pages.shape[0], float(c.scale), is_bf16,
             _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(k_pages),
             _ptr(v_pages), _ptr(page_table), _ptr(ctx_lens), n,
             _ptr(rows_arr), _ptr(out), _ptr(ws))
    if err:
        raise ValueError("oracle block_attn failed with code %d" % err)
    return (out, ws) if with_wsum else out


def unmask(logits: np.ndarray, mask: np.ndarray, k_commit: Optional[np.ndarray] = None,
           remaining_steps: int = 1):
    """Exact unmask: returns (ids int32 [B,S], commit uint8 [B,S], conf float64 [B,S])."""
    mask = _c(mask, np.uint8)
    B, S = mask.shape
    logits = _c(logits, np.float32).reshape(B * S, -1)
    V = logits.shape[1]
    ids = np.zeros((B, S), dtype=np.int32)
    commit = np.zeros((B, S), dtype=np.uint8)
    conf = np.zeros((B, S), dtype=np.float64)
    kc = None if k_commit is None else _c(k_commit, np.int32).reshape(B)
    err = _load().tto_unmask(B, S, V, _ptr(logits), _ptr(mask), _ptr(kc),
                             int(remaining_steps), _ptr(ids), _ptr(commit), _ptr(conf))
    if err:
        raise ValueError("oracle unmask failed with code %d" % err)
    return ids, commit, conf


def lmhead_logits(hidden: np.ndarray, weight: np.ndarray,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Exact LM-head logits in fp64: hidden [R, H] and weight [V, H] as bf16
    bit patterns (uint16); returns [len(rows) or R, V]."""
    hidden = _c(hidden, np.uint16)
    weight = _c(weight, np.uint16)
    R, H = hidden.shape
    V, H2 = weight.shape
    if H2 != H:
        raise ValueError("hidden and weight disagree on the hidden size")
    sel = None if rows is None else _c(np.asarray(rows, dtype=np.int32), np.int32)
    n = R if sel is None else sel.shape[0]
    out = np.zeros((n, V), dtype=np.float64)
    err = _load().tto_lmhead_logits(R, H, V, _ptr(hidden), _ptr(weight), _ptr(sel), n, _ptr(out))
    if err:
        raise ValueError("oracle lmhead_logits failed with code %d" % err)
    return out


def unmask_f64(logits: np.ndarray, mask: np.ndarray, k_commit: Optional[np.ndarray] = None,
               remaining_steps: int = 1):
    """The count-form unmask (as unmask()) on fp64 logits [B*S, V]."""
    mask = _c(mask, np.uint8)
    B, S = mask.shape
    logits = _c(logits, np.float64).reshape(B * S, -1)
    V = logits.shape[1]
    ids = np.zeros((B, S), dtype=np.int32)
    commit = np.zeros((B, S), dtype=np.uint8)
    conf = np.zeros((B, S), dtype=np.float64)
    kc = None if k_commit is None else _c(k_commit, np.int32).reshape(B)
    err = _load().tto_unmask_f64(B, S, V, _ptr(logits), _ptr(mask), _ptr(kc),
                                 int(remaining_steps), _ptr(ids), _ptr(commit), _ptr(conf))
    if err:
        raise ValueError("oracle unmask_f64 failed with code %d" % err)
    return ids, commit, conf


def lmhead_unmask(hidden: np.ndarray, weight: np.ndarray, mask: np.ndarray,
                  k_commit: Optional[np.ndarray] = None, remaining_steps: int = 1,
                  seqs: Optional[Sequence[int]] = None, with_logits: bool = False):
    """LM head then count-form unmask.  hidden [B*S, H] and weight [V, H] as
    bf16 bits, mask [B, S].  ``seqs`` restricts the evaluation to those
    sequences (the commit ranks within a sequence, so whole sequences are the
    unit); results then have len(seqs) rows of S."""
    mask = _c(mask, np.uint8)
    B, S = mask.shape
    if seqs is None:
        seqs = list(range(B))
    seqs = [int(b) for b in seqs]
    rows = [b * S + t for b in seqs for t in range(S)]
    logits = lmhead_logits(hidden, weight, rows)
    kc = None if k_commit is None else np.asarray(k_commit, dtype=np.int32).reshape(B)[seqs]
    res = unmask_f64(logits, mask[seqs], kc, remaining_steps)
    return res + (logits,) if with_logits else res


def unmask_threshold(logits: np.ndarray, mask: np.ndarray, gamma: float,
                     nsteps: Optional[np.ndarray] = None):
    """Threshold form of the commit rule: every masked position with confidence
    strictly above ``gamma`` is committed; when none is, the most confident
    masked position is (lower position on ties).  Returns (ids int32 [B,S],
    commit uint8 [B,S], conf float64 [B,S], nsteps int32 [B]) where nsteps is
    the input count (zeros if None) plus one for each sequence that had a
    masked position."""
    mask = _c(mask, np.uint8)
    B, S = mask.shape
    logits = _c(logits, np.float32).reshape(B * S, -1)
    V = logits.shape[1]
    ids = np.zeros((B, S), dtype=np.int32)
    commit = np.zeros((B, S), dtype=np.uint8)
    conf = np.zeros((B, S), dtype=np.float64)
    ns = np.zeros(B, np.int32) if nsteps is None else np.array(nsteps, dtype=np.int32, copy=True)
    err = _load().tto_unmask_threshold(B, S, V, _ptr(logits), _ptr(mask), float(gamma), _ptr(ids),
                                       _ptr(commit), _ptr(conf), _ptr(ns))
    if err:
        raise ValueError("oracle threshold unmask failed with code %d" % err)
    return ids, commit, conf, ns


def adaptive_unmask_loop(logits_per_step: Sequence[np.ndarray], B: int, S: int, gamma: float,
                         max_steps: int):
    """The adaptive-step sampler of one block ("Training and sampling",
    paperfeed review): starting from an all-masked block, each step commits by
    the threshold rule and clears the committed mask bits, until every
    sequence's block is resolved or ``max_steps`` steps have run (the pages'
    budget is 16).  Step s uses logits_per_step[s % len(logits_per_step)].

    Returns a dict with per-step ``ids``, ``commit``, ``conf``, ``mask`` (after
    the step), the final ``nsteps`` per sequence and ``steps`` run."""
    mask = np.ones((B, S), dtype=np.uint8)
    ns = np.zeros(B, np.int32)
    res = {"ids": [], "commit": [], "conf": [], "mask": []}
    s = 0
    while s < max_steps and mask.any():
        lg = logits_per_step[s % len(logits_per_step)]
        ids, commit, conf, ns = unmask_threshold(lg, mask, gamma, ns)
        mask = (mask & (1 - commit)).astype(np.uint8)
        res["ids"].append(ids); res["commit"].append(commit); res["conf"].append(conf)
        res["mask"].append(mask.copy())
        s += 1
    res["nsteps"] = ns
    res["steps"] = s
    return res


def kv_append(k_pages: np.ndarray, v_pages: np.ndarray, page_table: np.ndarray,
              ctx_lens: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray):
    """Block commit: write the block's keys/values at logical positions
    L_b .. L_b+S-1 of each sequence's paged cache and grow L_b by S.

    "The idea: freeze the reader, train the writer" (paperfeed review): once a
    block is resolved the context tower ingests it and updates its caches; the
    cache then grows by one committed block.  Returns new copies
    (k_pages, v_pages, ctx_lens); inputs are not modified.
    """
    k_pages = k_pages.copy()
    v_pages = v_pages.copy()
    ctx_lens = np.array(ctx_lens, dtype=np.int32, copy=True)
    B, S = k_blk.shape[0], k_blk.shape[1]
    ps = k_pages.shape[2]
    for b in range(B):
        L = int(ctx_lens[b])
        for t in range(S):
            pos = L + t
            page = int(page_table[b, pos // ps])
            if page < 0 or page >= k_pages.shape[0]:
                raise ValueError("no page allocated for position %d of sequence %d" % (pos, b))
            k_pages[page, :, pos % ps, :] = k_blk[b, t]
            v_pages[page, :, :, pos % ps] = v_blk[b, t]
        ctx_lens[b] = L + S
    return k_pages, v_pages, ctx_lens


def denoise_loop(loop, attn_rows=None, check_attn: bool = True):
    """Reference run of one block's denoise loop.

    For s = 1..T: every layer i computes block attention over its own context
    cache and the block's keys/values of that step; then the unmask commits
    ceil(#masked / (T - s + 1)) positions per sequence and clears their mask
    bits.  After step T every position is committed and each layer's cache
    ingests the block (the final step's block keys/values stand in for the
    context tower's own).  The synthetic loop has no model between steps, so
    attention outputs are produced for checking but not fed forward.

    Returns a dict with per-step ``ids``, ``commit``, ``conf``, ``mask`` (after
    the step), per-(step, layer) attention outputs for ``attn_rows`` (all rows
    when None, if ``check_attn``), and the appended pools and lengths.
    """
    B, S, T = loop.B, loop.S, loop.steps
    mask = np.ones((B, S), dtype=np.uint8)
    res = {"ids": [], "commit": [], "conf": [], "mask": [], "attn": []}
    for s in range(T):
        outs = []
        for i in range(loop.layers):
            if check_attn:
                outs.append(block_attn(loop.pools[i], rows=attn_rows, q=loop.q[s][i],
                                       k_blk=loop.k_blk[s][i], v_blk=loop.v_blk[s][i]))
        res["attn"].append(outs)
        ids, commit, conf = unmask(loop.logits[s], mask, None, T - s)
        mask = (mask & (1 - commit)).astype(np.uint8)
        res["ids"].append(ids); res["commit"].append(commit); res["conf"].append(conf)
        res["mask"].append(mask.copy())
    pools = []
    for i in range(loop.layers):
        p = loop.pools[i]
        pools.append(kv_append(p.k_pages, p.v_pages, p.page_table, p.ctx_lens,
                               loop.k_blk[T - 1][i], loop.v_blk[T - 1][i]))
    res["pools"] = pools
    return res
