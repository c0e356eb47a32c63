"""Python binding of libtt.so, the MI355X (gfx950) TwoTower denoiser
block-attention library.

Argument marshalling only: every entry point takes torch tensors that live on
the GPU, checks their dtype, contiguity and element counts, and passes raw
device pointers plus the current HIP stream to the C function of the same
name (include/tt.h).  All arithmetic runs in the library's HIP kernels; there
is no CPU fallback.  Importing this package does not load the library;
the first call does, and raises ``LibraryMissing`` if it has not been built
(``python -m two_tower_attention_amd.build`` or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtt.so")

TT_OK = 0
TT_BF16 = 0
TT_F32 = 1
TT_UNMASK_UPDATE_MASK = 1

EXPORTS = ("tt_block_attn_workspace_bytes", "tt_block_attn", "tt_chunk_attn", "tt_kv_append",
           "tt_unmask_workspace_bytes", "tt_unmask", "tt_unmask_noalloc", "tt_unmask_threshold",
           "tt_lmhead_unmask_workspace_bytes", "tt_lmhead_unmask", "tt_lmhead_unmask_threshold",
           "tt_status_str",
           "tt_last_error", "tt_abi_version")


class LibraryMissing(ImportError):
    pass


class TTError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (tt_status_str(status), status, msg))
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("block", ctypes.c_int32),
                ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_ctx_len", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libtt.so (no GPU needed to load it)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise LibraryMissing("libtt.so is not built at %s; run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    DP = ctypes.POINTER(AttnDesc)
    lib.tt_block_attn_workspace_bytes.argtypes = [DP, ctypes.POINTER(SZ)]
    lib.tt_block_attn.argtypes = [DP, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.tt_chunk_attn.argtypes = [DP, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.tt_kv_append.argtypes = [DP, P, P, P, P, P, P, P]
    lib.tt_unmask_workspace_bytes.argtypes = [I32, I32, I32, ctypes.POINTER(SZ)]
    lib.tt_unmask.argtypes = [P, P, P, I32, I32, I32, I32, P, P, P, ctypes.c_uint32, P, SZ, P]
    lib.tt_unmask_noalloc.argtypes = [P, P, P, I32, I32, I32, I32, P, P, P, ctypes.c_uint32, P]
    lib.tt_unmask_threshold.argtypes = [P, P, ctypes.c_float, I32, I32, I32, P, P, P, P,
                                        ctypes.c_uint32, P, SZ, P]
    lib.tt_lmhead_unmask_workspace_bytes.argtypes = [I32, I32, I32, I32, ctypes.POINTER(SZ)]
    lib.tt_lmhead_unmask.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, P, P, P,
                                     ctypes.c_uint32, P, SZ, P]
    lib.tt_lmhead_unmask_threshold.argtypes = [P, P, P, ctypes.c_float, I32, I32, I32, I32, P, P,
                                               P, P, ctypes.c_uint32, P, SZ, P]
    lib.tt_status_str.argtypes = [ctypes.c_int]
    lib.tt_status_str.restype = ctypes.c_char_p
    lib.tt_last_error.argtypes = []
    lib.tt_last_error.restype = ctypes.c_char_p
    lib.tt_abi_version.argtypes = []
    for name in ("tt_block_attn_workspace_bytes", "tt_block_attn", "tt_kv_append",
                 "tt_unmask_workspace_bytes", "tt_unmask", "tt_unmask_noalloc", "tt_unmask_threshold",
                 "tt_lmhead_unmask_workspace_bytes", "tt_lmhead_unmask",
                 "tt_lmhead_unmask_threshold", "tt_abi_version"):
        getattr(lib, name).restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def tt_status_str(status: int) -> str:
    return load_library().tt_status_str(int(status)).decode()


def tt_last_error() -> str:
    return load_library().tt_last_error().decode()


def _check(status: int):
    if status != TT_OK:
        raise TTError(status, tt_last_error())


def make_desc(B: int, S: int, Hq: int, Hkv: int, D: int, page_size: int, max_pages: int,
              num_pages: int, max_ctx_len: int, scale: float = 0.0,
              dtype: str = "bf16") -> AttnDesc:
    return AttnDesc(B, S, Hq, Hkv, D, page_size, max_pages, num_pages, max_ctx_len,
                    float(scale), TT_BF16 if dtype == "bf16" else TT_F32)


# ---------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _ptr(t, name, dtype=None, numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must have dtype %s, has %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s has %d elements, needs %d" % (name, t.numel(), numel))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _el(desc: AttnDesc):
    torch = _torch()
    return torch.bfloat16 if desc.dtype == TT_BF16 else torch.float32


def tt_block_attn_workspace_bytes(desc: AttnDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().tt_block_attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def tt_block_attn(desc: AttnDesc, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens,
                  out, workspace=None, stream=None) -> None:
    _attn("tt_block_attn", desc, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens, out,
          workspace, stream)


def tt_chunk_attn(desc: AttnDesc, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens,
                  out, workspace=None, stream=None) -> None:
    """Causal chunk ingest (see include/tt.h); same arguments as tt_block_attn."""
    _attn("tt_chunk_attn", desc, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens, out,
          workspace, stream)


def _attn(name, desc, q, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens, out, workspace,
          stream):
    torch = _torch()
    el = _el(desc)
    B, S, Hq, Hkv, D = desc.batch, desc.block, desc.heads_q, desc.heads_kv, desc.head_dim
    ctx = desc.max_ctx_len > 0
    P = desc.num_pages * Hkv * desc.page_size * D
    args = [_ptr(q, "q", el, B * S * Hq * D), _ptr(k_blk, "k_blk", el, B * S * Hkv * D),
            _ptr(v_blk, "v_blk", el, B * S * Hkv * D),
            _ptr(k_pages, "k_pages", el, P, allow_none=not ctx),
            _ptr(v_pages, "v_pages", el, P, allow_none=not ctx),
            _ptr(page_table, "page_table", torch.int32, B * desc.max_pages_per_seq,
                 allow_none=not ctx),
            _ptr(ctx_lens, "ctx_lens", torch.int32, B), _ptr(out, "out", el, B * S * Hq * D)]
    ws = _ptr(workspace, "workspace", allow_none=True)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(getattr(load_library(), name)(ctypes.byref(desc), *args, ws, nbytes, _stream(stream)))


def tt_kv_append(desc: AttnDesc, k_blk, v_blk, k_pages, v_pages, page_table, ctx_lens,
                 stream=None) -> None:
    torch = _torch()
    el = _el(desc)
    B, S, Hkv, D = desc.batch, desc.block, desc.heads_kv, desc.head_dim
    P = desc.num_pages * Hkv * desc.page_size * D
    _check(load_library().tt_kv_append(
        ctypes.byref(desc), _ptr(k_blk, "k_blk", el, B * S * Hkv * D),
        _ptr(v_blk, "v_blk", el, B * S * Hkv * D), _ptr(k_pages, "k_pages", el, P),
        _ptr(v_pages, "v_pages", el, P),
        _ptr(page_table, "page_table", torch.int32, B * desc.max_pages_per_seq),
        _ptr(ctx_lens, "ctx_lens", torch.int32, B), _stream(stream)))


def tt_unmask_workspace_bytes(batch: int, block: int, vocab: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().tt_unmask_workspace_bytes(batch, block, vocab, ctypes.byref(n)))
    return n.value


def tt_unmask(logits, mask, k_commit, remaining_steps: int, ids_out, commit_out,
              conf_out=None, flags: int = 0, workspace=None, stream=None) -> None:
    torch = _torch()
    B, S = mask.shape
    V = logits.shape[-1]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().tt_unmask(
        _ptr(logits, "logits", torch.float32, B * S * V), _ptr(mask, "mask", torch.uint8, B * S),
        _ptr(k_commit, "k_commit", torch.int32, B, allow_none=True), int(remaining_steps),
        B, S, V, _ptr(ids_out, "ids_out", torch.int32, B * S),
        _ptr(commit_out, "commit_out", torch.uint8, B * S),
        _ptr(conf_out, "conf_out", torch.float32, B * S, allow_none=True), int(flags),
        _ptr(workspace, "workspace", allow_none=True), nbytes, _stream(stream)))


def tt_unmask_noalloc(logits, mask, k_commit, remaining_steps: int, ids_out, commit_out,
                      conf_out=None, flags: int = 0, stream=None) -> None:
    """tt_unmask with its row partials in the library's static device array
    (no workspace; see include/tt.h)."""
    torch = _torch()
    B, S = mask.shape
    V = logits.shape[-1]
    _check(load_library().tt_unmask_noalloc(
        _ptr(logits, "logits", torch.float32, B * S * V), _ptr(mask, "mask", torch.uint8, B * S),
        _ptr(k_commit, "k_commit", torch.int32, B, allow_none=True), int(remaining_steps),
        B, S, V, _ptr(ids_out, "ids_out", torch.int32, B * S),
        _ptr(commit_out, "commit_out", torch.uint8, B * S),
        _ptr(conf_out, "conf_out", torch.float32, B * S, allow_none=True), int(flags),
        _stream(stream)))


def tt_unmask_threshold(logits, mask, gamma: float, ids_out, commit_out, conf_out=None,
                        nsteps=None, flags: int = 0, workspace=None, stream=None) -> None:
    """Threshold form of the commit rule (see include/tt.h)."""
    torch = _torch()
    B, S = mask.shape
    V = logits.shape[-1]
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().tt_unmask_threshold(
        _ptr(logits, "logits", torch.float32, B * S * V), _ptr(mask, "mask", torch.uint8, B * S),
        float(gamma), B, S, V, _ptr(ids_out, "ids_out", torch.int32, B * S),
        _ptr(commit_out, "commit_out", torch.uint8, B * S),
        _ptr(conf_out, "conf_out", torch.float32, B * S, allow_none=True),
        _ptr(nsteps, "nsteps", torch.int32, B, allow_none=True), int(flags),
        _ptr(workspace, "workspace", allow_none=True), nbytes, _stream(stream)))


def tt_lmhead_unmask_workspace_bytes(batch: int, block: int, vocab: int, hidden: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().tt_lmhead_unmask_workspace_bytes(batch, block, vocab, hidden,
                                                           ctypes.byref(n)))
    return n.value


def tt_lmhead_unmask(hidden, weight, mask, k_commit, remaining_steps: int, ids_out, commit_out,
                     conf_out=None, flags: int = 0, workspace=None, stream=None) -> None:
    """LM head fused with the count-form unmask (see include/tt.h)."""
    torch = _torch()
    B, S = mask.shape
    V, H = weight.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().tt_lmhead_unmask(
        _ptr(hidden, "hidden", torch.bfloat16, B * S * H), _ptr(weight, "weight", torch.bfloat16, V * H),
        _ptr(mask, "mask", torch.uint8, B * S),
        _ptr(k_commit, "k_commit", torch.int32, B, allow_none=True), int(remaining_steps),
        B, S, V, H, _ptr(ids_out, "ids_out", torch.int32, B * S),
        _ptr(commit_out, "commit_out", torch.uint8, B * S),
        _ptr(conf_out, "conf_out", torch.float32, B * S, allow_none=True), int(flags),
        _ptr(workspace, "workspace", allow_none=True), nbytes, _stream(stream)))


def tt_lmhead_unmask_threshold(hidden, weight, mask, gamma: float, ids_out, commit_out,
                               conf_out=None, nsteps=None, flags: int = 0, workspace=None,
                               stream=None) -> None:
    """LM head fused with the threshold-form unmask (see include/tt.h)."""
    torch = _torch()
    B, S = mask.shape
    V, H = weight.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().tt_lmhead_unmask_threshold(
        _ptr(hidden, "hidden", torch.bfloat16, B * S * H), _ptr(weight, "weight", torch.bfloat16, V * H),
        _ptr(mask, "mask", torch.uint8, B * S), float(gamma), B, S, V, H,
        _ptr(ids_out, "ids_out", torch.int32, B * S),
        _ptr(commit_out, "commit_out", torch.uint8, B * S),
        _ptr(conf_out, "conf_out", torch.float32, B * S, allow_none=True),
        _ptr(nsteps, "nsteps", torch.int32, B, allow_none=True), int(flags),
        _ptr(workspace, "workspace", allow_none=True), nbytes, _stream(stream)))
