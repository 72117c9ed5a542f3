"""Thin Python binding of libtreeverify.so (the C ABI in include/tree_verify.h).

Argument marshalling only: torch tensors supply device memory and the current HIP stream; every
step of the computation runs in the library's HIP kernels.  Output tensors that the caller does
not pass are allocated here with torch.  Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

TV_OK, TV_ERR_INVALID_ARG, TV_ERR_UNSUPPORTED, TV_ERR_WORKSPACE, TV_ERR_HIP = 0, -1, -2, -3, -4
TV_F32, TV_BF16 = 0, 1
TV_BAD_TREE, TV_OVERFLOW, TV_BAD_LEN, TV_BAD_PATH, TV_BAD_PAGE = 0x1, 0x2, 0x4, 0x8, 0x10
TV_BAD_TOKEN, TV_SYNC_TIMEOUT, TV_BAD_CONF, TV_FREE_FULL = 0x20, 0x40, 0x80, 0x100

EXPORTS = ("tv_status_string", "tree_build_mask", "tree_verify_attn_workspace_size",
           "tree_verify_attn", "tree_accept", "kv_compact_accepted", "tv_profile_attn_main",
           "tree_verify_step", "tree_verify_step_noalloc", "tree_verify_attn_paged",
           "kv_commit_paged",
           "tree_verify_step_paged",
           "tree_accept_stochastic", "tree_accept_stochastic_workspace_size",
           "tv_profile_accept_stochastic", "eagle2_node_count", "eagle2_expand",
           "eagle2_rerank", "lm_head_project", "lm_head_screen", "lm_head_rescore",
           "lm_head_topk")


class TreeVerifyError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({code})")
        self.code = code


_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _build.LIB


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libtreeverify.so (no build here: run __graft_entry__.build() or build.py first)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or _build.LIB
        if not os.path.exists(p):
            raise ImportError(f"libtreeverify.so not found at {p}; build it with "
                              "`python -m tree_attention_verification_attn_amd.build`")
        lib = ctypes.CDLL(p)
        _declare(lib)
        if path is None:
            _lib = lib
        return lib


def _declare(lib: ctypes.CDLL) -> None:
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.tv_status_string.argtypes = [I]
    lib.tv_status_string.restype = ctypes.c_char_p
    lib.tree_build_mask.argtypes = [P, I, I, P, P, P]
    lib.tree_build_mask.restype = I
    lib.tree_verify_attn_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.tree_verify_attn_workspace_size.restype = ctypes.c_size_t
    lib.tree_verify_attn.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P,
                                     ctypes.c_size_t, P]
    lib.tree_verify_attn.restype = I
    lib.tree_accept.argtypes = [P, P, P, I, I, P, P, P, P]
    lib.tree_accept.restype = I
    lib.kv_compact_accepted.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, P]
    lib.kv_compact_accepted.restype = I
    lib.tv_profile_attn_main.argtypes = [P, P]
    lib.tv_profile_attn_main.restype = I
    lib.tree_verify_step.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                     I, I, I, I, I, I, I, F, I, P, ctypes.c_size_t, P]
    lib.tree_verify_step.restype = I
    lib.tree_verify_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                             I, I, I, I, I, I, I, F, I, P]
    lib.tree_verify_step_noalloc.restype = I
    lib.tree_verify_attn_paged.argtypes = [P, P, P, I, P, I, I, P, P, P, P, P, P,
                                           I, I, I, I, I, I, F, I, P, ctypes.c_size_t, P]
    lib.tree_verify_attn_paged.restype = I
    lib.kv_commit_paged.argtypes = [P, I, I, P, P, P, P, P, P, P, I, I, I, P, P]
    lib.kv_commit_paged.restype = I
    lib.tree_verify_step_paged.argtypes = [P, P, P, P, P, P, I, P, I, I, P, P, P, P, P, P, P, P,
                                           P, P, P, P, I, I, I, I, I, I, F, I, P,
                                           ctypes.c_size_t, P]
    lib.tree_verify_step_paged.restype = I
    lib.tree_accept_stochastic.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, ctypes.c_size_t,
                                           P, P, P, P, P]
    lib.tree_accept_stochastic_workspace_size.argtypes = [I, I, I, I]
    lib.tree_accept_stochastic_workspace_size.restype = ctypes.c_size_t
    lib.tree_accept_stochastic.restype = I
    lib.tv_profile_accept_stochastic.argtypes = [P, P]
    lib.tv_profile_accept_stochastic.restype = I
    lib.eagle2_node_count.argtypes = [I, I, I]
    lib.eagle2_node_count.restype = I
    lib.eagle2_expand.argtypes = [P, P, P, I, I, I, I, P, P, P, I, P, P, P]
    lib.eagle2_expand.restype = I
    lib.eagle2_rerank.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, P]
    lib.eagle2_rerank.restype = I
    lib.lm_head_project.argtypes = [P, P, I, I, I, P, P]
    lib.lm_head_project.restype = I
    lib.lm_head_screen.argtypes = [P, P, P, I, I, I, I, I, P, P, P]
    lib.lm_head_screen.restype = I
    lib.lm_head_rescore.argtypes = [P, P, P, I, I, I, I, P, P, P]
    lib.lm_head_rescore.restype = I
    lib.lm_head_topk.argtypes = [P, P, I, I, I, I, P, P, P]
    lib.lm_head_topk.restype = I


def status_string(code: int) -> str:
    return load_library().tv_status_string(int(code)).decode()


def _check(fn: str, code: int) -> None:
    if code != TV_OK:
        raise TreeVerifyError(fn, code, status_string(code))


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TV_F32
    if t.dtype == torch.bfloat16:
        return TV_BF16
    raise TypeError(f"tree verification takes float32 or bfloat16 tensors, got {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def profile_attn_main(before: torch.cuda.Event | None, after: torch.cuda.Event | None) -> None:
    """Record `before`/`after` around every later tree_verify_attn main kernel (None, None: off).
    The events must have been recorded once (torch creates them lazily)."""
    ptr = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)  # noqa: E731
    _check("tv_profile_attn_main", load_library().tv_profile_attn_main(ptr(before), ptr(after)))


def profile_accept_stochastic(before: torch.cuda.Event | None,
                              after: torch.cuda.Event | None) -> None:
    """Record `before`/`after` around every later tree_accept_stochastic kernel (None: off)."""
    ptr = lambda e: None if e is None else ctypes.c_void_p(e.cuda_event)  # noqa: E731
    _check("tv_profile_accept_stochastic",
           load_library().tv_profile_accept_stochastic(ptr(before), ptr(after)))


def tree_build_mask(parent: torch.Tensor, anc_mask: torch.Tensor | None = None,
                    status: torch.Tensor | None = None, stream=None):
    """parent [B,T] int32 -> (anc_mask [B,T,W] uint64 as int64 storage, status [B] int32)."""
    _need(parent, "parent", torch.int32, 2)
    B, T = parent.shape
    W = (T + 63) // 64
    if anc_mask is None:
        anc_mask = torch.empty((B, T, W), dtype=torch.int64, device=parent.device)
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=parent.device)
    _need(anc_mask, "anc_mask", torch.int64, 3)
    _need(status, "status", torch.int32, 1)
    _check("tree_build_mask", load_library().tree_build_mask(
        _ptr(parent), B, T, _ptr(anc_mask), _ptr(status), _stream(stream)))
    return anc_mask, status


def tree_verify_attn_workspace_size(B: int, T: int, Hq: int, Hkv: int, D: int, Lmax: int,
                                    dtype: torch.dtype, split_keys: int = 0) -> int:
    code = TV_BF16 if dtype == torch.bfloat16 else TV_F32
    return int(load_library().tree_verify_attn_workspace_size(B, T, Hq, Hkv, D, Lmax, code,
                                                              split_keys))


def tree_verify_attn(q, k_cache, v_cache, cache_len, k_tree, v_tree, anc_mask, out=None,
                     lse=None, status=None, scale: float = 0.0, split_keys: int = 0,
                     workspace: torch.Tensor | None = None, with_lse: bool = True, stream=None):
    """Tree attention.  Returns (out [B,T,Hq,D], lse [B,T,Hq] float32 or None)."""
    _need(q, "q", None, 4)
    B, T, Hq, D = q.shape
    dt = _dtype_code(q)
    _need(k_cache, "k_cache", q.dtype, 4)
    _need(v_cache, "v_cache", q.dtype, 4)
    _need(k_tree, "k_tree", q.dtype, 4)
    _need(v_tree, "v_tree", q.dtype, 4)
    _need(cache_len, "cache_len", torch.int32, 1)
    _need(anc_mask, "anc_mask", torch.int64, 3)
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if (tuple(k_cache.shape) != (B, Hkv, Lmax, D) or tuple(v_cache.shape) != tuple(k_cache.shape)
            or tuple(k_tree.shape) != (B, T, Hkv, D) or tuple(v_tree.shape) != (B, T, Hkv, D)
            or tuple(cache_len.shape) != (B,) or tuple(anc_mask.shape) != (B, T, (T + 63) // 64)):
        raise ValueError("inconsistent tree_verify_attn shapes")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, 4)
    if lse is None and with_lse:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    ws_bytes = tree_verify_attn_workspace_size(B, T, Hq, Hkv, D, Lmax, q.dtype, split_keys)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tree_verify_attn", load_library().tree_verify_attn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(k_tree), _ptr(v_tree),
        _ptr(anc_mask), _ptr(out), _ptr(lse), _ptr(status), B, T, Hq, Hkv, D, Lmax, dt,
        float(scale), int(split_keys), _ptr(workspace), ws_have, _stream(stream)))
    return out, lse


def tree_accept(anc_mask, draft_tok, target_tok, accept_path=None, accept_len=None,
                bonus_tok=None, stream=None):
    """Greedy longest accepted path -> (accept_path [B,T], accept_len [B], bonus_tok [B])."""
    _need(anc_mask, "anc_mask", torch.int64, 3)
    _need(draft_tok, "draft_tok", torch.int32, 2)
    _need(target_tok, "target_tok", torch.int32, 2)
    B, T = draft_tok.shape
    if tuple(target_tok.shape) != (B, T) or tuple(anc_mask.shape) != (B, T, (T + 63) // 64):
        raise ValueError("inconsistent tree_accept shapes")
    dev = draft_tok.device
    accept_path = torch.empty((B, T), dtype=torch.int32, device=dev) if accept_path is None else accept_path
    accept_len = torch.empty((B,), dtype=torch.int32, device=dev) if accept_len is None else accept_len
    bonus_tok = torch.empty((B,), dtype=torch.int32, device=dev) if bonus_tok is None else bonus_tok
    _need(accept_path, "accept_path", torch.int32, 2)
    _need(accept_len, "accept_len", torch.int32, 1)
    _need(bonus_tok, "bonus_tok", torch.int32, 1)
    _check("tree_accept", load_library().tree_accept(
        _ptr(anc_mask), _ptr(draft_tok), _ptr(target_tok), B, T, _ptr(accept_path),
        _ptr(accept_len), _ptr(bonus_tok), _stream(stream)))
    return accept_path, accept_len, bonus_tok


def tree_accept_stochastic_workspace_size(B: int, T: int, V: int, workgroups_per_seq: int = 0) -> int:
    return int(load_library().tree_accept_stochastic_workspace_size(B, T, V, workgroups_per_seq))


def tree_accept_stochastic(anc_mask, draft_tok, p, q, u_acc, u_res, without_replacement=False,
                           workgroups_per_seq=0, workspace=None, accept_path=None, accept_len=None,
                           bonus_tok=None, status=None, stream=None):
    """Rejection-sampling acceptance over the tree: p, q [B,T,V] float32, u_acc, u_res [B,T]
    float64 -> (accept_path [B,T], accept_len [B], bonus_tok [B]).  `workspace` (uint8, zeroed
    once, then reused untouched) is allocated here when not given."""
    _need(anc_mask, "anc_mask", torch.int64, 3)
    _need(draft_tok, "draft_tok", torch.int32, 2)
    _need(p, "p", torch.float32, 3)
    _need(q, "q", torch.float32, 3)
    _need(u_acc, "u_acc", torch.float64, 2)
    _need(u_res, "u_res", torch.float64, 2)
    B, T = draft_tok.shape
    V = p.shape[2]
    if (tuple(anc_mask.shape) != (B, T, (T + 63) // 64) or tuple(p.shape) != (B, T, V)
            or tuple(q.shape) != (B, T, V) or tuple(u_acc.shape) != (B, T)
            or tuple(u_res.shape) != (B, T)):
        raise ValueError("inconsistent tree_accept_stochastic shapes")
    dev = draft_tok.device
    accept_path = torch.empty((B, T), dtype=torch.int32, device=dev) if accept_path is None else accept_path
    accept_len = torch.empty((B,), dtype=torch.int32, device=dev) if accept_len is None else accept_len
    bonus_tok = torch.empty((B,), dtype=torch.int32, device=dev) if bonus_tok is None else bonus_tok
    _need(accept_path, "accept_path", torch.int32, 2)
    _need(accept_len, "accept_len", torch.int32, 1)
    _need(bonus_tok, "bonus_tok", torch.int32, 1)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    need = tree_accept_stochastic_workspace_size(B, T, V, workgroups_per_seq)
    if workspace is None and need:
        workspace = torch.zeros((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tree_accept_stochastic", load_library().tree_accept_stochastic(
        _ptr(anc_mask), _ptr(draft_tok), _ptr(p), _ptr(q), _ptr(u_acc), _ptr(u_res), B, T, V,
        int(bool(without_replacement)), int(workgroups_per_seq), _ptr(workspace),
        ctypes.c_size_t(ws_bytes), _ptr(accept_path), _ptr(accept_len), _ptr(bonus_tok),
        _ptr(status), _stream(stream)))
    return accept_path, accept_len, bonus_tok


def kv_compact_accepted(k_cache, v_cache, cache_len, k_tree, v_tree, accept_path, accept_len,
                        cache_len_out=None, status=None, stream=None):
    """Append the accepted rows to the caches in place -> cache_len_out [B] int32."""
    _need(k_cache, "k_cache", None, 4)
    B, Hkv, Lmax, D = k_cache.shape
    dt = _dtype_code(k_cache)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    _need(cache_len, "cache_len", torch.int32, 1)
    _need(accept_path, "accept_path", torch.int32, 2)
    _need(accept_len, "accept_len", torch.int32, 1)
    T = accept_path.shape[1]
    dense = (T * Hkv * D, Hkv * D, D, 1)
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
        # may be a view into the cache itself (tree rows written in place during verification)
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != k_cache.dtype:
            raise ValueError(f"{name} must be a device tensor of the cache dtype")
        if tuple(t.shape) != (B, T, Hkv, D):
            raise ValueError(f"{name} must be [B,T,Hkv,D]")
        if any(sz > 1 and st != want for sz, st, want in zip(t.shape, t.stride(), dense)):
            raise ValueError(f"{name} must be laid out as a dense [B,T,Hkv,D] tensor")
    if tuple(v_cache.shape) != (B, Hkv, Lmax, D) or tuple(accept_len.shape) != (B,):
        raise ValueError("inconsistent kv_compact_accepted shapes")
    if cache_len_out is None:
        cache_len_out = torch.empty_like(cache_len)
    _need(cache_len_out, "cache_len_out", torch.int32, 1)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    _check("kv_compact_accepted", load_library().kv_compact_accepted(
        _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(cache_len_out), _ptr(k_tree),
        _ptr(v_tree), _ptr(accept_path), _ptr(accept_len), B, T, Hkv, D, Lmax, dt,
        _ptr(status), _stream(stream)))
    return cache_len_out


def tree_verify_step(parent, draft_tok, target_tok, q, k_cache, v_cache, cache_len, k_tree,
                     v_tree, cache_len_out=None, out=None, lse=None, anc_mask=None,
                     accept_path=None, accept_len=None, bonus_tok=None, status=None,
                     scale: float = 0.0, split_keys: int = 0,
                     workspace: torch.Tensor | None = None, with_lse: bool = True, stream=None):
    """One fused verification step (masks, attention, acceptance, compaction in place).

    Returns a dict with anc_mask, out, lse, accept_path, accept_len, bonus_tok, cache_len_out
    and status."""
    return _step(False, parent, draft_tok, target_tok, q, k_cache, v_cache, cache_len, k_tree,
                 v_tree, cache_len_out, out, lse, anc_mask, accept_path, accept_len, bonus_tok,
                 status, scale, split_keys, workspace, with_lse, stream)


def tree_verify_step_noalloc(parent, draft_tok, target_tok, q, k_cache, v_cache, cache_len,
                             k_tree, v_tree, cache_len_out=None, out=None, lse=None,
                             anc_mask=None, accept_path=None, accept_len=None, bonus_tok=None,
                             status=None, scale: float = 0.0, split_keys: int = 0,
                             with_lse: bool = True, stream=None):
    """tree_verify_step whose split-K workspace is the library's own device array: the library
    allocates nothing (outputs the caller does not pass are still allocated here, by torch)."""
    return _step(True, parent, draft_tok, target_tok, q, k_cache, v_cache, cache_len, k_tree,
                 v_tree, cache_len_out, out, lse, anc_mask, accept_path, accept_len, bonus_tok,
                 status, scale, split_keys, None, with_lse, stream)


def _step(noalloc, parent, draft_tok, target_tok, q, k_cache, v_cache, cache_len, k_tree,
          v_tree, cache_len_out, out, lse, anc_mask, accept_path, accept_len, bonus_tok, status,
          scale, split_keys, workspace, with_lse, stream):
    _need(parent, "parent", torch.int32, 2)
    _need(draft_tok, "draft_tok", torch.int32, 2)
    _need(target_tok, "target_tok", torch.int32, 2)
    _need(q, "q", None, 4)
    B, T, Hq, D = q.shape
    dt = _dtype_code(q)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_tree", k_tree),
                    ("v_tree", v_tree)):
        _need(t, name, q.dtype, 4)
    _need(cache_len, "cache_len", torch.int32, 1)
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    W = (T + 63) // 64
    if (tuple(k_cache.shape) != (B, Hkv, Lmax, D) or tuple(v_cache.shape) != tuple(k_cache.shape)
            or tuple(k_tree.shape) != (B, T, Hkv, D) or tuple(v_tree.shape) != (B, T, Hkv, D)
            or tuple(cache_len.shape) != (B,) or tuple(parent.shape) != (B, T)
            or tuple(draft_tok.shape) != (B, T) or tuple(target_tok.shape) != (B, T)):
        raise ValueError("inconsistent tree_verify_step shapes")
    dev = q.device
    new = lambda shape, dtype: torch.empty(shape, dtype=dtype, device=dev)  # noqa: E731
    anc_mask = new((B, T, W), torch.int64) if anc_mask is None else anc_mask
    out = torch.empty_like(q) if out is None else out
    if lse is None and with_lse:
        lse = new((B, T, Hq), torch.float32)
    accept_path = new((B, T), torch.int32) if accept_path is None else accept_path
    accept_len = new((B,), torch.int32) if accept_len is None else accept_len
    bonus_tok = new((B,), torch.int32) if bonus_tok is None else bonus_tok
    cache_len_out = torch.empty_like(cache_len) if cache_len_out is None else cache_len_out
    status = new((B,), torch.int32) if status is None else status
    _need(anc_mask, "anc_mask", torch.int64, 3)
    _need(out, "out", q.dtype, 4)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    for name, t in (("accept_len", accept_len), ("bonus_tok", bonus_tok),
                    ("cache_len_out", cache_len_out), ("status", status)):
        _need(t, name, torch.int32, 1)
    _need(accept_path, "accept_path", torch.int32, 2)
    args = (_ptr(parent), _ptr(draft_tok), _ptr(target_tok), _ptr(q), _ptr(k_cache),
            _ptr(v_cache), _ptr(cache_len), _ptr(cache_len_out), _ptr(k_tree), _ptr(v_tree),
            _ptr(anc_mask), _ptr(out), _ptr(lse), _ptr(accept_path), _ptr(accept_len),
            _ptr(bonus_tok), _ptr(status), B, T, Hq, Hkv, D, Lmax, dt, float(scale),
            int(split_keys))
    if noalloc:
        _check("tree_verify_step_noalloc",
               load_library().tree_verify_step_noalloc(*args, _stream(stream)))
    else:
        ws_bytes = tree_verify_attn_workspace_size(B, T, Hq, Hkv, D, Lmax, q.dtype, split_keys)
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
        ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check("tree_verify_step", load_library().tree_verify_step(
            *args, _ptr(workspace), ws_have, _stream(stream)))
    return dict(anc_mask=anc_mask, out=out, lse=lse, accept_path=accept_path,
                accept_len=accept_len, bonus_tok=bonus_tok, cache_len_out=cache_len_out,
                status=status)


def tree_verify_attn_paged(q, k_pool, v_pool, block_table, page_size: int, cache_len, tree_slot,
                           anc_mask, out=None, lse=None, status=None, scale: float = 0.0,
                           split_keys: int = 0, workspace: torch.Tensor | None = None,
                           with_lse: bool = True, stream=None):
    """Tree attention over a paged cache (pool [num_slots,Hkv,D], block table [B,max_pages])."""
    _need(q, "q", None, 4)
    B, T, Hq, D = q.shape
    dt = _dtype_code(q)
    _need(k_pool, "k_pool", q.dtype, 3)
    _need(v_pool, "v_pool", q.dtype, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_len, "cache_len", torch.int32, 1)
    _need(tree_slot, "tree_slot", torch.int32, 2)
    _need(anc_mask, "anc_mask", torch.int64, 3)
    num_slots, Hkv = k_pool.shape[0], k_pool.shape[1]
    max_pages = block_table.shape[1]
    if (tuple(k_pool.shape) != (num_slots, Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape)
            or block_table.shape[0] != B or tuple(tree_slot.shape) != (B, T)
            or tuple(cache_len.shape) != (B,) or tuple(anc_mask.shape) != (B, T, (T + 63) // 64)):
        raise ValueError("inconsistent tree_verify_attn_paged shapes")
    out = torch.empty_like(q) if out is None else out
    _need(out, "out", q.dtype, 4)
    if lse is None and with_lse:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    ws_bytes = tree_verify_attn_workspace_size(B, T, Hq, Hkv, D, max_pages * page_size, q.dtype,
                                               split_keys)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=q.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tree_verify_attn_paged", load_library().tree_verify_attn_paged(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), num_slots, _ptr(block_table), max_pages,
        int(page_size), _ptr(cache_len), _ptr(tree_slot), _ptr(anc_mask), _ptr(out), _ptr(lse),
        _ptr(status), B, T, Hq, Hkv, D, dt, float(scale), int(split_keys), _ptr(workspace),
        ws_have, _stream(stream)))
    return out, lse


def kv_commit_paged(block_table, cache_len, tree_slot, accept_path, accept_len, free_slots,
                    free_top, num_slots: int, page_size: int = 1, cache_len_out=None,
                    status=None, stream=None):
    """Pointer-swap commit (one-token pages); updates block_table, free_slots, free_top in place
    and returns cache_len_out [B] int32."""
    for name, t, nd in (("block_table", block_table, 2), ("cache_len", cache_len, 1),
                        ("tree_slot", tree_slot, 2), ("accept_path", accept_path, 2),
                        ("accept_len", accept_len, 1), ("free_slots", free_slots, 1),
                        ("free_top", free_top, 1)):
        _need(t, name, torch.int32, nd)
    B, max_pages = block_table.shape
    T = tree_slot.shape[1]
    if (tuple(cache_len.shape) != (B,) or tuple(tree_slot.shape) != (B, T)
            or tuple(accept_path.shape) != (B, T) or tuple(accept_len.shape) != (B,)
            or free_slots.numel() < num_slots or free_top.numel() != 1):
        raise ValueError("inconsistent kv_commit_paged shapes")
    cache_len_out = torch.empty_like(cache_len) if cache_len_out is None else cache_len_out
    _need(cache_len_out, "cache_len_out", torch.int32, 1)
    if status is not None:
        _need(status, "status", torch.int32, 1)
    _check("kv_commit_paged", load_library().kv_commit_paged(
        _ptr(block_table), max_pages, int(page_size), _ptr(cache_len), _ptr(cache_len_out),
        _ptr(tree_slot), _ptr(accept_path), _ptr(accept_len), _ptr(free_slots), _ptr(free_top),
        int(num_slots), B, T, _ptr(status), _stream(stream)))
    return cache_len_out


def tree_verify_step_paged(parent, draft_tok, target_tok, q, k_pool, v_pool, block_table,
                           cache_len, tree_slot, free_slots, free_top, page_size: int = 1,
                           cache_len_out=None, out=None, lse=None, anc_mask=None,
                           accept_path=None, accept_len=None, bonus_tok=None, status=None,
                           scale: float = 0.0, split_keys: int = 0,
                           workspace: torch.Tensor | None = None, with_lse: bool = True,
                           stream=None):
    """One fused verification step over a paged cache (masks, paged attention, acceptance,
    pointer-swap commit); updates block_table, free_slots and free_top in place.

    Returns a dict with anc_mask, out, lse, accept_path, accept_len, bonus_tok, cache_len_out
    and status."""
    for name, t, nd in (("parent", parent, 2), ("draft_tok", draft_tok, 2),
                        ("target_tok", target_tok, 2), ("block_table", block_table, 2),
                        ("cache_len", cache_len, 1), ("tree_slot", tree_slot, 2),
                        ("free_slots", free_slots, 1), ("free_top", free_top, 1)):
        _need(t, name, torch.int32, nd)
    _need(q, "q", None, 4)
    B, T, Hq, D = q.shape
    dt = _dtype_code(q)
    _need(k_pool, "k_pool", q.dtype, 3)
    _need(v_pool, "v_pool", q.dtype, 3)
    num_slots, Hkv = k_pool.shape[0], k_pool.shape[1]
    max_pages = block_table.shape[1]
    W = (T + 63) // 64
    if (tuple(k_pool.shape) != (num_slots, Hkv, D) or tuple(v_pool.shape) != tuple(k_pool.shape)
            or block_table.shape[0] != B or tuple(tree_slot.shape) != (B, T)
            or tuple(cache_len.shape) != (B,) or tuple(parent.shape) != (B, T)
            or tuple(draft_tok.shape) != (B, T) or tuple(target_tok.shape) != (B, T)
            or free_slots.numel() < num_slots or free_top.numel() != 1):
        raise ValueError("inconsistent tree_verify_step_paged shapes")
    dev = q.device
    new = lambda shape, dtype: torch.empty(shape, dtype=dtype, device=dev)  # noqa: E731
    anc_mask = new((B, T, W), torch.int64) if anc_mask is None else anc_mask
    out = torch.empty_like(q) if out is None else out
    if lse is None and with_lse:
        lse = new((B, T, Hq), torch.float32)
    accept_path = new((B, T), torch.int32) if accept_path is None else accept_path
    accept_len = new((B,), torch.int32) if accept_len is None else accept_len
    bonus_tok = new((B,), torch.int32) if bonus_tok is None else bonus_tok
    cache_len_out = torch.empty_like(cache_len) if cache_len_out is None else cache_len_out
    status = new((B,), torch.int32) if status is None else status
    _need(anc_mask, "anc_mask", torch.int64, 3)
    _need(out, "out", q.dtype, 4)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    for name, t in (("accept_len", accept_len), ("bonus_tok", bonus_tok),
                    ("cache_len_out", cache_len_out), ("status", status)):
        _need(t, name, torch.int32, 1)
    _need(accept_path, "accept_path", torch.int32, 2)
    ws_bytes = tree_verify_attn_workspace_size(B, T, Hq, Hkv, D, max_pages * page_size, q.dtype,
                                               split_keys)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("tree_verify_step_paged", load_library().tree_verify_step_paged(
        _ptr(parent), _ptr(draft_tok), _ptr(target_tok), _ptr(q), _ptr(k_pool), _ptr(v_pool),
        num_slots, _ptr(block_table), max_pages, int(page_size), _ptr(cache_len),
        _ptr(cache_len_out), _ptr(tree_slot), _ptr(anc_mask), _ptr(out), _ptr(lse),
        _ptr(accept_path), _ptr(accept_len), _ptr(bonus_tok), _ptr(free_slots), _ptr(free_top),
        _ptr(status), B, T, Hq, Hkv, D, dt, float(scale), int(split_keys), _ptr(workspace),
        ws_have, _stream(stream)))
    return dict(anc_mask=anc_mask, out=out, lse=lse, accept_path=accept_path,
                accept_len=accept_len, bonus_tok=bonus_tok, cache_len_out=cache_len_out,
                status=status)


def eagle2_node_count(depth: int, k: int, branch: int) -> int:
    """Nodes of the table after `depth` expansion levels (host arithmetic of the library)."""
    n = int(load_library().eagle2_node_count(depth, k, branch))
    if n < 0:
        raise ValueError(f"bad expansion shape depth={depth} k={k} branch={branch}")
    return n


def eagle2_new_table(B: int, n_max: int, k: int, device) -> dict:
    """Device buffers of the EAGLE-2 node table of B sequences: node_tok, node_parent,
    node_value [B, n_max], frontier [B, k] and status [B] (zeroed)."""
    return {
        "node_tok": torch.empty((B, n_max), dtype=torch.int32, device=device),
        "node_parent": torch.empty((B, n_max), dtype=torch.int32, device=device),
        "node_value": torch.empty((B, n_max), dtype=torch.float32, device=device),
        "frontier": torch.empty((B, k), dtype=torch.int32, device=device),
        "status": torch.zeros((B,), dtype=torch.int32, device=device),
    }


def eagle2_expand(table: dict, level: int, child_tok, child_conf, root_tok=None, stream=None):
    """Expansion level `level` (1, 2, ...) into `table` (from eagle2_new_table): child_tok
    [B,k,branch] int32 and child_conf [B,k,branch] float32 are the drafter's candidates for the
    frontier slots; root_tok [B] int32 at level 1.  Updates the table and its frontier."""
    _need(child_tok, "child_tok", torch.int32, 3)
    _need(child_conf, "child_conf", torch.float32, 3)
    B, k, branch = child_tok.shape
    if tuple(child_conf.shape) != (B, k, branch):
        raise ValueError("child_tok and child_conf shapes differ")
    for name in ("node_tok", "node_parent", "node_value", "frontier", "status"):
        _need(table[name], name)
    n_max = table["node_tok"].shape[1]
    if (tuple(table["frontier"].shape) != (B, k) or table["node_tok"].shape[0] != B
            or tuple(table["node_parent"].shape) != (B, n_max)
            or tuple(table["node_value"].shape) != (B, n_max)):
        raise ValueError("node table shapes do not match the drafter outputs")
    if root_tok is not None:
        _need(root_tok, "root_tok", torch.int32, 1)
    _check("eagle2_expand", load_library().eagle2_expand(
        _ptr(root_tok), _ptr(child_tok), _ptr(child_conf), B, int(level), k, branch,
        _ptr(table["node_tok"]), _ptr(table["node_parent"]), _ptr(table["node_value"]), n_max,
        _ptr(table["frontier"]), _ptr(table["status"]), _stream(stream)))


def eagle2_rerank(table: dict, n_nodes: int, T: int, out: dict | None = None, stream=None) -> dict:
    """Keep the T best of the table's first n_nodes nodes and flatten them -> dict of parent,
    tok, depth, node [B,T] int32 (the table's status is OR-ed)."""
    for name in ("node_tok", "node_parent", "node_value", "status"):
        _need(table[name], name)
    B, n_max = table["node_tok"].shape
    dev = table["node_tok"].device
    if out is None:
        out = {name: torch.empty((B, T), dtype=torch.int32, device=dev)
               for name in ("parent", "tok", "depth", "node")}
    for name in ("parent", "tok", "depth", "node"):
        _need(out[name], name, torch.int32, 2)
        if tuple(out[name].shape) != (B, T):
            raise ValueError(f"{name} must be [{B}, {T}]")
    _check("eagle2_rerank", load_library().eagle2_rerank(
        _ptr(table["node_tok"]), _ptr(table["node_parent"]), _ptr(table["node_value"]),
        int(n_nodes), n_max, B, int(T), _ptr(out["parent"]), _ptr(out["tok"]), _ptr(out["depth"]),
        _ptr(out["node"]), _ptr(table["status"]), _stream(stream)))
    return out


def _bf16_2d(t: torch.Tensor, name: str) -> None:
    _need(t, name, torch.bfloat16, 2)


def lm_head_project(h, B, u=None, stream=None):
    """u [M, r] float32 = B [r, d] h [M, d] (bfloat16 inputs)."""
    _bf16_2d(h, "h")
    _bf16_2d(B, "B")
    M, d = h.shape
    r = B.shape[0]
    if B.shape[1] != d:
        raise ValueError("h and B disagree on d")
    u = torch.empty((M, r), dtype=torch.float32, device=h.device) if u is None else u
    _need(u, "u", torch.float32, 2)
    _check("lm_head_project", load_library().lm_head_project(_ptr(h), _ptr(B), M, r, d, _ptr(u),
                                                            _stream(stream)))
    return u


def lm_head_screen(A, u, row_token, tile: int, k_tile: int, cand=None, cand_score=None,
                   stream=None):
    """Local top-k screening -> (cand [M, C] int32 tokens, cand_score [M, C] float32)."""
    _bf16_2d(A, "A")
    _need(u, "u", torch.float32, 2)
    _need(row_token, "row_token", torch.int32, 1)
    n, r = A.shape
    M = u.shape[0]
    if u.shape[1] != r or row_token.shape[0] != n:
        raise ValueError("inconsistent lm_head_screen shapes")
    C = -(-n // tile) * k_tile
    dev = A.device
    cand = torch.empty((M, C), dtype=torch.int32, device=dev) if cand is None else cand
    cand_score = (torch.empty((M, C), dtype=torch.float32, device=dev) if cand_score is None
                  else cand_score)
    _check("lm_head_screen", load_library().lm_head_screen(
        _ptr(A), _ptr(u), _ptr(row_token), M, r, n, int(tile), int(k_tile), _ptr(cand),
        _ptr(cand_score), _stream(stream)))
    return cand, cand_score


def lm_head_rescore(W, h, cand, logits=None, status=None, stream=None):
    """Exact candidate logits [M, C] float32 = W[cand] . h."""
    _bf16_2d(W, "W")
    _bf16_2d(h, "h")
    _need(cand, "cand", torch.int32, 2)
    V, d = W.shape
    M, C = cand.shape
    if h.shape != (M, d):
        raise ValueError("inconsistent lm_head_rescore shapes")
    logits = torch.empty((M, C), dtype=torch.float32, device=W.device) if logits is None else logits
    if status is not None:
        _need(status, "status", torch.int32, 1)
    _check("lm_head_rescore", load_library().lm_head_rescore(
        _ptr(W), _ptr(h), _ptr(cand), M, C, d, V, _ptr(logits), _ptr(status), _stream(stream)))
    return logits


def lm_head_topk(logits, cand, K: int, V: int, out_tok=None, out_conf=None, stream=None):
    """The drafter's children -> (tokens [M, K] int32, confidences [M, K] float32)."""
    _need(logits, "logits", torch.float32, 2)
    _need(cand, "cand", torch.int32, 2)
    M, C = cand.shape
    dev = cand.device
    out_tok = torch.empty((M, K), dtype=torch.int32, device=dev) if out_tok is None else out_tok
    out_conf = torch.empty((M, K), dtype=torch.float32, device=dev) if out_conf is None else out_conf
    _check("lm_head_topk", load_library().lm_head_topk(
        _ptr(logits), _ptr(cand), M, C, int(K), int(V), _ptr(out_tok), _ptr(out_conf),
        _stream(stream)))
    return out_tok, out_conf


def lm_head_two_stage(h, A, B, W, row_token, tile: int, k_tile: int, K: int, status=None,
                      stream=None) -> dict:
    """Both stages and the children, in four launches on one stream: dict of u, cand,
    cand_score, logits, tok, conf."""
    u = lm_head_project(h, B, stream=stream)
    cand, score = lm_head_screen(A, u, row_token, tile, k_tile, stream=stream)
    logits = lm_head_rescore(W, h, cand, status=status, stream=stream)
    tok, conf = lm_head_topk(logits, cand, K, W.shape[0], stream=stream)
    return dict(u=u, cand=cand, cand_score=score, logits=logits, tok=tok, conf=conf)
