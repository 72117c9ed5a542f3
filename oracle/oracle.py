"""ctypes wrapper of the plain-C fp64 oracle (``tree_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Builds ``libtree_oracle.so`` with gcc on first use; the functions
take and return numpy arrays.  Nothing here is shared with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

ORC_BAD_TREE = 0x1
ORC_OVERFLOW = 0x2
ORC_BAD_LEN = 0x4
ORC_BAD_PATH = 0x8
ORC_FREE_FULL = 0x100
ORC_BAD_TOKEN = 0x20
ORC_BAD_CONF = 0x80

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tree_oracle.c")
_LIB = os.path.join(_HERE, "libtree_oracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle (plain C, -O2, no fast-math so sums keep their written order)."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-shared", "-fPIC", "-pthread",
                           src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the oracle library, building it if it is missing or older than its source."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    i = ctypes.c_int
    lib.oracle_tree_paths.argtypes = [P, i, P, P]
    lib.oracle_tree_paths.restype = i
    lib.oracle_build_mask.argtypes = [P, i, i, P, P]
    lib.oracle_build_mask.restype = None
    lib.oracle_paged_gather.argtypes = [i, P, P, i, P, i, i, P, P, i, i, i, i, i, P, P, P, P]
    lib.oracle_paged_gather.restype = i
    lib.oracle_commit_paged.argtypes = [P, i, P, P, P, P, P, i, i, i, P, P, P]
    lib.oracle_commit_paged.restype = None
    lib.oracle_attention.argtypes = [i, P, P, P, P, P, P, P, i, i, i, i, i, i, ctypes.c_double,
                                     P, ctypes.c_long, P, P, i]
    lib.oracle_attention.restype = i
    lib.oracle_accept.argtypes = [P, P, P, i, i, P, P, P]
    lib.oracle_accept.restype = None
    lib.oracle_compact.argtypes = [i, P, P, P, P, P, P, P, P, i, i, i, i, i, P]
    lib.oracle_compact.restype = None
    lib.oracle_accept_stochastic.argtypes = [P, P, P, P, P, P, i, i, i, i, P, P, P, P]
    lib.oracle_accept_stochastic.restype = None
    lib.oracle_eagle2_rerank.argtypes = [P, P, P, i, i, i, i, P, P, P, P, P]
    lib.oracle_eagle2_rerank.restype = None
    lib.oracle_eagle2_build.argtypes = [P, P, P, i, i, i, i, i, P, P, P, i, P, P, P, P, P, P]
    lib.oracle_eagle2_build.restype = i
    lib.oracle_lm_project.argtypes = [P, P, i, i, i, P]
    lib.oracle_lm_project.restype = None
    lib.oracle_lm_scores.argtypes = [P, P, i, i, i, P]
    lib.oracle_lm_scores.restype = None
    lib.oracle_lm_screen.argtypes = [P, P, i, i, i, i, P, P]
    lib.oracle_lm_screen.restype = None
    lib.oracle_lm_rescore.argtypes = [P, P, P, i, i, i, i, P, P]
    lib.oracle_lm_rescore.restype = None
    lib.oracle_lm_logits_all.argtypes = [P, P, i, i, i, P, i]
    lib.oracle_lm_logits_all.restype = None
    lib.oracle_lm_topk.argtypes = [P, P, i, i, i, i, P, P]
    lib.oracle_lm_topk.restype = None
    return lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _elem_bits(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 32
    if a.dtype == np.uint16:
        return 16
    raise TypeError(f"oracle takes float32 or bfloat16 bits (uint16), got {a.dtype}")


def tree_paths(parent, lib=None) -> tuple[list[list[int]], int]:
    """Paths root..i of one tree and its status bits."""
    lib = lib or load()
    parent = _i32(parent)
    T = parent.shape[0]
    paths = np.empty((T, T), np.int32)
    plen = np.empty(T, np.int32)
    st = lib.oracle_tree_paths(_p(parent), T, _p(paths), _p(plen))
    return [list(map(int, paths[i, : plen[i]])) for i in range(T)], int(st)


def build_mask(parent, lib=None) -> tuple[np.ndarray, np.ndarray]:
    """anc_mask [B,T,W] uint64 and status [B] int32 for a [B,T] parent array."""
    lib = lib or load()
    parent = _i32(parent)
    B, T = parent.shape
    W = (T + 63) // 64
    anc = np.empty((B, T, W), np.uint64)
    status = np.empty(B, np.int32)
    lib.oracle_build_mask(_p(parent), B, T, _p(anc), _p(status))
    return anc, status


def attention(q, k_cache, v_cache, cache_len, k_tree, v_tree, parent, scale=None, rows=None,
              n_threads=None, lib=None) -> tuple[np.ndarray, np.ndarray]:
    """fp64 tree attention.  ``rows`` is an optional [n,3] array of (b, h, i); then the result
    is [n, D] and [n]; otherwise [B,T,Hq,D] and [B,T,Hq]."""
    lib = lib or load()
    q = np.ascontiguousarray(q)
    bits = _elem_bits(q)
    k_cache, v_cache, k_tree, v_tree = (np.ascontiguousarray(x, dtype=q.dtype)
                                        for x in (k_cache, v_cache, k_tree, v_tree))
    cache_len = _i32(cache_len)
    parent = _i32(parent)
    B, T, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    Lmax = k_cache.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if n_threads is None:
        n_threads = len(os.sched_getaffinity(0))
    if rows is not None:
        rows = _i32(rows).reshape(-1, 3)
        n = rows.shape[0]
        out = np.empty((n, D), np.float64)
        lse = np.empty(n, np.float64)
    else:
        n = B * T * Hq
        out = np.empty((B, T, Hq, D), np.float64)
        lse = np.empty((B, T, Hq), np.float64)
    rc = lib.oracle_attention(bits, _p(q), _p(k_cache), _p(v_cache), _p(cache_len), _p(k_tree),
                              _p(v_tree), _p(parent), B, T, Hq, Hkv, D, Lmax, float(scale),
                              _p(rows), n, _p(out), _p(lse), int(n_threads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return out, lse


def accept(parent, draft, target, lib=None) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """accept_path [B,T] (-1 padded), accept_len [B], bonus_tok [B]."""
    lib = lib or load()
    parent, draft, target = _i32(parent), _i32(draft), _i32(target)
    B, T = parent.shape
    path = np.empty((B, T), np.int32)
    n = np.empty(B, np.int32)
    bonus = np.empty(B, np.int32)
    lib.oracle_accept(_p(parent), _p(draft), _p(target), B, T, _p(path), _p(n), _p(bonus))
    return path, n, bonus


def compact(k_cache, v_cache, cache_len, k_tree, v_tree, accept_path, accept_len, status=None,
            lib=None):
    """In-place compaction of host copies; returns (cache_len_out, status)."""
    lib = lib or load()
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == v_cache.dtype == k_tree.dtype == v_tree.dtype
    B, Hkv, Lmax, D = k_cache.shape
    T = k_tree.shape[1]
    k_tree = np.ascontiguousarray(k_tree)
    v_tree = np.ascontiguousarray(v_tree)
    cache_len = _i32(cache_len)
    accept_path, accept_len = _i32(accept_path), _i32(accept_len)
    out_len = np.empty(B, np.int32)
    st = np.zeros(B, np.int32) if status is None else status
    lib.oracle_compact(k_cache.dtype.itemsize, _p(k_cache), _p(v_cache), _p(cache_len),
                       _p(out_len), _p(k_tree), _p(v_tree), _p(accept_path), _p(accept_len),
                       B, T, Hkv, D, Lmax, _p(st))
    return out_len, st


def paged_gather(k_pool, v_pool, table, page_size, cache_len, tree_slot, Lmax, fill=np.nan,
                 lib=None):
    """Dense copies (k_cache, v_cache [B,Hkv,Lmax,D], k_tree, v_tree [B,T,Hkv,D]) of the rows a
    paged cache names; cache rows past each prefix hold ``fill`` (bf16 pools: the NaN pattern)."""
    lib = lib or load()
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool, dtype=k_pool.dtype)
    table, cache_len, tree_slot = _i32(table), _i32(cache_len), _i32(tree_slot)
    num_slots, Hkv, D = k_pool.shape
    B, max_pages = table.shape
    T = tree_slot.shape[1]
    if k_pool.dtype == np.uint16:
        nan = np.uint16(0x7FC0)
        k_cache = np.full((B, Hkv, Lmax, D), nan, np.uint16)
    else:
        k_cache = np.full((B, Hkv, Lmax, D), fill, k_pool.dtype)
    v_cache = k_cache.copy()
    k_tree = np.empty((B, T, Hkv, D), k_pool.dtype)
    v_tree = np.empty_like(k_tree)
    rc = lib.oracle_paged_gather(k_pool.dtype.itemsize, _p(k_pool), _p(v_pool), num_slots,
                                 _p(table), max_pages, int(page_size), _p(cache_len),
                                 _p(tree_slot), B, T, Hkv, D, int(Lmax), _p(k_cache), _p(v_cache),
                                 _p(k_tree), _p(v_tree))
    if rc != 0:
        raise ValueError("a table entry or tree slot names a slot outside the pool")
    return k_cache, v_cache, k_tree, v_tree


def paged_attention(q, k_pool, v_pool, table, page_size, cache_len, tree_slot, parent,
                    scale=None, rows=None, n_threads=None, lib=None):
    """Tree attention over a paged cache: attention over the rows the table names."""
    cache_len = _i32(cache_len)
    Lmax = max(1, int(cache_len.max(initial=0)))
    kc, vc, kt, vt = paged_gather(k_pool, v_pool, table, page_size, cache_len, tree_slot, Lmax,
                                  lib=lib)
    return attention(q, kc, vc, cache_len, kt, vt, parent, scale=scale, rows=rows,
                     n_threads=n_threads, lib=lib)


def commit_paged(table, cache_len, tree_slot, accept_path, accept_len, num_slots, free_slots,
                 free_top, status=None, lib=None):
    """Pointer-swap commit on host copies (pages of one token): updates ``table``,
    ``free_slots`` and returns (cache_len_out, free_top, status)."""
    lib = lib or load()
    assert table.dtype == np.int32 and table.flags.c_contiguous
    assert free_slots.dtype == np.int32 and free_slots.flags.c_contiguous
    B, max_pages = table.shape
    tree_slot, cache_len = _i32(tree_slot), _i32(cache_len)
    accept_path, accept_len = _i32(accept_path), _i32(accept_len)
    T = tree_slot.shape[1]
    out_len = np.empty(B, np.int32)
    top = np.array([free_top], np.int32)
    st = np.zeros(B, np.int32) if status is None else status
    lib.oracle_commit_paged(_p(table), max_pages, _p(cache_len), _p(out_len), _p(tree_slot),
                            _p(accept_path), _p(accept_len), B, T, int(num_slots),
                            _p(free_slots), _p(top), _p(st))
    return out_len, int(top[0]), st


def accept_stochastic(parent, draft, p, q, u_acc, u_res, without_replacement=False, lib=None):
    """Rejection sampling over the draft tree (``oracle_accept_stochastic``): p and q are
    [B, T, V] float32 target and draft distributions, u_acc and u_res [B, T] float64 uniforms.
    Returns (accept_path [B,T], accept_len [B], bonus_tok [B], status [B])."""
    lib = lib or load()
    parent, draft = _i32(parent), _i32(draft)
    B, T = parent.shape
    p = np.ascontiguousarray(p, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    V = p.shape[-1]
    assert p.shape == (B, T, V) and q.shape == (B, T, V)
    u_acc = np.ascontiguousarray(u_acc, dtype=np.float64).reshape(B, T)
    u_res = np.ascontiguousarray(u_res, dtype=np.float64).reshape(B, T)
    path = np.empty((B, T), np.int32)
    alen = np.empty(B, np.int32)
    bonus = np.empty(B, np.int32)
    status = np.zeros(B, np.int32)
    lib.oracle_accept_stochastic(_p(parent), _p(draft), _p(p), _p(q), _p(u_acc), _p(u_res), B, T,
                                 V, int(bool(without_replacement)), _p(path), _p(alen), _p(bonus),
                                 _p(status))
    return path, alen, bonus, status


def eagle2_node_count(depth: int, k: int, branch: int) -> int:
    """Nodes of an EAGLE-2 expansion: the root, then branch children for each frontier node of
    every level, the frontier of level l being min(k, children of level l)."""
    n, F = 1, 1
    for _ in range(depth):
        n += F * branch
        F = min(k, F * branch)
    return n


def eagle2_build(root_tok, child_tok, child_conf, T, lib=None) -> dict:
    """EAGLE-2 tree construction (``oracle_eagle2_build``).  root_tok [B] int32; child_tok and
    child_conf [depth, B, k, branch] (int32, float32).  Returns a dict of numpy arrays:
    node_tok, node_parent, node_value [B, N]; frontier [depth, B, k]; parent, tok, depth,
    node [B, T]; status [B]."""
    lib = lib or load()
    root_tok = _i32(root_tok)
    child_tok = _i32(child_tok)
    child_conf = np.ascontiguousarray(child_conf, dtype=np.float32)
    depth, B, k, branch = child_tok.shape
    assert child_conf.shape == child_tok.shape and root_tok.shape == (B,)
    N = eagle2_node_count(depth, k, branch)
    if not 1 <= T <= N:
        raise ValueError(f"tree budget {T} outside [1, {N}]")
    r = {name: np.empty((B, N), dt) for name, dt in
         (("node_tok", np.int32), ("node_parent", np.int32), ("node_value", np.float32))}
    r["frontier"] = np.empty((depth, B, k), np.int32)
    for name in ("parent", "tok", "depth", "node"):
        r[name] = np.empty((B, T), np.int32)
    r["status"] = np.zeros(B, np.int32)
    n = lib.oracle_eagle2_build(_p(root_tok), _p(child_tok), _p(child_conf), B, depth, k, branch,
                                T, _p(r["node_tok"]), _p(r["node_parent"]), _p(r["node_value"]), N,
                                _p(r["frontier"]), _p(r["parent"]), _p(r["tok"]), _p(r["depth"]),
                                _p(r["node"]), _p(r["status"]))
    if n != N:
        raise AssertionError(f"oracle built {n} nodes, expected {N}")
    return r


def eagle2_rerank(node_tok, node_parent, node_value, T, lib=None) -> dict:
    """Reranking and flattening of given node tables [B, N] (``oracle_eagle2_rerank``).
    Returns parent, tok, depth, node [B, T] and status [B]."""
    lib = lib or load()
    node_tok, node_parent = _i32(node_tok), _i32(node_parent)
    node_value = np.ascontiguousarray(node_value, dtype=np.float32)
    B, N = node_tok.shape
    if not 1 <= T <= N:
        raise ValueError(f"tree budget {T} outside [1, {N}]")
    r = {name: np.empty((B, T), np.int32) for name in ("parent", "tok", "depth", "node")}
    r["status"] = np.zeros(B, np.int32)
    lib.oracle_eagle2_rerank(_p(node_tok), _p(node_parent), _p(node_value), N, N, B, T,
                             _p(r["parent"]), _p(r["tok"]), _p(r["depth"]), _p(r["node"]),
                             _p(r["status"]))
    return r


def _bf16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bfloat16 bit patterns (uint16), got {a.dtype}")
    return a


def lm_project(h, Bm, lib=None) -> np.ndarray:
    """u [M, r] float64 = B h (exact products, fp64 sum).  h [M, d] and B [r, d] are bfloat16
    bit patterns."""
    lib = lib or load()
    h, Bm = _bf16(h), _bf16(Bm)
    M, d = h.shape
    r = Bm.shape[0]
    assert Bm.shape[1] == d
    u = np.empty((M, r), np.float64)
    lib.oracle_lm_project(_p(h), _p(Bm), M, r, d, _p(u))
    return u


def lm_scores(A, u, lib=None) -> np.ndarray:
    """Approximate score of every stored row of A for every hidden state: [M, n] float64."""
    lib = lib or load()
    A = _bf16(A)
    u = np.ascontiguousarray(u, dtype=np.float64)
    n, r = A.shape
    M = u.shape[0]
    assert u.shape[1] == r
    s = np.empty((M, n), np.float64)
    lib.oracle_lm_scores(_p(A), _p(u), M, r, n, _p(s))
    return s


def lm_screen(A, u, row_token, tile, k_tile, lib=None) -> tuple[np.ndarray, np.ndarray]:
    """Local top-k screening: (cand [M, n_tiles*k_tile] int32 tokens, cand_score float64)."""
    lib = lib or load()
    s = lm_scores(A, u, lib=lib)
    row_token = _i32(row_token)
    M, n = s.shape
    assert row_token.shape == (n,)
    C = (n + tile - 1) // tile * k_tile
    cand = np.empty((M, C), np.int32)
    score = np.empty((M, C), np.float64)
    lib.oracle_lm_screen(_p(s), _p(row_token), M, n, int(tile), int(k_tile), _p(cand),
                         _p(score))
    return cand, score


def lm_rescore(W, h, cand, lib=None) -> tuple[np.ndarray, np.ndarray]:
    """Exact candidate logits [M, C] float64 (W's rows dotted with h) and status [M]."""
    lib = lib or load()
    W, h = _bf16(W), _bf16(h)
    cand = _i32(cand)
    V, d = W.shape
    M, C = cand.shape
    logits = np.empty((M, C), np.float64)
    status = np.zeros(M, np.int32)
    lib.oracle_lm_rescore(_p(W), _p(h), _p(cand), M, C, d, V, _p(logits), _p(status))
    return logits, status


def lm_logits_all(W, h, n_threads=None, lib=None) -> np.ndarray:
    """Exact logit of every vocabulary token for every hidden state: [M, V] float64."""
    lib = lib or load()
    W, h = _bf16(W), _bf16(h)
    V, d = W.shape
    M = h.shape[0]
    assert h.shape[1] == d
    if n_threads is None:
        n_threads = len(os.sched_getaffinity(0))
    logits = np.empty((M, V), np.float64)
    lib.oracle_lm_logits_all(_p(W), _p(h), M, d, V, _p(logits), int(n_threads))
    return logits


def lm_topk(logits, cand, K, V, lib=None) -> tuple[np.ndarray, np.ndarray]:
    """The K best valid candidates per hidden state (tokens [M, K] int32) and their softmax
    confidences over the candidates ([M, K] float64)."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    cand = _i32(cand)
    M, C = cand.shape
    tok = np.empty((M, K), np.int32)
    conf = np.empty((M, K), np.float64)
    lib.oracle_lm_topk(_p(logits), _p(cand), M, C, int(K), int(V), _p(tok), _p(conf))
    return tok, conf


def lm_head_two_stage(h, A, Bm, W, row_token, tile, k_tile, K, lib=None) -> dict:
    """Both stages and the children: dict of u, cand, cand_score, logits, status, tok, conf."""
    u = lm_project(h, Bm, lib=lib)
    cand, score = lm_screen(A, u, row_token, tile, k_tile, lib=lib)
    logits, status = lm_rescore(W, h, cand, lib=lib)
    tok, conf = lm_topk(logits, cand, K, W.shape[0], lib=lib)
    return dict(u=u, cand=cand, cand_score=score, logits=logits, status=status, tok=tok, conf=conf)
