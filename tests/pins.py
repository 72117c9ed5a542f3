"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes a loaded oracle library and raises ``AssertionError`` when the
oracle disagrees with something the pages or the mathematics fix:

* the worked tree and its printed mask row (tests/golden/worked_tree.txt);
* an independent closure formulation of "self plus ancestors" (boolean reachability through
  repeated parent steps) on every tree of up to 6 nodes and on random trees of up to 128;
* closed forms of attention (K = 0 with one-hot V rows; scale 0 gives the mean of the visible
  rows), textbook causal attention from ``torch.nn.functional.scaled_dot_product_attention`` on
  chain trees and single-node trees, and an explicit dense-mask softmax on random trees;
* hand-derived acceptance cases (tests/golden/accept_hand_cases.txt), the chain extremes and a
  brute-force enumeration of root-to-node paths;
* compaction against direct row selection, including tree rows that live inside the cache;
* paged gather and the pointer-swap commit against the pinned dense attention and copy;
* stochastic acceptance: hand-derived cases (tests/golden/stochastic_hand_cases.txt and a
  duplicate-sibling case), the page's losslessness claim checked exactly by enumerating every
  draft and integrating the uniforms out (one and two levels, both sibling modes), the reduction
  to the greedy rule for one-hot targets, and to a plain inverse-CDF draw (numpy.searchsorted)
  when q = p.

``test_oracle_pins.py`` runs every pin against the oracle; ``test_oracle_mutants.py`` runs them
against deliberately broken copies of the oracle source to show that each plausible mistake is
caught by at least one pin.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np

from oracle import oracle as O
from synth import bf16_bits_to_f32, f32_to_bf16_bits, random_parent, worked_tree_parent

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------------------------
# helpers (independent formulations)
# ----------------------------------------------------------------------------------------------
def closure_mask(parent: np.ndarray) -> np.ndarray:
    """Dense bool [T,T]: reach[i, j] iff j == i or j is reached from i by parent steps.
    Computed as the fixed point of R <- R | (R @ A) with A[i, parent(i)] = 1."""
    T = len(parent)
    A = np.zeros((T, T), dtype=np.int64)
    for i in range(T):
        if parent[i] >= 0:
            A[i, parent[i]] = 1
    R = np.eye(T, dtype=np.int64)
    while True:
        Rn = ((R + R @ A) > 0).astype(np.int64)
        if (Rn == R).all():
            return R.astype(bool)
        R = Rn


def bits_to_dense(anc_row: np.ndarray, T: int) -> np.ndarray:
    out = np.zeros(T, bool)
    for j in range(T):
        out[j] = (int(anc_row[j // 64]) >> (j % 64)) & 1
    return out


def read_worked_tree():
    rows = []
    tokens = None
    with open(os.path.join(GOLDEN, "worked_tree.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("tokens"):
                tokens = line.split()[1:]
                continue
            idx, tok, par, vis, src = line.split()
            rows.append((int(idx), tok, int(par), vis.split(","), src))
    return tokens, rows


def read_accept_cases():
    cases = []
    with open(os.path.join(GOLDEN, "accept_hand_cases.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rest = line.split(":", 1)
            draft, target, path, bonus = (x.strip() for x in rest.split("|"))
            cases.append((name, draft.split(), target.split(), [int(x) for x in path.split(",")],
                          bonus))
    return cases


def dense_tree_attention(q, k_cache, v_cache, cache_len, k_tree, v_tree, parent, scale):
    """Explicit masked softmax over [prefix ++ all T tree rows] with the closure mask; KV heads
    repeated G times (numpy, float64)."""
    q, k_cache, v_cache, k_tree, v_tree = (np.asarray(x, np.float64)
                                           for x in (q, k_cache, v_cache, k_tree, v_tree))
    B, T, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, T, Hq, D))
    lse = np.zeros((B, T, Hq))
    for b in range(B):
        L = int(cache_len[b])
        keys = np.concatenate([k_cache[b, :, :L, :], k_tree[b].transpose(1, 0, 2)], axis=1)
        vals = np.concatenate([v_cache[b, :, :L, :], v_tree[b].transpose(1, 0, 2)], axis=1)
        keys = np.repeat(keys, G, axis=0)  # [Hq, L+T, D]
        vals = np.repeat(vals, G, axis=0)
        vis = np.concatenate([np.ones((T, L), bool), closure_mask(parent[b])], axis=1)  # [T, L+T]
        s = np.einsum("thd,hkd->thk", q[b], keys) * scale
        s = np.where(vis[:, None, :], s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        w = np.exp(s - m)
        den = w.sum(axis=-1, keepdims=True)
        out[b] = np.einsum("thk,hkd->thd", w, vals) / den
        lse[b] = (m + np.log(den))[..., 0]
    return out, lse


def _rand(rng, shape, dtype):
    x = rng.standard_normal(size=shape).astype(np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def _as_f64(x, dtype):
    if dtype == "f32":
        return x.astype(np.float64)
    return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def small_case(rng, B=2, T=7, Hq=4, Hkv=2, D=16, Ls=(5, 9), dtype="f32", kind="random"):
    parent = np.stack([random_parent(rng, T, kind) for _ in range(B)])
    cache_len = np.array([Ls[b % len(Ls)] for b in range(B)], np.int32)
    Lmax = int(cache_len.max()) + T + 3
    nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
    store = np.float32 if dtype == "f32" else np.uint16
    k_cache = np.full((B, Hkv, Lmax, D), nan, store)
    v_cache = np.full((B, Hkv, Lmax, D), nan, store)
    for b in range(B):
        L = int(cache_len[b])
        k_cache[b, :, :L] = _rand(rng, (Hkv, L, D), dtype)
        v_cache[b, :, :L] = _rand(rng, (Hkv, L, D), dtype)
    q = _rand(rng, (B, T, Hq, D), dtype)
    k_tree = _rand(rng, (B, T, Hkv, D), dtype)
    v_tree = _rand(rng, (B, T, Hkv, D), dtype)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, cache_len=cache_len, k_tree=k_tree,
                v_tree=v_tree, parent=parent)


# ----------------------------------------------------------------------------------------------
# mask pins
# ----------------------------------------------------------------------------------------------
def pin_worked_tree_mask(lib):
    tokens, rows = read_worked_tree()
    parent = np.array([r[2] for r in rows], np.int32)
    assert (parent == worked_tree_parent()).all()
    anc, st = O.build_mask(parent[None], lib=lib)
    assert st[0] == 0
    for idx, tok, _par, vis, src in rows:
        got = [tokens[j] for j in range(len(tokens)) if bits_to_dense(anc[0, idx], 8)[j]]
        assert got == vis, (tok, got, vis, src)
    # the printed row: "good" sees exactly It, is, a, good -> bits 0, 1, 3, 6
    assert int(anc[0, 6, 0]) == 0b01001011


def pin_mask_closure_bruteforce(lib):
    for T in range(1, 7):
        for choice in itertools.product(*[range(i) for i in range(1, T)]):
            parent = np.array([-1, *choice], np.int32)
            anc, st = O.build_mask(parent[None], lib=lib)
            assert st[0] == 0
            R = closure_mask(parent)
            for i in range(T):
                assert (bits_to_dense(anc[0, i], T) == R[i]).all(), (parent, i)


def pin_mask_closure_random(lib):
    rng = np.random.default_rng(11)
    for T in (1, 2, 63, 64, 65, 100, 127, 128):
        for kind in ("random", "chain", "star", "deep"):
            parent = random_parent(rng, T, kind)
            anc, st = O.build_mask(parent[None], lib=lib)
            assert st[0] == 0
            assert anc.shape == (1, T, (T + 63) // 64)
            R = closure_mask(parent)
            for i in range(T):
                assert (bits_to_dense(anc[0, i], T) == R[i]).all(), (kind, T, i)
            # no bit at or beyond T
            for i in range(T):
                for w in range(anc.shape[2]):
                    hi = T - 64 * w
                    if hi < 64:
                        assert int(anc[0, i, w]) >> max(hi, 0) == 0


def pin_mask_invalid_trees(lib):
    bad = [[0, 0, 1], [-1, 1, 0], [-1, 0, 3], [-1, -1, 0], [-1, 0, 2]]
    for p in bad:
        parent = np.array(p, np.int32)
        anc, st = O.build_mask(parent[None], lib=lib)
        assert st[0] == O.ORC_BAD_TREE, p
        for i in range(len(p)):
            assert int(anc[0, i, 0]) == 1 << i, p


# ----------------------------------------------------------------------------------------------
# attention pins
# ----------------------------------------------------------------------------------------------
def pin_visibility_probe(lib):
    """K = 0, V rows one-hot: every visible key gets weight 1 / (#visible); the worked tree's
    "good" row (prefix 16) is 1/20 on columns 0..15 and 16 + {0, 1, 3, 6}."""
    parent = worked_tree_parent()
    T, L, D, Hq, Hkv = 8, 16, 64, 2, 1
    Lmax = L + T
    k_cache = np.zeros((1, Hkv, Lmax, D), np.float32)
    v_cache = np.zeros((1, Hkv, Lmax, D), np.float32)
    k_cache[0, 0, L:] = np.nan  # rows past the prefix must never be read
    v_cache[0, 0, L:] = np.nan
    for j in range(L):
        v_cache[0, 0, j, j] = 1.0
    k_tree = np.zeros((1, T, Hkv, D), np.float32)
    v_tree = np.zeros((1, T, Hkv, D), np.float32)
    for t in range(T):
        v_tree[0, t, 0, L + t] = 1.0
    q = np.random.default_rng(3).standard_normal((1, T, Hq, D)).astype(np.float32)
    out, lse = O.attention(q, k_cache, v_cache, np.array([L], np.int32), k_tree, v_tree,
                           parent[None], lib=lib)
    R = closure_mask(parent)
    for i in range(T):
        n_vis = L + int(R[i].sum())
        want = np.zeros(D)
        want[:L] = 1.0 / n_vis
        want[L + np.nonzero(R[i])[0]] = 1.0 / n_vis
        for h in range(Hq):
            assert np.abs(out[0, i, h] - want).max() < 1e-15, (i, h)
            assert abs(lse[0, i, h] - np.log(n_vis)) < 1e-14
    good = out[0, 6, 0]
    assert np.allclose(good[[0, 15, 16, 17, 19, 22]], 1 / 20) and good[[18, 20, 21, 23]].max() == 0


def pin_scale_zero_is_mean(lib):
    rng = np.random.default_rng(5)
    c = small_case(rng, B=2, T=6, Hq=4, Hkv=2, D=8)
    out, lse = O.attention(**c, scale=0.0, lib=lib)
    R = [closure_mask(c["parent"][b]) for b in range(2)]
    for b in range(2):
        L = int(c["cache_len"][b])
        for i in range(6):
            for h in range(4):
                kvh = h // 2
                rows = [c["v_cache"][b, kvh, j] for j in range(L)]
                rows += [c["v_tree"][b, j, kvh] for j in np.nonzero(R[b][i])[0]]
                want = np.mean(np.array(rows, np.float64), axis=0)
                assert np.abs(out[b, i, h] - want).max() < 1e-12
                assert abs(lse[b, i, h] - np.log(len(rows))) < 1e-12


def _sdpa_chain(q, k_cache, v_cache, L, k_tree, v_tree, scale):
    """Chain tree (node t's path is 0..t) as textbook causal attention of the last T positions
    of prefix ++ chain, via torch's CPU scaled_dot_product_attention with an explicit mask."""
    import torch

    T, Hq, D = q.shape
    Hkv = k_tree.shape[1]
    G = Hq // Hkv
    K = np.concatenate([k_cache[:, :L, :], k_tree.transpose(1, 0, 2)], axis=1)  # [Hkv, L+T, D]
    V = np.concatenate([v_cache[:, :L, :], v_tree.transpose(1, 0, 2)], axis=1)
    Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)
    Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
    Qt = torch.from_numpy(q.transpose(1, 0, 2).copy())  # [Hq, T, D]
    # query t sits at absolute position L + t and sees keys 0 .. L + t
    allowed = torch.arange(L + T)[None, :] <= (L + torch.arange(T))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=allowed,
                                                         scale=scale)
    s = (Qt @ Kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~allowed, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy().transpose(1, 0, 2), lse.numpy().T


def pin_chain_matches_causal_sdpa(lib):
    rng = np.random.default_rng(7)
    for dtype in ("f32", "bf16"):
        for (L, T, Hq, Hkv, D) in [(16, 8, 2, 1, 64), (33, 5, 4, 2, 32), (0, 4, 3, 3, 8)]:
            c = small_case(rng, B=1, T=T, Hq=Hq, Hkv=Hkv, D=D, Ls=(L,), dtype=dtype, kind="chain")
            out, lse = O.attention(**c, lib=lib)
            f = lambda x: _as_f64(x, dtype)  # noqa: E731
            want, want_lse = _sdpa_chain(f(c["q"][0]), f(c["k_cache"][0]), f(c["v_cache"][0]), L,
                                         f(c["k_tree"][0]), f(c["v_tree"][0]), 1 / np.sqrt(D))
            assert np.abs(out[0] - want).max() < 1e-12, (dtype, L, T)
            assert np.abs(lse[0] - want_lse).max() < 1e-12


def pin_single_node_is_decode(lib):
    """T = 1: ordinary decode attention of one query over prefix ++ itself."""
    import torch

    rng = np.random.default_rng(9)
    for L in (0, 1, 50):
        c = small_case(rng, B=1, T=1, Hq=4, Hkv=1, D=16, Ls=(L,))
        out, lse = O.attention(**c, lib=lib)
        K = np.concatenate([c["k_cache"][0, 0, :L], c["k_tree"][0, :, 0]], axis=0).astype(np.float64)
        V = np.concatenate([c["v_cache"][0, 0, :L], c["v_tree"][0, :, 0]], axis=0).astype(np.float64)
        Q = c["q"][0, 0].astype(np.float64)  # [Hq, D]
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[:, None, :], torch.from_numpy(K)[None].expand(4, -1, -1),
            torch.from_numpy(V)[None].expand(4, -1, -1), scale=0.25)
        assert np.abs(out[0, 0] - o.numpy()[:, 0, :]).max() < 1e-12


def pin_dense_mask_bruteforce(lib):
    rng = np.random.default_rng(13)
    for kind in ("random", "star", "deep"):
        for dtype in ("f32", "bf16"):
            c = small_case(rng, B=3, T=9, Hq=6, Hkv=2, D=12, Ls=(0, 4, 11), dtype=dtype, kind=kind)
            out, lse = O.attention(**c, lib=lib)
            f = {k: (_as_f64(v, dtype) if k in ("q", "k_cache", "v_cache", "k_tree", "v_tree")
                     else v) for k, v in c.items()}
            want, want_lse = dense_tree_attention(**f, scale=1 / np.sqrt(12))
            assert np.abs(out - want).max() < 1e-12, (kind, dtype)
            assert np.abs(lse - want_lse).max() < 1e-12


def pin_per_path_invariant(lib):
    """A tree pass equals verifying each root-to-node path on its own."""
    rng = np.random.default_rng(17)
    c = small_case(rng, B=1, T=10, Hq=4, Hkv=2, D=16, Ls=(12,), kind="random")
    out, lse = O.attention(**c, lib=lib)
    paths, st = O.tree_paths(c["parent"][0], lib=lib)
    assert st == 0
    for i in range(10):
        p = paths[i]
        n = len(p)
        sub = dict(q=c["q"][:, p], k_cache=c["k_cache"], v_cache=c["v_cache"],
                   cache_len=c["cache_len"], k_tree=c["k_tree"][:, p], v_tree=c["v_tree"][:, p],
                   parent=np.arange(-1, n - 1, dtype=np.int32)[None])
        o2, l2 = O.attention(**sub, lib=lib)
        assert np.abs(o2[0, n - 1] - out[0, i]).max() < 1e-13
        assert np.abs(l2[0, n - 1] - lse[0, i]).max() < 1e-13


def pin_selected_rows_match_full(lib):
    rng = np.random.default_rng(19)
    c = small_case(rng, B=2, T=5, Hq=4, Hkv=2, D=8, Ls=(3, 7))
    out, lse = O.attention(**c, lib=lib)
    rows = np.array([[1, 3, 4], [0, 0, 0], [1, 1, 2]], np.int32)
    o2, l2 = O.attention(**c, rows=rows, lib=lib)
    for r, (b, h, i) in enumerate(rows):
        assert (o2[r] == out[b, i, h]).all() and l2[r] == lse[b, i, h]


# ----------------------------------------------------------------------------------------------
# acceptance pins
# ----------------------------------------------------------------------------------------------
def pin_accept_hand_cases(lib):
    parent = worked_tree_parent()
    for name, draft, target, want_path, want_bonus in read_accept_cases():
        names = sorted(set(draft) | set(target))
        ids = {n: k for k, n in enumerate(names)}
        d = np.array([[ids[x] for x in draft]], np.int32)
        t = np.array([[ids[x] for x in target]], np.int32)
        path, n, bonus = O.accept(parent[None], d, t, lib=lib)
        assert list(path[0, : n[0]]) == want_path, name
        assert (path[0, n[0]:] == -1).all(), name
        assert bonus[0] == ids[want_bonus], name


def pin_accept_chain_extremes(lib):
    T = 9
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    draft = np.arange(100, 100 + T, dtype=np.int32)[None]
    target = np.roll(draft, -1, axis=1)
    target[0, -1] = 7
    path, n, bonus = O.accept(parent, draft, target, lib=lib)
    assert n[0] == T and list(path[0]) == list(range(T)) and bonus[0] == 7
    path, n, bonus = O.accept(parent, draft, np.full_like(draft, 5), lib=lib)
    assert n[0] == 1 and path[0, 0] == 0 and (path[0, 1:] == -1).all() and bonus[0] == 5


def _brute_accept(parent, draft, target):
    T = len(parent)
    kids = [[] for _ in range(T)]
    for i in range(1, T):
        kids[parent[i]].append(i)
    best = [0]

    def dfs(path):
        nonlocal best
        if len(path) > len(best) or (len(path) == len(best) and path[-1] < best[-1]):
            best = list(path)
        for c in kids[path[-1]]:
            if draft[c] == target[path[-1]]:
                dfs(path + [c])

    dfs([0])
    return best, int(target[best[-1]])


def pin_accept_bruteforce(lib):
    rng = np.random.default_rng(23)
    for trial in range(300):
        T = int(rng.integers(1, 14))
        parent = random_parent(rng, T, ["random", "star", "chain", "deep"][trial % 4])
        vocab = int(rng.integers(1, 4))
        draft = rng.integers(0, vocab, T).astype(np.int32)
        target = rng.integers(0, vocab, T).astype(np.int32)
        path, n, bonus = O.accept(parent[None], draft[None], target[None], lib=lib)
        want, wb = _brute_accept(parent, draft, target)
        assert list(path[0, : n[0]]) == want, (parent, draft, target)
        assert bonus[0] == wb


# ----------------------------------------------------------------------------------------------
# compaction pins
# ----------------------------------------------------------------------------------------------
def pin_compact_hand_case(lib):
    """Prefix 16, accepted path [0, 1, 3, 6]: cache rows 16..19 <- tree rows 0, 1, 3, 6."""
    D, T, L, Lmax = 4, 8, 16, 32
    k_cache = np.full((1, 1, Lmax, D), -1.0, np.float32)
    v_cache = np.full((1, 1, Lmax, D), -2.0, np.float32)
    k_tree = np.arange(T * D, dtype=np.float32).reshape(1, T, 1, D)
    v_tree = -k_tree
    path = np.array([[0, 1, 3, 6, -1, -1, -1, -1]], np.int32)
    out_len, st = O.compact(k_cache, v_cache, np.array([L], np.int32), k_tree, v_tree, path,
                            np.array([4], np.int32), lib=lib)
    assert out_len[0] == 20 and st[0] == 0
    for r, j in zip(range(16, 20), [0, 1, 3, 6]):
        assert (k_cache[0, 0, r] == k_tree[0, j, 0]).all() and (v_cache[0, 0, r] == v_tree[0, j, 0]).all()
    assert (k_cache[0, 0, :16] == -1).all() and (k_cache[0, 0, 20:] == -1).all()
    assert (v_cache[0, 0, 20:] == -2).all()


def pin_compact_alias(lib):
    """Tree rows stored in the cache itself at rows 16..23: the same result as from a copy."""
    D, T, L, Lmax = 4, 8, 16, 32
    base = np.random.default_rng(29).standard_normal((1, 1, Lmax, D)).astype(np.float32)
    k_cache = base.copy()
    v_cache = -base.copy()
    k_tree_copy = k_cache[0, 0, L:L + T].reshape(1, T, 1, D).copy()
    v_tree_copy = v_cache[0, 0, L:L + T].reshape(1, T, 1, D).copy()
    k_view = k_cache[0, 0, L:L + T].reshape(1, T, 1, D)
    v_view = v_cache[0, 0, L:L + T].reshape(1, T, 1, D)
    assert np.shares_memory(k_view, k_cache)
    path = np.array([[0, 1, 3, 6, -1, -1, -1, -1]], np.int32)
    out_len, st = O.compact(k_cache, v_cache, np.array([L], np.int32), k_view, v_view, path,
                            np.array([4], np.int32), lib=lib)
    assert out_len[0] == 20
    for r, j in enumerate([0, 1, 3, 6]):
        assert (k_cache[0, 0, L + r] == k_tree_copy[0, j, 0]).all()
        assert (v_cache[0, 0, L + r] == v_tree_copy[0, j, 0]).all()
    assert (k_cache[0, 0, :L] == base[0, 0, :L]).all()
    assert (k_cache[0, 0, L + 4:] == base[0, 0, L + 4:]).all()


def pin_compact_random(lib):
    rng = np.random.default_rng(31)
    B, T, Hkv, D = 5, 9, 3, 8
    cache_len = np.array([0, 3, 10, 20, 17], np.int32)
    Lmax = 26
    k_cache = rng.standard_normal((B, Hkv, Lmax, D)).astype(np.float32)
    v_cache = rng.standard_normal((B, Hkv, Lmax, D)).astype(np.float32)
    k_tree = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
    v_tree = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
    paths = np.full((B, T), -1, np.int32)
    lens = np.array([9, 2, 1, 7, 5], np.int32)  # sequence 3: 20 + 7 > 26 overflows
    for b in range(B):
        chosen = np.sort(rng.choice(T, size=lens[b], replace=False))
        chosen[0] = 0
        paths[b, : lens[b]] = np.sort(chosen)
    k0, v0 = k_cache.copy(), v_cache.copy()
    out_len, st = O.compact(k_cache, v_cache, cache_len, k_tree, v_tree, paths, lens, lib=lib)
    for b in range(B):
        L, n = int(cache_len[b]), int(lens[b])
        if L + n > Lmax:
            assert st[b] == O.ORC_OVERFLOW and out_len[b] == L
            assert (k_cache[b] == k0[b]).all() and (v_cache[b] == v0[b]).all()
            continue
        assert st[b] == 0 and out_len[b] == L + n
        want_k, want_v = k0[b].copy(), v0[b].copy()
        want_k[:, L:L + n] = k_tree[b, paths[b, :n]].transpose(1, 0, 2)
        want_v[:, L:L + n] = v_tree[b, paths[b, :n]].transpose(1, 0, 2)
        assert (k_cache[b] == want_k).all() and (v_cache[b] == want_v).all()
    # malformed lengths and path entries commit nothing
    k1 = k_cache.copy()
    st = np.zeros(B, np.int32)
    bad_len = np.array([-1, 3, 10, 20, 99], np.int32)
    bad_paths = paths.copy()
    bad_paths[1, 0] = T
    out_len, st = O.compact(k_cache, v_cache, bad_len, k_tree, v_tree, bad_paths,
                            np.array([1, 2, T + 1, 0, 1], np.int32), st, lib=lib)
    assert list(st) == [O.ORC_BAD_LEN, O.ORC_BAD_PATH, O.ORC_BAD_PATH, 0, O.ORC_BAD_LEN]
    assert (k_cache[[0, 1, 2, 4]] == k1[[0, 1, 2, 4]]).all()
    assert out_len[3] == 20


# ---- paged KV ("EAGLE-2 vs. Medusa" section 8) --------------------------------------------------
def _paged_from_dense(rng, k_cache, v_cache, cache_len, P, shuffle):
    """Pool + table holding the dense cache's rows 0..L_b-1 (pages of P tokens), built by plain
    numpy indexing; pages are placed in shuffled physical order when ``shuffle``."""
    B, Hkv, Lmax, D = k_cache.shape
    n_pages = [(-(-int(L) // P)) for L in cache_len]
    total = sum(n_pages)
    phys = rng.permutation(total) if shuffle else np.arange(total)
    max_pages = max(1, max(n_pages))
    table = np.full((B, max_pages), -1, np.int32)
    k_pool = np.zeros((total * P + 3, Hkv, D), k_cache.dtype)
    v_pool = np.zeros_like(k_pool)
    nxt = 0
    for b in range(B):
        for j in range(n_pages[b]):
            pg = int(phys[nxt])
            nxt += 1
            table[b, j] = pg
            for o in range(P):
                pos = j * P + o
                if pos < cache_len[b]:
                    k_pool[pg * P + o] = k_cache[b, :, pos]
                    v_pool[pg * P + o] = v_cache[b, :, pos]
    return k_pool, v_pool, table


def _with_tree_slots(rng, k_pool, v_pool, k_tree, v_tree):
    """Append the tree rows to the pool at shuffled slots; returns the pool and tree_slot."""
    B, T, Hkv, D = k_tree.shape
    base = k_pool.shape[0]
    order = rng.permutation(B * T)
    tree_slot = (base + order).reshape(B, T).astype(np.int32)
    kp = np.concatenate([k_pool, np.zeros((B * T, Hkv, D), k_pool.dtype)])
    vp = np.concatenate([v_pool, np.zeros((B * T, Hkv, D), v_pool.dtype)])
    for b in range(B):
        for j in range(T):
            kp[tree_slot[b, j]] = k_tree[b, j]
            vp[tree_slot[b, j]] = v_tree[b, j]
    return kp, vp, tree_slot


def pin_paged_gather_and_attention(lib):
    """Attention through a block table (any page size, pages in any physical order) equals the
    pinned dense attention on the same rows, bit for bit."""
    rng = np.random.default_rng(41)
    for P, shuffle, dtype in [(1, True, "f32"), (4, False, "f32"), (16, True, "bf16"),
                              (3, True, "f32")]:
        case = small_case(rng, B=3, T=9, Hq=4, Hkv=2, D=16, Ls=(0, 37), dtype=dtype)
        q, kc, vc, L, kt, vt, parent = (case[k] for k in
                                        ("q", "k_cache", "v_cache", "cache_len", "k_tree",
                                         "v_tree", "parent"))
        k_pool, v_pool, table = _paged_from_dense(rng, kc, vc, L, P, shuffle)
        k_pool, v_pool, tree_slot = _with_tree_slots(rng, k_pool, v_pool, kt, vt)
        gk, gv, gkt, gvt = O.paged_gather(k_pool, v_pool, table, P, L, tree_slot, kc.shape[2],
                                          lib=lib)
        for b in range(kc.shape[0]):
            n = int(L[b])
            assert (gk[b, :, :n] == kc[b, :, :n]).all() and (gv[b, :, :n] == vc[b, :, :n]).all()
        assert (gkt == kt).all() and (gvt == vt).all()
        o1, l1 = O.attention(q, kc, vc, L, kt, vt, parent, lib=lib)
        o2, l2 = O.paged_attention(q, k_pool, v_pool, table, P, L, tree_slot, parent, lib=lib)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), (P, shuffle, dtype)
    # an entry outside the pool is refused, not read
    bad = table.copy()
    bad[0, 0] = k_pool.shape[0]
    try:
        O.paged_gather(k_pool, v_pool, bad, P, np.maximum(L, 1), tree_slot, 64, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("out-of-pool page accepted")


def pin_commit_paged_hand_case(lib):
    """Worked tree, path [0, 2, 5] after a 3-token prefix, one-token pages."""
    table = np.full((1, 12), -1, np.int32)
    table[0, :3] = [40, 41, 42]
    tree_slot = np.array([[50, 51, 52, 53, 54, 55, 56, 57]], np.int32)
    path = np.array([[0, 2, 5, -1, -1, -1, -1, -1]], np.int32)
    free = np.full(64, -7, np.int32)
    out_len, top, st = O.commit_paged(table, np.array([3], np.int32), tree_slot, path,
                                      np.array([3], np.int32), 60, free, 10, lib=lib)
    assert list(table[0]) == [40, 41, 42, 50, 52, 55] + [-1] * 6
    assert out_len[0] == 6 and top == 15 and st[0] == 0
    assert list(free[10:15]) == [51, 53, 54, 56, 57] and (free[:10] == -7).all()
    # a free list with room for three of the five rejected slots: the table is still committed,
    # the first three slots are written, nothing at or past num_slots, and the sequence is told
    table[0, 3:] = -1
    free[:] = -7
    out_len, top, st = O.commit_paged(table, np.array([3], np.int32), tree_slot, path,
                                      np.array([3], np.int32), 60, free, 57, lib=lib)
    assert list(table[0]) == [40, 41, 42, 50, 52, 55] + [-1] * 6 and out_len[0] == 6
    assert top == 62 and st[0] == O.ORC_FREE_FULL
    assert list(free[57:60]) == [51, 53, 54] and (free[60:] == -7).all()
    # exactly full: no flag
    free[:] = -7
    table[0, 3:] = -1
    out_len, top, st = O.commit_paged(table, np.array([3], np.int32), tree_slot, path,
                                      np.array([3], np.int32), 60, free, 55, lib=lib)
    assert top == 60 and st[0] == 0 and list(free[55:60]) == [51, 53, 54, 56, 57]


def pin_commit_paged_matches_copy(lib):
    """After a pointer-swap commit, the rows the table names for positions 0..L+n-1 are exactly
    the cache the pinned copying compaction produces; the free list receives exactly the
    rejected nodes' slots; bad sequences commit nothing."""
    rng = np.random.default_rng(43)
    B, T, Hkv, D = 6, 9, 2, 8
    case = small_case(rng, B=B, T=T, Hq=2, Hkv=Hkv, D=D, Ls=(0, 20))
    kc, vc, L, kt, vt = (case[k] for k in ("k_cache", "v_cache", "cache_len", "k_tree", "v_tree"))
    k_pool, v_pool, table = _paged_from_dense(rng, kc, vc, L, 1, True)
    k_pool, v_pool, tree_slot = _with_tree_slots(rng, k_pool, v_pool, kt, vt)
    num_slots = k_pool.shape[0]
    max_pages = 26
    tbl = np.full((B, max_pages), -1, np.int32)
    tbl[:, :table.shape[1]] = table
    paths = np.full((B, T), -1, np.int32)
    lens = np.array([1, 4, 9, 2, 7, 3], np.int32)
    for b in range(B):
        chosen = np.sort(rng.choice(np.arange(1, T), size=lens[b] - 1, replace=False))
        paths[b, :lens[b]] = np.concatenate([[0], chosen])
    L = L.copy()
    L[4] = 20  # 20 + 7 = 27 > 26: overflow by one row
    free = np.full(num_slots + 8, -1, np.int32)
    t0 = tbl.copy()
    out_len, top, st = O.commit_paged(tbl, L, tree_slot, paths, lens, num_slots, free, 0, lib=lib)
    # the copying compaction on the dense view of the same data
    Lmax = max_pages
    dk = np.zeros((B, Hkv, Lmax, D), kc.dtype)
    dv = np.zeros_like(dk)
    for b in range(B):
        for p in range(min(int(L[b]), kc.shape[2])):
            dk[b, :, p] = kc[b, :, p]
            dv[b, :, p] = vc[b, :, p]
    want_len, want_st = O.compact(dk, dv, L, kt, vt, paths, lens, lib=lib)
    assert np.array_equal(out_len, want_len) and np.array_equal(st, want_st)
    rejected = []
    for b in range(B):
        if st[b]:
            assert (tbl[b] == t0[b]).all()
            continue
        for p in range(int(out_len[b])):
            if p < L[b]:
                continue
            slot = tbl[b, p]
            assert (k_pool[slot] == dk[b, :, p]).all() and (v_pool[slot] == dv[b, :, p]).all()
        rejected += [int(tree_slot[b, j]) for j in range(T) if j not in set(paths[b, :lens[b]])]
    assert top == len(rejected) and sorted(free[:top]) == sorted(rejected)
    # malformed paths, lengths and slots commit nothing
    tbl2 = t0.copy()
    dup = paths.copy()
    dup[1, 2] = dup[1, 1]
    slots = tree_slot.copy()
    slots[2, 5] = num_slots
    out_len, top2, st = O.commit_paged(tbl2, np.array([-1, 3, 3, 3, 3, 27], np.int32), slots,
                                       dup, lens, num_slots, free, 5, lib=lib)
    assert list(st[:3]) == [O.ORC_BAD_LEN, O.ORC_BAD_PATH, O.ORC_BAD_PATH]
    assert st[5] == O.ORC_BAD_LEN
    assert (tbl2[[0, 1, 2, 5]] == t0[[0, 1, 2, 5]]).all()


# ----------------------------------------------------------------------------------------------
# stochastic acceptance (lesty.tech "EAGLE-2 vs. Medusa", section 4: rejection sampling)
# ----------------------------------------------------------------------------------------------
def _frac(tok: str) -> float:
    from fractions import Fraction

    return float(Fraction(tok.strip()))


def read_stochastic_cases():
    cases = []
    with open(os.path.join(GOLDEN, "stochastic_hand_cases.txt"), encoding="utf-8") as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            f_ = [x.strip() for x in line.split("|")]
            name, mode = f_[0], int(f_[1])
            draft = [int(x) for x in f_[2].split()]
            rows = []
            for field in (f_[3], f_[4]):
                r = np.full((8, 4), 0.25)
                for ent in filter(None, (e.strip() for e in field.split(";"))):
                    node, vals = ent.split(":")
                    r[int(node)] = [_frac(v) for v in vals.split(",")]
                rows.append(r)
            u_acc = [_frac(x) for x in f_[5].split()]
            u_res = [_frac(x) for x in f_[6].split()]
            path = [int(x) for x in f_[7].split(",")]
            cases.append((name, mode, draft, rows[0], rows[1], u_acc, u_res, path, int(f_[8])))
    return cases


def pin_stochastic_hand_cases(lib):
    parent = worked_tree_parent()
    for name, mode, draft, p, q, u_acc, u_res, want_path, want_bonus in read_stochastic_cases():
        path, n, bonus, st = O.accept_stochastic(parent[None], np.array([draft]), p[None], q[None],
                                                 np.array([u_acc]), np.array([u_res]),
                                                 without_replacement=mode, lib=lib)
        assert list(path[0, : n[0]]) == want_path, (name, path[0, : n[0]])
        assert (path[0, n[0]:] == -1).all(), name
        assert bonus[0] == want_bonus, (name, bonus[0])
        assert st[0] == 0, name


def pin_stochastic_duplicate_siblings(lib):
    """Hand-derived (no program computed the expected values): a root with three children whose
    tokens are 0, 0 and 1; V = 4; p = [1/4, 1/4, 3/8, 1/8], q = [1/2, 1/8, 1/8, 1/4];
    u_acc = 3/4, 1/2, 0.9 for children 1..3; u_res = 1/2 everywhere; leaves' p uniform.

    Both modes: child 1 (token 0): 3/4 * 1/2 = 3/8 >= 1/4, rejected; residual
    max(0, p - q) = [0, 1/8, 1/4, 0] -> p_2 = [0, 1/3, 2/3, 0].
    Mode 0: child 2 (token 0) has p_2(0) = 0, rejected; residual max(0, p_2 - q) =
    [0, 5/24, 13/24, 0] -> p_3 = [0, 5/18, 13/18, 0]; child 3 (token 1): ratio (5/18)/(1/8) > 1,
    kept; node 3 is a leaf, uniform p, u_res 1/2 -> running sums 1/4, 1/2, 3/4 -> token 2.
    Path 0,3; bonus 2.
    Mode 1: q loses token 0: q_2 = [0, 1/4, 1/4, 1/2].  Child 2 (token 0 again): p_2(0) = 0,
    rejected; residual max(0, p_2 - q_2) = [0, 1/12, 5/12, 0] -> p_3 = [0, 1/6, 5/6, 0]; token 0
    is already out of q, so q_3 = q_2.  Child 3 (token 1): 0.9 * 1/4 = 0.225 >= 1/6, rejected;
    residual [0, 0, 7/12, 0] -> token 2.  Path 0; bonus 2."""
    parent = np.array([[-1, 0, 0, 0]], np.int32)
    draft = np.array([[0, 0, 0, 1]], np.int32)
    p = np.full((1, 4, 4), 0.25, np.float32)
    q = p.copy()
    p[0, 0] = [0.25, 0.25, 0.375, 0.125]
    q[0, 0] = [0.5, 0.125, 0.125, 0.25]
    u_acc = np.array([[0.5, 0.75, 0.5, 0.9]])
    u_res = np.full((1, 4), 0.5)
    for mode, want_path in ((0, [0, 3]), (1, [0])):
        path, n, bonus, st = O.accept_stochastic(parent, draft, p, q, u_acc, u_res,
                                                 without_replacement=mode, lib=lib)
        assert list(path[0, : n[0]]) == want_path and bonus[0] == 2 and st[0] == 0, (mode, path, bonus)


def walk_distribution(lib, parent, draft, p, q, mode):
    """Exact probability of every emitted token sequence (accepted tokens, then the bonus) of the
    stochastic walk, with the uniforms integrated out.  The oracle is used as a black box: every
    acceptance is monotone in its uniform (accepted below a threshold) and every draw is monotone
    in its uniform (inverse CDF), so each branch's probability is the length of a uniform interval
    found by bisection (to 2^-50)."""
    from collections import defaultdict

    T, V = len(parent), p.shape[-1]
    kids = {u: [c for c in range(u + 1, T) if parent[c] == u] for u in range(T)}
    u_acc, u_res = np.full(T, 0.5), np.full(T, 0.5)

    def run():
        path, n, bonus, _ = O.accept_stochastic(parent[None], draft[None], p[None], q[None],
                                                u_acc[None], u_res[None],
                                                without_replacement=mode, lib=lib)
        return list(path[0, : n[0]]), int(bonus[0])

    def edge(pred):  # sup{x in [0, 1): pred(x)} for pred true on a lower interval
        if not pred(0.0):
            return 0.0
        top = 1.0 - 2.0 ** -40
        if pred(top):
            return 1.0
        lo, hi = 0.0, top
        for _ in range(50):
            mid = 0.5 * (lo + hi)
            lo, hi = (mid, hi) if pred(mid) else (lo, mid)
        return lo

    out = defaultdict(float)

    def visit(u, prob, emitted):
        for c in kids[u]:
            if not 0 <= draft[c] < V:
                continue

            def accepted(x, c=c):
                u_acc[c] = x
                return c in run()[0]

            thr = edge(accepted)
            if thr > 0.0:
                u_acc[c] = 0.5 * thr
                visit(c, prob * thr, emitted + (int(draft[c]),))
            if thr >= 1.0:
                return
            u_acc[c] = 0.5 * (thr + 1.0)
            prob *= 1.0 - thr
        # no child accepted: the bonus draw at u
        lo = [0.0]
        for y in range(1, V):
            def below(x, y=y):
                u_res[u] = x
                return run()[1] < y
            lo.append(edge(below))
        lo.append(1.0)
        for y in range(V):
            if lo[y + 1] > lo[y]:
                out[emitted + (y,)] += prob * (lo[y + 1] - lo[y])

    visit(0, 1.0, ())
    return out


def _draft_tuples(q_row, k, mode):
    """Every ordered k-tuple of drafted tokens with its probability: independent draws from q
    (mode 0) or draws without replacement (mode 1)."""
    V = len(q_row)
    for tup in itertools.product(range(V), repeat=k):
        if mode and len(set(tup)) < k:
            continue
        w, used = 1.0, 0.0
        for x in tup:
            w *= q_row[x] / (1.0 - used) if mode else q_row[x]
            used += q_row[x]
        if w > 0.0:
            yield tup, w


def _rand_dist(rng, V, zeros=()):
    """A random distribution with the given zero entries whose values are multiples of 1/256
    summing to exactly one (exact in float32), so that losslessness can be checked to 1e-9."""
    live = [y for y in range(V) if y not in zeros]
    c = np.zeros(V, np.int64)
    for y in live[:-1]:
        c[y] = rng.integers(1, 256 // len(live) + 1)
    c[live[-1]] = 256 - c.sum()
    return (c / 256.0).astype(np.float32)


def pin_stochastic_lossless_one_level(lib):
    """The page's claim, checked exactly: with the children of a node drafted from q
    (independently for mode 0, without replacement for mode 1), the first emitted token is
    distributed exactly as p, whatever p and q are (zeros included)."""
    rng = np.random.default_rng(51)
    V = 4
    for mode in (0, 1):
        for k in (1, 2, 3):
            for trial in range(2):
                p0 = _rand_dist(rng, V, zeros=(trial,))
                q0 = _rand_dist(rng, V, zeros=((trial + 2) % V,))
                parent = np.array([-1] + [0] * k, np.int32)
                p = np.tile(p0, (k + 1, 1))
                q = np.tile(q0, (k + 1, 1))
                first = np.zeros(V)
                for tup, w in _draft_tuples(q0.astype(np.float64), k, mode):
                    draft = np.array([0, *tup], np.int32)
                    for seq, pr in walk_distribution(lib, parent, draft, p, q, mode).items():
                        first[seq[0]] += w * pr
                want = p0.astype(np.float64) / p0.astype(np.float64).sum()
                assert np.abs(first - want).max() < 1e-9, (mode, k, first, want)


def pin_stochastic_lossless_two_levels(lib):
    """Two levels: the root's two children are drafted from q_root, each child's own child from
    the draft distribution after that child's token.  The first emitted token follows p_root and,
    after a kept first token y, the second follows the target distribution after y."""
    rng = np.random.default_rng(52)
    V = 3
    P1, Q1 = _rand_dist(rng, V, zeros=(1,)), _rand_dist(rng, V)
    P2 = [_rand_dist(rng, V, zeros=((y + 1) % V,)) for y in range(V)]
    Q2 = [_rand_dist(rng, V, zeros=(y,)) for y in range(V)]
    parent = np.array([-1, 0, 0, 1, 2], np.int32)
    for mode in (0, 1):
        joint = np.zeros((V, V))
        first = np.zeros(V)
        for top, w in _draft_tuples(Q1.astype(np.float64), 2, mode):
            for g1, w1 in _draft_tuples(Q2[top[0]].astype(np.float64), 1, mode):
                for g2, w2 in _draft_tuples(Q2[top[1]].astype(np.float64), 1, mode):
                    draft = np.array([0, top[0], top[1], g1[0], g2[0]], np.int32)
                    p = np.stack([P1, P2[top[0]], P2[top[1]], P1, P1])
                    q = np.stack([Q1, Q2[top[0]], Q2[top[1]], Q1, Q1])
                    for seq, pr in walk_distribution(lib, parent, draft, p, q, mode).items():
                        first[seq[0]] += w * w1 * w2 * pr
                        if len(seq) >= 2:
                            joint[seq[0], seq[1]] += w * w1 * w2 * pr
        want1 = P1.astype(np.float64) / P1.astype(np.float64).sum()
        assert np.abs(first - want1).max() < 1e-9, (mode, first, want1)
        for y in range(V):
            if joint[y].sum() > 1e-12:
                cond = joint[y] / joint[y].sum()
                want2 = P2[y].astype(np.float64) / P2[y].astype(np.float64).sum()
                assert np.abs(cond - want2).max() < 1e-9, (mode, y, cond, want2)


def _distinct_sibling_tokens(rng, parent, V):
    T = len(parent)
    draft = np.zeros(T, np.int32)
    for u in range(T):
        kids = [c for c in range(u + 1, T) if parent[c] == u]
        draft[kids] = rng.choice(V, size=len(kids), replace=False)
    return draft


def pin_stochastic_onehot_is_greedy(lib):
    """A one-hot target distribution (temperature 0) turns rejection sampling into the greedy
    rule: with distinct sibling tokens the walk equals the pinned greedy acceptance, and the bonus
    is the target's token at the last kept node, whatever the uniforms and q."""
    rng = np.random.default_rng(53)
    V = 40
    for mode in (0, 1):
        for T in (1, 2, 9, 40, 100):
            B = 4
            parents = np.stack([random_parent(rng, T) for _ in range(B)]).astype(np.int32)
            draft = np.stack([_distinct_sibling_tokens(rng, parents[b], V) for b in range(B)])
            target = rng.integers(0, V, size=(B, T)).astype(np.int32)
            # make acceptances likely: a node's target is often one of its children's tokens
            for b in range(B):
                for u in range(T):
                    kids = [c for c in range(u + 1, T) if parents[b, c] == u]
                    if kids and rng.random() < 0.7:
                        target[b, u] = draft[b, rng.choice(kids)]
            p = np.zeros((B, T, V), np.float32)
            np.put_along_axis(p, target[..., None], 1.0, axis=2)
            q = rng.random((B, T, V)).astype(np.float32) + 0.01
            q /= q.sum(-1, keepdims=True)
            u_acc = rng.random((B, T)).astype(np.float32)
            u_res = rng.random((B, T)).astype(np.float32)
            path, n, bonus, st = O.accept_stochastic(parents, draft, p, q, u_acc, u_res,
                                                     without_replacement=mode, lib=lib)
            g_path, g_n, g_bonus = O.accept(parents, draft, target, lib=lib)
            assert np.array_equal(n, g_n) and np.array_equal(path, g_path), (mode, T)
            assert np.array_equal(bonus, g_bonus) and (st == 0).all(), (mode, T)


def pin_stochastic_q_equals_p(lib):
    """q = p: every tested child has ratio 1 and is kept, so the walk follows first children to a
    leaf, and the bonus is an ordinary inverse-CDF draw from the leaf's p
    (numpy.searchsorted over the running sums)."""
    rng = np.random.default_rng(54)
    V = 50
    for mode in (0, 1):
        for T in (1, 7, 60, 128):
            B = 3
            parents = np.stack([random_parent(rng, T) for _ in range(B)]).astype(np.int32)
            draft = rng.integers(3, V, size=(B, T)).astype(np.int32)  # tokens with mass
            p = rng.random((B, T, V)) ** 4
            p[..., :3] = 0.0
            p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
            u_acc = rng.random((B, T)).astype(np.float32)
            u_res = rng.random((B, T)).astype(np.float32)
            path, n, bonus, st = O.accept_stochastic(parents, draft, p, p.copy(), u_acc, u_res,
                                                     without_replacement=mode, lib=lib)
            for b in range(B):
                want = [0]
                while True:
                    kids = [c for c in range(T) if parents[b, c] == want[-1]]
                    if not kids:
                        break
                    want.append(kids[0])
                assert list(path[b, : n[b]]) == want, (mode, T, b)
                leaf = p[b, want[-1]].astype(np.float64)
                cdf = np.cumsum(leaf)
                y = int(np.searchsorted(cdf, u_res[b, want[-1]] * cdf[-1], side="right"))
                assert bonus[b] == y, (mode, T, b, bonus[b], y)


def pin_stochastic_bad_tokens(lib):
    """A child whose token is outside the vocabulary is skipped and flagged; the walk goes on as
    if it were absent (compared with the same tree without that child's token being tested)."""
    parent = worked_tree_parent()
    V = 4
    p = np.full((1, 8, V), 0.25, np.float32)
    q = p.copy()
    u = np.full((1, 8), 0.5, np.float32)
    draft = np.array([[0, 7, 2, 0, 0, -1, 0, 0]], np.int32)  # node 1 and node 5 are out of range
    path, n, bonus, st = O.accept_stochastic(parent[None], draft, p, q, u, u, lib=lib)
    assert list(path[0, : n[0]]) == [0, 2] and st[0] == O.ORC_BAD_TOKEN
    assert bonus[0] == 2  # uniform p at node 2, u_res 0.5: running sums 0.25, 0.5, 0.75 -> 2



# ----------------------------------------------------------------------------------------------
# EAGLE-2 draft tree construction (rainlin.net "EAGLE 系列", section 7)
# ----------------------------------------------------------------------------------------------
def read_eagle2_case():
    levels, frontiers, cases = {}, {}, []
    with open(os.path.join(GOLDEN, "eagle2_hand_case.txt"), encoding="utf-8") as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            f_ = [x.strip() for x in line.split("|")]
            if f_[0] == "shape":
                k, branch, depth, root = (int(x) for x in f_[1:5])
            elif f_[0] == "level":
                levels[(int(f_[1]), int(f_[2]))] = ([int(x) for x in f_[3].split()],
                                                    [_frac(x) for x in f_[4].split()])
            elif f_[0] == "values":
                values = [int(x) / 64 for x in f_[1].split()]
            elif f_[0] == "parents":
                parents = [int(x) for x in f_[1].split()]
            elif f_[0] == "frontier":
                frontiers[int(f_[1])] = [int(x) for x in f_[2].split()]
            elif f_[0] == "case":
                cases.append((int(f_[1]), *([int(x) for x in fld.split()] for fld in f_[2:6])))
    tok = np.zeros((depth, 1, k, branch), np.int32)
    conf = np.zeros((depth, 1, k, branch), np.float32)
    for (lvl, slot), (t, c) in levels.items():
        tok[lvl - 1, 0, slot] = t
        conf[lvl - 1, 0, slot] = c
    return dict(k=k, branch=branch, depth=depth, root=root, tok=tok, conf=conf, values=values,
                parents=parents, frontiers=frontiers, cases=cases)


def pin_eagle2_hand_case(lib):
    g = read_eagle2_case()
    for T, nodes, parents, depths, toks in g["cases"]:
        r = O.eagle2_build(np.array([g["root"]]), g["tok"], g["conf"], T, lib=lib)
        assert r["status"][0] == 0, f"T={T}: status {r['status'][0]}"
        assert list(r["node_parent"][0]) == g["parents"]
        assert list(r["node_value"][0].astype(np.float64)) == g["values"]
        for lvl, want in g["frontiers"].items():
            assert list(r["frontier"][lvl - 1, 0, : len(want)]) == want, f"frontier {lvl}"
        assert list(r["node"][0]) == nodes, f"T={T}: nodes {list(r['node'][0])}"
        assert list(r["parent"][0]) == parents, f"T={T}: parents {list(r['parent'][0])}"
        assert list(r["depth"][0]) == depths and list(r["tok"][0]) == toks, f"T={T}"


def _e2_inputs(rng, B, depth, k, branch, ties=False, vocab=50):
    """Drafter outputs for a small expansion: confidences are a softmax of normal logits, sorted
    best first as a top-`branch` returns them (``ties``: rounded to a few dyadic values)."""
    logits = rng.normal(0.0, 1.4, size=(depth, B, k, branch))
    e = np.exp(logits - logits.max(axis=-1, keepdims=True))
    conf = -np.sort(-(e / e.sum(axis=-1, keepdims=True)), axis=-1)
    if ties:
        conf = np.clip(np.round(conf * 4) / 4, 0.25, 1.0)
    tok = rng.integers(0, vocab, size=(depth, B, k, branch)).astype(np.int32)
    root = rng.integers(0, vocab, size=B).astype(np.int32)
    return root, tok, conf.astype(np.float32)


def _outranks(values, a, b):
    return values[a] > values[b] or (values[a] == values[b] and a < b)


def _check_e2_structure(r, root, tok, conf, depth, k, branch, T, brute=True):
    """Independent checks of one construction: node table against the drafter outputs, path
    products taken by walking each root path, the top-set properties of every frontier and of
    the kept set (and, on tiny tables, the maximum-sum subset by enumeration), and the flattened
    order against a breadth-first traversal with children visited in id order."""
    B = root.shape[0]
    for b in range(B):
        par, val, ntok = r["node_parent"][b], r["node_value"][b], r["node_tok"][b]
        N = len(par)
        # table layout: child c of frontier slot r at level l is node base + r*branch + c
        front, base = [0], 1
        for lvl in range(1, depth + 1):
            for slot, u in enumerate(front):
                for c in range(branch):
                    nid = base + slot * branch + c
                    assert par[nid] == u and ntok[nid] == tok[lvl - 1, b, slot, c]
            n_lvl = len(front) * branch
            level_ids = list(range(base, base + n_lvl))
            F = min(k, n_lvl)
            got = [int(x) for x in r["frontier"][lvl - 1, b, :F]]
            assert all(x == -1 for x in r["frontier"][lvl - 1, b, F:])
            vals = {i: float(val[i]) for i in level_ids}
            for pos, x in enumerate(got):  # best first, and every member beats every non-member
                assert x in vals
                for y in level_ids:
                    if y not in got:
                        assert _outranks(vals, x, y), f"level {lvl}: {x} does not beat {y}"
                if pos:
                    assert _outranks(vals, got[pos - 1], x)
            front, base = got, base + n_lvl
        assert base == N
        # values: float32 products along the root path, root first
        for i in range(N):
            path = []
            cur = i
            while cur != -1:
                path.append(cur)
                cur = int(par[cur])
            v = np.float32(1.0)
            for nd in path[::-1][1:]:  # root first, the root itself excluded
                v = np.float32(v * _conf_of(r, tok, conf, b, nd, depth, k, branch))
            assert val[i] == v, f"node {i}: value {val[i]} != path product {v}"
        # kept set: the T best nodes
        kept = [int(x) for x in r["node"][b]]
        assert len(set(kept)) == T
        vals = {i: float(val[i]) for i in range(N)}
        kept_set = set(kept)
        for x in kept:
            for y in range(N):
                if y not in kept_set:
                    assert _outranks(vals, x, y), f"kept {x} does not beat dropped {y}"
        if brute and len(set(vals.values())) == N and math.comb(N, T) <= 20000:
            best = max(itertools.combinations(range(N), T),
                       key=lambda S: sum(vals[i] for i in S))
            assert set(best) == kept_set
        # flattened order: breadth-first from the root, children in id order
        order, queue = [], [0]
        kids = {i: [] for i in range(N)}
        for i in range(1, N):
            kids[int(par[i])].append(i)
        while queue:
            u = queue.pop(0)
            order.append(u)
            queue.extend(c for c in kids[u] if c in kept_set)
        assert order == kept, f"flattened {kept} != breadth-first {order}"
        pos = {u: f for f, u in enumerate(order)}
        assert list(r["parent"][b]) == [-1] + [pos[int(par[u])] for u in order[1:]]
        assert list(r["tok"][b]) == [int(ntok[u]) for u in order]
        assert r["tok"][b][0] == root[b]
        dep = [0] * T
        for f in range(1, T):
            dep[f] = dep[r["parent"][b][f]] + 1
        assert list(r["depth"][b]) == dep


def _conf_of(r, tok, conf, b, nd, depth, k, branch):
    """The drafter confidence that created node nd (found from the frontier records)."""
    front, base = [0], 1
    for lvl in range(1, depth + 1):
        n_lvl = len(front) * branch
        if nd < base + n_lvl:
            slot, c = divmod(nd - base, branch)
            return np.float32(min(max(float(conf[lvl - 1, b, slot, c]), 0.0), 1.0))
        F = min(k, n_lvl)
        front = [int(x) for x in r["frontier"][lvl - 1, b, :F]]
        base += n_lvl
    raise AssertionError("node id past the table")


def pin_eagle2_bruteforce(lib):
    rng = np.random.default_rng(7)
    for trial in range(60):
        depth, k, branch = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = O.eagle2_node_count(depth, k, branch)
        T = int(rng.integers(1, N + 1))
        root, tok, conf = _e2_inputs(rng, 2, depth, k, branch, ties=trial % 3 == 0)
        r = O.eagle2_build(root, tok, conf, T, lib=lib)
        assert (r["status"] == 0).all()
        _check_e2_structure(r, root, tok, conf, depth, k, branch, T)
    # a larger expansion (the top-set and breadth-first checks only)
    root, tok, conf = _e2_inputs(rng, 2, 5, 4, 4)
    r = O.eagle2_build(root, tok, conf, 40, lib=lib)
    _check_e2_structure(r, root, tok, conf, 5, 4, 4, 40, brute=False)


def pin_eagle2_batch_independent(lib):
    rng = np.random.default_rng(8)
    root, tok, conf = _e2_inputs(rng, 4, 4, 3, 3)
    r = O.eagle2_build(root, tok, conf, 17, lib=lib)
    for b in range(4):
        rb = O.eagle2_build(root[b : b + 1], tok[:, b : b + 1], conf[:, b : b + 1], 17, lib=lib)
        for name in ("node_tok", "node_parent", "node_value", "parent", "tok", "depth", "node"):
            assert (rb[name][0] == r[name][b]).all(), name
        assert (rb["frontier"][:, 0] == r["frontier"][:, b]).all()


def pin_eagle2_chain(lib):
    """One child per node: the tree is a chain, and the kept prefix is the first T levels."""
    rng = np.random.default_rng(9)
    depth = 7
    root, tok, conf = _e2_inputs(rng, 1, depth, 3, 1)
    conf[:] = rng.uniform(0.05, 0.95, size=conf.shape).astype(np.float32)
    for T in (1, 4, depth + 1):
        r = O.eagle2_build(root, tok, conf, T, lib=lib)
        assert list(r["node"][0]) == list(range(T))
        assert list(r["parent"][0]) == list(range(-1, T - 1))
        assert list(r["depth"][0]) == list(range(T))
        assert list(r["tok"][0]) == [int(root[0])] + [int(tok[i, 0, 0, 0]) for i in range(T - 1)]
        v = np.float32(1.0)
        for i in range(1, depth + 1):
            v = np.float32(v * conf[i - 1, 0, 0, 0])
            assert r["node_value"][0, i] == v


def pin_eagle2_keep_everything(lib):
    """No pruning (k at least the widest level) and T = all nodes: the flattened tree is the
    complete branch-ary tree in breadth-first order, parent of position f = (f - 1) // branch,
    whatever the confidences."""
    rng = np.random.default_rng(10)
    for depth, branch in ((3, 2), (2, 4), (4, 3)):
        k = branch ** depth
        root, tok, conf = _e2_inputs(rng, 2, depth, k, branch)
        N = O.eagle2_node_count(depth, k, branch)
        assert N == sum(branch ** i for i in range(depth + 1))
        r = O.eagle2_build(root, tok, conf, N, lib=lib)
        for b in range(2):
            assert list(r["parent"][b]) == [-1] + [(f - 1) // branch for f in range(1, N)]
            # every drafted token appears once (level l uses the first branch**(l-1) slots)
            exp = []
            F = 1
            for lvl in range(depth):
                exp += [int(x) for x in tok[lvl, b, :F].ravel()]
                F *= branch
            assert sorted(int(x) for x in r["tok"][b][1:]) == sorted(exp)
            assert r["tok"][b][0] == root[b]


def pin_eagle2_equal_confidences(lib):
    """Every confidence 1/2: a level's values all tie, so every frontier is its first k
    children, and the kept set is the T smallest ids, already in flattened order."""
    rng = np.random.default_rng(11)
    for depth, k, branch, T in ((3, 2, 3, 12), (4, 3, 2, 18), (2, 5, 5, 9)):
        root, tok, conf = _e2_inputs(rng, 1, depth, k, branch)
        conf[:] = 0.5
        r = O.eagle2_build(root, tok, conf, T, lib=lib)
        assert list(r["node"][0]) == list(range(T))
        assert list(r["parent"][0]) == [int(x) for x in r["node_parent"][0, :T]]
        base, F = 1, 1
        for lvl in range(depth):
            n_lvl = F * branch
            F = min(k, n_lvl)
            assert list(r["frontier"][lvl, 0, :F]) == list(range(base, base + F))
            base += n_lvl


def pin_eagle2_bad_confidences(lib):
    """Confidences outside [0, 1] are flagged and used clamped: NaN and negatives as 0, values
    above one as 1 (-0.0 is a valid 0)."""
    rng = np.random.default_rng(12)
    root, tok, conf = _e2_inputs(rng, 2, 3, 3, 3)
    bad = conf.copy()
    bad[0, 0, 0, 1] = np.nan
    bad[1, 0, 1, 0] = -0.5
    bad[2, 0, 0, 2] = 1.5
    bad[1, 0, 0, 0] = np.inf
    bad[0, 1, 0, 2] = -0.0
    clamped = bad.copy()
    clamped[np.isnan(clamped)] = 0.0
    clamped = np.clip(clamped, 0.0, 1.0)
    clamped[0, 1, 0, 2] = 0.0
    rb = O.eagle2_build(root, tok, bad, 20, lib=lib)
    rc = O.eagle2_build(root, tok, clamped, 20, lib=lib)
    assert list(rb["status"]) == [O.ORC_BAD_CONF, 0] and list(rc["status"]) == [0, 0]
    for name in ("node_parent", "node_value", "frontier", "parent", "tok", "depth", "node"):
        assert np.array_equal(rb[name], rc[name]), name
    assert not np.signbit(rb["node_value"]).any()


def pin_eagle2_rerank_tables(lib):
    """Reranking of caller-built tables: a valid one (values never grow from parent to child)
    gives the top-set and breadth-first order; a table that is not such a tree is flagged and
    gets parent -1, token -1, depth 0, node -1 everywhere."""
    rng = np.random.default_rng(13)
    N, T = 30, 12
    par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, N)], np.int32)
    val = np.ones(N, np.float32)
    for i in range(1, N):
        val[i] = np.float32(val[par[i]] * np.float32(rng.choice([0.25, 0.5, 0.75, 1.0])))
    ntok = rng.integers(0, 100, size=N).astype(np.int32)
    r = O.eagle2_rerank(ntok[None], par[None], val[None], T, lib=lib)
    assert r["status"][0] == 0
    kept = [int(x) for x in r["node"][0]]
    vals = {i: float(val[i]) for i in range(N)}
    for x in kept:
        for y in set(range(N)) - set(kept):
            assert _outranks(vals, x, y)
    order, queue = [], [0]
    while queue:
        u = queue.pop(0)
        order.append(u)
        queue.extend(c for c in range(1, N) if par[c] == u and c in kept)
    assert order == kept
    bads = []
    p1 = par.copy(); p1[0] = 0; bads.append((p1, val))                      # root not a root
    p2 = par.copy(); p2[7] = 7; bads.append((p2, val))                      # parent not below
    p3 = par.copy(); p3[9] = -1; bads.append((p3, val))                     # second root
    v4 = val.copy(); c = int(np.argmax(par > 0)); v4[c] = val[par[c]] * 2   # child above parent
    bads.append((par, v4))
    for pb, vb in bads:
        rb = O.eagle2_rerank(np.stack([ntok, ntok]), np.stack([pb, par]), np.stack([vb, val]), T,
                             lib=lib)
        assert list(rb["status"]) == [O.ORC_BAD_TREE, 0]
        assert (rb["parent"][0] == -1).all() and (rb["tok"][0] == -1).all()
        assert (rb["depth"][0] == 0).all() and (rb["node"][0] == -1).all()
        assert list(rb["node"][1]) == kept


# ----------------------------------------------------------------------------------------------
# two-stage drafter LM head (jialefu.github.io, "EAGLE-4: Notes on the Efficient LM Head")
# ----------------------------------------------------------------------------------------------
def _bits(x) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _read_lm_hand_case():
    rec = {}
    with open(os.path.join(GOLDEN, "lm_head_hand_case.txt"), encoding="utf-8") as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            k, v = (x.strip() for x in line.split("|"))
            rec[k] = v
    return rec


def pin_lm_hand_case(lib):
    """The hand-derived case (tests/golden/lm_head_hand_case.txt): projection, the score of
    every stored row, tile boundaries and padding, ties to the smaller row, candidates mapped
    through the row shuffle, exact logits, children with ties to the smaller token, and
    confidences normalised over every valid candidate."""
    g = _read_lm_hand_case()
    num = lambda k: [float(x) for x in g[k].split()]  # noqa: E731
    d = int(g["d"])
    h = np.zeros((1, d), np.float32)
    h[0, 0] = float(g["h0"])
    b0 = num("B_col0")
    Bm = np.full((len(b0), d), 100.0, np.float32)
    Bm[:, 0] = b0
    A = np.array([[float(x) for x in row.split()] for row in g["A"].split(";")], np.float32)
    perm = np.array([int(x) for x in g["row_token"].split()], np.int32)
    w0 = num("W_col0")
    W = np.full((len(w0), d), 100.0, np.float32)
    W[:, 0] = w0
    tile, k_tile, K = int(g["tile"]), int(g["k_tile"]), int(g["K"])
    u = O.lm_project(_bits(h), _bits(Bm), lib=lib)
    assert list(u[0]) == num("u")
    assert list(O.lm_scores(_bits(A), u, lib=lib)[0]) == num("scores")
    res = O.lm_head_two_stage(_bits(h), _bits(A), _bits(Bm), _bits(W), perm, tile, k_tile, K,
                              lib=lib)
    assert list(res["cand"][0]) == [int(x) for x in g["cand"].split()]
    assert list(res["cand_score"][0]) == num("cand_score")
    assert list(res["logits"][0]) == num("logits") and res["status"][0] == 0
    assert list(res["tok"][0]) == [int(x) for x in g["children"].split()]
    Z = sum(math.exp(x) for x in num("Z_logits"))
    for j, lg in enumerate(num("children_logits")):
        assert abs(res["conf"][0, j] - math.exp(lg) / Z) <= 1e-15


def _int_lm_case(rng, M, d, r, n, lo=-3, hi=4):
    """Small-integer bfloat16 inputs: every product and partial sum is an integer below 2^24,
    so float32 arithmetic in any order is exact and equals numpy's int64 results."""
    h = rng.integers(lo, hi, size=(M, d))
    Bm = rng.integers(lo, hi, size=(r, d))
    A = rng.integers(lo, hi, size=(n, r))
    W = rng.integers(lo, hi, size=(n, d))
    perm = rng.permutation(n).astype(np.int32)
    return h, Bm, A, W, perm


def _lexsort_best(vals, keys2, k):
    """Indices of the k largest vals, ties to the smaller keys2 (numpy lexsort)."""
    order = np.lexsort((keys2, -np.asarray(vals, dtype=np.float64)))
    return order[:k]


def pin_lm_integer_bruteforce(lib):
    """Exact small-integer cases against numpy: u = B h, per-tile screening (top k_tile rows of
    each tile, ties to the smaller row, mapped through the row permutation), exact logits of the
    candidates, the K best (ties to the smaller token) and softmax confidences over the
    candidates."""
    from scipy.special import softmax

    rng = np.random.default_rng(31)
    for trial in range(25):
        M, d, r = int(rng.integers(1, 4)), 512 * int(rng.integers(1, 3)), int(rng.integers(1, 9))
        n, tile, k_tile = int(rng.integers(5, 60)), int(rng.integers(2, 12)), int(rng.integers(1, 4))
        h, Bm, A, W, perm = _int_lm_case(rng, M, d, r, n)
        K = int(rng.integers(1, 6))
        res = O.lm_head_two_stage(_bits(h), _bits(A[perm]), _bits(Bm), _bits(W), perm, tile, k_tile,
                                  K, lib=lib)
        u = h @ Bm.T  # [M, r], exact
        assert np.array_equal(res["u"], u.astype(np.float64))
        As = A[perm]  # row q of the shuffled head is token perm[q]
        scores = u @ As.T  # [M, n], exact
        n_tiles = -(-n // tile)
        for m in range(M):
            want = []
            for t in range(n_tiles):
                rows = np.arange(t * tile, min(n, (t + 1) * tile))
                best = rows[_lexsort_best(scores[m, rows], rows, k_tile)]
                want += [int(perm[q]) for q in best] + [-1] * (k_tile - len(best))
            assert list(res["cand"][m]) == want, (trial, m)
            valid = res["cand"][m] >= 0
            exact = (W[np.maximum(res["cand"][m], 0)] @ h[m]).astype(np.float64)
            assert np.array_equal(res["logits"][m][valid], exact[valid])
            want_s = [scores[m, perm.tolist().index(t)] if t >= 0 else -np.inf
                      for t in res["cand"][m]]
            assert np.array_equal(res["cand_score"][m], np.array(want_s, np.float64))
            assert np.isneginf(res["logits"][m][~valid]).all()
            vc = res["cand"][m][valid]
            top = vc[_lexsort_best(exact[valid], vc, K)]
            assert list(res["tok"][m][: len(top)]) == [int(x) for x in top]
            assert (res["tok"][m][len(top):] == -1).all()
            p = softmax(exact[valid])
            conf = {int(t): float(p[i]) for i, t in enumerate(vc)}
            for j, t in enumerate(res["tok"][m][: len(top)]):
                assert abs(res["conf"][m, j] - conf[int(t)]) <= 1e-12


def pin_lm_fp64_near_exact(lib):
    """Normal-valued bfloat16 inputs: u, the scores of every row and the logits of every token
    lie within n * 2^-53 * sum |x_i y_i| (plus the propagated error of u) of the exact rational
    values, computed with fractions.Fraction on a sample of entries."""
    from fractions import Fraction

    rng = np.random.default_rng(32)
    M, d, r, n = 2, 1024, 24, 30
    h = _bits(rng.standard_normal((M, d)))
    Bm = _bits(rng.standard_normal((r, d)))
    A = _bits(rng.standard_normal((n, r)))
    W = _bits(rng.standard_normal((n, d)))
    fr = lambda b: [Fraction(float(x)) for x in bf16_bits_to_f32(b).reshape(-1)]  # noqa: E731
    hq, Bq, Aq, Wq = fr(h), fr(Bm), fr(A), fr(W)
    f = lambda b: bf16_bits_to_f32(b).astype(np.float64)  # noqa: E731
    u = O.lm_project(h, Bm, lib=lib)
    s = O.lm_scores(A, u, lib=lib)
    L = O.lm_logits_all(W, h, n_threads=2, lib=lib)
    eps = 2.0 ** -53
    for m in range(M):
        hm = hq[m * d:(m + 1) * d]
        ue = [sum(Bq[i * d + k] * hm[k] for k in range(d)) for i in range(r)]
        mag_u = np.abs(f(Bm)) @ np.abs(f(h[m]))
        assert all(abs(Fraction(float(u[m, i])) - ue[i]) <= Fraction(d * eps * mag_u[i])
                   for i in range(r))
        for row in range(0, n, 7):
            se = sum(Aq[row * r + i] * ue[i] for i in range(r))
            bound = r * eps * float(np.abs(f(A[row])) @ np.abs(u[m])) + \
                float(np.abs(f(A[row])) @ (d * eps * mag_u)) * 1.01
            assert abs(Fraction(float(s[m, row])) - se) <= Fraction(bound)
        for v in range(0, n, 5):
            le = sum(Wq[v * d + k] * hm[k] for k in range(d))
            bound = d * eps * float(np.abs(f(W[v])) @ np.abs(f(h[m])))
            assert abs(Fraction(float(L[m, v])) - le) <= Fraction(bound)
    # the candidates' logits are the full head's logits at those tokens
    cand = rng.integers(0, n, size=(M, 9)).astype(np.int32)
    lg, st = O.lm_rescore(W, h, cand, lib=lib)
    assert (st == 0).all() and np.array_equal(lg, np.take_along_axis(L, cand, axis=1))


def pin_lm_exact_screen_keeps_global_best(lib):
    """A screening head equal to the full head (A = W, B = identity) with k_tile >= K keeps
    every token of the global top K, so the children equal the full vocabulary's best K
    (numpy over all of W h, ties to the smaller token), whatever the row shuffle."""
    rng = np.random.default_rng(33)
    for trial in range(10):
        M, d, n, K = 2, 512, int(rng.integers(20, 90)), int(rng.integers(1, 5))
        tile, k_tile = int(rng.integers(3, 10)), K + int(rng.integers(0, 3))
        h, _, _, W, perm = _int_lm_case(rng, M, d, 1, n, lo=-6, hi=7)
        eye = np.eye(d, dtype=np.int64)
        res = O.lm_head_two_stage(_bits(h), _bits(W[perm]), _bits(eye), _bits(W), perm, tile,
                                  k_tile, K, lib=lib)
        full = W @ h.T  # [n, M]
        for m in range(M):
            best = _lexsort_best(full[:, m], np.arange(n), K)
            assert list(res["tok"][m]) == [int(x) for x in best], (trial, m)


def pin_lm_padding_and_bad_tokens(lib):
    """A last tile shorter than k_tile pads with token -1 (score -inf); -1 candidates get -inf
    logits without a flag, out-of-range ones get -inf and ORC_BAD_TOKEN; the children skip them
    and pad with -1 / 0 when fewer than K valid candidates remain."""
    rng = np.random.default_rng(34)
    h, Bm, A, W, perm = _int_lm_case(rng, 2, 512, 4, 7)
    u = O.lm_project(_bits(h), _bits(Bm), lib=lib)
    cand, score = O.lm_screen(_bits(A), u, perm, 3, 2, lib=lib)  # tiles of 3, 3, 1 rows
    assert cand.shape == (2, 6) and (cand[:, 5] == -1).all() and np.isneginf(score[:, 5]).all()
    bad = cand.copy()
    bad[0, 0] = 7      # outside the vocabulary
    bad[1, 1] = -5
    logits, st = O.lm_rescore(_bits(W), _bits(h), bad, lib=lib)
    assert list(st) == [O.ORC_BAD_TOKEN, O.ORC_BAD_TOKEN]
    assert np.isneginf(logits[0, [0, 5]]).all() and np.isneginf(logits[1, [1, 5]]).all()
    tok, conf = O.lm_topk(logits, bad, 6, 7, lib=lib)
    assert list(tok[0, 4:]) == [-1, -1] and list(conf[0, 4:]) == [0.0, 0.0]
    assert set(tok[0, :4]) == set(int(x) for x in bad[0, 1:5])
    assert abs(conf[0].sum() - 1.0) < 1e-12

ALL_PINS = [
    pin_worked_tree_mask,
    pin_mask_closure_bruteforce,
    pin_mask_closure_random,
    pin_mask_invalid_trees,
    pin_visibility_probe,
    pin_scale_zero_is_mean,
    pin_chain_matches_causal_sdpa,
    pin_single_node_is_decode,
    pin_dense_mask_bruteforce,
    pin_per_path_invariant,
    pin_selected_rows_match_full,
    pin_accept_hand_cases,
    pin_accept_chain_extremes,
    pin_accept_bruteforce,
    pin_compact_hand_case,
    pin_compact_alias,
    pin_compact_random,
    pin_paged_gather_and_attention,
    pin_commit_paged_hand_case,
    pin_commit_paged_matches_copy,
    pin_stochastic_hand_cases,
    pin_stochastic_duplicate_siblings,
    pin_stochastic_bad_tokens,
    pin_stochastic_q_equals_p,
    pin_stochastic_onehot_is_greedy,
    pin_stochastic_lossless_one_level,
    pin_stochastic_lossless_two_levels,
    pin_eagle2_hand_case,
    pin_eagle2_chain,
    pin_eagle2_equal_confidences,
    pin_eagle2_keep_everything,
    pin_eagle2_bad_confidences,
    pin_eagle2_rerank_tables,
    pin_eagle2_batch_independent,
    pin_eagle2_bruteforce,
    pin_lm_hand_case,
    pin_lm_integer_bruteforce,
    pin_lm_fp64_near_exact,
    pin_lm_exact_screen_keeps_global_best,
    pin_lm_padding_and_bad_tokens,
]
