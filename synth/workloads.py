"""Seeded synthetic workloads shaped like the pages' verification workloads.

None of the pages' datasets (MT-bench, ShareGPT, HumanEval) nor any model
weights are available, and the verification path needs neither: it only needs
a draft tree, per-node draft and target tokens, a KV prefix and the q/k/v of
the tree tokens.  Everything here is drawn from ``numpy.random.default_rng``
seeded with ``SeedSequence([workload_id, b, stream, extra])`` where ``stream``
is 0 for the tree and tokens, 1 for q, 2 for k/v and 3 for the prefix length,
so every sequence of a batch is reproducible on its own.

Trees for the larger workloads follow the EAGLE-2 dynamic draft tree
(rainlin.net "EAGLE 系列", section 7: expand the top nodes of the deepest
layer by path-product confidence, then rerank all candidates and keep the
best, which stays a connected tree because a child's value never exceeds its
parent's).  Target tokens follow the calibration observation of section 6
(draft confidence approximates acceptance rate): the target picks a child of
an expanded node with probability equal to that child's confidence.

The worked 8-node tree It/is/has/a/the/to/good/be (rainlin.net section 4) is
``worked_tree_parent()``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
import math

import numpy as np

# Stream ids of the per-sequence seed sequences.
STREAM_TREE, STREAM_Q, STREAM_KV, STREAM_LEN = 0, 1, 2, 3

BF16_NAN_BITS = np.uint16(0x7FC0)
LLAMA3_VOCAB = 128256  # any vocabulary at least as large as the branch width works


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """Shape and tree recipe of one synthetic workload."""

    wid: int                 # numeric id, first element of every seed sequence
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    L_lo: int                # prefix length ~ U{L_lo..L_hi}; L_lo == L_hi means fixed
    L_hi: int
    T: int
    dtype: str               # "f32" or "bf16"
    tree: str                # "worked" or "eagle2"
    depth_max: int = 0
    topk: int = 0
    branch: int = 0
    vocab: int = LLAMA3_VOCAB
    desc: str = ""


WORKLOADS: dict[str, WorkloadSpec] = {
    s.name: s
    for s in [
        WorkloadSpec(1, "worked_tree_fp32", B=1, Hq=2, Hkv=1, D=64, L_lo=16, L_hi=16, T=8,
                     dtype="f32", tree="worked", vocab=1000,
                     desc="worked 8-node tree It/is/has/a/the/to/good/be, prefix 16, 2 query heads on 1 KV "
                          "head, head_dim 64, fp32"),
        WorkloadSpec(2, "llama8b_b1_L4096_T60", B=1, Hq=32, Hkv=8, D=128, L_lo=4096, L_hi=4096, T=60,
                     dtype="bf16", tree="eagle2", depth_max=6, topk=10, branch=10,
                     desc="Llama-3-8B-like layer: batch 1, 32/8 heads, head_dim 128, prefix 4096, 60-node "
                          "EAGLE-2 tree (depth<=6, top-10 expand, 10 children), bf16"),
        WorkloadSpec(3, "batch32_L512-4096_T60", B=32, Hq=32, Hkv=8, D=128, L_lo=512, L_hi=4096, T=60,
                     dtype="bf16", tree="eagle2", depth_max=6, topk=10, branch=10,
                     desc="continuous batch: 32 sequences, prefix U[512,4096], 32/8 heads, head_dim 128, "
                          "60-node EAGLE-2 tree per sequence, bf16"),
        WorkloadSpec(4, "llama70b_b8_L32768_T64", B=8, Hq=64, Hkv=8, D=128, L_lo=32768, L_hi=32768, T=64,
                     dtype="bf16", tree="eagle2", depth_max=8, topk=10, branch=10,
                     desc="70B-like layer, long context: batch 8, 64/8 heads, head_dim 128, prefix 32768, "
                          "64-node EAGLE-2 tree (depth<=8), bf16"),
        WorkloadSpec(5, "wide_b64_L1024-8192_T128", B=64, Hq=32, Hkv=8, D=128, L_lo=1024, L_hi=8192,
                     T=128, dtype="bf16", tree="eagle2", depth_max=10, topk=16, branch=16,
                     desc="wide-tree stress: batch 64, prefix U[1024,8192], 32/8 heads, head_dim 128, "
                          "128-node tree (depth<=10, 16-way expansion), bf16"),
    ]
}


def _rng(wid: int, b: int, stream: int, extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wid, b, stream, extra]))


# ----------------------------------------------------------------------------------------------
# bf16 storage helpers (input encoding only)
# ----------------------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------------------
# trees and tokens
# ----------------------------------------------------------------------------------------------
def worked_tree_parent() -> np.ndarray:
    """Parent array of the worked tree It/is/has/a/the/to/good/be in its flattened level order."""
    return np.array([-1, 0, 0, 1, 1, 2, 3, 5], dtype=np.int32)


def random_parent(rng: np.random.Generator, T: int, kind: str = "random") -> np.ndarray:
    """A valid level-ordered tree (parent[0] = -1, 0 <= parent[i] < i) of the given kind."""
    p = np.empty(T, dtype=np.int32)
    p[0] = -1
    if T == 1:
        return p
    if kind == "chain":
        p[1:] = np.arange(T - 1, dtype=np.int32)
    elif kind == "star":
        p[1:] = 0
    elif kind == "random":
        for i in range(1, T):
            p[i] = rng.integers(0, i)
    elif kind == "deep":  # mostly chain-like with occasional branches
        for i in range(1, T):
            p[i] = i - 1 if rng.random() < 0.8 else rng.integers(0, i)
    else:
        raise ValueError(kind)
    return p


def _children(parent: np.ndarray) -> list[list[int]]:
    kids: list[list[int]] = [[] for _ in range(len(parent))]
    for i in range(1, len(parent)):
        kids[int(parent[i])].append(i)
    return kids


def _worked_tree_tokens(rng: np.random.Generator, vocab: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Tokens for the worked tree: draft uniform in [0, vocab); a node with children gets, with
    probability 0.7, the token of one child picked uniformly, otherwise a uniform token that no
    child carries; a leaf gets a uniform token."""
    parent = worked_tree_parent()
    T = len(parent)
    draft = rng.integers(0, vocab, size=T).astype(np.int32)
    target = np.empty(T, dtype=np.int32)
    kids = _children(parent)
    for u in range(T):
        if kids[u] and rng.random() < 0.7:
            target[u] = draft[kids[u][int(rng.integers(0, len(kids[u])))]]
        else:
            child_toks = {int(draft[c]) for c in kids[u]}
            while True:
                tok = int(rng.integers(0, vocab))
                if tok not in child_toks:
                    break
            target[u] = tok
    return parent, draft, target


def eagle2_tree(rng: np.random.Generator, T: int, depth_max: int, topk: int, branch: int,
                vocab: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """EAGLE-2-style dynamic draft tree with calibrated synthetic targets.

    Expansion: at each level take the ``topk`` nodes of the deepest layer with the largest
    path-product value (ties: earlier-created node first) and give each ``branch`` children
    whose confidences are the softmax of ``branch`` N(0, variance 2) logits and whose tokens are
    distinct.  A child's value is its parent's value times its confidence.
    Rerank: keep the ``T`` nodes of largest value (ties: shallower, then earlier).  Because every
    confidence is below one, a parent always outranks its children, so the kept set is a tree.
    Flattening: order by (depth, flattened index of the parent, confidence rank among siblings).
    Targets: an expanded node's target is the token of one of its children (kept or not) drawn
    with probability equal to the child's confidence; an unexpanded node gets a uniform token.
    """
    depth = [0]
    par = [-1]
    value = [1.0]
    token = [int(rng.integers(0, vocab))]
    rank = [0]
    expanded: dict[int, tuple[list[int], np.ndarray]] = {}
    frontier = [0]
    for _level in range(1, depth_max + 1):
        chosen = sorted(frontier, key=lambda n: (-value[n], n))[:topk]
        new_frontier: list[int] = []
        for u in chosen:
            logits = rng.normal(0.0, math.sqrt(2.0), size=branch)
            e = np.exp(logits - logits.max())
            conf = e / e.sum()
            toks = rng.choice(vocab, size=branch, replace=False)
            order = np.argsort(-conf, kind="stable")
            kid_ids = []
            for r, ci in enumerate(order):
                nid = len(depth)
                depth.append(depth[u] + 1)
                par.append(u)
                value.append(value[u] * float(conf[ci]))
                token.append(int(toks[ci]))
                rank.append(r)
                kid_ids.append(nid)
                new_frontier.append(nid)
            expanded[u] = (kid_ids, conf[order])
        frontier = new_frontier
    n_all = len(depth)
    if T > n_all:
        raise ValueError(f"tree budget {T} exceeds {n_all} candidates")
    keep = sorted(range(n_all), key=lambda n: (-value[n], depth[n], n))[:T]
    keep_set = set(keep)
    for n in keep:
        if par[n] >= 0 and par[n] not in keep_set:
            raise AssertionError("reranked set is not ancestor-closed")
    flat_of: dict[int, int] = {}
    order_nodes = sorted(keep, key=lambda n: (depth[n], -1 if par[n] < 0 else 0, n))
    # assign flattened indices level by level so the parent's flattened index is known
    by_depth: dict[int, list[int]] = {}
    for n in order_nodes:
        by_depth.setdefault(depth[n], []).append(n)
    flat: list[int] = []
    for d in sorted(by_depth):
        level_nodes = sorted(by_depth[d], key=lambda n: (-1 if par[n] < 0 else flat_of[par[n]], rank[n]))
        for n in level_nodes:
            flat_of[n] = len(flat)
            flat.append(n)
    parent = np.array([-1 if par[n] < 0 else flat_of[par[n]] for n in flat], dtype=np.int32)
    draft = np.array([token[n] for n in flat], dtype=np.int32)
    target = np.empty(T, dtype=np.int32)
    for i, n in enumerate(flat):
        if n in expanded:
            kid_ids, conf = expanded[n]
            pick = int(rng.choice(len(kid_ids), p=conf / conf.sum()))
            target[i] = token[kid_ids[pick]]
        else:
            target[i] = int(rng.integers(0, vocab))
    return parent, draft, target


# ----------------------------------------------------------------------------------------------
# whole workloads
# ----------------------------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """Host arrays of one verification step.  Floating tensors are float32 arrays for
    ``dtype == "f32"`` and raw bfloat16 bit patterns (uint16) for ``dtype == "bf16"``."""

    spec: WorkloadSpec
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    Lmax: int
    dtype: str
    parent: np.ndarray       # [B,T] int32
    draft: np.ndarray        # [B,T] int32
    target: np.ndarray       # [B,T] int32
    cache_len: np.ndarray    # [B] int32
    q: np.ndarray            # [B,T,Hq,D]
    k_cache: np.ndarray      # [B,Hkv,Lmax,D]; rows >= cache_len[b] are NaN
    v_cache: np.ndarray
    k_tree: np.ndarray       # [B,T,Hkv,D]
    v_tree: np.ndarray

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def kv_prefix_bytes(self) -> int:
        elem = 4 if self.dtype == "f32" else 2
        return int(self.cache_len.astype(np.int64).sum()) * self.Hkv * self.D * 2 * elem


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def make_workload(spec: WorkloadSpec | str, extra_seed: int = 0, B: int | None = None,
                  T: int | None = None, L: tuple[int, int] | None = None,
                  Hq: int | None = None, Hkv: int | None = None, D: int | None = None,
                  dtype: str | None = None, parent_kind: str | None = None,
                  lmax_pad: int = 64, with_kv: bool = True) -> Workload:
    """Draw one workload.  Keyword overrides shrink or reshape a spec for tests (the tree
    recipe of the spec is kept unless ``parent_kind`` asks for a random shape instead)."""
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    B = spec.B if B is None else B
    T = spec.T if T is None else T
    Hq = spec.Hq if Hq is None else Hq
    Hkv = spec.Hkv if Hkv is None else Hkv
    D = spec.D if D is None else D
    dtype = spec.dtype if dtype is None else dtype
    L_lo, L_hi = (spec.L_lo, spec.L_hi) if L is None else L
    wid = spec.wid

    parent = np.empty((B, T), np.int32)
    draft = np.empty((B, T), np.int32)
    target = np.empty((B, T), np.int32)
    cache_len = np.empty(B, np.int32)
    for b in range(B):
        rt = _rng(wid, b, STREAM_TREE, extra_seed)
        if parent_kind is not None:
            p = random_parent(rt, T, parent_kind)
            small_vocab = 4  # small vocabulary: matches and duplicate siblings are frequent
            parent[b] = p
            draft[b] = rt.integers(0, small_vocab, size=T)
            target[b] = rt.integers(0, small_vocab, size=T)
        elif spec.tree == "worked":
            if T != 8:
                raise ValueError("the worked tree has 8 nodes")
            parent[b], draft[b], target[b] = _worked_tree_tokens(rt, spec.vocab)
        else:
            parent[b], draft[b], target[b] = eagle2_tree(rt, T, spec.depth_max, spec.topk,
                                                         spec.branch, spec.vocab)
        rl = _rng(wid, b, STREAM_LEN, extra_seed)
        cache_len[b] = L_lo if L_lo == L_hi else int(rl.integers(L_lo, L_hi + 1))

    Lmax = int(cache_len.max()) + T
    Lmax = ((Lmax + lmax_pad - 1) // lmax_pad) * lmax_pad

    store = np.float32 if dtype == "f32" else np.uint16
    nan = np.float32(np.nan) if dtype == "f32" else BF16_NAN_BITS
    q = np.empty((B, T, Hq, D), store)
    if with_kv:  # rows at and past each prefix are NaN (filled per sequence below)
        k_cache = np.empty((B, Hkv, Lmax, D), store)
        v_cache = np.empty((B, Hkv, Lmax, D), store)
    else:
        k_cache = v_cache = np.empty((0,), store)
    k_tree = np.empty((B, T, Hkv, D), store)
    v_tree = np.empty((B, T, Hkv, D), store)

    def draw(b):  # every sequence has its own generators, so the draws may run in any order
        q[b] = _normal(_rng(wid, b, STREAM_Q, extra_seed), (T, Hq, D), dtype)
        rkv = _rng(wid, b, STREAM_KV, extra_seed)
        Lb = int(cache_len[b])
        if with_kv:
            k_cache[b, :, :Lb] = _normal(rkv, (Hkv, Lb, D), dtype)
            v_cache[b, :, :Lb] = _normal(rkv, (Hkv, Lb, D), dtype)
            k_cache[b, :, Lb:] = nan
            v_cache[b, :, Lb:] = nan
        k_tree[b] = _normal(rkv, (T, Hkv, D), dtype)
        v_tree[b] = _normal(rkv, (T, Hkv, D), dtype)

    workers = min(B, 16, len(os.sched_getaffinity(0)))
    if workers > 1 and with_kv:
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(draw, range(B)))
    else:
        for b in range(B):
            draw(b)
    return Workload(spec=spec, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, Lmax=Lmax, dtype=dtype,
                    parent=parent, draft=draft, target=target, cache_len=cache_len, q=q,
                    k_cache=k_cache, v_cache=v_cache, k_tree=k_tree, v_tree=v_tree)


@dataclasses.dataclass
class PagedLayout:
    """A workload's K/V placed in a pool of token slots, for the paged entry points.

    k_pool / v_pool [num_slots, Hkv, D]; block_table [B, max_pages] names each sequence's pages
    (page_size positions each, physical pages in shuffled order, -1 past the prefix);
    tree_slot [B, T] names each tree node's slot (shuffled, after the prefix pages); the last
    ``spare`` slots are unused (room the free list can hand out)."""
    page_size: int
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_table: np.ndarray
    tree_slot: np.ndarray
    num_slots: int
    max_pages: int


def make_paged(w: "Workload", page_size: int, seed: int = 0, headroom: int | None = None,
               spare: int = 0) -> PagedLayout:
    """Place w's prefix rows and tree rows into a pool.  Pure data placement: slot and page
    numbers come from a seeded permutation; no value is computed.  ``headroom`` positions past
    each prefix get table room (default T, enough to commit a whole path)."""
    rng = np.random.default_rng(np.random.SeedSequence([w.spec.wid, 7, seed]))
    P = int(page_size)
    B, T, Hkv, D = w.B, w.T, w.Hkv, w.D
    L = np.clip(w.cache_len, 0, w.Lmax).astype(np.int64)
    headroom = T if headroom is None else headroom
    n_pages = [int(-(-int(x) // P)) for x in L]
    total_pages = sum(n_pages)
    max_pages = max(1, max(-(-(int(x) + headroom) // P) for x in L))
    phys = rng.permutation(total_pages)
    num_slots = total_pages * P + B * T + spare
    k_pool = np.zeros((num_slots, Hkv, D), w.k_cache.dtype)
    v_pool = np.zeros_like(k_pool)
    table = np.full((B, max_pages), -1, np.int32)
    nxt = 0
    for b in range(B):
        pages = phys[nxt:nxt + n_pages[b]]
        nxt += n_pages[b]
        table[b, :n_pages[b]] = pages
        if n_pages[b] == 0:
            continue
        pos = np.arange(int(L[b]))
        slots = pages[pos // P] * P + pos % P
        k_pool[slots] = w.k_cache[b, :, :L[b]].transpose(1, 0, 2)
        v_pool[slots] = w.v_cache[b, :, :L[b]].transpose(1, 0, 2)
    tree_slot = (total_pages * P + rng.permutation(B * T)).reshape(B, T).astype(np.int32)
    k_pool[tree_slot.reshape(-1)] = w.k_tree.reshape(B * T, Hkv, D)
    v_pool[tree_slot.reshape(-1)] = w.v_tree.reshape(B * T, Hkv, D)
    return PagedLayout(P, k_pool, v_pool, table, tree_slot, num_slots, max_pages)


STREAM_DIST = 5  # seed stream of the next-token distributions


@dataclasses.dataclass
class StochasticInputs:
    """Inputs of sampling-mode acceptance for a workload's trees.

    p / q [B, T, V] float32: the target and draft models' next-token distributions after every
    node; draft [B, T] int32: each non-root node's token, drawn from its parent's q
    (independently, or without replacement among siblings); u_acc / u_res [B, T] float64: the
    uniforms the acceptance tests and the bonus draws consume."""
    V: int
    without_replacement: bool
    p: np.ndarray
    q: np.ndarray
    draft: np.ndarray
    u_acc: np.ndarray
    u_res: np.ndarray


def make_stochastic(w: "Workload", V: int | None = None, without_replacement: bool = False,
                    seed: int = 0, spread: float = 2.0, draft_noise: float = 0.7,
                    peak: tuple[float, float] = (-2.0, 4.0)) -> StochasticInputs:
    """Next-token distributions and drafted tokens for w's tree shapes.  Pure input synthesis:
    target logits are N(0, spread^2) plus one to three peaked tokens raised by
    ln V + spread^2 / 2 + U(peak) (so the peak's share ranges from about 0.1 to 0.98, as in an
    LLM's sampling distribution); draft logits add N(0, draft_noise^2) noise to the target's.
    Both go through a softmax (float32 exponentials, float64 row sums) and are stored as
    float32.  The children of every node
    then draw their tokens from that node's draft distribution."""
    V = int(V or w.spec.vocab)
    B, T = w.B, w.T
    p = np.empty((B, T, V), np.float32)
    q = np.empty((B, T, V), np.float32)
    draft = np.zeros((B, T), np.int32)
    u_acc = np.empty((B, T), np.float64)
    u_res = np.empty((B, T), np.float64)
    lift = math.log(V) + 0.5 * spread * spread
    for b in range(B):
        rng = _rng(w.spec.wid, b, STREAM_DIST, seed)
        z = rng.standard_normal((T, V), dtype=np.float32) * np.float32(spread)
        for t in range(T):
            k = int(rng.integers(1, 4))
            z[t, rng.integers(0, V, size=k)] += np.float32(lift) + rng.uniform(*peak, size=k).astype(np.float32)
        zd = z + rng.standard_normal((T, V), dtype=np.float32) * np.float32(draft_noise)
        for src, dst in ((z, p), (zd, q)):
            e = np.exp(src - src.max(axis=1, keepdims=True))
            dst[b] = e / e.sum(axis=1, keepdims=True, dtype=np.float64)
        par = w.parent[b]
        for u in range(T):
            kids = [c for c in range(u + 1, T) if par[c] == u]
            if not kids:
                continue
            qu = q[b, u].astype(np.float64)
            qu /= qu.sum()
            draft[b, kids] = rng.choice(V, size=len(kids), replace=not without_replacement, p=qu)
        u_acc[b] = rng.random(T)
        u_res[b] = rng.random(T)
    return StochasticInputs(V, bool(without_replacement), p, q, draft, u_acc, u_res)


STREAM_DRAFTER = 6  # seed stream of the drafter outputs for device-side tree construction


@dataclasses.dataclass
class DraftLevels:
    """Drafter outputs consumed by EAGLE-2 tree construction, level by level.

    root_tok [B] int32: the root token of each sequence.  child_tok / child_conf
    [depth, B, k, branch] (int32, float32): at level l, the candidate children the drafter
    proposes for frontier slot r of sequence b (the root alone is slot 0 of level 1), with
    their confidences, best first as a top-`branch` returns them.  Sibling tokens are distinct.
    The drafter is synthetic, so its output for a slot does not depend on which node sits in
    that slot."""
    depth: int
    k: int
    branch: int
    root_tok: np.ndarray
    child_tok: np.ndarray
    child_conf: np.ndarray


def make_draft_levels(spec: WorkloadSpec | str, B: int | None = None, depth: int | None = None,
                      k: int | None = None, branch: int | None = None, seed: int = 0,
                      vocab: int | None = None, variance: float = 2.0) -> DraftLevels:
    """Seeded drafter outputs with a workload's expansion shape (overridable).  Each slot's
    confidences are the softmax (float64, stored float32) of `branch` N(0, variance) logits,
    the recipe of the workload trees; tokens are distinct draws from the vocabulary."""
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    B = spec.B if B is None else B
    depth = spec.depth_max if depth is None else depth
    k = spec.topk if k is None else k
    branch = spec.branch if branch is None else branch
    vocab = spec.vocab if vocab is None else vocab
    if min(depth, k, branch) < 1 or branch > vocab:
        raise ValueError("expansion shape needs depth, k, branch >= 1 and branch <= vocab")
    root = np.empty(B, np.int32)
    tok = np.empty((depth, B, k, branch), np.int32)
    conf = np.empty((depth, B, k, branch), np.float32)
    sd = math.sqrt(variance)
    for b in range(B):
        rng = _rng(spec.wid, b, STREAM_DRAFTER, seed)
        root[b] = rng.integers(0, vocab)
        logits = rng.normal(0.0, sd, size=(depth, k, branch))
        e = np.exp(logits - logits.max(axis=-1, keepdims=True))
        conf[:, b] = -np.sort(-(e / e.sum(axis=-1, keepdims=True)), axis=-1)
        for l in range(depth):
            for r in range(k):
                while True:
                    t = rng.integers(0, vocab, size=branch)
                    if len(np.unique(t)) == branch:
                        break
                tok[l, b, r] = t
    return DraftLevels(depth, k, branch, root, tok, conf)


STREAM_LM = 7  # seed stream of the drafter LM head's weights and hidden states


@dataclasses.dataclass
class LmHeadInputs:
    """Synthetic drafter LM head (bfloat16 bit patterns).

    h [M, d]: hidden states.  A [n, r]: the low-rank head's rows in shuffled order, row q
    belonging to token row_token[q] ([n] int32, a permutation).  B [r, d].  W [n, d]: the full
    head in token order, W = A_tok B plus full-rank noise, so the low-rank screening scores
    approximate the logits.  tile, k_tile, K: screening tile, candidates per tile, children."""
    name: str
    M: int
    d: int
    n: int
    r: int
    tile: int
    k_tile: int
    K: int
    h: np.ndarray
    A: np.ndarray
    B: np.ndarray
    W: np.ndarray
    row_token: np.ndarray


LM_HEADS = {
    # one EAGLE-2 expansion level at batch 1: the 10 frontier nodes' hidden states through a
    # Llama-3-8B-sized head (hidden 4096, vocabulary 128256), rank 256, tiles of 256 rows with
    # 4 candidates each (2004 candidates), 10 children per node
    "llama8b_head_M10": dict(wid=20, M=10, d=4096, n=LLAMA3_VOCAB, r=256, tile=256, k_tile=4,
                             K=10),
    # the same head for 64 hidden states at once (e.g. 64 sequences drafting one token each)
    "llama8b_head_M64": dict(wid=21, M=64, d=4096, n=LLAMA3_VOCAB, r=256, tile=256, k_tile=4,
                             K=10),
}


def make_lm_head(name: str = "llama8b_head_M10", seed: int = 0, noise: float = 1.0,
                 **override) -> LmHeadInputs:
    """Seeded drafter head.  h ~ N(0, 1); B ~ N(0, 1/d) so u = B h is about N(0, 1); the
    token-order factor A_tok ~ N(0, 9/r) so screening scores are about N(0, 9); W = A_tok B + E
    with E uniform of variance noise^2/d, so an exact logit is the screening score plus
    noise of variance about noise^2.  Rows of A are shuffled by a seeded permutation.
    `override` changes M, d, n, r, tile, k_tile or K (tests use small heads)."""
    cfg = dict(LM_HEADS[name])
    cfg.update(override)
    M, d, n, r = cfg["M"], cfg["d"], cfg["n"], cfg["r"]
    rng = _rng(cfg["wid"], 0, STREAM_LM, seed)
    h = rng.standard_normal((M, d), dtype=np.float32)
    Bf = rng.standard_normal((r, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    A_tok = rng.standard_normal((n, r), dtype=np.float32) * np.float32(3.0 / math.sqrt(r))
    perm = rng.permutation(n).astype(np.int32)
    W = np.empty((n, d), np.uint16)
    step = 8192
    for i0 in range(0, n, step):
        blk = A_tok[i0:i0 + step] @ Bf
        e = rng.random(blk.shape, dtype=np.float32)
        e -= np.float32(0.5)
        e *= np.float32(noise * math.sqrt(12.0 / d))
        blk += e
        # round to nearest even bfloat16 in place (the values are finite): as f32_to_bf16_bits
        u = blk.view(np.uint32)
        t = e.view(np.uint32)
        np.right_shift(u, np.uint32(16), out=t)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += u
        t >>= np.uint32(16)
        W[i0:i0 + step] = t
    return LmHeadInputs(name, M, d, n, r, cfg["tile"], cfg["k_tile"], cfg["K"],
                        f32_to_bf16_bits(h), f32_to_bf16_bits(A_tok[perm]), f32_to_bf16_bits(Bf),
                        W, perm)
