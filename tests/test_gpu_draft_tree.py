"""GPU parity of EAGLE-2 tree construction (eagle2_expand per level, then eagle2_rerank) against
the CPU oracle, through the C ABI.

Both sides rank nodes by the same float32 path products (parent value times confidence,
rounded to nearest even) with ties to the smaller node id, so the node tables (values compared
as bits), every level's frontier, the flattened tree and the status bits must agree exactly.
"""
import numpy as np
import pytest
import torch

import pins
from gpu_util import to_dev, to_host
from synth import make_draft_levels

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def run_device(root, tok, conf, T, n_max=None, corrupt=None):
    """Every expansion level, then the rerank, on the device.  `corrupt(level, table)` may edit
    the table between levels.  Returns host copies of the table, per-level frontiers, outputs
    and status."""
    import tree_attention_verification_attn_amd as tv

    depth, B, k, branch = tok.shape
    N = tv.eagle2_node_count(depth, k, branch)
    table = tv.eagle2_new_table(B, n_max or N, k, "cuda")
    tok_d, conf_d, root_d = to_dev(tok), to_dev(conf), to_dev(np.asarray(root, np.int32))
    fronts = []
    for lvl in range(1, depth + 1):
        if corrupt is not None:
            corrupt(lvl, table)
        tv.eagle2_expand(table, lvl, tok_d[lvl - 1], conf_d[lvl - 1],
                         root_tok=root_d if lvl == 1 else None)
        fronts.append(table["frontier"].clone())
    out = tv.eagle2_rerank(table, N, T)
    torch.cuda.synchronize()
    r = {name: to_host(t)[:, :N] for name, t in table.items()
         if name in ("node_tok", "node_parent", "node_value")}
    r["frontier"] = np.stack([to_host(f) for f in fronts])
    r["status"] = to_host(table["status"])
    r.update({name: to_host(t) for name, t in out.items()})
    return r


def check(root, tok, conf, T, label, n_max=None):
    from oracle import oracle as O

    depth, B, k, branch = tok.shape
    print(f"[case] draft tree {label} B={B} depth={depth} k={k} branch={branch} T={T}", flush=True)
    g = run_device(root, tok, conf, T, n_max=n_max)
    o = O.eagle2_build(root, tok, conf, T)
    for name in ("node_tok", "node_parent", "frontier", "parent", "tok", "depth", "node",
                 "status"):
        assert np.array_equal(g[name], o[name]), (label, name)
    assert np.array_equal(g["node_value"].view(np.uint32), o["node_value"].view(np.uint32)), label
    return g


def test_hand_case():
    gd = pins.read_eagle2_case()
    for T, nodes, parents, depths, toks in gd["cases"]:
        g = check(np.array([gd["root"]]), gd["tok"], gd["conf"], T, f"hand T={T}")
        assert list(g["node"][0]) == nodes and list(g["parent"][0]) == parents
        assert list(g["depth"][0]) == depths and list(g["tok"][0]) == toks


def test_random_small():
    rng = np.random.default_rng(21)
    for trial in range(40):
        depth, k, branch = (int(rng.integers(1, 5)), int(rng.integers(1, 6)),
                            int(rng.integers(1, 6)))
        from oracle import oracle as O

        N = O.eagle2_node_count(depth, k, branch)
        T = int(rng.integers(1, min(N, 128) + 1))
        B = int(rng.integers(1, 4))
        root, tok, conf = pins._e2_inputs(rng, B, depth, k, branch, ties=trial % 3 == 0)
        check(root, tok, conf, T, f"random {trial}")


@pytest.mark.parametrize("name", ["llama8b_b1_L4096_T60", "batch32_L512-4096_T60",
                                  "llama70b_b8_L32768_T64", "wide_b64_L1024-8192_T128"])
def test_workload_shapes(name):
    from synth import WORKLOADS

    d = make_draft_levels(name)
    g = check(d.root_tok, d.child_tok, d.child_conf, WORKLOADS[name].T, name)
    assert (g["status"] == 0).all()


def test_equal_confidences():
    d = make_draft_levels("wide_b64_L1024-8192_T128", B=4)
    conf = np.full_like(d.child_conf, 0.5)
    g = check(d.root_tok, d.child_tok, conf, 128, "equal confidences")
    assert (g["node"] == np.arange(128)).all()


def test_quantised_ties():
    d = make_draft_levels("llama8b_b1_L4096_T60", B=6, seed=3)
    conf = np.clip(np.round(d.child_conf * 8) / 8, 0.125, 1.0).astype(np.float32)
    check(d.root_tok, d.child_tok, conf, 60, "confidences in eighths")


def test_tiny_and_subnormal_values():
    d = make_draft_levels("llama70b_b8_L32768_T64", B=3, seed=4)
    conf = d.child_conf.copy()
    conf[1:, :, :, 1::2] = 1e-20  # two levels of these give 1e-40, a float32 subnormal
    conf[3, 1] = 3e-39            # subnormal confidences
    conf[5, 2, :, :3] = 0.0
    g = check(d.root_tok, d.child_tok, conf, 64, "tiny and subnormal")
    v = g["node_value"]
    assert ((v > 0) & (v < np.finfo(np.float32).tiny)).any()


def test_bad_confidences():
    from tree_attention_verification_attn_amd import TV_BAD_CONF

    d = make_draft_levels("llama8b_b1_L4096_T60", B=3, seed=5)
    conf = d.child_conf.copy()
    conf[0, 0, 0, 1] = np.nan
    conf[1, 0, 2, 0] = -0.5
    conf[2, 0, 0, 2] = 1.5
    conf[3, 0, 1, 1] = np.inf
    conf[1, 2, 0, 3] = -0.0
    g = check(d.root_tok, d.child_tok, conf, 60, "bad confidences")
    assert list(g["status"]) == [TV_BAD_CONF, 0, 0]


def test_degenerate_shapes():
    rng = np.random.default_rng(22)
    from oracle import oracle as O

    cases = [(3, 4, 3, 1), (2, 3, 5, 21), (20, 4, 1, 21), (1, 1, 1, 1), (1, 1, 7, 8),
             (5, 2, 2, 11)]
    for depth, k, branch, T in cases:
        N = O.eagle2_node_count(depth, k, branch)
        root, tok, conf = pins._e2_inputs(rng, 2, depth, k, branch)
        check(root, tok, conf, min(T, N), f"shape {depth}/{k}/{branch}")
    # a row stride larger than the table
    root, tok, conf = pins._e2_inputs(rng, 3, 3, 3, 3)
    check(root, tok, conf, 20, "padded rows", n_max=77)


def test_largest_shapes():
    rng = np.random.default_rng(23)
    for depth, k, branch, T in ((4, 32, 32, 128), (1, 1, 1024, 100), (16, 64, 16, 128)):
        root, tok, conf = pins._e2_inputs(rng, 2, depth, k, branch, vocab=128256)
        check(root, tok, conf, T, f"large {depth}/{k}/{branch}")


def test_bad_frontier_entries():
    """A frontier entry that is not a node of the previous level: its slot's children get parent
    -1 and value 0, TV_BAD_TREE is set, and the rerank rejects the table exactly as the oracle's
    rerank does on the same table."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    d = make_draft_levels("llama8b_b1_L4096_T60", B=3, seed=6)

    def corrupt(lvl, table):
        if lvl == 3:
            table["frontier"][1, 2] = 5   # a level-1 node, not of level 2
            table["frontier"][2, 0] = -7

    g = run_device(d.root_tok, d.child_tok, d.child_conf, 60, corrupt=corrupt)
    assert list(g["status"]) == [0, tv.TV_BAD_TREE, tv.TV_BAD_TREE]
    base = tv.eagle2_node_count(2, 10, 10)
    for b, slot in ((1, 2), (2, 0)):
        kids = slice(base + slot * 10, base + slot * 10 + 10)
        assert (g["node_parent"][b, kids] == -1).all() and (g["node_value"][b, kids] == 0).all()
    o = O.eagle2_rerank(g["node_tok"], g["node_parent"], g["node_value"], 60)
    for name in ("parent", "tok", "depth", "node"):
        assert np.array_equal(g[name], o[name]), name
    assert list(o["status"]) == [0, O.ORC_BAD_TREE, O.ORC_BAD_TREE]


def _rerank_both(ntok, npar, nval, T, label):
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    B, N = ntok.shape
    print(f"[case] rerank {label} B={B} N={N} T={T}", flush=True)
    table = {"node_tok": to_dev(ntok), "node_parent": to_dev(npar), "node_value": to_dev(nval),
             "status": torch.zeros(B, dtype=torch.int32, device="cuda")}
    out = tv.eagle2_rerank(table, N, T)
    torch.cuda.synchronize()
    o = O.eagle2_rerank(ntok, npar, nval, T)
    for name in ("parent", "tok", "depth", "node"):
        assert np.array_equal(to_host(out[name]), o[name]), (label, name)
    assert np.array_equal(to_host(table["status"]), o["status"]), label
    return o


def _random_table(rng, N, steps=(0.25, 0.5, 0.75, 1.0), kind="random"):
    if kind == "chain":
        par = np.arange(-1, N - 1, dtype=np.int32)
    else:
        par = np.array([-1] + [int(rng.integers(max(0, i - 40), i)) for i in range(1, N)],
                       np.int32)
    val = np.ones(N, np.float32)
    for i in range(1, N):
        val[i] = np.float32(val[par[i]] * np.float32(rng.choice(steps)))
    return rng.integers(0, 128256, size=N).astype(np.int32), par, val


def test_rerank_caller_tables():
    rng = np.random.default_rng(24)
    for N, T, kind in ((30, 12, "random"), (500, 128, "random"), (16384, 128, "random"),
                       (200, 128, "chain"), (128, 128, "random"), (7, 1, "random")):
        tabs = [_random_table(rng, N, kind=kind) for _ in range(3)]
        ntok, npar, nval = (np.stack(x) for x in zip(*tabs))
        _rerank_both(ntok, npar, nval, T, f"{kind} N={N}")
    # continuous values (few ties) and NaN / negative values counted as zero
    ntok, npar, nval = (np.stack(x) for x in zip(*[_random_table(
        rng, 300, steps=tuple(rng.uniform(0.2, 1.0, size=32))) for _ in range(2)]))
    nval[0, 250:] = np.nan
    nval[1, 200:260] = -1.0
    _rerank_both(ntok, npar, nval, 100, "NaN and negative values")


def test_rerank_invalid_tables():
    rng = np.random.default_rng(25)
    ntok, npar, nval = _random_table(rng, 300)
    bads = []
    p = npar.copy(); p[0] = 0; bads.append((p, nval))
    p = npar.copy(); p[77] = 77; bads.append((p, nval))
    p = npar.copy(); p[120] = 299; bads.append((p, nval))
    p = npar.copy(); p[50] = -1; bads.append((p, nval))
    v = nval.copy(); v[200] = v[npar[200]] * 1.5; bads.append((npar, v))
    for i, (p, v) in enumerate(bads):
        o = _rerank_both(np.stack([ntok, ntok]), np.stack([npar, p]), np.stack([nval, v]), 64,
                         f"invalid {i}")
        assert o["status"][1] != 0 and o["status"][0] == 0


def test_construction_feeds_verification():
    """The flattened trees are valid level-ordered trees: tree_build_mask accepts them and
    gives the oracle's masks."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    d = make_draft_levels("wide_b64_L1024-8192_T128", B=8, seed=7)
    g = run_device(d.root_tok, d.child_tok, d.child_conf, 128)
    anc, st = tv.tree_build_mask(to_dev(g["parent"]))
    torch.cuda.synchronize()
    o_anc, o_st = O.build_mask(g["parent"])
    assert (to_host(st) == 0).all() and (o_st == 0).all()
    assert np.array_equal(to_host(anc).view(np.uint64), o_anc)
    # a node's depth is the number of its ancestors: the mask's popcount minus one
    for b in range(8):
        for f in range(128):
            assert sum(bin(int(x)).count("1") for x in o_anc[b, f]) - 1 == g["depth"][b, f]
