"""GPU parity of tree_accept_stochastic (rejection sampling over the draft tree) against the CPU
oracle, through the C ABI.

The kernel and the oracle take every decision in fp64 on the same float32 distributions and
fp64 uniforms, so the accepted path, its length, the bonus token and the status bits must agree
exactly.  (They sum the vocabulary in different orders; a decision could only differ if a
uniform fell within ~1e-13 of a threshold, which none of these seeded inputs does.)
"""
import numpy as np
import pytest
import torch

import pins
from gpu_util import to_dev, to_host
from synth import make_stochastic, make_workload, worked_tree_parent

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _check(parent, draft, p, q, u_acc, u_res, mode, label, p_dev=None, q_dev=None, G=0,
           workspace=None):
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    B, T = draft.shape
    V = p.shape[-1]
    print(f"[case] stochastic {label} B={B} T={T} V={V} mode={mode} G={G}", flush=True)
    anc, st = tv.tree_build_mask(to_dev(np.asarray(parent, np.int32)))
    status = torch.zeros(B, dtype=torch.int32, device="cuda")
    path, n, bonus = tv.tree_accept_stochastic(
        anc, to_dev(np.asarray(draft, np.int32)), to_dev(p) if p_dev is None else p_dev,
        to_dev(q) if q_dev is None else q_dev, to_dev(np.asarray(u_acc, np.float64)),
        to_dev(np.asarray(u_res, np.float64)), without_replacement=mode, workgroups_per_seq=G,
        workspace=workspace, status=status)
    torch.cuda.synchronize()
    o_path, o_n, o_bonus, o_st = O.accept_stochastic(parent, draft, p, q, u_acc, u_res, mode)
    g_path, g_n, g_bonus, g_st = to_host(path), to_host(n), to_host(bonus), to_host(status)
    assert np.array_equal(g_n, o_n), (label, g_n, o_n)
    assert np.array_equal(g_path, o_path), label
    assert np.array_equal(g_bonus, o_bonus), (label, g_bonus, o_bonus)
    assert np.array_equal(g_st, o_st), (label, g_st, o_st)
    print(f"       mean accept_len {o_n.mean():.2f}", flush=True)
    return o_path, o_n, o_bonus


def test_hand_cases():
    parent = worked_tree_parent()[None]
    for name, mode, draft, p, q, u_acc, u_res, want_path, want_bonus in pins.read_stochastic_cases():
        path, n, bonus = _check(parent, np.array([draft]), p[None].astype(np.float32),
                                q[None].astype(np.float32), np.array([u_acc]),
                                np.array([u_res]), mode, name)
        assert list(path[0, : n[0]]) == want_path and bonus[0] == want_bonus, name


def test_duplicate_siblings():
    parent = np.array([[-1, 0, 0, 0]], np.int32)
    draft = np.array([[0, 0, 0, 1]], np.int32)
    p = np.full((1, 4, 4), 0.25, np.float32)
    q = p.copy()
    p[0, 0] = [0.25, 0.25, 0.375, 0.125]
    q[0, 0] = [0.5, 0.125, 0.125, 0.25]
    for mode in (0, 1):
        _check(parent, draft, p, q, np.array([[0.5, 0.75, 0.5, 0.9]]), np.full((1, 4), 0.5), mode,
               "duplicate siblings")


CASES = [  # label, B, T, V, parent kind, draft noise
    ("root_only", 2, 1, 37, "random", 0.7),
    ("two_nodes", 3, 2, 8, "random", 0.7),
    ("eagle_like", 4, 60, 1000, "random", 0.7),
    ("two_words_scalar_path", 3, 65, 4099, "random", 1.5),
    ("t128_v32000", 2, 128, 32000, "random", 0.7),
    ("star_many_rejections", 3, 40, 257, "star", 3.5),
    ("chain", 2, 30, 5000, "chain", 1.0),
    ("tiny_vocab", 6, 128, 5, "random", 1.0),
]


@pytest.mark.parametrize("label,B,T,V,kind,noise", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("G", [0, 3])
def test_random_trees(label, B, T, V, kind, noise, mode, G):
    w = make_workload("batch32_L512-4096_T60", B=B, T=T, L=(0, 8), Hq=2, Hkv=1, D=64,
                      dtype="f32", parent_kind=kind, extra_seed=31, with_kv=False)
    if mode and max(np.bincount(w.parent[w.parent >= 0], minlength=1).max(), 0) > V:
        pytest.skip("more siblings than tokens to draw without replacement")
    s = make_stochastic(w, V=V, without_replacement=mode, seed=7, draft_noise=noise)
    _check(w.parent, s.draft, s.p, s.q, s.u_acc, s.u_res, mode, label, G=G)


def test_edge_distributions():
    """Zero-mass rows, unnormalised p (empty residual), q = p, one-hot p, uniforms close to one,
    and out-of-vocabulary child tokens."""
    rng = np.random.default_rng(5)
    w = make_workload("batch32_L512-4096_T60", B=6, T=24, L=(0, 8), Hq=2, Hkv=1, D=64,
                      dtype="f32", parent_kind="random", extra_seed=32, with_kv=False)
    for mode in (0, 1):
        s = make_stochastic(w, V=300, without_replacement=mode, seed=8, draft_noise=1.5)
        p, q, draft = s.p.copy(), s.q.copy(), s.draft.copy()
        u_acc, u_res = s.u_acc.copy(), s.u_res.copy()
        p[0, :, :] = 0.0                      # sequence 0: no target mass anywhere -> bonus -1
        p[1] *= 0.5                           # sequence 1: p sums to 1/2 (empty residuals)
        q[2] = p[2]                           # sequence 2: q = p, every tried child kept
        hot = rng.integers(0, 300, size=24)   # sequence 3: one-hot targets
        p[3] = 0.0
        p[3, np.arange(24), hot] = 1.0
        u_acc[4] = 1.0 - 2.0 ** -30           # sequence 4: almost every child rejected
        u_res[4] = 1.0 - 2.0 ** -30
        draft[5, 1::3] = 300                  # sequence 5: some tokens outside the vocabulary
        draft[5, 2::5] = -3
        for G in (1, 4):
            _check(w.parent, draft, p, q, u_acc, u_res, mode, "edge distributions", G=G)


def test_unaligned_rows_use_the_scalar_path():
    import tree_attention_verification_attn_amd as tv  # noqa: F401

    w = make_workload("batch32_L512-4096_T60", B=3, T=20, L=(0, 8), Hq=2, Hkv=1, D=64,
                      dtype="f32", parent_kind="random", extra_seed=33, with_kv=False)
    s = make_stochastic(w, V=512, seed=9, draft_noise=1.5)
    n = s.p.size
    flat_p = torch.empty(n + 1, dtype=torch.float32, device="cuda")
    flat_q = torch.empty(n + 1, dtype=torch.float32, device="cuda")
    p_dev = flat_p[1:].view(s.p.shape)  # 4 bytes off a 16-byte boundary
    q_dev = flat_q[1:].view(s.q.shape)
    p_dev.copy_(torch.from_numpy(s.p))
    q_dev.copy_(torch.from_numpy(s.q))
    _check(w.parent, s.draft, s.p, s.q, s.u_acc, s.u_res, 0, "unaligned", p_dev=p_dev, q_dev=q_dev)


@pytest.mark.parametrize("name,mode,G", [("llama8b_b1_L4096_T60", 0, 0), ("llama8b_b1_L4096_T60", 1, 0),
                                         ("llama8b_b1_L4096_T60", 0, 1),
                                         ("batch32_L512-4096_T60", 0, 0)])
def test_full_size(name, mode, G):
    """The workloads' own trees with a Llama-3-sized vocabulary (128256), as the bench runs
    (automatic split: 32 workgroups per sequence at batch 1, 8 at batch 32)."""
    w = make_workload(name, with_kv=False)
    s = make_stochastic(w, without_replacement=mode)
    _check(w.parent, s.draft, s.p, s.q, s.u_acc, s.u_res, mode, name, G=G)


def test_workspace_is_left_zero_and_reusable():
    """Calls that share a workspace: each leaves it all zeros, and repeated calls agree."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=5, T=60, L=(0, 8), Hq=2, Hkv=1, D=64,
                      dtype="f32", parent_kind="random", extra_seed=34, with_kv=False)
    s = make_stochastic(w, V=40000, seed=10, draft_noise=2.5)
    G = 6
    need = tv.tree_accept_stochastic_workspace_size(w.B, w.T, s.V, G)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = None
    for rep in range(3):
        out = _check(w.parent, s.draft, s.p, s.q, s.u_acc, s.u_res, 0, f"reuse {rep}", G=G,
                     workspace=ws)
        assert int(torch.count_nonzero(ws)) == 0
        if first is None:
            first = out
        assert all(np.array_equal(x, y) for x, y in zip(out, first))
