"""GPU parity of the two-stage drafter LM head (lm_head_project, lm_head_screen,
lm_head_rescore, lm_head_topk) against the CPU oracle, through the C ABI.

Both sides compute every value that chooses a candidate or a child in float32 in the same
stated order (fused multiply-add chains; 64 segments combined by a fixed butterfly), so u,
the candidate tokens, their scores, the exact logits and the children must agree exactly.  The
confidences come from fp32 sums on the GPU and fp64 in the oracle: relative error <= 1e-5.
"""
import numpy as np
import pytest
import torch

import pins
from gpu_util import to_dev, to_host
from synth import bf16_bits_to_f32, make_lm_head

pytestmark = pytest.mark.gpu

TOL_CONF = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def run_both(h, A, Bm, W, perm, tile, k_tile, K, label, rows=None, cand_override=None):
    """Device and oracle two-stage heads on the same bits; `rows` limits the oracle (and the
    comparison) to some hidden states."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    M = h.shape[0]
    print(f"[case] lm head {label} M={M} d={h.shape[1]} n={A.shape[0]} r={A.shape[1]} "
          f"tile={tile} k_tile={k_tile} K={K}", flush=True)
    hd, Ad, Bd, Wd = (to_dev(x).view(torch.bfloat16) for x in (h.view(np.int16),
                                                                 A.view(np.int16),
                                                                 Bm.view(np.int16),
                                                                 W.view(np.int16)))
    status = torch.zeros(M, dtype=torch.int32, device="cuda")
    u = tv.lm_head_project(hd, Bd)
    cand, score = tv.lm_head_screen(Ad, u, to_dev(perm), tile, k_tile)
    if cand_override is not None:
        cand = to_dev(cand_override)
    logits = tv.lm_head_rescore(Wd, hd, cand, status=status)
    tok, conf = tv.lm_head_topk(logits, cand, K, W.shape[0])
    torch.cuda.synchronize()
    g = dict(u=to_host(u), cand=to_host(cand), cand_score=to_host(score), logits=to_host(logits),
             tok=to_host(tok), conf=to_host(conf), status=to_host(status))
    sel = np.arange(M) if rows is None else np.asarray(rows)
    o_u = O.lm_project(h[sel], Bm)
    assert np.array_equal(g["u"][sel].view(np.uint32), o_u.view(np.uint32)), label
    o_cand, o_score = O.lm_screen(A, o_u, perm, tile, k_tile)
    if cand_override is None:
        assert np.array_equal(g["cand"][sel], o_cand), label
        assert np.array_equal(g["cand_score"][sel], o_score), label
        c_use = o_cand
    else:
        c_use = cand_override[sel]
    o_logits, o_st = O.lm_rescore(W, h[sel], c_use)
    assert np.array_equal(g["logits"][sel].view(np.uint32), o_logits.view(np.uint32)), label
    assert np.array_equal(g["status"][sel], o_st), label
    o_tok, o_conf = O.lm_topk(o_logits, c_use, K, W.shape[0])
    assert np.array_equal(g["tok"][sel], o_tok), label
    err = np.abs(g["conf"][sel].astype(np.float64) - o_conf) / np.maximum(o_conf, 1e-30)
    assert (err[o_conf > 0] <= TOL_CONF).all() and (g["conf"][sel][o_conf == 0] == 0).all(), \
        (label, err.max())
    return g


def _rand(rng, shape, scale=1.0):
    return pins._bits(rng.standard_normal(shape) * scale)


def test_random_small():
    rng = np.random.default_rng(41)
    for trial in range(16):
        M = int(rng.integers(1, 13))
        d = 512 * int(rng.integers(1, 3))
        r = 8 * int(rng.integers(1, 40))
        n = int(rng.integers(50, 3000))
        tile = int(rng.choice([1, 7, 64, 100, 256]))
        k_tile = int(rng.integers(1, min(16, tile) + 1))
        K = int(rng.integers(1, 65))
        h, Bm = _rand(rng, (M, d)), _rand(rng, (r, d), 1 / np.sqrt(d))
        A, W = _rand(rng, (n, r)), _rand(rng, (n, d), 1 / np.sqrt(d))
        perm = rng.permutation(n).astype(np.int32)
        run_both(h, A, Bm, W, perm, tile, k_tile, K, f"random {trial}")


def test_small_integers_ties():
    """Integer-valued inputs: scores and logits tie often, exercising both tie rules."""
    rng = np.random.default_rng(42)
    for trial in range(6):
        M, d, r, n = 5, 512, 16, 700
        h, Bm, A, W, perm = pins._int_lm_case(rng, M, d, r, n, lo=-2, hi=3)
        run_both(pins._bits(h), pins._bits(A[perm]), pins._bits(Bm), pins._bits(W), perm, 64, 5,
                 12, f"integers {trial}")


def test_every_hidden_state_count():
    """Each compile-time chain count of the screening kernel (M rounded up to 2, 4, 6, 8, 10,
    12, 16, 24, 32, 48, 64)."""
    rng = np.random.default_rng(43)
    d, r, n = 512, 64, 900
    Bm, A, W = _rand(rng, (r, d), 1 / np.sqrt(d)), _rand(rng, (n, r)), _rand(rng, (n, d), 0.05)
    perm = rng.permutation(n).astype(np.int32)
    for M in (1, 3, 5, 7, 9, 11, 13, 17, 25, 33, 49, 64):
        run_both(_rand(rng, (M, d)), A, Bm, W, perm, 128, 3, 8, f"M={M}")


def test_padding_bad_tokens_and_short_lists():
    import tree_attention_verification_attn_amd as tv

    rng = np.random.default_rng(44)
    M, d, r, n = 3, 512, 32, 301  # tiles of 100 rows: the last one has a single row
    h, Bm = _rand(rng, (M, d)), _rand(rng, (r, d), 0.05)
    A, W = _rand(rng, (n, r)), _rand(rng, (n, d), 0.05)
    perm = rng.permutation(n).astype(np.int32)
    g = run_both(h, A, Bm, W, perm, 100, 4, 5, "padding")
    assert (g["cand"][:, -3:] == -1).all() and np.isneginf(g["cand_score"][:, -3:]).all()
    # bad candidates, and more children asked for than valid candidates
    bad = g["cand"].copy()
    bad[0, 0], bad[1, 2], bad[2, :] = n, -9, -1
    bad[2, 5] = int(perm[0])
    g2 = run_both(h, A, Bm, W, perm, 100, 4, 16, "bad tokens", cand_override=bad)
    assert list(g2["status"]) == [tv.TV_BAD_TOKEN, tv.TV_BAD_TOKEN, 0]
    assert g2["tok"][2, 0] == perm[0] and (g2["tok"][2, 1:] == -1).all()
    assert abs(g2["conf"][2, 0] - 1.0) <= 1e-6


@pytest.mark.parametrize("name", ["llama8b_head_M10", "llama8b_head_M64"])
def test_workload_full_size(name):
    x = make_lm_head(name)
    rows = None if x.M <= 10 else [0, 1, 17, 31, 32, 47, 62, 63]
    g = run_both(x.h, x.A, x.B, x.W, x.row_token, x.tile, x.k_tile, x.K, name, rows=rows)
    # the screening keeps most of the full head's best tokens (the synthetic head is close to
    # low rank): recall of the exact top 10 among the children
    full = bf16_bits_to_f32(x.W) @ bf16_bits_to_f32(x.h[:4]).T
    for m in range(4):
        top = set(np.argsort(-full[:, m])[:10].tolist())
        assert len(top & set(g["tok"][m].tolist())) >= 8


def test_children_feed_the_expansion():
    """The children of the frontier's hidden states are a valid expansion level."""
    import tree_attention_verification_attn_amd as tv

    rng = np.random.default_rng(45)
    k, branch, d, r, n = 10, 10, 512, 64, 5000
    h, Bm = _rand(rng, (k, d)), _rand(rng, (r, d), 1 / np.sqrt(d))
    A, W = _rand(rng, (n, r)), _rand(rng, (n, d), 0.2)
    perm = rng.permutation(n).astype(np.int32)
    g = run_both(h, A, Bm, W, perm, 250, 4, branch, "feeds eagle2_expand")
    table = tv.eagle2_new_table(1, tv.eagle2_node_count(2, k, branch), k, "cuda")
    tok, conf = to_dev(g["tok"]).view(1, k, branch), to_dev(g["conf"]).view(1, k, branch)
    tv.eagle2_expand(table, 1, tok, conf, root_tok=to_dev(np.array([7], np.int32)))
    tv.eagle2_expand(table, 2, tok, conf)
    torch.cuda.synchronize()
    assert to_host(table["status"])[0] == 0


@pytest.mark.parametrize("C,K", [(40, 10), (700, 16), (2004, 10), (8192, 64)])
def test_topk_repeated_tokens_and_ties(C, K):
    """lm_head_topk alone, on candidate lists that repeat tokens (a token's copies carry the
    same logit, as lm_head_rescore gives them) and hold many equal logits and invalid tokens.
    Each copy is a candidate of its own, as in the oracle: a repeated token can be chosen once
    per copy, and every copy counts in the softmax denominator."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    rng = np.random.default_rng(C + K)
    M, V = 5, 3000
    cand = rng.integers(0, V, (M, C)).astype(np.int32)
    # repeated tokens: copy some entries onto others
    src = rng.integers(0, C, (M, C // 4))
    dst = rng.integers(0, C, (M, C // 4))
    for m in range(M):
        cand[m, dst[m]] = cand[m, src[m]]
    cand[rng.random((M, C)) < 0.05] = -1
    cand[0, :3] = [V, V + 5, -7]  # out of range: invalid, not flagged here
    # logits on a coarse grid (many ties), one value per token
    table = (rng.integers(-20, 20, (M, V + 10)) * 0.25).astype(np.float32)
    logits = np.take_along_axis(table, np.clip(cand, 0, V + 9), axis=1).astype(np.float32)
    print(f"[case] lm topk repeated tokens M={M} C={C} K={K}", flush=True)
    tok, conf = tv.lm_head_topk(to_dev(logits), to_dev(cand), K, V)
    torch.cuda.synchronize()
    o_tok, o_conf = O.lm_topk(logits, cand, K, V)
    g_tok, g_conf = to_host(tok), to_host(conf).astype(np.float64)
    assert np.array_equal(g_tok, o_tok)
    err = np.abs(g_conf - o_conf) / np.maximum(o_conf, 1e-30)
    assert (err[o_conf > 0] <= TOL_CONF).all() and (g_conf[o_conf == 0] == 0).all(), err.max()
    # repeated tokens do come out more than once
    assert any(len(set(r[r >= 0].tolist())) < (r >= 0).sum() for r in g_tok)
