"""GPU parity of the two-stage drafter LM head (lm_head_project, lm_head_screen,
lm_head_rescore, lm_head_topk) against the CPU oracle, through the C ABI.

The oracle computes the page's definition exactly (fp64 dot products of the bfloat16 inputs):
u = B h, the score A u of every row, the local top-k of every tile of shuffled rows, the exact
logits W h, the children and their softmax confidences.  The kernels compute in float32, so
where two rows score within rounding of each other either choice is correct.  Parity is
therefore a validity check against the exact values, with the float32 rounding bound of the
kernels' arithmetic:

* every float32 value the GPU reports (u, candidate scores, logits) lies within its bound of
  the exact value.  A kernel dot product passes each term through at most n roundings
  (n = d/64 + 6 for u and the logits: 64-term chains of fused multiply-adds over d/64 pieces,
  then a six-level pairwise combination), so it errs by at most gamma_n sum |x_i y_i|,
  gamma_n = n u / (1 - n u), u = 2^-24.  A screening score on the matrix cores splits the
  float32 u exactly into three bfloat16 parts (each product with A exact) and passes each term
  through at most k + 3 ceil(r / k) roundings (k products inside its MFMA: 16 with blocks of 32
  hidden states, 32 with blocks of 16; then one per later MFMA), with the parts' magnitudes
  summing to at most (1 + 2^-8) |u|; ranks the MFMA kernel does not take run one chain over the
  rank index (r roundings).  So a screening score errs by at most gamma_n (1 + 2^-8)
  sum |A_i u_i| with n = max(r, 16 + 3 ceil(r / 16), 32 + 3 ceil(r / 32)), plus A times u's own
  error;
* every tile's candidates are distinct rows of that tile, as many as it has up to k_tile, named
  by their tokens through the row shuffle, best first by the GPU's scores; and no unchosen row
  of the tile beats a chosen one by more than both bounds: min over chosen (s + e) >=
  max over unchosen (s - e).  Where the tile's k_tile-th and next exact scores are further apart
  than that, the set is forced, and it must equal the oracle's;
* the children are the K best of the GPU's candidates by the same rule on the exact logits; the
  confidences are within the softmax's sensitivity to those bounds (relative exp(2E) - 1, E the
  largest logit bound of the hidden state, plus 1e-5 for float32 exponentials and sums) of the
  exact softmax over the GPU's candidates;
* out-of-vocabulary candidates get -inf and set TV_BAD_TOKEN.
"""
import numpy as np
import pytest
import torch

import pins
from gpu_util import to_dev, to_host
from synth import bf16_bits_to_f32, make_lm_head

pytestmark = pytest.mark.gpu

UNIT = 2.0 ** -24
TOL_CONF = 1e-5


def gamma(n: int) -> float:
    return n * UNIT / (1 - n * UNIT)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _f(b):
    return bf16_bits_to_f32(b).astype(np.float64)


def run_gpu(h, A, Bm, W, perm, tile, k_tile, K, cand_override=None):
    import tree_attention_verification_attn_amd as tv

    M = h.shape[0]
    hd, Ad, Bd, Wd = (to_dev(x.view(np.int16)).view(torch.bfloat16) for x in (h, A, Bm, W))
    status = torch.zeros(M, dtype=torch.int32, device="cuda")
    u = tv.lm_head_project(hd, Bd)
    cand, score = tv.lm_head_screen(Ad, u, to_dev(perm), tile, k_tile)
    if cand_override is not None:
        cand = to_dev(cand_override)
    logits = tv.lm_head_rescore(Wd, hd, cand, status=status)
    tok, conf = tv.lm_head_topk(logits, cand, K, W.shape[0])
    torch.cuda.synchronize()
    return dict(u=to_host(u), cand=to_host(cand), cand_score=to_host(score),
                logits=to_host(logits), tok=to_host(tok), conf=to_host(conf),
                status=to_host(status))


def check_screen(g, A, o_u, eps_u, perm, tile, k_tile, sel, o_cand):
    """Candidates of every tile of every selected hidden state; returns how many tiles had a
    forced set (and matched the oracle's)."""
    from oracle import oracle as O

    n, r = A.shape
    Ms = len(sel)
    s_ex = O.lm_scores(A, o_u)  # [Ms, n] exact
    absA = np.abs(_f(A))
    n_round = max(r, 16 + 3 * -(-r // 16), 32 + 3 * -(-r // 32))  # any screening path (docstring)
    eps_s = gamma(n_round) * (1 + 2.0 ** -8) * (np.abs(o_u) + eps_u) @ absA.T + eps_u @ absA.T
    n_tiles = -(-n // tile)
    pad = n_tiles * tile - n
    S = np.pad(s_ex, ((0, 0), (0, pad)), constant_values=-np.inf).reshape(Ms, n_tiles, tile)
    E = np.pad(eps_s, ((0, 0), (0, pad))).reshape(Ms, n_tiles, tile)
    cand = g["cand"][sel].reshape(Ms, n_tiles, k_tile)
    score = g["cand_score"][sel].astype(np.float64).reshape(Ms, n_tiles, k_tile)
    inv = np.empty(n, np.int64)
    inv[perm] = np.arange(n)
    rows_in = np.minimum(tile, n - np.arange(n_tiles) * tile)  # rows of each tile
    n_valid = np.minimum(k_tile, rows_in)
    slot = np.arange(k_tile)
    want_valid = slot[None, None, :] < n_valid[None, :, None]
    assert np.array_equal(cand >= 0, np.broadcast_to(want_valid, cand.shape)), "candidate count"
    assert np.isneginf(score[~want_valid.repeat(Ms, 0)]).all()
    assert (cand < n).all()
    row = np.where(cand >= 0, inv[np.maximum(cand, 0)], -1)
    loc = row - np.arange(n_tiles)[None, :, None] * tile
    assert ((loc >= 0) & (loc < tile))[cand >= 0].all(), "candidate outside its tile"
    # distinct rows, best first by the GPU's own scores
    srt = np.sort(np.where(cand >= 0, loc, -1 - slot[None, None, :]), axis=2)
    assert (np.diff(srt, axis=2) != 0).all(), "a row chosen twice"
    assert (np.diff(np.where(want_valid, score, -1e300), axis=2) <= 0).all(), "not best first"
    m_i, t_i, j_i = np.nonzero(cand >= 0)
    l_i = loc[m_i, t_i, j_i]
    ex = S[m_i, t_i, l_i]
    assert (np.abs(score[m_i, t_i, j_i] - ex) <= E[m_i, t_i, l_i]).all(), "candidate score"
    chosen = np.zeros(S.shape, bool)
    chosen[m_i, t_i, l_i] = True
    lo = np.where(chosen, S + E, np.inf).min(axis=2)
    real = np.isfinite(S)
    hi = np.where(~chosen & real, S - E, -np.inf).max(axis=2)
    assert (lo >= hi).all(), f"a tile's candidates are not its best rows ({(lo < hi).sum()})"
    # forced tiles (the exact top set beats every other row by more than both bounds) must
    # equal the oracle's candidates
    rank = np.argsort(np.argsort(-S, axis=2, kind="stable"), axis=2)
    top = rank < n_valid[None, :, None]
    fmin = np.where(top, S - E, np.inf).min(axis=2)
    fmax = np.where(~top & real, S + E, -np.inf).max(axis=2)
    forced = fmin > fmax
    oc = o_cand.reshape(Ms, n_tiles, k_tile)
    same = (np.sort(oc, axis=2) == np.sort(cand, axis=2)).all(axis=2)
    assert same[forced].all(), "a forced tile differs from the oracle's candidates"
    return int(forced.sum()), int(forced.size)


def check_children(g, L_all, eps_l, sel, K, V):
    """Logits of the GPU's candidates, the children and their confidences."""
    import tree_attention_verification_attn_amd as tv

    for i, m in enumerate(sel):
        cand = g["cand"][m]
        valid = (cand >= 0) & (cand < V)
        lg = g["logits"][m].astype(np.float64)
        assert np.isneginf(lg[~valid]).all()
        ex = L_all[i, cand[valid]]
        ec = eps_l[i, cand[valid]]
        assert (np.abs(lg[valid] - ex) <= ec).all(), "logit"
        bad = ((cand < -1) | (cand >= V)).any()
        assert (g["status"][m] & tv.TV_BAD_TOKEN) == (tv.TV_BAD_TOKEN if bad else 0)
        tok = g["tok"][m]
        nk = min(K, int(valid.sum()))
        assert (tok[nk:] == -1).all() and (g["conf"][m][nk:] == 0).all()
        kids = tok[:nk]
        assert (kids >= 0).all() and (kids < V).all()
        # each child is one copy of a valid candidate
        vals, cnt = np.unique(cand[valid], return_counts=True)
        kv, kc = np.unique(kids, return_counts=True)
        have = dict(zip(vals.tolist(), cnt.tolist()))
        assert all(have.get(t, 0) >= c for t, c in zip(kv.tolist(), kc.tolist())), "child copies"
        left = dict(have)
        for t in kids.tolist():
            left[t] -= 1
        k_ex, k_eps = L_all[i, kids], eps_l[i, kids]
        un = [t for t, c in left.items() for _ in range(c)]
        if un:
            assert (k_ex + k_eps).min() >= (L_all[i, un] - eps_l[i, un]).max(), "children"
        # best first by the GPU's own logits (every copy of a token has the same logit)
        glog = {int(t): float(v) for t, v in zip(cand[valid], lg[valid])}
        kl = np.array([glog[int(t)] for t in kids])
        assert (np.diff(kl) <= 0).all(), "children not best first"
        # confidences: softmax over every valid candidate copy, within its sensitivity
        mx = ex.max()
        z = np.exp(ex - mx).sum()
        want = np.exp(k_ex - mx) / z
        rel = np.expm1(2 * ec.max()) + TOL_CONF
        err = np.abs(g["conf"][m][:nk].astype(np.float64) - want)
        assert (err <= rel * want + 1e-30).all(), (err / want).max()


def run_both(h, A, Bm, W, perm, tile, k_tile, K, label, rows=None, cand_override=None):
    """Device head against the oracle's exact values; `rows` limits the check to some hidden
    states."""
    from oracle import oracle as O

    M, d = h.shape
    n, r = A.shape
    V = W.shape[0]
    print(f"[case] lm head {label} M={M} d={d} n={n} r={r} tile={tile} k_tile={k_tile} K={K}",
          flush=True)
    g = run_gpu(h, A, Bm, W, perm, tile, k_tile, K, cand_override)
    sel = np.arange(M) if rows is None else np.asarray(rows)
    depth = d // 64 + 6
    o_u = O.lm_project(h[sel], Bm)
    eps_u = gamma(depth) * (np.abs(_f(h[sel])) @ np.abs(_f(Bm)).T)
    assert (np.abs(g["u"][sel].astype(np.float64) - o_u) <= eps_u).all(), f"{label}: u"
    o_cand, _ = O.lm_screen(A, o_u, perm, tile, k_tile)
    forced = None
    if cand_override is None:
        forced = check_screen(g, A, o_u, eps_u, perm, tile, k_tile, sel, o_cand)
    L_all = O.lm_logits_all(W, h[sel])
    eps_l = gamma(depth) * (np.abs(_f(h[sel])) @ np.abs(_f(W)).T)
    check_children(g, L_all, eps_l, sel, K, V)
    if forced is not None:
        print(f"       forced tiles {forced[0]} of {forced[1]} equal the oracle's", flush=True)
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
    """Integer-valued inputs: every float32 sum is exact (the bounds still hold), and scores and
    logits tie often; tied rows may go either way, but the GPU's choice must be a best set."""
    rng = np.random.default_rng(42)
    for trial in range(9):
        M, d, r, n = 5, 512, 16, 700
        k_tile = (5, 4, 2)[trial % 3]  # rounds of maxima, then the sorting network
        h, Bm, A, W, perm = pins._int_lm_case(rng, M, d, r, n, lo=-2, hi=3)
        g = run_both(pins._bits(h), pins._bits(A[perm]), pins._bits(Bm), pins._bits(W), perm,
                     64, k_tile, 12, f"integers {trial} k_tile={k_tile}")
        # exact arithmetic: the GPU's values equal the exact ones
        assert np.array_equal(g["u"].astype(np.float64), (h @ Bm.T).astype(np.float64))


def test_every_hidden_state_count():
    """Each compile-time chain count of the screening kernel (M rounded up to 2, 4, 6, 8, 10,
    12, 16, 24, 32, 48, 64)."""
    rng = np.random.default_rng(43)
    d, r, n = 512, 64, 900
    Bm, A, W = _rand(rng, (r, d), 1 / np.sqrt(d)), _rand(rng, (n, r)), _rand(rng, (n, d), 0.05)
    perm = rng.permutation(n).astype(np.int32)
    for M in (1, 3, 5, 7, 9, 11, 13, 17, 25, 33, 49, 64):
        run_both(_rand(rng, (M, d)), A, Bm, W, perm, 128, 3, 8, f"M={M}")


def test_screen_kernel_boundary_and_largest_picks():
    """Ranks at and just past the matrix-core screening kernel's limit (256, then 272 on the
    float32 chains), the most hidden states and candidates per tile (64 and 16: the largest
    pick area), a short last tile, and ranks that are not multiples of 16."""
    rng = np.random.default_rng(46)
    d, n = 512, 1300
    for M, r, k_tile in ((64, 256, 16), (48, 272, 16), (33, 248, 16), (40, 200, 5)):
        h, Bm = _rand(rng, (M, d)), _rand(rng, (r, d), 1 / np.sqrt(d))
        A, W = _rand(rng, (n, r)), _rand(rng, (n, d), 0.05)
        perm = rng.permutation(n).astype(np.int32)
        run_both(h, A, Bm, W, perm, 256, k_tile, 12, f"M={M} r={r} k_tile={k_tile}")


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
    The logits are exact multiples of 1/4, so the children are unique up to the tie rule
    (larger logit, then smaller token; each copy a candidate of its own): they must equal the
    oracle's.  Confidences within 1e-5 relative of the oracle's fp64 softmax."""
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
    o_tok, o_conf = O.lm_topk(logits.astype(np.float64), cand, K, V)
    g_tok, g_conf = to_host(tok), to_host(conf).astype(np.float64)
    assert np.array_equal(g_tok, o_tok)
    err = np.abs(g_conf - o_conf) / np.maximum(o_conf, 1e-30)
    assert (err[o_conf > 0] <= TOL_CONF).all() and (g_conf[o_conf == 0] == 0).all(), err.max()
    # repeated tokens do come out more than once
    assert any(len(set(r[r >= 0].tolist())) < (r >= 0).sum() for r in g_tok)
