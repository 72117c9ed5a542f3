"""HIP-graph replays of the library's entry points give the eager results, bit for bit.

A caller (and the benchmark) may capture a step once and replay it.  Every kernel here is
deterministic and keeps no state between calls except the stochastic acceptance's exchange
workspace, which the last workgroup of each sequence clears again.  So each captured sequence of
calls is replayed several times.  Before each replay its outputs are poisoned (NaN, or an
impossible index), and the same entry points run eagerly on other inputs that share the
graph's workspace.  After each replay every output must equal the eager result bit for bit.  The
eager results themselves are checked against the oracle in the parity tests.  No memory is
cleared inside a graph: the poison and the clears between replays are eager torch fills.
"""
import numpy as np
import pytest
import torch

from gpu_util import to_dev, upload
from synth import make_draft_levels, make_paged, make_stochastic, make_workload

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8)


def _poison(t: torch.Tensor) -> None:
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(-7777)


def _replays_match_eager(label, run, outs, between, poison=None, clear=None):
    """Run `run` eagerly, capture it in a graph, then replay it REPLAYS times.  Before each
    replay: poison the tensors in `outs` (or call `poison`), zero those in `clear` (status words
    that the calls OR into), run `between` eagerly and synchronize."""
    clear = clear or []
    print(f"[case] graph {label}: eager run", flush=True)
    for t in clear:
        t.zero_()
    run()
    torch.cuda.synchronize()
    ref = {k: _bits(v).clone() for k, v in outs.items()}
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    print(f"[case] graph {label}: capture", flush=True)
    with torch.cuda.graph(graph, stream=stream):
        run()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        if poison is not None:
            poison()
        else:
            for v in outs.values():
                _poison(v)
        for t in clear:
            t.zero_()
        between()
        torch.cuda.synchronize()
        print(f"[case] graph {label}: replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(_bits(v), ref[k]), f"{label}: replay {rep} differs in {k}"


def _step_buffers(g, w):
    B, T, Hq, D = w.B, w.T, w.Hq, w.D
    dev = g["q"].device
    return dict(anc_mask=torch.empty((B, T, (T + 63) // 64), dtype=torch.int64, device=dev),
                out=torch.empty_like(g["q"]),
                lse=torch.empty((B, T, Hq), dtype=torch.float32, device=dev),
                accept_path=torch.empty((B, T), dtype=torch.int32, device=dev),
                accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                bonus_tok=torch.empty((B,), dtype=torch.int32, device=dev),
                cache_len_out=torch.empty((B,), dtype=torch.int32, device=dev),
                status=torch.empty((B,), dtype=torch.int32, device=dev))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_step_replays(dtype):
    """tree_verify_step with split-K partials (several splits per sequence, a zero-length
    prefix, ragged lengths), the compaction writing into the caches."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=6, T=60, L=(0, 700), Hq=8, Hkv=2, D=128,
                      dtype=dtype, extra_seed=40)
    w.cache_len[2] = 0
    w2 = make_workload("batch32_L512-4096_T60", B=6, T=60, L=(0, 700), Hq=8, Hkv=2, D=128,
                       dtype=dtype, extra_seed=41)
    g, g2 = upload(w), upload(w2)
    split = 128
    qdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ws = torch.empty((max(1, tv.tree_verify_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D,
                                                                max(w.Lmax, w2.Lmax), qdt,
                                                                split)),),
                     dtype=torch.uint8, device="cuda")
    bufs, bufs2 = _step_buffers(g, w), _step_buffers(g2, w2)

    def step(x, b):
        tv.tree_verify_step(x["parent"], x["draft"], x["target"], x["q"], x["k_cache"],
                            x["v_cache"], x["cache_len"], x["k_tree"], x["v_tree"],
                            split_keys=split, workspace=ws, **b)

    # the rows past each prefix that the compaction writes: accept_len of the eager run (the
    # buffers still hold it when the first poison comes)
    L = np.clip(w.cache_len, 0, w.Lmax)
    ends = []

    def poison():
        if not ends:
            ends.extend(np.minimum(L + bufs["accept_len"].cpu().numpy(), w.Lmax))
        for v in bufs.values():
            _poison(v)
        for b in range(w.B):
            g["k_cache"][b, :, int(L[b]):int(ends[b])].fill_(float("nan"))
            g["v_cache"][b, :, int(L[b]):int(ends[b])].fill_(float("nan"))

    outs = dict(bufs, k_cache=g["k_cache"], v_cache=g["v_cache"])
    _replays_match_eager(f"tree_verify_step {dtype}", lambda: step(g, bufs), outs,
                         lambda: step(g2, bufs2), poison=poison)
    assert int(bufs["status"].abs().sum()) == 0


def test_separate_calls_replay():
    """tree_build_mask, tree_verify_attn, tree_accept and kv_compact_accepted captured as one
    graph (a batch large enough for the longest-first dispatch of (sequence, chunk) pairs)."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=12, T=60, L=(64, 2000), Hq=8, Hkv=2, D=128,
                      extra_seed=42)
    w2 = make_workload("batch32_L512-4096_T60", B=12, T=60, L=(64, 2000), Hq=8, Hkv=2, D=128,
                       extra_seed=43)
    g, g2 = upload(w), upload(w2)
    bufs, bufs2 = _step_buffers(g, w), _step_buffers(g2, w2)
    ws_bytes = tv.tree_verify_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D,
                                                  max(w.Lmax, w2.Lmax), torch.bfloat16, 0)
    ws = torch.empty((max(1, ws_bytes),), dtype=torch.uint8, device="cuda")

    def calls(x, b):
        tv.tree_build_mask(x["parent"], anc_mask=b["anc_mask"], status=b["status"])
        tv.tree_verify_attn(x["q"], x["k_cache"], x["v_cache"], x["cache_len"], x["k_tree"],
                            x["v_tree"], b["anc_mask"], out=b["out"], lse=b["lse"],
                            status=b["status"], workspace=ws)
        tv.tree_accept(b["anc_mask"], x["draft"], x["target"], accept_path=b["accept_path"],
                       accept_len=b["accept_len"], bonus_tok=b["bonus_tok"])
        tv.kv_compact_accepted(x["k_cache"], x["v_cache"], x["cache_len"], x["k_tree"],
                               x["v_tree"], b["accept_path"], b["accept_len"],
                               cache_len_out=b["cache_len_out"], status=b["status"])

    _replays_match_eager("separate calls", lambda: calls(g, bufs), bufs,
                         lambda: calls(g2, bufs2))


def test_paged_attention_replays():
    """tree_verify_attn_paged on 16-token pages, then the greedy acceptance."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=5, T=60, L=(1, 900), Hq=8, Hkv=2, D=128,
                      extra_seed=44)
    pl = make_paged(w, 16, seed=12)
    g = upload(w)
    p = dict(k_pool=to_dev(pl.k_pool), v_pool=to_dev(pl.v_pool), table=to_dev(pl.block_table),
             tree_slot=to_dev(pl.tree_slot))
    bufs = _step_buffers(g, w)
    other = _step_buffers(g, w)
    cap = pl.block_table.shape[1] * pl.page_size
    ws = torch.empty((max(1, tv.tree_verify_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, cap,
                                                                torch.bfloat16, 96)),),
                     dtype=torch.uint8, device="cuda")

    def calls(b, split):
        tv.tree_build_mask(g["parent"], anc_mask=b["anc_mask"], status=b["status"])
        tv.tree_verify_attn_paged(g["q"], p["k_pool"], p["v_pool"], p["table"], pl.page_size,
                                  g["cache_len"], p["tree_slot"], b["anc_mask"], out=b["out"],
                                  lse=b["lse"], status=b["status"], split_keys=split,
                                  workspace=ws)
        tv.tree_accept(b["anc_mask"], g["draft"], g["target"], accept_path=b["accept_path"],
                       accept_len=b["accept_len"], bonus_tok=b["bonus_tok"])

    outs = {k: bufs[k] for k in ("anc_mask", "out", "lse", "accept_path", "accept_len",
                                 "bonus_tok", "status")}
    # between replays: the same call eagerly with another split of the prefix
    _replays_match_eager("paged attention", lambda: calls(bufs, 96), outs,
                         lambda: calls(other, 300))


def test_stochastic_acceptance_replays():
    """tree_accept_stochastic split over several workgroups per sequence: the exchange
    workspace is shared with eager calls between replays and must be left clear by each."""
    import tree_attention_verification_attn_amd as tv

    def inputs(seed):
        w = make_workload("batch32_L512-4096_T60", B=3, T=60, L=(0, 8), Hq=2, Hkv=1, D=64,
                          dtype="f32", parent_kind="random", extra_seed=seed, with_kv=False)
        s = make_stochastic(w, V=40000, seed=seed, draft_noise=2.5)
        anc, _ = tv.tree_build_mask(to_dev(np.asarray(w.parent, np.int32)))
        x = dict(anc=anc, draft=to_dev(np.asarray(s.draft, np.int32)), p=to_dev(s.p),
                 q=to_dev(s.q), u_acc=to_dev(np.asarray(s.u_acc, np.float64)),
                 u_res=to_dev(np.asarray(s.u_res, np.float64)))
        B, T = s.draft.shape
        b = dict(accept_path=torch.empty((B, T), dtype=torch.int32, device="cuda"),
                 accept_len=torch.empty((B,), dtype=torch.int32, device="cuda"),
                 bonus_tok=torch.empty((B,), dtype=torch.int32, device="cuda"),
                 status=torch.zeros((B,), dtype=torch.int32, device="cuda"))
        return x, b, s.V

    x, bufs, V = inputs(50)
    x2, bufs2, _ = inputs(51)
    G = 5
    need = tv.tree_accept_stochastic_workspace_size(3, 60, V, G)
    assert need > 0
    ws = torch.zeros((need,), dtype=torch.uint8, device="cuda")

    def call(y, b):
        tv.tree_accept_stochastic(y["anc"], y["draft"], y["p"], y["q"], y["u_acc"], y["u_res"],
                                  workgroups_per_seq=G, workspace=ws, **b)

    def poison():
        for k in ("accept_path", "accept_len", "bonus_tok"):
            _poison(bufs[k])

    _replays_match_eager("stochastic acceptance", lambda: call(x, bufs), bufs,
                         lambda: call(x2, bufs2), poison=poison, clear=[bufs["status"]])
    assert int(torch.count_nonzero(ws)) == 0


def test_tree_construction_replays():
    """Every eagle2_expand level and eagle2_rerank for a batch of sequences."""
    import tree_attention_verification_attn_amd as tv

    def inputs(seed):
        d = make_draft_levels("llama8b_b1_L4096_T60", B=5, seed=seed)
        depth, B, k, branch = d.child_tok.shape
        N = tv.eagle2_node_count(depth, k, branch)
        table = tv.eagle2_new_table(B, N, k, "cuda")
        out = {name: torch.empty((B, 60), dtype=torch.int32, device="cuda")
               for name in ("parent", "tok", "depth", "node")}
        return (d, N, table, out, to_dev(d.child_tok), to_dev(d.child_conf),
                to_dev(np.asarray(d.root_tok, np.int32)))

    a, b = inputs(60), inputs(61)

    def build(x):
        d, N, table, out, tok, conf, root = x
        for lvl in range(1, d.child_tok.shape[0] + 1):
            tv.eagle2_expand(table, lvl, tok[lvl - 1], conf[lvl - 1],
                             root_tok=root if lvl == 1 else None)
        tv.eagle2_rerank(table, N, 60, out=out)

    table, out = a[2], a[3]
    outs = dict(out, node_tok=table["node_tok"], node_parent=table["node_parent"],
                node_value=table["node_value"], frontier=table["frontier"],
                status=table["status"])

    def poison():
        for k, v in outs.items():
            if k != "status":
                _poison(v)

    _replays_match_eager("tree construction", lambda: build(a), outs, lambda: build(b),
                         poison=poison, clear=[table["status"], b[2]["status"]])
    assert int(table["status"].abs().sum()) == 0


def test_lm_head_replays():
    """The two-stage LM head's four launches with preallocated outputs."""
    import tree_attention_verification_attn_amd as tv
    from synth import make_lm_head

    x = make_lm_head("llama8b_head_M10", M=10, d=1024, n=20000, r=128, tile=200, k_tile=4, K=10)
    x2 = make_lm_head("llama8b_head_M10", seed=1, M=10, d=1024, n=20000, r=128, tile=200,
                      k_tile=4, K=10)

    def dev_inputs(y):
        return {k: to_dev(getattr(y, k).view(np.int16)).view(torch.bfloat16)
                for k in ("h", "A", "B", "W")} | {"perm": to_dev(y.row_token)}

    d1, d2 = dev_inputs(x), dev_inputs(x2)
    M, C = x.M, -(-x.n // x.tile) * x.k_tile

    def bufs():
        f = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")  # noqa: E731
        i = lambda *s: torch.empty(s, dtype=torch.int32, device="cuda")  # noqa: E731
        return dict(u=f(M, x.r), cand=i(M, C), score=f(M, C), logits=f(M, C), tok=i(M, x.K),
                    conf=f(M, x.K), status=torch.zeros(M, dtype=torch.int32, device="cuda"))

    b1, b2 = bufs(), bufs()

    def head(d, b):
        tv.lm_head_project(d["h"], d["B"], u=b["u"])
        tv.lm_head_screen(d["A"], b["u"], d["perm"], x.tile, x.k_tile, cand=b["cand"],
                          cand_score=b["score"])
        tv.lm_head_rescore(d["W"], d["h"], b["cand"], logits=b["logits"], status=b["status"])
        tv.lm_head_topk(b["logits"], b["cand"], x.K, x.n, out_tok=b["tok"], out_conf=b["conf"])

    def poison():
        for k, v in b1.items():
            if k != "status":
                _poison(v)

    _replays_match_eager("lm head", lambda: head(d1, b1), b1, lambda: head(d2, b2),
                         poison=poison, clear=[b1["status"], b2["status"]])
    assert int(b1["status"].abs().sum()) == 0


def test_fused_paged_step_replays():
    """tree_verify_step_paged with split-K partials and ragged prefixes: each replay, from the
    same block table and an empty free list, commits the same path into the same entries."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=6, T=60, L=(0, 700), Hq=8, Hkv=2, D=128,
                      extra_seed=46)
    w.target[:, :-1] = np.where(np.arange(w.T - 1) % 2 == 0, w.draft[:, 1:], w.target[:, :-1])
    w2 = make_workload("batch32_L512-4096_T60", B=6, T=60, L=(0, 700), Hq=8, Hkv=2, D=128,
                       extra_seed=47)
    pl, pl2 = make_paged(w, 1, seed=17), make_paged(w2, 1, seed=18)
    g, g2 = upload(w), upload(w2)
    split = 128

    def dev(p):
        return dict(k_pool=to_dev(p.k_pool), v_pool=to_dev(p.v_pool),
                    table=to_dev(p.block_table), slots=to_dev(p.tree_slot),
                    free=torch.full((p.num_slots,), -1, dtype=torch.int32, device="cuda"),
                    top=torch.zeros(1, dtype=torch.int32, device="cuda"))

    p, p2 = dev(pl), dev(pl2)
    table0 = p["table"].clone()
    ws = torch.empty((max(1, tv.tree_verify_attn_workspace_size(
        w.B, w.T, w.Hq, w.Hkv, w.D, max(pl.block_table.shape[1], pl2.block_table.shape[1]),
        torch.bfloat16, split)),), dtype=torch.uint8, device="cuda")
    bufs, bufs2 = _step_buffers(g, w), _step_buffers(g2, w2)

    def step(x, q, b):
        tv.tree_verify_step_paged(x["parent"], x["draft"], x["target"], x["q"], q["k_pool"],
                                  q["v_pool"], q["table"], x["cache_len"], q["slots"], q["free"],
                                  q["top"], split_keys=split, workspace=ws, **b)

    def reset():
        p["table"].copy_(table0)
        p["free"].fill_(-1)
        p["top"].zero_()

    print("[case] graph tree_verify_step_paged: eager run", flush=True)
    step(g, p, bufs)
    torch.cuda.synchronize()
    ref = {k: _bits(v).clone() for k, v in bufs.items()}
    ref_table, ref_top = p["table"].clone(), int(p["top"].item())
    ref_free = sorted(p["free"][:ref_top].tolist())
    assert int(bufs["status"].abs().sum()) == 0
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    print("[case] graph tree_verify_step_paged: capture", flush=True)
    with torch.cuda.graph(graph, stream=stream):
        step(g, p, bufs)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for v in bufs.values():
            _poison(v)
        reset()
        step(g2, p2, bufs2)  # another step eagerly in between: same workspace
        torch.cuda.synchronize()
        print(f"[case] graph tree_verify_step_paged: replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for k, v in bufs.items():
            assert torch.equal(_bits(v), ref[k]), f"replay {rep} differs in {k}"
        assert torch.equal(p["table"], ref_table), f"replay {rep}: block table differs"
        assert int(p["top"].item()) == ref_top
        assert sorted(p["free"][:ref_top].tolist()) == ref_free
