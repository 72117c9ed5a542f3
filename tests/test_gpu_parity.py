"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Every step is compared: ancestor masks, acceptance and compaction bit-exactly (cache bytes
included, with NaN-poisoned rows past every prefix), attention within max-abs 1e-5 (fp32) or
2e-2 (bf16).  Small workloads are compared on every output row; the full-size ones on sampled
rows, in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL_OUT, check_step, run_step, sample_rows, to_dev, to_host, upload
from synth import WORKLOADS, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _run_and_check(w, rows=None, split_keys=0, label=""):
    print(f"[case] {label} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} D={w.D} Lmax={w.Lmax} "
          f"{w.dtype} split_keys={split_keys}", flush=True)
    res = run_step(upload(w), split_keys=split_keys)
    stats = check_step(w, res, rows=rows, label=label)
    print(f"       max-abs err {stats['err']:.3e}  lse err {stats['lse_err']:.3e}", flush=True)
    return res, stats


# ---- the five workloads ----------------------------------------------------------------------
def test_worked_tree_fp32_full():
    w = make_workload("worked_tree_fp32")
    _run_and_check(w, label="worked_tree_fp32")


def test_llama8b_b1_full():
    w = make_workload("llama8b_b1_L4096_T60")
    _run_and_check(w, label="llama8b_b1_L4096_T60")


@pytest.mark.parametrize("name", ["batch32_L512-4096_T60", "llama70b_b8_L32768_T64",
                                  "wide_b64_L1024-8192_T128"])
def test_full_size_sampled(name):
    w = make_workload(name)
    _run_and_check(w, rows=sample_rows(w, 160, seed=1), label=name)


# ---- split-K invariance ----------------------------------------------------------------------
@pytest.mark.parametrize("split_keys", [64, 192, 1024, 100000])
def test_split_invariance(split_keys):
    w = make_workload("batch32_L512-4096_T60", B=6, extra_seed=3)
    _run_and_check(w, split_keys=split_keys, label=f"split {split_keys}")


def test_split_results_agree():
    w = make_workload("llama8b_b1_L4096_T60", extra_seed=4)
    outs = []
    for sk in (0, 64, 512, 4096):
        res = run_step(upload(w), split_keys=sk)
        outs.append(res["out"].view(np.uint16))
    base = outs[0].view(np.uint16)
    for o in outs[1:]:
        a = (base.astype(np.uint32) << 16).view(np.float32)
        b = (o.astype(np.uint32) << 16).view(np.float32)
        assert np.abs(a - b).max() <= TOL_OUT["bf16"]


# ---- merge ranking over more than 256 sequences ---------------------------------------------
def test_merge_ranks_more_than_256_sequences():
    """With few chunks per sequence the merge ranks the split sequences by ballots, 256 per pass:
    300 sequences, most split in two and some not split, so the ranking takes two passes and
    skips sequences in both.  The separate calls and the fused step agree bit for bit and match
    the oracle."""
    from gpu_util import run_step_fused

    w = make_workload("batch32_L512-4096_T60", B=300, T=8, L=(0, 120), Hq=2, Hkv=1, D=64,
                      parent_kind="random", extra_seed=91)
    w.cache_len[::7] = 0  # the tree tile alone: one chunk, written directly, never merged
    res, _ = _run_and_check(w, split_keys=64, label="300 sequences, split_keys 64")
    fused = run_step_fused(upload(w), split_keys=64)
    assert np.array_equal(res["out"].view(np.uint16), fused["out"].view(np.uint16))
    assert np.array_equal(res["lse"].view(np.uint32), fused["lse"].view(np.uint32))


# ---- every shape of the split-K merge ------------------------------------------------------
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
@pytest.mark.parametrize("target", [2, 4, 8, 20, 64])
def test_merge_shapes(dtype, D, target):
    """The merge loads 2, 4 or 8 chunks per round per thread, and beyond 8 chunks the four
    wavefronts of a workgroup share a piece and meet in LDS (beyond 32, in several rounds).
    Every such shape in both input types and head sizes.  G * T = 61 rows, so the second row of
    the last bf16 pair is padding.  A zero-length prefix (one chunk, written directly) sits next
    to sequences with many chunks."""
    L = (1200, 2500) if target == 64 else (600, 1200)
    w = make_workload("batch32_L512-4096_T60", B=3, T=61, L=L, Hq=3, Hkv=3, D=D, dtype=dtype,
                      parent_kind="random", extra_seed=70 + target)
    w.cache_len[1] = 0
    tiles = 1 + -(-w.Lmax // 64)
    chunk_tiles = -(-tiles // target)
    S = -(-tiles // chunk_tiles)
    lo = {2: 2, 4: 3, 8: 5, 20: 9, 64: 33}[target]
    assert lo <= S <= max(target, 16) or (target == 64 and S > 32), (tiles, S)
    _run_and_check(w, split_keys=64 * chunk_tiles, label=f"merge {dtype} D={D} S={S}")


# ---- ragged shapes and edge cases ------------------------------------------------------------
EDGE = [
    # (label, overrides)
    ("single_node_empty_prefix", dict(B=2, T=1, L=(0, 3), Hq=4, Hkv=2, D=128, dtype="bf16")),
    ("T128_two_mask_words", dict(B=3, T=128, L=(0, 700), Hq=8, Hkv=2, D=128, dtype="bf16",
                                 parent_kind="random")),
    ("T65_partial_second_tile", dict(B=2, T=65, L=(1, 130), Hq=4, Hkv=1, D=128, dtype="bf16",
                                     parent_kind="deep")),
    # depth 127: every pointer-jumping round of a mask build, pointers crossing mask words
    ("T128_chain", dict(B=2, T=128, L=(3, 200), Hq=4, Hkv=2, D=128, dtype="bf16",
                        parent_kind="chain")),
    ("row_blocks_4", dict(B=2, T=100, L=(63, 65), Hq=16, Hkv=2, D=128, dtype="bf16",
                          parent_kind="random")),
    ("d64_bf16", dict(B=3, T=20, L=(1, 300), Hq=12, Hkv=3, D=64, dtype="bf16",
                      parent_kind="star")),
    ("fp32_d128", dict(B=2, T=16, L=(5, 200), Hq=4, Hkv=2, D=128, dtype="f32",
                       parent_kind="random")),
    ("fp32_d64_chain", dict(B=2, T=40, L=(0, 129), Hq=2, Hkv=1, D=64, dtype="f32",
                            parent_kind="chain")),
    ("mha_no_grouping", dict(B=2, T=9, L=(64, 64), Hq=3, Hkv=3, D=128, dtype="bf16",
                             parent_kind="random")),
]


@pytest.mark.parametrize("label,kw", EDGE, ids=[e[0] for e in EDGE])
@pytest.mark.parametrize("split_keys", [0, 64])
def test_edge_case(label, kw, split_keys):
    w = make_workload("batch32_L512-4096_T60", extra_seed=11, **kw)
    _run_and_check(w, split_keys=split_keys, label=label)


def test_bad_trees_flagged():
    w = make_workload("batch32_L512-4096_T60", B=4, T=10, L=(20, 40), Hq=4, Hkv=2, D=128,
                      parent_kind="random", extra_seed=5)
    w.parent[1, 3] = 3   # self parent
    w.parent[2, 0] = 0   # root with a parent
    w.parent[3, 9] = -1  # second root
    res, _ = _run_and_check(w, label="bad trees")
    assert list(res["status"] & 1) == [0, 1, 1, 1]
    assert list(res["alen"][1:]) == [1, 1, 1]


def test_bad_cache_len_flagged_and_clamped():
    from synth import f32_to_bf16_bits

    w = make_workload("batch32_L512-4096_T60", B=3, T=8, L=(10, 30), Hq=4, Hkv=1, D=128,
                      parent_kind="random", extra_seed=6)
    # sequence 1 claims more rows than the cache holds: it is clamped to Lmax, so give every
    # row a finite value; sequence 2 claims a negative length and sees only its tree rows
    L1 = int(w.cache_len[1])
    rng = np.random.default_rng(60)
    fill = rng.standard_normal(w.k_cache[1, :, L1:].shape).astype(np.float32)
    w.k_cache[1, :, L1:] = f32_to_bf16_bits(fill)
    w.v_cache[1, :, L1:] = f32_to_bf16_bits(-fill)
    w.cache_len[1] = w.Lmax + 5
    w.cache_len[2] = -3
    res, _ = _run_and_check(w, label="bad cache_len")
    assert list(res["status"] & 4) == [0, 4, 4]
    assert list(res["new_len"][1:]) == [w.Lmax + 5, -3]


def test_compaction_overflow():
    w = make_workload("batch32_L512-4096_T60", B=2, T=30, L=(100, 100), Hq=4, Hkv=2, D=128,
                      parent_kind="chain", extra_seed=7, lmax_pad=1)
    w.target[:, :-1] = w.draft[:, 1:]  # every draft accepted: 30 rows
    w.target[0, 5] = -1                # sequence 0 stops after 6 nodes
    Lmax = w.Lmax - 1                  # sequence 1 needs 100 + 30 rows: one too many
    w.k_cache = np.ascontiguousarray(w.k_cache[:, :, :Lmax])
    w.v_cache = np.ascontiguousarray(w.v_cache[:, :, :Lmax])
    w.Lmax = Lmax
    res, _ = _run_and_check(w, label="overflow")
    assert res["status"][1] & 2 and not res["status"][0] & 2
    assert list(res["alen"]) == [6, 30] and list(res["new_len"]) == [106, 100]


# ---- aliasing ---------------------------------------------------------------------------------
def test_compaction_tree_rows_inside_cache():
    """Tree K/V written in place as the cache rows after the prefix (one sequence, one KV
    head): compaction must read all accepted rows before writing any."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    for dtype in ("f32", "bf16"):
        w = make_workload("worked_tree_fp32", dtype=dtype, D=128, extra_seed=8)
        L, T = int(w.cache_len[0]), w.T
        w.k_cache[0, 0, L:L + T] = w.k_tree[0, :, 0]
        w.v_cache[0, 0, L:L + T] = w.v_tree[0, :, 0]
        kc, vc = to_dev(w.k_cache), to_dev(w.v_cache)
        kt = kc[:, 0, L:L + T, :].reshape(1, T, 1, w.D)
        vt = vc[:, 0, L:L + T, :].reshape(1, T, 1, w.D)
        assert kt.data_ptr() == kc.data_ptr() + L * w.D * kc.element_size()
        path = np.full((1, T), -1, np.int32)
        path[0, :4] = [0, 1, 3, 6]
        alen = np.array([4], np.int32)
        new_len = tv.kv_compact_accepted(kc, vc, to_dev(w.cache_len), kt, vt, to_dev(path),
                                         to_dev(alen))
        torch.cuda.synchronize()
        hk, hv = w.k_cache.copy(), w.v_cache.copy()
        o_len, _ = O.compact(hk, hv, w.cache_len, w.k_tree, w.v_tree, path, alen)
        assert to_host(new_len)[0] == o_len[0] == L + 4
        bits = np.uint32 if dtype == "f32" else np.uint16
        assert np.array_equal(to_host(kc).view(bits), hk.view(bits))
        assert np.array_equal(to_host(vc).view(bits), hv.view(bits))


def test_compaction_cache_len_in_place():
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    w = make_workload("batch32_L512-4096_T60", B=5, T=12, L=(3, 90), Hq=8, Hkv=4, D=128,
                      parent_kind="chain", extra_seed=9)
    w.target[:, :-1] = w.draft[:, 1:]
    g = upload(w)
    o_path, o_len, _ = O.accept(w.parent, w.draft, w.target)
    cl = g["cache_len"]
    new_len = tv.kv_compact_accepted(g["k_cache"], g["v_cache"], cl, g["k_tree"], g["v_tree"],
                                     to_dev(o_path), to_dev(o_len), cache_len_out=cl)
    torch.cuda.synchronize()
    assert new_len.data_ptr() == cl.data_ptr()
    assert np.array_equal(to_host(cl), w.cache_len + o_len)
    kc = w.k_cache.copy()
    vc = w.v_cache.copy()
    O.compact(kc, vc, w.cache_len, w.k_tree, w.v_tree, o_path, o_len)
    assert np.array_equal(to_host(g["k_cache"]).view(np.uint16), kc.view(np.uint16))


# ---- canaries around every output -------------------------------------------------------------
def _guarded(shape, dtype, fill):
    n = int(np.prod(shape))
    pad = 4096
    buf = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(shape), pad


def test_output_canaries():
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=3, T=37, L=(1, 500), Hq=8, Hkv=2, D=128,
                      parent_kind="random", extra_seed=10)
    g = upload(w)
    B, T, Hq, D = w.B, w.T, w.Hq, w.D
    bufs = {}
    bufs["anc"] = _guarded((B, T, 1), torch.int64, -7)
    bufs["status"] = _guarded((B,), torch.int32, -7)
    bufs["out"] = _guarded((B, T, Hq, D), torch.bfloat16, -7.0)
    bufs["lse"] = _guarded((B, T, Hq), torch.float32, -7.0)
    bufs["path"] = _guarded((B, T), torch.int32, -7)
    bufs["alen"] = _guarded((B,), torch.int32, -7)
    bufs["bonus"] = _guarded((B,), torch.int32, -7)
    bufs["new_len"] = _guarded((B,), torch.int32, -7)
    for split_keys in (0, 64):
        anc, st = tv.tree_build_mask(g["parent"], bufs["anc"][1], bufs["status"][1])
        tv.tree_verify_attn(g["q"], g["k_cache"], g["v_cache"], g["cache_len"], g["k_tree"],
                            g["v_tree"], anc, out=bufs["out"][1], lse=bufs["lse"][1], status=st,
                            split_keys=split_keys)
        p, a, bo = tv.tree_accept(anc, g["draft"], g["target"], bufs["path"][1], bufs["alen"][1],
                                  bufs["bonus"][1])
        tv.kv_compact_accepted(g["k_cache"], g["v_cache"], g["cache_len"], g["k_tree"],
                               g["v_tree"], p, a, cache_len_out=bufs["new_len"][1], status=st)
        torch.cuda.synchronize()
        for name, (buf, _view, pad) in bufs.items():
            head, tail = buf[:pad].float().cpu(), buf[-pad:].float().cpu()
            assert (head == -7).all() and (tail == -7).all(), f"{name} guard overwritten"
