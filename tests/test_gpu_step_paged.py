"""GPU parity of tree_verify_step_paged (mask, paged attention, acceptance and pointer-swap
commit in two launches) through the C ABI.

The fused step must equal the four separate calls bit for bit: attention output and lse,
masks, path, bonus token, block table, lengths and status; the free list holds the same
slots (its order across sequences follows the atomics, so it is compared as a multiset).  The
separate calls are themselves pinned to the CPU oracle, and the fused step is also checked
against the oracle directly: attention within max-abs 1e-5 (fp32) / 2e-2 (bf16), everything
else exactly.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL_LSE, TOL_OUT, as_f64, sample_rows, to_dev, to_host, upload
from synth import make_paged, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _fused(w, pl, split_keys=0, spare_top=0, in_place_len=False):
    import tree_attention_verification_attn_amd as tv

    g = upload(w)
    table, slots = to_dev(pl.block_table), to_dev(pl.tree_slot)
    free = torch.full((pl.num_slots,), -1, dtype=torch.int32, device="cuda")
    top = torch.tensor([spare_top], dtype=torch.int32, device="cuda")
    res = tv.tree_verify_step_paged(
        g["parent"], g["draft"], g["target"], g["q"], to_dev(pl.k_pool), to_dev(pl.v_pool),
        table, g["cache_len"], slots, free, top, page_size=1,
        cache_len_out=g["cache_len"] if in_place_len else None, split_keys=split_keys)
    torch.cuda.synchronize()
    out = {k: to_host(v) for k, v in res.items()}
    out.update(table=to_host(table), free=to_host(free), top=int(to_host(top)[0]))
    return out


def _separate(w, pl, split_keys=0, spare_top=0):
    import tree_attention_verification_attn_amd as tv

    g = upload(w)
    table, slots = to_dev(pl.block_table), to_dev(pl.tree_slot)
    k_pool, v_pool = to_dev(pl.k_pool), to_dev(pl.v_pool)
    free = torch.full((pl.num_slots,), -1, dtype=torch.int32, device="cuda")
    top = torch.tensor([spare_top], dtype=torch.int32, device="cuda")
    anc, status = tv.tree_build_mask(g["parent"])
    o, lse = tv.tree_verify_attn_paged(g["q"], k_pool, v_pool, table, 1, g["cache_len"], slots,
                                       anc, status=status, split_keys=split_keys)
    path, alen, bonus = tv.tree_accept(anc, g["draft"], g["target"])
    new_len = tv.kv_commit_paged(table, g["cache_len"], slots, path, alen, free, top,
                                 pl.num_slots, status=status)
    torch.cuda.synchronize()
    return dict(anc_mask=to_host(anc), out=to_host(o), lse=to_host(lse),
                accept_path=to_host(path), accept_len=to_host(alen), bonus_tok=to_host(bonus),
                cache_len_out=to_host(new_len), status=to_host(status), table=to_host(table),
                free=to_host(free), top=int(to_host(top)[0]))


def _same(a, b, spare_top=0):
    for k in ("anc_mask", "out", "lse", "accept_path", "accept_len", "bonus_tok",
              "cache_len_out", "status", "table", "top"):
        x, y = np.asarray(a[k]), np.asarray(b[k])
        assert x.shape == y.shape, k
        assert np.array_equal(x.reshape(-1).view(np.uint8), y.reshape(-1).view(np.uint8)), k
    top = a["top"]
    assert sorted(a["free"][spare_top:top]) == sorted(b["free"][spare_top:top])
    assert (a["free"][:spare_top] == -1).all() and (a["free"][top:] == -1).all()


def _oracle_check(w, pl, res, rows=None, spare_top=0, rtol=0.0):
    from oracle import oracle as O

    o_out, o_lse = O.paged_attention(w.q, pl.k_pool, pl.v_pool, pl.block_table, 1, w.cache_len,
                                     pl.tree_slot, w.parent, rows=rows)
    got, got_lse = as_f64(res["out"]), res["lse"].astype(np.float64)
    if rows is not None:
        got = got[rows[:, 0], rows[:, 2], rows[:, 1]]
        got_lse = got_lse[rows[:, 0], rows[:, 2], rows[:, 1]]
    err, lerr = float(np.abs(got - o_out).max()), float(np.abs(got_lse - o_lse).max())
    print(f"       max-abs err {err:.3e}  lse err {lerr:.3e}", flush=True)
    excess = float((np.abs(got - o_out) - TOL_OUT[w.dtype] - rtol * np.abs(o_out)).max())
    assert excess <= 0 and lerr <= TOL_LSE[w.dtype], (err, lerr)
    o_path, o_len, o_bonus = O.accept(w.parent, w.draft, w.target)
    assert np.array_equal(res["accept_path"], o_path)
    assert np.array_equal(res["accept_len"], o_len)
    assert np.array_equal(res["bonus_tok"], o_bonus)
    h_table = pl.block_table.copy()
    h_free = np.full(pl.num_slots, -1, np.int32)
    o_new, o_top, o_st = O.commit_paged(h_table, w.cache_len, pl.tree_slot, o_path, o_len,
                                        pl.num_slots, h_free, spare_top)
    assert np.array_equal(res["table"], h_table)
    assert np.array_equal(res["cache_len_out"], o_new)
    assert np.array_equal(res["status"], o_st)
    assert res["top"] == o_top
    assert sorted(res["free"][spare_top:o_top]) == sorted(h_free[spare_top:o_top])


@pytest.mark.parametrize("name,kw,split_keys,sampled", [
    ("llama8b_b1_L4096_T60", {}, 0, False),
    ("batch32_L512-4096_T60", dict(B=6, L=(20, 700)), 0, False),
    ("batch32_L512-4096_T60", dict(B=5, T=33, L=(0, 300)), 64, False),
    ("wide_b64_L1024-8192_T128", dict(B=3, L=(10, 400)), 0, False),
    ("batch32_L512-4096_T60", {}, 0, True),
    ("llama70b_b8_L32768_T64", {}, 0, True),
    ("wide_b64_L1024-8192_T128", {}, 0, True),
], ids=["llama8b_b1", "batch6", "ragged_split64", "wide_T128", "batch32_full_sampled",
        "llama70b_full_sampled", "wide_full_sampled"])
def test_step_paged_matches_oracle(name, kw, split_keys, sampled):
    w = make_workload(name, **kw, extra_seed=41)
    # accept a few levels: some drafts equal their parent's target token
    w.target[:, :-1] = np.where(np.arange(w.T - 1) % 3 == 0, w.draft[:, 1:], w.target[:, :-1])
    pl = make_paged(w, 1, seed=12)
    print(f"[case] step_paged {name} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} D={w.D} {w.dtype} "
          f"split_keys={split_keys}", flush=True)
    res = _fused(w, pl, split_keys=split_keys, spare_top=3)
    rows = sample_rows(w, 120, seed=3) if sampled else None
    _oracle_check(w, pl, res, rows=rows, spare_top=3)


@pytest.mark.parametrize("split_keys", [0, 192])
def test_step_paged_matches_separate_calls_bitwise(split_keys):
    w = make_workload("batch32_L512-4096_T60", B=4, L=(100, 900), extra_seed=42)
    w.target[:, :-1] = np.where(np.arange(w.T - 1) % 2 == 0, w.draft[:, 1:], w.target[:, :-1])
    pl = make_paged(w, 1, seed=13)
    print(f"[case] step_paged bitwise split_keys={split_keys}", flush=True)
    _same(_fused(w, pl, split_keys=split_keys, spare_top=2),
          _separate(w, pl, split_keys=split_keys, spare_top=2), spare_top=2)


def test_step_paged_status_bits_match_separate_calls():
    """A bad page, a bad tree slot, a bad length, a bad tree and an overflow, one sequence
    each: the fused step reports the same bits as the four calls, and commits the same."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=6, T=12, L=(30, 40), Hq=4, Hkv=1, D=128,
                      parent_kind="chain", extra_seed=43)
    w.target[:, :-1] = w.draft[:, 1:]  # every node accepted
    pl = make_paged(w, 1, seed=14, headroom=12)
    pl.block_table[0, 5] = pl.num_slots + 3  # page past the pool
    pl.tree_slot[1, 4] = -1                  # tree slot before the pool
    w.cache_len[2] = -2                      # bad length
    w.parent[3, 2] = 2                       # self parent: not a tree
    w.cache_len[4] = pl.block_table.shape[1] - 5  # room for 5 rows only: overflow
    print("[case] step_paged status bits", flush=True)
    a, b = _fused(w, pl, spare_top=1), _separate(w, pl, spare_top=1)
    _same(a, b, spare_top=1)
    st = a["status"]
    assert st[0] & tv.TV_BAD_PAGE and st[1] & tv.TV_BAD_PAGE and st[1] & tv.TV_BAD_PATH
    assert st[2] & tv.TV_BAD_LEN and st[3] & tv.TV_BAD_TREE and st[4] & tv.TV_OVERFLOW
    assert st[5] == 0


def test_step_paged_in_place_length():
    w = make_workload("batch32_L512-4096_T60", B=3, T=20, L=(50, 500), extra_seed=44)
    w.target[:, :-1] = w.draft[:, 1:]
    pl = make_paged(w, 1, seed=15)
    print("[case] step_paged in-place length", flush=True)
    res = _fused(w, pl, in_place_len=True)
    _oracle_check(w, pl, res)


def test_step_paged_rejects_larger_pages():
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=2, T=8, L=(30, 40), Hq=4, Hkv=1, D=128,
                      extra_seed=45)
    pl = make_paged(w, 4, seed=16)
    g = upload(w)
    free = torch.full((pl.num_slots,), -1, dtype=torch.int32, device="cuda")
    top = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(tv.TreeVerifyError) as e:
        tv.tree_verify_step_paged(g["parent"], g["draft"], g["target"], g["q"],
                                  to_dev(pl.k_pool), to_dev(pl.v_pool), to_dev(pl.block_table),
                                  g["cache_len"], to_dev(pl.tree_slot), free, top, page_size=4)
    assert e.value.code == tv.TV_ERR_UNSUPPORTED


def test_step_paged_free_list_full():
    """A free list with room for only two of the rejected slots: the path is still committed,
    two slots are written, nothing past the list's end, and the sequence gets TV_FREE_FULL
    (batch 1, so which sequence found the list full is unique)."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("llama8b_b1_L4096_T60", L=(300, 300), extra_seed=46)
    w.target[:, :-1] = np.where(np.arange(w.T - 1) % 3 == 0, w.draft[:, 1:], w.target[:, :-1])
    pl = make_paged(w, 1, seed=18)
    spare_top = pl.num_slots - 2
    print(f"[case] step_paged free list full (top {spare_top} of {pl.num_slots})", flush=True)
    res = _fused(w, pl, spare_top=spare_top)
    assert res["status"][0] & tv.TV_FREE_FULL
    _oracle_check(w, pl, res, spare_top=spare_top)
    assert (res["free"][:spare_top] == -1).all()
    sep = _separate(w, pl, spare_top=spare_top)
    _same(res, sep, spare_top=spare_top)
