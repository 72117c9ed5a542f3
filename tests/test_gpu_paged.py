"""GPU parity of the paged-KV entry points (tree_verify_attn_paged, kv_commit_paged) against the
CPU oracle, through the C ABI.

Attention over a paged cache must match the oracle's attention over the rows the block table
names (max-abs 1e-5 fp32, 2e-2 bf16), and equal the dense kernel bit for bit when both cut the
prefix into the same chunks.  The pointer-swap commit must reproduce the oracle's block table,
lengths, status and free-list count exactly; the free list must hold exactly the rejected
slots (their order across sequences follows the atomics, so it is compared as a multiset).
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


def _paged_dev(pl):
    return dict(k_pool=to_dev(pl.k_pool), v_pool=to_dev(pl.v_pool),
                table=to_dev(pl.block_table), tree_slot=to_dev(pl.tree_slot))


def _check_attn(w, pl, split_keys=0, rows=None, label=""):
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    print(f"[case] paged {label} P={pl.page_size} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} "
          f"D={w.D} {w.dtype} split_keys={split_keys}", flush=True)
    g, p = upload(w), _paged_dev(pl)
    anc, status = tv.tree_build_mask(g["parent"])
    out, lse = tv.tree_verify_attn_paged(g["q"], p["k_pool"], p["v_pool"], p["table"],
                                         pl.page_size, g["cache_len"], p["tree_slot"], anc,
                                         status=status, split_keys=split_keys)
    torch.cuda.synchronize()
    assert (to_host(status) == 0).all(), to_host(status)
    o_out, o_lse = O.paged_attention(w.q, pl.k_pool, pl.v_pool, pl.block_table, pl.page_size,
                                     w.cache_len, pl.tree_slot, w.parent, rows=rows)
    got, got_lse = as_f64(to_host(out)), to_host(lse).astype(np.float64)
    if rows is not None:
        got = got[rows[:, 0], rows[:, 2], rows[:, 1]]
        got_lse = got_lse[rows[:, 0], rows[:, 2], rows[:, 1]]
    err = float(np.abs(got - o_out).max())
    lerr = float(np.abs(got_lse - o_lse).max())
    print(f"       max-abs err {err:.3e}  lse err {lerr:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= TOL_OUT[w.dtype] and lerr <= TOL_LSE[w.dtype], (err, lerr)
    return g, p, anc, out, lse


CASES = [
    ("p1_bf16_d128", 1, dict(B=3, T=60, L=(1, 700), Hq=8, Hkv=2, D=128, dtype="bf16")),
    ("p16_bf16_d128_t128", 16, dict(B=2, T=128, L=(0, 900), Hq=4, Hkv=2, D=128, dtype="bf16",
                                    parent_kind="random")),
    ("p64_bf16_d64", 64, dict(B=3, T=20, L=(63, 400), Hq=12, Hkv=3, D=64, dtype="bf16")),
    ("p256_bf16_d128", 256, dict(B=2, T=37, L=(200, 1100), Hq=8, Hkv=1, D=128, dtype="bf16")),
    ("p4_f32_d64", 4, dict(B=2, T=40, L=(0, 130), Hq=2, Hkv=1, D=64, dtype="f32",
                           parent_kind="chain")),
    ("p2_f32_d128", 2, dict(B=2, T=16, L=(5, 200), Hq=4, Hkv=2, D=128, dtype="f32")),
]


@pytest.mark.parametrize("label,P,kw", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("split_keys", [0, 64])
def test_paged_attention(label, P, kw, split_keys):
    w = make_workload("batch32_L512-4096_T60", **kw, extra_seed=21)
    _check_attn(w, make_paged(w, P, seed=3), split_keys=split_keys, label=label)


@pytest.mark.parametrize("name", ["llama8b_b1_L4096_T60", "batch32_L512-4096_T60"])
def test_paged_attention_full_size(name):
    w = make_workload(name)
    _check_attn(w, make_paged(w, 1, seed=4), rows=sample_rows(w, 120, seed=5), label=name)


def test_paged_equals_dense_bitwise():
    """Same rows, same chunks (fixed split_keys): the paged kernel reproduces the dense one bit
    for bit."""
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=4, T=60, L=(100, 1500), extra_seed=22)
    for P in (1, 32):
        g, p, anc, out, lse = _check_attn(w, make_paged(w, P, seed=6), split_keys=256,
                                          label=f"bitwise P={P}")
        out_d, lse_d = tv.tree_verify_attn(g["q"], g["k_cache"], g["v_cache"], g["cache_len"],
                                           g["k_tree"], g["v_tree"], anc, split_keys=256)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_d.view(torch.int16))
        assert torch.equal(lse, lse_d)


def test_paged_pool_over_4gb():
    """A bf16 pool larger than 4 GB per cache is addressed with 64-bit pointers (smaller pools
    take 32-bit offsets from the pool's base).  The workload's rows sit past the first 4 GB of
    an otherwise untouched pool; the result must equal the oracle's on the compact layout and,
    bit for bit, the same rows in a small pool."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    w = make_workload("batch32_L512-4096_T60", B=3, T=40, L=(20, 700), Hq=8, Hkv=2, D=128,
                      parent_kind="random", extra_seed=29)
    P = 16
    pl = make_paged(w, P, seed=13)
    slot_bytes = w.Hkv * w.D * 2
    shift_pages = -(-(1 << 32) // (slot_bytes * P))  # rows start past 4 GB
    shift = shift_pages * P
    big_slots = shift + pl.num_slots
    assert big_slots * slot_bytes > (1 << 32)
    print(f"[case] paged pool over 4 GB: {big_slots} slots, {2 * big_slots * slot_bytes / 2**30:.1f} GiB",
          flush=True)
    g = upload(w)
    kb = torch.empty((big_slots, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    kb[shift:] = to_dev(pl.k_pool)
    vb[shift:] = to_dev(pl.v_pool)
    table = np.where(pl.block_table >= 0, pl.block_table + shift_pages, -1).astype(np.int32)
    tslot = (pl.tree_slot + shift).astype(np.int32)
    anc, status = tv.tree_build_mask(g["parent"])
    out, lse = tv.tree_verify_attn_paged(g["q"], kb, vb, to_dev(table), P, g["cache_len"],
                                         to_dev(tslot), anc, status=status, split_keys=128)
    # the same rows in a compact pool (32-bit offsets)
    p = _paged_dev(pl)
    out_s, lse_s = tv.tree_verify_attn_paged(g["q"], p["k_pool"], p["v_pool"], p["table"], P,
                                             g["cache_len"], p["tree_slot"], anc, split_keys=128)
    torch.cuda.synchronize()
    assert (to_host(status) == 0).all(), to_host(status)
    assert torch.equal(out.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse, lse_s)
    o_out, o_lse = O.paged_attention(w.q, pl.k_pool, pl.v_pool, pl.block_table, P, w.cache_len,
                                     pl.tree_slot, w.parent)
    err = float(np.abs(as_f64(to_host(out)) - o_out).max())
    lerr = float(np.abs(to_host(lse).astype(np.float64) - o_lse).max())
    print(f"       max-abs err {err:.3e}  lse err {lerr:.3e}", flush=True)
    assert err <= TOL_OUT["bf16"] and lerr <= TOL_LSE["bf16"], (err, lerr)
    del kb, vb
    torch.cuda.empty_cache()


def test_paged_bad_entries_flagged_not_read():
    import tree_attention_verification_attn_amd as tv

    w = make_workload("batch32_L512-4096_T60", B=3, T=10, L=(30, 90), Hq=4, Hkv=1, D=128,
                      extra_seed=23)
    pl = make_paged(w, 4, seed=7)
    pl.block_table[1, 0] = pl.num_slots  # page past the pool
    pl.tree_slot[2, 3] = -5             # slot before the pool
    g, p = upload(w), _paged_dev(pl)
    anc, status = tv.tree_build_mask(g["parent"])
    out, lse = tv.tree_verify_attn_paged(g["q"], p["k_pool"], p["v_pool"], p["table"], 4,
                                         g["cache_len"], p["tree_slot"], anc, status=status)
    torch.cuda.synchronize()
    st = to_host(status)
    assert list(st & tv.TV_BAD_PAGE) == [0, tv.TV_BAD_PAGE, tv.TV_BAD_PAGE], st
    assert np.isfinite(as_f64(to_host(out))).all()


# ---- pointer-swap commit ----------------------------------------------------------------------
def _commit_case(w, pl, in_place=False, spare_top=0, label=""):
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    print(f"[case] commit {label} B={w.B} T={w.T}", flush=True)
    o_path, o_len, _ = O.accept(w.parent, w.draft, w.target)
    table = to_dev(pl.block_table)
    cl = to_dev(w.cache_len)
    free = torch.full((pl.num_slots,), -1, dtype=torch.int32, device="cuda")
    top = torch.tensor([spare_top], dtype=torch.int32, device="cuda")
    status = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    new_len = tv.kv_commit_paged(table, cl, to_dev(pl.tree_slot), to_dev(o_path),
                                 to_dev(o_len), free, top, pl.num_slots,
                                 cache_len_out=cl if in_place else None, status=status)
    torch.cuda.synchronize()
    h_table = pl.block_table.copy()
    h_free = np.full(pl.num_slots, -1, np.int32)
    o_new, o_top, o_st = O.commit_paged(h_table, w.cache_len, pl.tree_slot, o_path, o_len,
                                        pl.num_slots, h_free, spare_top)
    assert np.array_equal(to_host(table), h_table), f"{label}: block table differs"
    assert np.array_equal(to_host(new_len), o_new) and np.array_equal(to_host(status), o_st)
    assert int(to_host(top)[0]) == o_top
    got_free = to_host(free)
    assert sorted(got_free[spare_top:o_top]) == sorted(h_free[spare_top:o_top])
    assert (got_free[:spare_top] == -1).all() and (got_free[o_top:] == -1).all()
    return o_path, o_len


def test_commit_paged_matches_oracle():
    w = make_workload("batch32_L512-4096_T60", B=6, T=60, L=(20, 300), extra_seed=24)
    w.target[:, :-1] = np.where(np.arange(w.T - 1) % 3 == 0, w.draft[:, 1:], w.target[:, :-1])
    _commit_case(w, make_paged(w, 1, seed=8), spare_top=5, label="random trees")


def test_commit_paged_wide_tree_in_place_len():
    w = make_workload("wide_b64_L1024-8192_T128", B=5, L=(10, 90), extra_seed=25)
    _commit_case(w, make_paged(w, 1, seed=9), in_place=True, label="T=128, in-place length")


def test_commit_paged_bad_sequences():
    w = make_workload("batch32_L512-4096_T60", B=4, T=12, L=(30, 40), Hq=4, Hkv=1, D=128,
                      parent_kind="chain", extra_seed=26)
    w.target[:, :-1] = w.draft[:, 1:]  # every node accepted
    pl = make_paged(w, 1, seed=10, headroom=5)  # room for 5 more rows only: overflow
    pl.tree_slot[2, 4] = pl.num_slots + 1       # a slot outside the pool
    w.cache_len[3] = -2                         # bad length
    _commit_case(w, pl, label="overflow / bad slot / bad length")


def test_paged_step_commits_the_accepted_rows():
    """mask -> paged attention -> acceptance -> pointer-swap commit on the device: the rows
    the new table names after the prefix are the accepted nodes' rows, in path order."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    w = make_workload("llama8b_b1_L4096_T60", extra_seed=27)
    pl = make_paged(w, 1, seed=11)
    g, p = upload(w), _paged_dev(pl)
    anc, status = tv.tree_build_mask(g["parent"])
    tv.tree_verify_attn_paged(g["q"], p["k_pool"], p["v_pool"], p["table"], 1, g["cache_len"],
                              p["tree_slot"], anc, status=status)
    path, alen, bonus = tv.tree_accept(anc, g["draft"], g["target"])
    free = torch.full((pl.num_slots,), -1, dtype=torch.int32, device="cuda")
    top = torch.zeros(1, dtype=torch.int32, device="cuda")
    new_len = tv.kv_commit_paged(p["table"], g["cache_len"], p["tree_slot"], path, alen, free,
                                 top, pl.num_slots, status=status)
    torch.cuda.synchronize()
    o_path, o_len, _ = O.accept(w.parent, w.draft, w.target)
    n, L = int(o_len[0]), int(w.cache_len[0])
    assert int(to_host(new_len)[0]) == L + n and (to_host(status) == 0).all()
    table = to_host(p["table"])
    kp = pl.k_pool.view(np.uint16)
    for i in range(n):
        assert (kp[table[0, L + i]] == w.k_tree[0, o_path[0, i]].view(np.uint16)).all()
    assert int(to_host(top)[0]) == w.T - n
