"""Helpers shared by the GPU tests: upload synthetic workloads, run the HIP path through the C
ABI binding, run the CPU oracle on the same host bytes, compare."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O

# Tolerances.  Attention outputs: max-abs error 1e-5 for fp32 inputs and 2e-2 for bf16 inputs
# with fp32 accumulation.  lse carries no bf16 rounding of P (the row sums are accumulated from
# the fp32 probabilities), so it is held to 1e-3 for bf16 inputs and 1e-5 for fp32.
TOL_OUT = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = {"f32": 1e-5, "bf16": 1e-3}


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bfloat16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def upload(w) -> dict:
    return dict(parent=to_dev(w.parent), draft=to_dev(w.draft), target=to_dev(w.target),
                cache_len=to_dev(w.cache_len), q=to_dev(w.q), k_cache=to_dev(w.k_cache),
                v_cache=to_dev(w.v_cache), k_tree=to_dev(w.k_tree), v_tree=to_dev(w.v_tree))


def run_step(g: dict, split_keys: int = 0, tv=None):
    """mask -> attention -> acceptance -> compaction on the device; host copies of results."""
    import tree_attention_verification_attn_amd as tvmod

    tv = tv or tvmod
    anc, status = tv.tree_build_mask(g["parent"])
    out, lse = tv.tree_verify_attn(g["q"], g["k_cache"], g["v_cache"], g["cache_len"],
                                   g["k_tree"], g["v_tree"], anc, status=status,
                                   split_keys=split_keys)
    path, alen, bonus = tv.tree_accept(anc, g["draft"], g["target"])
    new_len = tv.kv_compact_accepted(g["k_cache"], g["v_cache"], g["cache_len"], g["k_tree"],
                                     g["v_tree"], path, alen, status=status)
    torch.cuda.synchronize()
    return dict(anc=to_host(anc).view(np.uint64), status=to_host(status), out=to_host(out),
                lse=to_host(lse), path=to_host(path), alen=to_host(alen), bonus=to_host(bonus),
                new_len=to_host(new_len), k_cache=to_host(g["k_cache"]),
                v_cache=to_host(g["v_cache"]))


def run_step_fused(g: dict, split_keys: int = 0, in_place_len: bool = False, tv=None):
    """The same step through the fused entry point tree_verify_step."""
    import tree_attention_verification_attn_amd as tvmod

    tv = tv or tvmod
    r = tv.tree_verify_step(g["parent"], g["draft"], g["target"], g["q"], g["k_cache"],
                            g["v_cache"], g["cache_len"], g["k_tree"], g["v_tree"],
                            cache_len_out=g["cache_len"] if in_place_len else None,
                            split_keys=split_keys)
    torch.cuda.synchronize()
    return dict(anc=to_host(r["anc_mask"]).view(np.uint64), status=to_host(r["status"]),
                out=to_host(r["out"]), lse=to_host(r["lse"]), path=to_host(r["accept_path"]),
                alen=to_host(r["accept_len"]), bonus=to_host(r["bonus_tok"]),
                new_len=to_host(r["cache_len_out"]), k_cache=to_host(g["k_cache"]),
                v_cache=to_host(g["v_cache"]))


def sample_rows(w, n_random: int, seed: int = 0) -> np.ndarray:
    """(b, h, i) rows: corners of every axis; one row of every 32-row group of every (sequence,
    KV head) unit, where a unit's rows are node * G + g over its G query heads (one wavefront of
    the main kernel owns such a group, eight of them a workgroup), so every wavefront of every
    work item that the kernel's longest-first and XCD-aware dispatch reorders is checked; plus
    uniform random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in {0, w.B - 1}:
        for h in {0, w.Hq - 1, w.G - 1, w.G % w.Hq}:
            for i in {0, w.T - 1, w.T // 2}:
                rows.add((b, h, i))
    GT = w.G * w.T
    for b in range(w.B):
        for kvh in range(w.Hkv):
            for r0 in range(0, GT, 32):
                r = int(rng.integers(r0, min(r0 + 32, GT)))
                rows.add((b, kvh * w.G + r % w.G, r // w.G))
    target = len(rows) + n_random
    while len(rows) < target:
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.T))))
    return np.array(sorted(rows), np.int32)


# Sharp softmax (a large explicit scale, peaked rows): an output row approaches one V row, whose
# entries reach 4..5 for N(0,1) values.  A bf16 output of that size carries up to 2^-8 of its
# value from its own rounding, and the bf16 rounding of P before P.V adds up to 2^-8 of
# sum p|v| / l, which is then about |o|.  Those cases are held to 2e-2 + 2^-7 |o|, elementwise.
RTOL_SHARP = {"f32": 0.0, "bf16": 2.0 ** -7}


def score_error_bound(w, scale: float | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Float32 rounding bound of the scores, per row (b, node, query head): a score
    scale * sum_d q_d k_d accumulated in float32 errs by at most (D + 3) 2^-24 scale
    sum_d |q_d k_d| (D products and sums, the scale, the log2(e) factor, the exponent).  Taken
    over every prefix and tree key of the row's KV head (a superset of the visible keys).
    Perturbing the scores by at most ds moves the softmax output by at most 2 ds max|v| and lse
    by at most ds.  Returns (ds [B, T, Hq], max|v| [B, T, Hq])."""
    scale = w.scale if scale is None else scale
    G = w.Hq // w.Hkv
    ds = np.zeros((w.B, w.T, w.Hq))
    vmax = np.zeros((w.B, w.T, w.Hq))
    for b in range(w.B):
        L = int(np.clip(w.cache_len[b], 0, w.Lmax))
        for kvh in range(w.Hkv):
            K = np.abs(np.concatenate([as_f64(w.k_cache[b, kvh, :L]), as_f64(w.k_tree[b, :, kvh])]))
            V = np.abs(np.concatenate([as_f64(w.v_cache[b, kvh, :L]), as_f64(w.v_tree[b, :, kvh])]))
            Q = np.abs(as_f64(w.q[b, :, kvh * G:(kvh + 1) * G]))  # [T, G, D]
            mag = (Q.reshape(-1, w.D) @ K.T).max(axis=1).reshape(w.T, G)
            ds[b, :, kvh * G:(kvh + 1) * G] = (w.D + 3) * 2.0 ** -24 * scale * mag
            vmax[b, :, kvh * G:(kvh + 1) * G] = V.max()
    return ds, vmax


def check_step(w, res: dict, rows: np.ndarray | None = None, label: str = "",
               rtol: float = 0.0, score_err: tuple | None = None) -> dict:
    """Compare a device step with the oracle.  Integer results and the cache bytes must match
    exactly; attention within the dtype's tolerance (all rows, or the sampled ones), plus
    `rtol` times the exact value's magnitude, plus (with `score_err` from score_error_bound)
    what the float32 rounding of the scores can move the output and lse by."""
    o_anc, o_st = O.build_mask(w.parent)
    assert np.array_equal(res["anc"], o_anc), f"{label}: ancestor mask differs"
    o_path, o_len, o_bonus = O.accept(w.parent, w.draft, w.target)
    assert np.array_equal(res["path"], o_path), f"{label}: accept_path differs"
    assert np.array_equal(res["alen"], o_len), f"{label}: accept_len differs"
    assert np.array_equal(res["bonus"], o_bonus), f"{label}: bonus_tok differs"

    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    o_st2 = o_st.copy()
    L_clamped = np.clip(w.cache_len, 0, w.Lmax).astype(np.int32)
    o_new_len, o_st2 = O.compact(kc, vc, w.cache_len, w.k_tree, w.v_tree, o_path, o_len, o_st2)
    bad_len = (w.cache_len < 0) | (w.cache_len > w.Lmax)
    o_st2 = o_st2 | np.where(bad_len, O.ORC_BAD_LEN, 0).astype(np.int32)
    assert np.array_equal(res["new_len"], o_new_len), f"{label}: cache_len_out differs"
    assert np.array_equal(res["status"], o_st2), f"{label}: status {res['status']} vs {o_st2}"
    bits = np.uint32 if kc.dtype == np.float32 else np.uint16
    assert np.array_equal(res["k_cache"].view(bits), kc.view(bits)), f"{label}: K cache differs"
    assert np.array_equal(res["v_cache"].view(bits), vc.view(bits)), f"{label}: V cache differs"

    out = as_f64(res["out"])
    if rows is None:
        o_out, o_lse = O.attention(w.q, w.k_cache, w.v_cache, L_clamped, w.k_tree, w.v_tree,
                                   w.parent)
        got, got_lse = out, res["lse"].astype(np.float64)
    else:
        o_out, o_lse = O.attention(w.q, w.k_cache, w.v_cache, L_clamped, w.k_tree, w.v_tree,
                                   w.parent, rows=rows)
        got = out[rows[:, 0], rows[:, 2], rows[:, 1]]
        got_lse = res["lse"][rows[:, 0], rows[:, 2], rows[:, 1]].astype(np.float64)
    err = float(np.abs(got - o_out).max())
    lerr = float(np.abs(got_lse - o_lse).max())
    assert np.isfinite(got).all(), f"{label}: non-finite attention output"
    tol_o, tol_l = TOL_OUT[w.dtype] + rtol * np.abs(o_out), np.full(o_lse.shape, TOL_LSE[w.dtype])
    if score_err is not None:
        ds, vmax = score_err
        if rows is not None:
            ds, vmax = ds[rows[:, 0], rows[:, 2], rows[:, 1]], vmax[rows[:, 0], rows[:, 2], rows[:, 1]]
        tol_o = tol_o + (2 * ds * vmax)[..., None]
        tol_l = tol_l + ds
    excess = float((np.abs(got - o_out) - tol_o).max())
    assert excess <= 0, f"{label}: attention max-abs error {err} (rtol {rtol})"
    assert (np.abs(got_lse - o_lse) <= tol_l).all(), f"{label}: lse max-abs error {lerr}"
    return dict(err=err, lse_err=lerr)
