"""GPU parity on the numeric edge cases of tree attention, through the C ABI.

* Split-K chunks in which a row sees no key at all: with 64-key chunks and T > 64, the second
  tree tile is a chunk of its own and the rows of nodes 0..63 hold none of their ancestors in
  it.  Such a chunk carries m = -inf, l = 0, O = 0 and must weigh nothing in the merge, also
  when the merge's chunk group holds nothing else.
* An explicit softmax scale (the ABI's `scale` argument) instead of the default 1/sqrt(D).
* Peaked rows: one key scores far above the rest of its row, late in a long chunk (after the
  running max is set) or as a tree ancestor at the start of the chunk.  40 above the row's
  other scores forces a rescale of the running sums; 100 above makes 2^(score - running max)
  overflow float32, which the lazy rescale must catch.

The sharp-softmax cases (scale 8/sqrt(D), peaked rows) are held to 2e-2 + 2^-7 |o| in bf16: an
output row then approaches a single V row, and the bf16 output type alone rounds a value of 4
by up to 0.016.  Their scores are large (tens to 100), so both types also get what the float32
rounding of a score of that size can move the output and lse by (gpu_util.score_error_bound).

Each case runs the four separate calls and the fused step (tree_verify_step) and compares
against the CPU oracle: masks, acceptance and cache bytes exactly, attention within max-abs
1e-5 (fp32) or 2e-2 (bf16), lse within 1e-5 / 1e-3.
"""
import numpy as np
import pytest
import torch

from gpu_util import (RTOL_SHARP, TOL_LSE, TOL_OUT, as_f64, check_step, run_step, run_step_fused,
                      score_error_bound, to_host, upload)
from oracle import oracle as O
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _run(w, fused, split_keys, label, rtol=0.0, score_err=None):
    print(f"[case] {label} fused={fused} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
          f"Lmax={w.Lmax} {w.dtype} split_keys={split_keys}", flush=True)
    g = upload(w)
    res = run_step_fused(g, split_keys=split_keys) if fused else run_step(g, split_keys=split_keys)
    stats = check_step(w, res, label=label, rtol=rtol, score_err=score_err)
    print(f"       max-abs err {stats['err']:.3e}  lse err {stats['lse_err']:.3e}", flush=True)
    return res


# ---- chunks without a visible key ------------------------------------------------------------
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("short_len", [0, 100, 192, 193])
def test_merge_chunk_without_visible_keys(fused, short_len):
    """T = 128 in 64-key chunks over a long Lmax: more than 8 chunks per row block, so the merge
    splits a row's chunks over four groups (group k takes chunks k, k + 4, ...).  A sequence
    with at most three prefix tiles leaves group 1 holding only chunk 1, the second tree tile,
    in which nodes 0..63 see nothing."""
    w = make_workload("wide_b64_L1024-8192_T128", B=3, L=(900, 1100), Hq=8, Hkv=2,
                      parent_kind="random", extra_seed=90)
    w.cache_len[1] = short_len
    tiles = 2 + -(-w.Lmax // 64)
    assert tiles > 8  # the plan's chunk count S at 64-key chunks
    _run(w, fused, 64, f"empty chunk L={short_len}")


# ---- explicit scale --------------------------------------------------------------------------
def _attn_with_scale(w, scale, split_keys, fused):
    import tree_attention_verification_attn_amd as tv

    g = upload(w)
    if fused:
        r = tv.tree_verify_step(g["parent"], g["draft"], g["target"], g["q"], g["k_cache"],
                                g["v_cache"], g["cache_len"], g["k_tree"], g["v_tree"],
                                scale=scale, split_keys=split_keys)
        out, lse = r["out"], r["lse"]
    else:
        anc, _ = tv.tree_build_mask(g["parent"])
        out, lse = tv.tree_verify_attn(g["q"], g["k_cache"], g["v_cache"], g["cache_len"],
                                       g["k_tree"], g["v_tree"], anc, scale=scale,
                                       split_keys=split_keys)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("scale_mul", [0.3, 8.0])
@pytest.mark.parametrize("split_keys", [0, 64])
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_explicit_scale(dtype, D, scale_mul, split_keys, fused):
    w = make_workload("batch32_L512-4096_T60", B=3, T=40, L=(50, 400), Hq=8, Hkv=2, D=D,
                      dtype=dtype, parent_kind="random", extra_seed=91)
    scale = float(np.float32(scale_mul / np.sqrt(D)))
    print(f"[case] scale {scale:.5f} {dtype} D={D} split_keys={split_keys} fused={fused}",
          flush=True)
    out, lse = _attn_with_scale(w, scale, split_keys, fused)
    o_out, o_lse = O.attention(w.q, w.k_cache, w.v_cache, w.cache_len, w.k_tree, w.v_tree,
                               w.parent, scale=scale)
    err = float(np.abs(as_f64(out) - o_out).max())
    lerr = float(np.abs(lse.astype(np.float64) - o_lse).max())
    print(f"       max-abs err {err:.3e}  lse err {lerr:.3e}", flush=True)
    assert np.isfinite(as_f64(out)).all()
    rtol = RTOL_SHARP[dtype] if scale_mul > 1 else 0.0
    ds, vmax = score_error_bound(w, scale) if scale_mul > 1 else (0.0, 0.0)
    tol_o = TOL_OUT[dtype] + rtol * np.abs(o_out) + np.asarray(2 * ds * vmax)[..., None]
    assert (np.abs(as_f64(out) - o_out) <= tol_o).all(), err
    assert (np.abs(lse.astype(np.float64) - o_lse) <= TOL_LSE[dtype] + ds).all(), lerr
    # the default scale differs from this one: the results must too (the argument is used)
    d_out, _ = _attn_with_scale(w, 0.0, split_keys, fused)
    assert np.abs(as_f64(d_out) - as_f64(out)).max() > 10 * TOL_OUT[dtype]


# ---- peaked rows -----------------------------------------------------------------------------
def _plant(w, b, t, h, key, peak, where):
    """Make key `key` (a prefix position, or a tree node) score `peak` for row (b, t, h):
    k = alpha q with alpha = peak / (scale |q|^2)."""
    G = w.Hq // w.Hkv
    kvh = h // G
    if w.dtype == "f32":
        qv = w.q[b, t, h].astype(np.float64)
    else:
        qv = bf16_bits_to_f32(w.q[b, t, h]).astype(np.float64)
    alpha = peak / (w.scale * float(qv @ qv))
    kv = (alpha * qv).astype(np.float32)
    bits = kv if w.dtype == "f32" else f32_to_bf16_bits(kv)
    if where == "late_prefix":
        w.k_cache[b, kvh, key] = bits
    else:
        w.k_tree[b, key, kvh] = bits


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("peak", [40.0, 100.0])
@pytest.mark.parametrize("where", ["late_prefix", "tree_ancestor"])
@pytest.mark.parametrize("split_keys", [0, 100000])
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_peaked_rows(dtype, peak, where, split_keys, fused):
    D = 128 if dtype == "bf16" else 64
    w = make_workload("batch32_L512-4096_T60", B=2, T=60, L=(1500, 2000), Hq=8, Hkv=2, D=D,
                      dtype=dtype, parent_kind="random", extra_seed=92)
    rng = np.random.default_rng(7)
    planted = []
    for b in range(w.B):
        for _ in range(3):
            if where == "late_prefix":
                t = int(rng.integers(w.T))
                key = int(w.cache_len[b]) - 1 - int(rng.integers(40))  # in the last tile(s)
            else:
                # a node whose parent sits in the second 32-key block, when there is one: the
                # running max is then already set by the first block when the peak arrives
                cands = [i for i in range(1, w.T) if w.parent[b, i] >= 32] or list(range(1, w.T))
                t = int(rng.choice(cands))
                key = int(w.parent[b, t])
            h = int(rng.integers(w.Hq))
            _plant(w, b, t, h, key, peak, where)
            planted.append((b, h, t))
    res = _run(w, fused, split_keys, f"peak {peak} {where}", rtol=RTOL_SHARP[dtype],
               score_err=score_error_bound(w))
    # the planted rows are dominated by their planted key: output close to that key's V row
    out = as_f64(res["out"])
    for b, h, t in planted:
        assert np.isfinite(out[b, t, h]).all()
