"""GPU parity of the fused verification step (tree_verify_step, through the C ABI) against
the CPU oracle, and against the four separate entry points.

The fused step runs the mask kernel, the attention main kernel and one kernel that merges the
split-K partials while other workgroups run the acceptance walk and the compaction.  Every
output is compared as in the separate-call tests: masks, acceptance, compaction and status bits
exactly (cache bytes included), attention within max-abs 1e-5 (fp32) or 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

from gpu_util import check_step, run_step, run_step_fused, sample_rows, to_dev, to_host, upload
from synth import make_workload
from test_gpu_parity import EDGE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _fused_check(w, rows=None, split_keys=0, label="", in_place_len=False):
    print(f"[case] fused {label} B={w.B} T={w.T} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
          f"Lmax={w.Lmax} {w.dtype} split_keys={split_keys} in_place={in_place_len}", flush=True)
    res = run_step_fused(upload(w), split_keys=split_keys, in_place_len=in_place_len)
    stats = check_step(w, res, rows=rows, label=label)
    print(f"       max-abs err {stats['err']:.3e}  lse err {stats['lse_err']:.3e}", flush=True)
    return res


def test_step_worked_tree_fp32():
    _fused_check(make_workload("worked_tree_fp32"), label="worked_tree_fp32")


def test_step_llama8b_b1():
    _fused_check(make_workload("llama8b_b1_L4096_T60"), label="llama8b_b1_L4096_T60")


@pytest.mark.parametrize("name", ["batch32_L512-4096_T60", "llama70b_b8_L32768_T64",
                                  "wide_b64_L1024-8192_T128"])
def test_step_full_size_sampled(name):
    w = make_workload(name)
    _fused_check(w, rows=sample_rows(w, 120, seed=2), label=name)


@pytest.mark.parametrize("split_keys", [64, 100000])
def test_step_split_settings(split_keys):
    w = make_workload("batch32_L512-4096_T60", B=5, extra_seed=11)
    _fused_check(w, split_keys=split_keys, label=f"split {split_keys}")


@pytest.mark.parametrize("label,kw", EDGE[:5], ids=[e[0] for e in EDGE[:5]])
def test_step_edge_cases(label, kw):
    _fused_check(make_workload("batch32_L512-4096_T60", **kw, extra_seed=12), split_keys=64,
                 label=label)


def test_step_matches_separate_calls_bitwise():
    """Same kernels, same arithmetic: the fused step reproduces the separate calls bit for
    bit, including the merged attention output and lse."""
    w = make_workload("batch32_L512-4096_T60", B=4, T=60, L=(100, 900), extra_seed=13)
    a = run_step(upload(w), split_keys=192)
    b = run_step_fused(upload(w), split_keys=192)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


def test_step_status_bits():
    w = make_workload("batch32_L512-4096_T60", B=4, T=10, L=(20, 40), Hq=4, Hkv=2, D=128,
                      parent_kind="random", extra_seed=14)
    w.parent[1, 3] = 3   # self parent
    w.cache_len[2] = -3  # negative prefix length
    res = _fused_check(w, label="status bits")
    assert list(res["status"] & 1) == [0, 1, 0, 0]
    assert list(res["status"] & 4) == [0, 0, 4, 0]


def test_step_overflow():
    w = make_workload("batch32_L512-4096_T60", B=2, T=30, L=(100, 100), Hq=4, Hkv=2, D=128,
                      parent_kind="chain", extra_seed=15, lmax_pad=1)
    w.target[:, :-1] = w.draft[:, 1:]
    w.target[0, 5] = -1
    Lmax = w.Lmax - 1
    w.k_cache = np.ascontiguousarray(w.k_cache[:, :, :Lmax])
    w.v_cache = np.ascontiguousarray(w.v_cache[:, :, :Lmax])
    w.Lmax = Lmax
    res = _fused_check(w, label="overflow")
    assert res["status"][1] & 2 and not res["status"][0] & 2
    assert list(res["new_len"]) == [106, 100]


def test_step_cache_len_in_place():
    w = make_workload("batch32_L512-4096_T60", B=5, T=12, L=(300, 900), Hq=8, Hkv=4, D=128,
                      parent_kind="chain", extra_seed=16)
    w.target[:, :-1] = w.draft[:, 1:]
    # the merge must not see the lengths the compaction writes: use a split setting
    _fused_check(w, split_keys=64, label="in-place cache_len", in_place_len=True)


def test_step_tree_rows_inside_cache():
    """Tree K/V stored in the cache's own tail: the step falls back to staged compaction."""
    import tree_attention_verification_attn_amd as tv
    from oracle import oracle as O

    w = make_workload("worked_tree_fp32", dtype="bf16", D=128, extra_seed=17)
    L, T = int(w.cache_len[0]), w.T
    w.k_cache[0, 0, L:L + T] = w.k_tree[0, :, 0]
    w.v_cache[0, 0, L:L + T] = w.v_tree[0, :, 0]
    g = upload(w)
    g["k_tree"] = g["k_cache"][:, 0, L:L + T, :].reshape(1, T, 1, w.D)
    g["v_tree"] = g["v_cache"][:, 0, L:L + T, :].reshape(1, T, 1, w.D)
    res = run_step_fused(g)
    o_path, o_len, _ = O.accept(w.parent, w.draft, w.target)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    o_new, _ = O.compact(kc, vc, w.cache_len, w.k_tree, w.v_tree, o_path, o_len)
    assert np.array_equal(res["path"], o_path) and np.array_equal(res["new_len"], o_new)
    assert np.array_equal(res["k_cache"].view(np.uint16), kc.view(np.uint16))
    assert np.array_equal(res["v_cache"].view(np.uint16), vc.view(np.uint16))
