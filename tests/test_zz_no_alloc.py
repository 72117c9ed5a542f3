"""tree_verify_step_noalloc (the step whose split-K workspace is the library's own device array)
against tree_verify_step with a caller workspace, through the C ABI.

Both run the same kernels with the same split plan, so every output must be bit-identical; the
no-allocation results are also checked against the CPU oracle (masks, acceptance and cache bytes
exactly, attention within max-abs 2e-2 / 1e-5).  Two calls in a row share the one array: the
second, on a smaller input with fewer chunks, must not see anything the first left behind."""
import numpy as np
import pytest
import torch

from gpu_util import check_step, to_host, upload
from synth import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tree_attention_verification_attn_amd as tv

    tv.load_library()


def _host(r, g):
    out = {k: to_host(v) for k, v in r.items()}
    out["anc_mask"] = out["anc_mask"].view(np.uint64)
    out["k_cache"], out["v_cache"] = to_host(g["k_cache"]), to_host(g["v_cache"])
    return out


def _step(w, noalloc, split_keys):
    import tree_attention_verification_attn_amd as tv

    g = upload(w)
    fn = tv.tree_verify_step_noalloc if noalloc else tv.tree_verify_step
    r = fn(g["parent"], g["draft"], g["target"], g["q"], g["k_cache"], g["v_cache"],
           g["cache_len"], g["k_tree"], g["v_tree"], split_keys=split_keys)
    torch.cuda.synchronize()
    return _host(r, g)


def _as_check(res):
    return dict(anc=res["anc_mask"], status=res["status"], out=res["out"], lse=res["lse"],
                path=res["accept_path"], alen=res["accept_len"], bonus=res["bonus_tok"],
                new_len=res["cache_len_out"], k_cache=res["k_cache"], v_cache=res["v_cache"])


CASES = [
    # (label, workload, overrides, split_keys)
    ("llama8b_b1_auto", "llama8b_b1_L4096_T60", {}, 0),
    ("batch6_split192", "batch32_L512-4096_T60", dict(B=6, L=(100, 1500)), 192),
    ("fp32_small_split64", "batch32_L512-4096_T60",
     dict(B=3, T=20, L=(5, 300), Hq=4, Hkv=2, D=64, dtype="f32", parent_kind="random"), 64),
]


def test_noalloc_matches_step_twice():
    """A large call, then a smaller one: bit-identical to tree_verify_step each time."""
    for label, name, kw, sk in CASES:
        w = make_workload(name, extra_seed=95, **kw)
        print(f"[case] noalloc {label} B={w.B} T={w.T} Lmax={w.Lmax} {w.dtype} split_keys={sk}",
              flush=True)
        a = _step(w, True, sk)
        b = _step(w, False, sk)
        for k in a:
            x, y = np.asarray(a[k]), np.asarray(b[k])
            assert x.shape == y.shape, (label, k)
            assert np.array_equal(x.reshape(-1).view(np.uint8), y.reshape(-1).view(np.uint8)), \
                (label, k)
        check_step(w, _as_check(a), label=label)


def test_noalloc_rejects_plans_beyond_its_array():
    import ctypes

    import tree_attention_verification_attn_amd as tv

    lib = tv.load_library()
    fake = ctypes.c_void_p(0x1000)
    # 64-key chunks over a 65536-token cache at batch 64: far more partials than the array holds
    need = lib.tree_verify_attn_workspace_size(64, 128, 32, 8, 128, 65536, tv.TV_BF16, 64)
    assert need > lib_limit()
    rc = lib.tree_verify_step_noalloc(*([fake] * 17), 64, 128, 32, 8, 128, 65536, tv.TV_BF16,
                                      ctypes.c_float(0.0), 64, None)
    assert rc == tv.TV_ERR_WORKSPACE


def lib_limit():
    import os
    import re

    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                       "tree_verify.h")
    m = re.search(r"#define TV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(hdr).read())
    return int(m.group(1)) << int(m.group(2))


def test_noalloc_step_replays_in_a_graph():
    """The use the entry point is for: the step captured in a HIP graph with no allocation in
    it (every output passed in).  Replays, with eager calls on other inputs in between that use
    the same device array, equal the eager result bit for bit."""
    import tree_attention_verification_attn_amd as tv
    from test_gpu_graph import _poison, _replays_match_eager, _step_buffers

    w = make_workload("batch32_L512-4096_T60", B=5, T=60, L=(0, 900), Hq=8, Hkv=2, D=128,
                      extra_seed=96)
    w2 = make_workload("batch32_L512-4096_T60", B=5, T=60, L=(0, 900), Hq=8, Hkv=2, D=128,
                       extra_seed=97)
    g, g2 = upload(w), upload(w2)
    bufs, bufs2 = _step_buffers(g, w), _step_buffers(g2, w2)
    split = 128

    def step(x, b):
        tv.tree_verify_step_noalloc(x["parent"], x["draft"], x["target"], x["q"], x["k_cache"],
                                    x["v_cache"], x["cache_len"], x["k_tree"], x["v_tree"],
                                    split_keys=split, **b)

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
    _replays_match_eager("tree_verify_step_noalloc", lambda: step(g, bufs), outs,
                         lambda: step(g2, bufs2), poison=poison)
    assert int(bufs["status"].abs().sum()) == 0
