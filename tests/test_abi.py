"""The C ABI of libtreeverify.so without a GPU: it loads, exports every function declared in
include/tree_verify.h, and reports host-checkable argument errors before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_verify.h")


@pytest.fixture(scope="module")
def lib():
    import tree_attention_verification_attn_amd as tv
    from tree_attention_verification_attn_amd import build

    if not os.path.exists(build.LIB):
        build.build_library()
    return tv.load_library()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_][a-z_0-9]*)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ("tree_build_mask", "tree_verify_attn", "tree_verify_attn_workspace_size",
               "tree_accept", "kv_compact_accepted", "tv_status_string"):
        assert fn in names


def test_library_exports_every_declared_function(lib):
    from tree_attention_verification_attn_amd import build

    out = subprocess.run(["nm", "-D", "--defined-only", build.LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for fn in declared_functions():
        assert fn in exported, fn
        assert hasattr(lib, fn)


def test_header_compiles_as_c():
    src = '#include "tree_verify.h"\nint main(void){return TV_OK + TV_F32 + TV_BAD_TREE * 0;}\n'
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-x", "c", "-I",
                    os.path.join(ROOT, "include"), "-", "-o", "/dev/null"], input=src, text=True,
                   check=True)


def test_status_strings(lib):
    import tree_attention_verification_attn_amd as tv

    for code in (tv.TV_OK, tv.TV_ERR_INVALID_ARG, tv.TV_ERR_UNSUPPORTED, tv.TV_ERR_WORKSPACE,
                 tv.TV_ERR_HIP, tv.TV_BAD_TREE, tv.TV_OVERFLOW, tv.TV_BAD_LEN, tv.TV_BAD_PATH,
                 tv.TV_BAD_PAGE, tv.TV_BAD_TOKEN, tv.TV_SYNC_TIMEOUT, tv.TV_BAD_CONF,
                 tv.TV_FREE_FULL):
        assert lib.tv_status_string(code)
    assert b"TV_BAD_TOKEN" in lib.tv_status_string(tv.TV_BAD_TOKEN)
    assert b"TV_FREE_FULL" in lib.tv_status_string(tv.TV_FREE_FULL)
    assert b"unknown" in lib.tv_status_string(12345)


# A fake non-null pointer: every call below must be rejected before it is dereferenced.
FAKE = ctypes.c_void_p(0x1000)


def test_build_mask_argument_errors(lib):
    assert lib.tree_build_mask(None, 1, 8, FAKE, FAKE, None) == -1
    assert lib.tree_build_mask(FAKE, 1, 8, None, FAKE, None) == -1
    assert lib.tree_build_mask(FAKE, 1, 8, FAKE, None, None) == -1
    assert lib.tree_build_mask(FAKE, 0, 8, FAKE, FAKE, None) == -1
    assert lib.tree_build_mask(FAKE, 1, 0, FAKE, FAKE, None) == -1
    assert lib.tree_build_mask(FAKE, 1, 129, FAKE, FAKE, None) == -1


def _attn(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, cl=FAKE, kt=FAKE, vt=FAKE, anc=FAKE, out=FAKE, lse=None,
             st=None, B=1, T=8, Hq=2, Hkv=1, D=64, Lmax=16, dt=0, scale=0.0, split=0, ws=None,
             wsb=0)
    a.update(kw)
    return lib.tree_verify_attn(a["q"], a["kc"], a["vc"], a["cl"], a["kt"], a["vt"], a["anc"],
                                a["out"], a["lse"], a["st"], a["B"], a["T"], a["Hq"], a["Hkv"],
                                a["D"], a["Lmax"], a["dt"], a["scale"], a["split"], a["ws"],
                                a["wsb"], None)


def test_attention_argument_errors(lib):
    for name in ("q", "kc", "vc", "cl", "kt", "vt", "anc", "out"):
        assert _attn(lib, **{name: None}) == -1, name
    assert _attn(lib, B=0) == -1
    assert _attn(lib, T=0) == -1
    assert _attn(lib, T=129) == -1
    assert _attn(lib, Hq=3, Hkv=2) == -1
    assert _attn(lib, Hkv=0) == -1
    assert _attn(lib, Lmax=-1) == -1
    assert _attn(lib, split=-64) == -1
    assert _attn(lib, D=96) == -2
    assert _attn(lib, dt=7) == -2
    # split-K over a long prefix needs a workspace
    need = lib.tree_verify_attn_workspace_size(1, 8, 2, 1, 64, 4096, 0, 256)
    assert need > 0
    assert _attn(lib, Lmax=4096, split=256) == -3
    assert _attn(lib, Lmax=4096, split=256, ws=FAKE, wsb=need - 1) == -3
    # row offsets are 32-bit within a (b, kvh) cache slab and a sequence's tree rows
    big = 1 << 62
    assert _attn(lib, Lmax=(1 << 24) + 1, D=128, dt=1, ws=FAKE, wsb=big) == -1
    assert _attn(lib, Lmax=(1 << 23) + 1, D=128, dt=0, ws=FAKE, wsb=big) == -1
    assert _attn(lib, T=128, Hq=131073, Hkv=131073, D=128, dt=1, ws=FAKE, wsb=big) == -1
    # rows are read and written 16 bytes at a time
    for name in ("q", "kc", "vc", "kt", "vt", "out"):
        assert _attn(lib, **{name: ctypes.c_void_p(0x1008)}) == -1, name


def test_workspace_size_rules(lib):
    ws = lib.tree_verify_attn_workspace_size
    # one chunk covers the prefix: no workspace
    assert ws(1, 8, 2, 1, 64, 16, 0, 1024) == 0
    # 1 tree tile + 64 prefix tiles in chunks of 4 tiles -> 17 chunks, one 256-row block:
    # S * 256 rows * (D fp32 partial O + 2 fp32 statistics), then one int32 chunk count per
    # sequence
    assert ws(1, 8, 2, 1, 64, 4096, 0, 256) == 17 * 256 * (64 * 4 + 8) + 1 * 4
    # G*T = 8*60 = 480 rows -> 2 row blocks of 256; 65 tiles in chunks of 32 -> 3 chunks;
    # the partial O is fp32 for bf16 inputs too
    assert ws(2, 60, 64, 8, 128, 4096, 1, 2048) == 2 * 8 * 2 * 3 * 256 * (128 * 4 + 8) + 2 * 4
    # bad arguments report 0
    assert ws(1, 8, 3, 2, 64, 4096, 0, 0) == 0
    assert ws(1, 8, 2, 1, 80, 4096, 0, 0) == 0


def test_step_argument_errors(lib):
    # 17 device pointers, then B, T, Hq, Hkv, D, Lmax, dtype, scale, split_keys, ws, ws_bytes,
    # stream
    base = [FAKE] * 17 + [1, 8, 2, 1, 64, 16, 0, 0.0, 0, None, 0, None]
    for i in list(range(12)) + list(range(13, 17)):  # every pointer but lse is required
        bad = list(base)
        bad[i] = None
        assert lib.tree_verify_step(*bad) == -1, i
    bad = list(base)
    bad[12] = None  # lse is optional
    bad[17] = 0     # B = 0 -> rejected before any launch
    assert lib.tree_verify_step(*bad) == -1
    bad = list(base)
    bad[21] = 96    # head_dim
    assert lib.tree_verify_step(*bad) == -2
    bad = list(base)
    bad[3] = ctypes.c_void_p(0x1008)  # q not 16-byte aligned
    assert lib.tree_verify_step(*bad) == -1
    # a (b, kvh) cache slab past 4 GiB (32-bit row offsets)
    bad = list(base)
    bad[21], bad[22], bad[23] = 128, (1 << 24) + 1, 1
    bad[26], bad[27] = FAKE, 1 << 62
    assert lib.tree_verify_step(*bad) == -1
    # partly overlapping cache_len / cache_len_out
    bad = list(base)
    bad[6] = ctypes.c_void_p(0x2000)
    bad[7] = ctypes.c_void_p(0x2002)
    bad[17] = 4
    assert lib.tree_verify_step(*bad) == -1


def test_paged_argument_errors(lib):
    def attn(**kw):
        a = dict(q=FAKE, kp=FAKE, vp=FAKE, ns=100, tb=FAKE, mp=4, P=16, cl=FAKE, ts=FAKE, anc=FAKE,
                 out=FAKE, B=1, T=8, Hq=2, Hkv=1, D=64, dt=0)
        a.update(kw)
        return lib.tree_verify_attn_paged(a["q"], a["kp"], a["vp"], a["ns"], a["tb"], a["mp"],
                                          a["P"], a["cl"], a["ts"], a["anc"], a["out"], None,
                                          None, a["B"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                          a["dt"], 0.0, 0, None, 0, None)
    for name in ("q", "kp", "vp", "tb", "cl", "ts", "anc", "out"):
        assert attn(**{name: None}) == -1, name
    assert attn(P=0) == -1 and attn(P=12) == -1  # page size: a power of two
    assert attn(ns=0) == -1 and attn(mp=0) == -1
    assert attn(D=96) == -2
    assert attn(mp=1 << 20, P=1 << 12) == -1  # table reach beyond 2^30 positions
    commit = [FAKE, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 1, 8, None, None]
    for i in (0, 3, 4, 5, 6, 7, 8, 9):
        bad = list(commit)
        bad[i] = None
        assert lib.kv_commit_paged(*bad) == -1, i
    bad = list(commit)
    bad[2] = 16  # pointer swap needs one-token pages
    assert lib.kv_commit_paged(*bad) == -2


def test_step_paged_argument_errors(lib):
    # parent, draft, target, q, k_pool, v_pool, num_slots, block_table, max_pages, page_size,
    # cache_len, cache_len_out, tree_slot, anc, out, lse, path, alen, bonus, free_slots,
    # free_top, status, B, T, Hq, Hkv, D, dtype, scale, split_keys, ws, ws_bytes, stream
    base = ([FAKE] * 6 + [100, FAKE, 16, 1] + [FAKE] * 12 +
            [1, 8, 2, 1, 64, 0, 0.0, 0, None, 0, None])
    ptrs = [0, 1, 2, 3, 4, 5, 7, 10, 11, 12, 13, 14, 16, 17, 18, 19, 20, 21]
    for i in ptrs:  # every pointer but lse is required
        bad = list(base)
        bad[i] = None
        assert lib.tree_verify_step_paged(*bad) == -1, i
    for i, v, code in ((9, 4, -2),   # the pointer-swap commit needs one-token pages
                       (9, 3, -1),   # page size: a power of two
                       (6, 0, -1),   # empty pool
                       (8, 0, -1),   # empty table
                       (26, 96, -2)):  # head_dim
        bad = list(base)
        bad[i] = v
        assert lib.tree_verify_step_paged(*bad) == code, (i, v)
    bad = list(base)  # partly overlapping cache_len / cache_len_out
    bad[10] = ctypes.c_void_p(0x2000)
    bad[11] = ctypes.c_void_p(0x2002)
    bad[22] = 4
    assert lib.tree_verify_step_paged(*bad) == -1


def test_accept_argument_errors(lib):
    assert lib.tree_accept(None, FAKE, FAKE, 1, 8, FAKE, FAKE, FAKE, None) == -1
    assert lib.tree_accept(FAKE, FAKE, FAKE, 1, 8, FAKE, None, FAKE, None) == -1
    assert lib.tree_accept(FAKE, FAKE, FAKE, 1, 129, FAKE, FAKE, FAKE, None) == -1
    assert lib.tree_accept(FAKE, FAKE, FAKE, 0, 8, FAKE, FAKE, FAKE, None) == -1


def test_compact_argument_errors(lib):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 1, 64, 32, 0, None, None]
    for i in range(8):
        bad = list(args)
        bad[i] = None
        assert lib.kv_compact_accepted(*bad) == -1, i
    bad = list(args)
    bad[11] = 80  # head_dim
    assert lib.kv_compact_accepted(*bad) == -2
    bad = list(args)
    bad[13] = 3  # dtype
    assert lib.kv_compact_accepted(*bad) == -2
    bad = list(args)
    bad[12] = -1  # Lmax
    assert lib.kv_compact_accepted(*bad) == -1


def test_binding_rejects_host_tensors():
    import torch

    import tree_attention_verification_attn_amd as tv

    with pytest.raises(ValueError):
        tv.tree_build_mask(torch.zeros((1, 8), dtype=torch.int32))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "tree_attention_verification_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower(), f


def test_stochastic_accept_argument_errors(lib):
    # anc, draft, p, q, u_acc, u_res, B, T, V, mode, G, workspace, bytes, path, len, bonus,
    # status, stream
    base = [FAKE] * 6 + [1, 8, 1000, 0, 1, None, 0] + [FAKE] * 3 + [None, None]
    for i in list(range(6)) + [13, 14, 15]:  # every pointer but workspace and status is required
        bad = list(base)
        bad[i] = None
        assert lib.tree_accept_stochastic(*bad) == -1, i
    for i, v in ((6, 0), (7, 0), (7, 129), (8, 0), (8, 1048577), (9, 2), (9, -1), (10, -1),
                 (10, 65)):
        bad = list(base)
        bad[i] = v
        assert lib.tree_accept_stochastic(*bad) == -1, (i, v)
    # two workgroups per sequence exchange sums through a workspace
    need = lib.tree_accept_stochastic_workspace_size(1, 8, 1000, 2)
    assert need == 8 * 2 * 16 + 4
    bad = list(base)
    bad[10] = 2
    assert lib.tree_accept_stochastic(*bad) == -3
    bad[11], bad[12] = FAKE, need - 1
    assert lib.tree_accept_stochastic(*bad) == -3


def test_stochastic_workspace_size_rules(lib):
    ws = lib.tree_accept_stochastic_workspace_size
    assert ws(4, 60, 1000, 1) == 0        # one workgroup per sequence: no exchange
    assert ws(4, 60, 1000, 0) == 0        # a 1000-token vocabulary is too small to split
    assert ws(2, 60, 128256, 3) == 2 * 60 * 3 * 16 + 2 * 4
    assert ws(0, 60, 1000, 0) == 0 and ws(1, 60, 1000, 65) == 0


def test_eagle2_node_count(lib):
    from oracle import oracle as O

    for depth, k, branch in ((0, 3, 3), (1, 10, 10), (6, 10, 10), (8, 10, 10), (10, 16, 16),
                             (5, 1, 4), (4, 7, 1)):
        assert lib.eagle2_node_count(depth, k, branch) == O.eagle2_node_count(depth, k, branch)
    assert lib.eagle2_node_count(-1, 3, 3) == -1 and lib.eagle2_node_count(2, 0, 3) == -1
    assert lib.eagle2_node_count(2000, 1024, 1024) == -1  # too many nodes


def test_eagle2_expand_argument_errors(lib):
    # root, tok, conf, B, level, k, branch, node_tok, node_parent, node_value, n_max, frontier,
    # status, stream
    base = [FAKE] * 3 + [2, 1, 10, 10] + [FAKE] * 3 + [111, FAKE, FAKE, None]
    for i in (1, 2, 7, 8, 9, 11, 12):
        bad = list(base)
        bad[i] = None
        assert lib.eagle2_expand(*bad) == -1, i
    bad = list(base)
    bad[0] = None  # the root token is needed at level 1 only
    assert lib.eagle2_expand(*bad) == -1
    for i, v in ((3, 0), (4, 0), (5, 0), (6, 0), (5, 103), (10, 10)):  # 103 * 10 > 1024
        bad = list(base)
        bad[i] = v
        assert lib.eagle2_expand(*bad) == -1, (i, v)
    bad = list(base)
    bad[4], bad[10] = 2, 110  # level 2 needs 1 + 10 + 100 = 111 nodes
    assert lib.eagle2_expand(*bad) == -1


def test_eagle2_rerank_argument_errors(lib):
    # tok, parent, value, n_nodes, n_max, B, T, parent_out, tok_out, depth_out, node_out,
    # status, stream
    base = [FAKE] * 3 + [511, 511, 1, 60] + [FAKE] * 5 + [None]
    for i in (0, 1, 2, 7, 8, 9, 10, 11):
        bad = list(base)
        bad[i] = None
        assert lib.eagle2_rerank(*bad) == -1, i
    for i, v in ((5, 0), (6, 0), (6, 129), (3, 59), (4, 510), (3, 16385)):
        bad = list(base)
        bad[i] = v
        if i == 3 and v > 511:
            bad[4] = v
        assert lib.eagle2_rerank(*bad) == -1, (i, v)


def test_lm_head_argument_errors(lib):
    # project: h, B, M, r, d, u, stream
    base = [FAKE, FAKE, 10, 256, 4096, FAKE, None]
    for i in (0, 1, 5):
        bad = list(base)
        bad[i] = None
        assert lib.lm_head_project(*bad) == -1, i
    for i, v in ((2, 0), (2, 65), (3, 0), (4, 0), (4, 4000), (4, 256)):
        bad = list(base)
        bad[i] = v
        assert lib.lm_head_project(*bad) == -1, (i, v)
    # screen: A, u, row_token, M, r, n, tile, k_tile, cand, score, stream
    base = [FAKE, FAKE, FAKE, 10, 256, 128256, 256, 4, FAKE, FAKE, None]
    for i in (0, 1, 2, 8, 9):
        bad = list(base)
        bad[i] = None
        assert lib.lm_head_screen(*bad) == -1, i
    for i, v in ((3, 0), (3, 65), (4, 0), (4, 12), (5, 0), (6, 0), (6, 257), (7, 0), (7, 17)):
        bad = list(base)
        bad[i] = v
        assert lib.lm_head_screen(*bad) == -1, (i, v)
    bad = list(base)
    bad[3], bad[4] = 64, 512  # 64 chains x 512 ranks x 4 B of u exceeds 64 KB of LDS
    assert lib.lm_head_screen(*bad) == -1
    # pointers read 16 bytes at a time must be 16-byte aligned
    odd = ctypes.c_void_p(0x1004)
    for i in (0, 1):
        bad = list(base)
        bad[i] = odd
        assert lib.lm_head_screen(*bad) == -1, i
    for i in (0, 1):
        bad = [FAKE, FAKE, 10, 256, 4096, FAKE, None]
        bad[i] = odd
        assert lib.lm_head_project(*bad) == -1, i
        bad = [FAKE, FAKE, FAKE, 10, 2004, 4096, 128256, FAKE, None, None]
        bad[i] = odd
        assert lib.lm_head_rescore(*bad) == -1, i
    # rescore: W, h, cand, M, C, d, V, logits, status, stream
    base = [FAKE, FAKE, FAKE, 10, 2004, 4096, 128256, FAKE, None, None]
    for i in (0, 1, 2, 7):
        bad = list(base)
        bad[i] = None
        assert lib.lm_head_rescore(*bad) == -1, i
    for i, v in ((3, 0), (3, 65), (4, 0), (5, 100), (6, 0)):
        bad = list(base)
        bad[i] = v
        assert lib.lm_head_rescore(*bad) == -1, (i, v)
    # topk: logits, cand, M, C, K, V, tok, conf, stream
    base = [FAKE, FAKE, 10, 2004, 10, 128256, FAKE, FAKE, None]
    for i in (0, 1, 6, 7):
        bad = list(base)
        bad[i] = None
        assert lib.lm_head_topk(*bad) == -1, i
    for i, v in ((2, 0), (3, 0), (3, 8193), (4, 0), (4, 65), (5, 0)):
        bad = list(base)
        bad[i] = v
        assert lib.lm_head_topk(*bad) == -1, (i, v)


def test_noalloc_rejects_plans_beyond_its_array(lib):
    """tree_verify_step_noalloc refuses, before any device call, a plan whose split-K partials
    exceed its fixed device array; the automatic plan of the largest workloads fits."""
    import re

    hdr = open(HEADER, encoding="utf-8").read()
    m = re.search(r"#define TV_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    limit = int(m.group(1)) << int(m.group(2))
    ws = lib.tree_verify_attn_workspace_size
    # 64-key chunks over a 65536-token cache at batch 64: far more partials than the array holds
    assert ws(64, 128, 32, 8, 128, 65536, 1, 64) > limit
    args = [FAKE] * 17 + [64, 128, 32, 8, 128, 65536, 1, ctypes.c_float(0.0), 64, None]
    assert lib.tree_verify_step_noalloc(*args) == -3
    # automatic plans: the worst case (511 units of two chunks each, fp32, D = 128) and the
    # 70B-like workload fit
    assert 0 < ws(511, 64, 1, 1, 128, 4096, 0, 0) <= limit
    assert 0 < ws(8, 64, 64, 8, 128, 32832, 1, 0) <= limit
