#!/usr/bin/env python3
"""Benchmark of the tree-verification step on one MI355X.

One step = tree_build_mask + tree_verify_attn + tree_accept + kv_compact_accepted (one layer)
over one batch of the chosen synthetic workload, all on one stream with the inputs resident in
HBM.  Copies of the input set are rotated so the bytes touched per sweep exceed twice the
256 MB Infinity Cache.  The default workload is the largest that fits one GPU: the wide-tree
batch (64 sequences, prefixes of 1024..8192 tokens, 128-node trees).  The timed region (K
steps) runs several times and the median is reported.  Prints one JSON line:

  value            KV-prefix bytes of the step / step time (GB/s), i.e. the prefix K/V read rate
                   of the whole verification step
  attn_kv_gbps     the same bytes / tree_verify_attn time alone
  tree_tokens_per_s, accepted_tokens_per_s   B*T and sum(accept_len) per second of step time
  roofline         the attention main kernel against MI355X's HBM (8 TB/s) or bf16 MFMA peak
  cpu_baseline     the CPU oracle on a bounded sample of the same workload
  other_workloads  the same fused step timed on the other multi-token workloads (--also)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synth import WORKLOADS, make_workload  # noqa: E402

DEFAULT_WORKLOAD = "wide_b64_L1024-8192_T128"
ALSO_WORKLOADS = "llama8b_b1_L4096_T60,batch32_L512-4096_T60,llama70b_b8_L32768_T64"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
MALL_BYTES = 256 << 20
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_main_hbm_counters.json")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--repeats", type=int, default=5,
                   help="times the K-step timed region is run; the median is reported")
    p.add_argument("--also", default=ALSO_WORKLOADS,
                   help="comma-separated workloads whose fused step is also timed and reported "
                        "under \"other_workloads\" ('' for none)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    p.add_argument("--split-keys", type=int, default=0, help="prefix keys per split (0 = auto)")
    p.add_argument("--graph-steps", type=int, default=0,
                   help="consecutive steps captured in one HIP graph, cycling the input sets "
                        "as the layers of a model would (0 = auto: the smallest multiple of the "
                        "set count that is >= 8)")
    p.add_argument("--api", choices=("fused", "separate"), default="fused",
                   help="time the step through tree_verify_step (two launches) or through the "
                        "four separate entry points; the other is timed too and reported")
    p.add_argument("--kv", choices=("dense", "paged"), default="dense",
                   help="dense caches, or a paged pool read through a block table with the path "
                        "committed by pointer swap (page size 1; kv_compact_accepted's copy is "
                        "timed beside it)")
    p.add_argument("--page-size", type=int, default=1,
                   help="tokens per page for --kv paged (the commit needs 1; larger pages time "
                        "mask + attention + acceptance)")
    p.add_argument("--accept", choices=("greedy", "stochastic"), default="greedy",
                   help="greedy acceptance (the fused step), or rejection sampling over the tree "
                        "(mask + attention + tree_accept_stochastic + compaction)")
    p.add_argument("--sampling", choices=("independent", "without-replacement"),
                   default="independent",
                   help="how siblings were drafted, for --accept stochastic")
    p.add_argument("--stoch-groups", type=int, default=0,
                   help="workgroups sharing each vocabulary sweep of a sequence for --accept "
                        "stochastic (0 = automatic)")
    p.add_argument("--vocab", type=int, default=0,
                   help="vocabulary of the next-token distributions (0 = the workload's, 128256)")
    p.add_argument("--construct", action="store_true",
                   help="also time device-side EAGLE-2 tree construction (every eagle2_expand "
                        "level, then eagle2_rerank) on the workload's expansion shape, and the "
                        "oracle's construction on the host; reported under \"construction\"")
    p.add_argument("--lm-head", metavar="HEAD", default=None,
                   help="also time the two-stage drafter LM head (lm_head_project, _screen, "
                        "_rescore, _topk) on a synthetic head (synth.LM_HEADS: llama8b_head_M10, "
                        "llama8b_head_M64); reported under \"lm_head\"")
    p.add_argument("--rotate", type=int, default=0, help="input copies to rotate (0 = auto)")
    p.add_argument("--mode", choices=("graph", "eager"), default="graph",
                   help="replay each step as a captured HIP graph, or launch eagerly")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a 1 GiB device-to-device copy 5 times (counter calibration)")
    p.add_argument("--pmc-summary", metavar="DIR",
                   help="summarise rocprofv3 --pmc runs under DIR/{fetch,write,cal_fetch,"
                        "cal_write} into " + os.path.relpath(COUNTERS_FILE, ROOT))
    return p.parse_args()


COPY_BYTES = 1 << 30


def copy_calibration() -> int:
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings scale the counters."""
    import torch

    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}))
    return 0


def _counter_avg(csv_path: str, kernel_sub: str, counter: str) -> float:
    import csv

    vals = []
    with open(csv_path, encoding="utf-8") as f:
        for row in csv.DictReader(f):
            if kernel_sub in row["Kernel_Name"] and row["Counter_Name"] == counter:
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples for kernels matching {kernel_sub!r} in {csv_path}")
    return float(np.mean(vals))


def pmc_summary(d: str, workload: str) -> int:
    """HBM bytes per attn_main launch = FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
    scaled by bytes / reading of the same counter on a plain copy of known size."""
    f = lambda sub: os.path.join(d, sub, "run_counter_collection.csv")  # noqa: E731
    fetch = _counter_avg(f("fetch"), "attn_main", "FETCH_SIZE")
    write = _counter_avg(f("write"), "attn_main", "WRITE_SIZE")
    cal_fetch = _counter_avg(f("cal_fetch"), "copyBuffer", "FETCH_SIZE")
    cal_write = _counter_avg(f("cal_write"), "copyBuffer", "WRITE_SIZE")
    fs, ws = COPY_BYTES / 1024 / cal_fetch, COPY_BYTES / 1024 / cal_write
    w = make_workload(workload, with_kv=False)
    L = np.clip(w.cache_len, 0, 1 << 30).astype(np.int64)
    alg = int(L.sum()) * w.Hkv * w.D * 2 * (2 if w.dtype == "bf16" else 4)
    rec = {
        "kernel": "attn_main",
        "kernel_source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": fetch,
        "write_kib_per_dispatch": write,
        "copy_fetch_kib": cal_fetch,
        "copy_write_kib": cal_write,
        "fetch_scale": fs,
        "write_scale": ws,
        "hbm_read_bytes_per_launch": fetch * fs * 1024,
        "hbm_write_bytes_per_launch": write * ws * 1024,
        "hbm_bytes_per_launch": (fetch * fs + write * ws) * 1024,
        "algorithmic_kv_bytes": alg,
        "read_over_algorithmic": fetch * fs * 1024 / alg,
    }
    data = {}
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE, encoding="utf-8") as fh:
            data = json.load(fh)
    data[workload] = rec
    os.makedirs(os.path.dirname(COUNTERS_FILE), exist_ok=True)
    with open(COUNTERS_FILE, "w", encoding="utf-8") as fh:
        json.dump(data, fh, indent=2, sort_keys=True)
    print(json.dumps(rec))
    return 0


# the sources attn_main is compiled from: the counters in COUNTERS_FILE hold while these are
# unchanged
ATTN_SOURCES = ("attn.hip", "tree_device.h", "tv_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_attention_verification_attn_amd", "csrc")
    for f in ATTN_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class StepSet:
    """Device buffers of one copy of the workload, plus pre-marshalled C-ABI argument tuples."""

    def __init__(self, tv, torch, w, base=None, split_keys=0, workspace=None, paged=None,
                 stoch=None, stoch_ws=None, stoch_groups=0):
        dev = torch.device("cuda:0")

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        if base is None:
            t = dict(parent=up(w.parent), draft=up(w.draft), target=up(w.target),
                     cache_len=up(w.cache_len), q=up(w.q), k_cache=up(w.k_cache),
                     v_cache=up(w.v_cache), k_tree=up(w.k_tree), v_tree=up(w.v_tree))
        else:
            t = {k: v.clone() for k, v in base.t.items()}
        B, T, Hq, D = w.B, w.T, w.Hq, w.D
        W = (T + 63) // 64
        t["anc"] = torch.empty((B, T, W), dtype=torch.int64, device=dev)
        t["status"] = torch.zeros((B,), dtype=torch.int32, device=dev)
        t["out"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
        t["path"] = torch.empty((B, T), dtype=torch.int32, device=dev)
        t["alen"] = torch.empty((B,), dtype=torch.int32, device=dev)
        t["bonus"] = torch.empty((B,), dtype=torch.int32, device=dev)
        t["cache_len_out"] = torch.empty((B,), dtype=torch.int32, device=dev)
        self.t = t
        P = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
        dt = tv.TV_BF16 if w.dtype == "bf16" else tv.TV_F32
        ws_bytes = 0 if workspace is None else workspace.numel()
        ws_ptr = None if workspace is None else P(workspace)
        self.lib = tv.load_library()
        self.mask_args = (P(t["parent"]), B, T, P(t["anc"]), P(t["status"]))
        self.attn_args = (P(t["q"]), P(t["k_cache"]), P(t["v_cache"]), P(t["cache_len"]),
                          P(t["k_tree"]), P(t["v_tree"]), P(t["anc"]), P(t["out"]), P(t["lse"]),
                          P(t["status"]), B, T, Hq, w.Hkv, D, w.Lmax, dt, ctypes.c_float(0.0),
                          split_keys, ws_ptr, ctypes.c_size_t(ws_bytes))
        self.accept_args = (P(t["anc"]), P(t["draft"]), P(t["target"]), B, T, P(t["path"]),
                            P(t["alen"]), P(t["bonus"]))
        self.compact_args = (P(t["k_cache"]), P(t["v_cache"]), P(t["cache_len"]),
                             P(t["cache_len_out"]), P(t["k_tree"]), P(t["v_tree"]), P(t["path"]),
                             P(t["alen"]), B, T, w.Hkv, D, w.Lmax, dt, P(t["status"]))
        self.step_args = (P(t["parent"]), P(t["draft"]), P(t["target"]), P(t["q"]),
                          P(t["k_cache"]), P(t["v_cache"]), P(t["cache_len"]),
                          P(t["cache_len_out"]), P(t["k_tree"]), P(t["v_tree"]), P(t["anc"]),
                          P(t["out"]), P(t["lse"]), P(t["path"]), P(t["alen"]), P(t["bonus"]),
                          P(t["status"]), B, T, Hq, w.Hkv, D, w.Lmax, dt, ctypes.c_float(0.0),
                          split_keys, ws_ptr, ctypes.c_size_t(ws_bytes))
        self.api = "fused"
        self.paged = paged
        if paged is not None:  # the same rows in a pool of token slots (synth.make_paged)
            if base is None:
                t["k_pool"], t["v_pool"] = up(paged.k_pool), up(paged.v_pool)
                t["table"], t["tree_slot"] = up(paged.block_table), up(paged.tree_slot)
            t["free"] = torch.full((paged.num_slots,), -1, dtype=torch.int32, device=dev)
            t["free_top"] = torch.zeros((1,), dtype=torch.int32, device=dev)
            mp = paged.block_table.shape[1]
            self.attn_paged_args = (P(t["q"]), P(t["k_pool"]), P(t["v_pool"]), paged.num_slots,
                                    P(t["table"]), mp, paged.page_size, P(t["cache_len"]),
                                    P(t["tree_slot"]), P(t["anc"]), P(t["out"]), P(t["lse"]),
                                    P(t["status"]), B, T, Hq, w.Hkv, D, dt, ctypes.c_float(0.0),
                                    split_keys, ws_ptr, ctypes.c_size_t(ws_bytes))
            self.commit_args = (P(t["table"]), mp, paged.page_size, P(t["cache_len"]),
                                P(t["cache_len_out"]), P(t["tree_slot"]), P(t["path"]),
                                P(t["alen"]), P(t["free"]), P(t["free_top"]), paged.num_slots,
                                B, T, P(t["status"]))
            # the fused paged step (one-token pages): the same four calls in two launches
            self.step_paged_args = (P(t["parent"]), P(t["draft"]), P(t["target"]), P(t["q"]),
                                    P(t["k_pool"]), P(t["v_pool"]), paged.num_slots,
                                    P(t["table"]), mp, paged.page_size, P(t["cache_len"]),
                                    P(t["cache_len_out"]), P(t["tree_slot"]), P(t["anc"]),
                                    P(t["out"]), P(t["lse"]), P(t["path"]), P(t["alen"]),
                                    P(t["bonus"]), P(t["free"]), P(t["free_top"]),
                                    P(t["status"]), B, T, Hq, w.Hkv, D, dt, ctypes.c_float(0.0),
                                    split_keys, ws_ptr, ctypes.c_size_t(ws_bytes))
            self.api = "paged_fused" if paged.page_size == 1 else "paged"
        self.stoch = stoch
        if stoch is not None:  # next-token distributions and uniforms (synth.make_stochastic)
            if base is None:
                t["p"], t["q"] = up(stoch.p), up(stoch.q)
                t["sdraft"] = up(stoch.draft)
                t["u_acc"], t["u_res"] = up(stoch.u_acc), up(stoch.u_res)
            sws = 0 if stoch_ws is None else stoch_ws.numel()
            self.stoch_args = (P(t["anc"]), P(t["sdraft"]), P(t["p"]), P(t["q"]), P(t["u_acc"]),
                               P(t["u_res"]), B, T, stoch.V, int(stoch.without_replacement),
                               stoch_groups,
                               None if stoch_ws is None else P(stoch_ws), ctypes.c_size_t(sws),
                               P(t["path"]), P(t["alen"]), P(t["bonus"]), P(t["status"]))
            self.api = "stochastic"

    def accept_stochastic(self, stream):
        rc = self.lib.tree_accept_stochastic(*self.stoch_args, stream)
        assert rc == 0, rc

    def attn_paged(self, stream):
        rc = self.lib.tree_verify_attn_paged(*self.attn_paged_args, stream)
        assert rc == 0, rc

    def fused_paged(self, stream):
        rc = self.lib.tree_verify_step_paged(*self.step_paged_args, stream)
        assert rc == 0, rc

    def commit(self, stream):
        if self.paged.page_size == 1:
            rc = self.lib.kv_commit_paged(*self.commit_args, stream)
            assert rc == 0, rc

    def mask(self, stream):
        rc = self.lib.tree_build_mask(*self.mask_args, stream)
        assert rc == 0, rc

    def attn(self, stream):
        rc = self.lib.tree_verify_attn(*self.attn_args, stream)
        assert rc == 0, rc

    def accept(self, stream):
        rc = self.lib.tree_accept(*self.accept_args, stream)
        assert rc == 0, rc

    def compact(self, stream):
        rc = self.lib.kv_compact_accepted(*self.compact_args, stream)
        assert rc == 0, rc

    def fused(self, stream):
        rc = self.lib.tree_verify_step(*self.step_args, stream)
        assert rc == 0, rc

    def step(self, stream):
        if self.api == "fused":
            self.fused(stream)
            return
        if self.api == "paged_fused":
            self.fused_paged(stream)
            return
        if self.api == "paged":
            self.mask(stream)
            self.attn_paged(stream)
            self.accept(stream)
            self.commit(stream)
            return
        if self.api == "stochastic":
            self.mask(stream)
            self.attn(stream)
            self.accept_stochastic(stream)
            self.compact(stream)
            return
        self.mask(stream)
        self.attn(stream)
        self.accept(stream)
        self.compact(stream)


def stochastic_work(parent, draft, path, alen, V) -> tuple[float, int]:
    """Vocabulary sweeps of tree_accept_stochastic's walks, read off its outputs, and their bytes.

    At every kept node but the last, each in-vocabulary child before the kept one was rejected
    (one sweep of p and q each); at the last node every such child was, and the bonus draw sweeps
    p (and q once a child was rejected there).  Returns (mean sweeps per sequence, bytes)."""
    B, T = parent.shape
    sweeps, nbytes = 0, 0
    for b in range(B):
        for i in range(int(alen[b])):
            u = int(path[b, i])
            kids = [c for c in range(u + 1, T) if parent[b, c] == u and 0 <= draft[b, c] < V]
            last = i + 1 == int(alen[b])
            rej = len(kids) if last else int(sum(c < int(path[b, i + 1]) for c in kids))
            sweeps += rej
            nbytes += rej * 8 * V
            if last:
                sweeps += 1
                nbytes += (8 if rej else 4) * V
    return sweeps / B, int(nbytes)


def construction_bench(tv, torch, w, stream, steps: int, warmup: int) -> dict:
    """Device-side EAGLE-2 tree construction on the workload's expansion shape: every
    eagle2_expand level, then eagle2_rerank, for the whole batch.  Timed as HIP graphs of
    constructions (whole job, inputs resident), per kernel by events between eager calls, and
    the oracle's construction of the same inputs on the host."""
    from synth import make_draft_levels

    d = make_draft_levels(w.spec.name)
    depth, B, k, branch = d.child_tok.shape
    N = tv.eagle2_node_count(depth, k, branch)
    T = w.T
    table = tv.eagle2_new_table(B, N, k, "cuda")
    tok = torch.from_numpy(d.child_tok).cuda()
    conf = torch.from_numpy(d.child_conf).cuda()
    root = torch.from_numpy(d.root_tok).cuda()
    out = {name: torch.empty((B, T), dtype=torch.int32, device="cuda")
           for name in ("parent", "tok", "depth", "node")}

    def expand(lvl, st):
        tv.eagle2_expand(table, lvl, tok[lvl - 1], conf[lvl - 1],
                         root_tok=root if lvl == 1 else None, stream=st)

    def build(st):
        for lvl in range(1, depth + 1):
            expand(lvl, st)
        tv.eagle2_rerank(table, N, T, out=out, stream=st)

    reps = 8
    with torch.cuda.stream(stream):
        build(stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                build(torch.cuda.current_stream())
        for _ in range(max(1, warmup // reps)):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_graphs = max(1, steps // reps)
        stream.synchronize()
        e0.record(stream)
        for _ in range(n_graphs):
            g.replay()
        e1.record(stream)
        e1.synchronize()
    t_build = e0.elapsed_time(e1) * 1e-3 / (n_graphs * reps)

    n_prof = 100
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(depth + 2)] for _ in range(n_prof)]
    for row in ev:
        for e in row:
            e.record(stream)
    stream.synchronize()
    with torch.cuda.stream(stream):
        for i in range(n_prof):
            ev[i][0].record(stream)
            for lvl in range(1, depth + 1):
                expand(lvl, stream)
                ev[i][lvl].record(stream)
            tv.eagle2_rerank(table, N, T, out=out, stream=stream)
            ev[i][depth + 1].record(stream)
        stream.synchronize()
    lv = [float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n_prof)])) * 1e3
          for j in range(depth + 1)]
    status = table["status"].cpu().numpy()

    # algorithmic bytes of one construction (the whole batch)
    byts, F = 0, 1
    for _ in range(depth):
        byts += B * (F * branch * (4 + 4 + 12) + 2 * F * 4 + k * 4)
        F = min(k, F * branch)
    byts += B * (N * 8 + T * 8 + T * 16)

    from oracle import oracle as O  # the CPU baseline leg

    O.eagle2_build(d.root_tok, d.child_tok, d.child_conf, T)
    n_cpu, t0 = 0, time.perf_counter()
    while n_cpu < 3 or time.perf_counter() - t0 < 2.0:
        O.eagle2_build(d.root_tok, d.child_tok, d.child_conf, T)
        n_cpu += 1
    t_cpu = (time.perf_counter() - t0) / n_cpu
    return {
        "levels": depth, "topk": k, "branch": branch, "nodes": N, "T": T, "B": B,
        "construction_us": t_build * 1e6,
        "trees_per_s": B / t_build,
        "expand_us_by_level": lv[:depth],
        "rerank_us": lv[depth],
        "algorithmic_bytes": byts,
        "achieved_gbps": byts / t_build / 1e9,
        "status_nonzero": int((status != 0).sum()),
        "cpu_baseline": {"construction_us": t_cpu * 1e6, "trees_per_s": B / t_cpu, "cores": 1,
                         "kind": "oracle",
                         "sample": f"the whole batch's construction, {n_cpu} runs"},
        "note": ("construction_us: graphs of 8 constructions replayed back to back (one "
                 "construction = every expand level and the rerank for the whole batch); the "
                 "per-kernel times come from events between eager calls, launch latency "
                 "included; latency-bound (a few KB per sequence per level)"),
    }


def lm_head_bench(tv, torch, name: str, stream, steps: int, warmup: int) -> dict:
    """The two-stage drafter LM head on a synthetic head: the four launches replayed as HIP
    graphs (inputs resident), per-kernel durations from events between eager calls, the
    roofline of the whole head against HBM, and the oracle on the host for a sample of hidden
    states."""
    from synth import make_lm_head

    x = make_lm_head(name)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    h, A, Bm, W = bf(x.h), bf(x.A), bf(x.B), bf(x.W)
    perm = torch.from_numpy(x.row_token).cuda()
    M, C = x.M, -(-x.n // x.tile) * x.k_tile
    u = torch.empty((M, x.r), dtype=torch.float32, device="cuda")
    cand = torch.empty((M, C), dtype=torch.int32, device="cuda")
    score = torch.empty((M, C), dtype=torch.float32, device="cuda")
    logits = torch.empty((M, C), dtype=torch.float32, device="cuda")
    tok = torch.empty((M, x.K), dtype=torch.int32, device="cuda")
    conf = torch.empty((M, x.K), dtype=torch.float32, device="cuda")

    calls = [
        lambda st: tv.lm_head_project(h, Bm, u=u, stream=st),
        lambda st: tv.lm_head_screen(A, u, perm, x.tile, x.k_tile, cand=cand, cand_score=score,
                                     stream=st),
        lambda st: tv.lm_head_rescore(W, h, cand, logits=logits, stream=st),
        lambda st: tv.lm_head_topk(logits, cand, x.K, x.n, out_tok=tok, out_conf=conf, stream=st),
    ]

    reps = 8
    with torch.cuda.stream(stream):
        for c in calls:
            c(stream)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            cs = torch.cuda.current_stream()
            for _ in range(reps):
                for c in calls:
                    c(cs)
        for _ in range(max(1, warmup // reps)):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_graphs = max(1, steps // reps)
        stream.synchronize()
        e0.record(stream)
        for _ in range(n_graphs):
            g.replay()
        e1.record(stream)
        e1.synchronize()
    t_head = e0.elapsed_time(e1) * 1e-3 / (n_graphs * reps)

    n_prof = 50
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_prof)]
    for row in ev:
        for e in row:
            e.record(stream)
    stream.synchronize()
    with torch.cuda.stream(stream):
        for i in range(n_prof):
            ev[i][0].record(stream)
            for j, c in enumerate(calls):
                c(stream)
                ev[i][j + 1].record(stream)
        stream.synchronize()
    per = [float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n_prof)])) * 1e3
           for j in range(4)]

    # algorithmic bytes: A, B and h once, the candidates' rows of W, the small outputs
    a_bytes = x.n * x.r * 2 + x.r * x.d * 2 + M * x.d * 2
    w_bytes = M * C * x.d * 2
    out_bytes = M * x.r * 4 * 2 + M * C * 4 * 5 + M * x.K * 8
    byts = a_bytes + w_bytes + out_bytes
    full_head_bytes = x.n * x.d * 2

    from oracle import oracle as O  # the CPU baseline leg

    rows = min(M, 2)
    t0 = time.perf_counter()
    O.lm_head_two_stage(x.h[:rows], x.A, x.B, x.W, x.row_token, x.tile, x.k_tile, x.K)
    t_cpu = (time.perf_counter() - t0) * M / rows
    return {
        "head": name, "M": M, "d": x.d, "vocab": x.n, "rank": x.r, "tile": x.tile,
        "k_tile": x.k_tile, "candidates": C, "children": x.K,
        "head_us": t_head * 1e6,
        "hidden_states_per_s": M / t_head,
        "kernel_us": {"lm_head_project": per[0], "lm_head_screen": per[1],
                      "lm_head_rescore": per[2], "lm_head_topk": per[3]},
        "algorithmic_bytes": byts,
        "roofline": {"bound": "hbm", "achieved": byts / t_head / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": byts / t_head / 1e9 / HBM_PEAK_GBS},
        "full_head_bytes": full_head_bytes,
        "full_head_us_at_hbm_peak": full_head_bytes / (HBM_PEAK_GBS * 1e9) * 1e6,
        "cpu_baseline": {"head_us": t_cpu * 1e6, "cores": 1, "kind": "oracle",
                         "sample": f"{rows} of {M} hidden states through both stages, scaled "
                                   f"to {M}"},
        "note": ("head_us: graphs of 8 heads (four launches each) replayed back to back; "
                 "kernel_us from events between eager calls (launch latency included); bytes: "
                 "A, B and h once plus the candidates' rows of W; full_head_* is what reading "
                 "the whole head once would take at the HBM peak, for context"),
    }


def other_workload_bench(tv, torch, name: str, args, stream) -> dict:
    """The fused step (tree_verify_step) on another workload, measured as the headline is:
    input sets rotated past twice the Infinity Cache, HIP graphs of consecutive steps, W warmup
    steps, `repeats` timed regions of K steps continuing the rotation (median reported), and
    the main kernel's own duration from its profiling hook over an eager pass."""
    print(f"[bench] also timing {name}", file=sys.stderr, flush=True)
    w = make_workload(name)
    kv_bytes = w.kv_prefix_bytes()
    L = np.clip(w.cache_len, 0, w.Lmax).astype(np.int64)
    flops = 4 * int(L.sum()) * w.Hq * w.T * w.D
    set_bytes = w.k_cache.nbytes + w.v_cache.nbytes + w.q.nbytes * 2 + w.k_tree.nbytes * 2
    free, _ = torch.cuda.mem_get_info()
    n_sets = max(1, min(math.ceil(2 * MALL_BYTES / max(kv_bytes, 1)), int(0.5 * free / set_bytes)))
    ws_bytes = tv.tree_verify_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.Lmax,
                                                  torch.bfloat16 if w.dtype == "bf16"
                                                  else torch.float32, 0)
    workspace = torch.zeros((ws_bytes,), dtype=torch.uint8, device="cuda") if ws_bytes else None
    sets = [StepSet(tv, torch, w, workspace=workspace)]
    for _ in range(n_sets - 1):
        sets.append(StepSet(tv, torch, w, base=sets[0], workspace=workspace))
    del w.k_cache, w.v_cache  # host copies are no longer needed
    gs = n_sets * math.ceil(8 / n_sets)
    graphs = {}

    def graph(n, start):
        key = (n, start % n_sets)
        if key not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for i in range(n):
                    sets[(start + i) % n_sets].fused(cs)
            graphs[key] = g
        return graphs[key]

    def plan(k, start):
        return [graph(gs, start)] * (k // gs) + ([graph(k % gs, start)] if k % gs else [])

    sptr = ctypes.c_void_p(stream.cuda_stream)
    with torch.cuda.stream(stream):
        for st in sets:
            st.fused(sptr)
    stream.synchronize()
    warm = plan(args.warmup, 0)
    plans = [plan(args.steps, args.warmup + r * args.steps) for r in range(args.repeats)]
    torch.cuda.synchronize()
    per = []
    with torch.cuda.stream(stream):
        for g in warm:
            g.replay()
        for pl in plans:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            stream.synchronize()
            e0.record(stream)
            for g in pl:
                g.replay()
            e1.record(stream)
            e1.synchronize()
            per.append(e0.elapsed_time(e1) / args.steps)
        # the main kernel's own duration, by its start and end timestamps
        n_prof = 50
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_prof)]
        for a, b in ev:
            a.record(stream)
            b.record(stream)
        stream.synchronize()
        for i, (a, b) in enumerate(ev):
            tv.profile_attn_main(a, b)
            sets[i % n_sets].fused(sptr)
        tv.profile_attn_main(None, None)
        stream.synchronize()
    t_main = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    ms = float(np.median(per))
    t_step = ms * 1e-3
    peak_tf = MFMA_PEAK_TFLOPS[w.dtype]
    hbm_bound = flops / kv_bytes < peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    res = {
        "workload": name, "desc": w.spec.desc, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv,
        "D": w.D, "prefix_tokens": int(L.sum()), "rotated_sets": n_sets, "graph_steps": gs,
        "ms_per_step": ms, "ms_per_step_repeats": per,
        "value_gbps": kv_bytes / t_step / 1e9,
        "hbm_frac": kv_bytes / t_step / 1e9 / HBM_PEAK_GBS,
        "tree_tokens_per_s": w.B * w.T / t_step,
        "attn_main_us": t_main * 1e6,
        "attn_main_bound": "hbm" if hbm_bound else "mfma",
        "attn_main_hbm_frac": kv_bytes / t_main / 1e9 / HBM_PEAK_GBS,
        "attn_main_mfma_frac": flops / t_main / 1e12 / peak_tf,
        "algorithmic_bytes": kv_bytes, "algorithmic_flops": flops,
    }
    del sets, graphs, workspace
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, kv_bytes: int, target_s: float) -> dict:
    """The oracle (never tuned) on a bounded random sample of attention rows."""
    from oracle import oracle as O

    cores = len(os.sched_getaffinity(0))
    total = w.B * w.T * w.Hq
    rng = np.random.default_rng(0)

    def rows_of(n):
        idx = rng.choice(total, size=n, replace=False)
        b = idx // (w.T * w.Hq)
        i = (idx // w.Hq) % w.T
        h = idx % w.Hq
        return np.stack([b, h, i], axis=1).astype(np.int32)

    L = np.clip(w.cache_len, 0, w.Lmax).astype(np.int32)
    n0 = min(total, 32 * cores)  # a probe long enough that thread start-up does not dominate
    t0 = time.perf_counter()
    O.attention(w.q, w.k_cache, w.v_cache, L, w.k_tree, w.v_tree, w.parent, rows=rows_of(n0),
                n_threads=cores)
    dt0 = max(time.perf_counter() - t0, 1e-3)
    n = int(min(total, max(n0, n0 * target_s / dt0)))
    rows = rows_of(n)
    reps = 1
    if n == total:  # the whole job is cheap: repeat it to reach the target CPU time
        reps = max(1, int(target_s / max(dt0 * total / n0, 1e-3)))
    t0 = time.perf_counter()
    for _ in range(reps):
        O.attention(w.q, w.k_cache, w.v_cache, L, w.k_tree, w.v_tree, w.parent, rows=rows,
                    n_threads=cores)
    dt = (time.perf_counter() - t0) / reps
    frac = n / total
    full_s = dt / frac
    return {
        "value": kv_bytes / full_s / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{n} of {total} (b, query head, node) attention rows drawn uniformly "
                   f"(seed 0), fp64, {reps} pass(es) of {dt:.2f} s wall each; rate = KV-prefix "
                   f"bytes of the whole step x {frac:.4f} / wall time per pass; mask, acceptance "
                   f"and compaction (microseconds) excluded"),
        "est_step_s": full_s,
        "tree_tokens_per_s": w.B * w.T / full_s,
    }


def main() -> int:
    args = parse_args()
    if args.pmc_summary:
        return pmc_summary(args.pmc_summary, args.workload)
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the verification step has no multi-GPU path "
              "(sequences and KV heads would shard across GPUs with no exchange, and one long "
              "prefix as split-K with one exchange of partials)", file=sys.stderr)
        return 2
    import torch

    import tree_attention_verification_attn_amd as tv

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    tv.load_library()
    torch.cuda.set_device(0)

    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    w = make_workload(args.workload)
    kv_bytes = w.kv_prefix_bytes()
    L = np.clip(w.cache_len, 0, w.Lmax).astype(np.int64)
    flops = 4 * int(L.sum()) * w.Hq * w.T * w.D  # QK^T and PV over the prefix
    elem = 2 if w.dtype == "bf16" else 4
    set_bytes = (w.k_cache.nbytes + w.v_cache.nbytes + w.q.nbytes * 2 + w.k_tree.nbytes * 2)
    if args.kv == "paged":
        set_bytes *= 2  # the pool holds the same rows again
    n_sets = args.rotate or max(1, math.ceil(2 * MALL_BYTES / max(kv_bytes, 1)))
    free, total_mem = torch.cuda.mem_get_info()
    n_sets = max(1, min(n_sets, int(0.5 * free / set_bytes)))

    ws_bytes = tv.tree_verify_attn_workspace_size(w.B, w.T, w.Hq, w.Hkv, w.D, w.Lmax,
                                                  torch.bfloat16 if w.dtype == "bf16"
                                                  else torch.float32, args.split_keys)
    paged = None
    if args.kv == "paged":
        from synth import make_paged

        paged = make_paged(w, args.page_size, seed=0)
        cap = paged.block_table.shape[1] * paged.page_size
        ws_bytes = max(ws_bytes, tv.tree_verify_attn_workspace_size(
            w.B, w.T, w.Hq, w.Hkv, w.D, cap,
            torch.bfloat16 if w.dtype == "bf16" else torch.float32, args.split_keys))
        args.api = "paged_fused" if args.page_size == 1 else "paged"
    stoch, stoch_ws = None, None
    if args.accept == "stochastic":
        if args.kv == "paged":
            raise SystemExit("--accept stochastic times the dense path; drop --kv paged")
        from synth import make_stochastic

        print("[bench] drawing next-token distributions", file=sys.stderr, flush=True)
        stoch = make_stochastic(w, V=args.vocab or None,
                                without_replacement=args.sampling == "without-replacement")
        set_bytes += stoch.p.nbytes + stoch.q.nbytes
        n_sets = max(1, min(n_sets, int(0.5 * free / set_bytes)))
        args.api = "stochastic"
        # one exchange workspace for every set: the calls are ordered on one stream, and each
        # leaves it all zeros for the next
        sws_bytes = tv.tree_accept_stochastic_workspace_size(w.B, w.T, stoch.V, args.stoch_groups)
        stoch_ws = torch.zeros((sws_bytes,), dtype=torch.uint8, device="cuda") if sws_bytes else None
    workspace = torch.zeros((max(ws_bytes, 1),), dtype=torch.uint8, device="cuda") if ws_bytes else None
    print(f"[bench] uploading {n_sets} input sets ({set_bytes / 2**20:.1f} MiB each), "
          f"workspace {ws_bytes / 2**20:.1f} MiB", file=sys.stderr, flush=True)
    sets = [StepSet(tv, torch, w, split_keys=args.split_keys, workspace=workspace, paged=paged,
                    stoch=stoch, stoch_ws=stoch_ws, stoch_groups=args.stoch_groups)]
    for _ in range(n_sets - 1):
        sets.append(StepSet(tv, torch, w, base=sets[0], split_keys=args.split_keys,
                            workspace=workspace, paged=paged, stoch=stoch, stoch_ws=stoch_ws,
                            stoch_groups=args.stoch_groups))
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    # whole graphs hold a multiple of the set count, so consecutive replays keep the rotation
    graph_steps = n_sets * math.ceil((args.graph_steps or 8) / n_sets)

    def time_api(api):
        """W untimed steps, then `repeats` timed regions of exactly K steps through `api`;
        returns (median ms per step, every region's ms per step, wall s of the median region).

        In graph mode a graph holds `graph_steps` consecutive steps on input sets s, s+1, ...
        (cycling, from a start set s); a run of k steps replays whole graphs, then one graph of
        the remainder.  Every run starts on the set after the last one the previous run used, so
        a timed region never begins on sets the warmup just touched."""
        for s in sets:
            s.api = api
        graphs = {}

        def graph_of(n, start):
            key = (n, start % n_sets)
            if key not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                    for i in range(n):
                        sets[(start + i) % n_sets].step(cs)
                graphs[key] = g
            return graphs[key]

        if args.mode == "graph":
            with torch.cuda.stream(stream):
                for s in sets:  # one eager step first so lazy initialisation is outside capture
                    s.step(sptr)
            stream.synchronize()

        def run_steps(k, start):
            """k steps from set `start`; graphs are captured before the first replay."""
            if args.mode == "graph":
                plan = [graph_of(graph_steps, start)] * (k // graph_steps)
                if k % graph_steps:  # whole graphs hold a multiple of the set count
                    plan.append(graph_of(k % graph_steps, start))
                return plan
            return [lambda i=i: sets[(start + i) % n_sets].step(sptr) for i in range(k)]

        def replay(plan):
            for g in plan:
                g.replay() if args.mode == "graph" else g()

        start = 0
        warm = run_steps(args.warmup, start)
        start += args.warmup
        plans = []
        for _ in range(args.repeats):
            plans.append(run_steps(args.steps, start))
            start += args.steps
        torch.cuda.synchronize()
        per, walls = [], []
        with torch.cuda.stream(stream):
            replay(warm)
            stream.synchronize()
            for plan in plans:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                t_wall = time.perf_counter()
                e0.record(stream)
                replay(plan)
                e1.record(stream)
                e1.synchronize()
                walls.append(time.perf_counter() - t_wall)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) / args.steps)
        mid = int(np.argsort(per)[len(per) // 2])
        return per[mid], per, walls[mid]

    other = {"fused": "separate", "separate": "fused", "paged_fused": "paged", "paged": None,
             "stochastic": None}[args.api]
    ms_other = time_api(other)[0] if other else None
    ms_per_step, ms_repeats, t_wall = time_api(args.api)
    t_step = ms_per_step * 1e-3

    # ---- per-call durations: a separate eager pass with events between the calls -------------
    # Events between eager calls include launch latency; the main kernel's own duration comes
    # from the library's profiling hook, whose events take that kernel's start and end
    # timestamps (hipExtLaunchKernel).
    n_prof = min(args.steps, 200)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(n_prof)]
    for row in ev:  # torch creates the underlying events on first record
        for e in row:
            e.record(stream)
    stream.synchronize()
    for s in sets:
        s.api = "separate"
    with torch.cuda.stream(stream):
        for i in range(n_prof):
            s = sets[i % n_sets]
            ei = ev[i]
            tv.profile_attn_main(ei[2], ei[3])
            ei[0].record(stream)
            s.mask(sptr)
            ei[1].record(stream)
            s.attn(sptr)
            ei[4].record(stream)
            s.accept(sptr)
            ei[5].record(stream)
            s.compact(sptr)
            ei[6].record(stream)
        tv.profile_attn_main(None, None)
        stream.synchronize()

    def avg(a, b):
        return float(np.mean([ev[i][a].elapsed_time(ev[i][b]) for i in range(n_prof)])) * 1e-3

    t_mask, t_attn, t_main, t_accept, t_compact = avg(0, 1), avg(1, 4), avg(2, 3), avg(4, 5), avg(5, 6)

    # the same for the fused step: its main kernel (which also builds the masks) and the whole
    # call (main kernel, then merge + acceptance + compaction)
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_prof)]
    for row in evf:
        for e in row:
            e.record(stream)
    stream.synchronize()
    with torch.cuda.stream(stream):
        for i in range(n_prof):
            s = sets[i % n_sets]
            ei = evf[i]
            tv.profile_attn_main(ei[1], ei[2])
            ei[0].record(stream)
            s.fused(sptr)
            ei[3].record(stream)
        tv.profile_attn_main(None, None)
        stream.synchronize()
    t_main_fused = float(np.mean([evf[i][1].elapsed_time(evf[i][2]) for i in range(n_prof)])) * 1e-3
    t_fused_call = float(np.mean([evf[i][0].elapsed_time(evf[i][3]) for i in range(n_prof)])) * 1e-3
    if args.api == "fused":
        t_main = t_main_fused

    # paged K/V: the same calls with the attention reading the pool through the block table and
    # the commit by pointer swap; the dense pass above timed the copying commit on the same path
    paged_breakdown = None
    if args.kv == "paged":
        evp = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(n_prof)]
        for row in evp:
            for e in row:
                e.record(stream)
        stream.synchronize()
        with torch.cuda.stream(stream):
            for i in range(n_prof):
                s = sets[i % n_sets]
                ei = evp[i]
                tv.profile_attn_main(ei[2], ei[3])
                ei[0].record(stream)
                s.mask(sptr)
                ei[1].record(stream)
                s.attn_paged(sptr)
                ei[4].record(stream)
                s.accept(sptr)
                ei[5].record(stream)
                s.commit(sptr)
                ei[6].record(stream)
            tv.profile_attn_main(None, None)
            stream.synchronize()

        def pavg(a, b):
            return float(np.mean([evp[i][a].elapsed_time(evp[i][b]) for i in range(n_prof)])) * 1e-3

        t_main = t_main_call = pavg(2, 3)
        # the fused paged step, its main kernel by the same hook
        step_paged_us = main_step_paged_us = None
        if paged.page_size == 1:
            evq = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                   for _ in range(n_prof)]
            for row in evq:
                for e in row:
                    e.record(stream)
            stream.synchronize()
            with torch.cuda.stream(stream):
                for i in range(n_prof):
                    ei = evq[i]
                    tv.profile_attn_main(ei[1], ei[2])
                    ei[0].record(stream)
                    sets[i % n_sets].fused_paged(sptr)
                    ei[3].record(stream)
                tv.profile_attn_main(None, None)
                stream.synchronize()
            step_paged_us = float(np.mean([evq[i][0].elapsed_time(evq[i][3])
                                           for i in range(n_prof)])) * 1e3
            main_step_paged_us = float(np.mean([evq[i][1].elapsed_time(evq[i][2])
                                                for i in range(n_prof)])) * 1e3
            if args.api == "paged_fused":  # the roofline takes the kernel the step runs
                t_main = main_step_paged_us * 1e-6
        paged_breakdown = {
            "page_size": paged.page_size, "num_slots": paged.num_slots,
            "max_pages": int(paged.block_table.shape[1]),
            "tree_verify_attn_paged_us": pavg(1, 4) * 1e6, "attn_main_paged_us": t_main_call * 1e6,
            "kv_commit_paged_us": pavg(5, 6) * 1e6 if paged.page_size == 1 else None,
            "kv_compact_accepted_copy_us": t_compact * 1e6,
            "tree_verify_step_paged_us": step_paged_us,
            "attn_main_step_paged_us": main_step_paged_us,
            "note": ("per-call times from events between eager calls (launch latency included); "
                     "attn_main_* from the kernel's own timestamps"),
        }

    # stochastic acceptance: the same calls with tree_accept_stochastic in place of tree_accept;
    # the kernel's own duration comes from its profiling hook
    stoch_breakdown = None
    if stoch is not None:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_prof)]
        for row in evs:
            for e in row:
                e.record(stream)
        stream.synchronize()
        with torch.cuda.stream(stream):
            for i in range(n_prof):
                s = sets[i % n_sets]
                ei = evs[i]
                s.mask(sptr)
                s.attn(sptr)
                tv.profile_accept_stochastic(ei[1], ei[2])
                ei[0].record(stream)
                s.accept_stochastic(sptr)
                ei[3].record(stream)
                s.compact(sptr)
            tv.profile_accept_stochastic(None, None)
            stream.synchronize()
        t_sk = float(np.mean([evs[i][1].elapsed_time(evs[i][2]) for i in range(n_prof)])) * 1e-3
        t_sc = float(np.mean([evs[i][0].elapsed_time(evs[i][3]) for i in range(n_prof)])) * 1e-3
        spath = sets[0].t["path"].cpu().numpy()
        slen = sets[0].t["alen"].cpu().numpy()
        sweeps, sbytes = stochastic_work(w.parent, stoch.draft, spath, slen, stoch.V)
        stoch_breakdown = {
            "vocab": stoch.V, "sampling": args.sampling,
            "workgroups_per_seq": (stoch_ws.numel() - 4 * w.B) // (16 * w.B * w.T)
            if stoch_ws is not None else 1,
            "mean_accept_len": float(slen.mean()),
            "vocab_sweeps_per_call": sweeps,
            "algorithmic_bytes_per_call": sbytes,
            "kernel_us": t_sk * 1e6,
            "call_us": t_sc * 1e6,
            "tree_accept_greedy_us": t_accept * 1e6,
            "achieved_gbps": sbytes / t_sk / 1e9,
            "hbm_frac": sbytes / t_sk / 1e9 / HBM_PEAK_GBS,
            "note": ("kernel_us from the kernel's own timestamps; call_us from events between "
                     "eager calls (launch latency included); bytes: p and q rows of every "
                     "vocabulary sweep the walk makes (one per rejected child, one for the bonus "
                     "draw)"),
        }

    construction = None
    if args.construct:
        print("[bench] timing EAGLE-2 tree construction", file=sys.stderr, flush=True)
        construction = construction_bench(tv, torch, w, stream, args.steps, args.warmup)

    lm_head = None
    if args.lm_head:
        print(f"[bench] timing the two-stage drafter LM head {args.lm_head}", file=sys.stderr,
              flush=True)
        lm_head = lm_head_bench(tv, torch, args.lm_head, stream, args.steps, args.warmup)

    alen = sets[0].t["alen"].cpu().numpy()
    status = sets[0].t["status"].cpu().numpy()
    if (status & ~0).any():
        print(f"[bench] warning: device status bits set: {np.unique(status)}", file=sys.stderr)

    # ---- roofline of the dominant kernel ------------------------------------------------------
    intensity = flops / kv_bytes
    peak_tf = MFMA_PEAK_TFLOPS[w.dtype]
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = None
    if os.path.exists(COUNTERS_FILE) and args.kv == "dense":  # counters of the dense kernel
        with open(COUNTERS_FILE, encoding="utf-8") as f:
            cnt = json.load(f)
        rec = cnt.get(args.workload)
        if rec and rec.get("kernel_source_hash") == kernel_source_hash():
            traffic = rec.get("hbm_bytes_per_launch")
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": kv_bytes / t_main / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t_main / 1e12, "peak": peak_tf,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["kernel"] = {"fused": "attn_main (tree_verify_step's instantiation, which also builds "
                               "the masks)",
                      "separate": "attn_main",
                      "paged": "attn_main (tree_verify_attn_paged's instantiation)",
                      "paged_fused": "attn_main (tree_verify_step_paged's instantiation, which "
                                     "also builds the masks)",
                      "stochastic": "attn_main"}[args.api]
    roof["kernel_us"] = t_main * 1e6
    roof["algorithmic_bytes"] = kv_bytes
    roof["algorithmic_flops"] = flops

    value = kv_bytes / t_step / 1e9
    result = {
        "metric": "tree-verify attn KV-read GB/s (% HBM peak) + verified tree tokens/sec",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_repeats": ms_repeats,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "desc": w.spec.desc, "B": w.B, "T": w.T,
                   "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "prefix_tokens": int(L.sum()),
                   "Lmax": w.Lmax, "layers": 1, "mode": args.mode, "rotated_sets": n_sets,
                   "split_keys": args.split_keys, "step_api": args.api, "kv": args.kv,
                   "accept": args.accept,
                   "graph_steps": graph_steps if args.mode == "graph" else None},
        "ms_per_step_by_api": ({args.api: ms_per_step, other: ms_other} if other
                               else {args.api: ms_per_step}),
        "paged": paged_breakdown,
        "stochastic": stoch_breakdown,
        "construction": construction,
        "lm_head": lm_head,
        "hbm_frac": value / HBM_PEAK_GBS,
        "attn_kv_gbps": kv_bytes / t_attn / 1e9,
        "attn_hbm_frac": kv_bytes / t_attn / 1e9 / HBM_PEAK_GBS,
        "attn_mfma_frac": flops / t_attn / 1e12 / peak_tf,
        "tree_tokens_per_s": w.B * w.T / t_step,
        "accepted_tokens_per_s": float(alen.sum()) / t_step,
        "step_breakdown_us": {"tree_build_mask": t_mask * 1e6, "tree_verify_attn": t_attn * 1e6,
                              "attn_main": avg(2, 3) * 1e6, "tree_accept": t_accept * 1e6,
                              "kv_compact_accepted": t_compact * 1e6},
        "fused_step_breakdown_us": {"tree_verify_step": t_fused_call * 1e6,
                                    "attn_main_with_masks": t_main_fused * 1e6},
        "wall_s_timed": t_wall,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, kv_bytes, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    others = [x for x in args.also.split(",") if x and x != args.workload]
    if others:
        del sets
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["other_workloads"] = {x: other_workload_bench(tv, torch, x, args, stream)
                                     for x in others}
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
