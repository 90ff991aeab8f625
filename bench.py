"""Benchmark of one tree-verification step on one MI355X.

A step is the whole hot path on one batch: the tree mask, the ancestor-masked
tree attention, the acceptance with its bonus token and the commit of the
accepted path.  By default it is one sv_verify_step launch (when the call
supports the workload); --separate-calls runs sv_build_tree_mask, then
sv_tree_attention beside sv_accept (whose walker commits the accepted path;
--separate-commit: its own sv_kv_commit launch) on a side stream, joined at the
end of the step (--no-overlap: all on one stream).  The default workload is
the EAGLE-style static tree at the Llama-3-8B attention shape (batch 1, 32
query / 8 KV heads, head_dim 128, 4096-token bf16 prefix, 60-node tree of
depth 6, vocab 128256, stochastic acceptance at T = 1).

Inputs are resident in HBM before timing starts.  R independent input
instances are cycled so that the working set (R x step bytes) exceeds twice
the 256 MB Infinity Cache and every step reads HBM, not a warm cache.  The
timed region is one replay of a HIP graph of exactly K steps (instances
cycled), repeated --reps times; ms_per_step is the median.  Stage times come
from graphs of K launches of one stage each.

Prints one JSON line: value = verified tree tokens/s (B*N / step time), with
the roofline of the dominant kernel measured live with HIP events on the
launch stream, a measured streaming-read ceiling, and the CPU oracle timed on
a bounded sample on the host (with the count of flagged stochastic draws).
"""
import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0   # dense bf16 MFMA peak of MI355X
VALU_FP32_TFLOPS = 157.3    # fp32 vector peak of MI355X
MALL_BYTES = 256 * 2**20
# batches up to this many logits rows run the step as one sv_verify_step launch, and stochastic
# or top-K walks over wide trees (the walk advances as rows resolve) up to ONE_LAUNCH_MAX_ROWS_WIDE
# (MI355X, one launch vs separate calls: eagle-static-8b 61 rows 33 vs 42 us, its batch 4 84 vs
# 94 us, batch 8 152 vs 154 us, batch 16 (976 rows) 254 vs 270 us; draft-target-chain-8b, 768
# rows, 467 vs 390 us; batched-paged-70b, 2112 rows, 586 vs 566 us; outcome-tree-8b, 4112 rows,
# 2900 vs 2749 us)
ONE_LAUNCH_MAX_ROWS = 256
ONE_LAUNCH_MAX_ROWS_WIDE = 1024


def threshold_rows(w, acc):
    """Logits rows a threshold walk must read: breadth first from the root row through the
    children whose path score p_r(token) products stay at or above the threshold."""
    import workloads as W
    T, tau = float(w.temperature), float(w.threshold)
    n = 0
    for b in range(w.B):
        par, tok = w.parents[b], w.tokens[b]
        kids = {}
        for i in range(w.N):
            kids.setdefault(int(par[i]) + 1, []).append(i)
        todo, seen = [(0, 1.0)], set()
        while todo:
            r, sc = todo.pop()
            seen.add(r)
            row = w.target_logits[b, r]
            x = (W.bf16_to_f32(row) if row.dtype == np.uint16 else row).astype(np.float64) / T
            p = np.exp(x - x.max())
            p /= p.sum()
            for c in kids.get(r, []):
                if 0 <= tok[c] < w.V and sc * p[tok[c]] >= tau and c + 1 in kids:
                    todo.append((c + 1, sc * p[tok[c]]))
        n += len(seen) + (0 if int(acc["stop_row"][b]) in seen else 1)
    return n


def algorithmic_bytes(w, acc):
    """Bytes each stage must move at minimum (per step), from the workload and its accept results."""
    e = 2 if w.dtype == "bf16" else 4
    el = 2 if w.target_logits.dtype == np.uint16 else 4
    B, N, Hq, Hkv, D, V = w.B, w.N, w.Hq, w.Hkv, w.D, w.V
    W = (N + 63) // 64
    L = w.prefix_len.astype(np.int64)
    attn = int(L.sum()) * Hkv * D * 2 * e + B * N * Hkv * D * 2 * e + 2 * B * N * Hq * D * e + B * N * W * 8
    if w.paged:
        attn += int(((L + w.block_size - 1) // w.block_size).sum()) * 4
    n_t = 2 if w.mode == "stochastic" else 1
    rows = 0
    if w.mode == "greedy":
        # the accepted path's rows, the stop row included: where the path goes next is known
        # only from the argmax of the row before, and no other row decides the result (sibling
        # tokens that tie would add the rows below the tie)
        rows = int((acc["accept_len"].astype(np.int64) + 1).sum())
    elif w.mode == "threshold":
        # the rows of the root and of every node whose path scores at least the threshold and
        # that has children (a deeper passing node can only be found through them), plus the
        # stop row when it has none
        rows = threshold_rows(w, acc)
    else:  # every row of a node with a child (and the draft rows in mode 1), plus the stop row
        for b in range(B):
            par = w.parents[b]
            needed = {0} | set((par[par >= 0] + 1).tolist())
            stop = int(acc["stop_row"][b])
            rows += len(needed) * n_t + (0 if stop in needed else 1)
    accept = rows * V * el
    A = acc["accept_len"].astype(np.int64)
    if w.tree_in_cache:  # the in-place commit moves only rows not already at their position
        moved = sum(int((acc["accept_rows"][b, :A[b]] - 1 != np.arange(A[b])).sum()) for b in range(B))
    else:
        moved = int(A.sum())
    commit = moved * Hkv * D * 2 * e * 2
    mask = 4 * B * N + B * N * (8 * W + 4 + 4 * w.max_depth)
    # attention flops: q.k and p.v over the prefix and each node's root path (2 flops per multiply-add)
    import workloads as W
    keys = sum(int(L[b]) * N + int(W.tree_depths(w.parents[b]).sum()) for b in range(B))
    attn_flops = 4 * Hq * D * keys
    return dict(mask=mask, attention=attn, accept=accept, commit=commit,
                total=mask + attn + accept + commit, attention_flops=attn_flops)


_CS = "tree_verification_sv_amd/csrc/"
# the sources whose device code each timed stage runs (a counter summary stays valid while they
# are unchanged)
KERNEL_SOURCES = {
    "verify_step": [_CS + f for f in ("sv_step.hip", "sv_accept_dev.h", "sv_attn_dev.h", "sv_mask_dev.h",
                                      "sv_commit_dev.h", "sv_common.h")],
    "attention": [_CS + f for f in ("sv_attention.hip", "sv_attn_dev.h", "sv_mask_dev.h", "sv_common.h")],
    "accept": [_CS + f for f in ("sv_accept.hip", "sv_accept_dev.h", "sv_commit_dev.h", "sv_common.h")],
}


def source_hash(files):
    """Hash of the kernel sources without their comments and with blank space collapsed, so that
    an edit of comments alone keeps a committed counter summary valid."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, kernel_src_hash, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or None when
    the summary is missing or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_src_hash:
        return None
    return d.get("bytes_per_launch")


def host_info():
    """Host threads available to this process and the CPU model, for the baseline lines."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def seq_slice(w, b):
    """Sequence b of a workload as a batch of one (the paged K/V pool is shared, not copied)."""
    import dataclasses
    sl = lambda x: None if x is None else x[b:b + 1]  # noqa: E731
    kw = dict(B=1, parents=sl(w.parents), tokens=sl(w.tokens), prefix_len=sl(w.prefix_len), q=sl(w.q),
              k_tree=sl(w.k_tree), v_tree=sl(w.v_tree), block_table=sl(w.block_table),
              target_logits=sl(w.target_logits), draft_logits=sl(w.draft_logits), u_accept=sl(w.u_accept),
              u_sample=sl(w.u_sample))
    if not w.paged:
        kw.update(k_cache=sl(w.k_cache), v_cache=sl(w.v_cache))
    return dataclasses.replace(w, **kw)


def cpu_baseline(cfg, budget_s=10.0, variant=None, over=None):
    """The CPU oracle as it stands on one step of the same workload, on one host thread and
    fanned out over host threads.

    Mask, acceptance and commit run on the whole batch; the attention runs on a seeded sample of
    query rows (b, node, head) sized to about ``budget_s`` seconds and is scaled linearly to all
    B*N*Hq rows (every row costs the same prefix pass up to its own few tree keys).  The
    all-threads line runs every stage in parallel: mask, acceptance and commit over sequences,
    the attention sample over row chunks.  Input generation is not timed.
    """
    import oracle
    import workloads as W
    from concurrent.futures import ThreadPoolExecutor
    w = W.config(cfg, seed=cfg * 1000, **(over or {}))
    if variant is not None:
        w = variant(w)
    nproc, cpu_model = host_info()
    total_rows = w.B * w.N * w.Hq
    t0 = time.perf_counter()
    oracle.build_tree_mask(w.parents, w.max_depth)
    t_mask = time.perf_counter() - t0
    # attention: time a small probe, then a sample that fills the budget
    probe = np.unique(W.randint(cfg, 91, 16, 0, total_rows - 1)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.tree_attention(w, sel=probe)
    per_row = (time.perf_counter() - t0) / probe.size
    n = int(min(total_rows, max(probe.size, budget_s / max(per_row, 1e-9))))
    sel = np.arange(total_rows, dtype=np.int64) if n >= total_rows else \
        np.unique(W.randint(cfg, 92, n, 0, total_rows - 1)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.tree_attention(w, sel=sel)
    t_attn = (time.perf_counter() - t0) * total_rows / sel.size
    t0 = time.perf_counter()
    acc = oracle.accept(w)
    t_acc = time.perf_counter() - t0
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    t0 = time.perf_counter()
    oracle.kv_commit(w, acc["accept_len"], acc["accept_rows"], kc, vc)
    t_com = time.perf_counter() - t0
    dt = t_mask + t_attn + t_acc + t_com
    scaled = "all rows" if sel.size == total_rows else f"{sel.size} of {total_rows} rows, scaled linearly"
    one = dict(value=round(w.B * w.N / dt, 3), unit="tokens/s", cores=1, kind="oracle", nproc=nproc,
               cpu_model=cpu_model,
               sample=f"one verification step of the {w.name} workload (B={w.B}, N={w.N}, "
                      f"L={int(w.prefix_len.max())}, V={w.V}, {w.mode} acceptance) on one host thread: mask, "
                      f"acceptance and commit on the whole batch ({t_mask + t_acc + t_com:.2f} s), fp64 attention "
                      f"on {scaled} ({t_attn:.1f} s for the step)")
    # every stage over host threads (the oracle's C code runs outside the interpreter lock)
    nthreads = max(1, min(16, nproc))
    seqs = [seq_slice(w, b) for b in range(w.B)]
    chunks = [c for c in np.array_split(sel, nthreads) if c.size]
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda s_: oracle.build_tree_mask(s_.parents, s_.max_depth), seqs))
        t_mask_mt = time.perf_counter() - t0
        t0 = time.perf_counter()
        list(ex.map(lambda c: oracle.tree_attention(w, sel=np.ascontiguousarray(c)), chunks))
        t_attn_mt = (time.perf_counter() - t0) * total_rows / sel.size
        t0 = time.perf_counter()
        accs = list(ex.map(oracle.accept, seqs))
        t_acc_mt = time.perf_counter() - t0
        kcs = [kc if w.paged else kc[b:b + 1] for b in range(w.B)]
        vcs = [vc if w.paged else vc[b:b + 1] for b in range(w.B)]
        t0 = time.perf_counter()
        list(ex.map(lambda i: oracle.kv_commit(seqs[i], accs[i]["accept_len"], accs[i]["accept_rows"], kcs[i], vcs[i]),
                    range(w.B)))
        t_com_mt = time.perf_counter() - t0
    dt_mt = t_mask_mt + t_attn_mt + t_acc_mt + t_com_mt
    many = dict(value=round(w.B * w.N / dt_mt, 3), unit="tokens/s", cores=nthreads, kind="oracle", nproc=nproc,
                cpu_model=cpu_model,
                sample=f"as cpu_baseline with every stage over {nthreads} host threads: mask, acceptance and "
                       f"commit over the {w.B} sequences ({t_mask_mt + t_acc_mt + t_com_mt:.2f} s), the attention "
                       f"sample over row chunks ({t_attn_mt:.1f} s for the step)")
    return one, many


def flagged_draws(ws):
    """Stochastic draws of the timed instances that the oracle flags (within 1e-6 of a threshold):
    the sequences excluded from exact comparison."""
    import oracle
    if ws[0].mode not in ("stochastic", "topk", "threshold"):
        return 0
    return int(sum(int(oracle.accept(w)["flagged"].sum()) for w in ws))


def stream_read_ceiling(dev, gib=2, reps=5):
    """A measured streaming-read ceiling: torch's sum over a fresh 2 GiB fp32 tensor (far larger
    than the 256 MB last-level cache), median of `reps` timed calls."""
    import torch
    x = torch.ones((gib << 30) // 4, dtype=torch.float32, device=dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    for _ in range(2):
        torch.sum(x, dim=0, out=out)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.sum(x, dim=0, out=out)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    del x
    ms = float(np.median(ts))
    return round((gib << 30) / (ms * 1e-3) / 1e9, 1)


def commit_layers(w, dev, acc, layers, K):
    """Time one sv_kv_commit over `layers` layers of the workload's cache shape (HIP events).

    Every layer shares the workload's tree, lengths, accepted rows and block table; the
    caches of the extra layers are plain device allocations (their contents do not change
    the work).  Replays are idempotent only in bytes moved, which is what is timed."""
    import torch
    import tree_verification_sv_amd as sv
    kc = dev["k_cache"].unsqueeze(0).repeat(layers, *([1] * dev["k_cache"].dim()))
    vc = dev["v_cache"].unsqueeze(0).repeat(layers, *([1] * dev["v_cache"].dim()))
    tic = w.tree_in_cache
    kt = None if tic else dev["k_tree"].unsqueeze(0).repeat(layers, *([1] * dev["k_tree"].dim()))
    vt = None if tic else dev["v_tree"].unsqueeze(0).repeat(layers, *([1] * dev["v_tree"].dim()))
    alen = torch.from_numpy(acc["accept_len"]).to(kc.device)
    arows = torch.from_numpy(np.ascontiguousarray(acc["accept_rows"])).to(kc.device)
    outs = dict(new_len=torch.empty(w.B, dtype=torch.int32, device=kc.device),
                committed_slots=torch.empty((w.B, w.max_depth), dtype=torch.int32, device=kc.device),
                status=torch.empty(w.B, dtype=torch.int32, device=kc.device))
    run = lambda: sv.sv_kv_commit(kc, vc, kt, vt, dev["prefix_len"], alen, arows, w.max_depth,  # noqa: E731
                                  block_table=dev["block_table"], paged=w.paged, num_blocks=w.num_blocks,
                                  outs=outs, tree_in_cache=tic, N=w.N, num_layers=layers)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    e = 2 if w.dtype == "bf16" else 4
    A = acc["accept_len"].astype(np.int64)
    if tic:  # rows already in place are not moved
        moved = sum(int((acc["accept_rows"][bb, :A[bb]] - 1 != np.arange(A[bb])).sum()) for bb in range(w.B))
    else:
        moved = int(A.sum())
    byts = layers * moved * w.Hkv * w.D * e * 2 * 2  # K and V rows, read + write
    return dict(layers=layers, ms=round(ms, 5), rows_moved_per_layer=moved, bytes=byts,
                gbs=round(byts / (ms * 1e-3) / 1e9, 1), tree_kv="in cache" if tic else "separate rows")


def time_extras(w, dev, acc, K_steps):
    """Time the operations around the step on this workload's shape (HIP events over a replayed
    graph of K launches each):
    the SSD outcome lookup (8 prepared outcomes of max_depth tokens per sequence), Saguaro
    reweighting (8 cached tokens per row of the draft logits) and the draft vocabulary subset
    (a 32000-id subset laid out over the target vocabulary)."""
    import torch
    import tree_verification_sv_amd as sv
    import workloads as W
    B, R, V, Dm = w.B, w.N + 1, w.V, w.max_depth
    d = "cuda:0"
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(d)  # noqa: E731
    K, P, C, Vd = 8, Dm, 8, 32000
    res = {}

    def timed(fn):
        """Average device time of one call: K_steps calls captured in a HIP graph and replayed,
        so that the host's per-call overhead (larger than these small kernels) is not timed."""
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(K_steps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        a.record(s)
        g.replay()
        b.record(s)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K_steps

    keys_r = t(W.randint(w.seed, 93, B * K, 0, w.N).reshape(B, K))
    keys_t = t(W.randint(w.seed, 94, B * K, 0, V - 1).reshape(B, K))
    prep = t(W.randint(w.seed, 95, B * K * P, 0, V - 1).reshape(B, K, P))
    nk = t(np.full(B, K))
    st, ot, no = t(acc["stop_row"]), t(acc["out_tokens"]), t(acc["num_out"])
    outs = dict(hit=torch.empty(B, dtype=torch.int32, device=d), branch=torch.empty(B, dtype=torch.int32, device=d),
                next_tokens=torch.empty((B, P), dtype=torch.int32, device=d),
                n_hits=torch.empty(1, dtype=torch.int32, device=d))
    ms = timed(lambda: sv.sv_outcome_lookup(st, ot, no, keys_r, keys_t, nk, prep, outs=outs))
    res["outcome_lookup"] = dict(ms=round(ms, 5), batch=B, keys=K, prepared_tokens=P)
    logits = dev["draft_logits"] if dev["draft_logits"] is not None else dev["target_logits"].clone()
    ct = t(W.randint(w.seed, 96, B * R * C, 0, V - 1).reshape(B, R, C))
    e = logits.element_size()
    ms = timed(lambda: sv.sv_saguaro_reweight(logits, ct, -0.5))
    res["saguaro_reweight"] = dict(ms=round(ms, 5), rows=B * R, cached_per_row=C)
    ids = np.argsort(W.u64(w.seed, 97, V))[:Vd]
    t2d = np.zeros(V, np.int32)
    t2d[ids] = np.arange(1, Vd + 1, dtype=np.int32)
    t2d_d = t(t2d)
    sub = logits[:, :, :Vd].contiguous()
    full = torch.empty_like(logits)
    ms = timed(lambda: sv.sv_draft_subset_logits(sub, t2d_d, out=full))
    byts = B * R * V * e + B * R * Vd * e + V * 4
    res["draft_subset"] = dict(ms=round(ms, 5), rows=B * R, subset=Vd, bytes=byts,
                               gbs=round(byts / (ms * 1e-3) / 1e9, 1), frac=round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--batch", type=int, default=0,
                    help="override the workload's batch (sequences of the same shape, each with its own tree)")
    ap.add_argument("--instances", type=int, default=0, help="input instances cycled (0: enough to defeat the MALL)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-overlap", action="store_true",
                    help="run the four stages back to back on one stream (default: acceptance and commit on a "
                         "side stream beside the attention, forked after the mask, except for stochastic wide "
                         "trees of more than 1024 rows)")
    ap.add_argument("--overlap", action="store_true",
                    help="the side-stream form also for stochastic wide trees of more than 1024 rows")
    ap.add_argument("--attention-side", action="store_true",
                    help="overlapped step with the attention on the side stream and acceptance + commit on the "
                         "launch stream")
    ap.add_argument("--separate-commit", action="store_true",
                    help="commit with its own sv_kv_commit launch (default: the acceptance kernel commits the "
                         "accepted path itself, one launch less; not with --tree-in-cache)")
    ap.add_argument("--mask-free-accept", action="store_true",
                    help="stochastic / top-K: the acceptance derives node depths from the parents itself and its "
                         "branch forks before the mask")
    ap.add_argument("--separate-calls", action="store_true",
                    help="run the step as separate library calls (mask, attention, acceptance, commit) instead "
                         "of one sv_verify_step launch")
    ap.add_argument("--one-launch", action="store_true",
                    help="run the step as one sv_verify_step launch whatever the batch (default: one launch for "
                         f"batches of at most {ONE_LAUNCH_MAX_ROWS} logits rows, or {ONE_LAUNCH_MAX_ROWS_WIDE} for "
                         "stochastic and top-K walks over wide trees, where the separate calls' launch gaps dominate; "
                         "the separate calls above that, where the two branches filling the device side by side "
                         "measured faster on MI355X)")
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions of the K-step graph (median reported)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--acceptance", choices=["greedy", "stochastic", "topk", "threshold"], default=None,
                    help="acceptance rule (default: the workload's own)")
    ap.add_argument("--threshold", type=float, default=1e-4, help="score threshold of --acceptance threshold")
    ap.add_argument("--tree-in-cache", action="store_true",
                    help="keep the tree tokens' K/V in the cache at positions prefix_len + t (attention reads them "
                         "there, the commit compacts the accepted path in place after the attention)")
    ap.add_argument("--commit-layers", type=int, default=0,
                    help="also time one layer-batched sv_kv_commit over this many layers of the workload's shape")
    ap.add_argument("--extras", action="store_true",
                    help="also time the SSD outcome lookup, Saguaro reweighting and draft vocabulary subset")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (reference kernel for PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: --gpus {args.gpus} is not supported "
              f"(sequences and KV heads shard with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from tree_verification_sv_amd.step import VerifyStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    over = {"B": args.batch} if args.batch else {}
    w0 = W.config(args.config, **over)
    # bytes one instance touches: the prefix K/V it reads plus its logits rows
    step_bytes_est = w0.target_logits.nbytes * 2 + int(w0.prefix_len.sum()) * w0.Hkv * w0.D * 2 * (2 if w0.dtype == "bf16" else 4)
    R = args.instances or max(1, min(32, int(np.ceil(2 * MALL_BYTES / max(step_bytes_est, 1)))))
    print(f"[bench] workload {w0.name} B={w0.B} N={w0.N} L={int(w0.prefix_len.max())} V={w0.V} "
          f"instances={R} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    ws = [w0] + [W.config(args.config, seed=args.config * 1000 + r, **over) for r in range(1, R)]
    def variant(w):
        if args.acceptance:
            w.mode = args.acceptance
            w.threshold = float(np.float32(args.threshold))
        return W.with_tree_in_cache(w) if args.tree_in_cache else w

    ws = [variant(w) for w in ws]
    w0 = ws[0]
    devs = [W.to_device(w, dev) for w in ws]
    steps = [VerifyStep(W.step_inputs(w, d)) for w, d in zip(ws, devs)]
    fused = not args.separate_commit and not args.tree_in_cache
    if fused:
        for s_ in steps:
            s_.fuse_commit(True)
    mask_free = args.mask_free_accept and w0.mode in ("stochastic", "topk")
    if mask_free:
        for s_ in steps:
            s_.mask_free_accept(True)
    one = False
    rows = w0.B * (w0.N + 1)
    wide = w0.mode in ("stochastic", "topk") and w0.N > 2 * w0.max_depth
    limit = ONE_LAUNCH_MAX_ROWS_WIDE if wide else ONE_LAUNCH_MAX_ROWS
    if not args.separate_calls and not mask_free and (args.one_launch or rows <= limit):
        one = all([s_.one_launch(True) for s_ in steps])
        if not one:
            print("[bench] sv_verify_step does not support this workload; timing the separate calls",
                  file=sys.stderr, flush=True)
            for s_ in steps:
                s_.one_launch(False)
    stream = torch.cuda.current_stream()

    # Stochastic wide trees of many rows run on one stream: most of their acceptance grid is
    # row groups that leave at their start (the rows of walks that have already finished), and
    # dispatched beside the attention they slow both (outcome-tree-8b, MI355X: 3.13 ms per step
    # overlapped against 2.58 ms on one stream).
    ov = not args.no_overlap and (args.overlap or not (wide and rows > ONE_LAUNCH_MAX_ROWS_WIDE))
    run = lambda i: steps[i % R].run(overlap=ov, attention_side=args.attention_side)  # noqa: E731
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    if args.copy_mib:  # untimed reference copy: its FETCH/WRITE counters calibrate the byte counts
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    accs = [{k: v.cpu().numpy() for k, v in s.acc.items()} for s in steps]
    byts = [algorithmic_bytes(w, a) for w, a in zip(ws, accs)]
    K = args.steps

    def capture(fn, n):
        """One HIP graph of n calls fn(i), captured on a side stream after one eager round."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(min(n, R)):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        return g

    def timed(g_or_fn, reps):
        """Per-repetition milliseconds of one graph replay (or one eager call of fn) on the launch stream."""
        ts = []
        for _ in range(reps):
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a_.record(stream)
            if callable(g_or_fn):
                g_or_fn()
            else:
                g_or_fn.replay()
            b_.record(stream)
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_))
        return ts

    # ---- timed region: exactly K steps per repetition (one graph of K steps cycling the
    # instances, or K eager steps), median of `reps` repetitions
    use_graph = not args.no_graph
    graph = None
    if use_graph:
        try:
            graph = capture(run, K)
        except Exception as ex:  # capture not available: fall back to eager launches
            print(f"[bench] graph capture failed ({ex}); timing eager launches", file=sys.stderr)
            graph, use_graph = None, False
    t0 = time.perf_counter()
    rep_ms = timed(graph if graph is not None else (lambda: [run(i) for i in range(K)]), args.reps)
    wall = time.perf_counter() - t0
    ms_step = float(np.median(rep_ms)) / K
    del graph

    # ---- per-stage durations: K launches of one stage in a graph of their own (median of reps)
    stage_ms = {}
    if one:
        stage_names = ("verify_step",)
        stage_fn = {"verify_step": lambda i: steps[i % R].run()}
    else:
        stage_names = ("build_mask", "attention", "accept") + (() if steps[0]._fused else ("kv_commit",))
        stage_fn = {nm: (lambda nm_: lambda i: getattr(steps[i % R], nm_)())(nm) for nm in stage_names}
    for name in stage_names:
        try:
            g = capture(stage_fn[name], K) if use_graph else None
        except Exception:
            g = None
        ts = timed(g if g is not None else (lambda: [stage_fn[name](i) for i in range(K)]), args.reps)
        stage_ms[name] = float(np.median(ts)) / K
        del g

    layered = commit_layers(ws[0], devs[0], accs[0], args.commit_layers, K) if args.commit_layers else None
    extras = time_extras(ws[0], devs[0], accs[0], K) if args.extras else None
    ceiling = stream_read_ceiling(dev)

    mean_bytes = {k: float(np.mean([bb[k] for bb in byts])) for k in byts[0]}
    B, N = w0.B, w0.N
    value = B * N / (ms_step * 1e-3)
    hbm_gbs = mean_bytes["total"] / (ms_step * 1e-3) / 1e9
    # the dominant kernel: the one-launch step itself, or the slower of attention and acceptance
    if one:
        dom, dom_bytes, dom_ms = "verify_step", mean_bytes["total"], stage_ms["verify_step"]
    else:
        dom = max(("attention", "accept"), key=lambda k: stage_ms[k])
        dom_bytes, dom_ms = mean_bytes[dom], stage_ms[dom]
    src = KERNEL_SOURCES[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4)}
    if dom == "attention":
        # the attention is a dense contraction: it is MFMA-bound when its flops at the dense peak take
        # longer than its bytes at the HBM peak (bf16 MFMA 2500 TFLOP/s; fp32 runs on the vector ALUs)
        fpeak = MFMA_BF16_TFLOPS if w0.dtype == "bf16" else VALU_FP32_TFLOPS
        flops = mean_bytes["attention_flops"]
        if flops / (fpeak * 1e12) > mean_bytes["attention"] / (HBM_PEAK_GBS * 1e9):
            tf = flops / (dom_ms * 1e-3) / 1e12
            roof = {"bound": "mfma" if w0.dtype == "bf16" else "alu", "kernel": dom, "achieved": round(tf, 1),
                    "peak": fpeak, "unit": "TFLOP/s", "frac": round(tf / fpeak, 4)}
    traffic = load_traffic(dom, source_hash(src), w0.name)
    result = {
        "metric": "verified tree tokens/sec + HBM GB/s (% peak), 8B-shape tree verify, 1 MI355X",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w0.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w0.name, "batch": B, "tree_nodes": N, "prefix_len": int(w0.prefix_len.max()),
                   "q_heads": w0.Hq, "kv_heads": w0.Hkv, "head_dim": w0.D, "vocab": w0.V, "max_depth": w0.max_depth,
                   "acceptance": w0.mode, "temperature": w0.temperature, "instances_cycled": R,
                   **({"threshold": w0.threshold} if w0.mode == "threshold" else {}),
                   "launch": ("hip_graph" if use_graph else "eager") + (" of one sv_verify_step launch per step"
                                                                        if one else " of the separate calls"),
                   "streams": "one" if (one or not ov) else
                              ("attention | accept after mask, commit after both" if w0.tree_in_cache else
                               "mask+attention | accept+commit" if mask_free else
                               "attention | accept+commit after mask"),
                   "tree_kv": "in cache at prefix_len + t" if w0.tree_in_cache else "separate rows",
                   "commit": "inside the acceptance" if steps[0]._fused else "sv_kv_commit"},
        "timing": {"reps": len(rep_ms), "ms_per_step_reps": [round(x / K, 5) for x in rep_ms],
                   "statistic": "median of the repetitions, each one replay of a graph of exactly K steps"},
        "accept_steps_per_s": round(B / (ms_step * 1e-3), 1),
        "hbm_gbs": round(hbm_gbs, 1),
        "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "stream_read_gbs": ceiling,
        "frac_of_stream_read": round(hbm_gbs / ceiling, 4) if ceiling else None,
        "bytes_per_step": {k: int(v) for k, v in mean_bytes.items() if k != "attention_flops"},
        "attention_flops_per_step": int(mean_bytes["attention_flops"]),
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "mean_accept_len": float(np.mean([a["accept_len"].mean() for a in accs])),
        "emitted_tokens_per_s": round(float(np.mean([a["num_out"].sum() for a in accs])) / (ms_step * 1e-3), 1),
        "roofline": {**roof, "traffic": traffic if roof["bound"] == "hbm" else None},
        "wall_s_timed": round(wall, 3),
    }
    if layered is not None:
        result["layered_commit"] = layered
    if extras is not None:
        result["extras"] = extras
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one step", file=sys.stderr, flush=True)
        result["flagged_draws"] = flagged_draws(ws)
        result["cpu_baseline"], result["cpu_baseline_all_cores"] = cpu_baseline(args.config, variant=variant,
                                                                                  over=over)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
