"""GPU vs oracle parity for the commit done by the acceptance kernel (sv_accept_args.commit).

The acceptance walker that finds a sequence's path also commits it; the result
must be the oracle's commit of the oracle's accepted path: new lengths,
committed slots, statuses and every cache byte, in every acceptance mode.
Sequences whose stochastic draws the oracle flags are excluded (their cache
positions L .. L + max_depth are masked on both sides).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import compare_accept, require_gpu, to_np

pytestmark = pytest.mark.gpu

SMALL = {
    1: dict(),
    2: dict(L=333, V=3001),
    3: dict(B=5, L=(40, 400), V=2500, N=32),
    4: dict(B=6, L=161, V=2999),
    5: dict(B=2, L=290, V=1500),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _mask_positions(w, cache, b):
    """Zero cache positions [L_b, L_b + max_depth) of sequence b (all heads), where they exist."""
    L = int(w.prefix_len[b])
    for pos in range(max(L, 0), L + w.max_depth):
        if w.paged:
            blk = pos // w.block_size
            if blk >= w.block_table.shape[1] or w.block_table[b, blk] <= 0:
                continue
            cache[w.block_table[b, blk], :, pos % w.block_size] = 0
        elif 0 <= pos < w.Lcap:
            cache[b, :, pos] = 0


def _run_fused(w):
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    print(f"[gpu] fused commit {w.name} B={w.B} N={w.N} V={w.V} mode={w.mode} paged={w.paged}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    step.fuse_commit(True)
    step.build_mask()
    step.accept()
    step.kv_commit()  # a no-op: the acceptance kernel has committed
    torch.cuda.synchronize()
    r = dict(acc={k: to_np(v) for k, v in step.acc.items()}, commit={k: to_np(v) for k, v in step.commit.items()},
             k_cache=to_np(dev["k_cache"]), v_cache=to_np(dev["v_cache"]))
    del step, dev
    return r


def _check(w):
    r = _run_fused(w)
    acc = oracle.accept(w)
    compare_accept(r["acc"], acc)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ref = oracle.kv_commit(w, acc["accept_len"], acc["accept_rows"], kc, vc)
    ok = acc["flagged"] == 0
    for k in ("new_len", "committed_slots", "status"):
        assert np.array_equal(r["commit"][k][ok], ref[k][ok]), k
    gk, gv = r["k_cache"], r["v_cache"]
    for b in np.nonzero(~ok)[0]:
        for c in (gk, gv, kc, vc):
            _mask_positions(w, c, int(b))
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
    return acc


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_fused_commit_small(cfg):
    acc = _check(W.config(cfg, **SMALL[cfg]))
    print(f"  accept_len {acc['accept_len'].tolist()}")


@pytest.mark.parametrize("cfg,mode", [(2, "topk"), (4, "topk"), (3, "threshold"), (2, "threshold")])
def test_fused_commit_other_modes(cfg, mode):
    w = W.config(cfg, **SMALL[cfg], **({"mode": mode} if mode == "topk" else {}))
    if mode == "threshold":
        w.mode, w.threshold = "threshold", float(np.float32(1e-6 if cfg == 2 else 1e-3))
    _check(w)


@pytest.mark.parametrize("cfg", [2, 3])
def test_fused_commit_full_size(cfg):
    _check(W.config(cfg))


@pytest.mark.parametrize("paged", [False, True])
def test_fused_commit_capacity_error(paged):
    """A sequence whose accepted path would pass the capacity gets status 6 and nothing written."""
    w = W.config(3 if paged else 1, **(SMALL[3] if paged else dict(plant=4)))
    cap = w.max_blocks * w.block_size if paged else w.Lcap
    w.prefix_len = w.prefix_len.copy()
    w.prefix_len[0] = cap - 1
    acc = _check(w)
    if acc["accept_len"][0] >= 2:
        ref = oracle.kv_commit(w, acc["accept_len"], acc["accept_rows"], w.k_cache.copy(), w.v_cache.copy())
        assert ref["status"][0] in ((5, 6) if paged else (6,))  # past the sequence's blocks, or the capacity
