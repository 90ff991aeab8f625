"""GPU vs oracle parity for acceptance without the mask outputs (sv_accept with NULL
anc_bits and depth, modes 0, 1 and 2): the kernel derives each node's depth from the parent
array by the mask's rule, so the outputs must equal the oracle's, and the GPU path that
reads the mask's depths, byte for byte -- on valid trees and on malformed ones (a parent
out of range, self and two-node cycles, paths longer than max_depth).  The mask outputs
are filled with garbage first: a read of them would show.  The overlapped step that forks
the acceptance before the mask, eager and as replayed graphs, equals the one-stream step.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import compare_accept, require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _accept(w, mask_free, fused=False):
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    print(f"[gpu] mask-free accept={mask_free} {w.name} B={w.B} N={w.N} V={w.V} mode={w.mode} "
          f"max_depth={w.max_depth} fused={fused}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    if fused:
        step.fuse_commit(True)
    if mask_free:
        step.mask_free_accept(True)
        step.mask["depth"].fill_(-3)  # not read
        step.mask["anc_bits"].fill_(-1)
    else:
        step.build_mask()
    step.accept()
    step.kv_commit()
    torch.cuda.synchronize()
    r = dict(acc={k: to_np(v) for k, v in step.acc.items()}, commit={k: to_np(v) for k, v in step.commit.items()},
             k_cache=to_np(dev["k_cache"]), v_cache=to_np(dev["v_cache"]))
    del step, dev
    return r


def _same(a, b):
    for k in a["acc"]:
        assert np.array_equal(a["acc"][k], b["acc"][k]), "acc." + k
    for k in a["commit"]:
        assert np.array_equal(a["commit"][k], b["commit"][k]), "commit." + k
    assert np.array_equal(a["k_cache"], b["k_cache"]) and np.array_equal(a["v_cache"], b["v_cache"])


def _malformed(w):
    """Plant malformed parent arrays in the first sequences (the rest stay valid)."""
    p = w.parents.copy()
    N = p.shape[1]
    p[0, N // 2] = N + 7        # parent out of range (above)
    if w.B > 1:
        p[1, 1] = -5            # parent out of range (below)
    if w.B > 2:
        p[2, N - 1] = N - 1     # self-parent
    if w.B > 3:
        p[3, 1], p[3, 2] = 2, 1  # two-node cycle
    w.parents = p
    return w


CASES = [
    ("cfg2-stochastic", lambda: W.config(2)),
    ("cfg4-stochastic", lambda: W.config(4, B=6, L=161, V=2999)),
    ("cfg5-stochastic", lambda: W.config(5, B=3, L=290, V=1500)),
    ("cfg2-topk", lambda: W.config(2, mode="topk")),
    ("cfg4-topk", lambda: W.config(4, B=6, L=161, V=2999, mode="topk")),
    ("cfg3-greedy", lambda: W.config(3, B=16, L=(16, 90))),
    ("cfg1-greedy", lambda: W.config(1, B=5, plant=[0, 1, 2, 3, 4])),
]


@pytest.mark.parametrize("name", [c[0] for c in CASES])
def test_mask_free_accept_matches_oracle(name):
    w = dict(CASES)[name]()
    got = _accept(w, True)
    ref = oracle.accept(w)
    n_flagged = compare_accept(got["acc"], ref)
    print(f"  accept_len {ref['accept_len'].tolist()[:8]} flagged {n_flagged}")
    _same(got, _accept(w, False))


@pytest.mark.parametrize("cfg,over", [(4, dict(B=6, L=161, V=2999)), (5, dict(B=5, L=290, V=1500)),
                                      (4, dict(B=6, L=161, V=2999, mode="topk")), (3, dict(B=8, L=(16, 90)))])
def test_mask_free_accept_malformed_trees(cfg, over):
    w = _malformed(W.config(cfg, **over))
    if cfg == 5:
        w.max_depth = 4  # the outcome tree reaches depth 10: deeper nodes are invalid
    got = _accept(w, True)
    ref = oracle.accept(w)
    compare_accept(got["acc"], ref)
    _same(got, _accept(w, False))
    assert (got["acc"]["accept_len"] <= w.max_depth).all()


@pytest.mark.parametrize("cfg,over", [(2, {}), (5, dict(B=2, L=290, V=1500)), (3, dict(B=8, L=(16, 90)))])
def test_mask_free_fused_commit(cfg, over):
    """The walker's commit with the depths derived in the kernel equals the commit after the mask."""
    w = W.config(cfg, **over)
    _same(_accept(w, True, fused=True), _accept(w, False, fused=True))


@pytest.mark.parametrize("cfg,over", [(2, {}), (4, dict(B=6, L=161, V=2999))])
def test_mask_free_overlapped_step_and_graph_replays(cfg, over):
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    w = W.config(cfg, **over)
    print(f"[gpu] mask-free step modes: {w.name} B={w.B} N={w.N} V={w.V} mode={w.mode}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    step.run()
    torch.cuda.synchronize()
    names = ["out"] + ["acc." + k for k in step.acc] + ["commit." + k for k in step.commit] + ["mask." + k for k in step.mask]

    def snap():
        ts = [step.out] + list(step.acc.values()) + list(step.commit.values()) + list(step.mask.values())
        r = {k: to_np(t).tobytes() for k, t in zip(names, ts)}
        r["k_cache"], r["v_cache"] = to_np(dev["k_cache"]).tobytes(), to_np(dev["v_cache"]).tobytes()
        return r

    ref = snap()

    def clobber():
        step.out.zero_()
        for v in list(step.acc.values()) + list(step.commit.values()) + list(step.mask.values()):
            v.fill_(-7)
        torch.cuda.synchronize()

    step.fuse_commit(True)
    step.mask_free_accept(True)
    clobber()
    step.run(overlap=True)
    torch.cuda.synchronize()
    bad = [k for k, v in snap().items() if v != ref[k]]
    assert not bad, f"mask-free overlapped step differs in {bad}"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run(overlap=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(overlap=True)
    torch.cuda.synchronize()
    for i in range(4):
        clobber()
        g.replay()
        torch.cuda.synchronize()
        bad = [k for k, v in snap().items() if v != ref[k]]
        assert not bad, f"mask-free graph replay {i} differs in {bad}"
    del g, step, dev
