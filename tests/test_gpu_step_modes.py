"""The step's launch modes on the GPU: the one-stream order, the overlapped order
(acceptance and commit on a side stream beside the attention, joined at the end), and
replays of a captured HIP graph of the overlapped order (the benchmark's mode) must give
identical bytes in every output.  The one-stream step itself is checked against the
oracle in test_gpu_parity.py.
"""
import numpy as np
import pytest

import workloads as W
from gpu_util import require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _snapshot(step, dev):
    r = {"out": to_np(step.out).tobytes(),
         "k_cache": to_np(dev["k_cache"]).tobytes(), "v_cache": to_np(dev["v_cache"]).tobytes()}
    for k, v in step.acc.items():
        r["acc." + k] = to_np(v).tobytes()
    for k, v in step.commit.items():
        r["commit." + k] = to_np(v).tobytes()
    for k, v in step.mask.items():
        r["mask." + k] = to_np(v).tobytes()
    return r


def _diff(a, b):
    return [k for k in a if a[k] != b[k]]


@pytest.mark.parametrize("cfg,over", [(2, {}), (3, dict(B=5, L=(40, 400), V=2500, N=32)), (4, dict(B=6, L=161, V=2999))])
def test_overlapped_step_and_graph_replays(cfg, over):
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    w = W.config(cfg, **over)
    print(f"[gpu] step modes: {w.name} B={w.B} N={w.N} V={w.V} mode={w.mode}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    step.run()
    torch.cuda.synchronize()
    ref = _snapshot(step, dev)

    def clobber():  # eager work between runs: every output overwritten
        step.out.zero_()
        for v in list(step.acc.values()) + list(step.commit.values()):
            v.fill_(-7)
        torch.cuda.synchronize()

    for accept_first in (True, False):
        clobber()
        step.run(overlap=True, accept_first=accept_first)
        torch.cuda.synchronize()
        bad = _diff(_snapshot(step, dev), ref)
        assert not bad, f"overlapped (accept_first={accept_first}) differs in {bad}"

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
        bad = _diff(_snapshot(step, dev), ref)
        assert not bad, f"graph replay {i} differs in {bad}"
    del g, step, dev


@pytest.mark.parametrize("cfg,over", [(2, {}), (3, dict(B=5, L=(40, 400), V=2500, N=32)), (5, dict(B=2, L=290, V=1500))])
def test_fused_commit_overlapped_and_graph_replays(cfg, over):
    """The benchmark's mode: the acceptance kernel commits, the attention runs beside it, the
    step is a replayed graph; every output equals the one-stream step with a separate commit."""
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    w = W.config(cfg, **over)
    print(f"[gpu] fused-commit step modes: {w.name} B={w.B} N={w.N} V={w.V} mode={w.mode}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    step.run()
    torch.cuda.synchronize()
    ref = _snapshot(step, dev)

    def clobber():
        step.out.zero_()
        for v in list(step.acc.values()) + list(step.commit.values()):
            v.fill_(-7)
        torch.cuda.synchronize()

    step.fuse_commit(True)
    for kw in (dict(), dict(overlap=True), dict(overlap=True, attention_side=True)):
        clobber()
        step.run(**kw)
        torch.cuda.synchronize()
        bad = _diff(_snapshot(step, dev), ref)
        assert not bad, f"fused commit {kw} differs in {bad}"
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
        bad = _diff(_snapshot(step, dev), ref)
        assert not bad, f"fused-commit graph replay {i} differs in {bad}"
    del g, step, dev
