"""GPU vs oracle parity for draft logits over a vocabulary subset (sv_draft_subset_logits).

Bar: every output entry bit-exact (including the -inf of ids outside the
subset); acceptance on the resulting draft logits bit-exact per draw except
oracle-flagged draws.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import compare_accept, require_gpu, run_step, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _t(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x).cuda()


def _subset_map(seed, V, Vd, junk=0):
    """A seeded subset of Vd target ids (Fisher-Yates order) as t2d [V]; junk entries out of range."""
    ids = np.argsort(W.u64(seed, 1, V))[:Vd]
    t2d = np.zeros(V, np.int32)
    t2d[ids] = np.arange(1, Vd + 1, dtype=np.int32)
    if junk:
        bad = np.argsort(W.u64(seed, 2, V))[:junk]
        t2d[bad] = np.where(np.arange(junk) % 2 == 0, -3, Vd + 5)
    return ids, t2d


@pytest.mark.parametrize("dtype,B,R,V,Vd,junk", [("bf16", 2, 7, 128256, 32000, 0), ("f32", 3, 5, 1001, 77, 40),
                                                 ("bf16", 1, 1, 4099, 4099, 0),
                                                 ("f32", 2, 3, 30011, 20000, 10)])  # 80 KB subset rows: global gather
def test_subset_logits_bitwise(dtype, B, R, V, Vd, junk):
    import torch
    import tree_verification_sv_amd as sv
    print(f"[gpu] draft subset {dtype} B={B} R={R} V={V} Vd={Vd}", flush=True)
    sub = W.normal(V, 3, (B, R, Vd), dtype, 3.0)
    _, t2d = _subset_map(V, V, Vd, junk)
    out = sv.sv_draft_subset_logits(_t(sub), _t(t2d))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out), oracle.draft_subset_logits(sub, t2d))


def test_acceptance_with_a_subset_drafter():
    import torch
    import tree_verification_sv_amd as sv
    w = W.config(4, B=32, L=40, V=3000)
    Vd = 700
    ids, t2d = _subset_map(77, w.V, Vd)
    sub = np.ascontiguousarray(w.draft_logits[:, :, ids])  # the drafter's own logits on its subset
    full = oracle.draft_subset_logits(sub, t2d)
    g = sv.sv_draft_subset_logits(_t(sub), _t(t2d))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(g), full)
    rows = (np.arange(w.B)[:, None] * (w.N + 1) + w.parents + 1).reshape(-1)
    toks = W.draft_tokens(4, 2, full.reshape(-1, w.V), rows, 1.0).reshape(w.B, w.N)
    assert np.isin(toks, ids).all()
    w2 = dataclasses.replace(w, draft_logits=full, tokens=toks)
    r = run_step(w2, stages=("mask", "accept"))
    ref = oracle.accept(w2)
    compare_accept(r["acc"], ref)
    assert ref["accept_len"].sum() > 0
