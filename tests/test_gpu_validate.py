"""Reference mode (SV_FLAG_VALIDATE), non-finite logits, the acceptance's bounded wait, and the
512-thread acceptance row groups on fp32 rows whose length is not a multiple of 16 bytes.

* Golden tree-mask cases on the GPU: bit-exact with the hand-derived values, and in reference
  mode the call raises SV_ERR_BAD_TREE exactly when a sequence is malformed.
* Non-finite rows: a NaN / +Inf logit or a row without a finite entry in a row the stochastic
  or top-K walk uses stops the walk there with status 8; -Inf entries alone are probability 0
  and the outputs still equal the oracle's.  Reference mode finds non-finite rows the greedy
  walk never reads.
* The timeout word of the acceptance workspace set from the host before a call: every
  sequence reports status 7, the kernel exits, and the next call equals the oracle again.
"""
import ctypes
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import compare_accept, require_gpu, run_step, to_np

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tree_mask_cases.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_golden_mask_cases_on_gpu_and_reference_mode():
    import torch
    import tree_verification_sv_amd as sv
    cases = json.load(open(GOLDEN))["cases"]
    for i, c in enumerate(cases):
        print(f"[gpu] golden mask case {i} parents={c['parents']} max_depth={c['max_depth']}", flush=True)
        par = torch.tensor([c["parents"]], dtype=torch.int32, device="cuda:0")
        m = sv.sv_build_tree_mask(par, c["max_depth"])
        torch.cuda.synchronize()
        assert to_np(m["anc_bits"]).view(np.uint64)[0, :, 0].tolist() == c["anc"]
        assert to_np(m["depth"])[0].tolist() == c["depth"]
        assert to_np(m["path_rows"])[0].tolist() == c["path_rows"]
        assert int(to_np(m["status"])[0]) == c["status"]
        if c["status"] == 0:
            sv.sv_build_tree_mask(par, c["max_depth"], out=m, validate=True)
        else:
            with pytest.raises(sv.SpecVerifyError, match="returned 3"):
                sv.sv_build_tree_mask(par, c["max_depth"], out=m, validate=True)
        assert int(to_np(m["status"])[0]) == c["status"]


def _accept(w, validate=False):
    import torch
    import tree_verification_sv_amd as sv
    d = W.to_device(w, "cuda:0")
    m = sv.sv_build_tree_mask(d["parents"], w.max_depth)
    kw = dict(draft_logits=d["draft_logits"], u_accept=d["u_accept"], u_sample=d["u_sample"],
              temperature=w.temperature)
    err = None
    try:
        o = sv.sv_accept(d["parents"], d["tokens"], m["anc_bits"], m["depth"], d["target_logits"], w.max_depth,
                         w.mode, validate=validate, **kw)
    except sv.SpecVerifyError as e:  # reference mode: outputs are still written before the raise
        err = e
        o = None
    torch.cuda.synchronize()
    return ({k: to_np(v) for k, v in o.items()} if o is not None else None), err


def _set(arr, b, r, v, value):
    """Set logits[b, r, v] (bf16 bit pattern or fp32) to a float value."""
    if arr.dtype == np.uint16:
        arr[b, r, v] = W.f32_to_bf16(np.array([value], np.float32))[0]
    else:
        arr[b, r, v] = np.float32(value)


@pytest.mark.parametrize("mode", ["stochastic", "topk"])
def test_nonfinite_rows_stop_the_walk(mode):
    w = W.config(2, B=5, L=64, V=5003, mode=mode)
    tl = w.target_logits.copy()
    _set(tl, 0, 0, 17, np.nan)                 # root row: NaN
    _set(tl, 1, 0, 4000, np.inf)               # root row: +Inf
    tl[2, 0, :] = W.f32_to_bf16(np.full(w.V, -np.inf, np.float32))  # root row: no finite entry
    for v in range(0, w.V, 7):                 # sequence 3: -Inf entries only (probability 0, valid)
        _set(tl, 3, 0, v, -np.inf)
    w.target_logits = tl
    got, _ = _accept(w)
    st = got["status"]
    assert st[:3].tolist() == [8, 8, 8], st
    assert got["stop_row"][:3].tolist() == [0, 0, 0] and got["accept_len"][:3].tolist() == [0, 0, 0]
    assert got["out_tokens"][:3, 0].tolist() == [0, 0, 0]
    # the valid sequences (3 with -Inf entries, 4 untouched) equal the oracle on the same inputs
    ref = oracle.accept(w)
    keep = np.array([3, 4])
    sub = {k: v[keep] for k, v in got.items()}
    rsub = {k: (v[keep] if isinstance(v, np.ndarray) and v.shape[:1] == (w.B,) else v) for k, v in ref.items()}
    compare_accept(sub, rsub)
    assert st[3:].tolist() == [0, 0]


def test_nonfinite_draft_row_stochastic():
    w = W.config(2, B=2, L=64, V=5003)
    dl = w.draft_logits.copy()
    _set(dl, 0, 0, 9, np.nan)
    w.draft_logits = dl
    got, _ = _accept(w)
    assert int(got["status"][0]) == 8 and int(got["status"][1]) == 0


def test_reference_mode_scans_rows_greedy_never_reads():
    """Greedy reads the root and the rows with children only: a NaN in a leaf's row goes unseen
    in performance mode and is reported by reference mode (status 8, SV_ERR_BAD_TREE)."""
    w = W.config(3, B=4, L=(16, 80), V=3001)
    par = w.parents[1]
    leaves = [i for i in range(w.N) if not (par == i).any()]
    tl = w.target_logits.copy()
    _set(tl, 1, leaves[0] + 1, 11, np.nan)
    w.target_logits = tl
    got, err = _accept(w, validate=False)
    assert err is None
    ref = oracle.accept(w)
    compare_accept(got, ref, allow_flagged=False)
    got2, err = _accept(w, validate=True)
    assert err is not None and "returned 3" in str(err)
    import torch
    import tree_verification_sv_amd as sv
    d = W.to_device(w, "cuda:0")
    m = sv.sv_build_tree_mask(d["parents"], w.max_depth)
    outs = sv.accept_outputs(w.B, w.max_depth, "cuda:0")
    with pytest.raises(sv.SpecVerifyError):
        sv.sv_accept(d["parents"], d["tokens"], m["anc_bits"], m["depth"], d["target_logits"], w.max_depth, "greedy",
                     outs=outs, validate=True)
    torch.cuda.synchronize()
    assert to_np(outs["status"]).tolist() == [0, 8, 0, 0]


def _ws_err_offset(B, N):
    """Byte offset of the acceptance workspace's timeout word (layout of sv_accept_workspace for
    modes 0-2: group exit counters, per-sequence counters, then the timeout word)."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    NG = (B * (N + 1) + 7) // 8 * 8
    return up(up(NG * 4) + B * 4)


@pytest.mark.parametrize("cfg,over", [(2, dict(B=2, L=64, V=5003)), (3, dict(B=4, L=(16, 80), V=3001)),
                                      (3, dict(B=16, L=(16, 80))), (3, dict(B=8, N=80, L=(16, 80), V=40000)),
                                      (4, dict(B=6, L=64, V=2999))])
def test_timeout_word_reports_status_7_then_recovers(cfg, over):
    """A timeout word set before the call: every sequence reports status 7, the workspace is left
    zeroed, and the next call matches the oracle (row groups with exchanges; greedy chains of two
    work-groups per sequence; the greedy row list)."""
    import torch
    import tree_verification_sv_amd as sv
    from tree_verification_sv_amd.step import VerifyStep
    w = W.config(cfg, **over)
    print(f"[gpu] forced timeout {w.name} B={w.B} N={w.N} V={w.V} mode={w.mode}", flush=True)
    d = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, d))
    step.build_mask()
    off = _ws_err_offset(w.B, w.N)
    assert off + 8 <= step.acc_ws.numel()
    step.acc_ws[off:off + 4].copy_(torch.tensor([1, 0, 0, 0], dtype=torch.uint8))  # timeout word = 1
    step.accept()
    torch.cuda.synchronize()
    assert to_np(step.acc["status"]).tolist() == [7] * w.B
    assert int(step.acc_ws.sum()) == 0, "the workspace is left zeroed"
    step.accept()
    torch.cuda.synchronize()
    ref = oracle.accept(w)
    compare_accept({k: to_np(v) for k, v in step.acc.items()}, ref)


def _outcome_f32(mode, B=8):
    """Outcome trees of 256 nodes at batch 8 (2056 rows: the 512-thread row groups) with fp32
    logits over a 1499-entry vocabulary (rows not on 16 bytes: the unaligned load path)."""
    par = np.stack([W.tree_outcome(31, offset=b * 1000) for b in range(B)])
    return W.build_workload("outcome-f32", B, par.shape[1], 8, 2, 64, 1499, "f32", mode, par, np.full(B, 32),
                            max_depth=10, seed=31, logit_sigma=3.0, target_from_draft_sigma=1.0,
                            token_rule="topk" if mode == "topk" else "sample")


@pytest.mark.parametrize("mode", ["stochastic", "topk"])
def test_wide_rows_fp32_ragged_mask_free_malformed_fused(mode):
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    for variant in ("plain", "malformed"):
        w = _outcome_f32(mode)
        assert w.B * (w.N + 1) >= 2048 and w.N >= 128
        if variant == "malformed":
            p = w.parents.copy()
            p[0, 100] = w.N + 3
            p[1, 5] = 5
            p[2, 1], p[2, 2] = 2, 1
            w.parents = p
        ref = oracle.accept(w)
        outs = []
        for mask_free, fused in ((False, False), (True, False), (True, True)):
            print(f"[gpu] wide fp32 {mode} {variant} mask_free={mask_free} fused={fused}", flush=True)
            d = W.to_device(w, "cuda:0")
            step = VerifyStep(W.step_inputs(w, d))
            if fused:
                step.fuse_commit(True)
            if mask_free:
                step.mask_free_accept(True)
                step.mask["depth"].fill_(-3)
            else:
                step.build_mask()
            step.accept()
            step.kv_commit()
            torch.cuda.synchronize()
            acc = {k: to_np(v) for k, v in step.acc.items()}
            compare_accept(acc, ref)
            outs.append((acc, {k: to_np(v) for k, v in step.commit.items()}, to_np(d["k_cache"]), to_np(d["v_cache"])))
            del step, d
        for o in outs[1:]:
            for k in o[0]:
                assert np.array_equal(o[0][k], outs[0][0][k]), k
            for k in o[1]:
                assert np.array_equal(o[1][k], outs[0][1][k]), k
            assert np.array_equal(o[2], outs[0][2]) and np.array_equal(o[3], outs[0][3])
