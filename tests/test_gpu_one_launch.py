"""The whole verification step in one launch (sv_verify_step) against the oracle and the
four-call step.

Acceptance, commit and mask outputs are integer / byte results of the same arithmetic as the
separate calls, so they must equal those calls' outputs bit for bit (and the oracle's, flagged
stochastic draws excluded).  The attention runs a different tiling (32-key tiles, its own split
plan), so it is held to the oracle at the bf16 tolerance with the relative-L2 and non-vacuity
checks.  Replays of a captured graph of the launch give the same bytes every time, and the
workspace is left zeroed after every call.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check_attention, compare_accept, out_f64, require_gpu, sample_rows, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(w, one, fused=True, mask_outputs=True):
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    print(f"[gpu] one-launch={one} {w.name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} V={w.V} paged={w.paged} "
          f"L=[{int(w.prefix_len.min())},{int(w.prefix_len.max())}] mode={w.mode} fused_commit={fused}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    if fused:
        step.fuse_commit(True)
    if one:
        assert step.one_launch(True, mask_outputs=mask_outputs), "sv_verify_step refused the arguments"
        for v in list(step.acc.values()) + list(step.mask.values()) + list(step.commit.values()):
            v.fill_(-7)
        step.out.fill_(7.0)
    step.run()
    torch.cuda.synchronize()
    r = dict(out=out_f64(step.out), astatus=to_np(step.attn_status),
             acc={k: to_np(v) for k, v in step.acc.items()}, mask={k: to_np(v) for k, v in step.mask.items()},
             commit={k: to_np(v) for k, v in step.commit.items()}, k_cache=to_np(dev["k_cache"]),
             v_cache=to_np(dev["v_cache"]))
    if one:
        r["ws_zero"] = _counters_zero(w, step.step_ws)
    del step, dev
    return r


def _counters_zero(w, ws):
    """The counters of the step's workspace are zero: the acceptance part at its start (exit
    counters, row words, exchange slots) and the attention's
    arrival and exit counters at its end (the split partials between them hold data)."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    B, N = w.B, w.N
    G = max(1, -(-w.V // (512 * 64)))
    NG = (B * (N + 1) + 7) // 8 * 8
    o = up(NG * 4)
    for n in (B * 4, 8, B * (N + 1) * 8, B * 4, B * 4, B * 4, NG * G * 2 * 64):
        o = up(o + n)
    units = B * w.Hkv * -(-(N * (w.Hq // w.Hkv)) // 256)
    tail = up(units * 4) + 256
    return int(ws[:o].sum()) == 0 and int(ws[-tail:].sum()) == 0


def _d64(B=3, N=40, V=4096, L=200, mode="stochastic"):
    par = np.stack([W.tree_random_recursive(41, N, 6, offset=b * N) for b in range(B)])
    return W.build_workload("d64-bf16", B, N, 8, 2, 64, V, "bf16", mode, par, np.full(B, L), max_depth=6, seed=41,
                            logit_sigma=3.0, token_rule="sample")


def _p_eq_q(w):
    """Draft logits equal to the target's: every first child is accepted, so the walks of wide
    trees stop at rows without children (drawn by the walker's work-group)."""
    w.draft_logits = w.target_logits.copy()
    return w


CASES = [
    ("eagle-static-8b", lambda: W.config(2)),
    ("eagle-static-8b-b3-p==q", lambda: _p_eq_q(W.config(2, B=3, L=100, V=12000))),
    ("outcome-tree-8b-small-p==q", lambda: _p_eq_q(W.config(5, B=2, L=300, V=2048))),
    ("eagle-static-8b-topk", lambda: W.config(2, mode="topk")),
    ("eagle-static-8b-b3-short", lambda: W.config(2, B=3, L=100, V=12000)),
    ("batched-paged-70b-small", lambda: W.config(3, B=6, L=(16, 300), V=8192)),
    ("chain-8b-small", lambda: W.config(4, B=5, L=300, V=4096)),
    ("outcome-tree-8b-small", lambda: W.config(5, B=2, L=300, V=2048)),
    ("d64", lambda: _d64()),
]


@pytest.mark.parametrize("name", [c[0] for c in CASES])
def test_one_launch_matches_oracle_and_separate_calls(name):
    w = dict(CASES)[name]()
    one = _run(w, True)
    sep = _run(w, False)
    assert one["ws_zero"], "the workspace is left zeroed"
    # acceptance: oracle (flagged excluded) and the separate calls, bit for bit
    ref = oracle.accept(w)
    n_flag = compare_accept(one["acc"], ref)
    for k in one["acc"]:
        assert np.array_equal(one["acc"][k], sep["acc"][k]), "acc." + k
    for k in one["commit"]:
        assert np.array_equal(one["commit"][k], sep["commit"][k]), "commit." + k
    assert np.array_equal(one["k_cache"], sep["k_cache"]) and np.array_equal(one["v_cache"], sep["v_cache"])
    for k in one["mask"]:
        assert np.array_equal(one["mask"][k], sep["mask"][k]), "mask." + k
    assert np.array_equal(one["astatus"], sep["astatus"])
    # attention: the oracle at the bf16 tolerance (all rows when small, a seeded sample otherwise)
    total = w.B * w.N * w.Hq
    sel = None if total * int(w.prefix_len.max()) <= 4096 * 60 * 32 else sample_rows(w, 400)
    ref_o = oracle.tree_attention(w, sel=sel)
    got = one["out"].reshape(-1, w.D)[sel] if sel is not None else one["out"]
    err, rel = check_attention(got.reshape(ref_o.shape), ref_o, w.dtype, name)
    print(f"  accept_len {ref['accept_len'].tolist()[:6]} flagged {n_flag} attention max-abs {err:.2e} rel-L2 {rel:.2e}")


def test_one_launch_malformed_trees():
    """Invalid nodes (parent out of range, cycles, too deep) see only themselves in the attention
    and are unusable in the acceptance -- the rule of sv_build_tree_mask, derived in the launch."""
    w = W.config(2, B=4, L=120, V=12000)
    p = w.parents.copy()
    N = w.N
    p[0, N // 2] = N + 3
    p[1, 3] = 3
    p[2, 5], p[2, 6] = 6, 5
    p[3, 1] = -4
    w.parents = p
    one = _run(w, True)
    sep = _run(w, False)
    for k in one["acc"]:
        assert np.array_equal(one["acc"][k], sep["acc"][k]), "acc." + k
    for k in one["mask"]:
        assert np.array_equal(one["mask"][k], sep["mask"][k]), "mask." + k
    compare_accept(one["acc"], oracle.accept(w))
    check_attention(one["out"], oracle.tree_attention(w), "bf16", "malformed")


def test_one_launch_without_mask_outputs_and_separate_commit():
    w = W.config(3, B=4, L=(16, 200), V=8192)
    one = _run(w, True, fused=False, mask_outputs=False)
    sep = _run(w, False, fused=False)
    for k in one["acc"]:
        assert np.array_equal(one["acc"][k], sep["acc"][k]), "acc." + k
    for k in one["commit"]:
        assert np.array_equal(one["commit"][k], sep["commit"][k]), "commit." + k
    assert np.array_equal(one["k_cache"], sep["k_cache"])


@pytest.mark.parametrize("cfg,over", [(2, {}), (5, dict(B=2, L=300, V=2048))])
def test_one_launch_graph_replays(cfg, over):
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    w = W.config(cfg, **over)
    print(f"[gpu] one-launch graph replays {w.name} B={w.B} N={w.N} V={w.V}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    step.fuse_commit(True)
    assert step.one_launch(True)
    step.run()
    torch.cuda.synchronize()
    outs = [step.out] + list(step.acc.values()) + list(step.commit.values()) + list(step.mask.values())

    def snap():
        r = [to_np(t).tobytes() for t in outs]
        return r + [to_np(dev["k_cache"]).tobytes(), to_np(dev["v_cache"]).tobytes()]

    ref = snap()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()
    for i in range(4):
        for t in outs:
            t.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert snap() == ref, f"graph replay {i} differs"
        assert _counters_zero(w, step.step_ws)
    del g, step, dev


def test_one_launch_refuses_unsupported_arguments():
    import torch
    import tree_verification_sv_amd as sv
    from tree_verification_sv_amd.step import VerifyStep
    w = W.config(2, B=1, L=64, V=5003)  # rows not on 16 bytes
    dev = W.to_device(w, "cuda:0")
    assert not VerifyStep(W.step_inputs(w, dev)).one_launch(True)
    w = W.config(1)  # fp32 attention and logits
    dev = W.to_device(w, "cuda:0")
    assert not VerifyStep(W.step_inputs(w, dev)).one_launch(True)
    w = W.with_tree_in_cache(W.config(2, B=1, L=64, V=4096))
    dev = W.to_device(w, "cuda:0")
    s = VerifyStep(W.step_inputs(w, dev))
    s._acc.commit = ctypes.addressof(s._com)  # a commit that would move rows the attention reads
    a = sv.sv_step_args()
    a.attn, a.accept = ctypes.addressof(s._attn), ctypes.addressof(s._acc)
    a.workspace, a.workspace_bytes = 256, 1 << 20
    assert sv.lib().sv_verify_step(ctypes.byref(a), None) == sv.SV_ERR_UNSUPPORTED
    torch.cuda.synchronize()
