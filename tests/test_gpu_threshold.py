"""GPU vs oracle parity for threshold acceptance (sv_accept mode SV_THRESHOLD).

Bar: accepted lengths, rows, tokens, stop rows and statuses bit-exact; path
scores within a relative 1e-5 of the threshold are flagged by the oracle and
excluded (their count is printed).  Thresholds and temperatures are rounded to
fp32 before the oracle sees them, as the library receives them.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _util import golden
from gpu_util import compare_accept, require_gpu, to_np

pytestmark = pytest.mark.gpu

SMALL = {
    2: dict(L=64, V=3001),
    3: dict(B=5, L=(40, 100), V=2500, N=32),
    4: dict(B=6, L=32, V=2999),
    5: dict(B=2, L=64, V=1500),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _f32(x):
    return float(np.float32(x))


def _gpu_threshold(w, tau, T, tokens=None, workspace=None, row_list=False):
    import torch
    import tree_verification_sv_amd as sv
    dev = W.to_device(w, "cuda:0")
    tok = dev["tokens"] if tokens is None else torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda()
    m = sv.sv_build_tree_mask(dev["parents"], w.max_depth)
    out = sv.sv_accept(dev["parents"], tok, m["anc_bits"], m["depth"], dev["target_logits"], w.max_depth,
                       mode="threshold", temperature=T, threshold=tau, workspace=workspace, row_list=row_list)
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in out.items()}


def _check(w, tau, T, tokens=None, row_list=False):
    tau, T = _f32(tau), _f32(T)
    print(f"[gpu] threshold {w.name} B={w.B} N={w.N} V={w.V} tau={tau:.3g} T={T:.3g} row_list={row_list}", flush=True)
    got = _gpu_threshold(w, tau, T, tokens, row_list=row_list)
    ref = oracle.accept(w, mode="threshold", temperature=T, threshold=tau, tokens=tokens)
    nflag = compare_accept(got, ref)
    print(f"  accept_len {got['accept_len'].tolist()[:16]} flagged {nflag}")
    return got, ref


@pytest.mark.parametrize("idx", range(len(golden("threshold_cases.json")["cases"])))
def test_golden_on_gpu(idx):
    from _util import ns
    c = golden("threshold_cases.json")["cases"][idx]
    target = np.asarray(c["target"], np.float32)[None]
    w = ns(B=1, N=len(c["parents"]), V=target.shape[-1], max_depth=c["max_depth"],
           parents=np.asarray([c["parents"]], np.int32), tokens=np.asarray([c["tokens"]], np.int32),
           target_logits=target, name="golden", q=None, k_cache=None, v_cache=None, k_tree=None, v_tree=None,
           prefix_len=np.zeros(1, np.int32), tree_in_cache=False)
    got = _gpu_threshold(w, c["threshold"], c["temperature"])
    assert got["accept_len"][0] == c["accept_len"], c["note"]
    assert got["accept_rows"][0].tolist() == c["accept_rows"], c["note"]
    assert got["out_tokens"][0].tolist() == c["out_tokens"], c["note"]
    assert got["stop_row"][0] == c["stop_row"] and got["status"][0] == c.get("status", 0)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_threshold_small(cfg):
    w = W.config(cfg, **SMALL[cfg])
    total = 0
    for tau in (1e-9, 1e-6, 1e-4, 1e-2, 0.3):
        got, _ = _check(w, tau, 1.0)
        total += int(got["accept_len"].sum())
    assert total > 0


@pytest.mark.parametrize("cfg", [2, 3])
def test_threshold_full_size(cfg):
    """Full size: batched-paged-70b follows the passing paths (chains); with SV_FLAG_ROW_LIST, and
    at eagle-static-8b, every needed row's statistics and one walk per sequence."""
    w = W.config(cfg)
    for tau in (1e-7, 1e-3):
        for row_list in (False, True):
            _check(w, tau, 1.0, row_list=row_list)


@pytest.mark.parametrize("over", [dict(B=24, N=40), dict(B=16, N=32, V=100000), dict(B=8, N=120)])
def test_threshold_chains(over):
    """Threshold chains (rows of many bytes): groups of up to eight work-groups per sequence follow
    the passing paths; several thresholds and a temperature, against the oracle."""
    w = W.config(3, L=(16, 80), **over)
    for T in (1.0, 0.7):
        for tau in (1e-6, 1e-3, 0.05):
            _check(w, tau, T)


def test_threshold_chains_fp32():
    """fp32 logits through the threshold chains (rows on 16 bytes, several slices per member)."""
    par = np.stack([W.tree_random_recursive(5, 20, 6, offset=b * 20) for b in range(32)])
    w = W.build_workload("fp32-thr", 32, 20, 4, 2, 64, 40000, "f32", "greedy", par, np.full(32, 8), max_depth=6,
                         seed=5, logit_sigma=1.0, token_rule="uniform", plant=W.plant_pairs(5, par), need_draft=False)
    for tau in (1e-6, 1e-3):
        _check(w, tau, 1.0)


def test_threshold_fp32_ragged_vocab_and_temperature():
    """fp32 logits whose rows are not 16-byte aligned (V = 1001), two temperatures."""
    par = np.stack([W.tree_random_recursive(3, 40, 6, offset=b * 40) for b in range(4)])
    w = W.build_workload("fp32-ragged", 4, 40, 4, 2, 64, 1001, "f32", "greedy", par, np.full(4, 8), max_depth=6,
                         seed=3, logit_sigma=1.0, token_rule="uniform", plant=W.plant_pairs(3, par), need_draft=False)
    for T in (0.5, 2.0):
        for tau in (1e-6, 1e-3, 0.05):
            _check(w, tau, T)


def test_threshold_cold_limit_matches_greedy_on_gpu():
    """T -> 0 with a threshold of 1/2 gives greedy acceptance (fp32 logits, planted matches)."""
    import torch
    from gpu_util import run_step
    par = np.stack([W.tree_random_recursive(8, 20, 6, offset=b * 20) for b in range(8)])
    w = W.build_workload("fp32-tree", 8, 20, 4, 2, 64, 500, "f32", "greedy", par, np.full(8, 16), max_depth=6,
                         seed=8, logit_sigma=3.0, token_rule="uniform", plant=W.plant_pairs(8, par), need_draft=False)
    g = run_step(w, stages=("mask", "accept"))["acc"]
    t, _ = _check(w, 0.5, 1e-4)
    for k in ("accept_len", "accept_rows", "out_tokens", "stop_row"):
        np.testing.assert_array_equal(t[k], g[k], err_msg=k)
    del torch


def test_threshold_bad_tokens_and_workspace_reuse():
    """Out-of-range tokens give status 4; a workspace used by threshold calls then serves a stochastic call."""
    import torch
    import tree_verification_sv_amd as sv
    w = W.config(2, L=64, V=3001)
    tok = w.tokens.copy()
    tok[0, 5] = w.V + 3
    tok[0, 17] = -1
    _check(w, 1e-6, 1.0, tokens=tok)
    dev = W.to_device(w, "cuda:0")
    m = sv.sv_build_tree_mask(dev["parents"], w.max_depth)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda:0")
    for tau in (1e-6, 1e-3):
        sv.sv_accept(dev["parents"], dev["tokens"], m["anc_bits"], m["depth"], dev["target_logits"], w.max_depth,
                     mode="threshold", temperature=1.0, threshold=tau, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0  # every call leaves the workspace zeroed
    out = sv.sv_accept(dev["parents"], dev["tokens"], m["anc_bits"], m["depth"], dev["target_logits"], w.max_depth,
                       mode="stochastic", draft_logits=dev["draft_logits"], u_accept=dev["u_accept"],
                       u_sample=dev["u_sample"], temperature=1.0, workspace=ws)
    torch.cuda.synchronize()
    compare_accept({k: to_np(v) for k, v in out.items()}, oracle.accept(w))
