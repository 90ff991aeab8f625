"""sv_accept_noalloc (library-owned workspace) against sv_accept (caller workspace), through the
C ABI: the same outputs, bit for bit, on two calls in a row -- the second on a smaller input -- in
every acceptance mode, plus the size limit and the argument errors."""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _run_pair(w, Dm=None):
    """Outputs of sv_accept (own workspace) and sv_accept_noalloc on the same inputs."""
    import torch
    import tree_verification_sv_amd as sv
    from tests.gpu_util import require_gpu, to_np
    dev = require_gpu()
    d = W.to_device(w, dev)
    mask = sv.sv_build_tree_mask(d["parents"], w.max_depth)
    outs = []
    for fn in ("sv_accept", "sv_accept_noalloc"):
        o = sv.accept_outputs(w.B, w.max_depth, dev)
        for v in o.values():
            v.fill_(-7)  # every output is written by the call
        a = sv.accept_args(d["parents"], d["tokens"], mask["anc_bits"], mask["depth"], d["target_logits"], w.max_depth,
                           w.mode, d.get("draft_logits"), d.get("u_accept"), d.get("u_sample"), w.temperature, o,
                           getattr(w, "threshold", 0.0))
        ws = None
        if fn == "sv_accept":
            need = sv.sv_accept_workspace(a)
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            a.workspace, a.workspace_bytes = ws.data_ptr(), need
        else:
            a.workspace, a.workspace_bytes = None, 0  # ignored by the no-allocation entry point
        rc = getattr(sv.lib(), fn)(ctypes.byref(a), sv._stream(None))
        assert rc == sv.SV_OK, f"{fn} returned {rc}"
        torch.cuda.synchronize()
        outs.append({k: to_np(v) for k, v in o.items()})
        del ws
    return outs


CASES = [
    # (config, overrides, mode) -- second of each pair is smaller
    (2, dict(B=3, L=64, V=20011), "stochastic"),
    (2, dict(B=1, L=64, V=5003), "stochastic"),
    (3, dict(B=6, L=(16, 80), V=9001), "greedy"),
    (3, dict(B=2, L=(16, 40), V=3001), "greedy"),
    (2, dict(B=2, L=64, V=12000, mode="topk"), "topk"),
    (2, dict(B=1, L=64, V=4000, mode="topk"), "topk"),
    (3, dict(B=16, N=32, L=(16, 80), V=100000), "greedy"),  # path chains (rows of many bytes)
    (3, dict(B=2, L=(16, 40), V=3001), "greedy"),
    (3, dict(B=8, N=80, L=(16, 80), V=40000), "greedy"),  # the row list (512 rows or more)
    (3, dict(B=3, L=(16, 40), V=5001), "greedy"),
]


@pytest.mark.parametrize("pair", [(0, 1), (2, 3), (4, 5), (6, 7), (8, 9)])
def test_noalloc_equals_sv_accept_twice(pair):
    for k in pair:  # two calls in a row, the second with the smaller input
        cfg, ov, mode = CASES[k]
        w = W.config(cfg, **ov)
        print(f"[noalloc] config {cfg} {ov} mode {w.mode} B={w.B} N={w.N} V={w.V}", flush=True)
        ref, got = _run_pair(w)
        for key in ref:
            assert np.array_equal(ref[key], got[key]), (key, ref[key][:2], got[key][:2])
            assert (got[key] != -7).all() or key in ("accept_rows",), key
        o = oracle.accept(w)
        ok = o["flagged"] == 0
        for key in ("accept_len", "accept_rows", "out_tokens", "num_out", "stop_row"):
            assert np.array_equal(got[key][ok], o[key][ok]), key


def test_noalloc_threshold_mode():
    # path chains (rows of many bytes), then the two-launch form on smaller inputs
    for ov in (dict(B=16, N=32, L=(16, 80), V=100000), dict(B=4, L=(16, 80), V=9001), dict(B=2, L=(16, 40), V=3001)):
        w = W.config(3, **ov)
        w.mode = "threshold"
        w.threshold = float(np.float32(1e-3))
        ref, got = _run_pair(w)
        for key in ref:
            assert np.array_equal(ref[key], got[key]), key


def test_noalloc_rejects_oversized_and_bad_arguments():
    import torch
    import tree_verification_sv_amd as sv
    from tests.gpu_util import require_gpu
    dev = require_gpu()
    w = W.config(2, B=1, L=64, V=4000)
    d = W.to_device(w, dev)
    mask = sv.sv_build_tree_mask(d["parents"], w.max_depth)
    o = sv.accept_outputs(w.B, w.max_depth, dev)
    a = sv.accept_args(d["parents"], d["tokens"], mask["anc_bits"], mask["depth"], d["target_logits"], w.max_depth,
                       w.mode, d["draft_logits"], d["u_accept"], d["u_sample"], w.temperature, o)
    big = sv.sv_accept_args.from_buffer_copy(a)
    big.B = 4096  # workspace of 4096 sequences of 61 rows is far above the 4 MiB array
    assert sv.sv_accept_workspace(big) > sv.SV_ACCEPT_SCRATCH_BYTES
    assert sv.lib().sv_accept_noalloc(ctypes.byref(big), sv._stream(None)) == sv.SV_ERR_SCRATCH_LIMIT
    bad = sv.sv_accept_args.from_buffer_copy(a)
    bad.mode = 9
    assert sv.lib().sv_accept_noalloc(ctypes.byref(bad), sv._stream(None)) == sv.SV_ERR_INVALID_ARGUMENT
    assert sv.lib().sv_accept_noalloc(None, sv._stream(None)) == sv.SV_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
