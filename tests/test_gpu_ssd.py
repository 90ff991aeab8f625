"""GPU vs oracle parity for the SSD outcome lookup and the Saguaro reweighting.

Bar: bit-exact hit flags, branches, gathered tokens, hit counts and reweighted
logits; acceptance on reweighted drafts bit-exact except oracle-flagged draws.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import compare_accept, require_gpu, run_step, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _t(x, dtype=np.int32):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x.astype(dtype) if x.dtype != dtype else x).cuda()


def _lookup_both(stop_row, out_tokens, num_out, key_row, key_token, n_keys, prepared=None):
    import torch
    import tree_verification_sv_amd as sv
    print(f"[gpu] outcome lookup B={len(stop_row)} K={np.shape(key_row)[1]}", flush=True)
    g = sv.sv_outcome_lookup(_t(stop_row), _t(out_tokens), _t(num_out), _t(key_row), _t(key_token), _t(n_keys),
                             None if prepared is None else _t(prepared))
    torch.cuda.synchronize()
    r = oracle.outcome_lookup(stop_row, out_tokens, num_out, key_row, key_token, n_keys, prepared)
    for k in ("hit", "branch", "n_hits") + (("next_tokens",) if prepared is not None else ()):
        np.testing.assert_array_equal(to_np(g[k]), r[k], err_msg=k)
    return r


def test_lookup_hand_cases_on_gpu():
    r = _lookup_both(np.array([2, 0, 1, 3]), np.array([[4, 7, 0, 0], [5, 0, 0, 0], [9, 9, 0, 0], [1, 1, 1, 8]]),
                     np.array([2, 1, 2, 4]), np.array([[1, 2, 2], [0, 0, 0], [1, 0, 0], [3, 3, 2]]),
                     np.array([[7, 7, 7], [4, 6, 3], [9, 0, 0], [8, 8, 8]]), np.array([3, 3, 0, 1]),
                     np.arange(24, dtype=np.int32).reshape(4, 3, 2) + 100)
    assert r["branch"].tolist() == [2, 0, 0, 1]


@pytest.mark.parametrize("B,K,P", [(1, 1, 0), (300, 8, 5), (4099, 16, 12)])
def test_lookup_random_tables(B, K, P):
    """Seeded random outcomes and tables with planted hits, duplicates, short tables and bad num_out."""
    Dm = 6
    seed = B + K
    stop_row = W.randint(seed, 1, B, 0, 20)
    num_out = W.randint(seed, 2, B, 0, Dm + 2)  # 0 and Dm + 2 are out of range: misses
    out_tokens = W.randint(seed, 3, B * (Dm + 1), 0, 9).reshape(B, Dm + 1)
    key_row = W.randint(seed, 4, B * K, 0, 20).reshape(B, K)
    key_token = W.randint(seed, 5, B * K, 0, 9).reshape(B, K)
    n_keys = W.randint(seed, 6, B, -1, K + 2)
    plant = W.randint(seed, 7, B, 0, 2 * K - 1)  # about half the sequences get their outcome planted
    for b in range(B):
        k = int(plant[b])
        if k < K and 1 <= num_out[b] <= Dm + 1:
            key_row[b, k] = stop_row[b]
            key_token[b, k] = out_tokens[b, num_out[b] - 1]
    prepared = W.randint(seed, 8, B * K * P, 0, 1000).reshape(B, K, P) if P else None
    r = _lookup_both(stop_row, out_tokens, num_out, key_row, key_token, n_keys, prepared)
    if B > 1:
        assert 0 < r["n_hits"][0] < B


@pytest.mark.parametrize("cfg", [2, 4])
def test_lookup_closed_loop_after_gpu_acceptance(cfg):
    """Tables from the oracle's outcomes (planted among decoys); the lookup runs on the GPU's own
    acceptance outputs and must find every planted outcome."""
    w = W.config(cfg, B=(32 if cfg == 4 else 2), L=40, V=2000)
    r = run_step(w, stages=("mask", "accept"))
    acc = oracle.accept(w)
    compare_accept(r["acc"], acc)
    ok = acc["flagged"] == 0
    B, K = w.B, 6
    bonus = acc["out_tokens"][np.arange(B), acc["num_out"] - 1]
    where = W.randint(cfg, 9, B, 0, K - 1)
    key_row = (acc["stop_row"][:, None] + 1 + np.arange(K)[None]) % (w.N + 1)
    key_token = np.tile(bonus[:, None], (1, K))
    key_row[np.arange(B), where] = acc["stop_row"]
    key_token[np.arange(B), where] = bonus
    g = r["acc"]
    ref = _lookup_both(g["stop_row"], g["out_tokens"], g["num_out"], key_row, key_token, np.full(B, K))
    assert (ref["hit"][ok] == 1).all() and np.array_equal(ref["branch"][ok], where[ok] + 1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reweight_bitwise(dtype):
    import torch
    import tree_verification_sv_amd as sv
    B, R, V, C = 5, 9, 3001, 7
    l = W.normal(11, 1, (B, R, V), dtype, 3.0)
    ct = W.randint(11, 2, B * R * C, -3, V + 3).reshape(B, R, C)
    ct[:, :, 3] = ct[:, :, 1]  # repeats count once
    shift = float(np.float32(np.log(0.25)))
    print(f"[gpu] saguaro reweight {dtype} B={B} R={R} V={V} C={C}", flush=True)
    d = _t(l) if dtype == "bf16" else _t(l, np.float32)
    sv.sv_saguaro_reweight(d, _t(ct), shift)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(d), oracle.saguaro_reweight(l, ct, shift))


def test_acceptance_on_reweighted_drafts():
    """Stochastic acceptance with Saguaro-reweighted drafts (tokens drawn from the reweighted rows)."""
    import dataclasses
    import torch
    import tree_verification_sv_amd as sv
    w = W.config(4, B=24, L=40, V=2000)
    C = 4
    ct = np.stack([np.argsort(-W.bf16_to_f32(w.target_logits[b]), axis=-1)[:, :C] for b in range(w.B)])
    shift = float(np.float32(np.log(0.3)))
    qw = oracle.saguaro_reweight(w.draft_logits, ct, shift)
    d = _t(w.draft_logits)
    sv.sv_saguaro_reweight(d, _t(ct), shift)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(d), qw)
    rows = (np.arange(w.B)[:, None] * (w.N + 1) + w.parents + 1).reshape(-1)
    toks = W.draft_tokens(4, 2, qw.reshape(-1, w.V), rows, 1.0).reshape(w.B, w.N)
    w2 = dataclasses.replace(w, draft_logits=qw, tokens=toks)
    r = run_step(w2, stages=("mask", "accept"))
    compare_accept(r["acc"], oracle.accept(w2))
