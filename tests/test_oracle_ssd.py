"""Pins for the oracle's SSD outcome lookup and Saguaro reweighting.

Definitions: 'Speculative Speculative Decoding' (gist.science summary), sec. 2:
the drafter prepares speculations for the likely outcomes of verification (how
many tokens are accepted and which bonus token is drawn); when verification
ends the real outcome hits that cache (the prepared tokens go straight to the
verifier) or misses (a fallback runs).  Sec. 3B: Saguaro sampling lowers the
draft probability of the tokens already in the cache, which raises the residual
mass on them, so the bonus token is more likely to be a cached one, while the
output distribution stays exact.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import workloads as W
from _util import ns


def test_lookup_hand_cases():
    Dm = 3
    stop_row = np.array([2, 0, 1, 3])
    out_tokens = np.array([[4, 7, 0, 0], [5, 0, 0, 0], [9, 9, 0, 0], [1, 1, 1, 8]])
    num_out = np.array([2, 1, 2, 4])
    key_row = np.array([[1, 2, 2], [0, 0, 0], [1, 0, 0], [3, 3, 2]])
    key_token = np.array([[7, 7, 7], [4, 6, 3], [9, 0, 0], [8, 8, 8]])
    n_keys = np.array([3, 3, 0, 1])
    prepared = np.arange(4 * 3 * 2, dtype=np.int32).reshape(4, 3, 2) + 100
    r = oracle.outcome_lookup(stop_row, out_tokens, num_out, key_row, key_token, n_keys, prepared)
    # seq 0: outcome (2, 7) matches keys 1 and 2 -> the lowest, branch 2; seq 1: (0, 5) absent;
    # seq 2: no valid keys; seq 3: (3, 8) is key 0 (keys past n_keys ignored)
    assert r["hit"].tolist() == [1, 0, 0, 1]
    assert r["branch"].tolist() == [2, 0, 0, 1]
    assert r["n_hits"][0] == 2
    assert r["next_tokens"].tolist() == [[102, 103], [0, 0], [0, 0], [118, 119]]
    assert Dm == out_tokens.shape[1] - 1


def test_lookup_bad_num_out_is_a_miss():
    r = oracle.outcome_lookup([1, 1], [[3, 3], [3, 3]], [0, 3], [[1], [1]], [[3], [3]], [1, 1])
    assert r["hit"].tolist() == [0, 0] and r["branch"].tolist() == [0, 0]


@pytest.mark.parametrize("cfg", [4, 2])
def test_lookup_closed_loop_with_acceptance(cfg):
    """Tables built from the acceptance oracle's own outcome (among decoys) always hit at the planted
    position; without it they always miss.  On a chain the stop row equals the accepted length."""
    w = W.config(cfg, B=(12 if cfg == 4 else 3), L=8, V=300)
    acc = oracle.accept(w)
    B, K = w.B, 5
    if cfg == 4:
        assert np.array_equal(acc["stop_row"], acc["accept_len"])
    bonus = acc["out_tokens"][np.arange(B), acc["num_out"] - 1]
    where = W.randint(cfg, 90, B, 0, K - 1)
    key_row = (acc["stop_row"][:, None] + 1 + np.arange(K)[None]) % (w.N + 1)  # decoys: other rows
    key_token = np.tile(bonus[:, None], (1, K))
    key_row[np.arange(B), where] = acc["stop_row"]
    key_token[np.arange(B), where] = bonus
    r = oracle.outcome_lookup(acc["stop_row"], acc["out_tokens"], acc["num_out"], key_row, key_token,
                              np.full(B, K))
    assert (r["hit"] == 1).all() and np.array_equal(r["branch"], where + 1)
    key_token[np.arange(B), where] = (bonus + 1) % w.V  # same row, another bonus token
    r = oracle.outcome_lookup(acc["stop_row"], acc["out_tokens"], acc["num_out"], key_row, key_token,
                              np.full(B, K))
    assert (r["hit"] == 0).all() and (r["branch"] == 0).all() and r["n_hits"][0] == 0


def test_reweight_touches_exactly_the_listed_tokens_fp32():
    l = W.normal(3, 1, (2, 3, 50), "f32", 2.0)
    ct = np.array([[[4, 4, 49], [-1, 50, 0], [7, 8, 9]], [[0, 1, 2], [3, 3, 3], [60, -5, 12]]], np.int32)
    shift = np.float32(-1.25)
    out = oracle.saguaro_reweight(l, ct, shift)
    want = l.copy()
    for b in range(2):
        for r in range(3):
            for v in set(int(x) for x in ct[b, r] if 0 <= x < 50):  # each distinct in-range token once
                want[b, r, v] = np.float32(want[b, r, v] + shift)
    np.testing.assert_array_equal(out, want)


def test_reweight_bf16_rounds_to_nearest_even():
    l = W.normal(4, 1, (1, 2, 40), "bf16", 3.0)
    ct = np.array([[[1, 5, 9], [2, 2, 39]]], np.int32)
    shift = np.float32(np.log(0.3))
    out = oracle.saguaro_reweight(l, ct, shift)
    f = W.bf16_to_f32(l)
    want = l.copy()
    for r, toks in enumerate(([1, 5, 9], [2, 39])):
        for v in toks:
            want[0, r, v] = W.f32_to_bf16(np.array([np.float32(f[0, r, v] + shift)], np.float32))[0]
    np.testing.assert_array_equal(out, want)
    assert (out != l).sum() == 5


def _softmax(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _saguaro_trials(rho, n, seed, p_rows, q_rows, cache):
    """Chain of one draft token drawn from the reweighted q'; verification with q' (exact by design)."""
    V = p_rows.shape[-1]
    ct = np.broadcast_to(np.asarray(cache, np.int32), (1, 2, len(cache)))
    qw = oracle.saguaro_reweight(q_rows[None].astype(np.float32), ct, np.float32(np.log(rho)))[0]
    par = np.zeros((n, 1), np.int32) - 1
    tgt = np.ascontiguousarray(np.broadcast_to(p_rows.astype(np.float32), (n, 2, V)))
    drf = np.ascontiguousarray(np.broadcast_to(qw, (n, 2, V)))
    toks = W.draft_tokens(seed, 2, drf.reshape(-1, V), np.arange(n) * 2, 1.0).reshape(n, 1)
    w = ns(B=n, N=1, parents=par, tokens=toks, target_logits=tgt, draft_logits=drf,
           u_accept=W.uniform24(seed, 11, (n, 2)), u_sample=W.uniform24(seed, 12, (n, 2)), max_depth=1,
           mode="stochastic", temperature=1.0)
    return oracle.accept(w)


@pytest.mark.slow
def test_saguaro_keeps_the_output_exact_and_raises_cache_hits():
    V, n = 16, 400_000
    p_rows = W.normal(41, 1, (2, V), "f32", 1.5)
    q_rows = W.normal(41, 2, (2, V), "f32", 1.5)
    cache = list(np.argsort(-_softmax(p_rows[0]))[:3])  # the three likeliest target tokens
    p0 = _softmax(p_rows[0])
    frac = {}
    for rho in (1.0, 0.2):
        r = _saguaro_trials(rho, n, 5 if rho == 1.0 else 6, p_rows, q_rows, cache)
        first = r["out_tokens"][:, 0]
        counts = np.bincount(first, minlength=V)
        assert stats.chisquare(counts, p0 * n).pvalue > 0.01  # still exactly p
        rej = r["accept_len"] == 0
        frac[rho] = float(np.isin(first[rej], cache).mean())  # the bonus after a rejection lands in the cache
    # residual mass on the cached tokens, closed form: sum_C max(0, p - q') / sum max(0, p - q')
    want = {}
    for rho in (1.0, 0.2):
        qw = _softmax(np.where(np.isin(np.arange(V), cache), q_rows[0] + np.log(rho), q_rows[0]))
        res = np.maximum(0, p0 - qw)
        want[rho] = res[cache].sum() / res.sum()
        assert abs(frac[rho] - want[rho]) < 0.005, (rho, frac[rho], want[rho])
    assert want[0.2] > want[1.0] + 0.01 and frac[0.2] > frac[1.0] + 0.01
