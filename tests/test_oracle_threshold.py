"""Pins for the oracle's threshold acceptance (mode 'threshold').

Definition: 'Accelerating Sonar Through Speculation', section 'Decodificacion
Especulativa': each prefix of the draft candidates is scored with a
probability and the longest prefix above an acceptance threshold is kept; the
target then supplies one more token.  Reading (also in the oracle header): a
prefix's score is the product of the target probabilities softmax(row / T) of
its tokens at their parent rows; the extra token is the stop row's argmax.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads as W
from _util import golden, ns, root_paths


def _case_ns(c):
    B, N = 1, len(c["parents"])
    target = np.asarray(c["target"], np.float32)[None]
    return ns(B=B, N=N, V=target.shape[-1], max_depth=c["max_depth"], parents=np.asarray([c["parents"]], np.int32),
              tokens=np.asarray([c["tokens"]], np.int32), target_logits=target, mode="threshold",
              temperature=c["temperature"], threshold=c["threshold"])


@pytest.mark.parametrize("idx", range(len(golden("threshold_cases.json")["cases"])))
def test_golden(idx):
    c = golden("threshold_cases.json")["cases"][idx]
    r = oracle.accept(_case_ns(c))
    assert r["accept_len"][0] == c["accept_len"], c["note"]
    assert r["accept_rows"][0].tolist() == c["accept_rows"], c["note"]
    assert r["out_tokens"][0].tolist() == c["out_tokens"], c["note"]
    assert r["num_out"][0] == c["num_out"] and r["stop_row"][0] == c["stop_row"], c["note"]
    assert r["status"][0] == c.get("status", 0)
    assert r["flagged"][0] == 0


def _fp32_tree_workload(seed, B=8, N=20, V=500):
    """fp32 logits (no bf16 ties), random recursive trees, planted argmax matches."""
    par = np.stack([W.tree_random_recursive(seed, N, 6, offset=b * N) for b in range(B)])
    return W.build_workload("fp32-tree", B, N, 4, 2, 64, V, "f32", "greedy", par, np.full(B, 16), max_depth=6,
                            seed=seed, logit_sigma=3.0, token_rule="uniform", plant=W.plant_pairs(seed, par),
                            need_draft=False)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_cold_limit_equals_greedy(seed):
    """As T -> 0 the target distribution becomes the point mass at the row's argmax, so a threshold of
    1/2 accepts exactly the argmax-matching prefixes: threshold acceptance equals greedy acceptance."""
    w = _fp32_tree_workload(seed)
    g = oracle.accept(w, mode="greedy")
    t = oracle.accept(w, mode="threshold", temperature=1e-4, threshold=0.5)
    assert (t["flagged"] == 0).all()
    for k in ("accept_len", "accept_rows", "out_tokens", "num_out", "stop_row", "status"):
        np.testing.assert_array_equal(t[k], g[k], err_msg=k)
    assert g["accept_len"].max() >= 2  # the planted matches make the comparison non-trivial


def test_zero_threshold_accepts_the_deepest_usable_node():
    w = _fp32_tree_workload(4)
    t = oracle.accept(w, mode="threshold", temperature=1.0, threshold=0.0)
    anc, depth, prow, _ = oracle.build_tree_mask(w.parents, w.max_depth)
    for b in range(w.B):
        i = int(np.argmax(depth[b]))  # deepest, lowest index on ties
        assert t["accept_len"][b] == depth[b, i] and t["stop_row"][b] == i + 1
        np.testing.assert_array_equal(t["accept_rows"][b], prow[b, i + 1])


def test_accepted_length_never_grows_with_the_threshold():
    w = _fp32_tree_workload(5, V=40)
    last = None
    for tau in (0.0, 1e-6, 1e-4, 1e-3, 0.01, 0.05, 0.1, 0.3, 0.6, 1.0):
        A = oracle.accept(w, mode="threshold", temperature=1.0, threshold=tau)["accept_len"]
        if last is not None:
            assert (A <= last).all()
        last = A
    assert (last == 0).all()  # no random token has probability 1


def _softmax(x):
    e = np.exp(x - x.max())
    return e / e.sum()


@pytest.mark.parametrize("seed", [6, 7])
def test_brute_force_small_vocab(seed):
    """Enumerate every root path of small trees over a 16-token vocabulary with numpy."""
    B, N, V = 6, 9, 16
    par = np.stack([W.tree_random_recursive(seed, N, 4, offset=b * N) for b in range(B)])
    w = W.build_workload("v16", B, N, 2, 1, 64, V, "f32", "greedy", par, np.full(B, 4), max_depth=4, seed=seed,
                         logit_sigma=1.0, token_rule="uniform", need_draft=False)
    for T, tau in itertools.product((0.7, 1.0, 1.6), (0.002, 0.01, 0.04)):
        r = oracle.accept(w, mode="threshold", temperature=T, threshold=tau)
        for b in range(B):
            tl = w.target_logits[b].astype(np.float64)
            best, best_i = 0, -1
            for i, path in sorted(root_paths(w.parents[b]).items()):
                s, ok = 1.0, True
                for t in path:
                    s *= _softmax(tl[w.parents[b, t] + 1] / T)[w.tokens[b, t]]
                    ok &= s >= tau
                if ok and len(path) > best:
                    best, best_i = len(path), i
            if r["flagged"][b]:
                continue
            assert r["accept_len"][b] == best
            assert r["stop_row"][b] == best_i + 1
            assert r["out_tokens"][b, best] == int(np.argmax(tl[best_i + 1]))
