"""Pins for the oracle's speculative acceptance (greedy and stochastic).

Definitions: 'Accelerating Sonar Through Speculation' (sections
'Decodificacion Especulativa', 'Objetivo-Borrador', 'EAGLE'): keep the
longest acceptable draft sequence, emit up to n+1 tokens with the bonus token
taken from the target logits after it, acceptance by comparing the full draft
and target distributions; 'Speculative Speculative Decoding' (sec. 3B residual
mass, sec. 5 exact output distribution).
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import workloads as W
from _util import golden, ns, root_paths


def _greedy_ns(parents, tokens, target, max_depth):
    par = np.asarray(parents, np.int32)[None]
    return ns(B=1, N=par.shape[1], parents=par, tokens=np.asarray(tokens, np.int32)[None],
              target_logits=np.asarray(target, np.float32)[None], max_depth=max_depth, mode="greedy")


@pytest.mark.parametrize("case", range(5))
def test_greedy_golden(case):
    c = golden("greedy_cases.json")["cases"][case]
    r = oracle.accept(_greedy_ns(c["parents"], c["tokens"], c["target"], c["max_depth"]))
    for k in ("accept_len", "num_out", "stop_row"):
        assert int(r[k][0]) == c[k], k
    assert r["accept_rows"][0].tolist() == c["accept_rows"]
    assert r["out_tokens"][0].tolist() == c["out_tokens"]


@pytest.mark.parametrize("case", range(3))
def test_stochastic_golden(case):
    c = golden("stochastic_cases.json")["cases"][case]
    par = np.asarray(c["parents"], np.int32)[None]
    w = ns(B=1, N=par.shape[1], parents=par, tokens=np.asarray(c["tokens"], np.int32)[None],
           target_logits=np.asarray(c["target"], np.float32)[None], draft_logits=np.asarray(c["draft"], np.float32)[None],
           u_accept=np.asarray(c["u_accept"], np.float32)[None], u_sample=np.asarray(c["u_sample"], np.float32)[None],
           max_depth=c["max_depth"], mode="stochastic", temperature=1.0)
    r = oracle.accept(w)
    for k in ("accept_len", "num_out", "stop_row"):
        assert int(r[k][0]) == c[k], k
    assert r["accept_rows"][0].tolist() == c["accept_rows"]
    assert r["out_tokens"][0].tolist() == c["out_tokens"]
    assert r["flagged"][0] == 0


def _brute_greedy(parents, tokens, target):
    """Enumerate every root-to-node path; keep the deepest fully matching one (lowest index on ties)."""
    amax = target.argmax(axis=-1)  # numpy returns the first maximum: lowest id on ties
    best_node, best_len = -1, 0
    for node, path in sorted(root_paths(parents).items()):
        if all(tokens[t] == amax[parents[t] + 1] for t in path) and len(path) > best_len:
            best_node, best_len = node, len(path)
    path = root_paths(parents)[best_node] if best_node >= 0 else []
    return best_len, [t + 1 for t in path], [int(tokens[t]) for t in path] + [int(amax[best_node + 1])], best_node + 1


@pytest.mark.parametrize("seed", range(6))
def test_greedy_brute_force(seed):
    """Planted batched trees: the oracle equals brute-force enumeration of all root paths."""
    w = W.config(3, seed=100 + seed, B=6, L=(8, 40), V=50, N=20)
    r = oracle.accept(w)
    T = W.bf16_to_f32(w.target_logits)
    for b in range(w.B):
        A, rows, toks, stop = _brute_greedy(w.parents[b], w.tokens[b], T[b])
        assert r["accept_len"][b] == A
        assert r["accept_rows"][b, :A].tolist() == rows and (r["accept_rows"][b, A:] == 0).all()
        assert r["out_tokens"][b, :A + 1].tolist() == toks and (r["out_tokens"][b, A + 1:] == 0).all()
        assert r["num_out"][b] == A + 1 and r["stop_row"][b] == stop
        assert 1 <= r["num_out"][b] <= w.max_depth + 1


def test_greedy_duplicate_tokens_with_ties():
    """Small vocab with many ties and duplicate sibling tokens still matches brute force."""
    for seed in range(10):
        par = W.tree_random_recursive(seed, 12, 5)
        toks = W.randint(seed, 3, 12, 0, 2).astype(np.int32)
        tgt = W.randint(seed, 4, 13 * 3, 0, 1).astype(np.float32).reshape(13, 3)
        r = oracle.accept(_greedy_ns(par, toks, tgt, 5))
        A, rows, out, stop = _brute_greedy(par, toks, tgt)
        assert (int(r["accept_len"][0]), int(r["stop_row"][0])) == (A, stop)
        assert r["out_tokens"][0, :A + 1].tolist() == out


@pytest.mark.parametrize("k", range(5))
def test_chain_planted_prefix_scan(k):
    """Tiny chain with target rows copied from the greedy drafter's rows for r < k: A = k."""
    w = W.config(1, plant=k)
    r = oracle.accept(w)
    amax = w.target_logits[0].argmax(-1)
    lead = 0
    while lead < w.N and w.tokens[0, lead] == amax[lead]:
        lead += 1
    assert r["accept_len"][0] == lead == k
    assert r["out_tokens"][0, k] == amax[k]


def test_target_equals_greedy_draft_accepts_deepest_path():
    """p rows = q rows and greedily drafted tokens: the whole deepest path is accepted."""
    par = W.tree_eagle_static(5)
    V = 300
    q = W.normal(5, 9, (61, V), "f32", 3.0)
    toks = q.argmax(-1)[par + 1].astype(np.int32)
    r = oracle.accept(_greedy_ns(par, toks, q, 6))
    d = W.tree_depths(par)
    # siblings drafted from the same row share a token, so every node matches
    assert r["accept_len"][0] == d.max()
    assert r["stop_row"][0] == int(np.argmax(d)) + 1


def test_bad_token_status_and_exclusion():
    par = W.tree_chain(3)
    tgt = np.zeros((4, 5), np.float32)
    r = oracle.accept(_greedy_ns(par, [0, 7, 0], tgt, 3))
    assert r["status"][0] == 4 and r["accept_len"][0] == 1


# ------------------------------------------------------------------ stochastic
def _stoch_batch(parents, p_rows, q_rows, n, seed, T=1.0):
    """n independent trials of one tree: tokens drawn i.i.d. from q of the parent row."""
    par = np.tile(np.asarray(parents, np.int32), (n, 1))
    N = par.shape[1]
    V = p_rows.shape[-1]
    tgt = np.ascontiguousarray(np.broadcast_to(p_rows.astype(np.float32), (n, N + 1, V)))
    drf = np.ascontiguousarray(np.broadcast_to(q_rows.astype(np.float32), (n, N + 1, V)))
    prow = (np.arange(n)[:, None] * (N + 1) + par + 1).reshape(-1)
    toks = W.draft_tokens(seed, 2, drf.reshape(-1, V), prow, T).reshape(n, N)
    return ns(B=n, N=N, parents=par, tokens=toks, target_logits=tgt, draft_logits=drf,
              u_accept=W.uniform24(seed, 11, (n, N + 1)), u_sample=W.uniform24(seed, 12, (n, N + 1)),
              max_depth=N, mode="stochastic", temperature=T)


def _softmax(x, T=1.0):
    x = np.asarray(x, np.float64) / T
    e = np.exp(x - x.max())
    return e / e.sum()


def _first_token_hist(parents, p_rows, q_rows, trials, seed, batch=200_000, T=1.0):
    V = p_rows.shape[-1]
    counts = np.zeros(V, np.int64)
    acc1 = 0
    flagged = 0
    for s in range(trials // batch):
        w = _stoch_batch(parents, p_rows, q_rows, batch, seed * 1000 + s, T)
        r = oracle.accept(w)
        counts += np.bincount(r["out_tokens"][:, 0], minlength=V)
        acc1 += int((r["accept_len"] >= 1).sum())
        flagged += int(r["flagged"].sum())
    return counts, acc1, flagged


@pytest.mark.slow
@pytest.mark.parametrize("shape", ["chain1", "chain3", "siblings3"])
def test_rejection_sampling_is_exact_chi_square(shape):
    """Vocab 16, 10^6 trials: the first emitted token follows p_root (chi-square p > 0.01)."""
    V = 16
    parents = {"chain1": [-1], "chain3": [-1, 0, 1], "siblings3": [-1, -1, -1]}[shape]
    N = len(parents)
    p_rows = W.normal(31, 1, (N + 1, V), "f32", 1.5)
    q_rows = W.normal(31, 2, (N + 1, V), "f32", 1.5)
    counts, acc1, flagged = _first_token_hist(parents, p_rows, q_rows, 1_000_000, seed=7)
    p0 = _softmax(p_rows[0])
    chi = stats.chisquare(counts, p0 * counts.sum())
    assert chi.pvalue > 0.01, (chi, counts, p0)
    # a wrong residual (plain p instead of max(0, p - q)) would fail: check the test has power
    q0 = _softmax(q_rows[0])
    assert stats.chisquare(counts, q0 * counts.sum()).pvalue < 1e-6


@pytest.mark.slow
def test_acceptance_probability_closed_form():
    """One child: P(A >= 1) = sum_v min(p(v), q(v)) within 4 sigma."""
    V = 16
    p_rows = W.normal(41, 1, (2, V), "f32", 1.0)
    q_rows = W.normal(41, 2, (2, V), "f32", 1.0)
    n = 1_000_000
    _, acc1, _ = _first_token_hist([-1], p_rows, q_rows, n, seed=9)
    P = np.minimum(_softmax(p_rows[0]), _softmax(q_rows[0])).sum()
    sigma = np.sqrt(P * (1 - P) / n)
    assert abs(acc1 / n - P) < 4 * sigma, (acc1 / n, P)


def test_temperature_applies_to_both_distributions():
    """At T=2 the first token follows softmax(l_p/2) (chi-square on 2e5 trials)."""
    V = 8
    p_rows = W.normal(51, 1, (3, V), "f32", 2.0)
    q_rows = W.normal(51, 2, (3, V), "f32", 2.0)
    counts, _, _ = _first_token_hist([-1, 0], p_rows, q_rows, 200_000, seed=5, T=2.0)
    assert stats.chisquare(counts, _softmax(p_rows[0], 2.0) * counts.sum()).pvalue > 0.01
    assert stats.chisquare(counts, _softmax(p_rows[0], 1.0) * counts.sum()).pvalue < 1e-6


def test_p_equals_q_accepts_everything():
    par = W.tree_eagle_static(8)
    V = 64
    rows = W.normal(8, 1, (61, V), "f32", 3.0)
    w = _stoch_batch(par, rows, rows, 500, seed=3)
    r = oracle.accept(w)
    # ratio is exactly 1 > u for every tested child: the walk takes the first child at every row
    first_child_chain = 0
    node = -1
    while True:
        kids = [i for i in range(len(par)) if par[i] == node]
        if not kids:
            break
        node = kids[0]
        first_child_chain += 1
    assert (r["accept_len"] == first_child_chain).all()


def test_flagging_near_threshold():
    c = golden("stochastic_cases.json")["cases"][2]
    par = np.asarray(c["parents"], np.int32)[None]
    tgt = np.asarray(c["target"], np.float32)[None]
    drf = np.asarray(c["draft"], np.float32)[None]
    ratio = float(np.exp(-2 * np.float64(np.float32(1.0986123))))  # (1/(1+3)) / (3/(1+3)) with fp32 ln3
    ua = np.array([[0.0, np.float32(ratio)]], np.float32)
    w = ns(B=1, N=1, parents=par, tokens=np.zeros((1, 1), np.int32), target_logits=tgt, draft_logits=drf,
           u_accept=ua, u_sample=np.array([[0.5, 0.0]], np.float32), max_depth=1, mode="stochastic", temperature=1.0)
    assert oracle.accept(w)["flagged"][0] == 1
    w.u_accept = np.array([[0.0, 0.9]], np.float32)
    assert oracle.accept(w)["flagged"][0] == 0
    # bonus sampling on the boundary: root residual is [0, 1]; u_s = 0 sits on C_{-1} = 0
    w.u_sample = np.array([[0.0, 0.0]], np.float32)
    assert oracle.accept(w)["flagged"][0] == 1


# ------------------------------------------------- deterministic (top-K) drafts
# The drafter proposes each child deterministically, so its proposal for child c
# is the point mass at tokens[c]: accept iff u < p_cur(x); a rejection zeroes x in
# p_cur and renormalises (sampling without replacement).  Because the first
# emitted token of any lossless scheme follows p_root, a child with a token of
# its own is accepted with probability exactly p_root(x).
@pytest.mark.parametrize("case", range(4))
def test_topk_golden(case):
    c = golden("topk_cases.json")["cases"][case]
    par = np.asarray(c["parents"], np.int32)[None]
    w = ns(B=1, N=par.shape[1], parents=par, tokens=np.asarray(c["tokens"], np.int32)[None],
           target_logits=np.asarray(c["target"], np.float32)[None], draft_logits=None,
           u_accept=np.asarray(c["u_accept"], np.float32)[None], u_sample=np.asarray(c["u_sample"], np.float32)[None],
           max_depth=c["max_depth"], mode="topk", temperature=1.0)
    r = oracle.accept(w)
    for k in ("accept_len", "num_out", "stop_row"):
        assert int(r[k][0]) == c[k], k
    assert r["accept_rows"][0].tolist() == c["accept_rows"]
    assert r["out_tokens"][0].tolist() == c["out_tokens"]
    assert r["flagged"][0] == 0


def _topk_batch(parents, tokens, p_rows, n, seed, T=1.0):
    par = np.tile(np.asarray(parents, np.int32), (n, 1))
    N = par.shape[1]
    V = p_rows.shape[-1]
    tgt = np.ascontiguousarray(np.broadcast_to(p_rows.astype(np.float32), (n, N + 1, V)))
    return ns(B=n, N=N, parents=par, tokens=np.tile(np.asarray(tokens, np.int32), (n, 1)), target_logits=tgt,
              draft_logits=None, u_accept=W.uniform24(seed, 11, (n, N + 1)),
              u_sample=W.uniform24(seed, 12, (n, N + 1)), max_depth=N, mode="topk", temperature=T)


@pytest.mark.slow
@pytest.mark.parametrize("T", [1.0, 2.0])
def test_topk_first_token_and_child_acceptance_exact(T):
    """Three sibling drafts with distinct tokens, 6e5 trials: the first emitted token
    follows p_root and child k is accepted with probability p_root(x_k) (chi-square)."""
    V = 16
    p_rows = W.normal(61, 1, (4, V), "f32", 1.5)
    p0 = _softmax(p_rows[0], T)
    toks = [int(x) for x in np.argsort(-p0, kind="stable")[:3]]  # the three most likely tokens
    counts = np.zeros(V, np.int64)
    which = np.zeros(4, np.int64)  # accepted child 0, 1, 2, or none
    for s in range(3):
        r = oracle.accept(_topk_batch([-1, -1, -1], toks, p_rows, 200_000, seed=900 + s, T=T))
        counts += np.bincount(r["out_tokens"][:, 0], minlength=V)
        first = np.where(r["accept_len"] >= 1, r["accept_rows"][:, 0] - 1, 3)
        which += np.bincount(first, minlength=4)
    assert stats.chisquare(counts, p0 * counts.sum()).pvalue > 0.01
    pk = np.array([p0[toks[0]], p0[toks[1]], p0[toks[2]], 1 - p0[toks].sum()])
    assert stats.chisquare(which, pk * which.sum()).pvalue > 0.01, (which, pk)
    # power: testing every child against p_root without renormalising after a rejection
    # gives p1, (1-p1) p2, (1-p1)(1-p2) p3 -- visibly different
    p1, p2, p3 = p0[toks]
    alt = np.array([p1, (1 - p1) * p2, (1 - p1) * (1 - p2) * p3, (1 - p1) * (1 - p2) * (1 - p3)])
    assert stats.chisquare(which, alt * which.sum()).pvalue < 1e-6


def test_topk_repeated_sibling_token_is_never_accepted():
    """Siblings with the same token: after the first is rejected its token has mass 0."""
    V = 8
    p_rows = W.normal(71, 1, (4, V), "f32", 1.0)
    r = oracle.accept(_topk_batch([-1, -1, -1], [3, 3, 6], p_rows, 50_000, seed=17))
    assert not (r["accept_rows"][:, 0] == 2).any()
    assert (r["accept_rows"][:, 0] == 1).any() and (r["accept_rows"][:, 0] == 3).any()


@pytest.mark.parametrize("seed", range(4))
def test_topk_chain_equals_stochastic_with_one_hot_draft(seed):
    """On a chain (one child per row) the deterministic draft is mode 1 with a draft row
    whose distribution is the point mass at the child's token (logit 0 there, -1e30
    elsewhere, so every other probability is exactly 0 in fp64)."""
    B, N, V = 300, 4, 32
    par = np.tile(W.tree_chain(N), (B, 1))
    tgt = W.normal(seed, 1, (B, N + 1, V), "f32", 1.0)
    toks = W.randint(seed, 3, B * N, 0, V - 1).astype(np.int32).reshape(B, N)
    drf = np.full((B, N + 1, V), -1e30, np.float32)
    for b in range(B):
        for i in range(N):
            drf[b, i, toks[b, i]] = 0.0  # row i is the parent row of node i on a chain
    ua, us = W.uniform24(seed, 11, (B, N + 1)), W.uniform24(seed, 12, (B, N + 1))
    common = dict(B=B, N=N, parents=par, tokens=toks, target_logits=tgt, u_accept=ua, u_sample=us, max_depth=N,
                  temperature=1.0)
    r1 = oracle.accept(ns(mode="stochastic", draft_logits=drf, **common))
    r2 = oracle.accept(ns(mode="topk", draft_logits=None, **common))
    for k in ("accept_len", "accept_rows", "out_tokens", "num_out", "stop_row", "status"):
        assert np.array_equal(r1[k], r2[k]), k
    assert (r1["accept_len"] > 0).any() and (r1["accept_len"] < N).any()


def test_topk_token_generator_orders_by_logit_then_id():
    """Siblings take the most likely ids of their parent row in turn, lowest id first on ties."""
    rng = np.random.default_rng(0)
    for _ in range(100):
        V = int(rng.integers(1, 40))
        n = int(rng.integers(1, V + 1))
        lg = np.zeros((1, 2, V), np.float32)
        lg[0, 0] = rng.integers(0, 4, V)
        got = W.topk_tokens(lg, np.full((1, n), -1, np.int32))[0]
        assert np.array_equal(got, np.argsort(-lg[0, 0], kind="stable")[:n])
