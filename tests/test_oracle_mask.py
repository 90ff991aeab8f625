"""Pins for the oracle's tree tensorisation (mask, depth, path rows, status).

Definitions: 'EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
NPUs', technical summary sec. 2 -- shifted indexing with a dummy root row 0,
ancestor index tables, range / acyclicity / depth checks; a token attends to
itself and its ancestors only.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _util import golden, root_paths


def _bits_to_set(words):
    s = set()
    for w, x in enumerate(words):
        x = int(x)
        for j in range(64):
            if (x >> j) & 1:
                s.add(64 * w + j)
    return s


def _relabel(parents, perm):
    """Rename node i to perm[i]; parents stay a valid tree but lose topological order."""
    N = len(parents)
    out = np.empty(N, dtype=np.int32)
    for i in range(N):
        p = parents[i]
        out[perm[i]] = -1 if p < 0 else perm[p]
    return out


@pytest.mark.parametrize("case", range(9))
def test_golden_cases(case):
    c = golden("tree_mask_cases.json")["cases"][case]
    par = np.array([c["parents"]], dtype=np.int32)
    anc, depth, prow, st = oracle.build_tree_mask(par, c["max_depth"])
    assert anc[0, :, 0].tolist() == c["anc"]
    assert depth[0].tolist() == c["depth"]
    assert prow[0].tolist() == c["path_rows"]
    assert int(st[0]) == c["status"]


def _trees():
    yield W.tree_chain(9)
    yield W.tree_star(7)
    yield W.tree_eagle_static(2)
    yield W.tree_random_recursive(3, 32, 6)
    yield W.tree_outcome(5)
    yield W.tree_random_recursive(11, 200, 16)


@pytest.mark.parametrize("ti", range(6))
@pytest.mark.parametrize("relabel", [False, True])
def test_brute_force_bfs(ti, relabel):
    """Ancestor sets, depths and path rows equal a breadth-first search from the root."""
    par = list(_trees())[ti]
    N = len(par)
    if relabel:
        perm = np.array(W.randint(7, 99, N, 0, 1 << 30)).argsort().astype(np.int32)
        par = _relabel(par, perm)
    paths = root_paths(par)
    assert len(paths) == N
    maxd = max(len(p) for p in paths.values())
    anc, depth, prow, st = oracle.build_tree_mask(par[None, :], maxd)
    assert st[0] == 0
    for i in range(N):
        assert _bits_to_set(anc[0, i]) == set(paths[i])
        assert depth[0, i] == len(paths[i])
        exp_rows = [t + 1 for t in paths[i]] + [0] * (maxd - len(paths[i]))
        assert prow[0, i + 1].tolist() == exp_rows
    assert prow[0, 0].tolist() == [0] * maxd
    # invariant: bits[i] = bits[parent] | {i}
    for i in range(N):
        want = {i} | (_bits_to_set(anc[0, par[i]]) if par[i] >= 0 else set())
        assert _bits_to_set(anc[0, i]) == want
    # no negative index anywhere
    assert (prow >= 0).all() and (depth >= 0).all()


def test_depth_limit_marks_only_deep_nodes():
    par = W.tree_chain(8)[None, :]
    anc, depth, prow, st = oracle.build_tree_mask(par, 5)
    assert st[0] == 3
    assert depth[0].tolist() == [1, 2, 3, 4, 5, 0, 0, 0]
    for i in range(5, 8):
        assert _bits_to_set(anc[0, i]) == {i}
        assert prow[0, i + 1].tolist() == [0] * 5


def test_fuzz_malformed_never_negative():
    """Random parent arrays over [-3, N+2]: statuses are the smallest failing code and all indices stay >= 0."""
    rng_draws = W.randint(21, 77, 64 * 24, -3, 26).reshape(64, 24).astype(np.int32)
    anc, depth, prow, st = oracle.build_tree_mask(rng_draws, 6)
    assert (prow >= 0).all() and (prow <= 24).all() and (depth >= 0).all() and (depth <= 6).all()
    for b in range(64):
        par = rng_draws[b]
        codes = []
        for i in range(24):
            # independent restatement of the three checks, by following pointers with a visited list
            seen, cur, code = [i], i, 0
            while True:
                p = int(par[cur])
                if p < -1 or p >= 24:
                    code = 1
                    break
                if p == -1:
                    break
                if p in seen:
                    code = 2
                    break
                if len(seen) + 1 > 6:
                    code = 3
                    break
                seen.append(p)
                cur = p
            codes.append(code)
            if code:
                assert depth[b, i] == 0 and _bits_to_set(anc[b, i]) == {i}
            else:
                assert depth[b, i] == len(seen)
        nz = [c for c in codes if c]
        assert st[b] == (min(nz) if nz else 0)


def test_batch_independence():
    a = W.tree_eagle_static(2)
    b = W.tree_chain(60)
    par = np.stack([a, b])
    anc, depth, prow, st = oracle.build_tree_mask(par, 60)
    anc1, depth1, _, _ = oracle.build_tree_mask(a[None], 60)
    assert (anc[0] == anc1[0]).all() and (depth[0] == depth1[0]).all()
    assert depth[1].tolist() == list(range(1, 61))
