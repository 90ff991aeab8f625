"""Pins for the oracle's cache-resident tree rows and the layer-batched commit.

Definition: 'EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
NPUs', technical summary sec. 2 ('Gestion de Cache KV Ramificada'): one cache
holds the committed prefix and the speculative per-branch state; the commit by
path indices reorders the accepted path in place and avoids memory moves that
are not needed; the commit by length keeps the first A steps.  With the tree
rows in the cache, node t's K/V is cache position L + t.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _util import root_paths


def _f64(a):
    return W.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _cache_rows(w, b, g, positions, which="k"):
    """K or V rows of logical positions of sequence b, KV head g (data lookup, no arithmetic)."""
    c = w.k_cache if which == "k" else w.v_cache
    if not w.paged:
        return c[b, g, positions]
    bs = w.block_size
    return np.stack([c[w.block_table[b, p // bs], g, p % bs] for p in positions])


def _causal_rows(q, k, v, scale):
    """Textbook causal attention of one head: query t sees keys 0..t (keys start with the prefix)."""
    T = q.shape[0]
    L = k.shape[0] - T
    s = scale * (q @ k.T)
    vis = np.tril(np.ones((T, k.shape[0]), bool), k=L)
    s = np.where(vis, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def _small(paged, N=12, B=2, seed=5, chain=False):
    if paged:
        w = W.config(3, seed=seed, B=B, L=(20, 70), V=32, N=N)
    else:
        w = W.config(4, seed=seed, B=B, L=37, V=32, N=N)
        w.max_depth = 6
        if not chain:
            w.parents = np.stack([W.tree_random_recursive(seed, N, 6, offset=b * N) for b in range(B)])
    if chain:
        w.parents = np.tile(W.tree_chain(N), (B, 1))
        w.max_depth = N
    return w


@pytest.mark.parametrize("paged", [False, True])
def test_chain_in_cache_is_causal_attention_over_the_cache(paged):
    """A chain whose rows sit at positions L.. of the cache is causal attention over cache[0, L+N)."""
    w = W.with_tree_in_cache(_small(paged, N=6, chain=True))
    out = oracle.tree_attention(w)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(w.prefix_len[b])
        pos = np.arange(L + w.N)
        for h in range(w.Hq):
            g = h // G
            k = _f64(_cache_rows(w, b, g, pos, "k"))
            v = _f64(_cache_rows(w, b, g, pos, "v"))
            ref = _causal_rows(_f64(w.q[b, :, h]), k, v, w.scale)
            np.testing.assert_allclose(out[b, :, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("paged", [False, True])
def test_each_path_in_cache_is_its_own_causal_sequence(paged):
    """Node i sees the prefix and its root path, read from cache positions L + t (brute force)."""
    w = W.with_tree_in_cache(_small(paged, N=10))
    out = oracle.tree_attention(w)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        L = int(w.prefix_len[b])
        for i, path in root_paths(w.parents[b]).items():
            pos = np.concatenate([np.arange(L), L + np.asarray(path)])
            for h in (0, w.Hq - 1):
                g = h // G
                k = _f64(_cache_rows(w, b, g, pos, "k"))
                v = _f64(_cache_rows(w, b, g, pos, "v"))
                q = _f64(w.q[b, path, h])
                ref = _causal_rows(q, k, v, w.scale)[-1]
                np.testing.assert_allclose(out[b, i, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("paged", [False, True])
def test_in_cache_equals_separate_tree_rows(paged):
    """Moving the tree rows into the cache changes no output bit (same keys, same order)."""
    w = _small(paged, N=10)
    wc = W.with_tree_in_cache(w)
    np.testing.assert_array_equal(oracle.tree_attention(wc), oracle.tree_attention(w))


@pytest.mark.parametrize("paged", [False, True])
def test_in_cache_leak(paged):
    """Non-ancestor tree positions and positions past L + N are invisible."""
    w = W.with_tree_in_cache(_small(paged, N=10))
    ref = oracle.tree_attention(w)
    w2 = W.with_tree_in_cache(_small(paged, N=10))
    bs = w.block_size
    for b in range(w.B):
        L = int(w.prefix_len[b])
        par = w.parents[b]
        # node 0's ancestors are itself only if it is a root child: perturb every non-ancestor of node 0
        anc0 = set(root_paths(par)[0])
        bad = [L + t for t in range(w.N) if t not in anc0] + [L + w.N]
        for p in bad:
            if w.paged:
                blk = w2.block_table[b, p // bs]
                if blk == 0:
                    continue
                w2.k_cache[blk, :, p % bs] = W.f32_to_bf16(np.full(w.D, 1e3, np.float32))
            else:
                if p >= w.Lcap:
                    continue
                w2.k_cache[b, :, p] = W.f32_to_bf16(np.full(w.D, 1e3, np.float32))
    out = oracle.tree_attention(w2)
    np.testing.assert_array_equal(out[:, 0], ref[:, 0])


def _commit_both(w, A, rows, mode=0):
    """Commit with separate tree rows and with the rows in the cache (copies of the caches)."""
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    r = oracle.kv_commit(w, A, rows, kc, vc, commit_mode=mode)
    wc = W.with_tree_in_cache(w)
    kc2, vc2 = wc.k_cache.copy(), wc.v_cache.copy()
    r2 = oracle.kv_commit(wc, A, rows, kc2, vc2, commit_mode=mode)
    return (kc, vc, r), (wc, kc2, vc2, r2)


@pytest.mark.parametrize("paged", [False, True])
def test_full_chain_commit_in_cache_moves_nothing(paged):
    w = _small(paged, N=6, chain=True)
    A = np.full(w.B, w.N, np.int32)
    rows = np.tile(np.arange(1, w.N + 1, dtype=np.int32), (w.B, 1))
    wc = W.with_tree_in_cache(w)
    kc, vc = wc.k_cache.copy(), wc.v_cache.copy()
    r = oracle.kv_commit(wc, A, rows, kc, vc)
    assert (r["status"] == 0).all() and (r["new_len"] == w.prefix_len + w.N).all()
    assert np.array_equal(kc, wc.k_cache) and np.array_equal(vc, wc.v_cache)


@pytest.mark.parametrize("paged", [False, True])
def test_length_mode_in_cache_moves_nothing(paged):
    w = _small(paged, N=6, chain=True)
    A = np.array([3, 0] if w.B == 2 else [3] * w.B, np.int32)
    wc = W.with_tree_in_cache(w)
    kc, vc = wc.k_cache.copy(), wc.v_cache.copy()
    r = oracle.kv_commit(wc, A, np.zeros((w.B, w.max_depth), np.int32), kc, vc, commit_mode=1)
    assert np.array_equal(kc, wc.k_cache) and np.array_equal(vc, wc.v_cache)
    assert (r["new_len"] == w.prefix_len + A).all()


@pytest.mark.parametrize("paged", [False, True])
def test_in_place_compaction_equals_append_of_path_rows(paged):
    """After the in-place commit, cache positions [0, L + A) equal those of the commit from
    separate tree rows (itself pinned to an append of the path rows)."""
    w = _small(paged, N=12, B=3, seed=11)
    acc = oracle.accept(w)
    # force deep paths: the deepest node of each tree and its path
    anc, depth, prow, _ = oracle.build_tree_mask(w.parents, w.max_depth)
    A = np.zeros(w.B, np.int32)
    rows = np.zeros((w.B, w.max_depth), np.int32)
    for b in range(w.B):
        i = int(np.argmax(depth[b]))
        A[b] = depth[b, i]
        rows[b] = prow[b, i + 1]
    (kc, vc, r), (wc, kc2, vc2, r2) = _commit_both(w, A, rows)
    assert (r["status"] == 0).all() and (r2["status"] == 0).all()
    np.testing.assert_array_equal(r["new_len"], r2["new_len"])
    np.testing.assert_array_equal(r["committed_slots"], r2["committed_slots"])
    for b in range(w.B):
        pos = np.arange(int(w.prefix_len[b]) + int(A[b]))
        for g in range(w.Hkv):
            ws = type("x", (), dict(paged=w.paged, block_table=w.block_table, block_size=w.block_size,
                                    k_cache=kc, v_cache=vc))
            wi = type("x", (), dict(paged=wc.paged, block_table=wc.block_table, block_size=wc.block_size,
                                    k_cache=kc2, v_cache=vc2))
            np.testing.assert_array_equal(_cache_rows(wi, b, g, pos, "k"), _cache_rows(ws, b, g, pos, "k"))
            np.testing.assert_array_equal(_cache_rows(wi, b, g, pos, "v"), _cache_rows(ws, b, g, pos, "v"))
    del acc


def test_compaction_with_descending_node_order():
    """A path whose node indices decrease (non-topological numbering) still compacts to the
    path rows: every source is read before any destination is written."""
    N, B = 5, 1
    w = _small(False, N=N, B=B, chain=True)
    # chain in reverse numbering: node 4 is the root child, node 0 the deepest
    w.parents = np.array([[1, 2, 3, 4, -1]], np.int32)
    anc, depth, prow, st = oracle.build_tree_mask(w.parents, w.max_depth)
    assert st[0] == 0 and list(prow[0, 1]) == [5, 4, 3, 2, 1]
    A = np.array([N], np.int32)
    rows = prow[:, 1].copy()
    (kc, vc, r), (wc, kc2, vc2, r2) = _commit_both(w, A, rows)
    L = int(w.prefix_len[0])
    for k in range(N):
        np.testing.assert_array_equal(kc2[0, :, L + k], w.k_tree[0, :, N - k])
        np.testing.assert_array_equal(vc2[0, :, L + k], w.v_tree[0, :, N - k])
    np.testing.assert_array_equal(kc2[0, :, :L + N], kc[0, :, :L + N])


@pytest.mark.parametrize("paged", [False, True])
def test_in_cache_capacity_and_block_errors_write_nothing(paged):
    w = _small(paged, N=6, chain=True)
    wc = W.with_tree_in_cache(w)
    A = np.full(w.B, 3, np.int32)
    rows = np.tile(np.array([1, 3, 5, 0, 0, 0], np.int32), (w.B, 1))[:, :w.max_depth]
    kc, vc = wc.k_cache.copy(), wc.v_cache.copy()
    plen = wc.prefix_len.copy()
    cap = wc.max_blocks * wc.block_size if paged else wc.Lcap
    plen[0] = cap - w.N + 1  # L + N exceeds the capacity by one
    r = oracle.kv_commit(wc, A, rows, kc, vc, prefix_len=plen)
    assert r["status"][0] == 6 and r["new_len"][0] == plen[0] and (r["committed_slots"][0] == 0).all()
    if paged:
        bt = wc.block_table.copy()
        L1 = int(wc.prefix_len[1])
        bt[1, (L1 + 4) // wc.block_size] = 0  # the block of source position L + 5 - 1 is the ghost
        kc, vc = wc.k_cache.copy(), wc.v_cache.copy()
        A1 = A.copy()
        A1[0] = 0  # sequence 0 commits nothing, so the caches must come back unchanged
        r = oracle.kv_commit(wc, A1, rows, kc, vc, block_table=bt)
        assert r["status"][1] == 5 and r["new_len"][1] == L1 and (r["committed_slots"][1] == 0).all()
        assert np.array_equal(kc, wc.k_cache) and np.array_equal(vc, wc.v_cache)


@pytest.mark.parametrize("tic", [False, True])
@pytest.mark.parametrize("paged", [False, True])
def test_layer_batched_commit_equals_per_layer_commits(paged, tic):
    """One call over 3 layers equals three single-layer calls on each layer's tensors."""
    layers = 3
    import dataclasses
    base = _small(paged, N=12, B=3, seed=20)
    ws = [base]
    for l in range(1, layers):  # every layer shares the tree, lengths and block table; own K/V data
        ws.append(dataclasses.replace(base, **{nm: W.normal(20 + l, 40 + i, getattr(base, nm).shape, base.dtype)
                                                for i, nm in enumerate(("k_cache", "v_cache", "k_tree", "v_tree"))}))
    if tic:
        ws = [W.with_tree_in_cache(x) for x in ws]
    w0 = ws[0]
    anc, depth, prow, _ = oracle.build_tree_mask(w0.parents, w0.max_depth)
    A = np.zeros(w0.B, np.int32)
    rows = np.zeros((w0.B, w0.max_depth), np.int32)
    for b in range(w0.B):
        i = int(np.argmax(depth[b])) if b != 1 else 0
        A[b] = depth[b, i]
        rows[b] = prow[b, i + 1]
    kc = np.stack([x.k_cache for x in ws])
    vc = np.stack([x.v_cache for x in ws])
    kt = None if tic else np.stack([x.k_tree for x in ws])
    vt = None if tic else np.stack([x.v_tree for x in ws])
    r = oracle.kv_commit(w0, A, rows, kc, vc, k_tree=kt, v_tree=vt, num_layers=layers)
    for l, x in enumerate(ws):
        k1, v1 = x.k_cache.copy(), x.v_cache.copy()
        r1 = oracle.kv_commit(x, A, rows, k1, v1)
        np.testing.assert_array_equal(kc[l], k1)
        np.testing.assert_array_equal(vc[l], v1)
        for key in ("new_len", "committed_slots", "status"):
            np.testing.assert_array_equal(r[key], r1[key])
    assert not np.array_equal(kc[0], kc[1])
