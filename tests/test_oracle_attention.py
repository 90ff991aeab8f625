"""Pins for the oracle's ancestor-masked GQA tree attention.

Definition: 'EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
NPUs', technical summary sec. 2 ('Ejecucion del Maestro con Mascara de Arbol
Fusionada'): each draft token attends to the committed prefix, to its
ancestors and to itself; tokens of other branches are invisible.  Softmax
attention with scale 1/sqrt(D) and query head h reading KV head h // (Hq/Hkv).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _util import ns, root_paths


def _tiny(parents, L, Hq=4, Hkv=2, D=8, seed=1, dtype="f32", B=1):
    par = np.tile(np.asarray(parents, dtype=np.int32), (B, 1))
    N = par.shape[1]
    Lcap = L + 8
    return ns(B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, parents=par, prefix_len=np.full(B, L, np.int32),
              max_depth=max(8, N), Lcap=Lcap,
              q=W.normal(seed, 1, (B, N, Hq, D), dtype),
              k_cache=W.normal(seed, 2, (B, Hkv, Lcap, D), dtype),
              v_cache=W.normal(seed, 3, (B, Hkv, Lcap, D), dtype),
              k_tree=W.normal(seed, 4, (B, Hkv, N + 1, D), dtype),
              v_tree=W.normal(seed, 5, (B, Hkv, N + 1, D), dtype))


def _f64(a):
    return W.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _causal_attention(q, k, v, scale):
    """Textbook causal attention for one head: query t sees keys 0..t.  q,k,v: [T, D]."""
    T = q.shape[0]
    s = scale * (q @ k.T)
    s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_equals_causal_attention(dtype):
    """A chain-shaped tree is ordinary causal attention over [prefix, chain]."""
    L, N = 13, 5
    w = _tiny(W.tree_chain(N), L, dtype=dtype)
    out = oracle.tree_attention(w)
    G = w.Hq // w.Hkv
    for h in range(w.Hq):
        g = h // G
        k = np.concatenate([_f64(w.k_cache[0, g, :L]), _f64(w.k_tree[0, g, 1:])])
        v = np.concatenate([_f64(w.v_cache[0, g, :L]), _f64(w.v_tree[0, g, 1:])])
        # prefix queries are never asked for; give them zero rows
        qq = np.concatenate([np.zeros((L, w.D)), _f64(w.q[0, :, h])])
        ref = _causal_attention(qq, k, v, w.scale)[L:]
        np.testing.assert_allclose(out[0, :, h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("tree", ["eagle", "outcome_small", "random"])
def test_each_path_equals_path_alone(tree):
    """Every root-to-node path, run alone as a causal sequence, gives the tree outputs of its nodes."""
    if tree == "eagle":
        par = W.tree_eagle_static(4, n_nodes=8, branch=3, depth=4)
    elif tree == "outcome_small":
        par = W.tree_outcome(6, budgets=(4, 2, 1, 1), k=2, max_depth=4)
    else:
        par = W.tree_random_recursive(9, 8, 4)
    L = 11
    w = _tiny(par, L, seed=3)
    out = oracle.tree_attention(w)
    G = w.Hq // w.Hkv
    for node, path in root_paths(par).items():
        for h in range(w.Hq):
            g = h // G
            rows = [t + 1 for t in path]
            k = np.concatenate([_f64(w.k_cache[0, g, :L]), _f64(w.k_tree[0, g, rows])])
            v = np.concatenate([_f64(w.v_cache[0, g, :L]), _f64(w.v_tree[0, g, rows])])
            qq = np.concatenate([np.zeros((L, w.D)), _f64(w.q[0, path, h])])
            ref = _causal_attention(qq, k, v, w.scale)[-1]
            np.testing.assert_allclose(out[0, node, h], ref, rtol=1e-12, atol=1e-13)


def test_no_cross_branch_leak():
    """Perturbing K/V of every non-ancestor tree row by +-1e3 changes no output bit."""
    par = W.tree_eagle_static(2)
    w = _tiny(par, 7, seed=5, D=16)
    base = oracle.tree_attention(w)
    paths = root_paths(par)
    for node in (0, 5, 17, 42, 59):
        anc = set(paths[node])
        w2 = _tiny(par, 7, seed=5, D=16)
        for t in range(len(par)):
            if t not in anc:
                sign = 1.0 if t % 2 else -1.0
                w2.k_tree[:, :, t + 1] += np.float32(sign * 1e3)
                w2.v_tree[:, :, t + 1] -= np.float32(sign * 1e3)
        o2 = oracle.tree_attention(w2)
        assert np.array_equal(o2[0, node], base[0, node])


def test_empty_prefix_star_returns_own_value():
    """L = 0 and every parent -1: a node sees only itself, so o = v_self exactly."""
    w = _tiny(W.tree_star(6), 0, seed=8)
    out = oracle.tree_attention(w)
    G = w.Hq // w.Hkv
    for i in range(6):
        for h in range(w.Hq):
            assert np.array_equal(out[0, i, h], w.v_tree[0, h // G, i + 1].astype(np.float64))


def test_equal_keys_give_mean_of_visible_values():
    """All keys identical -> uniform weights -> mean of the visible V rows."""
    par = W.tree_eagle_static(3, n_nodes=10, branch=3, depth=3)
    w = _tiny(par, 9, seed=2)
    w.k_cache[:] = w.k_cache[0, 0, 0]
    w.k_tree[:] = w.k_cache[0, 0, 0]
    out = oracle.tree_attention(w)
    G = w.Hq // w.Hkv
    for node, path in root_paths(par).items():
        for h in range(w.Hq):
            g = h // G
            vis = np.concatenate([w.v_cache[0, g, :9], w.v_tree[0, g, [t + 1 for t in path]]]).astype(np.float64)
            np.testing.assert_allclose(out[0, node, h], vis.mean(0), rtol=1e-13, atol=1e-14)


def test_two_keys_known_weights():
    """Hand example: scores 0 and ln 3 give weights 1/4 and 3/4."""
    D = 4
    w = _tiny([-1], 1, Hq=1, Hkv=1, D=D)
    w.scale = 1.0
    w.q[:] = 0
    w.q[0, 0, 0, 0] = 1.0
    w.k_cache[:] = 0
    w.k_tree[:] = 0
    w.k_tree[0, 0, 1, 0] = np.float32(np.log(3.0))
    w.v_cache[0, 0, 0] = [4, 0, 0, 0]
    w.v_tree[0, 0, 1] = [0, 8, 0, 0]
    out = oracle.tree_attention(w)[0, 0, 0]
    s = float(np.float32(np.log(3.0)))
    p1 = np.exp(s) / (1 + np.exp(s))
    np.testing.assert_allclose(out, [4 * (1 - p1), 8 * p1, 0, 0], rtol=1e-14)
    np.testing.assert_allclose(out, [1.0, 6.0, 0, 0], rtol=1e-7)


def test_gqa_grouping_consecutive_heads():
    """Query heads g*G .. g*G+G-1 read KV head g: swapping KV heads swaps those output groups."""
    w = _tiny(W.tree_chain(3), 5, Hq=4, Hkv=2)
    a = oracle.tree_attention(w)
    for name in ("k_cache", "v_cache", "k_tree", "v_tree"):
        x = getattr(w, name)
        setattr(w, name, np.ascontiguousarray(x[:, ::-1]))
    w.q = np.ascontiguousarray(w.q[:, :, [2, 3, 0, 1]])
    b = oracle.tree_attention(w)
    np.testing.assert_array_equal(a[:, :, [2, 3, 0, 1]], b)


def test_paged_equals_contiguous():
    """The same logical KV through a shuffled block table gives identical outputs."""
    wp = W.config(3, B=3, L=(20, 70), V=64, N=9)
    # build the contiguous twin from the paged pool
    B, Hkv, D, bs = wp.B, wp.Hkv, wp.D, wp.block_size
    Lcap = wp.max_blocks * bs
    kc = np.zeros((B, Hkv, Lcap, D), dtype=wp.k_cache.dtype)
    vc = np.zeros_like(kc)
    for b in range(B):
        for j in range(wp.max_blocks):
            blk = wp.block_table[b, j]
            kc[b, :, j * bs:(j + 1) * bs] = wp.k_cache[blk]
            vc[b, :, j * bs:(j + 1) * bs] = wp.v_cache[blk]
    wc = ns(B=B, N=wp.N, Hq=wp.Hq, Hkv=Hkv, D=D, parents=wp.parents, prefix_len=wp.prefix_len,
            max_depth=wp.max_depth, Lcap=Lcap, q=wp.q, k_cache=kc, v_cache=vc, k_tree=wp.k_tree, v_tree=wp.v_tree)
    sel = np.arange(0, B * wp.N * wp.Hq, 7)
    np.testing.assert_array_equal(oracle.tree_attention(wp, sel=sel), oracle.tree_attention(wc, sel=sel))


def test_selection_matches_full():
    w = _tiny(W.tree_eagle_static(2, n_nodes=12), 10, B=2)
    full = oracle.tree_attention(w).reshape(-1, w.D)
    sel = np.array([0, 5, 47, 95])
    np.testing.assert_array_equal(oracle.tree_attention(w, sel=sel), full[sel])


def test_peaky_query_selects_matching_key():
    """A query aligned with one key and scaled up puts (almost) all weight on that key's value."""
    D = 8
    w = _tiny([-1, 0], 6, Hq=1, Hkv=1, D=D, seed=4)
    w.k_cache[:] = 0
    w.k_tree[:] = 0
    w.k_cache[0, 0, 3, 2] = 1.0
    w.q[:] = 0
    w.q[0, :, 0, 2] = 200.0
    out = oracle.tree_attention(w)
    np.testing.assert_allclose(out[0, 1, 0], w.v_cache[0, 0, 3].astype(np.float64), atol=1e-20 + 1e-12)
