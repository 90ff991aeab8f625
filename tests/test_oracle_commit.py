"""Pins for the oracle's KV commit of the accepted branch.

Definition: 'EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
NPUs', technical summary sec. 2 ('Gestion de Cache KV Ramificada'): the
committed prefix is kept apart from speculative state; commit by length (keep
the first A steps) or by path indices (the accepted path's rows).
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _chain(paged, L=37, N=6, B=2):
    if paged:
        w = W.config(3, seed=9, B=B, L=(L, L + 20), V=32, N=N)
        w.parents = np.tile(W.tree_chain(N), (B, 1))
        return w
    return W.config(4, seed=9, B=B, L=L, V=32, N=N)


@pytest.mark.parametrize("paged", [False, True])
def test_full_acceptance_is_append(paged):
    w = _chain(paged)
    A = np.full(w.B, w.N, np.int32)
    rows = np.tile(np.arange(1, w.N + 1, dtype=np.int32), (w.B, 1))
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    r = oracle.kv_commit(w, A, rows, kc, vc)
    assert (r["status"] == 0).all() and (r["new_len"] == w.prefix_len + w.N).all()
    for b in range(w.B):
        L = int(w.prefix_len[b])
        for k in range(w.N):
            pos = L + k
            if paged:
                blk = w.block_table[b, pos // w.block_size]
                assert r["committed_slots"][b, k] == blk * w.block_size + pos % w.block_size
                np.testing.assert_array_equal(kc[blk, :, pos % w.block_size], w.k_tree[b, :, k + 1])
                np.testing.assert_array_equal(vc[blk, :, pos % w.block_size], w.v_tree[b, :, k + 1])
            else:
                assert r["committed_slots"][b, k] == pos
                np.testing.assert_array_equal(kc[b, :, pos], w.k_tree[b, :, k + 1])
                np.testing.assert_array_equal(vc[b, :, pos], w.v_tree[b, :, k + 1])
        # the prefix itself is untouched
        if not paged:
            np.testing.assert_array_equal(kc[b, :, :L], w.k_cache[b, :, :L])


@pytest.mark.parametrize("paged", [False, True])
def test_zero_acceptance_changes_nothing(paged):
    w = _chain(paged)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    r = oracle.kv_commit(w, np.zeros(w.B, np.int32), np.zeros((w.B, w.max_depth), np.int32), kc, vc)
    assert np.array_equal(kc, w.k_cache) and np.array_equal(vc, w.v_cache)
    assert (r["new_len"] == w.prefix_len).all() and (r["committed_slots"] == 0).all()


def test_only_path_rows_change_tree():
    w = W.config(3, seed=4, B=4, L=(16, 90), V=40, N=20)
    acc = oracle.accept(w)
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    r = oracle.kv_commit(w, acc["accept_len"], acc["accept_rows"], kc, vc)
    changed = np.argwhere((kc != w.k_cache).any(axis=-1))  # (block, head, offset)
    expect = set()
    for b in range(w.B):
        for k in range(int(acc["accept_len"][b])):
            s = int(r["committed_slots"][b, k])
            for h in range(w.Hkv):
                expect.add((s // w.block_size, h, s % w.block_size))
    assert set(map(tuple, changed.tolist())) <= expect
    assert (r["committed_slots"] >= 0).all()


def test_length_mode_equals_path_mode_on_chains():
    w = _chain(False, B=3)
    A = np.array([0, 3, 6], np.int32)
    rows = np.zeros((3, w.max_depth), np.int32)
    for b in range(3):
        rows[b, :A[b]] = np.arange(1, A[b] + 1)
    k1, v1 = w.k_cache.copy(), w.v_cache.copy()
    k2, v2 = w.k_cache.copy(), w.v_cache.copy()
    r1 = oracle.kv_commit(w, A, rows, k1, v1, commit_mode=0)
    r2 = oracle.kv_commit(w, A, np.zeros_like(rows), k2, v2, commit_mode=1)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    for k in r1:
        assert np.array_equal(r1[k], r2[k])


def test_errors_write_nothing():
    w = _chain(True, B=3)
    A = np.array([2, 2, 2], np.int32)
    rows = np.tile(np.array([1, 2, 0, 0, 0, 0], np.int32), (3, 1))
    bt = w.block_table.copy()
    L0 = int(w.prefix_len[0])
    bt[0, L0 // w.block_size] = 0                  # ghost block in a needed place -> 5
    rows[1, 1] = w.N + 3                           # row out of range -> 1
    plen = w.prefix_len.copy()
    plen[2] = w.max_blocks * w.block_size - 1       # second slot falls off the table -> 6
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    r = oracle.kv_commit(w, A, rows, kc, vc, prefix_len=plen, block_table=bt)
    assert r["status"].tolist() == [5, 1, 6]
    assert (r["new_len"] == plen).all() and (r["committed_slots"] == 0).all()
    assert np.array_equal(kc, w.k_cache) and np.array_equal(vc, w.v_cache)
