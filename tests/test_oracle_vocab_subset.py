"""Pins for the oracle's draft vocabulary subset (draft logits over a subset of the target vocabulary).

Definition: 'EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
NPUs', technical summary sec. 3, item 5: the drafter works on a cached subset of
the vocabulary.  Acceptance compares full distributions ('Accelerating Sonar
Through Speculation', 'Objetivo-Borrador'), so the draft distribution is taken
over the whole target vocabulary with probability 0 outside the subset.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import workloads as W
from _util import ns


def _t2d(V, ids):
    t = np.zeros(V, np.int32)
    t[np.asarray(ids)] = np.arange(1, len(ids) + 1, dtype=np.int32)
    return t


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_map_is_a_copy(dtype):
    sub = W.normal(1, 1, (2, 3, 40), dtype, 3.0)
    full = oracle.draft_subset_logits(sub, np.arange(1, 41, dtype=np.int32))
    np.testing.assert_array_equal(full, sub)


def test_subset_softmax_is_scattered_with_zeros_elsewhere():
    V, ids = 50, [3, 17, 4, 49, 0, 22]
    sub = W.normal(2, 1, (1, 2, len(ids)), "f32", 2.0)
    full = oracle.draft_subset_logits(sub, _t2d(V, ids))
    for r in range(2):
        f = full[0, r].astype(np.float64)
        e = np.exp(f - f.max())
        q_full = e / e.sum()
        s = sub[0, r].astype(np.float64)
        es = np.exp(s - s.max())
        q_sub = es / es.sum()
        want = np.zeros(V)
        want[ids] = q_sub
        np.testing.assert_allclose(q_full, want, rtol=1e-12, atol=0)


def test_out_of_range_map_entries_are_absent():
    sub = W.normal(3, 1, (1, 1, 4), "bf16", 1.0)
    t2d = np.array([0, 1, 5, -2, 4, 2], np.int32)  # 5 and -2 are not subset positions
    full = oracle.draft_subset_logits(sub, t2d)[0, 0]
    assert full[1] == sub[0, 0, 0] and full[4] == sub[0, 0, 3] and full[5] == sub[0, 0, 1]
    assert all(W.bf16_to_f32(full[[0, 2, 3]]) == -np.inf)


@pytest.mark.slow
def test_rejection_sampling_with_a_subset_drafter_is_exact():
    """Vocab 16, drafter on 6 ids: the first emitted token still follows p over all 16 ids."""
    V, n, ids = 16, 400_000, [1, 2, 5, 8, 11, 14]
    p_rows = W.normal(51, 1, (2, V), "f32", 1.5)
    sub = W.normal(51, 2, (1, 2, len(ids)), "f32", 1.5)
    q_rows = oracle.draft_subset_logits(sub, _t2d(V, ids))[0]
    tgt = np.ascontiguousarray(np.broadcast_to(p_rows, (n, 2, V)))
    drf = np.ascontiguousarray(np.broadcast_to(q_rows, (n, 2, V)))
    toks = W.draft_tokens(9, 2, drf.reshape(-1, V), np.arange(n) * 2, 1.0).reshape(n, 1)
    assert np.isin(toks, ids).all()  # the drafter never proposes an id outside its subset
    w = ns(B=n, N=1, parents=np.full((n, 1), -1, np.int32), tokens=toks, target_logits=tgt, draft_logits=drf,
           u_accept=W.uniform24(9, 11, (n, 2)), u_sample=W.uniform24(9, 12, (n, 2)), max_depth=1,
           mode="stochastic", temperature=1.0)
    r = oracle.accept(w)
    first = r["out_tokens"][:, 0]
    e = np.exp(p_rows[0] - p_rows[0].max())
    p0 = e / e.sum()
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, p0 * n).pvalue > 0.01
    assert (~np.isin(first, ids)).any()  # ids outside the subset reach the output through the residual
