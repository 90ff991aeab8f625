"""GPU vs oracle parity for cache-resident tree rows and the layer-batched commit.

The tree tokens' K/V sit in the cache at positions prefix_len + t: the attention
reads them there (contiguous or through the block table) and the commit
compacts the accepted path in place.  Bar: attention within the dtype's
tolerance (plus relative-L2 for bf16), everything else bit-exact, including
every byte of the caches after the commit.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check_attention, compare_accept, require_gpu, run_step, sample_rows, to_np

pytestmark = pytest.mark.gpu

SMALL = {
    1: dict(),
    2: dict(L=333, V=3001),
    3: dict(B=5, L=(40, 400), V=2500, N=32),
    4: dict(B=6, L=161, V=2999),
    5: dict(B=2, L=290, V=1500),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _commit_ok(w, r):
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ref = oracle.kv_commit(w, r["acc"]["accept_len"], r["acc"]["accept_rows"], kc, vc)
    for k in ("new_len", "committed_slots", "status"):
        assert np.array_equal(r["commit"][k], ref[k]), k
    assert np.array_equal(r["k_cache"], kc)
    assert np.array_equal(r["v_cache"], vc)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_step_tree_in_cache_small(cfg):
    w = W.with_tree_in_cache(W.config(cfg, **SMALL[cfg]))
    r = run_step(w)
    ref = oracle.tree_attention(w)
    err, rel = check_attention(r["out"], ref, w.dtype, f"config {cfg} tree in cache")
    print(f"  attention max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert (r["astatus"] == 0).all()
    acc = oracle.accept(w)
    compare_accept(r["acc"], acc)
    _commit_ok(w, r)


@pytest.mark.parametrize("cfg", [2, 3])
def test_step_tree_in_cache_full_size(cfg):
    """Full sizes of the EAGLE static tree (contiguous) and the batched paged workload."""
    w = W.with_tree_in_cache(W.config(cfg))
    r = run_step(w)
    n = {2: 10**9, 3: 160}[cfg]
    if n >= w.B * w.N * w.Hq:
        ref, got = oracle.tree_attention(w), r["out"]
    else:
        sel = sample_rows(w, n, seed=cfg)
        ref, got = oracle.tree_attention(w, sel=sel), r["out"].reshape(-1, w.D)[sel]
    err, rel = check_attention(got, ref, w.dtype, f"config {cfg} full, tree in cache")
    print(f"  attention max-abs {err:.2e} rel-L2 {rel:.2e}")
    compare_accept(r["acc"], oracle.accept(w))
    _commit_ok(w, r)


@pytest.mark.parametrize("paged", [False, True])
def test_tree_in_cache_capacity_status(paged):
    """prefix_len + N beyond the capacity: attention status 6 (prefix clamped), commit status 6."""
    w = W.with_tree_in_cache(W.config(3 if paged else 4, **(SMALL[3] if paged else SMALL[4])))
    cap = w.max_blocks * w.block_size if paged else w.Lcap
    w.prefix_len = w.prefix_len.copy()
    w.prefix_len[1] = cap - w.N + 1
    r = run_step(w)
    ref = oracle.tree_attention(w)
    check_attention(r["out"], ref, w.dtype, "clamped prefix")
    assert r["astatus"][1] == 6 and (np.delete(r["astatus"], 1) == 0).all()
    _commit_ok(w, r)
    assert r["commit"]["status"][1] == 6


def _dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(x).to("cuda:0")


def _layered(w, layers, seed):
    """Per-layer copies of a workload with their own K/V data (same tree, lengths, blocks)."""
    out = [w]
    for l in range(1, layers):
        out.append(dataclasses.replace(w, **{nm: W.normal(seed + l, 50 + i, getattr(w, nm).shape, w.dtype)
                                             for i, nm in enumerate(("k_cache", "v_cache", "k_tree", "v_tree"))}))
    return out


@pytest.mark.parametrize("tic", [False, True])
@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_layer_batched_commit(cfg, tic):
    """One sv_kv_commit over 4 layers vs the oracle over the same stacked caches."""
    import torch
    import tree_verification_sv_amd as sv
    layers = 4
    w = W.config(cfg, **SMALL[cfg])
    acc = oracle.accept(w)
    # a mix of accepted lengths: the walk's result, a forced deepest path and nothing
    anc, depth, prow, _ = oracle.build_tree_mask(w.parents, w.max_depth)
    A, rows = acc["accept_len"].copy(), acc["accept_rows"].copy()
    i = int(np.argmax(depth[0]))
    A[0], rows[0] = depth[0, i], prow[0, i + 1]
    if w.B > 1:
        A[-1], rows[-1] = 0, 0
    ws = _layered(w, layers, seed=70 + cfg)
    if tic:
        ws = [W.with_tree_in_cache(x) for x in ws]
    w0 = ws[0]
    kc = np.stack([x.k_cache for x in ws])
    vc = np.stack([x.v_cache for x in ws])
    kt = None if tic else np.stack([x.k_tree for x in ws])
    vt = None if tic else np.stack([x.v_tree for x in ws])
    print(f"[gpu] layered commit {w.name} layers={layers} tree_in_cache={tic} A={A.tolist()}", flush=True)
    dev = W.to_device(w0, "cuda:0")
    kc_d, vc_d = _dev(kc), _dev(vc)
    kt_d = None if tic else _dev(kt)
    vt_d = None if tic else _dev(vt)
    A_d = torch.from_numpy(A.astype(np.int32)).to("cuda:0")
    rows_d = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int32)).to("cuda:0")
    out = sv.sv_kv_commit(kc_d, vc_d, kt_d, vt_d, dev["prefix_len"], A_d, rows_d, w0.max_depth,
                          block_table=dev["block_table"], paged=w0.paged, num_blocks=w0.num_blocks,
                          tree_in_cache=tic, N=w0.N, num_layers=layers)
    torch.cuda.synchronize()
    kc_ref, vc_ref = kc.copy(), vc.copy()
    ref = oracle.kv_commit(w0, A, rows, kc_ref, vc_ref, k_tree=kt, v_tree=vt, num_layers=layers)
    for k in ("new_len", "committed_slots", "status"):
        assert np.array_equal(to_np(out[k]), ref[k]), k
    assert np.array_equal(to_np(kc_d), kc_ref)
    assert np.array_equal(to_np(vc_d), vc_ref)
    assert (ref["status"] == 0).all()
