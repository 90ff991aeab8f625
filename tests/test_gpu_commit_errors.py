"""sv_kv_commit on crafted accepted paths (through the C ABI) against the oracle's commit:
valid paths, accepted lengths beyond max_depth, ghost source rows, ghost or missing blocks,
capacity overflow, commit by length, and nothing to commit.  Status codes, new lengths,
committed slots and every cache byte must match; nothing is written for a failing sequence.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import require_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(w, A, rows, plen, bt, mode):
    import torch
    import tree_verification_sv_amd as sv
    print(f"[gpu] commit {w.name} B={w.B} paged={w.paged} mode={mode} A={A.tolist()} L={plen.tolist()}", flush=True)
    dev = W.to_device(w, "cuda:0")
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to("cuda:0")
    out = sv.sv_kv_commit(dev["k_cache"], dev["v_cache"], dev["k_tree"], dev["v_tree"], d(plen), d(A), d(rows),
                          w.max_depth, block_table=d(bt) if bt is not None else None, paged=w.paged,
                          num_blocks=w.num_blocks, commit_mode=mode)
    torch.cuda.synchronize()
    got = {k: to_np(v) for k, v in out.items()}
    got["k_cache"], got["v_cache"] = to_np(dev["k_cache"]), to_np(dev["v_cache"])
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ref = oracle.kv_commit(w, A, rows, kc, vc, commit_mode=mode, prefix_len=plen, block_table=bt)
    for k in ("status", "new_len", "committed_slots"):
        assert np.array_equal(got[k], ref[k]), (k, got[k], ref[k])
    assert np.array_equal(got["k_cache"], kc) and np.array_equal(got["v_cache"], vc)
    return ref


def test_commit_paged_error_paths():
    w = W.config(3, B=6, L=(40, 400), V=2500, N=32)
    Dm = w.max_depth
    plen = w.prefix_len.astype(np.int32).copy()
    bt = w.block_table.copy()
    A = np.array([4, Dm + 1, 3, 4, 5, 0], np.int32)
    rows = np.zeros((w.B, Dm), np.int32)
    rows[0, :4] = [3, 7, 12, 20]
    rows[2, :3] = [2, 0, 5]                  # ghost source row at position 1
    rows[3, :4] = [1, 2, 3, 4]
    bt[3, (int(plen[3]) + 2) // 16] = 0      # ghost block at or before position 2
    rows[4, :5] = [5, 6, 7, 8, 9]
    plen[4] = w.max_blocks * 16 - 2          # positions 2.. beyond the block table
    ref = _run(w, A, rows, plen, bt, 0)
    assert ref["status"][0] == 0 and ref["status"][1] == 1 and ref["status"][2] == 1
    assert ref["status"][3] == 5 and ref["status"][4] in (5, 6) and ref["status"][5] == 0


def test_commit_contiguous_capacity_and_length_mode():
    w = W.config(4, B=6, L=161, V=2999)
    Dm = w.max_depth
    plen = w.prefix_len.astype(np.int32).copy()
    A = np.array([Dm, 2, 3, 0, 1, Dm], np.int32)
    rows = np.zeros((w.B, Dm), np.int32)
    for b in range(w.B):
        rows[b, :A[b]] = np.arange(1, A[b] + 1)
    plen[2] = w.Lcap - 1                     # position 1 is past the capacity
    plen[4] = -3                             # negative prefix length
    for mode in (0, 1):
        ref = _run(w, A, rows, plen, None, mode)
        assert ref["status"][2] == 6 and ref["status"][4] == 1 and ref["status"][0] == 0
