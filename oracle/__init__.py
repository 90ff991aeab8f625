"""CPU oracle for tree speculative-decoding verification -- TEST INFRASTRUCTURE.

Thin ctypes marshalling around ``oracle.c`` (plain scalar C, fp64).  Only the
tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package; the product path never does.  The oracle shares no code
with the GPU library; both are fed from the seeded generators in ``workloads``.

Parity pins live in ``tests/test_oracle_*.py``.  Per-draw outcomes of the
stochastic acceptance walk follow one sampling convention (sibling order,
uniform layout, inverse-CDF order); that convention itself is "parity
unpinned" by the pages -- only its distribution is pinned (chi-square tests).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-shared", "-fPIC",
                               os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _AttnArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("D", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_double),
                ("paged", ctypes.c_int32), ("Lcap", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_tree", ctypes.c_void_p), ("v_tree", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("prefix_len", ctypes.c_void_p), ("parents", ctypes.c_void_p), ("max_depth", ctypes.c_int32),
                ("sel", ctypes.c_void_p), ("n_sel", ctypes.c_int64), ("out", ctypes.c_void_p),
                ("tree_in_cache", ctypes.c_int32)]


class _AcceptArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("V", ctypes.c_int32), ("max_depth", ctypes.c_int32),
                ("logits_dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("temperature", ctypes.c_double),
                ("parents", ctypes.c_void_p), ("tokens", ctypes.c_void_p), ("target_logits", ctypes.c_void_p),
                ("draft_logits", ctypes.c_void_p), ("u_accept", ctypes.c_void_p), ("u_sample", ctypes.c_void_p),
                ("accept_len", ctypes.c_void_p), ("accept_rows", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
                ("num_out", ctypes.c_void_p), ("stop_row", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("flagged", ctypes.c_void_p), ("threshold", ctypes.c_double)]


class _CommitArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("max_depth", ctypes.c_int32), ("commit_mode", ctypes.c_int32),
                ("paged", ctypes.c_int32), ("Lcap", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("k_tree", ctypes.c_void_p), ("v_tree", ctypes.c_void_p), ("prefix_len", ctypes.c_void_p),
                ("accept_len", ctypes.c_void_p), ("accept_rows", ctypes.c_void_p), ("new_len", ctypes.c_void_p),
                ("committed_slots", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("tree_in_cache", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("cache_layer_stride", ctypes.c_int64), ("tree_layer_stride", ctypes.c_int64)]


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.orc_build_tree_mask.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P]
        lib.orc_build_tree_mask.restype = ctypes.c_int
        lib.orc_tree_attention.argtypes = [ctypes.POINTER(_AttnArgs)]
        lib.orc_tree_attention.restype = ctypes.c_int
        lib.orc_accept.argtypes = [ctypes.POINTER(_AcceptArgs)]
        lib.orc_accept.restype = ctypes.c_int
        lib.orc_kv_commit.argtypes = [ctypes.POINTER(_CommitArgs)]
        lib.orc_kv_commit.restype = ctypes.c_int
        i32 = ctypes.c_int32
        lib.orc_outcome_lookup.argtypes = [i32, i32, i32, i32] + [P] * 11
        lib.orc_outcome_lookup.restype = ctypes.c_int
        lib.orc_saguaro_reweight.argtypes = [P, i32, i32, i32, i32, P, i32, ctypes.c_float]
        lib.orc_saguaro_reweight.restype = ctypes.c_int
        lib.orc_draft_subset_logits.argtypes = [P, i32, i32, i32, P, i32, i32, P]
        lib.orc_draft_subset_logits.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype in (np.uint16, np.int16):
        return 1
    raise TypeError(a.dtype)


def build_tree_mask(parents: np.ndarray, max_depth: int):
    """-> anc_bits [B,N,W] uint64, depth [B,N], path_rows [B,N+1,max_depth], status [B]."""
    parents = np.ascontiguousarray(parents, dtype=np.int32)
    B, N = parents.shape
    W = (N + 63) // 64
    anc = np.zeros((B, N, W), dtype=np.uint64)
    depth = np.zeros((B, N), dtype=np.int32)
    path_rows = np.zeros((B, N + 1, max_depth), dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    rc = _L().orc_build_tree_mask(_p(parents), B, N, max_depth, _p(anc), _p(depth), _p(path_rows), _p(status))
    if rc != 0:
        raise ValueError("orc_build_tree_mask rejected its arguments")
    return anc, depth, path_rows, status


def tree_attention(w, sel: Optional[np.ndarray] = None, parents: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 attention output; [B,N,Hq,D] or [len(sel), D] for flat (b*N+i)*Hq+h indices."""
    parents = np.ascontiguousarray(w.parents if parents is None else parents, dtype=np.int32)
    a = _AttnArgs()
    a.B, a.N, a.Hq, a.Hkv, a.D = w.B, w.N, w.Hq, w.Hkv, w.D
    a.dtype = _dt(w.q)
    a.scale = float(w.scale)
    a.paged = int(bool(w.paged))
    a.Lcap, a.block_size, a.max_blocks, a.num_blocks = w.Lcap, w.block_size, w.max_blocks, w.num_blocks
    keep = [np.ascontiguousarray(x) if x is not None else None
            for x in (w.q, w.k_cache, w.v_cache, w.k_tree, w.v_tree, w.block_table, w.prefix_len)]
    a.q, a.k_cache, a.v_cache, a.k_tree, a.v_tree, a.block_table = [_p(x) for x in keep[:6]]
    plen = np.ascontiguousarray(w.prefix_len, dtype=np.int32)
    a.prefix_len = _p(plen)
    a.parents = _p(parents)
    a.max_depth = w.max_depth
    a.tree_in_cache = int(bool(getattr(w, "tree_in_cache", False)))
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int64)
        out = np.zeros((sel.size, w.D), dtype=np.float64)
        a.sel, a.n_sel = _p(sel), sel.size
    else:
        out = np.zeros((w.B, w.N, w.Hq, w.D), dtype=np.float64)
        a.sel, a.n_sel = None, 0
    a.out = _p(out)
    if _L().orc_tree_attention(ctypes.byref(a)) != 0:
        raise ValueError("orc_tree_attention rejected its arguments")
    return out


def accept(w, mode: Optional[str] = None, temperature: Optional[float] = None, tokens=None, parents=None,
           target=None, draft=None, u_accept=None, u_sample=None, threshold: Optional[float] = None) -> dict:
    mode = w.mode if mode is None else mode
    T = w.temperature if temperature is None else temperature
    parents = np.ascontiguousarray(w.parents if parents is None else parents, dtype=np.int32)
    tokens = np.ascontiguousarray(w.tokens if tokens is None else tokens, dtype=np.int32)
    target = np.ascontiguousarray(w.target_logits if target is None else target)
    draft = w.draft_logits if draft is None else draft
    draft = np.ascontiguousarray(draft) if draft is not None else None
    ua = w.u_accept if u_accept is None else u_accept
    us = w.u_sample if u_sample is None else u_sample
    B, N = parents.shape
    V = target.shape[-1]
    Dm = w.max_depth
    out = dict(accept_len=np.zeros(B, np.int32), accept_rows=np.zeros((B, Dm), np.int32),
               out_tokens=np.zeros((B, Dm + 1), np.int32), num_out=np.zeros(B, np.int32),
               stop_row=np.zeros(B, np.int32), status=np.zeros(B, np.int32), flagged=np.zeros(B, np.int32))
    a = _AcceptArgs()
    a.B, a.N, a.V, a.max_depth = B, N, V, Dm
    a.logits_dtype = _dt(target)
    a.mode = {"greedy": 0, "stochastic": 1, "topk": 2, "threshold": 3}[mode]
    a.temperature = float(T)
    a.threshold = float(getattr(w, "threshold", 0.0) if threshold is None else threshold)
    a.parents, a.tokens, a.target_logits = _p(parents), _p(tokens), _p(target)
    if a.mode in (1, 2):
        ua = np.ascontiguousarray(ua, dtype=np.float32)
        us = np.ascontiguousarray(us, dtype=np.float32)
        a.draft_logits = _p(draft) if a.mode == 1 else None
        a.u_accept, a.u_sample = _p(ua), _p(us)
    for k in out:
        setattr(a, k, _p(out[k]))
    if _L().orc_accept(ctypes.byref(a)) != 0:
        raise ValueError("orc_accept rejected its arguments")
    return out


def kv_commit(w, accept_len: np.ndarray, accept_rows: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
              commit_mode: int = 0, prefix_len=None, block_table=None, k_tree=None, v_tree=None,
              num_layers: int = 1) -> dict:
    """Commits into the given caches in place (pass copies); returns new_len, committed_slots, status.

    num_layers > 1: k_cache / v_cache (and k_tree / v_tree unless the tree rows are
    in the cache) carry a leading layer dimension; every layer is committed."""
    B, N, Dm = w.B, w.N, w.max_depth
    tic = bool(getattr(w, "tree_in_cache", False))
    plen = np.ascontiguousarray(w.prefix_len if prefix_len is None else prefix_len, dtype=np.int32)
    bt = w.block_table if block_table is None else block_table
    bt = np.ascontiguousarray(bt, dtype=np.int32) if bt is not None else None
    alen = np.ascontiguousarray(accept_len, dtype=np.int32)
    arows = np.ascontiguousarray(accept_rows, dtype=np.int32)
    kt = w.k_tree if k_tree is None else k_tree
    vt = w.v_tree if v_tree is None else v_tree
    kt = None if tic else np.ascontiguousarray(kt)
    vt = None if tic else np.ascontiguousarray(vt)
    out = dict(new_len=np.zeros(B, np.int32), committed_slots=np.zeros((B, Dm), np.int32),
               status=np.zeros(B, np.int32))
    a = _CommitArgs()
    a.B, a.N, a.Hkv, a.D = B, N, w.Hkv, w.D
    a.elem_bytes = k_cache.itemsize
    a.max_depth, a.commit_mode = Dm, commit_mode
    a.paged = int(bool(w.paged))
    a.Lcap, a.block_size, a.max_blocks, a.num_blocks = w.Lcap, w.block_size, w.max_blocks, w.num_blocks
    assert k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]
    a.k_cache, a.v_cache, a.block_table = _p(k_cache), _p(v_cache), _p(bt)
    a.k_tree, a.v_tree = _p(kt), _p(vt)
    a.prefix_len, a.accept_len, a.accept_rows = _p(plen), _p(alen), _p(arows)
    a.new_len, a.committed_slots, a.status = _p(out["new_len"]), _p(out["committed_slots"]), _p(out["status"])
    a.tree_in_cache = int(tic)
    a.num_layers = num_layers
    if num_layers > 1:
        a.cache_layer_stride = k_cache[0].size
        a.tree_layer_stride = 0 if tic else kt[0].size
    if _L().orc_kv_commit(ctypes.byref(a)) != 0:
        raise ValueError("orc_kv_commit rejected its arguments")
    return out


def outcome_lookup(stop_row, out_tokens, num_out, key_row, key_token, n_keys, prepared=None) -> dict:
    """SSD outcome lookup; key_* [B,K], prepared [B,K,P] or None.  -> hit, branch, next_tokens, n_hits."""
    c = lambda x: np.ascontiguousarray(x, dtype=np.int32)  # noqa: E731
    stop_row, out_tokens, num_out, key_row, key_token, n_keys = map(c, (stop_row, out_tokens, num_out, key_row,
                                                                         key_token, n_keys))
    B, K = key_row.shape
    Dm = out_tokens.shape[1] - 1
    P = 0 if prepared is None else prepared.shape[2]
    prepared = None if prepared is None else c(prepared)
    out = dict(hit=np.zeros(B, np.int32), branch=np.zeros(B, np.int32), n_hits=np.zeros(1, np.int32),
               next_tokens=np.zeros((B, P), np.int32) if P else None)
    rc = _L().orc_outcome_lookup(B, K, P, Dm, _p(stop_row), _p(out_tokens), _p(num_out), _p(key_row), _p(key_token),
                                 _p(n_keys), _p(prepared), _p(out["hit"]), _p(out["branch"]), _p(out["next_tokens"]),
                                 _p(out["n_hits"]))
    if rc != 0:
        raise ValueError("orc_outcome_lookup rejected its arguments")
    return out


def saguaro_reweight(draft_logits: np.ndarray, cache_tokens: np.ndarray, shift: float) -> np.ndarray:
    """Returns a reweighted copy of draft_logits [B,R,V] (fp32 or bf16 bits); cache_tokens [B,R,C]."""
    out = np.ascontiguousarray(draft_logits).copy()
    ct = np.ascontiguousarray(cache_tokens, dtype=np.int32)
    B, R, V = out.shape
    rc = _L().orc_saguaro_reweight(_p(out), B, R, V, _dt(out), _p(ct), ct.shape[2], float(np.float32(shift)))
    if rc != 0:
        raise ValueError("orc_saguaro_reweight rejected its arguments")
    return out


def draft_subset_logits(sub: np.ndarray, t2d: np.ndarray) -> np.ndarray:
    """Full-vocabulary draft logits [B,R,V] from subset logits [B,R,Vd] and t2d [V] (j+1, 0 = absent)."""
    sub = np.ascontiguousarray(sub)
    t2d = np.ascontiguousarray(t2d, dtype=np.int32)
    B, R, Vd = sub.shape
    V = t2d.size
    full = np.empty((B, R, V), dtype=sub.dtype)
    if _L().orc_draft_subset_logits(_p(sub), B, R, Vd, _p(t2d), V, _dt(sub), _p(full)) != 0:
        raise ValueError("orc_draft_subset_logits rejected its arguments")
    return full
