"""Python binding of libspecverify: argument marshalling only.

Every function here forwards torch tensors (device pointers) and the current
HIP stream to the C-ABI entry point of the same name in ``libspecverify.so``
(declared in ``include/specverify.h``).  All computation runs in the library's
HIP kernels; if the library is not built this module raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libspecverify.so")
_lib = None

SV_OK, SV_ERR_INVALID_ARGUMENT, SV_ERR_UNSUPPORTED, SV_ERR_BAD_TREE, SV_ERR_HIP, SV_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4, 5
SV_ACCEPT_SCRATCH_BYTES = 4 << 20
SV_F32, SV_BF16 = 0, 1
SV_GREEDY, SV_STOCHASTIC, SV_TOPK_DRAFT, SV_THRESHOLD = 0, 1, 2, 3
_MODES = {"greedy": SV_GREEDY, "stochastic": SV_STOCHASTIC, "topk": SV_TOPK_DRAFT, "threshold": SV_THRESHOLD}
SV_COMMIT_PATH, SV_COMMIT_LENGTH = 0, 1
SV_FLAG_VALIDATE = 1
SV_FLAG_ROW_LIST = 2
SV_SEQ_NONFINITE = 8

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = ["sv_api.hip", "sv_mask.hip", "sv_attention.hip", "sv_accept.hip", "sv_threshold.hip", "sv_commit.hip",
           "sv_ssd.hip", "sv_vocab.hip", "sv_step.hip"]


class SpecVerifyError(RuntimeError):
    pass


def build(verbose: bool = False) -> str:
    """Compile libspecverify.so for gfx950 with hipcc (in-tree)."""
    srcs = [os.path.join(_HERE, "csrc", s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", os.path.join(_ROOT, "include"), *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise SpecVerifyError("hipcc failed:\n" + r.stderr[-4000:])
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# ------------------------------------------------------------ C structures
class sv_attn_args(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("D", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("paged", ctypes.c_int32), ("Lcap", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_tree", ctypes.c_void_p), ("v_tree", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("prefix_len", ctypes.c_void_p), ("anc_bits", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("status", ctypes.c_void_p),
                ("tree_in_cache", ctypes.c_int32)]


class sv_accept_args(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("V", ctypes.c_int32), ("max_depth", ctypes.c_int32),
                ("logits_dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("temperature", ctypes.c_float),
                ("parents", ctypes.c_void_p), ("tokens", ctypes.c_void_p), ("anc_bits", ctypes.c_void_p),
                ("depth", ctypes.c_void_p), ("target_logits", ctypes.c_void_p), ("draft_logits", ctypes.c_void_p),
                ("u_accept", ctypes.c_void_p), ("u_sample", ctypes.c_void_p), ("accept_len", ctypes.c_void_p),
                ("accept_rows", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p), ("num_out", ctypes.c_void_p),
                ("stop_row", ctypes.c_void_p), ("status", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("threshold", ctypes.c_float), ("commit", ctypes.c_void_p),
                ("flags", ctypes.c_uint32)]


class sv_commit_args(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_depth", ctypes.c_int32), ("commit_mode", ctypes.c_int32),
                ("paged", ctypes.c_int32), ("Lcap", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("k_tree", ctypes.c_void_p), ("v_tree", ctypes.c_void_p), ("prefix_len", ctypes.c_void_p),
                ("accept_len", ctypes.c_void_p), ("accept_rows", ctypes.c_void_p), ("new_len", ctypes.c_void_p),
                ("committed_slots", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("tree_in_cache", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("cache_layer_stride", ctypes.c_int64), ("tree_layer_stride", ctypes.c_int64)]


class sv_step_args(ctypes.Structure):
    _fields_ = [("attn", ctypes.c_void_p), ("accept", ctypes.c_void_p), ("anc_bits", ctypes.c_void_p),
                ("depth", ctypes.c_void_p), ("path_rows", ctypes.c_void_p), ("mask_status", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class sv_outcome_args(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("K", ctypes.c_int32), ("P", ctypes.c_int32), ("max_depth", ctypes.c_int32),
                ("stop_row", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p), ("num_out", ctypes.c_void_p),
                ("key_row", ctypes.c_void_p), ("key_token", ctypes.c_void_p), ("n_keys", ctypes.c_void_p),
                ("prepared", ctypes.c_void_p), ("hit", ctypes.c_void_p), ("branch", ctypes.c_void_p),
                ("next_tokens", ctypes.c_void_p), ("n_hits", ctypes.c_void_p)]


EXPORTS = ["sv_build_tree_mask", "sv_tree_attention_workspace", "sv_tree_attention", "sv_accept_workspace",
           "sv_accept", "sv_accept_noalloc", "sv_kv_commit", "sv_verify_step_workspace", "sv_verify_step", "sv_outcome_lookup", "sv_saguaro_reweight", "sv_draft_subset_logits",
           "sv_status_string", "sv_version"]


def lib():
    """Load libspecverify.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SpecVerifyError("libspecverify.so is not built: run __graft_entry__.build() or "
                                  "tree_verification_sv_amd.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        L.sv_build_tree_mask.argtypes = [P, i32, i32, i32, P, P, P, P, ctypes.c_uint32, P]
        L.sv_build_tree_mask.restype = i32
        L.sv_tree_attention_workspace.argtypes = [ctypes.POINTER(sv_attn_args)]
        L.sv_tree_attention_workspace.restype = ctypes.c_size_t
        L.sv_tree_attention.argtypes = [ctypes.POINTER(sv_attn_args), P]
        L.sv_tree_attention.restype = i32
        L.sv_accept_workspace.argtypes = [ctypes.POINTER(sv_accept_args)]
        L.sv_accept_workspace.restype = ctypes.c_size_t
        L.sv_accept.argtypes = [ctypes.POINTER(sv_accept_args), P]
        L.sv_accept.restype = i32
        L.sv_accept_noalloc.argtypes = [ctypes.POINTER(sv_accept_args), P]
        L.sv_accept_noalloc.restype = i32
        L.sv_kv_commit.argtypes = [ctypes.POINTER(sv_commit_args), P]
        L.sv_kv_commit.restype = i32
        L.sv_verify_step_workspace.argtypes = [ctypes.POINTER(sv_step_args)]
        L.sv_verify_step_workspace.restype = ctypes.c_size_t
        L.sv_verify_step.argtypes = [ctypes.POINTER(sv_step_args), P]
        L.sv_verify_step.restype = i32
        L.sv_outcome_lookup.argtypes = [ctypes.POINTER(sv_outcome_args), P]
        L.sv_outcome_lookup.restype = i32
        L.sv_saguaro_reweight.argtypes = [P, i32, i32, i32, i32, P, i32, ctypes.c_float, P]
        L.sv_saguaro_reweight.restype = i32
        L.sv_draft_subset_logits.argtypes = [P, i32, i32, i32, P, i32, i32, P, P]
        L.sv_draft_subset_logits.restype = i32
        L.sv_status_string.argtypes = [i32]
        L.sv_status_string.restype = ctypes.c_char_p
        L.sv_version.argtypes = []
        L.sv_version.restype = i32
        _lib = L
    return _lib


# ------------------------------------------------------------ marshalling helpers
def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda:
        raise SpecVerifyError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise SpecVerifyError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise SpecVerifyError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _check(rc, what):
    if rc != SV_OK:
        msg = lib().sv_status_string(rc).decode()
        raise SpecVerifyError(f"{what} returned {rc} ({msg})")


def _elem(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise SpecVerifyError(f"unsupported element type {t.dtype}")


def _alloc_workspace(nbytes, device):
    torch = _torch()
    if nbytes == 0:
        return None
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------ entry points
def sv_build_tree_mask(parents, max_depth: int, out: Optional[dict] = None, stream=None, validate=False) -> dict:
    """parents [B,N] int32 -> dict(anc_bits [B,N,W] int64 (uint64 bits), depth, path_rows, status).

    validate: reference mode (SV_FLAG_VALIDATE) -- the call waits and raises on a malformed tree."""
    torch = _torch()
    B, N = parents.shape
    W = (N + 63) // 64
    dev = parents.device
    if out is None:
        out = dict(anc_bits=torch.empty((B, N, W), dtype=torch.int64, device=dev),
                   depth=torch.empty((B, N), dtype=torch.int32, device=dev),
                   path_rows=torch.empty((B, N + 1, max_depth), dtype=torch.int32, device=dev),
                   status=torch.empty((B,), dtype=torch.int32, device=dev))
    rc = lib().sv_build_tree_mask(_ptr(parents, torch.int32, "parents"), B, N, max_depth,
                                  _ptr(out["anc_bits"], torch.int64, "anc_bits"), _ptr(out["depth"], torch.int32),
                                  _ptr(out.get("path_rows"), torch.int32), _ptr(out["status"], torch.int32),
                                  SV_FLAG_VALIDATE if validate else 0, _stream(stream))
    _check(rc, "sv_build_tree_mask")
    return out


def attn_args(q, k_cache, v_cache, k_tree, v_tree, anc_bits, prefix_len, out, block_table=None, scale=None,
              paged=False, num_blocks=0, status=None, tree_in_cache=False) -> sv_attn_args:
    torch = _torch()
    B, N, Hq, D = q.shape
    Hkv = k_cache.shape[1]  # [B,Hkv,Lcap,D] or [num_blocks,Hkv,bs,D]
    a = sv_attn_args()
    a.B, a.N, a.Hq, a.Hkv, a.D = B, N, Hq, Hkv, D
    a.dtype = _elem(q)
    a.scale = float(1.0 / (D ** 0.5)) if scale is None else float(scale)
    a.paged = int(bool(paged))
    if paged:
        a.Lcap = 0
        a.block_size = k_cache.shape[2]
        a.max_blocks = block_table.shape[1]
        a.num_blocks = num_blocks or k_cache.shape[0]
    else:
        a.Lcap = k_cache.shape[2]
        a.block_size, a.max_blocks, a.num_blocks = 16, 0, 0
    a.tree_in_cache = int(bool(tree_in_cache))
    if tree_in_cache:
        k_tree = v_tree = None  # the tree rows are cache positions prefix_len + t
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_tree, "k_tree"), (v_tree, "v_tree"), (out, "out")):
        if t is not None and t.dtype != q.dtype:
            raise SpecVerifyError(f"{nm} dtype {t.dtype} differs from q dtype {q.dtype}")
    a.q, a.k_cache, a.v_cache = _ptr(q, name="q"), _ptr(k_cache, name="k_cache"), _ptr(v_cache, name="v_cache")
    a.k_tree, a.v_tree = _ptr(k_tree, name="k_tree"), _ptr(v_tree, name="v_tree")
    a.block_table = _ptr(block_table, torch.int32, "block_table")
    a.prefix_len = _ptr(prefix_len, torch.int32, "prefix_len")
    a.anc_bits = _ptr(anc_bits, torch.int64, "anc_bits")
    a.out = _ptr(out, name="out")
    a.status = _ptr(status, torch.int32, "status")
    return a


def sv_tree_attention_workspace(args: sv_attn_args) -> int:
    return int(lib().sv_tree_attention_workspace(ctypes.byref(args)))


def sv_tree_attention(q, k_cache, v_cache, k_tree, v_tree, anc_bits, prefix_len, block_table=None, scale=None,
                      paged=False, num_blocks=0, out=None, workspace=None, status=None, stream=None,
                      tree_in_cache=False):
    """Ancestor-masked GQA tree attention; returns out [B,N,Hq,D] (dtype of q).

    tree_in_cache: node t's K/V is cache position prefix_len + t (k_tree / v_tree ignored)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    a = attn_args(q, k_cache, v_cache, k_tree, v_tree, anc_bits, prefix_len, out, block_table, scale, paged,
                  num_blocks, status, tree_in_cache)
    need = sv_tree_attention_workspace(a)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = _alloc_workspace(need, q.device)
    a.workspace = _ptr(workspace) if need else None
    a.workspace_bytes = need
    _check(lib().sv_tree_attention(ctypes.byref(a), _stream(stream)), "sv_tree_attention")
    return out


def accept_args(parents, tokens, anc_bits, depth, target_logits, max_depth, mode, draft_logits=None,
                u_accept=None, u_sample=None, temperature=1.0, outs=None, threshold=0.0, flags=0) -> sv_accept_args:
    torch = _torch()
    B, N = parents.shape
    V = target_logits.shape[-1]
    a = sv_accept_args()
    a.B, a.N, a.V, a.max_depth = B, N, V, max_depth
    a.logits_dtype = _elem(target_logits)
    if mode in _MODES:
        mode = _MODES[mode]
    if mode not in _MODES.values():
        raise SpecVerifyError(f"unknown acceptance mode {mode!r}")
    a.mode = mode
    a.temperature = float(temperature)
    a.threshold = float(threshold)
    a.flags = int(flags)
    a.parents, a.tokens = _ptr(parents, torch.int32, "parents"), _ptr(tokens, torch.int32, "tokens")
    a.anc_bits, a.depth = _ptr(anc_bits, torch.int64, "anc_bits"), _ptr(depth, torch.int32, "depth")
    a.target_logits = _ptr(target_logits, name="target_logits")
    if a.mode == SV_STOCHASTIC:
        if draft_logits.dtype != target_logits.dtype:
            raise SpecVerifyError("draft and target logits must share a dtype")
        a.draft_logits = _ptr(draft_logits, name="draft_logits")
    if a.mode in (SV_STOCHASTIC, SV_TOPK_DRAFT):
        a.u_accept = _ptr(u_accept, torch.float32, "u_accept")
        a.u_sample = _ptr(u_sample, torch.float32, "u_sample")
    for k in ("accept_len", "accept_rows", "out_tokens", "num_out", "stop_row", "status"):
        setattr(a, k, _ptr(outs[k], torch.int32, k))
    return a


def accept_outputs(B, max_depth, device):
    torch = _torch()
    return dict(accept_len=torch.empty(B, dtype=torch.int32, device=device),
                accept_rows=torch.empty((B, max_depth), dtype=torch.int32, device=device),
                out_tokens=torch.empty((B, max_depth + 1), dtype=torch.int32, device=device),
                num_out=torch.empty(B, dtype=torch.int32, device=device),
                stop_row=torch.empty(B, dtype=torch.int32, device=device),
                status=torch.empty(B, dtype=torch.int32, device=device))


def sv_accept_workspace(args: sv_accept_args) -> int:
    return int(lib().sv_accept_workspace(ctypes.byref(args)))


def sv_accept(parents, tokens, anc_bits, depth, target_logits, max_depth, mode="greedy", draft_logits=None,
              u_accept=None, u_sample=None, temperature=1.0, outs=None, workspace=None, stream=None,
              threshold=0.0, validate=False, row_list=False) -> dict:
    """Speculative acceptance + bonus token; returns the dict of int32 device outputs.

    validate: reference mode (SV_FLAG_VALIDATE) -- logits rows are scanned for non-finite values and
    the call waits and raises SpecVerifyError when a sequence reports a non-zero status.
    row_list: SV_FLAG_ROW_LIST -- greedy and threshold batches resolve every needed row instead of
    following the accepted paths (same results)."""
    B = parents.shape[0]
    if outs is None:
        outs = accept_outputs(B, max_depth, parents.device)
    a = accept_args(parents, tokens, anc_bits, depth, target_logits, max_depth, mode, draft_logits, u_accept,
                    u_sample, temperature, outs, threshold,
                    (SV_FLAG_VALIDATE if validate else 0) | (SV_FLAG_ROW_LIST if row_list else 0))
    need = sv_accept_workspace(a)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = _alloc_workspace(need, parents.device)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = need
    _check(lib().sv_accept(ctypes.byref(a), _stream(stream)), "sv_accept")
    return outs


def commit_args(k_cache, v_cache, k_tree, v_tree, prefix_len, accept_len, accept_rows, max_depth, new_len,
                committed_slots, status, block_table=None, paged=False, num_blocks=0,
                commit_mode=SV_COMMIT_PATH, tree_in_cache=False, N=None, num_layers=1) -> sv_commit_args:
    """num_layers > 1: k_cache / v_cache (and k_tree / v_tree) carry a leading layer dimension.
    tree_in_cache: the tree rows are cache positions prefix_len + t; N must be given."""
    torch = _torch()
    layered = num_layers > 1
    kc1 = k_cache[0] if layered else k_cache  # one layer's cache
    B = prefix_len.shape[0]
    Hkv, D = kc1.shape[1], kc1.shape[3]
    if tree_in_cache:
        if N is None:
            raise SpecVerifyError("tree_in_cache needs the tree size N")
        k_tree = v_tree = None
    else:
        kt1 = k_tree[0] if layered else k_tree
        N = kt1.shape[2] - 1
    a = sv_commit_args()
    a.B, a.N, a.Hkv, a.D = B, N, Hkv, D
    a.dtype = _elem(k_cache)
    a.max_depth, a.commit_mode = max_depth, commit_mode
    a.paged = int(bool(paged))
    if paged:
        a.Lcap, a.block_size, a.max_blocks = 0, kc1.shape[2], block_table.shape[1]
        a.num_blocks = num_blocks or kc1.shape[0]
    else:
        a.Lcap, a.block_size, a.max_blocks, a.num_blocks = kc1.shape[2], 16, 0, 0
    a.tree_in_cache = int(bool(tree_in_cache))
    a.num_layers = num_layers
    if layered:
        a.cache_layer_stride = kc1.numel()
        a.tree_layer_stride = 0 if tree_in_cache else k_tree[0].numel()
    for t, nm in ((v_cache, "v_cache"), (k_tree, "k_tree"), (v_tree, "v_tree")):
        if t is not None and t.dtype != k_cache.dtype:
            raise SpecVerifyError(f"{nm} dtype {t.dtype} differs from k_cache dtype {k_cache.dtype}")
    a.k_cache, a.v_cache = _ptr(k_cache, name="k_cache"), _ptr(v_cache, name="v_cache")
    a.block_table = _ptr(block_table, torch.int32, "block_table")
    a.k_tree, a.v_tree = _ptr(k_tree, name="k_tree"), _ptr(v_tree, name="v_tree")
    a.prefix_len = _ptr(prefix_len, torch.int32, "prefix_len")
    a.accept_len = _ptr(accept_len, torch.int32, "accept_len")
    a.accept_rows = _ptr(accept_rows, torch.int32, "accept_rows")
    a.new_len = _ptr(new_len, torch.int32, "new_len")
    a.committed_slots = _ptr(committed_slots, torch.int32, "committed_slots")
    a.status = _ptr(status, torch.int32, "status")
    return a


def sv_kv_commit(k_cache, v_cache, k_tree, v_tree, prefix_len, accept_len, accept_rows, max_depth,
                 block_table=None, paged=False, num_blocks=0, commit_mode=SV_COMMIT_PATH, outs=None,
                 stream=None, tree_in_cache=False, N=None, num_layers=1) -> dict:
    """Commit the accepted rows into the caches in place; returns new_len, committed_slots, status."""
    torch = _torch()
    B = prefix_len.shape[0]
    dev = k_cache.device
    if outs is None:
        outs = dict(new_len=torch.empty(B, dtype=torch.int32, device=dev),
                    committed_slots=torch.empty((B, max_depth), dtype=torch.int32, device=dev),
                    status=torch.empty(B, dtype=torch.int32, device=dev))
    a = commit_args(k_cache, v_cache, k_tree, v_tree, prefix_len, accept_len, accept_rows, max_depth,
                    outs["new_len"], outs["committed_slots"], outs["status"], block_table, paged, num_blocks,
                    commit_mode, tree_in_cache, N, num_layers)
    _check(lib().sv_kv_commit(ctypes.byref(a), _stream(stream)), "sv_kv_commit")
    return outs


def sv_outcome_lookup(stop_row, out_tokens, num_out, key_row, key_token, n_keys, prepared=None, outs=None,
                      stream=None) -> dict:
    """SSD outcome lookup on device; returns hit, branch (k+1 or 0), next_tokens (or None), n_hits."""
    torch = _torch()
    B, K = key_row.shape
    Dm = out_tokens.shape[1] - 1
    P = 0 if prepared is None else prepared.shape[2]
    dev = key_row.device
    if outs is None:
        outs = dict(hit=torch.empty(B, dtype=torch.int32, device=dev),
                    branch=torch.empty(B, dtype=torch.int32, device=dev),
                    next_tokens=torch.empty((B, P), dtype=torch.int32, device=dev) if P else None,
                    n_hits=torch.empty(1, dtype=torch.int32, device=dev))
    a = sv_outcome_args()
    a.B, a.K, a.P, a.max_depth = B, K, P, Dm
    i32 = torch.int32
    a.stop_row, a.out_tokens, a.num_out = (_ptr(stop_row, i32, "stop_row"), _ptr(out_tokens, i32, "out_tokens"),
                                           _ptr(num_out, i32, "num_out"))
    a.key_row, a.key_token, a.n_keys = (_ptr(key_row, i32, "key_row"), _ptr(key_token, i32, "key_token"),
                                        _ptr(n_keys, i32, "n_keys"))
    a.prepared = _ptr(prepared, i32, "prepared")
    a.hit, a.branch = _ptr(outs["hit"], i32, "hit"), _ptr(outs["branch"], i32, "branch")
    a.next_tokens = _ptr(outs.get("next_tokens"), i32, "next_tokens")
    a.n_hits = _ptr(outs.get("n_hits"), i32, "n_hits")
    _check(lib().sv_outcome_lookup(ctypes.byref(a), _stream(stream)), "sv_outcome_lookup")
    return outs


def sv_saguaro_reweight(draft_logits, cache_tokens, shift: float, stream=None):
    """In-place Saguaro reweighting of draft_logits [B,R,V] at the tokens cache_tokens [B,R,C]."""
    torch = _torch()
    B, R, V = draft_logits.shape
    C = cache_tokens.shape[2]
    rc = lib().sv_saguaro_reweight(_ptr(draft_logits, name="draft_logits"), B, R, V, _elem(draft_logits),
                                   _ptr(cache_tokens, torch.int32, "cache_tokens"), C, float(shift), _stream(stream))
    _check(rc, "sv_saguaro_reweight")
    return draft_logits


def sv_draft_subset_logits(sub_logits, t2d, out=None, stream=None):
    """Full-vocabulary draft logits [B,R,V] from subset logits [B,R,Vd] and t2d [V] (j+1, 0 = absent)."""
    torch = _torch()
    B, R, Vd = sub_logits.shape
    V = t2d.shape[0]
    if out is None:
        out = torch.empty((B, R, V), dtype=sub_logits.dtype, device=sub_logits.device)
    if out.dtype != sub_logits.dtype:
        raise SpecVerifyError("out and sub_logits must share a dtype")
    rc = lib().sv_draft_subset_logits(_ptr(sub_logits, name="sub_logits"), B, R, Vd, _ptr(t2d, torch.int32, "t2d"),
                                      V, _elem(sub_logits), _ptr(out, name="out"), _stream(stream))
    _check(rc, "sv_draft_subset_logits")
    return out


def sv_status_string(code: int) -> str:
    return lib().sv_status_string(code).decode()


def sv_version() -> int:
    return int(lib().sv_version())
