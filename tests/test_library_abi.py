"""CPU checks of the C-ABI library: it loads, exports every declared symbol, and
rejects bad arguments synchronously (no GPU needed: nothing is launched)."""
import ctypes
import os
import re

import pytest

import tree_verification_sv_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "specverify.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("sv_build_tree_mask", "sv_tree_attention", "sv_accept", "sv_kv_commit"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sv.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(sv.EXPORTS) == set(_declared())


def test_bad_arguments_rejected_without_launch():
    L = sv.lib()
    # N = 0, max_depth = 0 and N > 256 are argument errors
    assert L.sv_build_tree_mask(None, 1, 0, 4, None, None, None, None, 0, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert L.sv_build_tree_mask(None, 1, 4, 0, None, None, None, None, 0, None) == sv.SV_ERR_INVALID_ARGUMENT
    assert L.sv_build_tree_mask(None, 1, 257, 4, None, None, None, None, 0, None) == sv.SV_ERR_INVALID_ARGUMENT
    # B = 0 is a no-op
    assert L.sv_build_tree_mask(None, 0, 4, 4, None, None, None, None, 0, None) == sv.SV_OK
    a = sv.sv_attn_args()
    a.B, a.N, a.Hq, a.Hkv, a.D, a.dtype, a.scale = 1, 4, 8, 3, 128, sv.SV_BF16, 0.088
    assert L.sv_tree_attention(ctypes.byref(a), None) == sv.SV_ERR_INVALID_ARGUMENT  # Hq % Hkv
    a.Hkv, a.D = 2, 96
    assert L.sv_tree_attention(ctypes.byref(a), None) == sv.SV_ERR_UNSUPPORTED
    a.D = 128
    assert L.sv_tree_attention(ctypes.byref(a), None) == sv.SV_ERR_INVALID_ARGUMENT  # null pointers
    acc = sv.sv_accept_args()
    acc.B, acc.N, acc.V, acc.max_depth, acc.mode = 1, 4, 10, 17, 0
    assert L.sv_accept(ctypes.byref(acc), None) == sv.SV_ERR_INVALID_ARGUMENT
    acc.max_depth, acc.mode = 4, 1
    assert L.sv_accept(ctypes.byref(acc), None) == sv.SV_ERR_INVALID_ARGUMENT  # null pointers
    c = sv.sv_commit_args()
    c.B, c.N, c.Hkv, c.D, c.dtype, c.max_depth, c.commit_mode = 1, 4, 2, 64, sv.SV_F32, 4, 7
    assert L.sv_kv_commit(ctypes.byref(c), None) == sv.SV_ERR_INVALID_ARGUMENT
    assert sv.sv_status_string(sv.SV_ERR_UNSUPPORTED) == "unsupported shape or type"


def test_workspace_queries():
    a = sv.sv_attn_args()
    a.B, a.N, a.Hq, a.Hkv, a.D, a.dtype, a.scale = 1, 60, 32, 8, 128, sv.SV_BF16, 0.088
    a.Lcap = 4112
    n = sv.sv_tree_attention_workspace(a)
    assert n % 4 == 0 and n > 0  # batch-1 tree splits the prefix, so partials are needed
    a.dtype = sv.SV_F32
    assert sv.sv_tree_attention_workspace(a) == 0
    acc = sv.sv_accept_args()
    acc.B, acc.N, acc.V = 2, 60, 128256
    small = sv.sv_accept_workspace(acc)
    acc.B = 64
    big = sv.sv_accept_workspace(acc)
    assert small % 256 == 0 and big > small  # per-row results and per-sequence counters grow with B
    assert big - small >= 62 * 61 * 8 - 512  # up to 256-byte alignment of each region


def test_no_product_module_imports_the_oracle():
    """The product package and the bench's GPU path never import the oracle."""
    pkg = os.path.join(ROOT, "tree_verification_sv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "oracle." not in txt.replace("the oracle", ""), f


def test_tree_in_cache_and_layer_arguments_rejected_without_launch():
    L = sv.lib()
    a = sv.sv_attn_args()
    a.B, a.N, a.Hq, a.Hkv, a.D, a.dtype, a.scale = 1, 60, 32, 8, 128, sv.SV_BF16, 0.088
    a.Lcap, a.tree_in_cache = 59, 1  # the cache cannot hold the tree rows
    assert L.sv_tree_attention(ctypes.byref(a), None) == sv.SV_ERR_INVALID_ARGUMENT
    a.tree_in_cache = 2
    assert L.sv_tree_attention(ctypes.byref(a), None) == sv.SV_ERR_INVALID_ARGUMENT
    a.Lcap, a.tree_in_cache = 4160, 1  # valid shape, but no pointers
    assert L.sv_tree_attention(ctypes.byref(a), None) == sv.SV_ERR_INVALID_ARGUMENT
    assert sv.sv_tree_attention_workspace(a) > 0
    c = sv.sv_commit_args()
    c.B, c.N, c.Hkv, c.D, c.dtype, c.max_depth, c.commit_mode, c.Lcap = 1, 4, 2, 64, sv.SV_F32, 4, 0, 64
    c.num_layers = 3  # several layers need positive layer strides
    assert L.sv_kv_commit(ctypes.byref(c), None) == sv.SV_ERR_INVALID_ARGUMENT
    c.cache_layer_stride, c.tree_layer_stride = 1 << 20, 0
    assert L.sv_kv_commit(ctypes.byref(c), None) == sv.SV_ERR_INVALID_ARGUMENT
    c.tree_in_cache = 1  # the tree stride is not needed with the rows in the cache; pointers still are
    assert L.sv_kv_commit(ctypes.byref(c), None) == sv.SV_ERR_INVALID_ARGUMENT
    c.num_layers = -1
    assert L.sv_kv_commit(ctypes.byref(c), None) == sv.SV_ERR_INVALID_ARGUMENT


def test_accept_without_mask_outputs_only_in_walk_modes():
    """NULL anc_bits and depth are allowed in modes 0, 1 and 2 (depths and root paths derived in
    the kernel); threshold acceptance reads the mask outputs and rejects them before any launch."""
    L = sv.lib()
    acc = sv.sv_accept_args()
    acc.B, acc.N, acc.V, acc.max_depth, acc.temperature, acc.threshold = 1, 4, 10, 4, 1.0, 0.5
    acc.logits_dtype = sv.SV_F32
    fake = 1 << 20  # never dereferenced: the call returns before any launch
    for k in ("parents", "tokens", "target_logits", "draft_logits", "u_accept", "u_sample", "accept_len",
              "accept_rows", "out_tokens", "num_out", "stop_row", "status", "workspace"):
        setattr(acc, k, fake)
    acc.workspace_bytes = 1 << 20
    for mode in (sv.SV_THRESHOLD,):
        acc.mode = mode
        acc.anc_bits, acc.depth = None, None
        assert L.sv_accept(ctypes.byref(acc), None) == sv.SV_ERR_INVALID_ARGUMENT
        acc.anc_bits = fake
        assert L.sv_accept(ctypes.byref(acc), None) == sv.SV_ERR_INVALID_ARGUMENT  # depth still NULL
