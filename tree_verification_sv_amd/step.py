"""One verification step: the library calls in dependency order.

``VerifyStep`` owns the output and workspace buffers (allocated once through
torch), so repeated ``run()`` calls allocate nothing and issue the C-ABI calls
sv_build_tree_mask -> sv_tree_attention -> sv_accept -> sv_kv_commit, or, after
``fuse_commit()``, three calls with the commit done inside sv_accept.  Nothing
here computes; it marshals arguments and orders streams.

Attention and acceptance both read only the mask outputs and the step's
inputs, and the commit writes cache slots at positions >= prefix_len, which
the attention never reads.  ``run(overlap=True)`` therefore forks after the
mask: acceptance and commit go to a side stream while the attention runs on
the caller's stream, and the caller's stream waits for the side stream at the
end (a fork/join that HIP graph capture records as a DAG).  The attention is
issued first by default (``accept_first=False``): measured on MI355X, the step
is shorter when the attention's work-groups take the compute units first and
the acceptance fills them as they free up.  With the tree rows in the cache the
commit moves rows the attention reads, so it follows the join.  Stochastic
acceptance over wide trees of many rows is faster without the fork: most of
its row groups leave at their start once their sequence's walk has finished,
and those dispatches beside the attention slow both.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

from . import (SV_COMMIT_PATH, SV_GREEDY, SV_STOCHASTIC, SV_TOPK_DRAFT, _check, _stream, accept_args, accept_outputs, attn_args,
               commit_args, lib, sv_accept_workspace, sv_step_args, sv_tree_attention_workspace)


@dataclass
class StepInputs:
    """Device tensors of one verification batch (see include/specverify.h for layouts)."""
    parents: object
    tokens: object
    q: object
    k_cache: object
    v_cache: object
    k_tree: object
    v_tree: object
    prefix_len: object
    target_logits: object
    max_depth: int
    mode: str = "greedy"
    temperature: float = 1.0
    draft_logits: Optional[object] = None
    u_accept: Optional[object] = None
    u_sample: Optional[object] = None
    block_table: Optional[object] = None
    paged: bool = False
    num_blocks: int = 0
    scale: Optional[float] = None
    commit_mode: int = SV_COMMIT_PATH
    tree_in_cache: bool = False  # tree K/V rows are cache positions prefix_len + t (k_tree / v_tree unused)
    threshold: float = 0.0       # acceptance threshold of mode "threshold"


class VerifyStep:
    def __init__(self, x: StepInputs):
        import torch
        self.x = x
        B, N = x.parents.shape
        dev = x.parents.device
        W = (N + 63) // 64
        Dm = x.max_depth
        self.B, self.N = B, N
        self.mask = dict(anc_bits=torch.empty((B, N, W), dtype=torch.int64, device=dev),
                         depth=torch.empty((B, N), dtype=torch.int32, device=dev),
                         path_rows=torch.empty((B, N + 1, Dm), dtype=torch.int32, device=dev),
                         status=torch.empty((B,), dtype=torch.int32, device=dev))
        self.out = torch.empty_like(x.q)
        self.attn_status = torch.empty((B,), dtype=torch.int32, device=dev)
        self.acc = accept_outputs(B, Dm, dev)
        self.commit = dict(new_len=torch.empty(B, dtype=torch.int32, device=dev),
                           committed_slots=torch.empty((B, Dm), dtype=torch.int32, device=dev),
                           status=torch.empty(B, dtype=torch.int32, device=dev))
        # argument blocks are built once; pointers stay valid for the tensors' lifetime
        self._attn = attn_args(x.q, x.k_cache, x.v_cache, x.k_tree, x.v_tree, self.mask["anc_bits"], x.prefix_len,
                               self.out, x.block_table, x.scale, x.paged, x.num_blocks, self.attn_status,
                               x.tree_in_cache)
        need = sv_tree_attention_workspace(self._attn)
        self.attn_ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self._attn.workspace = self.attn_ws.data_ptr() if need else None
        self._attn.workspace_bytes = need
        self._acc = accept_args(x.parents, x.tokens, self.mask["anc_bits"], self.mask["depth"], x.target_logits, Dm,
                                x.mode, x.draft_logits, x.u_accept, x.u_sample, x.temperature, self.acc,
                                x.threshold)
        need = sv_accept_workspace(self._acc)
        self.acc_ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)  # counters start at zero
        self._acc.workspace = self.acc_ws.data_ptr()
        self._acc.workspace_bytes = need
        self._com = commit_args(x.k_cache, x.v_cache, x.k_tree, x.v_tree, x.prefix_len, self.acc["accept_len"],
                                self.acc["accept_rows"], Dm, self.commit["new_len"], self.commit["committed_slots"],
                                self.commit["status"], x.block_table, x.paged, x.num_blocks, x.commit_mode,
                                x.tree_in_cache, N)
        self._L = lib()
        self._one = None  # sv_step_args of the one-launch step (see one_launch())
        self._fused = False
        self._mask_free = False
        self._side = None
        self._ev_fork = self._ev_join = None

    def _side_stream(self):
        import torch
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.x.parents.device)  # default priority
            self._ev_fork = torch.cuda.Event()
            self._ev_join = torch.cuda.Event()
        return self._side

    # individual stages (same stream)
    def build_mask(self, stream=None):
        m = self.mask
        _check(self._L.sv_build_tree_mask(self.x.parents.data_ptr(), self.B, self.N, self.x.max_depth,
                                          m["anc_bits"].data_ptr(), m["depth"].data_ptr(), m["path_rows"].data_ptr(),
                                          m["status"].data_ptr(), 0, _stream(stream)), "sv_build_tree_mask")

    def attention(self, stream=None):
        _check(self._L.sv_tree_attention(ctypes.byref(self._attn), _stream(stream)), "sv_tree_attention")

    def accept(self, stream=None):
        _check(self._L.sv_accept(ctypes.byref(self._acc), _stream(stream)), "sv_accept")

    def kv_commit(self, stream=None):
        if self._fused:  # done by the acceptance kernel
            return
        _check(self._L.sv_kv_commit(ctypes.byref(self._com), _stream(stream)), "sv_kv_commit")

    def fuse_commit(self, on: bool = True):
        """Let the acceptance kernel commit the accepted path itself (one launch less); kv_commit()
        and run() then skip the separate commit.  Not with the tree rows in the cache."""
        if on and self.x.tree_in_cache:
            raise ValueError("the fused commit needs the tree rows in their own tensor")
        self._acc.commit = ctypes.addressof(self._com) if on else None
        self._fused = on

    def mask_free_accept(self, on: bool = True):
        """Let the acceptance derive node depths from the parent array itself (every mode but
        "threshold": sv_accept gets NULL anc_bits and depth), so that it does not wait for the
        mask; run(overlap=True) then forks before the mask and the acceptance branch starts at once."""
        if on and self._acc.mode not in (SV_GREEDY, SV_STOCHASTIC, SV_TOPK_DRAFT):
            raise ValueError("threshold acceptance needs the mask outputs")
        self._acc.anc_bits = None if on else self.mask["anc_bits"].data_ptr()
        self._acc.depth = None if on else self.mask["depth"].data_ptr()
        self._mask_free = on

    def one_launch(self, on: bool = True, mask_outputs: bool = True):
        """Run the step as one sv_verify_step launch: the mask (written to self.mask when
        mask_outputs), the attention, the acceptance and -- after fuse_commit() -- the commit.
        Returns False (and stays off) when the call does not support these arguments."""
        import torch
        if not on:
            self._one = None
            return False
        a = sv_step_args()
        a.attn = ctypes.addressof(self._attn)
        a.accept = ctypes.addressof(self._acc)
        if mask_outputs:
            m = self.mask
            a.anc_bits, a.depth = m["anc_bits"].data_ptr(), m["depth"].data_ptr()
            a.path_rows, a.mask_status = m["path_rows"].data_ptr(), m["status"].data_ptr()
        need = int(self._L.sv_verify_step_workspace(ctypes.byref(a)))
        if need == 0:
            self._one = None
            return False
        self.step_ws = torch.zeros(need, dtype=torch.uint8, device=self.x.parents.device)  # counters start at zero
        a.workspace, a.workspace_bytes = self.step_ws.data_ptr(), need
        self._one = a
        return True

    def run(self, stream=None, overlap=False, accept_first=False, attention_side=False):
        if self._one is not None:  # the whole step in one launch (stream order only)
            _check(self._L.sv_verify_step(ctypes.byref(self._one), _stream(stream)), "sv_verify_step")
            if not self._fused:
                self.kv_commit(stream)
            return
        if overlap and self._com.new_len == self._attn.prefix_len:
            # the commit beside the attention writes new_len while the attention reads prefix_len
            raise ValueError("new_len must not alias prefix_len when the commit overlaps the attention")
        if not overlap:
            self.build_mask(stream)
            self.attention(stream)
            self.accept(stream)
            self.kv_commit(stream)
            return
        import torch
        main = stream if stream is not None else torch.cuda.current_stream()
        side = self._side_stream()
        # with the tree rows in the cache the commit moves rows the attention reads,
        # so it follows the join instead of running beside the attention
        late_commit = self.x.tree_in_cache
        if self._mask_free:
            # the acceptance reads no mask output: its branch forks before the mask
            self._ev_fork.record(main)
            side.wait_event(self._ev_fork)
            self.accept(side)
            if not late_commit:
                self.kv_commit(side)
            self.build_mask(main)
            self.attention(main)
            self._ev_join.record(side)
            main.wait_event(self._ev_join)
            if late_commit:
                self.kv_commit(main)
            return
        self.build_mask(main)
        self._ev_fork.record(main)
        side.wait_event(self._ev_fork)
        if attention_side and not late_commit:
            # acceptance -> commit stay on the caller's stream right after the mask (no
            # cross-stream wait on the longer branch); the attention takes the side stream
            self.attention(side)
            self.accept(main)
            self.kv_commit(main)
        elif accept_first:
            self.accept(side)
            if not late_commit:
                self.kv_commit(side)
            self.attention(main)
        else:
            self.attention(main)
            self.accept(side)
            if not late_commit:
                self.kv_commit(side)
        self._ev_join.record(side)
        main.wait_event(self._ev_join)
        if late_commit:
            self.kv_commit(main)
