"""Seeded synthetic workloads for tree speculative-decoding verification.

This module only draws inputs: trees (parent arrays), draft tokens, logits,
queries, KV caches, block tables and the uniforms the acceptance rule consumes.
It holds none of the verification arithmetic, so the CPU oracle and the GPU
library can both be fed from it without sharing any computation.

Every random quantity comes from the counter-based SplitMix64 streams of
``svgen.c`` keyed by (seed, stream id), so any tensor is reproducible from the
seed alone.  bf16 tensors are returned as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsvgen.so")
_lib = None

# stream ids: one per tensor role
S_TREE, S_TOKENS, S_Q, S_KC, S_VC, S_KT, S_VT = 1, 2, 3, 4, 5, 6, 7
S_TGT, S_DRF, S_PERT, S_UACC, S_USMP, S_PLEN, S_PERM, S_PLANT = 8, 9, 10, 11, 12, 13, 14, 15
S_KC2, S_VC2 = 16, 17  # cache positions added when the tree rows move into the cache

VOCAB_LLAMA3 = 128256


def build(force: bool = True) -> str:
    """Compile libsvgen.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "svgen.c")
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        u64, i64, d, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.svg_stream_key.argtypes = [u64, u64]
        lib.svg_stream_key.restype = u64
        lib.svg_u64.argtypes = [u64, u64, u64, i64, p]
        lib.svg_uniform24_f32.argtypes = [u64, u64, u64, i64, p]
        lib.svg_normal_f32.argtypes = [u64, u64, u64, i64, d, d, p]
        lib.svg_normal_bf16.argtypes = [u64, u64, u64, i64, d, d, p]
        lib.svg_perturb_bf16.argtypes = [u64, u64, i64, p, d, p]
        lib.svg_perturb_f32.argtypes = [u64, u64, i64, p, d, p]
        lib.svg_draft_tokens.argtypes = [u64, u64, p, ctypes.c_int, i64, p, i64, d, p]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- raw draws
def u64(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    if n:
        _L().svg_u64(seed, stream, offset, n, _ptr(out))
    return out


def uniform24(seed: int, stream: int, shape, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    if out.size:
        _L().svg_uniform24_f32(seed, stream, offset, out.size, _ptr(out))
    return out


def normal(seed: int, stream: int, shape, dtype: str, sigma: float = 1.0, mean: float = 0.0,
           offset: int = 0) -> np.ndarray:
    """mean + sigma*N(0,1); dtype 'f32' -> float32, 'bf16' -> uint16 bit patterns."""
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        if out.size:
            _L().svg_normal_f32(seed, stream, offset, out.size, mean, sigma, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        if out.size:
            _L().svg_normal_bf16(seed, stream, offset, out.size, mean, sigma, _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def perturb(seed: int, stream: int, base: np.ndarray, sigma: float) -> np.ndarray:
    """dtype-preserving base + sigma*N(0,1), rounded to the base's dtype."""
    base = np.ascontiguousarray(base)
    out = np.empty_like(base)
    if base.dtype == np.uint16:
        _L().svg_perturb_bf16(seed, stream, base.size, _ptr(base), sigma, _ptr(out))
    elif base.dtype == np.float32:
        _L().svg_perturb_f32(seed, stream, base.size, _ptr(base), sigma, _ptr(out))
    else:
        raise ValueError(base.dtype)
    return out


def draft_tokens(seed: int, stream: int, logits: np.ndarray, rows: np.ndarray, T: float) -> np.ndarray:
    """One drafted token per requested row of ``logits`` viewed as [R, V].

    T > 0 samples from softmax(logits/T) (Gumbel-max); T <= 0 is greedy drafting
    (argmax, lowest id on ties).
    """
    logits = np.ascontiguousarray(logits)
    V = logits.shape[-1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty(rows.size, dtype=np.int32)
    dt = 0 if logits.dtype == np.float32 else 1
    if rows.size:
        _L().svg_draft_tokens(seed, stream, _ptr(logits), dt, V, _ptr(rows), rows.size, T, _ptr(out))
    return out


def topk_tokens(logits: np.ndarray, parents: np.ndarray) -> np.ndarray:
    """Deterministic drafts: the children of row r (ascending node index) take the
    1st, 2nd, ... most likely ids of logits row r (viewed as [B, N+1, V]; the lowest
    id first among equal logits)."""
    B, N = parents.shape
    out = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        kids = {}
        for i in range(N):
            kids.setdefault(int(parents[b, i]) + 1, []).append(i)
        for r, ch in kids.items():
            row = logits[b, r]
            row = bf16_to_f32(row) if row.dtype == np.uint16 else row.astype(np.float32)
            n = min(len(ch), row.size)
            kth = np.partition(row, row.size - n)[row.size - n]  # the n-th largest value
            above = np.nonzero(row > kth)[0]
            cand = np.concatenate([above, np.nonzero(row == kth)[0][:n - above.size]])
            order = cand[np.lexsort((cand, -row[cand]))]  # descending value, then ascending id
            order = np.concatenate([order, np.zeros(len(ch) - n, np.int64)])
            for k, i in enumerate(ch):
                out[b, i] = order[k]
    return out


def randint(seed: int, stream: int, n: int, lo: int, hi: int, offset: int = 0) -> np.ndarray:
    """Integers uniform on [lo, hi] (inclusive) by multiply-shift on the top 32 bits."""
    span = hi - lo + 1
    raw = u64(seed, stream, n, offset) >> np.uint64(32)
    return (lo + ((raw * np.uint64(span)) >> np.uint64(32)).astype(np.int64)).astype(np.int64)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (finite inputs)."""
    x = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    x = x + np.uint64(0x7FFF) + ((x >> np.uint64(16)) & np.uint64(1))
    return (x >> np.uint64(16)).astype(np.uint16)


# ---------------------------------------------------------------- trees
def tree_chain(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def tree_star(n: int) -> np.ndarray:
    return np.full(n, -1, dtype=np.int32)


def tree_depths(parents: np.ndarray) -> np.ndarray:
    """Depths of a topologically ordered parent array (parent index < child index)."""
    d = np.zeros(len(parents), dtype=np.int32)
    for i, p in enumerate(parents):
        d[i] = 1 if p < 0 else d[p] + 1
    return d


def tree_eagle_static(seed: int, n_nodes: int = 60, branch: int = 4, depth: int = 6, stream_off: int = 0) -> np.ndarray:
    """Top-``n_nodes`` of the complete ``branch``-ary candidate tree of ``depth`` levels.

    Each sibling group receives ``branch`` seeded uniform scores sorted in
    descending order (child 0 is the drafter's top-1 guess); a candidate's
    priority is the product of scores on its root path.  The top ``n_nodes``
    by priority (ties to the lower breadth-first index) are kept; because every
    score is < 1 the kept set is closed under taking ancestors.  Kept nodes
    are renumbered in breadth-first order, so parents precede children.
    """
    # candidate list in BFS order: (parent candidate, priority)
    cand_parent = []
    cand_prio = []
    level = [(-1, 1.0)]  # the root, a virtual candidate
    level_ids = [-1]
    draws = u64(seed, S_TREE, sum(branch ** d for d in range(depth)) * branch, offset=stream_off)
    di = 0
    for _ in range(depth):
        nxt_ids = []
        for pid, (_, prio) in zip(level_ids, level):
            s = (draws[di:di + branch] >> np.uint64(11)).astype(np.float64) + 1.0
            s = s / 9007199254740994.0  # strictly inside (0, 1)
            di += branch
            s = np.sort(s)[::-1]
            for j in range(branch):
                cand_parent.append(pid)
                cand_prio.append(prio * s[j])
                nxt_ids.append(len(cand_parent) - 1)
        level = [(cand_parent[c], cand_prio[c]) for c in nxt_ids]
        level_ids = nxt_ids
    prio = np.array(cand_prio)
    order = np.lexsort((np.arange(len(prio)), -prio))  # primary: -prio, secondary: bfs index
    keep = np.sort(order[:n_nodes])
    new_id = {int(c): i for i, c in enumerate(keep)}
    parents = np.array([new_id[cand_parent[c]] if cand_parent[c] >= 0 else -1 for c in keep], dtype=np.int32)
    return parents


def tree_random_recursive(seed: int, n: int, max_depth: int, offset: int = 0) -> np.ndarray:
    """Parent of node i uniform over {-1} U {j < i : depth(j) < max_depth}."""
    draws = u64(seed, S_TREE, n, offset=offset) >> np.uint64(32)
    parents = np.empty(n, dtype=np.int32)
    depth = np.empty(n, dtype=np.int32)
    for i in range(n):
        opts = [-1] + [j for j in range(i) if depth[j] < max_depth]
        k = int((int(draws[i]) * len(opts)) >> 32)
        p = opts[k]
        parents[i] = p
        depth[i] = 1 if p < 0 else depth[p] + 1
    return parents


def tree_outcome(seed: int, budgets=(137, 68, 34, 17), k: int = 4, max_depth: int = 10, offset: int = 0) -> np.ndarray:
    """Outcome tree: one root child per prepared outcome branch, each grown best-first.

    Branch j holds ``budgets[j]`` nodes (its first node at depth 1 included).
    Expanding a node offers ``k`` children whose seeded scores are sorted in
    descending order; the frontier is popped by highest product of scores
    (ties to the earlier insertion).  Nodes are renumbered by (depth, branch,
    insertion order), so parents precede children.
    """
    import heapq
    draws = u64(seed, S_TREE, sum(budgets) * k + 8, offset=offset)
    di = 0
    nodes = []  # (depth, branch, order, parent_node_index)
    for bj, budget in enumerate(budgets):
        heap = [(-1.0, 0, -1, 1)]  # (-priority, insertion counter, parent node, depth)
        counter = 1
        taken = 0
        while heap and taken < budget:
            negp, _, par, d = heapq.heappop(heap)
            idx = len(nodes)
            nodes.append((d, bj, taken, par))
            taken += 1
            if d < max_depth:
                s = (draws[di:di + k] >> np.uint64(11)).astype(np.float64) + 1.0
                s = np.sort(s / 9007199254740994.0)[::-1]
                di += k
                for j in range(k):
                    heapq.heappush(heap, (negp * s[j], counter, idx, d + 1))
                    counter += 1
    order = sorted(range(len(nodes)), key=lambda i: (nodes[i][0], nodes[i][1], nodes[i][2]))
    new_id = {old: new for new, old in enumerate(order)}
    parents = np.array([new_id[nodes[o][3]] if nodes[o][3] >= 0 else -1 for o in order], dtype=np.int32)
    return parents


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass
class Workload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    V: int
    dtype: str          # 'f32' | 'bf16' for q / kv / logits
    mode: str           # 'greedy' | 'stochastic'
    temperature: float
    max_depth: int
    paged: bool
    Lcap: int           # contiguous capacity per sequence (0 when paged)
    block_size: int
    max_blocks: int
    num_blocks: int
    parents: np.ndarray
    tokens: np.ndarray
    prefix_len: np.ndarray
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_tree: np.ndarray
    v_tree: np.ndarray
    block_table: Optional[np.ndarray]
    target_logits: np.ndarray
    draft_logits: Optional[np.ndarray]
    u_accept: Optional[np.ndarray]
    u_sample: Optional[np.ndarray]
    scale: float = 0.0
    seed: int = 0
    tree_in_cache: bool = False  # tree K/V rows stored in the cache at positions prefix_len + t
    threshold: float = 0.0       # acceptance threshold when mode == 'threshold'

    def __post_init__(self):
        if not self.scale:
            self.scale = float(np.float32(1.0 / np.sqrt(self.D)))


def _parent_rows(parents: np.ndarray) -> np.ndarray:
    return parents.astype(np.int64) + 1


def build_workload(name: str, B: int, N: int, Hq: int, Hkv: int, D: int, V: int, dtype: str, mode: str,
                   parents: np.ndarray, prefix_len: np.ndarray, max_depth: int, seed: int,
                   paged: bool = False, block_size: int = 16, temperature: float = 1.0,
                   logit_sigma: float = 3.0, target_from_draft_sigma: Optional[float] = None,
                   token_rule: str = "sample", plant: Optional[np.ndarray] = None,
                   need_draft: Optional[bool] = None, lcap_extra: Optional[int] = None) -> Workload:
    """Assemble one workload.

    parents: [B, N] int32.  prefix_len: [B].
    token_rule: 'sample' (draft from q of the parent row, temperature T),
                'greedy' (argmax of the draft parent row), 'uniform' (uniform ids),
                'topk' (siblings take the top ids of the draft parent row in turn).
    target_from_draft_sigma: if set, target = draft + N(0, sigma) (rounded to dtype),
                otherwise target and draft are independent N(0, logit_sigma).
    plant: optional [B] int array of planted match counts (greedy acceptance);
                see ``plant_greedy_matches``.
    """
    parents = np.ascontiguousarray(parents, dtype=np.int32).reshape(B, N)
    prefix_len = np.ascontiguousarray(prefix_len, dtype=np.int32).reshape(B)
    if need_draft is None:
        need_draft = mode == "stochastic" or token_rule in ("sample", "greedy", "topk")
    rows = N + 1
    # logits
    if need_draft or target_from_draft_sigma is not None:
        draft = normal(seed, S_DRF, (B, rows, V), dtype, sigma=logit_sigma)
    else:
        draft = None
    if target_from_draft_sigma is not None:
        target = perturb(seed, S_PERT, draft, target_from_draft_sigma)
    else:
        target = normal(seed, S_TGT, (B, rows, V), dtype, sigma=logit_sigma)
    # tokens
    if token_rule == "uniform":
        tokens = randint(seed, S_TOKENS, B * N, 0, V - 1).astype(np.int32).reshape(B, N)
    elif token_rule == "topk":
        tokens = topk_tokens(draft, parents)
    else:
        prow = (np.arange(B, dtype=np.int64)[:, None] * rows + _parent_rows(parents)).reshape(-1)
        T = temperature if token_rule == "sample" else 0.0
        tokens = draft_tokens(seed, S_TOKENS, draft.reshape(B * rows, V), prow, T).reshape(B, N)
    if plant is not None:
        target = plant_greedy_matches(target, parents, tokens, plant, dtype)
    if mode == "greedy" and not need_draft:
        draft = None
    # attention tensors
    q = normal(seed, S_Q, (B, N, Hq, D), dtype)
    k_tree = normal(seed, S_KT, (B, Hkv, N + 1, D), dtype)
    v_tree = normal(seed, S_VT, (B, Hkv, N + 1, D), dtype)
    k_tree[:, :, 0, :] = 0  # ghost row
    v_tree[:, :, 0, :] = 0
    if not paged:
        extra = max_depth if lcap_extra is None else lcap_extra
        Lcap = int(((int(prefix_len.max()) + extra + 15) // 16) * 16)
        k_cache = normal(seed, S_KC, (B, Hkv, Lcap, D), dtype)
        v_cache = normal(seed, S_VC, (B, Hkv, Lcap, D), dtype)
        block_table = None
        max_blocks = 0
        num_blocks = 0
    else:
        Lcap = 0
        need = (prefix_len.astype(np.int64) + max_depth + block_size - 1) // block_size
        num_blocks = int(need.sum()) + 1
        max_blocks = int(need.max())
        perm = np.arange(1, num_blocks, dtype=np.int64)
        # Fisher-Yates with seeded draws
        draws = u64(seed, S_PERM, len(perm)) >> np.uint64(32)
        for i in range(len(perm) - 1, 0, -1):
            j = int((int(draws[i]) * (i + 1)) >> 32)
            perm[i], perm[j] = perm[j], perm[i]
        block_table = np.zeros((B, max_blocks), dtype=np.int32)
        pos = 0
        for b in range(B):
            block_table[b, :need[b]] = perm[pos:pos + need[b]]
            pos += need[b]
        k_cache = normal(seed, S_KC, (num_blocks, Hkv, block_size, D), dtype)
        v_cache = normal(seed, S_VC, (num_blocks, Hkv, block_size, D), dtype)
        k_cache[0] = 0  # ghost block
        v_cache[0] = 0
    if mode in ("stochastic", "topk"):
        u_accept = uniform24(seed, S_UACC, (B, rows))
        u_sample = uniform24(seed, S_USMP, (B, rows))
    else:
        u_accept = u_sample = None
    return Workload(name=name, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=V, dtype=dtype, mode=mode,
                    temperature=temperature, max_depth=max_depth, paged=paged, Lcap=Lcap,
                    block_size=block_size, max_blocks=max_blocks, num_blocks=num_blocks,
                    parents=parents, tokens=tokens, prefix_len=prefix_len, q=q, k_cache=k_cache,
                    v_cache=v_cache, k_tree=k_tree, v_tree=v_tree, block_table=block_table,
                    target_logits=target, draft_logits=draft, u_accept=u_accept, u_sample=u_sample,
                    seed=seed)


def plant_greedy_matches(target: np.ndarray, parents: np.ndarray, tokens: np.ndarray, plant: np.ndarray,
                         dtype: str) -> np.ndarray:
    """Make the first plant[b] nodes of a seeded root-to-leaf path match greedily.

    For sequence b a leaf is picked (the deepest node of the tree with the
    lowest index, unless ``plant`` carries a (leaf, k) pair), and for the first
    k nodes on its root path the target logit of the node's token in its
    parent row is raised to (row maximum + 1), rounded to the logits dtype.
    """
    target = target.copy()
    B, N = parents.shape
    plant = np.asarray(plant)
    for b in range(B):
        if plant.ndim == 2:
            leaf, k = int(plant[b, 0]), int(plant[b, 1])
        else:
            d = tree_depths(parents[b])
            leaf, k = int(np.argmax(d)), int(plant[b])
        path = []
        cur = leaf
        while cur >= 0:
            path.append(cur)
            cur = int(parents[b, cur])
        path = path[::-1]
        for node in path[:k]:
            row = int(parents[b, node]) + 1
            if dtype == "bf16":
                rmax = float(bf16_to_f32(target[b, row]).max())
                target[b, row, tokens[b, node]] = f32_to_bf16(np.array([rmax + 1.0], dtype=np.float32))[0]
            else:
                rmax = float(target[b, row].max())
                target[b, row, tokens[b, node]] = np.float32(rmax + 1.0)
    return target


def plant_pairs(seed: int, parents: np.ndarray) -> np.ndarray:
    """Seeded (leaf, k) per sequence: leaf uniform over leaves, k uniform on {0..depth(leaf)}."""
    B, N = parents.shape
    out = np.zeros((B, 2), dtype=np.int64)
    r = u64(seed, S_PLANT, 2 * B) >> np.uint64(32)
    for b in range(B):
        par = parents[b]
        has_child = np.zeros(N, dtype=bool)
        for p in par:
            if p >= 0:
                has_child[p] = True
        leaves = np.nonzero(~has_child)[0]
        leaf = int(leaves[(int(r[2 * b]) * len(leaves)) >> 32])
        d = tree_depths(par)[leaf]
        k = (int(r[2 * b + 1]) * (int(d) + 1)) >> 32
        out[b] = (leaf, k)
    return out


# ------------------------------------------------- the five named workloads
def config(cfg: int, seed: Optional[int] = None, **ov) -> Workload:
    """The five verification workloads, optionally shrunk with overrides.

    Overrides: B, L (prefix length, or (lo, hi) range for the batched one), V,
    N / budgets (tree size), plant (greedy planting counts for the tiny chain),
    mode ('topk' for the stochastic ones: deterministic drafts, siblings take the
    top ids of the draft parent row).
    """
    seed = cfg if seed is None else seed
    if cfg == 1:  # tiny chain, fp32, greedy
        B = ov.get("B", 1)
        N = ov.get("N", 4)
        V = ov.get("V", 4096)
        L = ov.get("L", 256)
        par = np.tile(tree_chain(N), (B, 1))
        plant = ov.get("plant")
        w = build_workload("tiny-chain", B, N, 8, 2, 64, V, "f32", "greedy", par, np.full(B, L), max_depth=max(N, 1),
                           seed=seed, logit_sigma=2.0, token_rule="greedy", need_draft=True)
        if plant is not None:
            # target row r := draft row r for r < k, so the chain matches k times
            k = np.broadcast_to(np.asarray(plant), (B,))
            for b in range(B):
                w.target_logits[b, :k[b]] = w.draft_logits[b, :k[b]]
        return w
    if cfg == 2:  # EAGLE-style static tree, 8B shape, stochastic
        B = ov.get("B", 1)
        V = ov.get("V", VOCAB_LLAMA3)
        L = ov.get("L", 4096)
        n_nodes = ov.get("N", 60)
        par = np.stack([tree_eagle_static(seed, n_nodes=n_nodes, stream_off=b * 100003) for b in range(B)])
        mode = ov.get("mode", "stochastic")
        return build_workload("eagle-static-8b", B, n_nodes, 32, 8, 128, V, "bf16", mode, par,
                              np.full(B, L), max_depth=6, seed=seed, logit_sigma=3.0,
                              token_rule="topk" if mode == "topk" else "sample")
    if cfg == 3:  # batched paged, 70B shape, greedy + commit
        B = ov.get("B", 64)
        V = ov.get("V", VOCAB_LLAMA3)
        lo, hi = ov.get("L", (512, 8192))
        N = ov.get("N", 32)
        par = np.stack([tree_random_recursive(seed, N, 6, offset=b * N) for b in range(B)])
        L = randint(seed, S_PLEN, B, lo, hi)
        plant = plant_pairs(seed, par)
        return build_workload("batched-paged-70b", B, N, 64, 8, 128, V, "bf16", "greedy", par, L, max_depth=6,
                              seed=seed, paged=True, block_size=16, logit_sigma=3.0, token_rule="uniform",
                              plant=plant, need_draft=False)
    if cfg == 4:  # linear draft-target chain, 8B shape, stochastic
        B = ov.get("B", 128)
        V = ov.get("V", VOCAB_LLAMA3)
        L = ov.get("L", 2048)
        N = ov.get("N", 5)
        par = np.tile(tree_chain(N), (B, 1))
        mode = ov.get("mode", "stochastic")
        return build_workload("draft-target-chain-8b", B, N, 32, 8, 128, V, "bf16", mode, par,
                              np.full(B, L), max_depth=N, seed=seed, logit_sigma=3.0,
                              target_from_draft_sigma=1.0, token_rule="topk" if mode == "topk" else "sample")
    if cfg == 5:  # SSD outcome tree, 8B shape, 32K prefix, stochastic
        B = ov.get("B", 16)
        V = ov.get("V", VOCAB_LLAMA3)
        L = ov.get("L", 32768)
        budgets = ov.get("budgets", (137, 68, 34, 17))
        par = np.stack([tree_outcome(seed, budgets=budgets, offset=b * 4099) for b in range(B)])
        N = par.shape[1]
        mode = ov.get("mode", "stochastic")
        return build_workload("ssd-outcome-tree-8b", B, N, 32, 8, 128, V, "bf16", mode, par,
                              np.full(B, L), max_depth=10, seed=seed, logit_sigma=3.0,
                              target_from_draft_sigma=1.0, token_rule="topk" if mode == "topk" else "sample")
    raise ValueError(cfg)


def with_tree_in_cache(w: Workload) -> Workload:
    """The same workload with the tree tokens' K/V stored inside the cache.

    Node t's K/V row (tree row t+1) is written to cache position prefix_len[b] + t
    of its sequence; the caches grow so that every sequence holds prefix_len + N
    positions (contiguous: a larger Lcap; paged: extra blocks appended to the pool
    and to the sequence's block table).  New cache positions outside the tree rows
    get seeded normals.  k_tree / v_tree become None.  Data placement only.
    """
    import dataclasses
    L = w.prefix_len.astype(np.int64)
    if not w.paged:
        Lcap = int(((int(L.max()) + w.N + 15) // 16) * 16)
        Lcap = max(Lcap, w.Lcap)
        shape = (w.B, w.Hkv, Lcap, w.D)
        kc = normal(w.seed, S_KC2, shape, w.dtype)
        vc = normal(w.seed, S_VC2, shape, w.dtype)
        kc[:, :, :w.Lcap] = w.k_cache
        vc[:, :, :w.Lcap] = w.v_cache
        for b in range(w.B):
            kc[b, :, L[b]:L[b] + w.N] = w.k_tree[b, :, 1:]
            vc[b, :, L[b]:L[b] + w.N] = w.v_tree[b, :, 1:]
        return dataclasses.replace(w, Lcap=Lcap, k_cache=kc, v_cache=vc, k_tree=None, v_tree=None,
                                   tree_in_cache=True)
    bs = w.block_size
    have = (w.block_table > 0).sum(axis=1)
    need = np.maximum((L + w.N + bs - 1) // bs, have)
    extra = int((need - have).sum())
    num_blocks = w.num_blocks + extra
    max_blocks = max(int(need.max()), w.max_blocks)
    bt = np.zeros((w.B, max_blocks), dtype=np.int32)
    bt[:, :w.max_blocks] = w.block_table
    nxt = w.num_blocks
    for b in range(w.B):
        for k in range(int(have[b]), int(need[b])):
            bt[b, k] = nxt
            nxt += 1
    shape = (num_blocks, w.Hkv, bs, w.D)
    kc = normal(w.seed, S_KC2, shape, w.dtype)
    vc = normal(w.seed, S_VC2, shape, w.dtype)
    kc[:w.num_blocks] = w.k_cache
    vc[:w.num_blocks] = w.v_cache
    kc[0] = 0
    vc[0] = 0
    for b in range(w.B):
        for t in range(w.N):
            pos = int(L[b]) + t
            blk = int(bt[b, pos // bs])
            kc[blk, :, pos % bs] = w.k_tree[b, :, t + 1]
            vc[blk, :, pos % bs] = w.v_tree[b, :, t + 1]
    return dataclasses.replace(w, num_blocks=num_blocks, max_blocks=max_blocks, block_table=bt, k_cache=kc,
                               v_cache=vc, k_tree=None, v_tree=None, tree_in_cache=True)


# ------------------------------------------------- host -> device transfer
def to_device(w: Workload, device="cuda:0"):
    """Copy a workload's arrays to device tensors (bf16 bit patterns become torch.bfloat16)."""
    import torch

    def t(x, dt=None):
        if x is None:
            return None
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
        if x.dtype == np.uint64:
            return torch.from_numpy(x.view(np.int64)).to(device)
        return torch.from_numpy(x).to(device)

    return dict(parents=t(w.parents), tokens=t(w.tokens), q=t(w.q), k_cache=t(w.k_cache), v_cache=t(w.v_cache),
                k_tree=t(w.k_tree), v_tree=t(w.v_tree), prefix_len=t(w.prefix_len.astype(np.int32)),
                target_logits=t(w.target_logits), draft_logits=t(w.draft_logits), u_accept=t(w.u_accept),
                u_sample=t(w.u_sample), block_table=t(w.block_table))


def step_inputs(w: Workload, dev: dict):
    """StepInputs for the library's VerifyStep from a workload and its device copy."""
    from tree_verification_sv_amd.step import StepInputs
    return StepInputs(parents=dev["parents"], tokens=dev["tokens"], q=dev["q"], k_cache=dev["k_cache"],
                      v_cache=dev["v_cache"], k_tree=dev["k_tree"], v_tree=dev["v_tree"],
                      prefix_len=dev["prefix_len"], target_logits=dev["target_logits"], max_depth=w.max_depth,
                      mode=w.mode, temperature=w.temperature, draft_logits=dev["draft_logits"],
                      u_accept=dev["u_accept"], u_sample=dev["u_sample"], block_table=dev["block_table"],
                      paged=w.paged, num_blocks=w.num_blocks, scale=w.scale, tree_in_cache=w.tree_in_cache,
                      threshold=w.threshold)
