"""Small helpers shared by the tests (no verification arithmetic here)."""
import json
import os
import types

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def ns(**kw):
    """A workload-like namespace for hand-built cases."""
    d = dict(paged=False, Lcap=0, block_size=16, max_blocks=0, num_blocks=0, block_table=None,
             mode="greedy", temperature=1.0, draft_logits=None, u_accept=None, u_sample=None)
    d.update(kw)
    if "scale" not in d and "D" in d:
        d["scale"] = float(np.float32(1.0 / np.sqrt(d["D"])))
    return types.SimpleNamespace(**d)


def children_lists(parents):
    N = len(parents)
    ch = {r: [] for r in range(N + 1)}
    for i, p in enumerate(parents):
        ch[int(p) + 1].append(i)
    return ch


def root_paths(parents):
    """All root-to-node paths of a well-formed tree by breadth-first search from the root."""
    ch = children_lists(parents)
    paths = {}
    frontier = [(c, [c]) for c in ch[0]]
    while frontier:
        nxt = []
        for node, path in frontier:
            paths[node] = path
            for c in ch[node + 1]:
                nxt.append((c, path + [c]))
        frontier = nxt
    return paths
