"""GPU (HIP path through the C ABI) vs CPU oracle parity, stage by stage and end to end.

Bar: bit-exact for masks, depths, path rows, statuses, accepted lengths, rows,
tokens, stop rows, committed slots, new lengths and committed cache bytes;
attention within max-abs 1e-4 (fp32) or 2e-2 (bf16) plus relative-L2 <= 1e-2
for bf16; stochastic draws the oracle flags (within 1e-6 of a threshold) are
excluded from the exact comparison and counted.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import (attention_check_rejects_zero, check_attention, compare_accept, require_gpu, run_step,
                      sample_rows)

pytestmark = pytest.mark.gpu

# shrunk variants the oracle finishes in seconds; ragged prefix lengths and tails on purpose
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


def _mask_ok(w, r):
    anc, depth, prow, st = oracle.build_tree_mask(w.parents, w.max_depth)
    assert np.array_equal(r["anc"], anc)
    assert np.array_equal(r["depth"], depth)
    assert np.array_equal(r["path_rows"], prow)
    assert np.array_equal(r["mstatus"], st)


def _commit_ok(w, r):
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ref = oracle.kv_commit(w, r["acc"]["accept_len"], r["acc"]["accept_rows"], kc, vc)
    for k in ("new_len", "committed_slots", "status"):
        assert np.array_equal(r["commit"][k], ref[k]), k
    assert np.array_equal(r["k_cache"], kc)
    assert np.array_equal(r["v_cache"], vc)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_step_small(cfg):
    """All four stages on shrunk workloads, every output compared."""
    w = W.config(cfg, **SMALL[cfg])
    r = run_step(w)
    _mask_ok(w, r)
    ref = oracle.tree_attention(w)
    err, rel = check_attention(r["out"], ref, w.dtype, f"config {cfg}")
    print(f"  attention max-abs {err:.2e} rel-L2 {rel:.2e}")
    acc = oracle.accept(w)
    nflag = compare_accept(r["acc"], acc)
    print(f"  accept_len {r['acc']['accept_len'].tolist()} flagged {nflag}")
    _commit_ok(w, r)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_step_full_size(cfg):
    """All four stages at the full workload sizes; attention on a seeded sample of rows."""
    w = W.config(cfg)
    r = run_step(w)
    _mask_ok(w, r)
    n = {1: 10**9, 2: 10**9, 3: 160, 4: 300, 5: 96}[cfg]
    if n >= w.B * w.N * w.Hq:
        ref = oracle.tree_attention(w)
        got = r["out"]
    else:
        sel = sample_rows(w, n, seed=cfg)
        ref = oracle.tree_attention(w, sel=sel)
        got = r["out"].reshape(-1, w.D)[sel]
    err, rel = check_attention(got, ref, w.dtype, f"config {cfg} full")
    assert attention_check_rejects_zero(ref) or w.dtype == "f32"
    print(f"  attention max-abs {err:.2e} rel-L2 {rel:.2e} on {got.shape[0]} rows")
    acc = oracle.accept(w)
    nflag = compare_accept(r["acc"], acc)
    print(f"  mean accept_len {r['acc']['accept_len'].mean():.3f} flagged {nflag}/{w.B}")
    assert nflag <= max(1, w.B // 10)
    _commit_ok(w, r)


@pytest.mark.parametrize("k", range(5))
def test_greedy_planted_chain(k):
    w = W.config(1, plant=k)
    r = run_step(w, ("mask", "accept"))
    acc = oracle.accept(w)
    compare_accept(r["acc"], acc, allow_flagged=False)
    assert r["acc"]["accept_len"][0] == k


def test_mask_fuzz_and_shapes():
    """Random, deep, wide and malformed parent arrays: bit-exact tensorisation and status."""
    cases = [
        W.randint(5, 1, 64 * 40, -3, 42).astype(np.int32).reshape(64, 40),
        np.stack([W.tree_random_recursive(s, 256, 16) for s in range(8)]),
        np.stack([W.tree_chain(16)] * 3),
        np.stack([W.tree_star(256)] * 2),
        np.stack([W.tree_outcome(s) for s in range(4)]),
    ]
    for par in cases:
        B, N = par.shape
        for maxd in (1, 6, 16):
            w = W.Workload(name="mask", B=B, N=N, Hq=1, Hkv=1, D=64, V=1, dtype="f32", mode="greedy",
                           temperature=1.0, max_depth=maxd, paged=False, Lcap=0, block_size=16, max_blocks=0,
                           num_blocks=0, parents=par, tokens=np.zeros_like(par), prefix_len=np.zeros(B, np.int32),
                           q=np.zeros((1,), np.float32), k_cache=np.zeros((1,), np.float32),
                           v_cache=np.zeros((1,), np.float32), k_tree=np.zeros((1,), np.float32),
                           v_tree=np.zeros((1,), np.float32), block_table=None, target_logits=np.zeros((1,), np.float32),
                           draft_logits=None, u_accept=None, u_sample=None)
            import torch
            import tree_verification_sv_amd as sv
            print(f"[gpu] mask fuzz B={B} N={N} max_depth={maxd}", flush=True)
            out = sv.sv_build_tree_mask(torch.from_numpy(np.ascontiguousarray(par)).cuda(), maxd)
            torch.cuda.synchronize()
            anc, depth, prow, st = oracle.build_tree_mask(par, maxd)
            assert np.array_equal(out["anc_bits"].cpu().numpy().view(np.uint64), anc)
            assert np.array_equal(out["depth"].cpu().numpy(), depth)
            assert np.array_equal(out["path_rows"].cpu().numpy(), prow)
            assert np.array_equal(out["status"].cpu().numpy(), st)


def test_leak_free_on_gpu():
    """Perturbing K/V of non-ancestor tree rows by +-1e3 leaves every output bit unchanged."""
    from _util import root_paths
    w = W.config(2, L=40, V=64)
    r0 = run_step(w, ("mask", "attention"))
    paths = root_paths(w.parents[0])
    node = max(paths, key=lambda n: len(paths[n]))
    anc = set(paths[node])
    for t in range(w.N):
        if t not in anc:
            w.k_tree[0, :, t + 1] = W.f32_to_bf16(W.bf16_to_f32(w.k_tree[0, :, t + 1]) + 1e3)
            w.v_tree[0, :, t + 1] = W.f32_to_bf16(W.bf16_to_f32(w.v_tree[0, :, t + 1]) - 1e3)
    r1 = run_step(w, ("mask", "attention"))
    assert np.array_equal(r0["out"][0, node], r1["out"][0, node])


@pytest.mark.parametrize("variant", ["peaky", "short_prefix", "empty_prefix", "d64", "gqa1", "n256", "lpt_b256",
                                     "lpt_b257"])
def test_attention_variants(variant):
    """Non-vacuity and edge shapes: sharp softmax, tree-dominated keys, L = 0, D = 64, G = 1, N = 256;
    paged batches of 256 and 257 ragged sequences with many equal lengths (one work-group per
    (sequence, KV head): the longest-first order at 256, the plain order above it)."""
    if variant.startswith("lpt_"):
        w = W.config(3, B=int(variant[5:]), L=(16, 80), V=64)
    elif variant == "peaky":
        w = W.config(2, L=700, V=64)
        w.q = W.f32_to_bf16(W.bf16_to_f32(w.q) * 8.0)
    elif variant == "short_prefix":
        w = W.config(2, L=37, V=64)
    elif variant == "empty_prefix":
        w = W.config(4, B=3, L=0, V=64)
    elif variant == "d64":
        par = np.stack([W.tree_eagle_static(3, n_nodes=20)] * 2)
        w = W.build_workload("d64", 2, 20, 8, 2, 64, 50, "bf16", "greedy", par, np.array([100, 257]), 6, seed=3,
                             token_rule="uniform", need_draft=False)
    elif variant == "gqa1":
        par = np.stack([W.tree_random_recursive(4, 24, 6)] * 3)
        w = W.build_workload("gqa1", 3, 24, 4, 4, 128, 50, "bf16", "greedy", par, np.array([65, 1, 300]), 6,
                             seed=4, token_rule="uniform", need_draft=False)
    else:
        par = np.stack([W.tree_random_recursive(7, 256, 16)])
        w = W.build_workload("n256", 1, 256, 32, 8, 128, 50, "bf16", "greedy", par, np.array([200]), 16, seed=7,
                             token_rule="uniform", need_draft=False)
    r = run_step(w, ("mask", "attention"))
    ref = oracle.tree_attention(w)
    err, rel = check_attention(r["out"], ref, w.dtype, variant)
    assert attention_check_rejects_zero(ref)
    print(f"  {variant}: max-abs {err:.2e} rel-L2 {rel:.2e} |ref|max {np.abs(ref).max():.3f}")


def test_attention_fp32_paths():
    """fp32 inputs (generic kernel) on a ragged tree with a paged cache."""
    w = W.config(3, B=3, L=(10, 100), V=64, N=12)
    for name in ("q", "k_cache", "v_cache", "k_tree", "v_tree"):
        setattr(w, name, np.ascontiguousarray(W.bf16_to_f32(getattr(w, name))))
    w.dtype = "f32"
    r = run_step(w, ("mask", "attention"))
    check_attention(r["out"], oracle.tree_attention(w), "f32", "fp32 paged")


def test_invalid_inputs_report_status():
    """Malformed trees, out-of-range tokens, ghost blocks and overlong prefixes: codes, no fault."""
    w = W.config(3, B=4, L=(30, 90), V=300, N=16)
    w.parents[0, 5] = 99            # parent out of range
    w.parents[1, 3] = 3             # self-parent cycle
    w.tokens[2, 0] = 300            # token id == V
    w.block_table[3, 0] = 0         # ghost block in a needed position
    r = run_step(w)
    _mask_ok(w, r)
    assert r["mstatus"][0] == 1 and r["mstatus"][1] == 2
    assert r["acc"]["status"][2] == 4
    assert r["astatus"][3] == 5
    acc = oracle.accept(w)
    compare_accept(r["acc"], acc, allow_flagged=False)
    _commit_ok(w, r)
    assert np.isfinite(r["out"]).all()


@pytest.mark.parametrize("shape", ["chain1", "chain3", "siblings3"])
def test_chi_square_gpu(shape):
    """Vocab 16, 10^6 trials on the GPU: the first emitted token follows p_root."""
    from scipy import stats
    import torch
    from tree_verification_sv_amd.step import StepInputs, VerifyStep
    V = 16
    parents = {"chain1": [-1], "chain3": [-1, 0, 1], "siblings3": [-1, -1, -1]}[shape]
    N = len(parents)
    p_rows = W.normal(31, 1, (N + 1, V), "f32", 1.5)
    q_rows = W.normal(31, 2, (N + 1, V), "f32", 1.5)
    n = 250_000
    counts = np.zeros(V, np.int64)
    for s in range(4):
        par = np.tile(np.asarray(parents, np.int32), (n, 1))
        prow = (np.arange(n)[:, None] * (N + 1) + par + 1).reshape(-1)
        drf = np.ascontiguousarray(np.broadcast_to(q_rows, (n, N + 1, V)))
        tgt = np.ascontiguousarray(np.broadcast_to(p_rows, (n, N + 1, V)))
        toks = W.draft_tokens(700 + s, 2, drf.reshape(-1, V), prow, 1.0).reshape(n, N)
        ua = W.uniform24(700 + s, 11, (n, N + 1))
        us = W.uniform24(700 + s, 12, (n, N + 1))
        import tree_verification_sv_amd as sv
        d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
        print(f"[gpu] chi-square {shape} batch {s}", flush=True)
        m = sv.sv_build_tree_mask(d(par), N)
        acc = sv.sv_accept(d(par), d(toks), m["anc_bits"], m["depth"], d(tgt), N, mode="stochastic",
                           draft_logits=d(drf), u_accept=d(ua), u_sample=d(us), temperature=1.0)
        torch.cuda.synchronize()
        counts += np.bincount(acc["out_tokens"][:, 0].cpu().numpy(), minlength=V)
    p0 = np.exp(p_rows[0].astype(np.float64) - p_rows[0].max())
    p0 /= p0.sum()
    chi = stats.chisquare(counts, p0 * counts.sum())
    assert chi.pvalue > 0.01, chi


@pytest.mark.parametrize("B,N,V,form", [(20, 32, 3001, "auto"), (20, 32, 3001, "list"), (16, 40, 40000, "auto"),
                                        (16, 40, 40000, "list"), (24, 24, 300, "auto"), (600, 3, 4096, "auto"),
                                        (600, 3, 4096, "list"), (2, 255, 1000, "auto"), (40, 40, 100000, "auto"),
                                        (40, 40, 100000, "list"), (48, 24, 98311, "auto"), (48, 24, 98311, "list"),
                                        (8, 255, 98305, "auto"), (8, 255, 98305, "list"), (6, 200, 98311, "auto"),
                                        (6, 200, 98311, "list"), (12, 100, 40000, "auto"),
                                        (1100, 3, 1024, "auto"), (300, 15, 70000, "auto")])
def test_greedy_row_streamer(B, N, V, form):
    """Greedy batches of at least 512 rows, each row read whole.  Where the batch's needed rows
    are many bytes (form "auto": (40, 40, 100000), (48, 24, 98311), (8, 255, 98305),
    (6, 200, 98311), and the batches beyond the list), a group of work-groups per sequence follows
    its accepted path row by row; otherwise, or with SV_FLAG_ROW_LIST (form "list"), whole rows of the batch's
    needed-row list are streamed, the first by work-group index and the rest taken from a
    device-wide counter (two rows ahead for rows of one or two slices, one row ahead from three
    slices on), several rows per work-group, leaf stop rows handed back into the walker's
    stream.  Rows off 16 bytes, vocabularies smaller than one slice, wide trees."""
    import tree_verification_sv_amd as sv
    w = W.config(3, B=B, N=N, V=V, L=(16, 80))
    assert w.B * (w.N + 1) >= 512 and w.mode == "greedy"
    print(f"[gpu] greedy streamer B={w.B} N={w.N} V={w.V} form={form}", flush=True)
    r = run_step(w, ("mask", "accept"), acc_flags=sv.SV_FLAG_ROW_LIST if form == "list" else 0)
    compare_accept(r["acc"], oracle.accept(w), allow_flagged=False)

def _tied_siblings(w):
    """Every sibling of a node that matches its parent row's argmax gets that node's token, so
    rows have several matching children: the accepted node is then the deepest match, lowest
    index on ties, over several matching branches."""
    rows = W.bf16_to_f32(w.target_logits) if w.target_logits.dtype == np.uint16 else w.target_logits
    am = rows.argmax(axis=2)  # first index of the maximum: the lowest id on ties
    tok = w.tokens.copy()
    for b in range(w.B):
        par = w.parents[b]
        for i in range(w.N):
            if tok[b, i] == am[b, par[i] + 1]:
                tok[b, par == par[i]] = tok[b, i]
    w.tokens = tok
    return w


@pytest.mark.parametrize("form", ["auto", "list"])
def test_greedy_tied_siblings(form):
    """Greedy batches whose rows have several matching children (equal sibling tokens): the
    chains follow every matching child breadth first, the row list resolves every needed row;
    both must give the oracle's deepest match with the lowest index."""
    import tree_verification_sv_amd as sv
    w = _tied_siblings(W.config(3, B=24, N=40, L=(16, 80)))
    par = w.parents
    multi = 0
    for b in range(w.B):
        rows = W.bf16_to_f32(w.target_logits[b]).argmax(axis=1)
        m = w.tokens[b] == rows[par[b] + 1]
        multi += sum(int(m[par[b] == p].sum()) > 1 for p in set(par[b].tolist()))
    assert multi > 0, "no row with several matching children"
    print(f"[gpu] greedy tied siblings B={w.B} N={w.N} form={form} rows with ties={multi}", flush=True)
    r = run_step(w, ("mask", "accept"), acc_flags=sv.SV_FLAG_ROW_LIST if form == "list" else 0)
    compare_accept(r["acc"], oracle.accept(w), allow_flagged=False)

def _fill_rows(w, picks):
    """Overwrite logits rows: (b, r, kind) with kind 'ninf' (every entry -inf), 'nan' (every entry
    NaN) or 'mixed' (NaN at the first 8 ids and every 1000th, the rest unchanged)."""
    x = w.target_logits.copy()
    bf = x.dtype == np.uint16
    ninf, nan = (np.uint16(0xFF80), np.uint16(0x7FC0)) if bf else (np.float32(-np.inf), np.float32(np.nan))
    for b, r, kind in picks:
        if kind == "ninf":
            x[b, r, :] = ninf
        elif kind == "nan":
            x[b, r, :] = nan
        else:
            x[b, r, :8] = nan
            x[b, r, ::1000] = nan
    w.target_logits = x
    return w


@pytest.mark.parametrize("form,over", [("groups", dict(B=6, N=32, V=70000)), ("list", dict(B=8, N=80, V=40000)),
                                       ("chain", dict(B=24, N=40))])
def test_greedy_nonfinite_rows(form, over):
    """Greedy argmax over rows with -inf and NaN entries, as the oracle takes it: a NaN is never
    the maximum and a row without an entry above -inf has argmax 0 -- for root rows and for the
    stop rows of the unmodified batch, through row groups with exchanges, the row list and the
    path chains."""
    w = W.config(3, L=(16, 80), **over)
    picks = [(0, 0, "ninf"), (1, 0, "nan"), (2, 0, "mixed")]
    ref0 = oracle.accept(w)
    kinds = ("ninf", "nan", "mixed")
    picks += [(b, int(ref0["stop_row"][b]), kinds[b % 3]) for b in range(3, w.B)]
    w = _fill_rows(w, picks)
    ref = oracle.accept(w)
    print(f"[gpu] greedy non-finite rows form={form} B={w.B} N={w.N} V={w.V}", flush=True)
    r = run_step(w, ("mask", "accept"))
    compare_accept(r["acc"], ref, allow_flagged=False)


def test_threshold_bonus_nonfinite_stop_rows():
    """Threshold acceptance whose stop rows have no usable children and hold -inf or NaN entries:
    those rows enter no score, so the accepted paths stay, and the bonus is their argmax as the
    oracle takes it (NaN never the maximum, id 0 when no entry is above -inf)."""
    w = W.config(3, B=16, N=32, V=3001, L=(16, 80))
    w.mode = "threshold"
    w.threshold = float(np.float32(1e-3))
    ref0 = oracle.accept(w)
    kinds = ("ninf", "nan", "mixed")
    picks = []
    for b in range(w.B):
        sr = int(ref0["stop_row"][b])
        if sr > 0 and not (w.parents[b] == sr - 1).any():  # a stop row without children
            picks.append((b, sr, kinds[len(picks) % 3]))
    assert len(picks) >= 3, "too few leaf stop rows"
    w = _fill_rows(w, picks)
    ref = oracle.accept(w)
    assert np.array_equal(ref["accept_len"], ref0["accept_len"])
    print(f"[gpu] threshold non-finite stop rows: {len(picks)}", flush=True)
    r = run_step(w, ("mask", "accept"))
    compare_accept(r["acc"], ref, allow_flagged=True)

@pytest.mark.parametrize("B,N,V", [(32, 20, 40000), (40, 20, 33333), (8, 80, 70000), (10, 60, 50001)])
def test_greedy_rows_fp32(B, N, V):
    """fp32 logits in both greedy forms of batches of at least 512 rows: per-sequence chains
    (the first two shapes) and the streamed row list (the last two, and SV_FLAG_ROW_LIST),
    several slices per row, rows on and off 16 bytes."""
    import tree_verification_sv_amd as sv
    seed = 31 + B
    par = np.stack([W.tree_random_recursive(seed, N, 6, offset=b * N) for b in range(B)])
    w = W.build_workload("greedy-f32", B, N, 8, 2, 64, V, "f32", "greedy", par, np.full(B, 64), max_depth=6,
                         seed=seed, logit_sigma=3.0, token_rule="uniform", plant=W.plant_pairs(seed, par),
                         need_draft=False)
    ref = oracle.accept(w)
    for flags in (0, sv.SV_FLAG_ROW_LIST):
        print(f"[gpu] greedy fp32 B={B} N={N} V={V} flags={flags}", flush=True)
        r = run_step(w, ("mask", "accept"), acc_flags=flags)
        compare_accept(r["acc"], ref, allow_flagged=False)
