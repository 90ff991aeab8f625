"""Helpers for the GPU parity tests: run a verification step through the C ABI and
compare with the CPU oracle.  Imported only by tests marked ``gpu``."""
import numpy as np
import pytest

import oracle
import workloads as W


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    import tree_verification_sv_amd as sv
    sv.lib()  # raises if libspecverify.so is missing: never a silent fallback
    return "cuda:0"


def to_np(t):
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_f64(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_step(w, stages=("mask", "attention", "accept", "commit"), acc_flags=0):
    """Run the chosen stages of one verification step on cuda:0; return numpy results.
    acc_flags: extra sv_accept flags (SV_FLAG_ROW_LIST)."""
    import torch
    from tree_verification_sv_amd.step import VerifyStep
    print(f"[gpu] {w.name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} V={w.V} paged={w.paged} "
          f"L=[{int(w.prefix_len.min())},{int(w.prefix_len.max())}] mode={w.mode} stages={stages}", flush=True)
    dev = W.to_device(w, "cuda:0")
    step = VerifyStep(W.step_inputs(w, dev))
    step._acc.flags |= acc_flags
    if "mask" in stages:
        step.build_mask()
    if "attention" in stages:
        step.attention()
    if "accept" in stages:
        step.accept()
    if "commit" in stages:
        step.kv_commit()
    torch.cuda.synchronize()
    r = dict(anc=to_np(step.mask["anc_bits"]).view(np.uint64), depth=to_np(step.mask["depth"]),
             path_rows=to_np(step.mask["path_rows"]), mstatus=to_np(step.mask["status"]))
    if "attention" in stages:
        r["out"] = out_f64(step.out)
        r["astatus"] = to_np(step.attn_status)
    if "accept" in stages:
        r["acc"] = {k: to_np(v) for k, v in step.acc.items()}
    if "commit" in stages:
        r["commit"] = {k: to_np(v) for k, v in step.commit.items()}
        r["k_cache"] = to_np(dev["k_cache"])
        r["v_cache"] = to_np(dev["v_cache"])
    del step, dev
    return r


def check_attention(got, ref, dtype, what=""):
    """Max-abs tolerance of the dtype plus relative-L2 and non-vacuity checks."""
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 1e-4, f"{what}: fp32 max-abs {err.max():.3e}"
        return float(err.max()), 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert err.max() <= 2e-2, f"{what}: bf16 max-abs {err.max():.3e}"
    assert rel <= 1e-2, f"{what}: bf16 relative-L2 {rel:.3e}"
    return float(err.max()), rel


def attention_check_rejects_zero(ref):
    """The combined check must fail an all-zero output (guards against a vacuous tolerance)."""
    try:
        check_attention(np.zeros_like(ref), ref, "bf16")
    except AssertionError:
        return True
    return False


def sample_rows(w, n, seed=0):
    """Seeded sample of flat (b*N + i)*Hq + h indices, always including the corners."""
    total = w.B * w.N * w.Hq
    idx = set(int(x) for x in W.randint(seed, 77, n, 0, total - 1))
    idx |= {0, total - 1, (w.N - 1) * w.Hq, w.Hq - 1}
    return np.array(sorted(idx), dtype=np.int64)


def compare_accept(got, ref, allow_flagged=True):
    ok = np.ones_like(ref["accept_len"], dtype=bool)
    if allow_flagged:
        ok = ref["flagged"] == 0
    for k in ("accept_len", "accept_rows", "out_tokens", "num_out", "stop_row", "status"):
        a, b = got[k][ok], ref[k][ok]
        if not np.array_equal(a, b):
            bad = np.nonzero(~np.all((got[k] == ref[k]).reshape(len(ok), -1), axis=1) & ok)[0]
            raise AssertionError(f"accept field {k} differs on sequences {bad[:10].tolist()}: "
                                 f"gpu {got[k][bad[:3]].tolist()} oracle {ref[k][bad[:3]].tolist()}")
    return int((~ok).sum())
