"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the fp64
oracle on exactly the same seeded inputs, and compare."""
import sys

import numpy as np
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd.segmla import Plan

TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}
# Absolute error bound of the natural-log log-sum-exp (the statistic the split merge consumes).
# The fp32 path carries no rounding beyond fp32; the bf16 path rounds the segment-rotated RoPE
# query to bf16 (about 2^-9 |s_rope| per score) and the E4M3 path also rounds code x scale to
# bf16 (about 2^-9 |s| per score): on the synthetic workloads |s| is a few units. Measured over
# the named parity cases (softmax scale 1): at most 8.7e-7 (fp32), 8.8e-4 (bf16) and 5.0e-3
# (E4M3). Seeded random layers reach 1.5e-3 per unit of scale on bf16 where sink + window heads
# see one or two keys (the lse is then about one score, whose rounding is not averaged over many
# keys). The bounds hold at scale 1 and grow with it (lse_tol_of). Tests that drive the scores
# far larger pass their own bound.
LSE_TOL = {"f32": 1e-5, "bf16": 2e-3, "e4m3": 1e-2}


def tol_of(cfg):
    return TOL["e4m3"] if cfg["kv_dtype"] == "e4m3" else TOL[cfg["dtype"]]


def lse_tol_of(cfg):
    """LSE_TOL at softmax scale sigma = 1. lse = log sum_k exp(sigma s_k), so a rounding error
    in the score s_k enters multiplied by sigma: the bound scales with max(1, sigma)."""
    base = LSE_TOL["e4m3"] if cfg["kv_dtype"] == "e4m3" else LSE_TOL[cfg["dtype"]]
    return base * max(1.0, float(cfg.get("softmax_scale", 1.0)))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class _Rows:
    """Row-wise lazy host view of a device tensor (the oracle indexes q / Zc by row)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, i):
        return self.t[int(i)].double().cpu().numpy()


def oracle_inputs(inp, lazy=False):
    """The oracle's view of the generated inputs: stored values upcast exactly to fp64."""
    d = {k: v for k, v in inp.items() if not torch.is_tensor(v)}
    cfg = inp["cfg"]
    if cfg["kv_dtype"] == "e4m3":
        d["latent"] = O.e4m3_b128_values(inp["kv"].cpu().numpy(), inp["kv_scale"].cpu().numpy(),
                                         inp["kv_rope"].double().cpu().numpy())
    else:
        d["latent"] = inp["kv"].double().cpu().numpy()
    d["w"] = inp["w"].double().cpu().numpy()
    d["scores"] = inp["scores"].cpu().numpy()
    if lazy:
        d["q"] = _Rows(inp["q"])
        d["z_cached"] = _Rows(inp["z_cached"])
    else:
        d["q"] = inp["q"].double().cpu().numpy()
        d["z_cached"] = inp["z_cached"].double().cpu().numpy()
    return d


def run_gpu(inp, split_keys=0, with_lse=True, plan=None):
    """Plan + build + forward through the C ABI; outputs pre-filled with a NaN sentinel."""
    cfg = inp["cfg"]
    T, H = inp["T"], cfg["n_heads"]
    own = plan is None
    if own:
        plan = Plan.for_inputs(inp, split_keys)
        plan.build(inp["scores"])
    dt = inp["q"].dtype
    out = torch.full((T, H, inp["d_v"]), float("nan"), dtype=dt, device="cuda")
    z = torch.full((T, H, cfg["d_state"]), float("nan"), dtype=dt, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
    plan.forward(inp, out, z, lse)
    torch.cuda.synchronize()
    return plan, out, z, lse


def compare(cfg, ref, out, z, lse, zc_rows, rows=None, lse_tol=None):
    """Assert parity of one forward against the oracle result `ref` (computed on `rows`).
    Returns (max rel err of O, of Z, max abs err of lse or 0)."""
    lse_tol = lse_tol_of(cfg) if lse_tol is None else lse_tol
    tol = tol_of(cfg)
    rows = ref["rows"] if rows is None else rows
    o = out[torch.as_tensor(rows, device=out.device)].double().cpu().numpy()
    zz = z[torch.as_tensor(rows, device=z.device)].double().cpu().numpy()
    comp = ref["computed"]
    # (a window of Local-only rows outside A computes nothing: every z row is a copy)
    e_o = O.rel_err_rows(o[comp], ref["O"][comp]) if comp.any() else np.zeros(1)
    assert np.all(np.isfinite(o[comp])), "non-finite merged output"
    assert e_o.max() <= tol, "O max rel err %.3g > %.1g" % (e_o.max(), tol)
    # Local heads outside A are never written to `out`
    assert np.all(np.isnan(o[~comp])), "out written for a Local head outside A"
    e_z = O.rel_err_rows(zz[comp], ref["Z"][comp]) if comp.any() else np.zeros(1)
    assert e_z.max() <= tol, "Z max rel err %.3g > %.1g" % (e_z.max(), tol)
    # replaced, never added: copied rows are bit-equal to the cached state
    if (~comp).any():
        np.testing.assert_array_equal(zz[~comp], ref["Z"][~comp])
    e_l = 0.0
    if lse is not None:
        ls = lse[torch.as_tensor(rows, device=lse.device)].double().cpu().numpy()
        e_l = float(np.abs(ls[comp] - ref["lse"][comp]).max()) if comp.any() else 0.0
        assert e_l <= lse_tol, "lse max abs err %.3g > %.1g" % (e_l, lse_tol)
        assert np.all(np.isnan(ls[~comp]))
    return float(e_o.max()), float(e_z.max()), e_l
