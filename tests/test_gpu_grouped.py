"""GPU parity of the grouped projected state (segmla_layer.group_heads >= 2).

z holds one vector per group of heads: on rows of A the sum of all of the group's head
projections, elsewhere the group's Global heads plus the cached Local contribution (the cache
holds one vector per group). Checked against the fp64 oracle's grouped state within the
layer's tolerance per (row, group), with `out` and `lse` checked as in the per-head tests.
"""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import lse_tol_of, oracle_inputs, run_gpu, say, tol_of
from workload import make_inputs
from workload.configs import GROUPED_CONFIGS

pytestmark = pytest.mark.gpu


def _check(cfg, ref, out, z, lse, rows):
    tol = tol_of(cfg)
    idx = torch.as_tensor(rows, device=out.device)
    o = out[idx].double().cpu().numpy()
    comp = ref["computed"]
    assert np.all(np.isfinite(o[comp])) and np.all(np.isnan(o[~comp]))
    # (a window of Local-only rows outside A computes no head: z is the cache alone)
    e_o = O.rel_err_rows(o[comp], ref["O"][comp]) if comp.any() else np.zeros(1)
    assert e_o.max() <= tol, "O max rel err %.3g" % e_o.max()
    zz = z[idx].double().cpu().numpy()
    assert np.all(np.isfinite(zz))
    e_z = O.rel_err_rows(zz.reshape(-1, zz.shape[-1]), ref["Z"].reshape(-1, zz.shape[-1]))
    assert e_z.max() <= tol, "grouped Z max rel err %.3g" % e_z.max()
    ls = lse[idx].double().cpu().numpy()
    e_l = float(np.abs(ls[comp] - ref["lse"][comp]).max()) if comp.any() else 0.0
    assert e_l <= lse_tol_of(cfg), "lse max abs err %.3g > %.1g" % (e_l, lse_tol_of(cfg))
    return float(e_o.max()), float(e_z.max()), e_l


def _run(inp, split_keys=0, q_range=None):
    cfg = inp["cfg"]
    plan = Plan.for_inputs(inp, split_keys, q_range=q_range)
    plan.build(inp["scores"])
    q0, q1 = q_range if q_range else (0, inp["T"])
    G = cfg["group_heads"]
    dt = inp["q"].dtype
    out = torch.full((q1 - q0, cfg["n_heads"], inp["d_v"]), float("nan"), dtype=dt, device="cuda")
    z = torch.full((q1 - q0, cfg["n_heads"] // G, cfg["d_state"]), float("nan"), dtype=dt,
                   device="cuda")
    lse = torch.full((q1 - q0, cfg["n_heads"]), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(inp, out, z, lse)
    torch.cuda.synchronize()
    return plan, out, z, lse


@pytest.mark.parametrize("cfg,split", [(GROUPED_CONFIGS[0], 0), (GROUPED_CONFIGS[0], 64),
                                       (GROUPED_CONFIGS[1], 0), (GROUPED_CONFIGS[1], 128),
                                       (GROUPED_CONFIGS[2], 0)],
                         ids=lambda x: x["name"] if isinstance(x, dict) else str(x))
def test_grouped_parity(cfg, split):
    say("case grouped %s split=%d" % (cfg["name"], split))
    inp = make_inputs(cfg, "cuda")
    plan, out, z, lse = _run(inp, split)
    ref = O.layer_forward_grouped(oracle_inputs(inp))
    np.testing.assert_array_equal(plan.protected(), ref["A"])
    plan.close()
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % _check(cfg, ref, out, z, lse, np.arange(inp["T"])))


@pytest.mark.parametrize("q0,q1", [(0, 1), (300, 500), (-1, 0)], ids=str)
def test_grouped_windows(q0, q1):
    """Row windows with grouped state, the last row (decode) included."""
    cfg = GROUPED_CONFIGS[1]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    if q0 < 0:
        q0, q1 = T - 1, T
    say("case grouped window %s [%d, %d)" % (cfg["name"], q0, q1))
    plan, out, z, lse = _run(inp, q_range=(q0, q1))
    ref = O.layer_forward_grouped(oracle_inputs(inp), rows=np.arange(q0, q1))
    plan.close()
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % _check(cfg, ref, out, z, lse, np.arange(q1 - q0)))


def test_grouped_full_size_32k_sampled():
    """The 32K layer with grouped state in the launch configuration the bench times."""
    cfg = GROUPED_CONFIGS[3]
    say("case grouped full-size %s" % cfg["name"])
    inp = make_inputs(cfg, "cuda")
    plan, out, z, lse = _run(inp)
    A = plan.protected()
    plan.close()
    rng = np.random.default_rng(8)
    T = inp["T"]
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 6, replace=False),
                                     rng.choice(A, 6, replace=False)]))
    ref = O.layer_forward_grouped(oracle_inputs(inp, lazy=True), rows=rows)
    np.testing.assert_array_equal(A, ref["A"])
    say("  %d rows, max rel err O %.2e Z %.2e, lse max abs err %.2e" % ((len(rows),) + _check(cfg, ref, out[rows], z[rows],
                                                                          lse[rows], np.arange(len(rows)))))


@pytest.mark.parametrize("q0,q1,split", [(0, None, 0), (250, 420, 128), (-1, None, 0)], ids=str)
def test_grouped_paged_windows_compose(q0, q1, split):
    """The features together: grouped state over a paged latent pool (48-row pages, documents
    of equal length sharing pages), in row windows and with key splits."""
    cfg = GROUPED_CONFIGS[1]
    inp = make_inputs(cfg, "cuda", pool="paged:48")
    T = inp["T"]
    if q0 < 0:
        q0 = T - 3
    q1 = T if q1 is None else q1
    say("case grouped paged %s [%d, %d) split=%d" % (cfg["name"], q0, q1, split))
    plan, out, z, lse = _run(inp, split, q_range=(q0, q1))
    oi = oracle_inputs(inp)
    ref = O.layer_forward_grouped(oi, rows=np.arange(q0, q1))
    np.testing.assert_array_equal(plan.protected(), ref["A"])
    seg, pool_row = plan.geometry()
    np.testing.assert_array_equal(pool_row, ref["geom"]["pool_of_row"])
    plan.close()
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % _check(cfg, ref, out, z, lse, np.arange(q1 - q0)))


def test_grouped_decode_128k_last_row():
    """The 128K layer's last row with grouped state: split keys, the wide merge and the
    matrix-vector projection summing each group's heads."""
    cfg = GROUPED_CONFIGS[4]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    say("case grouped decode %s [%d, %d)" % (cfg["name"], T - 1, T))
    plan, out, z, lse = _run(inp, q_range=(T - 1, T))
    ref = O.layer_forward_grouped(oracle_inputs(inp, lazy=True), rows=np.arange(T - 1, T))
    plan.close()
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % _check(cfg, ref, out, z, lse, np.arange(1)))
