"""GPU parity of sink + window heads under relocation (head role 2): every row attends the
sink (the first n_sink request positions) and its recent window [t - w, t] (RedKnot explainer,
"Insight 1: heads have different jobs"), across relocated segments, next to Global heads (full
causal context on every row) and Local heads (rows of A; the cached contribution elsewhere).

Against the fp64 oracle, which masks the dense attention over physically re-rotated keys:
geometry and A bit-exact, O and Z within the dtype tolerance row by row, lse within its bound,
copied Local rows bit-equal to the cache, and the pair counts of all three roles exact."""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import compare, oracle_inputs, run_gpu, say, tol_of
from tests.test_gpu_parity import _oracle_in_chunks, _sample_rows
from workload import make_inputs
from workload.configs import FLASH_32K_WINDOW, SWA_32K, WINDOW_CONFIGS

pytestmark = pytest.mark.gpu


def _pairs_ref(cfg, T, A, q0=0, q1=None):
    q1 = T if q1 is None else q1
    hg, hw = len(cfg["global_heads"]), len(cfg["window_heads"])
    g, l_ = O.flops_pairs_window(q0, q1, A, hg, cfg["n_heads"] - hg - hw)
    return g, l_, hw * O.window_pairs(q0, q1, cfg["n_sink"], cfg["window"])


def _case(cfg, pool="identity", split_keys=0):
    say("case %s pool=%s split_keys=%d (sink %d, window %d)"
        % (cfg["name"], pool, split_keys, cfg["n_sink"], cfg["window"]))
    inp = make_inputs(cfg, "cuda", pool=pool)
    plan, out, z, lse = run_gpu(inp, split_keys)
    ref = O.layer_forward(oracle_inputs(inp))
    seg, pool_row = plan.geometry()
    np.testing.assert_array_equal(seg, ref["geom"]["seg_of_row"])
    np.testing.assert_array_equal(pool_row, ref["geom"]["pool_of_row"])
    np.testing.assert_array_equal(plan.protected(), ref["A"])
    assert ref["computed"][:, cfg["window_heads"]].all()
    e = compare(cfg, ref, out, z, lse, None)
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)
    assert plan.pairs() == _pairs_ref(cfg, inp["T"], ref["A"])
    plan.close()


@pytest.mark.parametrize("cfg", WINDOW_CONFIGS, ids=lambda c: c["name"])
def test_window_heads_parity(cfg):
    _case(cfg)


@pytest.mark.parametrize("ci,pool", [(0, "shuffled"), (1, "shuffled"), (1, "paged:16"),
                                     (2, "paged:48"), (3, "aliased"), (4, "paged:32")],
                         ids=lambda x: WINDOW_CONFIGS[x]["name"] if isinstance(x, int) else x)
def test_window_heads_pool_placement(ci, pool):
    """Windows whose keys sit on other pool rows or on pages (a page break inside the sink, the
    gap or the window; unused pool rows hold NaN, so a read outside the visible keys fails)."""
    _case(WINDOW_CONFIGS[ci], pool=pool)


@pytest.mark.parametrize("ci,split", [(0, 64), (1, 128), (3, 64)])
def test_window_heads_with_key_splits(ci, split):
    """Key splits of the full-context streams beside the (never split) window stream."""
    _case(WINDOW_CONFIGS[ci], split_keys=split)


@pytest.mark.parametrize("ci,q0,q1", [(1, 300, 700), (1, 945, 946), (2, 0, 1), (2, 500, 520),
                                      (0, 100, 274)])
def test_window_heads_row_windows(ci, q0, q1):
    """Row-window plans (chunked prefill, decode): the window heads of the window's rows only."""
    cfg = WINDOW_CONFIGS[ci]
    say("case %s rows [%d, %d)" % (cfg["name"], q0, q1))
    inp = make_inputs(cfg, "cuda")
    H, L = cfg["n_heads"], q1 - q0
    plan = Plan.for_inputs(inp, q_range=(q0, q1))
    plan.build(inp["scores"])
    dt = inp["q"].dtype
    out = torch.full((L, H, inp["d_v"]), float("nan"), dtype=dt, device="cuda")
    z = torch.full((L, H, cfg["d_state"]), float("nan"), dtype=dt, device="cuda")
    lse = torch.full((L, H), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(inp, out, z, lse)
    torch.cuda.synchronize()
    ref = O.layer_forward(oracle_inputs(inp), rows=np.arange(q0, q1))
    assert plan.pairs() == _pairs_ref(cfg, inp["T"], ref["A"], q0, q1)
    plan.close()
    e = compare(cfg, ref, out, z, lse, None, rows=np.arange(L))
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


def test_window_heads_grouped_state():
    """Grouped projected state: a group's sink + window heads are summed with its Global heads
    on every row; its Local heads only on rows of A (the cached group vector elsewhere)."""
    cfg = dict(WINDOW_CONFIGS[1], name="flash_window_small_grouped_bf16", group_heads=8)
    say("case %s" % cfg["name"])
    inp = make_inputs(cfg, "cuda")
    T, H, G = inp["T"], cfg["n_heads"], 8
    plan = Plan.for_inputs(inp)
    plan.build(inp["scores"])
    out = torch.full((T, H, inp["d_v"]), float("nan"), dtype=inp["q"].dtype, device="cuda")
    z = torch.full((T, H // G, cfg["d_state"]), float("nan"), dtype=inp["q"].dtype, device="cuda")
    plan.forward(inp, out, z)
    torch.cuda.synchronize()
    plan.close()
    ref = O.layer_forward_grouped(oracle_inputs(inp))
    e = O.rel_err_rows(z.double().cpu().numpy().reshape(-1, cfg["d_state"]),
                       ref["Z"].reshape(-1, cfg["d_state"]))
    assert e.max() <= tol_of(cfg), "grouped Z max rel err %.3g" % e.max()
    say("  grouped Z max rel err %.2e" % e.max())


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [FLASH_32K_WINDOW, SWA_32K], ids=lambda c: c["name"])
def test_window_heads_full_size_sampled(cfg):
    """The 32K layer with 56 sink + window heads (w = 256, 4 sink tokens) beside its 8 Global
    heads, and the same request as an SWA-128 layer: geometry and A on every row, outputs on
    sampled rows (every segment's first and last row, the new rows, rows inside and outside A)."""
    say("case full-size %s" % cfg["name"])
    inp = make_inputs(cfg, "cuda")
    plan, out, z, lse = run_gpu(inp)
    oi = oracle_inputs(inp, lazy=True)
    g = O.geometry(oi["kinds"], oi["lens"], oi["offsets"], oi["pool_rows"], oi["n_pool"])
    prot = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"], (),
                            oi["scores"])
    np.testing.assert_array_equal(plan.protected(), prot["A"])
    assert plan.pairs() == _pairs_ref(cfg, inp["T"], prot["A"])
    rows = _sample_rows(inp, prot["A"], np.random.default_rng(7))
    say("  %d sampled rows" % len(rows))
    ref = _oracle_in_chunks(oi, rows)
    e = compare(cfg, ref, out, z, lse, None, rows=rows)
    say("  max rel err O %.2e Z %.2e (tol %.0e), lse max abs err %.2e" % (e[0], e[1], tol_of(cfg), e[2]))
    plan.close()
