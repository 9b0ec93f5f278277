"""Plan reuse across windows of one request (segmla_plan_set_window): the geometry, RoPE
tables, row maps and protected set built once serve every chunk of a chunked prefill and
every row of a decode walk (RedKnot-MLA paper, TP8 fast-path paragraph: repeated document
bundles reuse compact segment-pointer geometry); only the window's part is redone."""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd import segmla as S
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import compare, oracle_inputs, run_gpu, say, tol_of
from workload import CONFIGS, SMALL_CONFIGS, make_inputs
from workload.configs import WINDOW_CONFIGS

pytestmark = pytest.mark.gpu


def _outputs(inp, n):
    cfg = inp["cfg"]
    H, dt = cfg["n_heads"], inp["q"].dtype
    nan = float("nan")
    return (torch.full((n, H, inp["d_v"]), nan, dtype=dt, device="cuda"),
            torch.full((n, H, cfg["d_state"]), nan, dtype=dt, device="cuda"),
            torch.full((n, H), nan, dtype=torch.float32, device="cuda"))


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


@pytest.mark.parametrize("cfg", [SMALL_CONFIGS[0], SMALL_CONFIGS[1], SMALL_CONFIGS[4],
                                 WINDOW_CONFIGS[1], WINDOW_CONFIGS[0]], ids=lambda c: c["name"])
def test_chunked_prefill_reuses_the_plan(cfg):
    """One plan built for the first chunk, moved chunk by chunk over the request. Each chunk's
    out, z and lse equal those of a plan created for that chunk alone, bit for bit (the same
    tiles, work list and split), A stays the request's, the pair counts follow the chunk, and the
    rows match the whole-request forward within the dtype tolerance (bit for bit is not promised
    there: the bf16 kernel's lazy rescale is decided per wavefront, so a row's rounding can
    depend on which rows share its wavefront, and a chunk can group them differently)."""
    say("case chunked prefill %s" % cfg["name"])
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    whole, out, z, lse = run_gpu(inp, -1)
    A = whole.protected()
    cap = S.segmla_plan_workspace_bytes(whole.handle)
    whole.close()
    cuts = sorted({0, 5, 6, min(130, T // 3), T // 2, T - 3, T})
    plan = Plan.for_inputs(inp, split_keys=-1, q_range=(cuts[0], cuts[1]))
    plan.build(inp["scores"], min_bytes=cap)
    hg, hw = len(cfg["global_heads"]), len(cfg.get("window_heads", ()))
    tol = tol_of(cfg)
    for k, (q0, q1) in enumerate(zip(cuts[:-1], cuts[1:])):
        if k > 0:
            plan.set_window(q0, q1)
        o, zz, ls = _outputs(inp, q1 - q0)
        plan.forward(inp, o, zz, ls)
        fresh = Plan.for_inputs(inp, split_keys=-1, q_range=(q0, q1))
        fresh.build(inp["scores"])
        o2, z2, l2 = _outputs(inp, q1 - q0)
        fresh.forward(inp, o2, z2, l2)
        torch.cuda.synchronize()
        fresh.close()
        say("  chunk [%d, %d)" % (q0, q1))
        np.testing.assert_array_equal(plan.protected(), A)
        g, l_ = O.flops_pairs_window(q0, q1, A, hg, cfg["n_heads"] - hg - hw)
        w = hw * O.window_pairs(q0, q1, cfg.get("n_sink", 0), cfg.get("window", 0))
        assert plan.pairs() == (g, l_, w)
        assert torch.equal(_bits(o), _bits(o2)) and torch.equal(_bits(ls), _bits(l2))
        assert torch.equal(_bits(zz), _bits(z2))
        a, b = o.double().cpu().numpy(), out[q0:q1].double().cpu().numpy()
        comp = np.isfinite(b).all(-1)
        np.testing.assert_array_equal(np.isfinite(a).all(-1), comp)
        assert O.rel_err_rows(a[comp], b[comp]).max() <= tol
        a, b = zz.double().cpu().numpy(), z[q0:q1].double().cpu().numpy()
        assert O.rel_err_rows(a.reshape(-1, a.shape[-1]), b.reshape(-1, b.shape[-1])).max() <= tol
    plan.close()


@pytest.mark.parametrize("ci", [2, 1])
def test_decode_walk_reuses_the_plan(ci):
    """A plan created for the request's final length and its first decode row, then moved row by
    row to the end: every row against the fp64 oracle (the window re-targeting keeps the
    request's geometry and A; the key split follows each window's length)."""
    cfg = CONFIGS[ci]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    n = 6
    say("case decode walk %s rows [%d, %d)" % (cfg["name"], T - n, T))
    plan = Plan.for_inputs(inp, q_range=(T - n, T - n + 1))
    plan.build(inp["scores"])
    outs = []
    for t in range(T - n, T):
        if t > T - n:
            plan.set_window(t, t + 1)
        o, zz, ls = _outputs(inp, 1)
        plan.forward(inp, o, zz, ls)
        outs.append((o, zz, ls))
    torch.cuda.synchronize()
    assert S.segmla_plan_get_info(plan.handle)["q_begin"] == T - 1
    plan.close()
    oi = oracle_inputs(inp, lazy=True)
    ref = O.layer_forward(oi, rows=np.arange(T - n, T))
    out = torch.cat([x[0] for x in outs])
    z = torch.cat([x[1] for x in outs])
    lse = torch.cat([x[2] for x in outs])
    e = compare(cfg, ref, out, z, lse, None, rows=np.arange(n))
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


def test_set_window_capacity_and_errors():
    """A window whose part of the workspace does not fit the built workspace is refused with
    SEGMLA_E_WORKSPACE and leaves the plan on its window (its forward is unchanged); invalid
    windows are SEGMLA_E_SHAPE."""
    cfg = SMALL_CONFIGS[1]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    plan = Plan.for_inputs(inp, split_keys=-1, q_range=(10, 12))
    plan.build(inp["scores"])
    o1, z1, l1 = _outputs(inp, 2)
    plan.forward(inp, o1, z1, l1)
    for q0, q1, want in ((0, T, S.SEGMLA_E_WORKSPACE), (5, 3, S.SEGMLA_E_SHAPE),
                         (0, T + 1, S.SEGMLA_E_SHAPE), (-1, 4, S.SEGMLA_E_SHAPE)):
        with pytest.raises(S.SegmlaError) as e:
            S.segmla_plan_set_window(plan.handle, q0, q1)
        assert e.value.status == want, (q0, q1)
    assert S.segmla_plan_get_info(plan.handle)["q_begin"] == 10
    o2, z2, l2 = _outputs(inp, 2)
    plan.forward(inp, o2, z2, l2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o1.nan_to_num(7)), _bits(o2.nan_to_num(7)))
    assert torch.equal(_bits(z1), _bits(z2)) and torch.equal(_bits(l1.nan_to_num(7)), _bits(l2.nan_to_num(7)))
    plan.close()
