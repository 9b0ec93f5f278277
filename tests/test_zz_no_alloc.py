"""segmla_forward_noalloc (plan build + forward with the workspace in the library's own device
array) against segmla_plan_build + segmla_forward on the same inputs, bit for bit. The no-alloc
calls run back to back with shrinking inputs, so each reuses the array the previous call left
behind: a stale value it depended on would show up as a difference."""
import pytest
import torch

from segmented_attention_amd import segmla as S
from tests.gpu_common import say
from workload import CONFIGS, SMALL_CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _outputs(inp, q_range):
    cfg = inp["cfg"]
    q0, q1 = q_range or (0, inp["T"])
    n, H, dt = q1 - q0, cfg["n_heads"], inp["q"].dtype
    nan = float("nan")
    return (torch.full((n, H, inp["d_v"]), nan, dtype=dt, device="cuda"),
            torch.full((n, H, cfg["d_state"]), nan, dtype=dt, device="cuda"),
            torch.full((n, H), nan, dtype=torch.float32, device="cuda"))


def _same(a, b):
    return torch.equal(a.float().nan_to_num(7.0), b.float().nan_to_num(7.0))


# whole 1088-row request -> a decode row with 64-key splits (the decode kernel, then the merge
# and projection in one kernel) -> 4-row window with key splits (partials, merge, thin
# projection) -> the 274-row fp32 layer: each call's workspace is smaller than the last
CASES = [(SMALL_CONFIGS[2], None, 0), (SMALL_CONFIGS[1], (945, 946), 64),
         (SMALL_CONFIGS[1], (942, 946), 256), (CONFIGS[0], None, 0)]


def test_noalloc_matches_plan_build_and_forward():
    runs = []
    for cfg, q_range, split in CASES:
        inp = make_inputs(cfg, "cuda")
        plan = S.Plan.for_inputs(inp, split_keys=split, q_range=q_range)
        ws = S.segmla_plan_workspace_bytes(plan.handle)
        assert ws <= S.NOALLOC_MAX_BYTES
        q = inp["q"] if q_range is None else inp["q"][q_range[0]:q_range[1]]
        runs.append((cfg, q_range, inp, plan, q, ws, _outputs(inp, q_range)))
    assert all(a[5] > b[5] for a, b in zip(runs, runs[1:])), [r[5] for r in runs]
    # the no-alloc calls, back to back on one stream (unbuilt plans)
    for cfg, q_range, inp, plan, q, ws, (o, z, l) in runs:
        say("case noalloc %s window=%s workspace=%d" % (cfg["name"], q_range, ws))
        S.segmla_forward_noalloc(plan.handle, inp["scores"], q, inp["kv"], inp["w"], o, z,
                                 inp.get("z_cached"), inp.get("kv_scale"), inp.get("kv_rope"), l)
    torch.cuda.synchronize()
    for cfg, q_range, inp, plan, q, ws, (o, z, l) in runs:
        # the plan is left unbuilt by the no-alloc call
        with pytest.raises(S.SegmlaError) as e:
            plan.forward(inp, *_outputs(inp, q_range)[:2])
        assert e.value.status == S.SEGMLA_E_STATE
        plan.build(inp["scores"])
        o1, z1, l1 = _outputs(inp, q_range)
        plan.forward(inp, o1, z1, l1)
        torch.cuda.synchronize()
        assert torch.isfinite(z1.float()).all()
        assert _same(o, o1) and _same(z, z1) and _same(l, l1), cfg["name"]
        say("  %s: no-alloc outputs equal plan_build + forward" % cfg["name"])
    # a built plan keeps its own workspace across a no-alloc call of another plan
    cfg, q_range, inp, plan, q, ws, _ = runs[0]
    other = runs[-1]
    o3, z3, l3 = _outputs(other[2], None)
    S.segmla_forward_noalloc(other[3].handle, other[2]["scores"], other[4], other[2]["kv"],
                             other[2]["w"], o3, z3, other[2]["z_cached"], None, None, l3)
    o4, z4, l4 = _outputs(inp, q_range)
    plan.forward(inp, o4, z4, l4)
    o5, z5, l5 = _outputs(inp, q_range)
    S.segmla_forward_noalloc(plan.handle, inp["scores"], q, inp["kv"], inp["w"], o5, z5,
                             inp["z_cached"], None, None, l5)
    torch.cuda.synchronize()
    o, z, l = runs[0][6]
    assert _same(o4, o) and _same(z4, z) and _same(l4, l)
    assert _same(o5, o) and _same(z5, z) and _same(l5, l)
    for r in runs:
        r[3].close()


def test_noalloc_on_random_layers():
    """The seeded random layers (every dtype, head roles, pool placements, key splits, dirty
    rows), each through segmla_forward_noalloc and through plan_build + forward: bit for bit."""
    from tests.test_gpu_random_layers import CASES

    done = 0
    for cfg, pool, split in CASES:
        inp = make_inputs(cfg, "cuda", pool=pool)
        plan = S.Plan.for_inputs(inp, split_keys=split)
        ws = S.segmla_plan_workspace_bytes(plan.handle)
        if ws > S.NOALLOC_MAX_BYTES:
            plan.close()
            continue
        say("case noalloc %s pool=%s split=%d workspace=%d" % (cfg["name"], pool, split, ws))
        o, z, l = _outputs(inp, None)
        S.segmla_forward_noalloc(plan.handle, inp["scores"], inp["q"], inp["kv"], inp["w"], o, z,
                                 inp.get("z_cached"), inp.get("kv_scale"), inp.get("kv_rope"), l)
        plan.build(inp["scores"])
        o1, z1, l1 = _outputs(inp, None)
        plan.forward(inp, o1, z1, l1)
        torch.cuda.synchronize()
        assert _same(o, o1) and _same(z, z1) and _same(l, l1), cfg["name"]
        plan.close()
        done += 1
    assert done >= 12, done
