"""GPU parity of the decode attention kernel (one-row windows with a key split, bf16 latent).

A one-row window has at most 64 query vectors per tile (one row x the full-context heads), so
the library runs it on a kernel whose two wave sets walk alternate 32-key tiles of each key
range and merge their running (max, sum, output) states at the end by the log-sum-exp rule
(RedKnot-MLA paper, relocation paragraph). These tests force key splits on the small layers (whole
multiples of 64 keys) so that every shape of that walk occurs: a row's last split holding a
single tile (the second set only runs its masked stand-in), splits of an odd and an even number
of tiles (segment boundaries cut extra tiles), splits that cross segment boundaries
(each set changes RoPE frame on its own, possibly skipping the segment the other set took), the
causal edge inside the last tile, and rows inside and outside the protected set. Every window
is checked against the fp64 oracle row.
"""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd import segmla as S
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import compare, oracle_inputs, say
from workload import SMALL_CONFIGS, make_inputs
from workload.configs import WINDOW_CONFIGS

pytestmark = pytest.mark.gpu

# bf16 layers: Flash-like, long, many short documents, nope-only values, and sink + window heads
# beside the full-context ones (their W tiles take the window grid; the rest decodes here)
CFGS = [SMALL_CONFIGS[1], SMALL_CONFIGS[2], SMALL_CONFIGS[3], SMALL_CONFIGS[5],
        WINDOW_CONFIGS[1], WINDOW_CONFIGS[4]]


def _rows(inp):
    """The last row, a document-interior row, a document's first row, a row of A and a row
    outside it (when the request has one)."""
    T = inp["T"]
    offs = [int(o) for o in inp["offsets"]]
    plan = Plan.for_inputs(inp)
    plan.build(inp["scores"])
    A = plan.protected()
    plan.close()
    inA = np.zeros(T, dtype=bool)
    inA[A] = True
    rows = {T - 1, offs[len(offs) // 2] + 7, offs[-2] if len(offs) > 2 else T // 2}
    a_mid = [int(r) for r in A if 100 < r < T - 50]
    if a_mid:
        rows.add(a_mid[len(a_mid) // 2])
    out_mid = np.flatnonzero(~inA[100:T - 50])
    if out_mid.size:
        rows.add(100 + int(out_mid[out_mid.size // 2]))
    return sorted(r for r in rows if 0 < r < T)


@pytest.mark.parametrize("cfg", CFGS, ids=lambda c: c["name"])
@pytest.mark.parametrize("split_keys", [64, 128, 192, 512])
def test_decode_rows_match_oracle(cfg, split_keys):
    inp = make_inputs(cfg, "cuda")
    H = cfg["n_heads"]
    oi = oracle_inputs(inp)
    for t in _rows(inp):
        say("case decode %s row %d split %d" % (cfg["name"], t, split_keys))
        plan = Plan.for_inputs(inp, split_keys, q_range=(t, t + 1))
        plan.build(inp["scores"])
        info = S.segmla_plan_get_info(plan.handle)
        assert info["n_split"] == (t + split_keys) // split_keys, (info["n_split"], t, split_keys)
        dt = inp["q"].dtype
        out = torch.full((1, H, inp["d_v"]), float("nan"), dtype=dt, device="cuda")
        z = torch.full((1, H, cfg["d_state"]), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((1, H), float("nan"), dtype=torch.float32, device="cuda")
        plan.forward(inp, out, z, lse)
        torch.cuda.synchronize()
        plan.close()
        ref = O.layer_forward(oi, rows=np.arange(t, t + 1))
        e = compare(cfg, ref, out, z, lse, None, rows=np.arange(1))
        say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


@pytest.mark.parametrize("cfg,page_rows", [(SMALL_CONFIGS[1], 32), (SMALL_CONFIGS[3], 48),
                                           (SMALL_CONFIGS[5], 40)],
                         ids=lambda x: x["name"] if isinstance(x, dict) else str(x))
@pytest.mark.parametrize("split_keys", [64, 192])
def test_decode_rows_on_paged_pool(cfg, page_rows, split_keys):
    """The decode kernel over a paged latent pool: shuffled pages, some of a size that does not
    divide the 32-key tile, so a segment's keys arrive in runs that cut tiles (each run keeps
    its segment's RoPE frame, and the two sets may meet a run boundary at different steps)."""
    from tests.test_gpu_paged import _paged_copy
    base = make_inputs(cfg, "cuda")
    inp = _paged_copy(base, page_rows, cfg["seed"] + 1)
    H = cfg["n_heads"]
    oi = oracle_inputs(inp)
    for t in _rows(base):
        say("case decode paged %s pages %d row %d split %d" % (cfg["name"], page_rows, t, split_keys))
        plan = Plan.for_inputs(inp, split_keys, q_range=(t, t + 1))
        plan.build(inp["scores"])
        dt = inp["q"].dtype
        out = torch.full((1, H, inp["d_v"]), float("nan"), dtype=dt, device="cuda")
        z = torch.full((1, H, cfg["d_state"]), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((1, H), float("nan"), dtype=torch.float32, device="cuda")
        plan.forward(inp, out, z, lse)
        torch.cuda.synchronize()
        plan.close()
        ref = O.layer_forward(oi, rows=np.arange(t, t + 1))
        e = compare(cfg, ref, out, z, lse, None, rows=np.arange(1))
        say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)
