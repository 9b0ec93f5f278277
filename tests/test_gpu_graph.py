"""HIP graph capture of the forward (segmla_forward on a captured stream).

The forward enqueues kernels only (no host synchronisation, memory set or host copy), so a
caller can capture it once and replay it, e.g. a serving loop's decode step. Each case captures
one forward, then replays it three times with eager work in between (the NaN fills of its
outputs and an eager forward of the same plan into other buffers, with synchronisations), and
checks every replay against the eager forward bit for bit: the decode path (the decode kernel,
the wide split merge and the matrix-vector projection), a whole small request (prefill tiles
with the replacement copy in the attention grid, the operand-order copy of W and the MFMA
projection), the E4M3 latent, and sink + window heads.
"""
import pytest
import torch

from segmented_attention_amd.segmla import Plan
from tests.gpu_common import say
from workload import CONFIGS, SMALL_CONFIGS, make_inputs
from workload.configs import WINDOW_CONFIGS

pytestmark = pytest.mark.gpu


def _bufs(inp, n):
    cfg = inp["cfg"]
    H, dt = cfg["n_heads"], inp["q"].dtype
    nan = float("nan")
    return (torch.full((n, H, inp["d_v"]), nan, dtype=dt, device="cuda"),
            torch.full((n, H, cfg["d_state"]), nan, dtype=dt, device="cuda"),
            torch.full((n, H), nan, dtype=torch.float32, device="cuda"))


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


CASES = [("decode_32k_last_row", CONFIGS[1], "last"),
         ("flash_small_whole", SMALL_CONFIGS[1], None),
         ("pro_small_fp8_whole", SMALL_CONFIGS[4], None),
         ("flash_window_small_whole", WINDOW_CONFIGS[1], None)]


@pytest.mark.parametrize("name,cfg,window", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, cfg, window):
    say("case graph %s" % name)
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    q_range = (T - 1, T) if window == "last" else None
    n = 1 if window == "last" else T
    plan = Plan.for_inputs(inp, q_range=q_range)
    plan.build(inp["scores"])
    ref = _bufs(inp, n)
    plan.forward(inp, *ref)
    torch.cuda.synchronize()
    out, z, lse = _bufs(inp, n)
    other = _bufs(inp, n)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.forward(inp, out, z, lse)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (out, z, lse) + other:
            t.fill_(float("nan"))
        plan.forward(inp, *other)  # eager work on the same plan between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((out, z, lse) + other, ref + ref, ("out", "z", "lse") * 2):
            assert torch.equal(_bits(got), _bits(want)), "replay %d: %s differs" % (rep, what)
        say("  replay %d equal" % rep)
    del g
    plan.close()
