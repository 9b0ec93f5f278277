"""GPU parity of row-window plans (segmla_plan_create_range): chunked prefill and decode.

A window plan computes the request rows [q_begin, q_end) with their full causal context over
all segments, and the whole request's protected set A. Without a key split every (row, head)
result depends only on that row's own keys, so windows that cover the request in pieces must
give the whole-request forward's rows bit for bit. Every window must also match the fp64 oracle
on its rows, including decode windows (a few rows at the end of a long request, where the
library splits the key axis and merges the partials).
"""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import compare, oracle_inputs, run_gpu, say
from workload import CONFIGS, SMALL_CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _run_window(inp, q0, q1, split_keys=0):
    cfg = inp["cfg"]
    H, L = cfg["n_heads"], q1 - q0
    plan = Plan.for_inputs(inp, split_keys, q_range=(q0, q1))
    plan.build(inp["scores"])
    dt = inp["q"].dtype
    out = torch.full((L, H, inp["d_v"]), float("nan"), dtype=dt, device="cuda")
    z = torch.full((L, H, cfg["d_state"]), float("nan"), dtype=dt, device="cuda")
    lse = torch.full((L, H), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(inp, out, z, lse)
    torch.cuda.synchronize()
    return plan, out, z, lse


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def _check_pairs(plan, inp, A, q0, q1):
    cfg = inp["cfg"]
    hg = len(cfg["global_heads"])
    assert plan.pairs() == O.flops_pairs_window(q0, q1, A, hg, cfg["n_heads"] - hg) + (0.0,)


@pytest.mark.parametrize("cfg", [SMALL_CONFIGS[0], SMALL_CONFIGS[1], SMALL_CONFIGS[3],
                                 SMALL_CONFIGS[4], SMALL_CONFIGS[5]], ids=lambda c: c["name"])
def test_windows_compose_to_whole_request_bitwise(cfg):
    say("case windows %s" % cfg["name"])
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    plan, out, z, lse = run_gpu(inp, -1)  # never split: per-row results are order independent
    A = plan.protected()
    plan.close()
    rng = np.random.default_rng(cfg["seed"])
    cuts = sorted(set(rng.integers(2, T - 1, 5).tolist()) | {1, T - 1})  # 1-row windows at both ends
    edges = [0] + cuts + [T]
    for q0, q1 in zip(edges[:-1], edges[1:]):
        say("  window [%d, %d)" % (q0, q1))
        p, o, zz, ls = _run_window(inp, q0, q1, -1)
        np.testing.assert_array_equal(p.protected(), A)  # A stays the whole request's
        _check_pairs(p, inp, A, q0, q1)
        p.close()
        assert torch.equal(_bits(o), _bits(out[q0:q1])), "out differs from the whole request's rows"
        assert torch.equal(_bits(ls), _bits(lse[q0:q1])), "lse differs from the whole request's rows"
        if cfg["dtype"] == "f32" or q1 - q0 > THIN_ROWS:
            assert torch.equal(_bits(zz), _bits(z[q0:q1])), "z differs from the whole request's rows"
        else:  # the thin projection: same operands, another summation order
            _check_thin_z(cfg, A, q0, q1, zz, z[q0:q1])


THIN_ROWS = 8  # windows up to this many rows project with the matrix-vector kernel


def _check_thin_z(cfg, A, q0, q1, zw, zr):
    H = cfg["n_heads"]
    comp = np.zeros((q1 - q0, H), dtype=bool)
    comp[:, cfg["global_heads"]] = True
    comp[np.isin(np.arange(q0, q1), A)] = True
    a, b = zw.double().cpu().numpy(), zr.double().cpu().numpy()
    assert np.all(np.isfinite(a[comp]))
    e = O.rel_err_rows(a[comp], b[comp])
    assert e.max() <= 1e-2, "thin projection rel err %.3g" % e.max()
    np.testing.assert_array_equal(a[~comp], b[~comp])  # copied rows: bit for bit


@pytest.mark.parametrize("cfg,q0,q1", [(SMALL_CONFIGS[1], 300, 700), (SMALL_CONFIGS[1], 0, 1),
                                       (SMALL_CONFIGS[0], 80, 81), (SMALL_CONFIGS[4], 200, 530),
                                       (SMALL_CONFIGS[6], 100, 282)],
                         ids=lambda x: x["name"] if isinstance(x, dict) else str(x))
def test_window_parity_with_oracle(cfg, q0, q1):
    """A window in the middle of the request (crossing segment boundaries) against the oracle,
    with the library's own choice of key split."""
    say("case window %s [%d, %d)" % (cfg["name"], q0, q1))
    inp = make_inputs(cfg, "cuda")
    plan, out, z, lse = _run_window(inp, q0, q1)
    ref = O.layer_forward(oracle_inputs(inp), rows=np.arange(q0, q1))
    _check_pairs(plan, inp, ref["A"], q0, q1)
    plan.close()
    e = compare(cfg, ref, out, z, lse, None, rows=np.arange(q1 - q0))
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


@pytest.mark.parametrize("ci,where", [(1, "last_row"), (1, "last_4_rows"), (1, "doc_interior_row"),
                                      (1, "doc_start_row"), (2, "last_row"), (2, "last_8_rows"),
                                      (4, "last_row")],
                         ids=lambda x: CONFIGS[x]["name"] if isinstance(x, int) else x)
def test_decode_windows(ci, where):
    """Decode-shaped windows on the 32K, 128K and 64K-fp8 layers: one or a few rows against
    the whole context, so the key axis is split over many workgroups and merged, and the
    projection takes the matrix-vector path (the 128K last row is the timed decode)."""
    cfg = CONFIGS[ci]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    offs = np.asarray(inp["offsets"])
    q0, q1 = {"last_row": (T - 1, T), "last_4_rows": (T - 4, T), "last_8_rows": (T - 8, T),
              "doc_interior_row": (int(offs[3]) + 1000, int(offs[3]) + 1001),
              "doc_start_row": (int(offs[5]), int(offs[5]) + 1)}[where]
    say("case decode %s [%d, %d)" % (where, q0, q1))
    plan, out, z, lse = _run_window(inp, q0, q1)
    oi = oracle_inputs(inp, lazy=True)
    ref = O.layer_forward(oi, rows=np.arange(q0, q1))
    _check_pairs(plan, inp, ref["A"], q0, q1)
    plan.close()
    e = compare(cfg, ref, out, z, lse, None, rows=np.arange(q1 - q0))
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


@pytest.mark.parametrize("ci,n_rows", [(1, 1), (1, 2), (4, 1)],
                         ids=["32k_last_row", "32k_last_2_rows", "64k_e4m3_last_row"])
def test_merge_of_hundreds_of_splits(ci, n_rows):
    """Decode windows with 64-key splits: 518 (32K layer) and 1028 (64K layer) partials per
    vector, so the many-split merge makes several passes over the splits and reads more than
    256 (max, sum) pairs per vector. The 32K layer's last row takes the decode kernel (bf16
    partials); two rows, and the E4M3 latent, take the prefill kernel (fp32 partials)."""
    from segmented_attention_amd import segmla as S
    cfg = CONFIGS[ci]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    q0, q1 = T - n_rows, T
    say("case many-split merge %s [%d, %d) split 64" % (cfg["name"], q0, q1))
    plan, out, z, lse = _run_window(inp, q0, q1, 64)
    n_split = S.segmla_plan_get_info(plan.handle)["n_split"]
    assert n_split == (T + 63) // 64 and n_split > 256, n_split
    ref = O.layer_forward(oracle_inputs(inp, lazy=True), rows=np.arange(q0, q1))
    plan.close()
    e = compare(cfg, ref, out, z, lse, None, rows=np.arange(n_rows))
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


def test_misaligned_tensor_is_rejected():
    """A tensor pointer off a 16-byte boundary is refused before any launch."""
    from segmented_attention_amd import segmla as S
    cfg = SMALL_CONFIGS[1]
    inp = make_inputs(cfg, "cuda")
    T, H = inp["T"], cfg["n_heads"]
    plan = Plan.for_inputs(inp, q_range=(T - 1, T))
    plan.build(inp["scores"])
    n = H * inp["d_v"]
    big = torch.zeros(n + 8, dtype=inp["q"].dtype, device="cuda")
    out = big[1:1 + n].view(1, H, inp["d_v"])  # 2 bytes past an aligned start
    z = torch.zeros((1, H, cfg["d_state"]), dtype=inp["q"].dtype, device="cuda")
    with pytest.raises(S.SegmlaError) as ei:
        plan.forward(inp, out, z)
    assert ei.value.status == S.SEGMLA_E_SHAPE
    plan.close()
    torch.cuda.synchronize()
    assert torch.count_nonzero(big).item() == 0 and torch.count_nonzero(z).item() == 0


@pytest.mark.parametrize("ci,n_rows", [(1, 12), (2, 8), (3, 6), (4, 6)],
                         ids=["32k_12_rows", "128k_8_rows", "many_short_6_rows", "64k_e4m3_6_rows"])
def test_decode_rows_at_seeded_positions(ci, n_rows):
    """One-row windows at seeded positions anywhere in the full-size layers (documents,
    their edges, rows in and outside A, the 256-segment layer, the E4M3 latent), each with the
    library's own key split, against the oracle."""
    cfg = CONFIGS[ci]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    oi = oracle_inputs(inp, lazy=True)
    for r in np.random.default_rng([ci, 0xDEC]).integers(1, T, n_rows):
        q0, q1 = int(r), int(r) + 1
        say("case decode %s row %d" % (cfg["name"], q0))
        plan, out, z, lse = _run_window(inp, q0, q1)
        plan.close()
        ref = O.layer_forward(oi, rows=np.arange(q0, q1))
        e = compare(cfg, ref, out, z, lse, None, rows=np.arange(1))
        say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)
