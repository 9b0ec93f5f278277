"""GPU parity of the paged latent pool (segmla_plan_create_paged).

Every segment's rows sit on a list of pool pages; the plan cuts segments into runs that are
contiguous in the pool. Pages whose size is a multiple of the key tile (32 keys in the bf16 /
E4M3 kernel, 64 in the fp32 one) keep the tiling of each segment unchanged, so the forward
over a paged copy of a request equals the contiguous forward bit for bit (without a key
split). Any page size must match the fp64 oracle, and the row maps must name the logical
segment and the paged pool row of every request row. Unused pool pages hold NaN, so a read
through a wrong page fails.
"""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from tests.gpu_common import compare, oracle_inputs, run_gpu, say, tol_of
from workload import CONFIGS, SMALL_CONFIGS, make_inputs
from workload.gen import page_placement, pool_rows_of

pytestmark = pytest.mark.gpu


def _same(a, b):
    """Equal values, NaN where the other has NaN (untouched sentinel slots)."""
    a, b = a.float(), b.float()
    return bool(torch.all((a == b) | (torch.isnan(a) & torch.isnan(b))))


def _paged_copy(inp, page_rows, seed):
    """The request of `inp` with its latent and cached state moved onto shuffled pages."""
    pages, n_pool, first = page_placement(inp["kinds"], inp["lens"], page_rows, seed,
                                          share_docs=False)
    dst = torch.as_tensor(pool_rows_of(inp["lens"], pages), device="cuda")
    seg = np.repeat(np.arange(len(inp["lens"])), inp["lens"])
    src = torch.as_tensor(inp["pool_rows"][seg] + np.arange(inp["T"]) - inp["offsets"][seg],
                          device="cuda")
    alt = dict(inp)
    alt["pages"], alt["n_pool"], alt["pool_rows"] = pages, n_pool, first
    for k in ("kv", "kv_scale", "kv_rope", "z_cached"):
        if k in inp:
            t = inp[k]
            fill = 0x7F if t.dtype == torch.uint8 else float("nan")  # E4M3 NaN code
            x = torch.full((n_pool,) + tuple(t.shape[1:]), fill, dtype=t.dtype, device="cuda")
            x[dst] = t[src]
            alt[k] = x
    return alt


@pytest.mark.parametrize("cfg,page_rows", [(CONFIGS[0], 64), (SMALL_CONFIGS[1], 64),
                                           (SMALL_CONFIGS[3], 32), (SMALL_CONFIGS[4], 128),
                                           (SMALL_CONFIGS[5], 64)],
                         ids=lambda x: x["name"] if isinstance(x, dict) else str(x))
def test_paged_equals_contiguous_bitwise(cfg, page_rows):
    say("case paged-bitwise %s page_rows=%d" % (cfg["name"], page_rows))
    inp = make_inputs(cfg, "cuda")
    p1, o1, z1, l1 = run_gpu(inp, -1)
    A = p1.protected()
    p1.close()
    alt = _paged_copy(inp, page_rows, 11)
    p2, o2, z2, l2 = run_gpu(alt, -1)
    np.testing.assert_array_equal(p2.protected(), A)
    seg, pool_row = p2.geometry()
    np.testing.assert_array_equal(seg, np.repeat(np.arange(len(inp["lens"])), inp["lens"]))
    np.testing.assert_array_equal(pool_row, pool_rows_of(inp["lens"], alt["pages"]))
    p2.close()
    assert _same(o1, o2), "out differs"
    assert _same(z1, z2), "z differs"
    assert _same(l1, l2), "lse differs"


@pytest.mark.parametrize("cfg,pool,split", [
    (CONFIGS[0], "paged:5", 0), (SMALL_CONFIGS[0], "paged:16", 64),
    (SMALL_CONFIGS[1], "paged:48", 0), (SMALL_CONFIGS[1], "paged:64", 128),
    (SMALL_CONFIGS[3], "paged:1", 0), (SMALL_CONFIGS[4], "paged:96", 0),
    (SMALL_CONFIGS[6], "paged:40", 0)],
    ids=lambda x: x["name"] if isinstance(x, dict) else str(x))
def test_paged_parity_with_oracle(cfg, pool, split):
    """Shuffled pages with documents of equal length sharing their pages; page sizes that are
    not multiples of the key tile (partial tiles at page breaks), single-row pages, and key
    splits that start inside a page."""
    say("case paged %s %s split=%d" % (cfg["name"], pool, split))
    inp = make_inputs(cfg, "cuda", pool=pool)
    plan, out, z, lse = run_gpu(inp, split)
    ref = O.layer_forward(oracle_inputs(inp))
    seg, pool_row = plan.geometry()
    np.testing.assert_array_equal(seg, ref["geom"]["seg_of_row"])
    np.testing.assert_array_equal(pool_row, ref["geom"]["pool_of_row"])
    np.testing.assert_array_equal(plan.protected(), ref["A"])
    plan.close()
    e = compare(cfg, ref, out, z, lse, None)
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


def test_paged_full_size_32k_sampled():
    """The 32K layer on 256-row pages in the launch configuration the bench times: maps and A
    bit-exact on every row, outputs on sampled rows against the oracle."""
    cfg = CONFIGS[1]
    say("case paged full-size %s" % cfg["name"])
    inp = make_inputs(cfg, "cuda", pool="paged:256")
    plan, out, z, lse = run_gpu(inp)
    oi = oracle_inputs(inp, lazy=True)
    g = O.geometry(oi["kinds"], oi["lens"], oi["offsets"], oi["pool_rows"], oi["n_pool"],
                   oi["pages"])
    prot = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"],
                            (), oi["scores"])
    seg, pool_row = plan.geometry()
    np.testing.assert_array_equal(seg, g["seg_of_row"])
    np.testing.assert_array_equal(pool_row, g["pool_of_row"])
    np.testing.assert_array_equal(plan.protected(), prot["A"])
    rng = np.random.default_rng(5)
    T = inp["T"]
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 6, replace=False),
                                     rng.choice(prot["A"], 6, replace=False)]))
    ref = O.layer_forward(oi, rows=rows)
    plan.close()
    e = compare(cfg, ref, out, z, lse, None, rows=rows)
    say("  %d sampled rows, max rel err O %.2e Z %.2e (tol %.0e), lse max abs err %.2e"
        % (len(rows), e[0], e[1], tol_of(cfg), e[2]))
