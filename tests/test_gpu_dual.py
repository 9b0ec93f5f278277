"""GPU parity of the compressed-history (dual-pool) attention of the DeepSeek-V4 CSA and HCA
layers ("Reading notes on DeepSeek-V4 serving in TensorRT-LLM", section 1, the dual-pool kernel
paragraph) over relocated segments: every row's raw window and its compressed entries (all the
available ones, or the row's list) in one softmax, against the fp64 oracle on every (row, head)
of the small layers and on sampled rows of the 32K layer.

Cases cover: windows of 0, 5, 40 and 127 keys (one-tile windows start the entry walk in the
prologue); entry ratios 3, 4 and 16 (segments whose length is not a multiple of the ratio);
contiguous, shuffled and paged latent pools and contiguous or shuffled compressed pools; lists
in Indexer order (ascending), shuffled, with repeated ids, with an id that is not available
(the walk stops there) and with -1 padding; 64, 96 (a partial head block) and 128 heads; values
with and without RoPE dims; row windows (a prefill chunk and the last row), also reached by
moving a built plan's window; and capture of the forward in a HIP graph.
"""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd.segmla import Dual, Plan
from tests.gpu_common import lse_tol_of, oracle_inputs, say, tol_of
from workload import CONFIGS, SMALL_CONFIGS, make_dual_inputs, make_inputs

pytestmark = pytest.mark.gpu


def _lists_variant(dual, mode, n_entries, seed):
    """Rewrite the generated lists: 'shuffle' permutes each row's ids; 'dups+cut' repeats
    a few ids, and on every third row places an unavailable id (past the last entry, or -1)
    inside the list with the length raised to the full width."""
    if mode is None:
        return dual
    cidx = dual["cidx"].cpu().numpy().copy()
    clen = dual["clen"].cpu().numpy().copy()
    rng = np.random.default_rng(seed)
    K = cidx.shape[1]
    for t in range(cidx.shape[0]):
        n = int(clen[t])
        if mode == "shuffle" and n > 1:
            cidx[t, :n] = rng.permutation(cidx[t, :n])
        elif mode == "dups+cut":
            if n >= 2 and n < K:
                cidx[t, n] = cidx[t, int(rng.integers(0, n))]
                clen[t] = n = n + 1
            if t % 3 == 0 and n >= 1:
                at = int(rng.integers(0, n))
                cidx[t, at + 1:] = cidx[t, at:K - 1].copy()
                cidx[t, at] = n_entries + 5 if t % 2 else -1
                clen[t] = K
    out = dict(dual)
    out["cidx"] = torch.from_numpy(cidx).to(dual["cidx"].device)
    out["clen"] = torch.from_numpy(clen).to(dual["clen"].device)
    return out


def _run(inp, dual, q_range=None):
    """Plan (+ build) and one dual-pool forward through the C ABI on the plan's window rows;
    outputs pre-filled with NaN."""
    T, H = inp["T"], inp["cfg"]["n_heads"]
    q0, q1 = q_range if q_range is not None else (0, T)
    plan = Plan.for_inputs(inp, q_range=q_range)
    plan.build(inp["scores"])
    d = Dual.for_inputs(plan, dual)
    d.build()
    out = torch.full((q1 - q0, H, inp["d_v"]), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((q1 - q0, H), float("nan"), dtype=torch.float32, device="cuda")
    cidx = dual["cidx"][q0:q1] if dual["top_k"] else None
    clen = dual["clen"][q0:q1] if dual["top_k"] else None
    d.forward(inp["q"][q0:q1], inp["kv"], dual["ckv"], out, cidx, clen, lse)
    torch.cuda.synchronize()
    n_entries = d.n_entries
    d.close()
    plan.close()
    return out, lse, n_entries


def _oracle(inp, dual, rows):
    oi = oracle_inputs(inp, lazy=True)
    dd = dict(dual, centries=dual["ckv"].double().cpu().numpy())
    lists = lens = None
    if dual["top_k"]:
        lists = dual["cidx"][torch.as_tensor(rows, device=dual["cidx"].device)].cpu().numpy()
        lens = dual["clen"][torch.as_tensor(rows, device=dual["clen"].device)].cpu().numpy()
    return O.dual_pool_forward(oi, dd, rows, lists, lens)


def _check(cfg, ref, out, lse, sel):
    o = out[torch.as_tensor(sel, device=out.device)].double().cpu().numpy()
    ls = lse[torch.as_tensor(sel, device=lse.device)].double().cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ls)), "non-finite output"
    e_o = O.rel_err_rows(o, ref["O"])
    e_l = float(np.abs(ls - ref["lse"]).max())
    say("  max rel err O %.2e (tol %.0e), lse max abs err %.2e, keys per row %d..%d"
        % (e_o.max(), tol_of(cfg), e_l, ref["n_keys"].min(), ref["n_keys"].max()))
    assert e_o.max() <= tol_of(cfg), "O max rel err %.3g" % e_o.max()
    assert e_l <= lse_tol_of(cfg), "lse max abs err %.3g" % e_l


def _heads(cfg, n):
    return dict(cfg, name="%s_h%d" % (cfg["name"], n), n_heads=n,
                global_heads=[h for h in range(n) if h % 8 == 0])


CASES = [
    # name, cfg, raw pool, compressed pool, ratio, window, top_k, list variant
    ("flash_hca4", SMALL_CONFIGS[1], "identity", "identity", 4, 127, 0, None),
    ("flash_csa4", SMALL_CONFIGS[1], "identity", "identity", 4, 127, 40, None),
    ("flash_csa4_w5_shuffled", SMALL_CONFIGS[1], "shuffled", "shuffled", 4, 5, 40, "shuffle"),
    ("long_hca16_w0", SMALL_CONFIGS[2], "identity", "shuffled", 16, 0, 0, None),
    ("many_short_csa3_paged", SMALL_CONFIGS[3], "paged:48", "shuffled", 3, 40, 33, "dups+cut"),
    ("vnope_csa4", SMALL_CONFIGS[5], "identity", "identity", 4, 127, 100, None),
    ("heads96_csa4", _heads(SMALL_CONFIGS[1], 96), "identity", "identity", 4, 127, 40, "dups+cut"),
    ("heads128_hca4_w40", _heads(SMALL_CONFIGS[1], 128), "shuffled", "identity", 4, 40, 0, None),
    ("heads16_csa2_w127", _heads(SMALL_CONFIGS[2], 16), "identity", "identity", 2, 127, 64, "shuffle"),
]


@pytest.mark.parametrize("name,cfg,pool,cpool,ratio,window,top_k,variant", CASES,
                         ids=[c[0] for c in CASES])
def test_dual_pool_matches_oracle(name, cfg, pool, cpool, ratio, window, top_k, variant):
    say("case dual %s" % name)
    inp = make_inputs(cfg, "cuda", pool=pool)
    dual = make_dual_inputs(inp, ratio, window, top_k, "cuda", pool=cpool)
    T = inp["T"]
    n_entries = int((np.asarray(inp["lens"]) // ratio).sum())
    dual = _lists_variant(dual, variant, n_entries, cfg["seed"])
    out, lse, n_dev = _run(inp, dual)
    assert n_dev == n_entries
    rows = np.arange(T)
    _check(cfg, _oracle(inp, dual, rows), out, lse, rows)


@pytest.mark.parametrize("top_k", [0, 40])
def test_dual_pool_row_windows(top_k):
    """A prefill chunk and the last row (decode) of the request: the plan's window rows only."""
    cfg = SMALL_CONFIGS[1]
    inp = make_inputs(cfg, "cuda")
    dual = make_dual_inputs(inp, 4, 127, top_k, "cuda")
    T = inp["T"]
    for q_range in ((200, 520), (T - 1, T)):
        say("case dual window %s top_k %d" % (q_range, top_k))
        out, lse, _ = _run(inp, dual, q_range)
        rows = np.arange(*q_range)
        _check(cfg, _oracle(inp, dual, rows), out, lse, rows - q_range[0])


def test_dual_pool_full_size_32k():
    """The 32K Flash-like layer as a CSA layer (ratio 4, 128-token window, 512-entry lists) and
    as an HCA layer (ratio 128): every row computed in the launch the bench times, sampled rows
    against the oracle (the first and last row of every segment, the question rows and 64
    seeded rows)."""
    cfg = CONFIGS[1]
    inp = make_inputs(cfg, "cuda")
    T = inp["T"]
    offs = np.asarray(inp["offsets"], dtype=np.int64)
    lens = np.asarray(inp["lens"], dtype=np.int64)
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([offs, offs + lens - 1, np.arange(T - 128, T),
                                     rng.integers(0, T, 64)]))
    for ratio, top_k in ((4, 512), (128, 0)):
        say("case dual full-size %s ratio %d top_k %d (%d sampled rows)"
            % (cfg["name"], ratio, top_k, len(rows)))
        dual = make_dual_inputs(inp, ratio, 127, top_k, "cuda")
        out, lse, _ = _run(inp, dual)
        _check(cfg, _oracle(inp, dual, rows), out, lse, rows)


def test_dual_pool_moved_window_and_graph_replays():
    """A plan built for the whole request, moved to a chunk and then to the last row with
    segmla_plan_set_window: the dual-pool forward follows the plan's window. The last-row
    forward captured in a HIP graph and replayed three times, with eager work in between
    (NaN fills, an eager forward into other buffers), equals the eager forward bit for bit."""
    cfg = SMALL_CONFIGS[1]
    inp = make_inputs(cfg, "cuda")
    dual = make_dual_inputs(inp, 4, 127, 40, "cuda")
    T, H = inp["T"], cfg["n_heads"]
    plan = Plan.for_inputs(inp)
    plan.build(inp["scores"])
    d = Dual.for_inputs(plan, dual)
    d.build()
    for q0, q1 in ((300, 700), (T - 1, T)):
        say("case dual moved window (%d, %d)" % (q0, q1))
        plan.set_window(q0, q1)
        out = torch.full((q1 - q0, H, inp["d_v"]), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((q1 - q0, H), float("nan"), dtype=torch.float32, device="cuda")
        args = (inp["q"][q0:q1], inp["kv"], dual["ckv"])
        lists = (dual["cidx"][q0:q1], dual["clen"][q0:q1])
        d.forward(*args, out, *lists, lse)
        torch.cuda.synchronize()
        rows = np.arange(q0, q1)
        _check(cfg, _oracle(inp, dual, rows), out, lse, rows - q0)
    # graph capture of the last-row forward
    ref_o, ref_l = out.clone(), lse.clone()
    g_o, g_l = torch.empty_like(out), torch.empty_like(lse)
    e_o, e_l = torch.empty_like(out), torch.empty_like(lse)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.forward(*args, g_o, *lists, g_l)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (g_o, g_l, e_o, e_l):
            t.fill_(float("nan"))
        d.forward(*args, e_o, *lists, e_l)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in ((g_o, ref_o), (g_l, ref_l), (e_o, ref_o), (e_l, ref_l)):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32))
        say("  replay %d equal" % rep)
    del g
    d.close()
    plan.close()
