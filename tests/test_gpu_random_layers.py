"""GPU parity on seeded random layers: combinations of shapes, roles and placements that the
named configurations do not spell out one by one.

Each layer draws, from its own seed:
* the latent and io dtypes (fp32, bf16, or an E4M3 latent with bf16 io);
* the head count and the state width (64 to 512), and for fp32 the nope and RoPE widths;
* the head roles: Global, Local and, in some layers, sink + window heads;
* one to seven segments of any kind and order (prefix, document, new), many of them a few
  rows long, so that key tiles, segment runs and protected-row edges fall anywhere;
* the protected-row rule (edge rows, tail rows, Indexer budget, in half of the layers a few
  caller-listed dirty rows, unsorted and repeated) and values with or without the RoPE dims;
* the softmax scale (1, 0.6 or 1.7) and the RoPE base (10000, 500 or 10^6);
* the latent pool placement (identity, shuffled with gaps, or aliased documents) and the key
  split (none, 64 or 128 keys).

Every (row, head) of the forward is compared with the fp64 oracle, to the tolerances of the
named layers, and the geometry and the protected rows bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from segmented_attention_amd import segmla as S
from segmented_attention_amd.segmla import Plan
from tests.gpu_common import compare, oracle_inputs, run_gpu, say
from workload import make_inputs
from workload.configs import _cfg, _windowed

N_LAYERS = 18  # layers 16 and 17 are bf16 and E4M3 layers with 192 and 256 heads


def random_layer(k):
    """The k-th random layer: (cfg, pool placement, split_keys)."""
    rng = np.random.default_rng([k, 0x5E6])
    kind = str(rng.choice(["f32", "bf16", "e4m3"], p=[0.3, 0.45, 0.25]))
    if k in (16, 17):
        kind = ("bf16", "e4m3")[k % 2]
    segs = []
    for _ in range(int(rng.integers(1, 8))):
        sk = str(rng.choice(["prefix", "doc", "new"], p=[0.15, 0.7, 0.15]))
        n = int(rng.integers(1, 6)) if rng.random() < 0.3 else int(rng.integers(6, 140))
        segs.append((sk, n))
    if kind == "f32":
        H = int(rng.choice([1, 5, 8, 12]))
        d_nope, d_rope = int(rng.choice([16, 64, 96])), int(rng.choice([4, 16, 32]))
        d_state = int(rng.choice([16, 64, 96]))
    else:
        H = int(rng.choice([8, 40, 64, 128])) if k not in (16, 17) else (192, 256)[k % 2]
        d_nope, d_rope = 512, 64
        d_state = int(rng.choice([192, 512]))
        wrng = np.random.default_rng([k, 0xD57])
        if wrng.random() < 0.4:  # state widths the named layers do not use
            d_state = int(wrng.choice([64, 128, 256]))
    cfg = _cfg("random_%02d_%s" % (k, kind), None, "f32" if kind == "f32" else "bf16", H, d_nope,
               d_rope, d_state, segs, edge_rows=int(rng.choice([0, 4, 16])),
               tail_rows=int(rng.choice([0, 8, 64])),
               budget_permille=int(rng.choice([0, 100, 300])), seed=200 + k,
               v_has_rope=int(rng.integers(0, 2)), kv_dtype="e4m3" if kind == "e4m3" else None)
    frac = float(rng.choice([0.0, 0.15, 0.5, 1.0]))
    roles = rng.random(H)
    glob = [h for h in range(H) if roles[h] < frac]
    if rng.random() < 0.3 and len(glob) < H:  # some of the other heads as sink + window heads
        win = [h for h in range(H) if h not in glob and rng.random() < 0.5]
        if win:
            cfg = _windowed(cfg, cfg["name"] + "_win", win, n_sink=int(rng.choice([0, 3])),
                            window=int(rng.choice([1, 17, 64])), global_heads=glob)
    cfg["global_heads"] = glob
    pool = str(rng.choice(["identity", "shuffled", "aliased"]))
    split = int(rng.choice([0, 0, 64, 128]))
    # caller-listed dirty rows (forced into A), unsorted and possibly repeated, in half of the
    # layers; drawn from a stream of their own
    drng = np.random.default_rng([k, 0xD17])
    if drng.random() < 0.5:
        T = sum(n for _, n in segs)
        cfg["dirty_rows"] = [int(x) for x in drng.integers(0, T, int(drng.integers(1, 8)))]
    # softmax scale and RoPE base (the named layers use 1 and 10000), from a stream of their own
    srng = np.random.default_rng([k, 0x5CA])
    cfg["softmax_scale"] = float(srng.choice([1.0, 1.0, 0.6, 1.7]))
    cfg["rope_base"] = float(srng.choice([10000.0, 10000.0, 500.0, 1e6]))
    return cfg, pool, split


CASES = [random_layer(k) for k in range(N_LAYERS)]


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(N_LAYERS), ids=[c[0]["name"] for c in CASES])
def test_random_layer_matches_oracle(k):
    cfg, pool, split = CASES[k]
    say("case %s H=%d segments=%s pool=%s split=%d global=%d window=%d" % (
        cfg["name"], cfg["n_heads"], cfg["segments"], pool, split, len(cfg["global_heads"]),
        len(cfg.get("window_heads", ()))))
    inp = make_inputs(cfg, "cuda", pool=pool)
    plan, out, z, lse = run_gpu(inp, split)
    ref = O.layer_forward(oracle_inputs(inp))
    seg, pool_row = plan.geometry()
    np.testing.assert_array_equal(seg, ref["geom"]["seg_of_row"])
    np.testing.assert_array_equal(pool_row, ref["geom"]["pool_of_row"])
    np.testing.assert_array_equal(plan.protected(), ref["A"])
    e = compare(cfg, ref, out, z, lse, None)
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)
    plan.close()


def random_window(k, T):
    """The k-th layer's row window: one row (decode-shaped, keys split every 64) or a range of
    rows, anywhere in the request; (q0, q1, split_keys)."""
    rng = np.random.default_rng([k, 0x3D0])
    if rng.random() < 0.5:
        q0 = int(rng.integers(0, T))
        return q0, q0 + 1, 64
    q0 = int(rng.integers(0, T))
    q1 = int(rng.integers(q0 + 1, T + 1))
    return q0, q1, int(rng.choice([0, 64]))


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(N_LAYERS), ids=[c[0]["name"] for c in CASES])
def test_random_layer_window_matches_oracle(k):
    """A row window of the same random layer (a plan created for those rows only): its rows
    against the oracle's rows of the whole request."""
    cfg, pool, _ = CASES[k]
    inp = make_inputs(cfg, "cuda", pool=pool)
    T, H = inp["T"], cfg["n_heads"]
    q0, q1, split = random_window(k, T)
    say("case %s window [%d, %d) of %d split=%d" % (cfg["name"], q0, q1, T, split))
    plan = Plan.for_inputs(inp, split, q_range=(q0, q1))
    plan.build(inp["scores"])
    dt = inp["q"].dtype
    out = torch.full((q1 - q0, H, inp["d_v"]), float("nan"), dtype=dt, device="cuda")
    z = torch.full((q1 - q0, H, cfg["d_state"]), float("nan"), dtype=dt, device="cuda")
    lse = torch.full((q1 - q0, H), float("nan"), dtype=torch.float32, device="cuda")
    plan.forward(inp, out, z, lse)
    torch.cuda.synchronize()
    ref = O.layer_forward(oracle_inputs(inp), rows=np.arange(q0, q1))
    np.testing.assert_array_equal(plan.protected(), ref["A"])
    plan.close()
    e = compare(cfg, ref, out, z, lse, None, rows=np.arange(q1 - q0))
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)


def grouped_paged_variant(k):
    """The k-th layer with a grouped projected state (a group size drawn from the divisors 2..8
    of H; None when H has none) over a paged latent pool, and a row window (the whole request
    or a seeded range); (cfg, pool, q0, q1, split_keys) or None."""
    cfg = CASES[k][0]
    H = cfg["n_heads"]
    sizes = [g for g in range(2, min(H, 8) + 1) if H % g == 0]
    if not sizes:
        return None
    rng = np.random.default_rng([k, 0x6A9])
    cfg = dict(cfg, name=cfg["name"] + "_grouped_paged", group_heads=int(rng.choice(sizes)))
    pool = "paged:%d" % int(rng.choice([1, 16, 48, 64]))
    T = sum(n for _, n in cfg["segments"])
    q0, q1 = 0, T
    if rng.random() < 0.5:
        q0 = int(rng.integers(0, T))
        q1 = int(rng.integers(q0 + 1, T + 1))
    return cfg, pool, q0, q1, int(rng.choice([0, 64]))


GP = [v for v in (grouped_paged_variant(k) for k in range(N_LAYERS)) if v is not None]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(GP)), ids=[v[0]["name"] for v in GP])
def test_random_layer_grouped_paged_matches_oracle(i):
    """Grouped projected state over a paged latent pool, on a row window of a random layer:
    z per group against the oracle's grouped state, out and lse per head."""
    from tests.test_gpu_grouped import _check, _run

    cfg, pool, q0, q1, split = GP[i]
    say("case %s G=%d pool=%s window [%d, %d) split=%d" % (cfg["name"], cfg["group_heads"], pool,
                                                          q0, q1, split))
    inp = make_inputs(cfg, "cuda", pool=pool)
    plan, out, z, lse = _run(inp, split, q_range=(q0, q1))
    ref = O.layer_forward_grouped(oracle_inputs(inp), rows=np.arange(q0, q1))
    np.testing.assert_array_equal(plan.protected(), ref["A"])
    plan.close()
    say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % _check(cfg, ref, out, z, lse,
                                                                      np.arange(q1 - q0)))


def moved_windows(k, T):
    """Four windows, in seeded order, that one plan of the k-th layer is moved through: single
    rows and ranges anywhere in the request; and the key split of that plan."""
    rng = np.random.default_rng([k, 0x4E1])
    wins = []
    for _ in range(4):
        q0 = int(rng.integers(0, T))
        q1 = q0 + 1 if rng.random() < 0.5 else int(rng.integers(q0 + 1, T + 1))
        wins.append((q0, q1))
    return wins, int(rng.choice([0, 64]))


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(N_LAYERS), ids=[c[0]["name"] for c in CASES])
def test_random_layer_plan_moved_over_windows(k):
    """One plan of a random layer, built once, moved by set_window through four seeded windows
    (rows before and after the previous window, single rows and ranges); each window's rows
    against the oracle, and A stays the request's."""
    cfg, pool, _ = CASES[k]
    inp = make_inputs(cfg, "cuda", pool=pool)
    T, H = inp["T"], cfg["n_heads"]
    wins, split = moved_windows(k, T)
    whole = Plan.for_inputs(inp, split)
    cap = S.segmla_plan_workspace_bytes(whole.handle)
    whole.close()
    plan = Plan.for_inputs(inp, split, q_range=wins[0])
    plan.build(inp["scores"], min_bytes=cap)
    oi = oracle_inputs(inp)
    dt = inp["q"].dtype
    for i, (q0, q1) in enumerate(wins):
        say("case %s window %d [%d, %d) of %d split=%d" % (cfg["name"], i, q0, q1, T, split))
        if i > 0:
            plan.set_window(q0, q1)
        out = torch.full((q1 - q0, H, inp["d_v"]), float("nan"), dtype=dt, device="cuda")
        z = torch.full((q1 - q0, H, cfg["d_state"]), float("nan"), dtype=dt, device="cuda")
        lse = torch.full((q1 - q0, H), float("nan"), dtype=torch.float32, device="cuda")
        plan.forward(inp, out, z, lse)
        torch.cuda.synchronize()
        ref = O.layer_forward(oi, rows=np.arange(q0, q1))
        np.testing.assert_array_equal(plan.protected(), ref["A"])
        e = compare(cfg, ref, out, z, lse, None, rows=np.arange(q1 - q0))
        say("  max rel err O %.2e Z %.2e, lse max abs err %.2e" % e)
    plan.close()


E4 = [v for v in GP if v[0]["dtype"] == "bf16" and v[0]["d_state"] % 128 == 0]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(E4)), ids=[v[0]["name"] + "_e4m3_state" for v in E4])
def test_random_layer_e4m3_state(i):
    """The grouped state of the same variants emitted as 1x128 E4M3 blocks: the oracle's
    quantizer applied to the library's own bf16 state gives the library's codes and scales bit
    for bit, and the decoded state matches the fp64 grouped oracle within 6e-2."""
    from tests.test_gpu_e4m3_state import E4M3_TOL, _run as run_state

    cfg, pool, q0, q1, split = E4[i]
    say("case %s e4m3 state G=%d pool=%s window [%d, %d) split=%d" % (
        cfg["name"], cfg["group_heads"], pool, q0, q1, split))
    inp = make_inputs(cfg, "cuda", pool=pool)
    out_b, z_b, _ = run_state(inp, cfg, (q0, q1), split)
    out_e, codes, scales = run_state(inp, dict(cfg, z_e4m3=1), (q0, q1), split)
    assert torch.equal(out_b.view(torch.int16), out_e.view(torch.int16))
    want_c, want_s = O.quantize_e4m3_b128_fp32(z_b.float().cpu().numpy())
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(got_s.view(np.uint32), want_s.view(np.uint32))
    np.testing.assert_array_equal(got_c, want_c)
    deq = (O.e4m3_decode(got_c).reshape(*got_c.shape[:-1], -1, 128)
           * got_s[..., None].astype(np.float64)).reshape(got_c.shape)
    ref = O.layer_forward_grouped(oracle_inputs(inp), rows=np.arange(q0, q1))
    e = O.rel_err_rows(deq.reshape(-1, deq.shape[-1]), ref["Z"].reshape(-1, deq.shape[-1]))
    say("  decoded state max rel err %.3g" % e.max())
    assert e.max() <= E4M3_TOL


def dual_variant(k):
    """The k-th layer as a compressed-history (CSA / HCA) layer, for bf16 and E4M3 layers (an
    E4M3 layer keeps its shapes with a bf16 latent; the dual-pool path takes bf16 only): entry
    ratio, raw window, list width (0: HCA, every available entry), compressed-pool placement,
    list rewrite and row window drawn from the seed; (cfg, pool, ratio, window, top_k, cpool,
    variant, q0, q1) or None."""
    cfg, pool, _ = CASES[k]
    if cfg["dtype"] != "bf16":
        return None
    rng = np.random.default_rng([k, 0xD0A])
    cfg = dict(cfg, name=cfg["name"] + "_dual", kv_dtype="bf16")
    ratio = int(rng.choice([1, 2, 3, 4, 16]))
    window = int(rng.choice([0, 5, 40, 127]))
    top_k = int(rng.choice([0, 0, 7, 40, 100]))
    cpool = str(rng.choice(["identity", "shuffled"]))
    variant = str(rng.choice(["none", "shuffle", "dups+cut"])) if top_k else "none"
    T = sum(n for _, n in cfg["segments"])
    q0, q1 = 0, T
    if rng.random() < 0.5:
        q0 = int(rng.integers(0, T))
        q1 = q0 + 1 if rng.random() < 0.5 else int(rng.integers(q0 + 1, T + 1))
    return cfg, pool, ratio, window, top_k, cpool, variant, q0, q1


DUAL = [v for v in (dual_variant(k) for k in range(N_LAYERS)) if v is not None]


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(len(DUAL)), ids=[v[0]["name"] for v in DUAL])
def test_random_layer_dual_pool_matches_oracle(i):
    """The compressed-history attention of a random layer's rows (raw window and compressed
    entries in one softmax) against the oracle, every (row, head) of the window."""
    from tests.test_gpu_dual import _check, _lists_variant, _oracle, _run
    from workload import make_dual_inputs

    cfg, pool, ratio, window, top_k, cpool, variant, q0, q1 = DUAL[i]
    say("case %s pool=%s ratio=%d window=%d top_k=%d cpool=%s lists=%s rows [%d, %d)" % (
        cfg["name"], pool, ratio, window, top_k, cpool, variant, q0, q1))
    inp = make_inputs(cfg, "cuda", pool=pool)
    dual = make_dual_inputs(inp, ratio, window, top_k, "cuda", pool=cpool)
    n_entries = int((np.asarray(inp["lens"]) // ratio).sum())
    dual = _lists_variant(dual, None if variant == "none" else variant, n_entries, cfg["seed"])
    out, lse, n_dev = _run(inp, dual, q_range=(q0, q1))
    assert n_dev == n_entries
    rows = np.arange(q0, q1)
    _check(cfg, _oracle(inp, dual, rows), out, lse, np.arange(q1 - q0))


@pytest.mark.gpu
@pytest.mark.parametrize("k", range(N_LAYERS), ids=[c[0]["name"] for c in CASES])
def test_random_layer_window_graph_replays(k):
    """The forward of each random layer's seeded window captured in a HIP graph and replayed
    twice, with eager forwards of the same plan in between: every replay equals the eager
    forward bit for bit."""
    from tests.test_gpu_graph import _bits, _bufs

    cfg, pool, _ = CASES[k]
    inp = make_inputs(cfg, "cuda", pool=pool)
    q0, q1, split = random_window(k, inp["T"])
    say("case %s graph of window [%d, %d) split=%d" % (cfg["name"], q0, q1, split))
    plan = Plan.for_inputs(inp, split, q_range=(q0, q1))
    plan.build(inp["scores"])
    ref = _bufs(inp, q1 - q0)
    plan.forward(inp, *ref)
    torch.cuda.synchronize()
    got, other = _bufs(inp, q1 - q0), _bufs(inp, q1 - q0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.forward(inp, *got)
    torch.cuda.synchronize()
    for rep in range(2):
        for t in got + other:
            t.fill_(float("nan"))
        plan.forward(inp, *other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(got + other, ref + ref):
            assert torch.equal(_bits(a), _bits(b)), "replay %d differs" % rep
    del g
    plan.close()


def test_random_layers_cover_the_combinations():
    """(CPU) The seeds reach every dtype, every pool placement, split and unsplit runs, window heads,
    layers without Global heads and layers with one-row segments."""
    kinds = {c["kv_dtype"] if c["kv_dtype"] == "e4m3" else c["dtype"] for c, _, _ in CASES}
    assert kinds == {"f32", "bf16", "e4m3"}
    assert {p for _, p, _ in CASES} == {"identity", "shuffled", "aliased"}
    assert {s > 0 for _, _, s in CASES} == {True, False}
    assert any(c.get("window_heads") for c, _, _ in CASES)
    assert any(not c["global_heads"] for c, _, _ in CASES)
    assert any(n == 1 for c, _, _ in CASES for _, n in c["segments"])
    assert {c["d_state"] for c, _, _ in CASES if c["dtype"] == "bf16"} >= {64, 192, 512}
    assert {c["softmax_scale"] != 1.0 for c, _, _ in CASES} == {True, False}
    assert {c["rope_base"] != 10000.0 for c, _, _ in CASES} == {True, False}
    dirty = [c["dirty_rows"] for c, _, _ in CASES if c.get("dirty_rows")]
    assert len(dirty) >= 4 and any(len(set(d)) < len(d) or d != sorted(d) for d in dirty)
    wins = [random_window(k, sum(n for _, n in CASES[k][0]["segments"])) for k in range(N_LAYERS)]
    # one-row windows with a key split on bf16 layers (the decode kernel), and longer windows
    assert any(q1 - q0 == 1 and q1 > s > 0 and CASES[k][0]["kv_dtype"] == "bf16"
               for k, (q0, q1, s) in enumerate(wins))
    assert any(q1 - q0 > 1 for q0, q1, _ in wins)
    assert len(DUAL) >= 10 and {v[4] > 0 for v in DUAL} == {True, False}
    assert len(E4) >= 4
    assert len(GP) >= 10 and {v[2] == 0 and v[3] == sum(n for _, n in v[0]["segments"]) for v in GP} == {True, False}
