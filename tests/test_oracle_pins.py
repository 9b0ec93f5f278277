"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test checks the oracle against something independent of its own code:
a brute-force formulation, a library routine, an identity of the mathematics
or a value derived by hand from the pages. A plausible mistake in the oracle
(dropped term, wrong sign or index, off-by-one causality, transposed
operand, wrong tie rule) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from workload import CONFIGS, SMALL_CONFIGS, make_inputs, segment_table
from workload.gen import pool_placement

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _oracle_inputs(inp):
    """Torch inputs -> the fp64 arrays the oracle consumes (stored values upcast exactly)."""
    d = dict(inp)
    if inp["cfg"]["kv_dtype"] == "e4m3":
        d["latent"] = O.e4m3_b128_values(inp["kv"].numpy(), inp["kv_scale"].numpy(),
                                         inp["kv_rope"].double().numpy())
    else:
        d["latent"] = inp["kv"].double().numpy()
    d["q"] = inp["q"].double().numpy()
    d["w"] = inp["w"].double().numpy()
    d["z_cached"] = inp["z_cached"].double().numpy()
    d["scores"] = inp["scores"].numpy()
    return d


def _geom(cfg, mode="identity"):
    kinds, lens, offsets = segment_table(cfg)
    pr, n_pool = pool_placement(lens, mode, cfg["seed"])
    return O.geometry(kinds, lens, offsets, pr, n_pool)


# ---------------------------------------------------------------- protected rows
def _golden_intervals(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = map(int, line.split())
            rows.extend(range(a, b))
    return np.array(rows, dtype=np.int64)


def test_tiny_worked_example():
    cfg = CONFIGS[0]
    g = _geom(cfg)
    assert g["T"] == 274
    p = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"])
    ref = _golden_intervals("tiny_fp32_protected_rows.txt")
    np.testing.assert_array_equal(p["A"], ref)
    gp, lp = O.flops_pairs(g["T"], p["A"], 1, 7)
    assert (gp, lp) == (37675, 82908)


def test_window_pair_counts():
    """Pairs of a row window: brute-force count of (row, head, key) triples on the tiny layer,
    the whole request as one window, and windows covering it in pieces summing to the whole."""
    cfg = CONFIGS[0]
    g = _geom(cfg)
    T = g["T"]
    A = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"])["A"]
    in_a = np.zeros(T, bool)
    in_a[A] = True
    assert O.flops_pairs_window(0, T, A, 1, 7) == O.flops_pairs(T, A, 1, 7)
    for q0, q1 in [(0, 1), (5, 9), (100, 274), (273, 274), (17, 200)]:
        bg = bl = 0
        for t in range(q0, q1):
            for key in range(t + 1):  # causal: keys 0..t
                bg += 1
                bl += 7 * in_a[t]
        assert O.flops_pairs_window(q0, q1, A, 1, 7) == (bg, bl)
    cuts = [0, 3, 66, 67, 150, 266, T]
    parts = [O.flops_pairs_window(a, b, A, 1, 7) for a, b in zip(cuts[:-1], cuts[1:])]
    assert tuple(map(sum, zip(*parts))) == O.flops_pairs(T, A, 1, 7)


@pytest.mark.parametrize("idx,expect", [(1, (2432, 999, 3431)), (2, (38784, 0, 38784)),
                                        (4, (4224, 12416, 16640))])
def test_workload_protected_sizes(idx, expect):
    """|F|, need and |A| derived by hand from the rule for the long workloads."""
    cfg = CONFIGS[idx]
    g = _geom(cfg)
    scores = np.random.default_rng(idx).integers(0, 2**32, g["T"], dtype=np.uint64)
    p = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"],
                         scores=scores)
    assert (int(p["forced"].sum()), p["need"], len(p["A"])) == expect


def _brute_forced(g, b, tau, dirty):
    """Row-by-row membership predicate, written independently of the interval painting."""
    T = g["T"]
    out = np.zeros(T, dtype=bool)
    dirty = set(int(d) for d in dirty)
    for t in range(T):
        i = int(np.searchsorted(g["offsets"], t, side="right") - 1)
        j = t - int(g["offsets"][i])
        n = int(g["lens"][i])
        kind = int(g["kinds"][i])
        edge = kind == O.SEG_DOC and g["offsets"][i] != 0 and (j < b or j >= n - b)
        out[t] = kind == O.SEG_NEW or t in dirty or edge or t >= T - tau
    return out


def _random_geometry(rng):
    n = int(rng.integers(1, 9))
    kinds = rng.choice([0, 1, 1, 1, 2], n).astype(np.uint8)
    if rng.random() < 0.5:
        kinds[0] = 0
    lens = rng.integers(1, 40, n).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return O.geometry(kinds, lens, offsets, offsets, int(lens.sum()))


@pytest.mark.parametrize("seed", range(40))
def test_protected_fuzz(seed):
    rng = np.random.default_rng([77, seed])
    g = _random_geometry(rng)
    T = g["T"]
    b = int(rng.integers(0, 12))
    tau = int(rng.integers(0, 30))
    beta = int(rng.integers(0, 1001))
    dirty = rng.choice(T, int(rng.integers(0, 3)), replace=False) if T > 2 else []
    # adversarial scores half the time: few distinct values, so the row tie-break decides
    if seed % 2:
        scores = rng.integers(0, 3, T).astype(np.uint64)
    else:
        scores = rng.integers(0, 2**32, T, dtype=np.uint64)
    p = O.protected_rows(g, b, tau, beta, dirty, scores)
    forced = _brute_forced(g, b, tau, dirty)
    np.testing.assert_array_equal(p["forced"], forced)
    cand = g["kinds"][g["seg_of_row"]] != O.SEG_NEW
    K = math.ceil(beta * int(cand.sum()) / 1000)
    assert p["K"] == K
    sel = p["indexer"]
    assert int(sel.sum()) == max(0, K - int((forced & cand).sum()))
    assert not np.any(sel & (forced | ~cand))
    # every chosen row beats every unchosen eligible row in (score desc, row asc)
    elig = np.nonzero(cand & ~forced & ~sel)[0]
    for x in np.nonzero(sel)[0]:
        for y in elig:
            assert (scores[x] > scores[y]) or (scores[x] == scores[y] and x < y)
    np.testing.assert_array_equal(p["A"], np.nonzero(forced | sel)[0])


def test_protected_all_equal_scores_take_smallest_rows():
    cfg = SMALL_CONFIGS[1]
    g = _geom(cfg)
    T = g["T"]
    p = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"],
                         scores=np.full(T, 12345, dtype=np.uint64))
    elig = np.nonzero((g["kinds"][g["seg_of_row"]] != O.SEG_NEW) & ~p["forced"])[0]
    np.testing.assert_array_equal(np.nonzero(p["indexer"])[0], elig[:p["need"]])


# ----------------------------------------------------------------------------- RoPE
def test_rotation_group_identities():
    theta = O.rope_theta(64, 10000.0)
    rng = np.random.default_rng(5)
    a, b = rng.uniform(-2e5, 2e5, 2)
    Ra, Rb, Rab = O.rot_blocks(a, theta), O.rot_blocks(b, theta), O.rot_blocks(a + b, theta)
    eye = np.broadcast_to(np.eye(2), Ra.shape)
    np.testing.assert_allclose(np.swapaxes(Ra, -1, -2) @ Ra, eye, atol=1e-15, rtol=0)
    # the product identity carries the rounding of the angles (|a|*theta ~ 2e5 rad)
    np.testing.assert_allclose(Ra @ Rb, Rab, atol=1e-9, rtol=0)
    small = O.rot_blocks(3.0, theta) @ O.rot_blocks(4.0, theta)
    np.testing.assert_allclose(small, O.rot_blocks(7.0, theta), atol=1e-15, rtol=0)
    # theta_0 = 1 and theta_{last} = base^{-(d-2)/d}
    assert theta[0] == 1.0 and math.isclose(theta[-1], 10000.0 ** (-62 / 64))
    # counter-clockwise convention: R(pi/2) maps (1, 0) to (0, 1) on pair 0
    x = np.zeros(64)
    x[0] = 1.0
    y = O.apply_blocks(O.rot_blocks(math.pi / 2, theta), x)
    assert abs(y[0]) < 1e-15 and abs(y[1] - 1.0) < 1e-15


# ----------------------------------------------------------- brute force, tiny case
def _rot2(angle):
    c, s = math.cos(angle), math.sin(angle)
    return np.array([[c, -s], [s, c]])


def test_brute_force_tiny():
    """T = 11, d_nope = d_rope = 2, H = 2: raw unrotated vectors, explicit 2x2 matrices,
    softmax without max subtraction."""
    rng = np.random.default_rng(3)
    kinds = np.array([0, 1, 1, 2], dtype=np.uint8)
    lens = np.array([2, 3, 4, 2])
    offsets = np.array([0, 2, 5, 9])
    T, H, base = 11, 2, 10000.0
    theta0 = 1.0  # d_rope = 2: a single pair with theta_0 = 1
    kh = rng.normal(size=(T, 4))      # true (unrotated) key content per request row
    qh = rng.normal(size=(T, H, 4))   # true (unrotated) query content
    seg = np.repeat(np.arange(4), lens)
    j = np.arange(T) - offsets[seg]
    # stored latent: documents at canonical j, prefix/new at request position
    stored_pos = np.where(kinds[seg] == 1, j, np.arange(T))
    lat = kh.copy()
    q = qh.copy()
    for p in range(T):
        lat[p, 2:] = _rot2(stored_pos[p] * theta0) @ kh[p, 2:]
        for h in range(H):
            q[p, h, 2:] = _rot2(p * theta0) @ qh[p, h, 2:]
    W = rng.normal(size=(H, 3, 4))
    cfg = dict(d_nope=2, d_rope=2, rope_base=base, softmax_scale=0.7, v_has_rope=1,
               edge_rows=1, tail_rows=2, budget_permille=0)
    inp = dict(cfg=cfg, kinds=kinds, lens=lens, offsets=offsets, pool_rows=offsets, n_pool=T,
               head_is_global=np.array([1, 1], dtype=np.uint8), q=q, latent=lat, w=W,
               z_cached=np.zeros((T, 0, 3)), scores=np.zeros(T))
    res = O.layer_forward(inp)
    for t in range(T):
        for h in range(H):
            sc = []
            for p in range(t + 1):
                k_true = np.concatenate([kh[p, :2], _rot2(p * theta0) @ kh[p, 2:]])
                sc.append(0.7 * float(q[t, h] @ k_true))
            e = np.exp(np.array(sc))
            P = e / e.sum()
            o = np.zeros(4)
            u = np.zeros(4)
            for p in range(t + 1):
                o[:2] += P[p] * kh[p, :2]
                o[2:] += P[p] * (_rot2(p * theta0) @ kh[p, 2:])
                # projected-state input: RoPE part in the frame relative to the query
                u[:2] += P[p] * kh[p, :2]
                u[2:] += P[p] * (_rot2((p - t) * theta0) @ kh[p, 2:])
            np.testing.assert_allclose(res["O"][t, h], o, rtol=0, atol=1e-13)
            np.testing.assert_allclose(res["Z"][t, h], W[h] @ u, rtol=0, atol=1e-12)
            # scores depend on relative position only
            rel = qh[t, h, :2] @ kh[:t + 1, :2].T + np.array(
                [qh[t, h, 2:] @ _rot2((p - t) * theta0) @ kh[p, 2:] for p in range(t + 1)])
            np.testing.assert_allclose(np.array(sc), 0.7 * rel, rtol=0, atol=1e-12)


# ------------------------------------------------------------------- library routine
def test_sdpa_float64_pin():
    cfg = CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    res = O.layer_forward(inp)
    g = res["geom"]
    keys = O.relocated_keys(inp["latent"], g, cfg["d_nope"], cfg["d_rope"], cfg["rope_base"])
    kt = torch.from_numpy(keys)[None, None]            # [1, 1, T, d]
    for h in range(cfg["n_heads"]):
        qt = torch.from_numpy(np.ascontiguousarray(inp["q"][:, h]))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, kt, is_causal=True, scale=cfg["softmax_scale"])[0, 0].numpy()
        rows = res["computed"][:, h]
        np.testing.assert_allclose(res["O"][rows, h], ref[rows], rtol=0, atol=1e-12)
    assert res["computed"][:, 0].all()                  # the Global head covers every row
    assert res["computed"][:, 1].sum() == len(res["A"])


# ------------------------------------------------------- segmented fp64 computation
def _segmented_fp64(inp, rows, rng, visible=None):
    """The method itself in fp64, written independently: for each visible segment
    rotate q's RoPE part by -rot_i, attend the stored latent in place, restore the
    partial output's phase by +rot_i, then merge (max, sum, partial) statistics with
    a log-sum-exp merge taken in a random segment order. visible(t, positions) -> bool
    mask restricts the keys (request positions) a row sees; segments with none are skipped."""
    cfg = inp["cfg"]
    dn, dr, base, sig = cfg["d_nope"], cfg["d_rope"], cfg["rope_base"], cfg["softmax_scale"]
    k = np.arange(dr // 2)
    theta = base ** (-2.0 * k / dr)

    def rot(x, ang):  # rotate pairs of x[..., dn:] by angles ang[k]
        y = x.copy()
        c, s = np.cos(ang), np.sin(ang)
        xe, xo = x[..., dn::2], x[..., dn + 1::2]
        y[..., dn::2] = xe * c - xo * s
        y[..., dn + 1::2] = xe * s + xo * c
        return y

    kinds, lens, offs, pr = inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"]
    lat = inp["latent"]
    pages = inp.get("pages")

    def seg_rows(i, n):  # pool rows of segment i's first n rows
        if pages is None:
            return np.arange(pr[i], pr[i] + n)
        P, j = pages["page_rows"], np.arange(n)
        return pages["page_table"][pages["page_start"][i] + j // P] * P + j % P

    out = {}
    for t in rows:
        stats = []
        for i in range(len(lens)):
            if offs[i] > t:
                break
            nvis = min(int(lens[i]), t - int(offs[i]) + 1)
            rot_i = float(offs[i]) if kinds[i] == 1 else 0.0
            C = lat[seg_rows(i, nvis)]
            if visible is not None:
                keep = visible(t, int(offs[i]) + np.arange(nvis))
                if not keep.any():
                    continue
                C = C[keep]
            q = rot(inp["q"][t], -rot_i * theta)            # [H, d]
            s = sig * q @ C.T
            m = s.max(axis=1)
            e = np.exp(s - m[:, None])
            part = rot(e @ C, rot_i * theta)
            stats.append((m, e.sum(axis=1), part))
        order = rng.permutation(len(stats))
        M = np.max([stats[i][0] for i in order], axis=0)
        num = sum(np.exp(stats[i][0] - M)[:, None] * stats[i][2] for i in order)
        den = sum(np.exp(stats[i][0] - M) * stats[i][1] for i in order)
        out[t] = num / den[:, None]
    return out


@pytest.mark.parametrize("cfg,mode", [(CONFIGS[0], "identity"), (SMALL_CONFIGS[0], "shuffled"),
                                      (SMALL_CONFIGS[0], "aliased"), (SMALL_CONFIGS[0], "paged:16"),
                                      (CONFIGS[0], "paged:7")])
def test_relocation_identity(cfg, mode):
    inp = _oracle_inputs(make_inputs(cfg, "cpu", pool=mode))
    T = inp["T"]
    rows = sorted(set([0, 1, T - 1] + list(np.random.default_rng(1).choice(T, 25, replace=False))))
    res = O.layer_forward(inp, rows=rows, A_override=np.arange(T))
    seg = _segmented_fp64(inp, rows, np.random.default_rng(9))
    for i, t in enumerate(rows):
        np.testing.assert_allclose(res["O"][i], seg[t], rtol=0, atol=1e-10)


def test_stored_frame_equivalence():
    """A document stored at canonical positions and placed at Delta gives the same
    outputs as the same rows given as a prefix-kind segment stored at request
    positions (rope part pre-rotated by R(Delta))."""
    cfg = SMALL_CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    g = O.geometry(inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"], inp["n_pool"])
    theta = O.rope_theta(cfg["d_rope"], cfg["rope_base"])
    alt = dict(inp)
    lat = inp["latent"].copy()
    kinds = inp["kinds"].copy()
    for i in range(len(kinds)):
        if kinds[i] == 1:
            s, n, p0 = int(inp["offsets"][i]), int(inp["lens"][i]), int(inp["pool_rows"][i])
            R = O.rot_blocks(np.arange(s, s + n) - np.arange(n) + 0.0, theta)  # R(Delta)
            lat[p0:p0 + n, cfg["d_nope"]:] = O.apply_blocks(R, lat[p0:p0 + n, cfg["d_nope"]:])
            kinds[i] = 0
    alt["latent"], alt["kinds"] = lat, kinds
    T = g["T"]
    a = O.layer_forward(inp, A_override=np.arange(T))
    b = O.layer_forward(alt, A_override=np.arange(T))
    np.testing.assert_allclose(a["O"], b["O"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a["Z"], b["Z"], rtol=0, atol=1e-12)


def test_projected_state_shift_invariance():
    """Rotating every output's RoPE part by R(c) while moving the query position
    from t to t + c leaves the projected state unchanged."""
    rng = np.random.default_rng(4)
    dn, dr, base = 8, 16, 10000.0
    theta = O.rope_theta(dr, base)
    Orows = rng.normal(size=(5, 3, dn + dr))
    t = np.array([0, 3, 17, 400, 12345])
    W = rng.normal(size=(3, 6, dn + dr))
    c = 9876.0
    shifted = Orows.copy()
    shifted[..., dn:] = O.apply_blocks(O.rot_blocks(np.full((5, 1), c), theta), Orows[..., dn:])
    z0 = O.project_rows(Orows, t, [0, 1, 2], W, dn, dr, base, True)
    z1 = O.project_rows(shifted, t + c, [0, 1, 2], W, dn, dr, base, True)
    np.testing.assert_allclose(z0, z1, rtol=0, atol=1e-9)
    # without the inverse RoPE the state would not be shift invariant
    zr = O.project_rows(shifted, t, [0, 1, 2], W, dn, dr, base, True)
    assert np.max(np.abs(zr - z0)) > 1e-3


# ----------------------------------------------------------------------- replacement
def test_exact_cache_identity_and_overwrite():
    """With the cached Local state equal to full recomputation, the replaced state
    equals full recomputation whatever A is (exactness of the projected-state sum,
    RedKnot-MLA paper, projected-state paragraph); NaN-poisoned cached rows inside A
    never reach the output (overwrite, never add); rows outside A copy the cache."""
    cfg = SMALL_CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    T = inp["T"]
    full = O.layer_forward(inp, A_override=np.arange(T))
    g = full["geom"]
    local = np.nonzero(inp["head_is_global"] == 0)[0]
    zc = np.full_like(inp["z_cached"], np.nan)
    zc[g["pool_of_row"]] = full["Z"][:, local]
    res = O.layer_forward(inp, zc_override=zc)
    np.testing.assert_allclose(res["Z"], full["Z"], rtol=0, atol=1e-12)
    outside = np.setdiff1d(np.arange(T), res["A"])
    np.testing.assert_array_equal(res["Z"][outside][:, local], full["Z"][outside][:, local])
    poisoned = inp["z_cached"].copy()
    A = res["A"]
    poisoned[g["pool_of_row"][A]] = np.nan
    res2 = O.layer_forward(inp, zc_override=poisoned)
    assert np.isfinite(res2["Z"]).all()
    notA = np.setdiff1d(np.arange(T), A)
    np.testing.assert_array_equal(res2["Z"][notA][:, local],
                                  inp["z_cached"][g["pool_of_row"][notA]])


# ---------------------------------------------------------------------------- ledger
def test_head_row_ceilings_printed_values():
    """Flash 3F-37R-3F with 56/64 Local heads: 75.29 %; Pro 3F-55R-3F with 112/128:
    78.89 % (RedKnot-MLA paper, profiles paragraph; explainer, DeepSeek-V4 section)."""
    assert round(100 * O.head_row_ceiling(3, 37, 3, 64, 56), 2) == 75.29
    assert round(100 * O.head_row_ceiling(3, 55, 3, 128, 112), 2) == 78.89
    assert O.head_row_ceiling(3, 37, 3, 64, 56) == 2072 / 2752
    lg, ph, op = O.ledger(3, 37, 3, 64, 56, 274, np.arange(274))
    assert ph == 0.0 and op == 0.0
    lg, ph, op = O.ledger(0, 1, 0, 8, 7, 4, np.array([3]))
    # dense triples 8*10 = 80; computed 1*10 + 7*4 = 38
    assert ph == 7 * 3 / (8 * 4) and op == 1 - 38 / 80


# ------------------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0xB8] == -1.0


def test_e4m3_generator_roundtrip_error():
    """The stored E4M3 + fp32 scale rows reproduce the drawn values to the
    format's half-ulp bound (relative 2^-4 for normals)."""
    cfg = SMALL_CONFIGS[4]
    inp = make_inputs(cfg, "cpu")
    vals = O.e4m3_b128_values(inp["kv"].numpy(), inp["kv_scale"].numpy(),
                              inp["kv_rope"].double().numpy())
    assert np.isfinite(vals).all()
    sc = inp["kv_scale"].double().numpy()
    amax = np.abs(vals[:, :512]).reshape(-1, 4, 128).max(-1)
    np.testing.assert_allclose(amax, 448 * sc, rtol=2 ** -4)


def _e4m3_finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_e4m3_encode_inverts_decode():
    """Every finite code (both zeros included) encodes back from its own value."""
    codes = _e4m3_finite_codes()
    np.testing.assert_array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


def test_e4m3_encode_nearest_even_by_brute_force():
    """Against a brute-force search over all finite codes: the nearest value, and on an exact
    tie (every midpoint between neighbouring positive codes, both signs) the code with an even
    mantissa field."""
    codes = _e4m3_finite_codes()
    pos = codes[codes < 0x80]
    pv = O.e4m3_decode(pos)
    order = np.argsort(pv)
    pv, pos = pv[order], pos[order]
    mids = (pv[1:] + pv[:-1]) / 2.0
    rng = np.random.default_rng(7)
    xs = np.concatenate([mids, -mids, rng.uniform(-463.0, 463.0, 4000), rng.uniform(-0.03, 0.03, 4000)])
    allv = O.e4m3_decode(codes)
    got = O.e4m3_encode(xs)
    for x, g in zip(xs, got):
        d = np.abs(allv - x)
        best = codes[d == d.min()]
        best = best[(best & 0x80) == (0x80 if x < 0 else 0)] if best.size > 1 else best
        if best.size > 1:  # a tie: the even mantissa
            best = best[(best & 1) == 0]
        assert best.size == 1 and g == best[0], (x, g, best)


def test_e4m3_encode_matches_torch_cast():
    """The same rounding as torch's float8_e4m3fn cast (round to nearest even) on fp32 values
    within the format's range."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-460, 460, 50000), rng.standard_normal(50000) * 2.0,
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 50000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(x.astype(np.float64)), ref)


def test_quantize_e4m3_b128_blocks():
    """Each block's largest magnitude becomes +-448 exactly (code 0x7E / 0xFE), the scale is
    the fp32 quotient amax / 448, an all-zero block has scale 1 and zero codes, and every value
    comes back within half a code step (relative 2^-4 for normals, 2^-10 * scale below 2^-6 *
    scale)."""
    rng = np.random.default_rng(3)
    z = (rng.standard_normal((5, 3, 512)) * np.exp(rng.uniform(-6, 6, (5, 3, 1)))).astype(np.float32)
    z[2, 1, 128:256] = 0.0
    codes, scale = O.quantize_e4m3_b128_fp32(z)
    assert codes.shape == z.shape and scale.shape == (5, 3, 4) and scale.dtype == np.float32
    zb = z.reshape(5, 3, 4, 128)
    amax = np.abs(zb).max(-1)
    np.testing.assert_array_equal(scale, np.where(amax > 0, amax / np.float32(448), np.float32(1)))
    assert scale[2, 1, 1] == 1.0 and np.all(codes.reshape(5, 3, 4, 128)[2, 1, 1] == 0)
    cb = codes.reshape(5, 3, 4, 128)
    k = np.abs(zb).argmax(-1)
    top = np.take_along_axis(cb, k[..., None], -1)[..., 0]
    nz = amax > 0
    assert np.all(np.isin(top[nz], [0x7E, 0xFE]))
    back = O.e4m3_decode(cb) * scale[..., None].astype(np.float64)
    err = np.abs(back - zb)
    bound = np.maximum(2.0 ** -4 * np.abs(zb), 2.0 ** -10 * scale[..., None])
    assert np.all(err <= bound * (1 + 1e-6))


@pytest.mark.parametrize("page_rows", [1, 5, 32])
def test_paged_pool_equals_contiguous(page_rows):
    """The same latent rows and cached state placed on shuffled pages instead of contiguous
    segment ranges: the oracle's results are identical (every row read through the page
    list lands on the row it stands for; unused pages hold NaN)."""
    from workload.gen import page_placement
    cfg = SMALL_CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    pages, n_pool, _ = page_placement(inp["kinds"], inp["lens"], page_rows, 5, share_docs=False)
    # the page list's pool row of every request row, written out here from the definition
    P = page_rows
    rows = []
    for i, L in enumerate(inp["lens"]):
        for j in range(int(L)):
            rows.append(int(pages["page_table"][pages["page_start"][i] + j // P]) * P + j % P)
    rows = np.asarray(rows)
    assert len(np.unique(rows)) == inp["T"]
    src = inp["pool_rows"][np.repeat(np.arange(len(inp["lens"])), inp["lens"])] + \
        (np.arange(inp["T"]) - np.repeat(inp["offsets"], inp["lens"]))
    paged = dict(inp)
    paged["pages"], paged["n_pool"] = pages, n_pool
    paged["latent"] = np.full((n_pool, inp["latent"].shape[1]), np.nan)
    paged["latent"][rows] = inp["latent"][src]
    paged["z_cached"] = np.full((n_pool,) + inp["z_cached"].shape[1:], np.nan)
    paged["z_cached"][rows] = inp["z_cached"][src]
    a, b = O.layer_forward(inp), O.layer_forward(paged)
    np.testing.assert_array_equal(a["A"], b["A"])
    for k in ("O", "Z", "lse"):
        np.testing.assert_array_equal(a[k], b[k])


def test_grouped_state_is_the_group_sum_of_per_head_state():
    """Grouped state (Eq. 3, z = z_L + z_G) against the per-head oracle: with the grouped cache
    holding each group's sum of the per-head cached Local rows, the grouped z of every row is the
    sum over the group's heads of the per-head z (computed heads on rows of A, Global heads plus
    the cache elsewhere), for groups with and without a Global head."""
    from workload.configs import GROUPED_CONFIGS
    cfg = GROUPED_CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    G, H = cfg["group_heads"], cfg["n_heads"]
    gmask = np.asarray(inp["head_is_global"]).astype(bool)
    local = np.nonzero(~gmask)[0]
    rng = np.random.default_rng(4)
    zc_h = rng.standard_normal((inp["n_pool"], len(local), cfg["d_state"]))
    zc_g = np.zeros((inp["n_pool"], H // G, cfg["d_state"]))
    for li, h in enumerate(local):
        zc_g[:, h // G] += zc_h[:, li]
    per_head = O.layer_forward(dict(inp, z_cached=zc_h))
    grouped = O.layer_forward_grouped(dict(inp, z_cached=zc_g))
    np.testing.assert_array_equal(grouped["A"], per_head["A"])
    ref = per_head["Z"].reshape(len(per_head["rows"]), H // G, G, -1).sum(axis=2)
    np.testing.assert_allclose(grouped["Z"], ref, rtol=0, atol=1e-12)
    assert not gmask[G:2 * G].any()  # the second group has no Global head
    outside = np.setdiff1d(np.arange(inp["T"]), per_head["A"])
    np.testing.assert_allclose(grouped["Z"][outside, 1], zc_g[grouped["geom"]["pool_of_row"][outside], 1],
                               rtol=0, atol=0)


def test_rope_blocks_on_zero_rows():
    """The RoPE helper on an empty set of rows (a request whose segments hold no compressed
    entry) returns an empty result instead of failing."""
    theta = O.rope_theta(64, 10000.0)
    R = O.rot_blocks(np.zeros(0), theta)
    y = O.apply_blocks(R, np.zeros((0, 64)))
    assert y.shape == (0, 64)


def test_grouped_state_without_local_heads_reads_no_cache():
    """A grouped layer whose heads are all Global has no Local contribution (Eq. 3 with
    z_L = 0): its grouped z is the group sum of the per-head z on every row, whatever the
    cached state holds (here NaN: it is not read)."""
    from workload.configs import GROUPED_CONFIGS
    cfg = dict(GROUPED_CONFIGS[0], name="tiny_fp32_grouped_all_global",
               global_heads=list(range(GROUPED_CONFIGS[0]["n_heads"])))
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    G, H = cfg["group_heads"], cfg["n_heads"]
    per_head = O.layer_forward(dict(inp, z_cached=np.zeros((inp["n_pool"], 0, cfg["d_state"]))))
    nan_cache = np.full((inp["n_pool"], H // G, cfg["d_state"]), np.nan)
    grouped = O.layer_forward_grouped(dict(inp, z_cached=nan_cache))
    assert len(grouped["A"]) < inp["T"]  # rows outside A exist
    ref = per_head["Z"].reshape(len(per_head["rows"]), H // G, G, -1).sum(axis=2)
    np.testing.assert_allclose(grouped["Z"], ref, rtol=0, atol=1e-12)


def test_grouped_exact_cache_identity():
    """When the cached Local contribution of every group equals the full recomputation's (the
    cache was produced in the same context), the grouped state equals full recomputation on
    every row, whatever A is (Eq. 4 as an exact linear identity)."""
    from workload.configs import GROUPED_CONFIGS
    cfg = GROUPED_CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    G, H, T = cfg["group_heads"], cfg["n_heads"], inp["T"]
    full = O.layer_forward(inp, A_override=np.arange(T))  # every head on every row
    gmask = np.asarray(inp["head_is_global"]).astype(bool)
    zc_g = np.full((inp["n_pool"], H // G, cfg["d_state"]), np.nan)
    pool = full["geom"]["pool_of_row"]
    for g in range(H // G):
        heads = [h for h in range(g * G, (g + 1) * G) if not gmask[h]]
        zc_g[pool, g] = full["Z"][:, heads].sum(axis=1)
    grouped = O.layer_forward_grouped(dict(inp, z_cached=zc_g))
    ref = full["Z"].reshape(T, H // G, G, -1).sum(axis=2)
    assert len(grouped["A"]) < T
    np.testing.assert_allclose(grouped["Z"], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------ error metric
def test_rel_err_rows_hand_values():
    """The pass/fail metric of every parity check: per (row, head), the L2 norm of the error
    over the channel axis divided by the L2 norm of the reference over the same axis (the
    per-head output L2 norm of the stated tolerances, taken row by row). Hand-computed
    values: a wrong axis, a denominator taken from x instead of ref, a missing square root
    or a mean instead of a sum each change at least one of them."""
    ref = np.array([[3.0, 4.0], [0.0, 5.0], [1.0, 0.0]])
    # identical rows: zero error
    np.testing.assert_array_equal(O.rel_err_rows(ref, ref), [0.0, 0.0, 0.0])
    # row 0 off by (0, 0); row 1 x = 0 (error = the whole row, ratio 1); row 2 x = 3 ref
    x = np.array([[3.0, 4.0], [0.0, 0.0], [3.0, 0.0]])
    np.testing.assert_array_equal(O.rel_err_rows(x, ref), [0.0, 1.0, 2.0])
    # denominator is ||ref||, not ||x||: x = 2 ref gives 1 (||x||-based would give 0.5)
    np.testing.assert_array_equal(O.rel_err_rows(2 * ref, ref), [1.0, 1.0, 1.0])
    # a known error vector per row: ||(0.3, 0.4)|| / ||(3, 4)|| = 0.5 / 5 = 0.1
    got = O.rel_err_rows(ref + np.array([[0.3, 0.4], [1.2, 0.0], [0.0, 0.25]]), ref)
    np.testing.assert_allclose(got, [0.1, 0.24, 0.25], rtol=0, atol=1e-15)
    # three axes [rows, heads, channels]: one value per (row, head), reduced over the last
    # axis only; the same numbers along the other two axes would give other values
    ref3 = np.zeros((2, 3, 4))
    ref3[..., 0] = 2.0                       # ||ref|| = 2 for every (row, head)
    x3 = ref3.copy()
    x3[1, 2, 3] = 1.0                        # one error of 1 in (row 1, head 2)
    e3 = O.rel_err_rows(x3, ref3)
    assert e3.shape == (2, 3)
    expect = np.zeros((2, 3))
    expect[1, 2] = 0.5
    np.testing.assert_array_equal(e3, expect)
    # a zero reference row with a nonzero x is an infinite relative error, never a pass
    assert O.rel_err_rows(np.array([[1e-3, 0.0]]), np.array([[0.0, 0.0]]))[0] > 1e100


# ------------------------------------------------------------------ sink + window heads
def test_window_printed_example():
    """RedKnot explainer, "Insight 1: heads have different jobs": with a window of w = 256,
    token 1000 of a local head needs tokens 744-1000 and the sink."""
    vis = O.window_visible(1000, n_sink=4, window=256)
    assert len(vis) == 1001
    np.testing.assert_array_equal(np.nonzero(vis)[0], np.r_[0:4, 744:1001])
    # a row inside the sink's reach sees a contiguous prefix; row 0 sees itself
    np.testing.assert_array_equal(np.nonzero(O.window_visible(200, 4, 256))[0], np.arange(201))
    np.testing.assert_array_equal(np.nonzero(O.window_visible(0, 0, 0))[0], [0])
    np.testing.assert_array_equal(np.nonzero(O.window_visible(10, 0, 0))[0], [10])
    assert O.window_pairs(1000, 1001, 4, 256) == 261


def _role_inputs(cfg, roles, n_sink, window, pool="identity"):
    inp = _oracle_inputs(make_inputs(cfg, "cpu", pool=pool))
    inp["head_is_global"] = np.asarray(roles, dtype=np.uint8)
    inp["cfg"] = dict(cfg, n_sink=n_sink, window=window)
    n_local = int(np.sum(np.asarray(roles) == 0))
    inp["z_cached"] = inp["z_cached"][:, :n_local]
    return inp


def test_window_brute_force_tiny():
    """Sink + window heads on an 11-row request (d_nope = d_rope = 2): raw unrotated vectors,
    explicit 2x2 matrices, the key set enumerated position by position, unshifted softmax."""
    rng = np.random.default_rng(5)
    kinds = np.array([0, 1, 1, 2], dtype=np.uint8)
    lens = np.array([2, 3, 4, 2])
    offsets = np.array([0, 2, 5, 9])
    T, H, n_sink, w = 11, 3, 2, 3
    kh = rng.normal(size=(T, 4))
    qh = rng.normal(size=(T, H, 4))
    seg = np.repeat(np.arange(4), lens)
    j = np.arange(T) - offsets[seg]
    stored_pos = np.where(kinds[seg] == 1, j, np.arange(T))
    lat, q = kh.copy(), qh.copy()
    for p in range(T):
        lat[p, 2:] = _rot2(stored_pos[p]) @ kh[p, 2:]
        for h in range(H):
            q[p, h, 2:] = _rot2(p) @ qh[p, h, 2:]
    Wp = rng.normal(size=(H, 3, 4))
    cfg = dict(d_nope=2, d_rope=2, rope_base=10000.0, softmax_scale=0.9, v_has_rope=1,
               edge_rows=1, tail_rows=2, budget_permille=0, n_sink=n_sink, window=w)
    inp = dict(cfg=cfg, kinds=kinds, lens=lens, offsets=offsets, pool_rows=offsets, n_pool=T,
               head_is_global=np.array([2, 1, 2], dtype=np.uint8), q=q, latent=lat, w=Wp,
               z_cached=np.zeros((T, 0, 3)), scores=np.zeros(T))
    res = O.layer_forward(inp)
    assert res["computed"].all()
    for t in range(T):
        for h in (0, 2):
            keys = [p for p in range(t + 1) if p < n_sink or t - w <= p]
            sc = np.array([0.9 * float(q[t, h] @ np.concatenate([kh[p, :2], _rot2(p) @ kh[p, 2:]]))
                           for p in keys])
            P = np.exp(sc) / np.exp(sc).sum()
            o, u = np.zeros(4), np.zeros(4)
            for pk, p in zip(P, keys):
                o[:2] += pk * kh[p, :2]
                o[2:] += pk * (_rot2(p) @ kh[p, 2:])
                u[:2] += pk * kh[p, :2]
                u[2:] += pk * (_rot2(p - t) @ kh[p, 2:])
            np.testing.assert_allclose(res["O"][t, h], o, rtol=0, atol=1e-13)
            np.testing.assert_allclose(res["Z"][t, h], Wp[h] @ u, rtol=0, atol=1e-12)
            np.testing.assert_allclose(res["lse"][t, h], np.log(np.exp(sc).sum()), rtol=0, atol=1e-12)


def test_window_special_cases():
    """A window reaching row 0 (or a sink covering the request) is full causal attention; a
    zero window without sink is each row attending to itself alone (O = the row's own value,
    whatever the query)."""
    cfg = CONFIGS[0]
    T = 274
    roles = [1, 2, 2, 0, 0, 2, 0, 0]
    full = O.layer_forward(_role_inputs(cfg, [1 if r == 2 else r for r in roles], 0, 0))
    for n_sink, w in ((0, T), (T, 0), (5, T - 1)):
        res = O.layer_forward(_role_inputs(cfg, roles, n_sink, w))
        for h in (1, 2, 5):
            np.testing.assert_allclose(res["O"][:, h], full["O"][:, h], rtol=0, atol=1e-13)
            np.testing.assert_allclose(res["Z"][:, h], full["Z"][:, h], rtol=0, atol=1e-12)
    inp = _role_inputs(cfg, roles, 0, 0)
    res = O.layer_forward(inp)
    keys = O.relocated_keys(inp["latent"], res["geom"], cfg["d_nope"], cfg["d_rope"], cfg["rope_base"])
    for h in (1, 2, 5):
        np.testing.assert_allclose(res["O"][:, h], keys, rtol=0, atol=1e-13)
        np.testing.assert_allclose(res["lse"][:, h], np.einsum("td,td->t", inp["q"][:, h], keys),
                                   rtol=0, atol=1e-12)
    # Local heads outside A still copy the cache and Global heads keep full context
    np.testing.assert_allclose(res["O"][:, 0], full["O"][:, 0], rtol=0, atol=1e-13)


def test_window_sdpa_float64_pin():
    """Library routine: torch scaled_dot_product_attention in float64 with an explicit boolean
    mask (key p visible from row t iff p <= t and (p < n_sink or p >= t - w)), built here
    from the index grids, on the physically re-rotated keys."""
    cfg = SMALL_CONFIGS[0]
    roles = [1, 2, 0, 2, 0, 0, 2, 0]
    n_sink, w = 3, 40
    inp = _role_inputs(cfg, roles, n_sink, w)
    res = O.layer_forward(inp)
    keys = O.relocated_keys(inp["latent"], res["geom"], cfg["d_nope"], cfg["d_rope"], cfg["rope_base"])
    T = len(keys)
    tt, pp = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    mask = torch.from_numpy((pp <= tt) & ((pp < n_sink) | (pp >= tt - w)))
    kt = torch.from_numpy(keys)[None, None]
    for h in (1, 3, 6):
        qt = torch.from_numpy(np.ascontiguousarray(inp["q"][:, h]))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, kt, attn_mask=mask, scale=cfg["softmax_scale"])[0, 0].numpy()
        np.testing.assert_allclose(res["O"][:, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["identity", "shuffled", "paged:16"])
def test_window_relocation_identity(mode):
    """Sink + window heads under relocation: the independent segmented fp64 computation (rotate
    q per segment, attend the stored latent, restore the phase, log-sum-exp merge) restricted
    to each row's window equals the oracle on physically re-rotated keys, across windows that
    span segment boundaries."""
    cfg = SMALL_CONFIGS[0]
    roles = [2] * 8
    n_sink, w = 2, 60
    inp = _role_inputs(cfg, roles, n_sink, w, pool=mode)
    T = inp["T"]
    rows = sorted(set([0, 1, 5, 70, 71, T - 1] + list(np.random.default_rng(2).choice(T, 20, replace=False))))
    res = O.layer_forward(inp, rows=rows)
    seg = _segmented_fp64(inp, rows, np.random.default_rng(3),
                          visible=lambda t, pos: (pos < n_sink) | (pos >= t - w))
    for i, t in enumerate(rows):
        np.testing.assert_allclose(res["O"][i], seg[t], rtol=0, atol=1e-10)


def test_window_pairs_brute_force():
    for n_sink, w in ((0, 0), (4, 256), (3, 10), (1000, 5)):
        for q0, q1 in ((0, 1), (0, 300), (250, 700), (999, 1300)):
            brute = sum(1 for t in range(q0, q1) for p in range(t + 1) if p < n_sink or p >= t - w)
            assert O.window_pairs(q0, q1, n_sink, w) == brute
