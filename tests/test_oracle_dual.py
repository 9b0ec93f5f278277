"""Pins of the oracle's compressed-history (dual-pool) attention against things other than
itself: hand-counted entry availability, brute force with explicit 2x2 rotations on a tiny
request, torch's float64 attention with an explicit additive mask, the sink + window oracle it
reduces to, and the method's own per-segment computation (rotate q, attend the stored rows in
place, restore the phase, log-sum-exp merge) written independently.

Source: "Reading notes on DeepSeek-V4 serving in TensorRT-LLM", section 1 (the hybrid attention
bullets and the dual-pool kernel paragraph); relocation as in the RedKnot-MLA paper, relocation
paragraph (Eq. 5).
"""
import math

import numpy as np
import pytest
import torch

from oracle import segmla_oracle as O
from workload import CONFIGS, SMALL_CONFIGS, make_dual_inputs, make_inputs


def _oracle_inputs(inp):
    d = dict(inp)
    d["latent"] = inp["kv"].double().numpy()
    d["q"] = inp["q"].double().numpy()
    return d


def _dual(dual_inp):
    d = dict(dual_inp)
    d["centries"] = dual_inp["ckv"].double().numpy()
    return d


def _rot2(angle):
    c, s = math.cos(angle), math.sin(angle)
    return np.array([[c, -s], [s, c]])


def test_entry_availability_hand_counted():
    """Segments of 6, 9 and 4 rows at offsets 0, 6, 15 compressed 4 to 1: 1, 2 and 1 entries.
    Segment 1's entries stand for its rows 0..3 and 4..7 (request rows 6..9 and 10..13), so
    request row 9 is the first to see the first of them and row 13 the second. With disjoint
    windows of 128 (HCA), a 300-row document holds 2 entries, seen from rows 127 and 255."""
    g = O.geometry([0, 1, 2], [6, 9, 4], [0, 6, 15], [0, 6, 15], 19)
    ce = O.compressed_entries(g, 4, [10, 0, 5], 11)
    assert ce["n"] == 4
    np.testing.assert_array_equal(ce["seg"], [0, 1, 1, 2])
    np.testing.assert_array_equal(ce["pool"], [10, 0, 1, 5])
    np.testing.assert_array_equal(ce["first_row"], [3, 9, 13, 18])
    np.testing.assert_array_equal(O.entries_of_row(ce, 12), [0, 1])
    np.testing.assert_array_equal(O.entries_of_row(ce, 13), [0, 1, 2])
    np.testing.assert_array_equal(O.entries_of_row(ce, 2), [])
    # a list is read up to its first id that is not available at the row
    np.testing.assert_array_equal(O.entries_of_row(ce, 13, [2, 0, 3, 1], 4), [2, 0])
    np.testing.assert_array_equal(O.entries_of_row(ce, 18, [2, 0, 2, -1, 1], 5), [2, 0, 2])
    np.testing.assert_array_equal(O.entries_of_row(ce, 18, [3, 1, 0], 2), [3, 1])
    g = O.geometry([1, 2], [300, 100], [0, 300], [0, 300], 400)
    ce = O.compressed_entries(g, 128, [0, 2], 2)
    np.testing.assert_array_equal(ce["first_row"], [127, 255])
    np.testing.assert_array_equal(ce["count"], [2, 0])
    with pytest.raises(ValueError):
        O.compressed_entries(g, 128, [0, 2], 1)


def test_dual_brute_force_tiny():
    """An 11-row request (d_nope = d_rope = 2, theta_0 = 1), entries of 2 rows: the true
    request-frame content of every raw row and entry is drawn, stored in its segment's frame
    (documents canonical, prefix and new rows at request positions), and each row's key list
    is enumerated by hand; softmax without max subtraction."""
    rng = np.random.default_rng(11)
    kinds = np.array([0, 1, 1, 2], dtype=np.uint8)
    lens = np.array([2, 3, 4, 2])
    offsets = np.array([0, 2, 5, 9])
    T, H, m, w = 11, 2, 2, 2
    shift = np.where(kinds == 1, offsets, 0)           # stored frame -> request frame
    kh = rng.normal(size=(T, 4))                        # raw rows, request frame content
    qh = rng.normal(size=(T, H, 4))
    seg = np.repeat(np.arange(4), lens)
    lat = kh.copy()
    q = qh.copy()
    for p in range(T):
        lat[p, 2:] = _rot2(p - shift[seg[p]]) @ kh[p, 2:]
        for h in range(H):
            q[p, h, 2:] = _rot2(p) @ qh[p, h, 2:]
    # entries per segment: floor(len / 2) = 1, 1, 2, 1; pool rows reversed per segment
    cnt = lens // m
    cpool_rows = np.array([5, 3, 0, 2])
    n_cpool = 6
    ce_true = rng.normal(size=(n_cpool, 4))            # request-frame content of each pool row
    cent = ce_true.copy()
    entry_seg, entry_first = [], []
    for i in range(4):
        for j in range(cnt[i]):
            r = cpool_rows[i] + j
            cent[r, 2:] = _rot2(-shift[i]) @ ce_true[r, 2:]
            entry_seg.append((i, r))
            entry_first.append(offsets[i] + m * j + m - 1)
    cfg = dict(d_nope=2, d_rope=2, rope_base=10000.0, softmax_scale=0.8, v_has_rope=1)
    inp = dict(cfg=cfg, kinds=kinds, lens=lens, offsets=offsets, pool_rows=offsets, n_pool=T,
               q=q, latent=lat)
    dual = dict(ratio=m, window=w, cpool_rows=cpool_rows, n_cpool=n_cpool, centries=cent)
    lists = [rng.permutation(len(entry_seg)) for _ in range(T)]
    lens_l = [int(rng.integers(0, len(entry_seg) + 1)) for _ in range(T)]
    for mode in ("hca", "csa"):
        res = O.dual_pool_forward(inp, dual, np.arange(T), *(
            (None, None) if mode == "hca" else (lists, lens_l)))
        for t in range(T):
            if mode == "hca":
                ents = [e for e in range(len(entry_seg)) if entry_first[e] <= t]
            else:
                ents = []
                for e in lists[t][:lens_l[t]]:
                    if entry_first[e] > t:
                        break
                    ents.append(e)
            keys = [np.concatenate([kh[p, :2], _rot2(p) @ kh[p, 2:]])
                    for p in range(max(0, t - w), t + 1)]
            keys += [ce_true[entry_seg[e][1]] for e in ents]
            assert res["n_keys"][t] == len(keys)
            for h in range(H):
                sc = np.array([0.8 * float(q[t, h] @ k) for k in keys])
                e = np.exp(sc)
                o = sum(pe * k for pe, k in zip(e / e.sum(), keys))
                np.testing.assert_allclose(res["O"][t, h], o, rtol=0, atol=1e-13)
                np.testing.assert_allclose(res["lse"][t, h], np.log(e.sum()), rtol=0, atol=1e-12)


def test_dual_hca_ratio_one_sdpa_float64():
    """Library routine: with ratio 1 and the compressed pool equal to the latent pool, HCA
    sees every raw key p <= t once as an entry and the window's keys once more, which is
    softmax attention over the keys p <= t with log(2) added to the window's scores: torch
    scaled_dot_product_attention in float64 with that additive mask, built here from the index
    grids, on the physically re-rotated keys."""
    cfg = CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    w = 17
    dual = dict(ratio=1, window=w, cpool_rows=inp["pool_rows"], n_cpool=inp["n_pool"],
                centries=inp["latent"])
    T = inp["T"]
    res = O.dual_pool_forward(inp, dual, np.arange(T))
    g = O.geometry(inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"], inp["n_pool"])
    keys = O.relocated_keys(inp["latent"], g, cfg["d_nope"], cfg["d_rope"], cfg["rope_base"])
    tt, pp = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    bias = np.where(pp > tt, -np.inf, np.where(pp >= tt - w, math.log(2.0), 0.0))
    kt = torch.from_numpy(keys)[None, None]
    for h in range(cfg["n_heads"]):
        qt = torch.from_numpy(np.ascontiguousarray(inp["q"][:, h]))[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, kt, attn_mask=torch.from_numpy(bias), scale=cfg["softmax_scale"])[0, 0].numpy()
        np.testing.assert_allclose(res["O"][:, h], ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(res["n_keys"], np.arange(T) + 1 + np.minimum(np.arange(T), w) + 1)


def test_dual_empty_lists_are_the_window_heads():
    """CSA rows whose lists are empty attend the recent window alone: the sink + window oracle
    with no sink (pinned separately against brute force and torch)."""
    cfg = SMALL_CONFIGS[0]
    inp = _oracle_inputs(make_inputs(cfg, "cpu"))
    dual = _dual(make_dual_inputs(make_inputs(cfg, "cpu"), 4, 30, 8))
    T = inp["T"]
    rows = np.arange(0, T, 7)
    res = O.dual_pool_forward(inp, dual, rows, [np.zeros(8, dtype=np.int64)] * len(rows),
                              [0] * len(rows))
    g = O.geometry(inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"], inp["n_pool"])
    keys = O.relocated_keys(inp["latent"], g, cfg["d_nope"], cfg["d_rope"], cfg["rope_base"])
    d_v = cfg["d_nope"] + cfg["d_rope"]
    Ow, lw = O.attend_rows_window(inp["q"][rows], rows, keys, cfg["softmax_scale"], d_v, 0, 30)
    np.testing.assert_allclose(res["O"], Ow, rtol=0, atol=1e-13)
    np.testing.assert_allclose(res["lse"], lw, rtol=0, atol=1e-12)


def test_dual_list_forms():
    """A CSA list holding every available entry is HCA; the order of a list does not matter;
    an unavailable id cuts the list where it stands; a repeated id counts twice, which is the
    entry's score raised by log(2)."""
    cfg = SMALL_CONFIGS[0]
    raw = make_inputs(cfg, "cpu", pool="shuffled")
    inp = _oracle_inputs(raw)
    dual = _dual(make_dual_inputs(raw, 4, 20, 8, pool="shuffled"))
    T = inp["T"]
    rng = np.random.default_rng(4)
    rows = np.array(sorted(set([3, 4, 40, T - 1] + list(rng.choice(T, 12, replace=False)))))
    hca = O.dual_pool_forward(inp, dual, rows)
    ce = hca["ce"]
    full = [O.entries_of_row(ce, t) for t in rows]
    csa = O.dual_pool_forward(inp, dual, rows, full, [len(x) for x in full])
    np.testing.assert_allclose(csa["O"], hca["O"], rtol=0, atol=1e-13)
    shuf = [rng.permutation(x) for x in full]
    csa2 = O.dual_pool_forward(inp, dual, rows, shuf, [len(x) for x in shuf])
    np.testing.assert_allclose(csa2["O"], hca["O"], rtol=0, atol=1e-13)
    short = [x[:3] for x in full]
    csa4 = O.dual_pool_forward(inp, dual, rows, short, [len(x) for x in short])
    for bad in (-1, ce["n"]):
        cut = [np.concatenate([x[:3], [bad], x[3:]]) for x in full]
        csa3 = O.dual_pool_forward(inp, dual, rows, cut, [len(x) for x in cut])
        np.testing.assert_allclose(csa3["O"], csa4["O"], rtol=0, atol=1e-13)
    # an entry not yet available (the last one, seen only from its last row on) cuts too
    i0 = int(np.flatnonzero(rows < ce["first_row"][-1])[-1])
    cut = [np.concatenate([full[i0][:3], [ce["n"] - 1], full[i0][3:]])]
    csa5 = O.dual_pool_forward(inp, dual, rows[i0:i0 + 1], cut, [len(cut[0])])
    np.testing.assert_allclose(csa5["O"], csa4["O"][i0:i0 + 1], rtol=0, atol=1e-13)
    # a repeated id: the same as adding log(2) to that entry's score, written out here
    i = int(np.flatnonzero([len(x) >= 2 for x in full])[-1])
    t, x = int(rows[i]), full[i]
    rep = O.dual_pool_forward(inp, dual, rows[i:i + 1], [np.concatenate([x, x[1:2]])], [len(x) + 1])
    g = O.geometry(inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"], inp["n_pool"])
    keys = O.relocated_keys(inp["latent"], g, cfg["d_nope"], cfg["d_rope"], cfg["rope_base"])
    ekeys = O.relocated_entries(dual["centries"], g, ce, cfg["d_nope"], cfg["d_rope"], cfg["rope_base"])
    K = np.concatenate([keys[max(0, t - 20):t + 1], ekeys[x]])
    bias = np.zeros(len(K))
    bias[len(K) - len(x) + 1] = math.log(2.0)
    s = cfg["softmax_scale"] * inp["q"][t] @ K.T + bias
    p = np.exp(s - s.max(axis=1, keepdims=True))
    np.testing.assert_allclose(rep["O"][0], (p @ K) / p.sum(axis=1, keepdims=True), rtol=0, atol=1e-13)


def _segmented_dual(inp, dual, rows, lists, list_lens, rng):
    """The method in fp64, written independently of the oracle: the row's keys are grouped by
    segment (raw window rows by request position, entries by the segment that holds them);
    per segment the query's RoPE part is rotated by -rot_i, scores are taken against the
    stored rows in place, the partial output's RoPE part is rotated back by +rot_i, and the
    (max, sum, partial) statistics are merged by a log-sum-exp merge in a random order."""
    cfg = inp["cfg"]
    dn, dr, base, sig = cfg["d_nope"], cfg["d_rope"], cfg["rope_base"], cfg["softmax_scale"]
    theta = base ** (-2.0 * np.arange(dr // 2) / dr)

    def rot(x, ang):
        y = x.copy()
        c, s = np.cos(ang), np.sin(ang)
        y[..., dn::2] = x[..., dn::2] * c - x[..., dn + 1::2] * s
        y[..., dn + 1::2] = x[..., dn::2] * s + x[..., dn + 1::2] * c
        return y

    kinds, lens, offs, pr = inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"]
    m, w = dual["ratio"], dual["window"]
    cnt = [int(n) // m for n in lens]
    cbase = np.concatenate([[0], np.cumsum(cnt)])
    out = {}
    for r, t in enumerate(rows):
        groups = {}
        for p in range(max(0, t - w), t + 1):
            i = int(np.searchsorted(offs, p, side="right") - 1)
            groups.setdefault(i, []).append(inp["latent"][pr[i] + p - offs[i]])
        if lists is None:
            ids = [c for i in range(len(lens)) for c in range(cbase[i], cbase[i + 1])
                   if offs[i] + m * (c - cbase[i]) + m - 1 <= t]
        else:
            ids = []
            for c in list(lists[r])[:list_lens[r]]:
                i = int(np.searchsorted(cbase, c, side="right") - 1) if 0 <= c < cbase[-1] else -1
                if i < 0 or offs[i] + m * (c - cbase[i]) + m - 1 > t:
                    break
                ids.append(c)
        for c in ids:
            i = int(np.searchsorted(cbase, c, side="right") - 1)
            groups.setdefault(i, []).append(dual["centries"][dual["cpool_rows"][i] + c - cbase[i]])
        stats = []
        for i, C in groups.items():
            C = np.array(C)
            rot_i = float(offs[i]) if kinds[i] == 1 else 0.0
            qr = rot(inp["q"][t], -rot_i * theta)
            s = sig * qr @ C.T
            mx = s.max(axis=1)
            e = np.exp(s - mx[:, None])
            stats.append((mx, e.sum(axis=1), rot(e @ C, rot_i * theta)))
        order = rng.permutation(len(stats))
        M = np.max([stats[i][0] for i in order], axis=0)
        num = sum(np.exp(stats[i][0] - M)[:, None] * stats[i][2] for i in order)
        den = sum(np.exp(stats[i][0] - M) * stats[i][1] for i in order)
        out[t] = num / den[:, None]
    return out


@pytest.mark.parametrize("pool,ratio,top_k", [("identity", 4, 0), ("shuffled", 4, 6),
                                              ("shuffled", 3, 0), ("identity", 16, 3)])
def test_dual_relocation_identity(pool, ratio, top_k):
    """The oracle (physically re-rotated raw rows and entries, one dense softmax) equals the
    method's per-segment rotate / attend / restore / merge computation, over windows and lists
    that span segment boundaries, on contiguous and shuffled pools."""
    cfg = SMALL_CONFIGS[0]
    raw = make_inputs(cfg, "cpu", pool=pool)
    inp = _oracle_inputs(raw)
    dual = _dual(make_dual_inputs(raw, ratio, 25, top_k, pool=pool))
    T = inp["T"]
    rows = sorted(set([0, 1, 9, 60, 61, T - 1] + list(np.random.default_rng(6).choice(T, 14, replace=False))))
    lists = lens_l = None
    if top_k:
        lists = [dual["cidx"][t].numpy() for t in rows]
        lens_l = [int(dual["clen"][t]) for t in rows]
    res = O.dual_pool_forward(inp, dual, rows, lists, lens_l)
    seg = _segmented_dual(inp, dual, rows, lists, lens_l, np.random.default_rng(8))
    for i, t in enumerate(rows):
        np.testing.assert_allclose(res["O"][i], seg[t], rtol=0, atol=1e-10)
