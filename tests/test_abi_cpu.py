"""C-ABI checks that need no GPU: exported symbols, host validation and error paths,
host-side sizing of the protected set, and the analytic ledger.

Every call here returns before any HIP call is made (validation happens first), so it
runs on a machine without a GPU.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import segmla_oracle as O
from workload import CONFIGS, SMALL_CONFIGS, segment_table
from workload.configs import FLASH_TAIL32K
from workload.gen import pool_placement

S = pytest.importorskip("segmented_attention_amd.segmla")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(S.LIB_PATH):
        pytest.skip("libsegmla.so not built")
    return S.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "segmla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(segmla_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    decl = _declared()
    assert len(decl) >= 13
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(S.EXPORTED) == decl


def test_abi_version_and_status_strings(L):
    assert S.segmla_abi_version() == 5
    for st in range(-9, 1):
        assert S.segmla_status_string(st) not in ("", "unknown status")
    assert S.segmla_status_string(-100) == "unknown status"


def _create(cfg, **over):
    kinds, lens, offsets = segment_table(cfg)
    pr, n_pool = pool_placement(lens, "identity", cfg["seed"])
    glob = np.zeros(cfg["n_heads"], np.uint8)
    glob[cfg["global_heads"]] = 1
    args = dict(kinds=kinds, lens=lens, offsets=offsets, pool_rows=pr, n_pool=n_pool,
                n_heads=cfg["n_heads"], head_is_global=glob, d_nope=cfg["d_nope"],
                d_rope=cfg["d_rope"], d_state=cfg["d_state"], v_has_rope=cfg["v_has_rope"],
                kv_dtype=S._DT[cfg["kv_dtype"]], io_dtype=S._DT[cfg["dtype"]],
                edge_rows=cfg["edge_rows"], tail_rows=cfg["tail_rows"],
                budget_permille=cfg["budget_permille"])
    args.update(over)
    return S.segmla_plan_create(**args)


def _status(cfg, **over):
    try:
        p = _create(cfg, **over)
    except S.SegmlaError as e:
        return e.status
    S.segmla_plan_destroy(p)
    return S.SEGMLA_OK


@pytest.mark.parametrize("cfg", CONFIGS + SMALL_CONFIGS + [FLASH_TAIL32K], ids=lambda c: c["name"])
def test_plan_rows_match_oracle(L, cfg):
    """|A| = |F| + need is fixed on the host by geometry and the protection rule."""
    p = _create(cfg)
    try:
        T, nA = S.segmla_plan_rows(p)
        kinds, lens, offsets = segment_table(cfg)
        g = O.geometry(kinds, lens, offsets, offsets, int(lens.sum()))
        scores = np.random.default_rng(0).integers(0, 2**32, g["T"], dtype=np.uint64)
        ref = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"],
                               scores=scores)
        assert T == g["T"] and nA == len(ref["A"])
        assert S.segmla_plan_workspace_bytes(p) > 0
    finally:
        S.segmla_plan_destroy(p)


def test_range_errors(L):
    """Row windows: 0 <= q_begin < q_end <= T (q_end = -1: T); |A| stays the request's."""
    cfg = SMALL_CONFIGS[1]
    kinds, lens, offsets = segment_table(cfg)
    T = int(lens.sum())
    full = _create(cfg)
    try:
        T0, nA0 = S.segmla_plan_rows(full)
    finally:
        S.segmla_plan_destroy(full)
    for rng in [(0, T), (0, -1), (0, 1), (T - 1, T), (37, 300)]:
        p = _create(cfg, q_range=rng)
        try:
            assert S.segmla_plan_rows(p) == (T0, nA0)
            assert S.segmla_plan_workspace_bytes(p) > 0
        finally:
            S.segmla_plan_destroy(p)
    for rng in [(-1, 5), (5, 5), (6, 5), (0, T + 1), (T, T + 1)]:
        assert _status(cfg, q_range=rng) == S.SEGMLA_E_SHAPE, rng


def test_paged_pool_errors(L):
    """Paged pool: every page a segment uses must be listed and lie inside the pool; a valid
    page list gives the same |A| and rows as the contiguous pool (A does not depend on where
    the rows are stored)."""
    from workload.gen import page_placement
    cfg = SMALL_CONFIGS[1]
    kinds, lens, offsets = segment_table(cfg)
    full = _create(cfg)
    try:
        rows0 = S.segmla_plan_rows(full)
    finally:
        S.segmla_plan_destroy(full)
    for P in (1, 32, 48, 64):
        pages, n_pool, _ = page_placement(kinds, lens, P, 3)
        p = _create(cfg, pages=pages, n_pool=n_pool, pool_rows=np.zeros(len(lens), np.int64))
        try:
            assert S.segmla_plan_rows(p) == rows0
        finally:
            S.segmla_plan_destroy(p)
    pages, n_pool, _ = page_placement(kinds, lens, 64, 3)

    def st(**pg):
        d = dict(pages)
        d.update(pg)
        return _status(cfg, pages=d, n_pool=n_pool)
    assert st() == S.SEGMLA_OK
    assert st(page_rows=0) == S.SEGMLA_E_GEOMETRY
    bad = pages["page_start"].copy()
    bad[-1] = len(pages["page_table"])  # the last segment's pages past the list
    assert st(page_start=bad) == S.SEGMLA_E_GEOMETRY
    bad = pages["page_start"].copy()
    bad[0] = -1
    assert st(page_start=bad) == S.SEGMLA_E_GEOMETRY
    tbl = pages["page_table"].copy()
    tbl[0] = n_pool // 64  # one page past the pool
    assert st(page_table=tbl) == S.SEGMLA_E_GEOMETRY
    tbl[0] = -1
    assert st(page_table=tbl) == S.SEGMLA_E_GEOMETRY
    from workload.gen import pool_rows_of
    last = int(pool_rows_of(lens, pages).max())  # the highest pool row any segment uses
    assert _status(cfg, pages=pages, n_pool=last + 1) == S.SEGMLA_OK
    assert _status(cfg, pages=pages, n_pool=last) == S.SEGMLA_E_GEOMETRY


def test_paged_pool_smaller_than_one_page(L):
    """A pool smaller than the rows a segment uses on its first page is rejected (the check
    must not round a negative room up to page 0): one 50-row document on 64-row pages needs
    pool rows 0..49, so n_pool = 32 or 49 is an error and 50 is enough."""
    cfg = dict(SMALL_CONFIGS[1], segments=[("doc", 50)])
    one = dict(page_rows=64, page_start=np.array([0], np.int64),
               page_table=np.array([0], np.int64))
    for n_pool, want in ((32, S.SEGMLA_E_GEOMETRY), (49, S.SEGMLA_E_GEOMETRY),
                         (50, S.SEGMLA_OK), (64, S.SEGMLA_OK)):
        got = _status(cfg, kinds=[1], lens=[50], offsets=[0], pool_rows=[0], n_pool=n_pool,
                      pages=one, edge_rows=0, tail_rows=0, budget_permille=0)
        assert got == want, (n_pool, got)
    # the unpaged geometry gives the same verdicts
    for n_pool, want in ((49, S.SEGMLA_E_GEOMETRY), (50, S.SEGMLA_OK)):
        got = _status(cfg, kinds=[1], lens=[50], offsets=[0], pool_rows=[0], n_pool=n_pool,
                      edge_rows=0, tail_rows=0, budget_permille=0)
        assert got == want, (n_pool, got)
    # a page index so large that page * rows overflows int64 is rejected, not wrapped
    huge = dict(one, page_table=np.array([2**62], np.int64))
    assert _status(cfg, kinds=[1], lens=[50], offsets=[0], pool_rows=[0], n_pool=64,
                   pages=huge, edge_rows=0, tail_rows=0, budget_permille=0) == S.SEGMLA_E_GEOMETRY


def test_group_heads_errors(L):
    """Grouped state: group_heads 0 or 1 is per head; G >= 2 must divide n_heads; negative is
    an error. A valid grouping changes neither T nor |A|."""
    cfg = SMALL_CONFIGS[1]  # 64 heads
    base = _create(cfg)
    try:
        rows0 = S.segmla_plan_rows(base)
    finally:
        S.segmla_plan_destroy(base)
    for G in (0, 1, 2, 8, 64):
        p = _create(cfg, group_heads=G)
        try:
            assert S.segmla_plan_rows(p) == rows0
        finally:
            S.segmla_plan_destroy(p)
    for G in (-1, 3, 7, 65):
        assert _status(cfg, group_heads=G) == S.SEGMLA_E_SHAPE, G


def test_e4m3_state_errors(L):
    """The E4M3 output of the projected state needs bf16 io, grouped state and d_state a
    multiple of 128 (else SEGMLA_E_SHAPE); the plan reports it, and a forward without the scale
    buffer is SEGMLA_E_NULL before any device work; the binding asks for uint8 codes and the
    scales."""
    import torch
    cfg = SMALL_CONFIGS[1]  # bf16, 64 heads, d_state 512
    assert _status(cfg, group_heads=8, z_e4m3=1) == S.SEGMLA_OK
    assert _status(cfg, group_heads=0, z_e4m3=1) == S.SEGMLA_E_SHAPE
    assert _status(cfg, group_heads=8, z_e4m3=2) == S.SEGMLA_E_SHAPE
    assert _status(cfg, group_heads=8, z_e4m3=1, d_state=192) == S.SEGMLA_E_SHAPE
    assert _status(SMALL_CONFIGS[0], group_heads=4, z_e4m3=1) == S.SEGMLA_E_SHAPE  # fp32 io
    p = _create(cfg, group_heads=8, z_e4m3=1)
    try:
        info = S.segmla_plan_get_info(p)
        assert info["z_e4m3"] == 1 and info["z_slots"] == 8
        T = info["T"]
        lib = S.lib()
        need = S.segmla_plan_workspace_bytes(p)
        p0 = _create(cfg, group_heads=8)
        try:  # the bf16 state before quantization: T x 8 groups x 512 x 2 bytes more workspace
            assert need - S.segmla_plan_workspace_bytes(p0) >= T * 8 * 512 * 2
        finally:
            S.segmla_plan_destroy(p0)
        bf = torch.bfloat16
        good = dict(q=torch.zeros(T, 64, 576, dtype=bf), kv=torch.zeros(T, 576, dtype=bf),
                    w=torch.zeros(64, 512, 576, dtype=bf), out=torch.zeros(T, 64, 576, dtype=bf),
                    z=torch.zeros(T, 8, 512, dtype=torch.uint8),
                    z_cached=torch.zeros(T, 8, 512, dtype=bf),
                    z_scale=torch.zeros(T, 8, 4, dtype=torch.float32))

        def err(**over):
            args = dict(good)
            args.update(over)
            with pytest.raises(ValueError) as e:
                S.segmla_forward(p, **args)
            return str(e.value)
        assert "q must be on the GPU" in err()
        assert "z has dtype" in err(z=torch.zeros(T, 8, 512, dtype=bf))
        assert "z_scale is required" in err(z_scale=None)
        assert "z_scale holds" in err(z_scale=torch.zeros(T, 8, 3))
        if _no_gpu():  # a built plan needs a device; the NULL check comes first on the host
            t = S.Tensors()
            assert lib.segmla_forward(p, ctypes.byref(t), None) == S.SEGMLA_E_STATE
    finally:
        S.segmla_plan_destroy(p)
    p = _create(cfg, group_heads=8)
    try:
        with pytest.raises(ValueError, match="z_scale is given"):
            S.segmla_forward(p, q=None, kv=None, w=None, out=None, z=None,
                             z_scale=torch.zeros(4))
    finally:
        S.segmla_plan_destroy(p)


def test_geometry_errors(L):
    cfg = SMALL_CONFIGS[1]
    kinds, lens, offsets = segment_table(cfg)
    pr, n_pool = pool_placement(lens, "identity", 0)
    bad_off = offsets.copy()
    bad_off[2] += 1
    assert _status(cfg, offsets=bad_off) == S.SEGMLA_E_GEOMETRY
    first = offsets.copy()
    first += 3
    assert _status(cfg, offsets=first) == S.SEGMLA_E_GEOMETRY
    zero_len = lens.copy()
    zero_len[1] = 0
    assert _status(cfg, lens=zero_len) == S.SEGMLA_E_GEOMETRY
    bad_kind = kinds.copy()
    bad_kind[0] = 7
    assert _status(cfg, kinds=bad_kind) == S.SEGMLA_E_GEOMETRY
    out_of_pool = pr.copy()
    out_of_pool[-1] = n_pool - lens[-1] + 1
    assert _status(cfg, pool_rows=out_of_pool) == S.SEGMLA_E_GEOMETRY
    neg_pool = pr.copy()
    neg_pool[0] = -1
    assert _status(cfg, pool_rows=neg_pool) == S.SEGMLA_E_GEOMETRY
    assert _status(cfg, n_pool=0) == S.SEGMLA_E_GEOMETRY
    # aliased pool ranges are legal
    alias = pr.copy()
    alias[2] = alias[1]
    assert _status(cfg, pool_rows=alias) == S.SEGMLA_OK
    # an empty request (no segment) has no rows to compute
    none = np.zeros(0, np.int64)
    assert _status(cfg, kinds=np.zeros(0, np.uint8), lens=np.zeros(0, np.int32), offsets=none,
                   pool_rows=none) == S.SEGMLA_E_GEOMETRY


def test_shape_dtype_protect_errors(L):
    cfg = SMALL_CONFIGS[1]
    assert _status(cfg, n_heads=0, head_is_global=np.zeros(0, np.uint8)) == S.SEGMLA_E_SHAPE
    assert _status(cfg, d_rope=63) == S.SEGMLA_E_SHAPE
    assert _status(cfg, d_state=0) == S.SEGMLA_E_SHAPE
    assert _status(cfg, v_has_rope=2) == S.SEGMLA_E_SHAPE
    assert _status(cfg, rope_base=1.0) == S.SEGMLA_E_SHAPE
    assert _status(cfg, softmax_scale=0.0) == S.SEGMLA_E_SHAPE
    assert _status(cfg, softmax_scale=float("nan")) == S.SEGMLA_E_SHAPE
    glob = np.zeros(cfg["n_heads"], np.uint8)
    glob[3] = 3                                   # roles are 0, 1 or 2
    assert _status(cfg, head_is_global=glob) == S.SEGMLA_E_SHAPE
    glob[3] = 2                                   # a sink + window head
    assert _status(cfg, head_is_global=glob, n_sink=4, window=16) == S.SEGMLA_OK
    assert _status(cfg, head_is_global=glob, n_sink=-1, window=16) == S.SEGMLA_E_SHAPE
    assert _status(cfg, head_is_global=glob, n_sink=0, window=-1) == S.SEGMLA_E_SHAPE
    assert _status(cfg, split_keys=100) == S.SEGMLA_E_SHAPE
    assert _status(cfg, split_keys=-2) == S.SEGMLA_E_SHAPE
    assert _status(cfg, kv_dtype=9) == S.SEGMLA_E_DTYPE
    assert _status(cfg, io_dtype=S.SEGMLA_E4M3_B128) == S.SEGMLA_E_DTYPE
    assert _status(cfg, io_dtype=S.SEGMLA_F32) == S.SEGMLA_E_UNSUPPORTED
    assert _status(cfg, d_nope=256) == S.SEGMLA_E_UNSUPPORTED
    assert _status(cfg, d_state=100) == S.SEGMLA_E_UNSUPPORTED
    tiny = CONFIGS[0]
    assert _status(tiny, io_dtype=S.SEGMLA_BF16) == S.SEGMLA_E_UNSUPPORTED
    assert _status(tiny, d_nope=63) == S.SEGMLA_E_UNSUPPORTED
    assert _status(cfg, edge_rows=-1) == S.SEGMLA_E_PROTECT
    assert _status(cfg, tail_rows=-5) == S.SEGMLA_E_PROTECT
    assert _status(cfg, budget_permille=1001) == S.SEGMLA_E_PROTECT
    assert _status(cfg, budget_permille=-1) == S.SEGMLA_E_PROTECT
    kinds, lens, _ = segment_table(cfg)
    assert _status(cfg, dirty_rows=[int(lens.sum())]) == S.SEGMLA_E_PROTECT
    assert _status(cfg, dirty_rows=[-1]) == S.SEGMLA_E_PROTECT
    assert _status(cfg, dirty_rows=[3, 3, 5]) == S.SEGMLA_OK


def test_dirty_rows_counted_once(L):
    cfg = dict(SMALL_CONFIGS[1], budget_permille=0)
    p = _create(cfg)
    q = _create(cfg, dirty_rows=[100, 100, 101, 5])   # 100, 101 lie inside no forced range
    try:
        kinds, lens, offsets = segment_table(cfg)
        g = O.geometry(kinds, lens, offsets, offsets, int(lens.sum()))
        ref = O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], 0, [100, 101, 5])
        assert S.segmla_plan_rows(q)[1] == len(ref["A"])
        assert S.segmla_plan_rows(q)[1] > S.segmla_plan_rows(p)[1]
    finally:
        S.segmla_plan_destroy(p)
        S.segmla_plan_destroy(q)


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="passes fake device addresses; host-only check")
def test_null_and_state_errors(L):
    lib = S.lib()
    h = ctypes.c_void_p()
    assert lib.segmla_plan_create(None, None, None, 10, ctypes.byref(h)) == S.SEGMLA_E_NULL
    cfg = SMALL_CONFIGS[4]
    kinds, lens, offsets = segment_table(cfg)
    g = O.geometry(kinds, lens, offsets, offsets, int(lens.sum()))
    assert O.protected_rows(g, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"],
                            scores=np.zeros(g["T"]))["need"] > 0
    p = _create(cfg)
    try:
        t = S.Tensors()
        # not built yet -> state error, before any device work
        assert lib.segmla_forward(p, ctypes.byref(t), None) == S.SEGMLA_E_STATE
        assert lib.segmla_forward(None, ctypes.byref(t), None) == S.SEGMLA_E_NULL
        # NULL / misaligned / short workspace, missing scores -> rejected before any HIP call
        assert lib.segmla_plan_build(p, None, 0, None, None) == S.SEGMLA_E_WORKSPACE
        assert lib.segmla_plan_build(p, ctypes.c_void_p(0x1008), 1 << 40, None, None) == \
            S.SEGMLA_E_WORKSPACE
        need = S.segmla_plan_workspace_bytes(p)
        assert lib.segmla_plan_build(p, ctypes.c_void_p(0x10000), need - 1, None, None) == \
            S.SEGMLA_E_WORKSPACE
        assert lib.segmla_plan_build(p, ctypes.c_void_p(0x10000), need, None, None) == \
            S.SEGMLA_E_PROTECT
        buf = (ctypes.c_int32 * 4)()
        assert lib.segmla_copy_protected(p, buf, 4, None) == S.SEGMLA_E_STATE
        out = (ctypes.c_double * 3)()
        assert lib.segmla_plan_pairs(p, out, None) == S.SEGMLA_E_STATE
    finally:
        S.segmla_plan_destroy(p)
    S.segmla_plan_destroy(None)


@pytest.mark.skipif(not _no_gpu(), reason="passes fake device addresses; host-only check")
def test_lse_merge_argument_errors(L):
    lib = S.lib()
    P = ctypes.c_void_p
    assert lib.segmla_lse_merge(None, P(16), 1, 1, 4, P(16), 0, None, None) == S.SEGMLA_E_NULL
    assert lib.segmla_lse_merge(P(16), P(16), 0, 1, 4, P(16), 0, None, None) == S.SEGMLA_E_SHAPE
    assert lib.segmla_lse_merge(P(16), P(16), 1, 1, 5000, P(16), 0, None, None) == S.SEGMLA_E_SHAPE
    assert lib.segmla_lse_merge(P(16), P(16), 1, 1, 4, P(16), 2, None, None) == S.SEGMLA_E_DTYPE
    assert lib.segmla_lse_merge(P(16), P(16), 1, 0, 4, P(16), 0, None, None) == S.SEGMLA_OK


def test_ledger_matches_printed_ceilings(L):
    lg, ph, op = S.segmla_ledger(3, 37, 3, 64, 56, 1000, 250)
    assert round(100 * lg, 2) == 75.29
    assert ph == 56 * 750 / (64 * 1000)
    assert np.isnan(op)
    lg, _, _ = S.segmla_ledger(3, 55, 3, 128, 112, 10, 1)
    assert round(100 * lg, 2) == 78.89
    T = 274
    A = _golden_tiny_a()
    g_pairs, l_pairs = O.flops_pairs(T, A, 1, 7)
    lg, ph, op = S.segmla_ledger(0, 1, 0, 8, 7, T, len(A), float(g_pairs), float(l_pairs))
    ref = O.ledger(0, 1, 0, 8, 7, T, A)
    assert np.allclose((lg, ph, op), ref, rtol=0, atol=1e-15)
    with pytest.raises(S.SegmlaError):
        S.segmla_ledger(0, 0, 0, 8, 7, T, 10)
    with pytest.raises(S.SegmlaError):
        S.segmla_ledger(3, 37, 3, 8, 9, T, 10)


def _golden_tiny_a():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "tiny_fp32_protected_rows.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b = map(int, line.split())
            rows.extend(range(a, b))
    return np.array(rows)


def test_product_path_does_not_import_oracle():
    """The package and the C sources never reference the oracle."""
    pkg = os.path.join(ROOT, "segmented_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, f)


def test_binding_rejects_bad_tensors(L):
    """The binding checks every tensor before the C call (the ABI sees raw addresses only):
    host tensors, wrong dtypes, non-contiguous views and undersized buffers raise ValueError
    with the tensor's name, and segmla_plan_get_info reports the shapes the checks use."""
    import torch
    cfg = SMALL_CONFIGS[1]                      # bf16 io, bf16 latent, 64 heads
    p = _create(cfg)
    try:
        info = S.segmla_plan_get_info(p)
        T = int(segment_table(cfg)[1].sum())
        assert info["T"] == T and (info["q_begin"], info["q_end"]) == (0, T)
        assert info["n_heads"] == 64 and info["n_global"] == 8 and info["n_local"] == 56
        assert info["d_v"] == 576 and info["d_state"] == 512 and info["z_slots"] == 64
        assert info["zc_slots"] == 56 and info["n_pool"] == T
        assert info["workspace_bytes"] == S.segmla_plan_workspace_bytes(p)
        bf = torch.bfloat16
        good = dict(q=torch.zeros(T, 64, 576, dtype=bf), kv=torch.zeros(T, 576, dtype=bf),
                    w=torch.zeros(64, 512, 576, dtype=bf), out=torch.zeros(T, 64, 576, dtype=bf),
                    z=torch.zeros(T, 64, 512, dtype=bf), z_cached=torch.zeros(T, 56, 512, dtype=bf))

        def err(**over):
            args = dict(good)
            args.update(over)
            with pytest.raises(ValueError) as e:
                S.segmla_forward(p, **args)
            return str(e.value)
        assert "q must be on the GPU" in err()        # every check passes but the device
        assert "q has dtype" in err(q=good["q"].float())
        assert "kv must be contiguous" in err(kv=torch.zeros(576, T, dtype=bf).t())
        assert "out holds" in err(out=torch.zeros(T - 1, 64, 576, dtype=bf))
        assert "z_cached is required" in err(z_cached=None)
        assert "lse has dtype" in err(lse=torch.zeros(T, 64, dtype=bf))
        assert "w must be a torch tensor" in err(w=np.zeros((64, 512, 576)))
        with pytest.raises(ValueError, match="workspace must be on the GPU"):
            S.segmla_plan_build(p, torch.zeros(info["workspace_bytes"], dtype=torch.uint8))
        with pytest.raises(ValueError, match="workspace holds"):
            S.segmla_plan_build(p, torch.zeros(16, dtype=torch.uint8))
    finally:
        S.segmla_plan_destroy(p)
    # the standalone merge: fp16 output is not an accepted dtype (no silent bf16 reading)
    po, pm = torch.zeros(2, 4, 8), torch.zeros(2, 4, 2)
    with pytest.raises(ValueError, match="out has dtype"):
        S.segmla_lse_merge(po, pm, torch.zeros(4, 8, dtype=torch.float16))
    with pytest.raises(ValueError, match="partial_ml holds"):
        S.segmla_lse_merge(po, torch.zeros(2, 4, 1), torch.zeros(4, 8))
    with pytest.raises(ValueError, match="partial_o must be on the GPU"):
        S.segmla_lse_merge(po, pm, torch.zeros(4, 8))


def test_noalloc_rejects_oversized_workspace(L):
    """segmla_forward_noalloc refuses a plan whose workspace exceeds the library's array before
    anything is enqueued or any tensor is touched (the addresses here are never dereferenced);
    a plan that fits passes the size check and reaches the tensor checks."""
    cfg = SMALL_CONFIGS[1]
    big = _create(cfg, split_keys=64)  # 15 key splits: the partials alone take ~600 MB
    small = _create(CONFIGS[1])        # the 32K layer: its budget needs 999 Indexer rows
    try:
        assert S.segmla_plan_workspace_bytes(big) > S.NOALLOC_MAX_BYTES
        assert S.segmla_plan_workspace_bytes(small) <= S.NOALLOC_MAX_BYTES
        t = S.Tensors(*([16] * 9))
        score = ctypes.c_void_p(16)
        assert L.segmla_forward_noalloc(big, score, ctypes.byref(t), None) == S.SEGMLA_E_WORKSPACE
        assert L.segmla_forward_noalloc(big, None, ctypes.byref(t), None) == S.SEGMLA_E_WORKSPACE
        assert L.segmla_forward_noalloc(small, None, ctypes.byref(t), None) == S.SEGMLA_E_PROTECT
        t_bad = S.Tensors(*([16] * 6 + [24, 16, 16]))  # out off a 16-byte boundary
        assert L.segmla_forward_noalloc(small, score, ctypes.byref(t_bad), None) == S.SEGMLA_E_SHAPE
        assert L.segmla_forward_noalloc(None, score, ctypes.byref(t), None) == S.SEGMLA_E_NULL
        # every check passed: without a visible GPU the device step fails, and says so
        import torch
        if not torch.cuda.is_available():
            assert L.segmla_forward_noalloc(small, score, ctypes.byref(t), None) == S.SEGMLA_E_HIP
    finally:
        S.segmla_plan_destroy(big)
        S.segmla_plan_destroy(small)


def test_set_window_needs_a_built_plan(L):
    """segmla_plan_set_window on an unbuilt plan is SEGMLA_E_STATE (before any argument is
    used), on no plan SEGMLA_E_NULL; nothing is enqueued either way."""
    p = _create(SMALL_CONFIGS[1])
    try:
        assert L.segmla_plan_set_window(p, 0, 5, None) == S.SEGMLA_E_STATE
        assert L.segmla_plan_set_window(p, 7, 3, None) == S.SEGMLA_E_STATE
        assert L.segmla_plan_set_window(None, 0, 5, None) == S.SEGMLA_E_NULL
    finally:
        S.segmla_plan_destroy(p)


def test_prefetch_argument_errors(L):
    """Prefetch calls fail explicitly: no prefetcher or no output slot is SEGMLA_E_NULL; without
    a visible GPU the prefetcher cannot get its stream and says so (SEGMLA_E_HIP)."""
    r = S.CopyRange(16, 32, 1, 8, 8, 8)
    assert L.segmla_prefetch(None, ctypes.byref(r), 1, None) == S.SEGMLA_E_NULL
    assert L.segmla_prefetch_wait(None, None) == S.SEGMLA_E_NULL
    assert L.segmla_prefetcher_create(None) == S.SEGMLA_E_NULL
    ms = ctypes.c_float()
    assert L.segmla_prefetch_elapsed(None, ctypes.byref(ms)) == S.SEGMLA_E_NULL
    L.segmla_prefetcher_destroy(None)
    import torch
    if not torch.cuda.is_available():
        h = ctypes.c_void_p()
        assert L.segmla_prefetcher_create(ctypes.byref(h)) == S.SEGMLA_E_HIP and not h.value


def test_dual_pool_errors(L):
    """Compressed-history attention (segmla_dual_*): the compressed geometry is validated at
    create time (ratio, window, list width, pool size: SEGMLA_E_SHAPE; a segment's entries
    outside the pool: SEGMLA_E_GEOMETRY; an fp32 or E4M3 layer: SEGMLA_E_UNSUPPORTED), the entry
    count is the sum of floor(len / ratio) over segments, a forward of an unbuilt object is
    SEGMLA_E_STATE, and the binding checks every tensor (lists required exactly when top_k > 0)."""
    import torch
    cfg = SMALL_CONFIGS[1]
    kinds, lens, offsets = segment_table(cfg)
    T = int(lens.sum())
    p = _create(cfg)
    lib = S.lib()
    try:
        cpr = np.concatenate([[0], np.cumsum(lens // 4)[:-1]])
        n_c = int((lens // 4).sum())

        def st(ratio=4, window=127, top_k=8, rows=cpr, n_cpool=n_c):
            try:
                d = S.segmla_dual_create(p, ratio, window, top_k, rows, n_cpool)
            except S.SegmlaError as e:
                return e.status
            S.segmla_dual_destroy(d)
            return S.SEGMLA_OK
        assert st() == S.SEGMLA_OK
        assert st(ratio=0) == S.SEGMLA_E_SHAPE
        assert st(window=-1) == S.SEGMLA_E_SHAPE
        assert st(top_k=-1) == S.SEGMLA_E_SHAPE
        assert st(n_cpool=-1) == S.SEGMLA_E_SHAPE
        assert st(n_cpool=2 ** 31) == S.SEGMLA_E_SHAPE
        assert st(n_cpool=n_c - 1) == S.SEGMLA_E_GEOMETRY
        assert st(rows=cpr - 1) == S.SEGMLA_E_GEOMETRY
        assert st(ratio=10 ** 6, n_cpool=0, rows=np.zeros_like(cpr)) == S.SEGMLA_OK  # no entries
        dp = S.DualPool(4, 127, 8, n_c, None)
        h = ctypes.c_void_p()
        assert lib.segmla_dual_create(p, ctypes.byref(dp), ctypes.byref(h)) == S.SEGMLA_E_NULL
        d = S.segmla_dual_create(p, 4, 127, 8, cpr, n_c)
        try:
            ws, ne = S.segmla_dual_sizes(d)
            assert ne == n_c and ws % 256 == 0 and ws >= 16 * (n_c + len(lens))
            info = S.segmla_plan_get_info(p)
            bf = torch.bfloat16
            good = dict(q=torch.zeros(T, 64, 576, dtype=bf), kv=torch.zeros(T, 576, dtype=bf),
                        ckv=torch.zeros(n_c, 576, dtype=bf), out=torch.zeros(T, 64, 576, dtype=bf),
                        cidx=torch.zeros(T, 8, dtype=torch.int32),
                        clen=torch.zeros(T, dtype=torch.int32))

            def err(top_k=8, **over):
                args = dict(good)
                args.update(over)
                with pytest.raises(ValueError) as e:
                    S.segmla_dual_forward(d, info, top_k, n_c, **args)
                return str(e.value)
            assert "q must be on the GPU" in err()
            assert "ckv holds" in err(ckv=torch.zeros(n_c - 1, 576, dtype=bf))
            assert "cidx is required" in err(cidx=None)
            assert "cidx has dtype" in err(cidx=torch.zeros(T, 8, dtype=torch.int64))
            assert "clen holds" in err(clen=torch.zeros(T - 1, dtype=torch.int32))
            assert "every available entry" in err(top_k=0)
            assert "out has dtype" in err(out=torch.zeros(T, 64, 576))
            if _no_gpu():  # unbuilt plan and object: nothing is enqueued
                t = S.DualTensors(*([8192] * 6 + [None]))
                assert lib.segmla_dual_forward(d, ctypes.byref(t), None) == S.SEGMLA_E_STATE
                t = S.DualTensors(8192, 8192, 8192, None, None, 8192, None)
                assert lib.segmla_dual_forward(d, ctypes.byref(t), None) == S.SEGMLA_E_NULL
                # a workspace off the 256-byte grid or too small, before any copy
                assert lib.segmla_dual_build(d, ctypes.c_void_p(4096 + 8), ws, None) == S.SEGMLA_E_WORKSPACE
                assert lib.segmla_dual_build(d, ctypes.c_void_p(4096), ws - 256, None) == S.SEGMLA_E_WORKSPACE
        finally:
            S.segmla_dual_destroy(d)
    finally:
        S.segmla_plan_destroy(p)
    for c in (SMALL_CONFIGS[0], SMALL_CONFIGS[4]):  # fp32 layer, E4M3 latent
        q = _create(c)
        try:
            k2, l2, _ = segment_table(c)
            with pytest.raises(S.SegmlaError) as e:
                S.segmla_dual_create(q, 4, 127, 0, np.zeros(len(l2), np.int64), 10 ** 6)
            assert e.value.status == S.SEGMLA_E_UNSUPPORTED
        finally:
            S.segmla_plan_destroy(q)
