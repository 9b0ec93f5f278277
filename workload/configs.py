"""Request shapes for segment-relocated MLA attention.

The five named workloads follow the long-context shapes of the RedKnot-MLA
paper (arXiv 2609.07008): DeepSeek-V4-Flash-like layers with 64 logical heads
(one Global head per group of eight, the "profiles" paragraph) and a
Pro-like layer with 128 heads, a packed latent of 512 "nope" + 64 RoPE dims,
documents cached at canonical positions and placed at request offsets, and
the protected-row rule (query/new rows, first/last rows of each relocated
document, Indexer rows, recent tail) with a 10/20/25 % controller budget.

The SMALL_CONFIGS keep the same structure at sizes the fp64 oracle finishes in
seconds; they still span several 64-key tiles, several segments and ragged
segment ends.

Segment kinds: "prefix" (a system prefix computed in the request), "doc" (a
cached document built alone at positions 0..n-1) and "new" (question rows).
"""
import numpy as np

TAG_LEN = 6  # seed tag for the document-length draw of the many-short-segments workload


def _docs(n, length):
    return [("doc", length)] * n


def _many_short_lengths(seed, n, lo, hi):
    return [int(x) for x in np.random.default_rng([seed, TAG_LEN]).integers(lo, hi + 1, n)]


def _cfg(name, index, dtype, n_heads, d_nope, d_rope, d_state, segments, edge_rows,
         tail_rows, budget_permille, seed, v_has_rope=1, kv_dtype=None):
    d_qk = d_nope + d_rope
    return dict(
        name=name, index=index,
        dtype=dtype,                       # io dtype: "f32" or "bf16"
        kv_dtype=kv_dtype or dtype,        # latent storage: "f32", "bf16" or "e4m3"
        n_heads=n_heads,
        global_heads=[h for h in range(n_heads) if h % 8 == 0],
        d_nope=d_nope, d_rope=d_rope, d_state=d_state, v_has_rope=v_has_rope,
        segments=list(segments),
        edge_rows=edge_rows, tail_rows=tail_rows, budget_permille=budget_permille,
        seed=seed, rope_base=10000.0, softmax_scale=1.0,
        q_std=1.0 / np.sqrt(d_qk),
    )


CONFIGS = [
    # 0: tiny fp32 layer: 8 heads (7 Local / 1 Global), 64 + 16 dims.
    _cfg("tiny_fp32", 0, "f32", 8, 64, 16, 64,
         [("prefix", 16), ("doc", 50), ("doc", 80), ("doc", 120), ("new", 8)],
         edge_rows=8, tail_rows=32, budget_permille=0, seed=0),
    # 1: Flash-like bf16 layer, 32K context: prefix + 8 x 4096 documents + 128 question rows.
    _cfg("flash_32k_bf16", 1, "bf16", 64, 512, 64, 512,
         [("prefix", 256)] + _docs(8, 4096) + [("new", 128)],
         edge_rows=128, tail_rows=512, budget_permille=100, seed=1),
    # 2: long-context bf16 layer, 128K context: 32 x 4096 documents + 512 question rows.
    _cfg("long_128k_bf16", 2, "bf16", 64, 512, 64, 512,
         _docs(32, 4096) + [("new", 512)],
         edge_rows=128, tail_rows=32768, budget_permille=200, seed=2),
    # 3: many short segments: 256 documents with lengths uniform in [128, 1024].
    _cfg("many_short_bf16", 3, "bf16", 64, 512, 64, 512,
         [("doc", n) for n in _many_short_lengths(3, 256, 128, 1024)] + [("new", 64)],
         edge_rows=128, tail_rows=512, budget_permille=250, seed=3),
    # 4: Pro-like layer: 128 heads (112 / 16), latent nope dims in E4M3 with one fp32
    #    scale per 128 values, RoPE dims bf16; 16 x 4096 documents + 256 question rows.
    _cfg("pro_64k_fp8", 4, "bf16", 128, 512, 64, 512,
         _docs(16, 4096) + [("new", 256)],
         edge_rows=128, tail_rows=512, budget_permille=250, seed=4, kv_dtype="e4m3"),
]

# The 32K-tail variant of the Flash-like layer (labelled, not one of the five).
FLASH_TAIL32K = dict(CONFIGS[1], name="flash_32k_tail32k_bf16", index=None, tail_rows=32768)

# The Global-head work of the 128K layer alone: its 8 Global heads over every request row,
# the same segments and protected-row rule (the 128K throughput target is stated on this part).
LONG_128K_GLOBAL = dict(CONFIGS[2], name="long_128k_global_bf16", index=None, n_heads=8,
                        global_heads=list(range(8)))

SMALL_CONFIGS = [
    _cfg("tiny_fp32_ragged", None, "f32", 8, 64, 16, 64,
         [("prefix", 5), ("doc", 1), ("doc", 70), ("doc", 3), ("doc", 129), ("new", 9)],
         edge_rows=8, tail_rows=20, budget_permille=300, seed=10),
    _cfg("flash_small_bf16", None, "bf16", 64, 512, 64, 512,
         [("prefix", 40), ("doc", 300), ("doc", 257), ("doc", 129), ("doc", 200), ("new", 20)],
         edge_rows=16, tail_rows=64, budget_permille=100, seed=11),
    _cfg("long_small_bf16", None, "bf16", 64, 512, 64, 512,
         _docs(8, 128) + [("new", 64)],
         edge_rows=16, tail_rows=512, budget_permille=200, seed=12),
    _cfg("many_short_small_bf16", None, "bf16", 64, 512, 64, 512,
         [("doc", n) for n in _many_short_lengths(13, 24, 5, 60)] + [("new", 12)],
         edge_rows=8, tail_rows=32, budget_permille=250, seed=13),
    _cfg("pro_small_fp8", None, "bf16", 128, 512, 64, 512,
         [("doc", 200), ("doc", 130), ("doc", 96), ("doc", 64), ("new", 40)],
         edge_rows=16, tail_rows=48, budget_permille=250, seed=14, kv_dtype="e4m3"),
    _cfg("flash_small_vnope_bf16", None, "bf16", 64, 512, 64, 512,
         [("prefix", 17), ("doc", 150), ("doc", 99), ("new", 11)],
         edge_rows=16, tail_rows=40, budget_permille=150, seed=15, v_has_rope=0),
    # E4M3 latent with nope-only values, ragged segment lengths (partial key tiles)
    _cfg("pro_small_vnope_fp8", None, "bf16", 128, 512, 64, 512,
         [("prefix", 9), ("doc", 77), ("doc", 33), ("doc", 150), ("new", 13)],
         edge_rows=8, tail_rows=24, budget_permille=200, seed=16, kv_dtype="e4m3", v_has_rope=0),
]


# Grouped projected state (z and the cache hold one vector per group of heads): the tiny layer
# in groups of 4 (group 1 has no Global head: its rows outside A are the cache alone), and the
# Flash-like and Pro-like layers in groups of 8 (one Global head each).
GROUPED_CONFIGS = [
    dict(_cfg("tiny_fp32_grouped", None, "f32", 8, 64, 16, 64,
              [("prefix", 12), ("doc", 40), ("doc", 75), ("new", 6)],
              edge_rows=8, tail_rows=16, budget_permille=200, seed=20), group_heads=4),
    dict(_cfg("flash_small_grouped_bf16", None, "bf16", 64, 512, 64, 512,
              [("prefix", 33), ("doc", 200), ("doc", 257), ("doc", 120), ("new", 21)],
              edge_rows=16, tail_rows=48, budget_permille=150, seed=21), group_heads=8),
    dict(_cfg("pro_small_grouped_fp8", None, "bf16", 128, 512, 64, 512,
              [("prefix", 9), ("doc", 140), ("doc", 95), ("new", 13)],
              edge_rows=8, tail_rows=24, budget_permille=250, seed=22, kv_dtype="e4m3"),
         group_heads=8),
    dict(CONFIGS[1], name="flash_32k_grouped_bf16", index=None, group_heads=8),
    dict(CONFIGS[2], name="long_128k_grouped_bf16", index=None, group_heads=8),
]


def _windowed(cfg, name, window_heads, n_sink, window, global_heads=None, seed=None, **over):
    """cfg with sink + window heads (role 2): key p visible from row t iff p <= t and
    (p < n_sink or p >= t - window) (RedKnot explainer, "Insight 1: heads have different jobs").
    The remaining heads keep their roles (Global where listed, else Local)."""
    g = cfg["global_heads"] if global_heads is None else list(global_heads)
    w = sorted(window_heads)
    assert not set(w) & set(g)
    return dict(cfg, name=name, index=None, global_heads=g, window_heads=w, n_sink=n_sink,
                window=window, seed=cfg["seed"] if seed is None else seed, **over)


# Sink + window heads under relocation. The small layers mix all three roles (Global, Local,
# sink + window) with windows that cross segment boundaries; the SWA layers give every head a
# 128-token window without sink (DeepSeek-V4's sliding-window layers, TensorRT-LLM reading
# notes: dense attention over the most recent 128 raw tokens).
WINDOW_CONFIGS = [
    _windowed(_cfg("tiny_window_fp32", None, "f32", 8, 64, 16, 64,
                   [("prefix", 16), ("doc", 50), ("doc", 80), ("doc", 120), ("new", 8)],
                   edge_rows=8, tail_rows=32, budget_permille=100, seed=30),
              "tiny_window_fp32", [1, 4, 6], n_sink=4, window=20),
    _windowed(SMALL_CONFIGS[1], "flash_window_small_bf16", [h for h in range(64) if h % 8 in (1, 2, 3)],
              n_sink=4, window=96, seed=31),
    _windowed(SMALL_CONFIGS[1], "swa_small_bf16", list(range(64)), n_sink=0, window=127,
              global_heads=[], seed=32),
    _windowed(SMALL_CONFIGS[4], "pro_window_small_fp8", [h for h in range(128) if h % 8 in (1, 2)],
              n_sink=4, window=64, seed=33),
    _windowed(SMALL_CONFIGS[5], "flash_window_small_vnope_bf16", [h for h in range(64) if h % 4 == 1],
              n_sink=0, window=50, seed=34),
    # tiny windows (a row and its predecessor) and a sink that covers a whole segment
    _windowed(SMALL_CONFIGS[0], "tiny_window_edge_fp32", [2, 3, 5], n_sink=9, window=1, seed=35),
]

# Full-size: the Flash-like 32K layer with its 56 non-Global heads as sink + window heads (the
# explainer's w = 256 example, 4 sink tokens), and the same request as an SWA-128 layer.
FLASH_32K_WINDOW = _windowed(CONFIGS[1], "flash_32k_window_bf16",
                             [h for h in range(64) if h % 8 != 0], n_sink=4, window=256)
SWA_32K = _windowed(CONFIGS[1], "swa_32k_bf16", list(range(64)), n_sink=0, window=127,
                    global_heads=[])


def config_by_name(name):
    for c in (CONFIGS + SMALL_CONFIGS + GROUPED_CONFIGS + WINDOW_CONFIGS +
              [FLASH_TAIL32K, LONG_128K_GLOBAL, FLASH_32K_WINDOW, SWA_32K]):
        if c["name"] == name:
            return c
    raise KeyError(name)


def segment_table(cfg):
    """(kinds, lens, offsets) of the request, segments placed contiguously from 0."""
    kind_code = {"prefix": 0, "doc": 1, "new": 2}
    kinds = np.array([kind_code[k] for k, _ in cfg["segments"]], dtype=np.uint8)
    lens = np.array([n for _, n in cfg["segments"]], dtype=np.int32)
    offsets = np.zeros(len(lens), dtype=np.int64)
    offsets[1:] = np.cumsum(lens[:-1], dtype=np.int64)
    return kinds, lens, offsets
