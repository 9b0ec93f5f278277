"""Seeded synthetic tensors for one layer of segment-relocated MLA attention.

Every tensor is drawn by torch's generator on the requested device, in chunks
of rows with one seed per (workload seed, tensor tag, chunk), so a run is
reproducible and the chunk size does not depend on memory. Distributions:
latent ~ N(0, 1); q ~ N(0, 1) / sqrt(d_nope + d_rope); each head's projection
slice ~ N(0, 1) / sqrt(d_v); the cached projected Local state ~ N(0, 1);
Indexer scores uniform over uint32 (a stand-in for a trained Indexer: picking
the top scores then draws a uniformly random subset of rows).

The E4M3 latent follows the 1x128 E4M3 + fp32-scale storage format described
for DeepSeek-V4's FP8 dataflow (TensorRT-LLM reading notes, Part I): each row's
512 nope values are split into blocks of 128, the block scale is amax / 448 in
fp32 (1 when amax is 0) and the code is torch's round-to-nearest-even cast of
value / scale to float8_e4m3fn; the RoPE dims are kept in bf16. This is the
artifact's storage format (producer side), not part of the attention method.
"""
import numpy as np
import torch

from .configs import segment_table

SEG_PREFIX, SEG_DOC, SEG_NEW = 0, 1, 2

TAG_Q, TAG_LAT, TAG_W, TAG_ZC, TAG_SCORE, TAG_POOL, TAG_PAGES = 1, 2, 3, 4, 5, 7, 8
TAG_CKV, TAG_CIDX, TAG_CPOOL = 9, 10, 11
CHUNK_ROWS = 2048

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _seed(seed, tag, chunk):
    return (int(seed) * 1_000_003 + int(tag) * 10_007 + int(chunk)) % (2**63 - 1)


def _gen(device, seed, tag, chunk):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, tag, chunk))
    return g


def randn_rows(shape, seed, tag, device, dtype, std=1.0):
    """N(0, std^2) tensor of `shape`, drawn CHUNK_ROWS rows at a time in fp32."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    for ci, r0 in enumerate(range(0, rows, CHUNK_ROWS)):
        n = min(CHUNK_ROWS, rows - r0)
        x = torch.randn((n,) + tuple(shape[1:]), generator=_gen(device, seed, tag, ci),
                        device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[r0:r0 + n] = x.to(dtype)
    return out


def uint32_scores(n, seed, device):
    """Uniform uint32 values, returned as an int32 tensor holding the same bits."""
    g = _gen(device, seed, TAG_SCORE, 0)
    x = torch.randint(0, 2**32, (n,), generator=g, device=device, dtype=torch.int64)
    x = torch.where(x >= 2**31, x - 2**32, x)
    return x.to(torch.int32)


def quantize_e4m3_b128(x):
    """fp32 [rows, d] (d a multiple of 128) -> (codes uint8 [rows, d], scales fp32 [rows, d/128])."""
    rows, d = x.shape
    xb = x.reshape(rows, d // 128, 128)
    amax = xb.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (xb / scale.unsqueeze(-1)).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(rows, d)
    return codes, scale.to(torch.float32)


def pool_placement(lens, mode, seed):
    """First pool row of each segment and the pool size.

    identity: pool row = request row. shuffled: segment blocks in a random order
    with random gaps (unused pool rows). aliased: every document whose length
    equals an earlier document's reuses that document's pool range (the same
    cached document placed twice in one request).
    """
    n = len(lens)
    if mode == "identity":
        pr = np.zeros(n, dtype=np.int64)
        pr[1:] = np.cumsum(lens[:-1], dtype=np.int64)
        return pr, int(np.sum(lens, dtype=np.int64))
    rng = np.random.default_rng([seed, TAG_POOL])
    if mode == "shuffled":
        order = rng.permutation(n)
        gaps = rng.integers(0, 9, n)
        pr = np.zeros(n, dtype=np.int64)
        cur = int(rng.integers(0, 9))
        for i in order:
            pr[i] = cur
            cur += int(lens[i]) + int(gaps[i])
        return pr, cur
    if mode == "aliased":
        pr = np.zeros(n, dtype=np.int64)
        first_of_len = {}
        cur = 0
        for i in range(n):
            n_i = int(lens[i])
            if n_i in first_of_len and i > 0:
                pr[i] = first_of_len[n_i]
            else:
                pr[i] = cur
                first_of_len.setdefault(n_i, cur)
                cur += n_i
        return pr, cur
    raise ValueError(mode)


def page_placement(kinds, lens, page_rows, seed, share_docs=True):
    """Paged pool: segment i's rows on ceil(len_i / page_rows) pages listed at
    page_table[page_start[i] ...]. Pages come from a shuffled list of pages with unused ones
    among them; every third segment takes consecutive pages instead (runs longer than a page);
    a document as long as an earlier document shares that document's pages (the same cached
    document placed twice). Returns (pages dict, n_pool, pool row of each segment's first row)."""
    rng = np.random.default_rng([seed, TAG_PAGES])
    n = len(lens)
    npg = (np.asarray(lens, dtype=np.int64) + page_rows - 1) // page_rows
    need = int(npg.sum())
    n_shuf = need + need // 3 + 2
    free = [int(g) for g in rng.permutation(n_shuf)]
    next_block = n_shuf  # consecutive pages are taken past the shuffled ones
    page_start = np.zeros(n, dtype=np.int64)
    table, first_doc_of_len = [], {}
    for i in range(n):
        L = int(lens[i])
        if share_docs and kinds[i] == 1 and L in first_doc_of_len:
            page_start[i] = page_start[first_doc_of_len[L]]
            continue
        if kinds[i] == 1:
            first_doc_of_len[L] = i
        page_start[i] = len(table)
        if i % 3 == 0:
            table += list(range(next_block, next_block + int(npg[i])))
            next_block += int(npg[i])
        else:
            table += [free.pop() for _ in range(int(npg[i]))]
    table = np.asarray(table, dtype=np.int64)
    first_rows = table[page_start] * page_rows
    return dict(page_rows=page_rows, page_start=page_start, page_table=table), \
        next_block * page_rows, first_rows


def pool_rows_of(lens, pages):
    """Pool row of every request row under a page placement (the pages' definition)."""
    P = pages["page_rows"]
    out = []
    for i, L in enumerate(lens):
        j = np.arange(int(L), dtype=np.int64)
        out.append(pages["page_table"][pages["page_start"][i] + j // P] * P + j % P)
    return np.concatenate(out)


def make_inputs(cfg, device="cpu", pool="identity", with_scores=True):
    """All inputs of one layer forward for workload `cfg` on `device`. pool: identity,
    shuffled, aliased, or paged:<rows per page>."""
    kinds, lens, offsets = segment_table(cfg)
    T = int(np.sum(lens, dtype=np.int64))
    seed = cfg["seed"]
    pages = None
    if pool.startswith("paged:"):
        pages, n_pool, pool_rows = page_placement(kinds, lens, int(pool.split(":")[1]), seed)
    else:
        pool_rows, n_pool = pool_placement(lens, pool, seed)
    H = cfg["n_heads"]
    d_nope, d_rope = cfg["d_nope"], cfg["d_rope"]
    d_qk = d_nope + d_rope
    d_v = d_qk if cfg["v_has_rope"] else d_nope
    head_is_global = np.zeros(H, dtype=np.uint8)   # each head's role: 0 Local, 1 Global,
    head_is_global[cfg["global_heads"]] = 1         # 2 sink + window
    head_is_global[list(cfg.get("window_heads", ()))] = 2
    n_local = int(np.sum(head_is_global == 0))
    io = _TORCH_DT[cfg["dtype"]]

    used = np.zeros(n_pool, dtype=bool)
    if pages is not None:
        used[pool_rows_of(lens, pages)] = True
    else:
        for p, n in zip(pool_rows, lens):
            used[p:p + n] = True
    unused = torch.from_numpy(~used).to(device)

    out = dict(cfg=cfg, kinds=kinds, lens=lens, offsets=offsets, pool_rows=pool_rows,
               n_pool=n_pool, T=T, head_is_global=head_is_global, n_local=n_local, d_v=d_v)
    if pages is not None:
        out["pages"] = pages
    out["q"] = randn_rows((T, H, d_qk), seed, TAG_Q, device, io, std=cfg["q_std"])
    lat = randn_rows((n_pool, d_qk), seed, TAG_LAT, device, torch.float32)
    if cfg["kv_dtype"] == "e4m3":
        codes, scales = quantize_e4m3_b128(lat[:, :d_nope])
        rope = lat[:, d_nope:].to(torch.bfloat16)
        if bool(unused.any()):
            codes[unused] = 0x7F  # E4M3 NaN code
            scales[unused] = float("nan")
            rope[unused] = float("nan")
        out["kv"], out["kv_scale"], out["kv_rope"] = codes, scales, rope
    else:
        lat = lat.to(_TORCH_DT[cfg["kv_dtype"]])
        if bool(unused.any()):
            lat[unused] = float("nan")
        out["kv"] = lat
    del lat
    out["w"] = randn_rows((H, cfg["d_state"], d_v), seed, TAG_W, device, io,
                          std=1.0 / np.sqrt(d_v))
    G = cfg.get("group_heads", 0)
    slots = H // G if G >= 2 else n_local  # grouped state: one cached vector per group
    out["z_cached"] = randn_rows((n_pool, slots, cfg["d_state"]), seed, TAG_ZC, device, io)
    if with_scores:
        out["scores"] = uint32_scores(T, seed, device)
    return out


def make_dual_inputs(inp, ratio, window, top_k, device="cpu", pool="identity"):
    """A compressed pool and Indexer lists for the compressed-history (dual-pool) layers, next
    to the inputs `inp` of make_inputs.

    Pool layout: segment i gets a block of ceil(len_i / ratio) + 1 rows (room for every entry
    it can hold), the blocks in segment order back to back (identity) or in a random order
    with random gaps (shuffled); rows ~ N(0, 1) in the latent's dtype (bf16 or fp32), rows
    outside every block NaN.

    Lists (top_k > 0): a stand-in for an Indexer's top-K picks. Row t draws from the ids
    [0, n_t) with n_t = (t + 1) // ratio (the entries of a request whose segments are multiples
    of `ratio` long): all of them when n_t <= top_k, else one uniformly drawn id from each of
    top_k equal strata of [0, n_t) (ascending, no repeats). cidx int32 [T][top_k] (unused
    slots -1), clen int32 [T]."""
    cfg = inp["cfg"]
    lens = np.asarray(inp["lens"], dtype=np.int64)
    T = int(inp["T"])
    seed = cfg["seed"]
    blk = -(-lens // int(ratio)) + 1
    n = len(lens)
    cpool_rows = np.zeros(n, dtype=np.int64)
    if pool == "identity":
        cpool_rows[1:] = np.cumsum(blk[:-1])
        n_cpool = int(blk.sum())
    elif pool == "shuffled":
        rng = np.random.default_rng([seed, TAG_CPOOL])
        cur = int(rng.integers(0, 5))
        for i in rng.permutation(n):
            cpool_rows[i] = cur
            cur += int(blk[i]) + int(rng.integers(0, 5))
        n_cpool = cur
    else:
        raise ValueError(pool)
    d_qk = cfg["d_nope"] + cfg["d_rope"]
    dt = _TORCH_DT[cfg["kv_dtype"]] if cfg["kv_dtype"] in _TORCH_DT else torch.bfloat16
    ckv = randn_rows((n_cpool, d_qk), seed, TAG_CKV, device, torch.float32)
    used = np.zeros(n_cpool, dtype=bool)
    for r, b in zip(cpool_rows, blk):
        used[r:r + b] = True
    if not used.all():
        ckv[torch.from_numpy(~used).to(device)] = float("nan")
    out = dict(ratio=int(ratio), window=int(window), top_k=int(top_k), cpool_rows=cpool_rows,
               n_cpool=int(n_cpool), ckv=ckv.to(dt))
    if top_k > 0:
        g = _gen(device, seed, TAG_CIDX, 0)
        nt = torch.div(torch.arange(1, T + 1, device=device, dtype=torch.int64), int(ratio),
                       rounding_mode="floor")
        k = torch.arange(top_k, device=device, dtype=torch.int64)
        u = torch.rand((T, top_k), generator=g, device=device, dtype=torch.float64)
        strat = torch.floor((k[None, :] + u) * nt[:, None].double() / top_k).to(torch.int64)
        every = k[None, :].expand(T, top_k)
        ids = torch.where((nt >= top_k)[:, None], strat, every)
        clen = torch.clamp(nt, max=top_k)
        ids = torch.where(k[None, :] < clen[:, None], ids, torch.full_like(ids, -1))
        out["cidx"] = ids.to(torch.int32).contiguous()
        out["clen"] = clen.to(torch.int32).contiguous()
    return out
