"""Plain fp64 CPU oracle for segment-relocated MLA attention.

TEST INFRASTRUCTURE ONLY. This module is imported by tests/, by
__graft_entry__.smoke() and by the cpu_baseline leg of bench.py, and by
nothing else: the library's product path never calls it. It shares no code
with the HIP path; the only code both sides use is the seeded input generator
in the `workload` package, which holds none of the method's arithmetic.

It computes, slowly and in the most direct way, what the GPU path computes:

* geometry: the request is a list of segments placed contiguously; each row has
  a segment, a canonical index j inside it and a latent-pool row.
* the protected row set A (RedKnot-MLA paper, protected-row paragraph, Eq. 6):
  question/new rows, dirty rows, the first and last b rows of each relocated
  document, the recent tail, then Indexer rows chosen by top score up to the
  controller budget of candidate rows.
* attention by *physical* re-rotation, not by the method's query rotation:
  every cached key's RoPE part is moved to its request position with
  K(p_new) = R(p_new) R(p_old)^-1 K(p_old) (RedKnot explainer, "Insight 1:
  heads have different jobs", key re-rotation equation), the request is
  concatenated, and dense causal softmax attention runs over it. By RoPE
  orthogonality (RedKnot-MLA paper, relocation paragraph, Eq. 5) the method's
  rotate-query / attend-canonical / restore-output / LSE-merge computes the
  same thing, which is why this is its oracle.
* the projected state (RedKnot-MLA paper, head-partition and projected-state
  paragraphs, Eq. 2-3): inverse output RoPE at the query position, then each
  head's slice of the bias-free first output projection; Local heads outside
  A take their cached contribution unchanged (replacement, never addition,
  protected-row paragraph).
* sink + window heads (RedKnot explainer, "Insight 1: heads have different
  jobs": a local head sees the sink tokens and the recent window,
  W(i) = S_sink U [i - w, i]): the same dense attention with the keys outside
  that set masked out, on every row, over the same physically re-rotated keys.
* compressed-history layers of DeepSeek-V4 (TensorRT-LLM reading notes,
  section 1: CSA / HCA): per segment, entries of m rows stored in a second
  pool; each row attends its recent raw window and its compressed entries
  (all available ones for HCA, its Indexer list for CSA) in one dense
  softmax, entries re-rotated physically by their segment's shift.

Readings of points the pages leave open (each listed in the design notes):
values are the full latent row (keys = values, RoPE dims last); RoPE pairs
(2k, 2k+1) with theta_k = base^(-2k/d_rope); documents are stored at
canonical positions 0..n-1, prefix and new segments at their request
positions; a key p is visible from row t iff p <= t; softmax scale sigma is a
parameter (1 in the workloads).

Pinned by tests/test_oracle_pins.py against: a brute-force tiny case with
explicit rotation matrices and an unshifted softmax, torch's
scaled_dot_product_attention (float64, CPU), an independent fp64 segmented
computation (RoPE relocation identity), rotation-group identities, shift
invariance of the projected state, the exact-cache identity of the
replacement, brute-force membership of the protected set, the worked example
of the tiny workload, the printed head-row ceilings (75.29 % / 78.89 %) and
torch's float8_e4m3fn decoding.
"""
import numpy as np

SEG_PREFIX, SEG_DOC, SEG_NEW = 0, 1, 2


# --------------------------------------------------------------------------- geometry
def geometry(kinds, lens, offsets, pool_rows, n_pool, pages=None):
    """Integer layout of a request (segment list in request order).

    The pool is either contiguous per segment (segment i at pool rows pool_rows[i] + j) or,
    with `pages` = dict(page_rows, page_start, page_table), paged: row j of segment i sits on
    page page_table[page_start[i] + j // page_rows] at offset j % page_rows (RedKnot-MLA
    paper, fused-consumer paragraph: each cached segment paged in once, attended in place).

    Returns dict(T, seg_of_row, canon, pool_of_row, relocated, stored_pos_base).
    A document is relocated when it sits at a nonzero offset (RedKnot-MLA
    paper, relocation paragraph: a document built at 0..n_i-1 placed at
    offset Delta_i). Documents keep canonical positions in the pool; prefix and
    new segments are computed in the request, so their stored RoPE phase is
    already the request position (stored_pos_base = offset).
    """
    kinds = np.asarray(kinds, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    pool_rows = np.asarray(pool_rows, dtype=np.int64)
    n = len(kinds)
    if n < 1 or len(lens) != n or len(offsets) != n or len(pool_rows) != n:
        raise ValueError("segment arrays must be non-empty and of equal length")
    if np.any(lens < 1):
        raise ValueError("every segment needs at least one row")
    if offsets[0] != 0 or np.any(offsets[1:] != offsets[:-1] + lens[:-1]):
        raise ValueError("segments must be contiguous from request position 0")
    if np.any((kinds < 0) | (kinds > 2)):
        raise ValueError("unknown segment kind")
    T = int(offsets[-1] + lens[-1])
    seg_of_row = np.repeat(np.arange(n, dtype=np.int64), lens)
    canon = np.arange(T, dtype=np.int64) - offsets[seg_of_row]
    if pages is None:
        if np.any(pool_rows < 0) or np.any(pool_rows + lens > n_pool):
            raise ValueError("segment pool range out of bounds")
        pool_of_row = pool_rows[seg_of_row] + canon
    else:
        P = int(pages["page_rows"])
        start = np.asarray(pages["page_start"], dtype=np.int64)
        table = np.asarray(pages["page_table"], dtype=np.int64)
        entry = start[seg_of_row] + canon // P
        if P < 1 or np.any(entry < 0) or np.any(entry >= len(table)):
            raise ValueError("page list out of bounds")
        pool_of_row = table[entry] * P + canon % P
        if np.any(pool_of_row < 0) or np.any(pool_of_row >= n_pool):
            raise ValueError("paged pool row out of bounds")
    relocated = (kinds == SEG_DOC) & (offsets != 0)
    stored_pos_base = np.where(kinds == SEG_DOC, 0, offsets)
    return dict(T=T, n_seg=n, kinds=kinds, lens=lens, offsets=offsets, pool_rows=pool_rows,
                seg_of_row=seg_of_row, canon=canon, pool_of_row=pool_of_row,
                relocated=relocated, stored_pos_base=stored_pos_base)


# ---------------------------------------------------------------------- protected rows
def protected_rows(geom, edge_rows, tail_rows, budget_permille, dirty_rows=(), scores=None):
    """Protected row set A (RedKnot-MLA paper, protected-row paragraph, Eq. 6).

    Forced rows F = question/new rows, dirty rows, the first and last
    `edge_rows` rows of every relocated document, and the last `tail_rows`
    request rows. Candidates C = rows of cached segments (prefix and
    documents). The controller budget is K = ceil(budget_permille * |C| / 1000)
    candidate rows; the Indexer fills the remaining need = max(0, K - |F & C|)
    with the highest-scoring candidates outside F, ties going to the smaller
    row. Forced rows are never dropped, so |A| may exceed the budget.
    Returns dict(A, forced, indexer, K, need).
    """
    T = geom["T"]
    kinds, lens, offsets = geom["kinds"], geom["lens"], geom["offsets"]
    forced = np.zeros(T, dtype=bool)
    row_kind = kinds[geom["seg_of_row"]]
    forced[row_kind == SEG_NEW] = True
    dirty = np.asarray(list(dirty_rows), dtype=np.int64)
    if dirty.size:
        if np.any((dirty < 0) | (dirty >= T)):
            raise ValueError("dirty row out of range")
        forced[dirty] = True
    b = int(edge_rows)
    for i in range(geom["n_seg"]):
        if geom["relocated"][i]:
            s, n = int(offsets[i]), int(lens[i])
            forced[s:s + min(b, n)] = True
            forced[s + max(0, n - b):s + n] = True
    if tail_rows > 0:
        forced[max(0, T - int(tail_rows)):] = True
    cand = row_kind != SEG_NEW
    n_cand = int(cand.sum())
    K = (int(budget_permille) * n_cand + 999) // 1000
    need = max(0, K - int((forced & cand).sum()))
    chosen = np.zeros(T, dtype=bool)
    if need > 0:
        if scores is None:
            raise ValueError("Indexer scores are required when the budget needs rows")
        sc = np.asarray(scores).astype(np.int64) & 0xFFFFFFFF  # uint32 bit pattern
        pool = np.nonzero(cand & ~forced)[0]
        # highest score first; equal scores -> smaller row first
        order = np.lexsort((pool, -sc[pool]))
        chosen[pool[order[:need]]] = True
    A = np.nonzero(forced | chosen)[0].astype(np.int64)
    return dict(A=A, forced=forced, indexer=chosen, K=K, need=need)


# ------------------------------------------------------------------------------ RoPE
def rope_theta(d_rope, base):
    """theta_k = base^(-2k/d_rope), k = 0 .. d_rope/2 - 1, in fp64."""
    k = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * k / float(d_rope))


def rot_blocks(pos, theta):
    """Explicit 2x2 rotation blocks R(pos * theta_k): array [..., d_rope/2, 2, 2].

    R = [[cos, -sin], [sin, cos]] acting on the pair (x_2k, x_2k+1).
    """
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    R = np.empty(ang.shape + (2, 2), dtype=np.float64)
    R[..., 0, 0] = c
    R[..., 0, 1] = -s
    R[..., 1, 0] = s
    R[..., 1, 1] = c
    return R


def apply_blocks(R, x_rope):
    """Apply per-pair 2x2 blocks R [..., d_rope/2, 2, 2] to x_rope [..., d_rope]."""
    xp = x_rope.reshape(x_rope.shape[:-1] + (x_rope.shape[-1] // 2, 2))  # also for zero rows
    y = np.einsum("...kab,...kb->...ka", R, xp)
    return y.reshape(x_rope.shape)


# ------------------------------------------------------------------------- attention
def relocated_keys(latent, geom, d_nope, d_rope, base):
    """Request-ordered keys k_p (fp64 [T, d_nope + d_rope]) by physical re-rotation.

    k_p = [c^nope, R(p) R(p_stored)^-1 c^rope] with p the request position and
    p_stored the position the stored latent row was encoded at (its canonical
    index j for a document, p itself for prefix/new rows).
    """
    theta = rope_theta(d_rope, base)
    lat = np.asarray(latent, dtype=np.float64)[geom["pool_of_row"]]
    p = np.arange(geom["T"], dtype=np.float64)
    p_stored = (geom["stored_pos_base"][geom["seg_of_row"]] + geom["canon"]).astype(np.float64)
    R_new = rot_blocks(p, theta)
    R_old_inv = np.swapaxes(rot_blocks(p_stored, theta), -1, -2)  # R^-1 = R^T
    M = np.einsum("tkab,tkbc->tkac", R_new, R_old_inv)
    keys = lat.copy()
    keys[:, d_nope:] = apply_blocks(M, lat[:, d_nope:])
    return keys


def attend_rows(q_rows, t_rows, keys, sigma, d_v):
    """Dense causal softmax attention for chosen query rows.

    q_rows fp64 [n, Hs, d_qk] (stored queries, already at their request
    positions), t_rows [n] request positions, keys fp64 [T, d_qk]; values are
    the first d_v dims of the keys. Key p is visible from row t iff p <= t.
    Returns (O [n, Hs, d_v], lse [n, Hs]) with lse = log sum_p exp(sigma q.k_p).
    """
    n, Hs, _ = q_rows.shape
    O = np.empty((n, Hs, d_v), dtype=np.float64)
    lse = np.empty((n, Hs), dtype=np.float64)
    for i in range(n):
        t = int(t_rows[i])
        K = keys[:t + 1]
        s = sigma * (q_rows[i] @ K.T)              # [Hs, t+1]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        O[i] = (e @ K[:, :d_v]) / l
        lse[i] = (m + np.log(l))[:, 0]
    return O, lse


def window_visible(t, n_sink, window):
    """Keys a sink + window head sees from request row t (RedKnot explainer, "Insight 1: heads
    have different jobs": W(i) = S_sink U [i - w, i]): boolean mask over positions 0..t, key p
    visible iff p < n_sink (the sink, the first n_sink request positions) or p >= t - window
    (the recent window, t itself included)."""
    p = np.arange(int(t) + 1)
    return (p < int(n_sink)) | (p >= int(t) - int(window))


def attend_rows_window(q_rows, t_rows, keys, sigma, d_v, n_sink, window):
    """attend_rows restricted to the sink + window key set of each row (window_visible)."""
    n, Hs, _ = q_rows.shape
    O = np.empty((n, Hs, d_v), dtype=np.float64)
    lse = np.empty((n, Hs), dtype=np.float64)
    for i in range(n):
        t = int(t_rows[i])
        K = keys[:t + 1][window_visible(t, n_sink, window)]
        s = sigma * (q_rows[i] @ K.T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        O[i] = (e @ K[:, :d_v]) / l
        lse[i] = (m + np.log(l))[:, 0]
    return O, lse


# --------------------------------------------------------------------- projected state
def project_rows(O_rows, t_rows, heads, W, d_nope, d_rope, base, v_has_rope):
    """Per-head projected contribution Z[t,h] = W_h u (fp64 [n, Hs, d_state]).

    u = [O^nope, R(-t) O^rope]: inverse output RoPE at the query position,
    then the head's slice W_h [d_state, d_v] of the bias-free first output
    projection (RedKnot-MLA paper, head-partition paragraph, Eq. 2).
    With values of nope dims only there is no RoPE part to undo.
    """
    u = np.array(O_rows, dtype=np.float64, copy=True)
    if v_has_rope:
        R_inv = np.swapaxes(rot_blocks(np.asarray(t_rows, dtype=np.float64),
                                       rope_theta(d_rope, base)), -1, -2)
        u[..., d_nope:] = apply_blocks(R_inv[:, None], u[..., d_nope:])
    Wh = np.asarray(W, dtype=np.float64)[list(heads)]          # [Hs, d_state, d_v]
    return np.einsum("hzv,nhv->nhz", Wh, u)


def layer_forward(inp, rows=None, A_override=None, zc_override=None):
    """Oracle of one layer forward on rows `rows` (default: every request row).

    `inp` holds numpy/fp64-convertible arrays: kinds, lens, offsets, pool_rows,
    n_pool, head_is_global, q [T,H,d_qk], latent [n_pool, d_qk] (already
    decoded to values), w [H, d_state, d_v], z_cached [n_pool, H_L, d_state],
    scores [T], and cfg (d_nope, d_rope, rope_base, softmax_scale, v_has_rope,
    edge_rows, tail_rows, budget_permille, and n_sink / window when some head
    has role 2).

    head_is_global holds each head's role: 1 Global (every row, full causal context),
    0 Local (rows of A with full causal context; elsewhere the cached contribution is
    copied), 2 sink + window (every row, keys window_visible(t, n_sink, window)).

    Returns dict(geom, prot, A, rows, O [n,H,d_v] (NaN where a Local head is not
    computed), lse [n,H], Z [n,H,d_state], computed [n,H] bool).
    """
    cfg = inp["cfg"]
    d_nope, d_rope = cfg["d_nope"], cfg["d_rope"]
    base, sigma = cfg["rope_base"], cfg["softmax_scale"]
    v_rope = bool(cfg["v_has_rope"])
    d_v = d_nope + d_rope if v_rope else d_nope
    geom = geometry(inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"], inp["n_pool"],
                    inp.get("pages"))
    prot = protected_rows(geom, cfg["edge_rows"], cfg["tail_rows"], cfg["budget_permille"],
                          cfg.get("dirty_rows", ()), inp.get("scores"))
    A = prot["A"] if A_override is None else np.asarray(A_override, dtype=np.int64)
    in_A = np.zeros(geom["T"], dtype=bool)
    in_A[A] = True
    T = geom["T"]
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    role = np.asarray(inp["head_is_global"]).astype(np.int64)
    if np.any((role < 0) | (role > 2)):
        raise ValueError("head roles are 0 (Local), 1 (Global) or 2 (sink + window)")
    H = len(role)
    local_heads = np.nonzero(role == 0)[0]
    win_heads = np.nonzero(role == 2)[0]
    n_sink, window = int(cfg.get("n_sink", 0)), int(cfg.get("window", 0))
    local_index = np.full(H, -1, dtype=np.int64)
    local_index[local_heads] = np.arange(len(local_heads))

    keys = relocated_keys(inp["latent"], geom, d_nope, d_rope, base)
    q = inp["q"]
    W = inp["w"]
    Zc = inp["z_cached"] if zc_override is None else zc_override
    n = len(rows)
    O = np.full((n, H, d_v), np.nan)
    lse = np.full((n, H), np.nan)
    Z = np.empty((n, H, W.shape[1]), dtype=np.float64)
    computed = np.zeros((n, H), dtype=bool)
    for i, t in enumerate(rows):
        # full causal context: Global heads, and Local heads on rows of A
        heads = np.nonzero((role == 1) | ((role == 0) & in_A[t]))[0]
        qrow = np.asarray(q[t], dtype=np.float64)
        if len(heads):
            o, ls = attend_rows(qrow[heads][None], [t], keys, sigma, d_v)
            O[i, heads] = o[0]
            lse[i, heads] = ls[0]
            computed[i, heads] = True
            Z[i, heads] = project_rows(o, [t], heads, W, d_nope, d_rope, base, v_rope)[0]
        if len(win_heads):  # sink + window heads, every row
            o, ls = attend_rows_window(qrow[win_heads][None], [t], keys, sigma, d_v, n_sink, window)
            O[i, win_heads] = o[0]
            lse[i, win_heads] = ls[0]
            computed[i, win_heads] = True
            Z[i, win_heads] = project_rows(o, [t], win_heads, W, d_nope, d_rope, base, v_rope)[0]
        if not in_A[t]:
            zc_row = np.asarray(Zc[geom["pool_of_row"][t]], dtype=np.float64)
            Z[i, local_heads] = zc_row[local_index[local_heads]]
    return dict(geom=geom, prot=prot, A=A, rows=rows, O=O, lse=lse, Z=Z, computed=computed)


class _NoCache:
    """Stand-in cached state whose every row is zero (used to take the computed heads alone)."""

    def __init__(self, n_local, d_state):
        self.row = np.zeros((n_local, d_state))

    def __getitem__(self, i):
        return self.row


def layer_forward_grouped(inp, rows=None):
    """Oracle of the grouped projected state (RedKnot-MLA paper, projected-state paragraph,
    Eq. 3: z = z_L + z_G, with the producer retaining the projected Local contribution).

    Heads gG .. gG+G-1 form group g (G = cfg["group_heads"]). For request row t:
    z[t][g] = sum over the group's Global and sink + window heads of W_h u_h(t)
              + (t in A ? sum over its Local heads of W_h u_h(t) : z_cached[pool_row(t)][g]),
    with z_cached [n_pool, n_groups, d_state] the cached Local contribution per group. A layer
    without Local heads has no Local contribution (z_L = 0 in Eq. 3), so nothing cached is added
    and z_cached is not read. O, lse and A are those of layer_forward. Returns its dict with
    Z [n, n_groups, d_state].
    """
    cfg = inp["cfg"]
    G = int(cfg["group_heads"])
    role = np.asarray(inp["head_is_global"]).astype(np.int64)
    H = len(role)
    none = _NoCache(int((role == 0).sum()), cfg["d_state"])
    res = layer_forward(inp, rows=rows, zc_override=none)  # Local heads outside A add 0
    geom, A = res["geom"], res["A"]
    in_A = np.zeros(geom["T"], dtype=bool)
    in_A[A] = True
    Zh = res["Z"]                                             # [n, H, d_state]
    Zg = Zh.reshape(len(res["rows"]), H // G, G, -1).sum(axis=2)
    if (role == 0).any():
        Zc = inp["z_cached"]
        for i, t in enumerate(res["rows"]):
            if not in_A[t]:
                Zg[i] += np.asarray(Zc[geom["pool_of_row"][t]], dtype=np.float64)
    res["Z"] = Zg
    return res


# ---------------------------------------------------------------------------- ledger
def head_row_ceiling(f_front, r, f_back, n_heads, n_local):
    """Logical head-row eligibility ceiling (RedKnot-MLA paper, profiles paragraph,
    Eq. 8): the reusable-layer share times the Local-head share."""
    return (r / (f_front + r + f_back)) * (n_local / n_heads)


def ledger(f_front, r, f_back, n_heads, n_local, T, A):
    """The three analytic namespaces kept apart (RedKnot-MLA paper, namespaces
    paragraph): logical head-row saving, physical token-row saving of one
    reusable layer (Local heads' rows outside A) and the analytic attention
    operator saving (1 - computed (row, head, key) triples / dense triples)."""
    A = np.asarray(A, dtype=np.int64)
    logical = head_row_ceiling(f_front, r, f_back, n_heads, n_local)
    physical = n_local * (T - len(A)) / (n_heads * T)
    n_global = n_heads - n_local
    dense = n_heads * T * (T + 1) / 2.0
    computed = n_global * T * (T + 1) / 2.0 + n_local * float(np.sum(A + 1))
    return logical, physical, 1.0 - computed / dense


# -------------------------------------------------- compressed history (dual-pool layers)
def compressed_entries(geom, ratio, cpool_rows, n_cpool):
    """Compressed entries of a request for the DeepSeek-V4 CSA and HCA layers ("Reading notes on
    DeepSeek-V4 serving in TensorRT-LLM", section 1: besides the recent raw tokens, such a layer
    attends a history compressed m to 1; HCA pools disjoint windows of m' tokens).

    Reading (the pages say nothing of relocation here): compression runs per segment when the
    segment is stored, so a cached document is compressed alone at its canonical positions and
    segment i holds floor(len_i / m) entries. Entry j of segment i stands for the segment's rows
    [m j, m j + m), lies at compressed-pool row cpool_rows[i] + j, is encoded in the segment's
    stored RoPE frame (like its raw rows) and becomes available to request row t once its last
    row, offset_i + m j + m - 1, is <= t. Entries are numbered in request order, segment by
    segment.

    Returns dict(n, seg [n], j [n], pool [n], first_row [n] (the first request row that sees
    the entry), base [n_seg] (id of each segment's entry 0), count [n_seg])."""
    m = int(ratio)
    if m < 1:
        raise ValueError("ratio must be >= 1")
    lens, offsets = geom["lens"], geom["offsets"]
    cpool_rows = np.asarray(cpool_rows, dtype=np.int64)
    count = lens // m
    if np.any(cpool_rows < 0) or np.any(cpool_rows + count > int(n_cpool)):
        raise ValueError("compressed pool range out of bounds")
    base = np.zeros(len(lens), dtype=np.int64)
    base[1:] = np.cumsum(count[:-1])
    seg = np.repeat(np.arange(len(lens), dtype=np.int64), count)
    j = np.arange(int(count.sum()), dtype=np.int64) - base[seg]
    return dict(n=int(count.sum()), m=m, seg=seg, j=j, pool=cpool_rows[seg] + j,
                first_row=offsets[seg] + m * j + m - 1, base=base, count=count)


def relocated_entries(centries, geom, ce, d_nope, d_rope, base):
    """Entry keys in the request frame by physical re-rotation (fp64 [n, d_nope + d_rope]): an
    entry of segment i moves by its segment's phase shift, R(offset_i - stored_pos_base_i), the
    same move relocated_keys gives every raw row of that segment (R(p) R(p_stored)^-1 =
    R(p - p_stored), and p - p_stored is constant over a segment)."""
    theta = rope_theta(d_rope, base)
    lat = np.asarray(centries, dtype=np.float64)[ce["pool"]]
    shift = (geom["offsets"] - geom["stored_pos_base"])[ce["seg"]].astype(np.float64)
    keys = lat.copy()
    keys[:, d_nope:] = apply_blocks(rot_blocks(shift, theta), lat[:, d_nope:])
    return keys


def entries_of_row(ce, t, ids=None, n_list=None):
    """Entry ids one row attends. HCA (ids None): every entry available at row t, in id order.
    CSA: the row's Indexer list ids[:n_list] (the pages' per-query list length over a fixed-width
    buffer), read up to, not including, the first id that is not an entry available at row t
    (negative, past the last entry, or not yet available); an id listed twice counts twice."""
    avail = ce["first_row"] <= int(t)
    if ids is None:
        return np.flatnonzero(avail)
    out = []
    for c in np.asarray(ids, dtype=np.int64)[:max(0, int(n_list))]:
        if c < 0 or c >= ce["n"] or not avail[c]:
            break
        out.append(int(c))
    return np.asarray(out, dtype=np.int64)


def dual_pool_rows(q_rows, t_rows, keys, ekeys, ce, sigma, d_v, window, lists=None, list_lens=None):
    """One softmax over two key pools ("Reading notes on DeepSeek-V4 serving in TensorRT-LLM",
    section 1, the dual-pool kernel paragraph): for row t, the raw keys p with
    max(0, t - window) <= p <= t (keys: relocated_keys) and the compressed entries of
    entries_of_row (ekeys: relocated_entries), all heads sharing the key set. Values are the
    first d_v dims of each key. Returns (O [n, Hs, d_v], lse [n, Hs])."""
    n, Hs, _ = q_rows.shape
    O = np.empty((n, Hs, d_v), dtype=np.float64)
    lse = np.empty((n, Hs), dtype=np.float64)
    for i in range(n):
        t = int(t_rows[i])
        lo = max(0, t - int(window))
        ids = entries_of_row(ce, t, None if lists is None else lists[i],
                             None if list_lens is None else list_lens[i])
        K = np.concatenate([keys[lo:t + 1], ekeys[ids]], axis=0)
        s = sigma * (q_rows[i] @ K.T)
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        l = e.sum(axis=1, keepdims=True)
        O[i] = (e @ K[:, :d_v]) / l
        lse[i] = (mx + np.log(l))[:, 0]
    return O, lse


def dual_pool_forward(inp, dual, rows, lists=None, list_lens=None):
    """Oracle of the dual-pool attention on request rows `rows` (every head of q). `inp` as for
    layer_forward (q, latent, geometry, cfg), `dual` = dict(ratio, window, cpool_rows, n_cpool,
    centries fp64 [n_cpool, d_qk]); lists / list_lens: per row of `rows`, the CSA list and its
    length (None: HCA). Returns dict(O, lse, ce, n_keys [n] (keys attended per head))."""
    cfg = inp["cfg"]
    d_nope, d_rope = cfg["d_nope"], cfg["d_rope"]
    base, sigma = cfg["rope_base"], cfg["softmax_scale"]
    d_v = d_nope + d_rope if cfg["v_has_rope"] else d_nope
    geom = geometry(inp["kinds"], inp["lens"], inp["offsets"], inp["pool_rows"], inp["n_pool"],
                    inp.get("pages"))
    ce = compressed_entries(geom, dual["ratio"], dual["cpool_rows"], dual["n_cpool"])
    rows = np.asarray(rows, dtype=np.int64)
    keys = relocated_keys(inp["latent"], geom, d_nope, d_rope, base)
    ekeys = relocated_entries(dual["centries"], geom, ce, d_nope, d_rope, base)
    q = np.stack([np.asarray(inp["q"][int(t)], dtype=np.float64) for t in rows])
    O, lse = dual_pool_rows(q, rows, keys, ekeys, ce, sigma, d_v, dual["window"], lists, list_lens)
    n_keys = np.array([min(int(t), int(dual["window"])) + 1 +
                       len(entries_of_row(ce, t, None if lists is None else lists[i],
                                          None if list_lens is None else list_lens[i]))
                       for i, t in enumerate(rows)], dtype=np.int64)
    return dict(O=O, lse=lse, ce=ce, n_keys=n_keys)


# ------------------------------------------------------------------------------ E4M3
def e4m3_decode(codes):
    """OCP E4M3 (float8_e4m3fn) code -> fp64 value, from the format definition:
    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_b128_values(codes, scales, rope):
    """Dequantized latent rows: nope = code value * block scale (blocks of 128),
    RoPE dims as stored."""
    v = e4m3_decode(codes)
    rows, d = v.shape
    v = v.reshape(rows, d // 128, 128) * np.asarray(scales, dtype=np.float64)[..., None]
    return np.concatenate([v.reshape(rows, d), np.asarray(rope, dtype=np.float64)], axis=1)


def e4m3_encode(x):
    """fp64 values of magnitude below 464 -> the nearest OCP E4M3 code, ties to the code with
    an even mantissa, from the format definition (see e4m3_decode): below 2^-6 the codes step by
    2^-9 (subnormals, m * 2^-9), in the binade [2^E, 2^(E+1)) by 2^(E-3). A value that rounds up
    to the next power of two gets that binade's first code. The sign is kept for zeros."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    E = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a < 2.0 ** -6, 2.0 ** -9, np.power(2.0, E - 3.0))
    v = np.rint(a / step) * step  # rint: round half to even, on the step count
    sub = v < 2.0 ** -6
    Ev = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    m = np.where(sub, 0, np.rint(v / np.power(2.0, Ev) * 8.0 - 8.0))
    code = np.where(sub, np.rint(v / 2.0 ** -9), (Ev + 7.0) * 8.0 + m).astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_e4m3_b128_fp32(z):
    """Projected state -> 1x128 E4M3 blocks for the next projection ("Reading notes on
    DeepSeek-V4 serving in TensorRT-LLM", Part I, FP8 dataflow bullet), in fp32 as the producer
    computes it: per block of 128 channels the amax (exact), scale = amax / 448 rounded to fp32
    (1 for an all-zero block), each quotient value / scale rounded to fp32, then the nearest E4M3
    code. z: [..., d] with d a multiple of 128 (taken as fp32). Returns (codes uint8 [..., d],
    scales fp32 [..., d / 128])."""
    z = np.asarray(z, dtype=np.float32)
    lead, d = z.shape[:-1], z.shape[-1]
    zb = z.reshape(*lead, d // 128, 128)
    amax = np.abs(zb).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = (zb / scale[..., None]).astype(np.float32)
    return e4m3_encode(y.astype(np.float64)).reshape(*lead, d), scale


# --------------------------------------------------------------------------- helpers
def flops_pairs(T, A, n_global, n_local):
    """(Global, Local) counts of computed (row, head, key) triples."""
    A = np.asarray(A, dtype=np.int64)
    g = n_global * T * (T + 1) // 2
    l_ = n_local * int(np.sum(A + 1))
    return g, l_


def window_pairs(q0, q1, n_sink, window):
    """Keys one sink + window head attends over the request rows [q0, q1): sum of |W(t)|."""
    return int(sum(int(window_visible(t, n_sink, window).sum()) for t in range(q0, q1)))


def flops_pairs_window(q0, q1, A, n_global, n_local):
    """(Global, Local) counts of computed (row, head, key) triples when only the request rows
    [q0, q1) are computed: each such row t sees t + 1 keys; Local heads only on rows of A."""
    A = np.asarray(A, dtype=np.int64)
    g = n_global * (q1 * (q1 + 1) - q0 * (q0 + 1)) // 2
    inw = A[(A >= q0) & (A < q1)]
    l_ = n_local * int(np.sum(inw + 1))
    return g, l_


def rel_err_rows(x, ref):
    """Per-(row, head) relative L2 error ||x - ref|| / ||ref|| over the channel axis."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(np.sum((x - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    return num / np.maximum(den, 1e-300)

