/*
 * segmla.h - C ABI of libsegmla, segment-relocated MLA attention for AMD MI355X (gfx950).
 *
 * One reusable MLA layer of RedKnot-MLA (arXiv 2609.07008): logical heads are
 * split into Local and Global roles (head-partition paragraph, Eq. 1). All heads
 * share one packed latent row per token. Cached documents were built alone at
 * canonical positions 0..n_i-1 and are placed at request offsets Delta_i
 * (relocation paragraph, Eq. 5). For every computed (query row, head) the library
 * rotates the query's RoPE part by -Delta_i per segment, attends the canonical
 * latent in place, restores the partial output's phase and merges segments with
 * a stable log-sum-exp merge. Global heads run on every row, Local heads only
 * on the protected row set A (protected-row paragraph, Eq. 6). The epilogue then
 * undoes output RoPE at the query position, applies each head's slice of the
 * bias-free first output projection (Eq. 2) and writes a request-ordered
 * projected state. On rows outside A, Local heads' slots receive their cached
 * contribution unchanged (replacement, never addition).
 *
 * Conventions shared by every entry point
 *  - Ownership: the caller owns all device memory, including the workspace. The
 *    library never allocates or frees device memory. A plan is host memory owned
 *    by the library until segmla_plan_destroy.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = default stream).
 *    All device work is enqueued on it with no hidden synchronization; only the
 *    segmla_copy_* calls synchronize that stream.
 *  - Errors: arguments are validated on the host before anything is enqueued; on
 *    any status other than SEGMLA_OK and SEGMLA_E_HIP nothing has been written to
 *    caller memory and no work has been enqueued, so the caller chooses the fallback
 *    (there is never a silent one). SEGMLA_E_HIP reports a HIP call or launch that
 *    failed after validation: work enqueued earlier in the same call may still run,
 *    so after SEGMLA_E_HIP from segmla_plan_build the plan stays unbuilt (the
 *    workspace contents are undefined) and after SEGMLA_E_HIP from segmla_forward
 *    the outputs are undefined. Faults of enqueued kernels surface at the caller's
 *    next synchronization.
 *  - Immutability: the latent pool, the cached projected state and the Indexer
 *    scores are read only.
 *  - Aliasing: segment pool ranges may alias (one document placed twice); outputs
 *    and the workspace must not alias any input or each other.
 *  - Row and head indices are int32; pool indices are int64; T < 2^31.
 */
#ifndef SEGMLA_H
#define SEGMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SEGMLA_ABI_VERSION 5

typedef enum segmla_status {
  SEGMLA_OK = 0,
  SEGMLA_E_NULL = -1,        /* a required pointer is NULL */
  SEGMLA_E_GEOMETRY = -2,    /* malformed segment list (see segmla_geometry) */
  SEGMLA_E_SHAPE = -3,       /* invalid head / latent / state sizes or role mask */
  SEGMLA_E_DTYPE = -4,       /* unknown dtype or unsupported dtype combination */
  SEGMLA_E_PROTECT = -5,     /* invalid protection parameters, or scores missing */
  SEGMLA_E_WORKSPACE = -6,   /* workspace NULL, too small or not 256-byte aligned */
  SEGMLA_E_HIP = -7,         /* a HIP runtime call or kernel launch failed */
  SEGMLA_E_UNSUPPORTED = -8, /* valid request outside what the kernels implement */
  SEGMLA_E_STATE = -9        /* plan not built yet */
} segmla_status;

typedef enum segmla_seg_kind {
  SEGMLA_SEG_PREFIX = 0, /* computed in the request; latent stored at request positions */
  SEGMLA_SEG_DOC = 1,    /* cached document; latent stored at canonical positions 0..n-1 */
  SEGMLA_SEG_NEW = 2     /* question / new rows; latent stored at request positions */
} segmla_seg_kind;

typedef enum segmla_dtype {
  SEGMLA_F32 = 0,
  SEGMLA_BF16 = 1,
  SEGMLA_E4M3_B128 = 2 /* latent only: nope dims as OCP E4M3 codes with one fp32 scale per 128
                          values, RoPE dims bf16 (DeepSeek-V4 FP8 dataflow, TensorRT-LLM
                          reading notes, Part I) */
} segmla_dtype;

/* Segment list of one request, host memory, read only during segmla_plan_create.
 * Segment i covers request rows [offset[i], offset[i] + len[i]) and latent-pool
 * rows [pool_row[i], pool_row[i] + len[i]). Requirements (else SEGMLA_E_GEOMETRY):
 * n_seg >= 1; len[i] >= 1; offset[0] = 0 and offset[i+1] = offset[i] + len[i];
 * 0 <= pool_row[i] and pool_row[i] + len[i] <= n_pool; kind[i] a segmla_seg_kind;
 * T = offset[n-1] + len[n-1] < 2^31. A DOC at a nonzero offset is "relocated". */
typedef struct segmla_geometry {
  int32_t n_seg;
  const int64_t *pool_row;
  const int32_t *len;
  const int64_t *offset;
  const uint8_t *kind;
} segmla_geometry;

/* Layer shape and roles (RedKnot-MLA paper, head-partition paragraph). The latent
 * row holds d_nope dims followed by d_rope RoPE dims. RoPE pairs are (2k, 2k+1)
 * with theta_k = rope_base^(-2k/d_rope). Values are the full latent row when
 * v_has_rope = 1 (d_v = d_nope + d_rope), else its nope dims (d_v = d_nope).
 * Supported: kv_dtype F32 with io_dtype F32 (any even d_rope, d_nope + d_rope
 * <= 1024, d_state <= 1024); kv_dtype BF16 or E4M3_B128 with io_dtype BF16 and
 * d_nope = 512, d_rope = 64, d_state a multiple of 64. Other combinations return
 * SEGMLA_E_UNSUPPORTED. */
typedef struct segmla_layer {
  int32_t n_heads;               /* H >= 1 */
  int32_t d_nope;                /* >= 0 */
  int32_t d_rope;                /* even, >= 2 */
  int32_t d_state;               /* rows of each head's projection slice, >= 1 */
  int32_t v_has_rope;            /* 1 or 0, see above */
  const uint8_t *head_is_global; /* host [n_heads], each head's role, read at plan_create:
                                    1 Global (every row, full causal context), 0 Local (rows
                                    of A with full context, the cached contribution elsewhere),
                                    2 sink + window (every row, keys of W(t) below; projected
                                    like a Global head, never cached) */
  double rope_base;              /* > 1 */
  float softmax_scale;           /* sigma multiplying q.k, > 0 */
  int32_t kv_dtype;              /* segmla_dtype of the latent pool */
  int32_t io_dtype;              /* segmla_dtype of q, W, cached state, out and z */
  int32_t split_keys;            /* 0: library decides; -1: never split the key range;
                                    > 0 (a multiple of 64): each work item covers at most
                                    this many keys and split partials are merged by the
                                    log-sum-exp merge */
  int32_t group_heads;           /* 0 or 1: per-head projected state (z and z_cached hold
                                    one vector per head / per Local head); G >= 2, dividing
                                    n_heads: grouped state (RedKnot-MLA paper, projected-
                                    state paragraph, Eq. 3, z = z_L + z_G): heads gG .. gG+G-1
                                    form group g, z holds one vector per group, the sum of
                                    its heads' projections, and z_cached the group's cached
                                    Local contribution (else SEGMLA_E_SHAPE) */
  int32_t n_sink;                /* sink + window heads (RedKnot explainer, "Insight 1: heads
                                    have different jobs", W(i) = S_sink U [i - w, i]): key p
                                    is visible from row t iff p <= t and (p < n_sink or
                                    p >= t - window); n_sink >= 0 request positions */
  int32_t window;                /* w >= 0; both unused when no head has role 2 */
  int32_t z_e4m3;                /* 0: z in io_dtype. 1: the grouped state is emitted for the
                                    next projection as 1x128 E4M3 blocks ("Reading notes on
                                    DeepSeek-V4 serving in TensorRT-LLM", Part I, FP8
                                    dataflow bullet): per (row, group) and block of 128
                                    channels, scale = amax / 448 (fp32) and code = the OCP E4M3
                                    value of channel / scale, rounded to nearest even; the
                                    block is quantized from the bf16 state z would otherwise
                                    hold. Requires io_dtype BF16, group_heads >= 2 and
                                    d_state a multiple of 128 (else SEGMLA_E_SHAPE) */
} segmla_layer;

/* Protected-row rule (RedKnot-MLA paper, protected-row paragraph, Eq. 6):
 * A = new rows U dirty rows U first/last edge_rows rows of every relocated
 * document U the last tail_rows request rows (the forced set F), then, when
 * budget_permille > 0, the Indexer rows: with C = prefix + document rows and
 * K = ceil(budget_permille * |C| / 1000), the max(0, K - |F & C|) rows of C \ F
 * with the largest score (ties: smaller row first). Forced rows are kept even
 * when they exceed K. Requirements (else SEGMLA_E_PROTECT): edge_rows, tail_rows
 * >= 0; 0 <= budget_permille <= 1000; n_dirty >= 0; each dirty row in [0, T). */
typedef struct segmla_protect {
  int32_t edge_rows;
  int32_t tail_rows;
  int32_t budget_permille;
  int32_t n_dirty;
  const int32_t *dirty_rows; /* host [n_dirty], may be NULL when n_dirty = 0 */
} segmla_protect;

/* Device tensors of one forward, all row-major and caller-owned. A plan computes the
 * request rows of its window [q_begin, q_end) (the whole request [0, T) for
 * segmla_plan_create); q, out, z and lse hold those rows only, row t at index t - q_begin.
 * Every pointer is 16-byte aligned (the kernels move 16-byte vectors), else
 * segmla_forward returns SEGMLA_E_SHAPE.
 *  q        [q_end - q_begin][H][d_nope + d_rope] io_dtype, stored post-RoPE at request
 *           position t
 *  kv       F32/BF16: [n_pool][d_nope + d_rope]; E4M3_B128: codes uint8 [n_pool][d_nope]
 *  kv_scale E4M3_B128 only: fp32 [n_pool][d_nope / 128], else NULL
 *  kv_rope  E4M3_B128 only: bf16 [n_pool][d_rope], else NULL
 *  w        [H][d_state][d_v] io_dtype, head h's slice of the first output projection
 *  z_cached [n_pool][H_L][d_state] io_dtype, cached projected contribution of the Local
 *           heads (in head order), indexed by latent-pool row; may be NULL when H_L = 0
 *  out      [q_end - q_begin][H][d_v] io_dtype: merged head outputs in request phase;
 *           written for Global and sink + window heads on every row and for Local heads
 *           on rows in A only
 *  z        [q_end - q_begin][H][d_state] io_dtype: projected state, every (row, head)
 *           written
 *  lse      optional fp32 [q_end - q_begin][H]: natural-log log-sum-exp of sigma*q.k for
 *           every computed (row, head); NULL to skip
 * With grouped state (group_heads = G >= 2, n_groups = H / G): z is
 * [q_end - q_begin][n_groups][d_state] with z[t][g] = the sum over the group's Global and
 * sink + window heads of W_h u_h plus, on rows in A, the sum over its Local heads of W_h u_h, or else
 * z_cached[pool_row(t)][g]; z_cached is [n_pool][n_groups][d_state] (may be NULL when H_L = 0).
 * With z_e4m3 = 1: z holds the codes, uint8 [q_end - q_begin][n_groups][d_state], and
 *  z_scale  fp32 [q_end - q_begin][n_groups][d_state / 128] their block scales (z[t][g][c]
 *           stands for decode(code) * z_scale[t][g][c / 128]); NULL otherwise. */
typedef struct segmla_tensors {
  const void *q;
  const void *kv;
  const float *kv_scale;
  const void *kv_rope;
  const void *w;
  const void *z_cached;
  void *out;
  void *z;
  float *lse;
  float *z_scale;
} segmla_tensors;

typedef struct segmla_plan segmla_plan;

/* Validate geometry, roles and protection and size the plan (host only: nothing is
 * enqueued; the one HIP call reads the current device's compute-unit count, which the
 * key-range split spreads short work lists over, and 256 is assumed when no device is
 * visible). n_pool = rows of the latent pool. On success *out_plan owns a new plan. */
segmla_status segmla_plan_create(const segmla_geometry *geom, const segmla_layer *layer,
                                 const segmla_protect *prot, int64_t n_pool,
                                 segmla_plan **out_plan);

/* The same for the window of request rows [q_begin, q_end) only: chunked prefill, or
 * decode (a few new rows at the end of a long request). Every window row attends to its
 * full causal context [0, t] over all segments (relocation paragraph: rotate, attend the
 * stored latent in place, restore, merge), and the protected set A is the whole
 * request's, so windows that cover the request in pieces give the rows of the whole-request
 * forward. The latent pool must hold every row the window sees. Few window rows and a
 * long context split the key axis (merged by the log-sum-exp merge). Host only;
 * 0 <= q_begin < q_end <= T, else SEGMLA_E_SHAPE; q_end = -1 means T. */
segmla_status segmla_plan_create_range(const segmla_geometry *geom, const segmla_layer *layer,
                                       const segmla_protect *prot, int64_t n_pool,
                                       int64_t q_begin, int64_t q_end, segmla_plan **out_plan);

/* Paged latent pool (RedKnot-MLA paper, relocation and fused-consumer paragraphs: each cached
 * segment is paged in once and attended in place). The pool is cut into pages of page_rows
 * rows; page g holds pool rows [g * page_rows, (g + 1) * page_rows). Segment i's rows sit on
 * ceil(len[i] / page_rows) pages listed in order at page_table[page_start[i] ...]: row j of
 * segment i is pool row page_table[page_start[i] + j / page_rows] * page_rows + j % page_rows,
 * and the same row of the cached projected state z_cached. Pages may be shared between
 * segments (the same cached document placed twice). Host memory, read only during plan
 * creation. Requirements (else SEGMLA_E_GEOMETRY): page_rows >= 1; page_table and page_start
 * non-NULL (else SEGMLA_E_NULL); 0 <= page_start[i] and page_start[i] + ceil(len[i] /
 * page_rows) <= n_entries; every pool row a segment uses lies in [0, n_pool). Pages of a
 * multiple of 32 rows keep every 32-key tile of the attention whole. */
typedef struct segmla_pages {
  int32_t page_rows;
  int64_t n_entries;          /* entries of page_table */
  const int64_t *page_start;  /* [n_seg] */
  const int64_t *page_table;  /* [n_entries] page indices */
} segmla_pages;

/* segmla_plan_create_range over a paged latent pool: geom->pool_row is ignored (may be
 * NULL); `pages` places every segment's rows. Everything else as segmla_plan_create_range. */
segmla_status segmla_plan_create_paged(const segmla_geometry *geom, const segmla_pages *pages,
                                       const segmla_layer *layer, const segmla_protect *prot,
                                       int64_t n_pool, int64_t q_begin, int64_t q_end,
                                       segmla_plan **out_plan);

/* Device workspace bytes segmla_plan_build needs (host only). */
segmla_status segmla_plan_workspace_bytes(const segmla_plan *plan, size_t *bytes);

/* Host only, no synchronization: request rows T and |A|. |A| = |F| + need is fixed
 * by geometry and protection; only which Indexer rows are chosen needs the scores. */
segmla_status segmla_plan_rows(const segmla_plan *plan, int64_t *n_rows, int64_t *n_protected);

/* Shapes a forward of this plan reads and writes (host only, no synchronization), so that a
 * binding can check caller tensors before passing raw pointers: in elements, q holds
 * window_rows * n_heads * (d_nope + d_rope) io values, out window_rows * n_heads * d_v, z
 * window_rows * z_slots * d_state, lse window_rows * n_heads (fp32), w n_heads * d_state *
 * d_v, z_cached n_pool * zc_slots * d_state (io dtype); the latent n_pool rows (see
 * segmla_tensors); indexer_score T values. z_slots = n_heads (per-head state) or the number
 * of groups; zc_slots = the Local heads or the number of groups. */
typedef struct segmla_plan_info {
  int64_t T;               /* request rows */
  int64_t q_begin, q_end;  /* computed window */
  int64_t n_pool;          /* latent-pool rows the plan was validated against */
  int64_t n_protected;     /* |A| */
  int64_t workspace_bytes; /* as segmla_plan_workspace_bytes */
  int32_t n_heads, n_global, n_local, n_window;
  int32_t d_nope, d_rope, d_v, d_state;
  int32_t z_slots, zc_slots;
  int32_t kv_dtype, io_dtype;
  int32_t n_split;         /* key-range splits of the attention (1: none) */
  int32_t z_e4m3;          /* the layer's z_e4m3 */
} segmla_plan_info;
segmla_status segmla_plan_get_info(const segmla_plan *plan, segmla_plan_info *info);

/* Build the plan's device descriptors into `workspace` (>= segmla_plan_workspace_bytes,
 * 256-byte aligned): segment descriptors and RoPE tables (fp64-built), the row maps,
 * the protected set A and the ordered work list. indexer_score: device uint32 [T],
 * required iff the budget needs Indexer rows, else may be NULL. The workspace must
 * stay allocated and unmodified while the plan is used. It also holds forward scratch
 * (key-range split partials; with bf16 io and a window of more than 8 rows, a copy of W in
 * the projection's operand order, H * d_state * d_v * 2 bytes; with z_e4m3, the bf16 state
 * before quantization), so forwards of one plan must
 * not overlap: run them in order on one stream. */
segmla_status segmla_plan_build(segmla_plan *plan, void *workspace, size_t workspace_bytes,
                                const uint32_t *indexer_score, void *stream);

/* Re-target a built plan to another window [q_begin, q_end) of the same request (q_end = -1:
 * T): the next chunk of a chunked prefill, or the next decode row on a plan created for the
 * request's final length (a window's rows attend keys [0, t] only, so rows after the window
 * need no latent yet). The segment descriptors, RoPE tables, row maps and the protected set A
 * are the request's and are kept (RedKnot-MLA paper, TP8 fast-path paragraph: repeated
 * document bundles reuse compact segment-pointer geometry); only the window's RoPE rows, its
 * ranges in A and in the complement, the work list and the key-range split are redone, on
 * `stream`, ahead of the forwards that follow there. The window's workspace part must fit the
 * workspace the plan was built into (the key split is coarsened until it does), else
 * SEGMLA_E_WORKSPACE and the plan is unchanged; 0 <= q_begin < q_end <= T, else SEGMLA_E_SHAPE;
 * an unbuilt plan gives SEGMLA_E_STATE. Afterwards segmla_plan_workspace_bytes, _pairs and
 * _get_info describe the new window. */
segmla_status segmla_plan_set_window(segmla_plan *plan, int64_t q_begin, int64_t q_end,
                                     void *stream);

/* One layer forward (per-segment rotate / attend / restore, LSE merge, replacement
 * epilogue) on a built plan. A plan may run many forwards with new tensors. */
segmla_status segmla_forward(const segmla_plan *plan, const segmla_tensors *t, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): segmla_plan_build followed by
 * segmla_forward in one call, with the plan's workspace in a device array that the library
 * itself holds, SEGMLA_NOALLOC_MAX_BYTES per GPU, instead of caller memory. The caller
 * passes only the Indexer scores (as for segmla_plan_build) and the forward's tensors (as for
 * segmla_forward). Nothing is allocated: the array is part of the library's device code and
 * each GPU keeps its copy from the first call there until the process ends. A plan whose
 * workspace (segmla_plan_workspace_bytes) exceeds SEGMLA_NOALLOC_MAX_BYTES returns
 * SEGMLA_E_WORKSPACE before anything is enqueued. Every call on one GPU uses that GPU's one
 * array, which keeps the last call's contents: calls that overlap on one GPU (on different
 * streams or from several host threads) race and must be ordered by the caller, e.g. on one
 * stream. The plan itself is left as it was: a plan built with segmla_plan_build keeps its own
 * workspace, and an unbuilt plan stays unbuilt. No event profiling is recorded. */
#define SEGMLA_NOALLOC_MAX_BYTES (96ull << 20)
segmla_status segmla_forward_noalloc(segmla_plan *plan, const uint32_t *indexer_score,
                                     const segmla_tensors *t, void *stream);

/* Copy A (sorted ascending, |A| rows) to host memory; synchronizes `stream`. */
segmla_status segmla_copy_protected(const segmla_plan *plan, int32_t *host_rows, int64_t cap,
                                    void *stream);

/* Copy the device row maps to host memory for inspection: seg_of_row[T] (segment of
 * each request row) and pool_of_row[T] (latent-pool row of each request row); either
 * may be NULL. cap = capacity in elements of each array. Synchronizes `stream`. */
segmla_status segmla_copy_geometry(const segmla_plan *plan, int32_t *seg_of_row,
                                   int64_t *pool_of_row, int64_t cap, void *stream);

/* Stable log-sum-exp merge of split attention partials (RedKnot-MLA paper,
 * relocation paragraph). For each vector v < n_vec and split s < n_split:
 * partial_ml[s][v] = (m, l) with m the max of sigma*q.k over the split's keys
 * (natural log units, -inf when the split saw no key) and l = sum exp(sigma*q.k - m);
 * partial_o[s][v][0..d) = sum exp(sigma*q.k - m) * value (unnormalized, request phase).
 * Writes out[v][0..d) = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s in out_dtype
 * (F32 or BF16) and, if lse != NULL, lse[v] = M + log(sum_s e^(m_s - M) l_s) with
 * M = max_s m_s. A vector that saw no key at all gets out = 0 and lse = -inf.
 * All pointers are device memory; 1 <= n_split, 1 <= d <= 4096. */
segmla_status segmla_lse_merge(const float *partial_o, const float *partial_ml, int32_t n_split,
                               int64_t n_vec, int32_t d, void *out, int32_t out_dtype,
                               float *lse, void *stream);

/* Number of (row, head, key) triples the forward computes, by role: out[0] Global
 * heads (every window row), out[1] Local heads (window rows in A), out[2] sink + window
 * heads (every window row, |W(t)| keys each). Needs a built plan; copies the device-side
 * sum over A and synchronizes `stream`. */
segmla_status segmla_plan_pairs(const segmla_plan *plan, double out[3], void *stream);

/* The analytic ledger, namespaces kept apart (RedKnot-MLA paper, namespaces
 * paragraph; head-row ceiling Eq. 8). Host only:
 * out[0] logical head-row saving (r / (f_front + r + f_back)) * (h_local / h);
 * out[1] physical token-row saving of one reusable layer, h_local * (T - n_protected) / (h * T);
 * out[2] analytic attention operator saving of one reusable layer,
 *        1 - (global_pairs + local_pairs) / (h * T * (T + 1) / 2), with the pair counts
 *        (global_pairs: every head computed on every row, Global and sink + window)
 *        of segmla_plan_pairs; NaN when local_pairs < 0.
 * Wall-clock time, the fourth namespace, is measured by the caller. */
segmla_status segmla_ledger(int32_t f_front, int32_t r, int32_t f_back, int32_t h,
                            int32_t h_local, int64_t T, int64_t n_protected,
                            double global_pairs, double local_pairs, double out[3]);

/* Stage timing with HIP events on the forward's stream (tracing aid). enable = 1 creates the
 * plan's events and zeroes the totals; 0 stops recording. While enabled, each forward and
 * build records events around its stages, and the next forward first waits for the previous
 * forward's last event (so at most one profiled forward is in flight). Host only apart from
 * the event calls; returns SEGMLA_E_HIP if event creation fails. */
segmla_status segmla_profile_enable(segmla_plan *plan, int32_t enable);

/* Wait for the last recorded events and return accumulated milliseconds per stage since
 * segmla_profile_enable(plan, 1): ms[0] attention kernel (rotate / attend / restore / merge),
 * ms[1] split-partial merge kernel, ms[2] epilogue (projection + cached-state copy),
 * ms[3] plan build (geometry, protected rows, work list); *n_forward = profiled forwards. */
segmla_status segmla_profile_read(segmla_plan *plan, double ms[4], int64_t *n_forward,
                                  int64_t *n_build);

/* Artifact prefetch (RedKnot-MLA paper, TP8 fast-path paragraph: while a layer runs, a
 * dedicated stream prefetches the tiles of a future layer group, and device events, not host
 * polling, guard their consumption). A prefetcher owns one stream of default priority and its
 * events. segmla_prefetch stages row ranges, e.g. the latent rows and cached projected state
 * of the segments a later layer reads, from host memory (pinned) or device memory into device
 * buffers: the transfers start once all work enqueued on `after_stream` before the call has
 * finished (the destination may be buffers that work read) and run beside work enqueued there
 * afterwards. segmla_prefetch_wait makes `stream` wait for the transfers on the device; work
 * enqueued on it afterwards sees the staged rows. Each prefetch call replaces the previous
 * one's events. The library allocates no device memory: all buffers are the caller's. */
typedef struct segmla_copy_range {
  const void *src;      /* first source row: host (pinned) or device memory */
  void *dst;            /* first destination row: device memory */
  int64_t rows;         /* rows to copy, >= 0 */
  int64_t row_bytes;    /* bytes per row, >= 1 */
  int64_t src_stride;   /* bytes from one source row to the next, >= row_bytes */
  int64_t dst_stride;   /* bytes from one destination row to the next, >= row_bytes */
} segmla_copy_range;
typedef struct segmla_prefetcher segmla_prefetcher;

/* Create a prefetcher (its stream and events); SEGMLA_E_HIP if the runtime refuses. */
segmla_status segmla_prefetcher_create(segmla_prefetcher **out);
/* Enqueue the transfers of n_ranges ranges (SEGMLA_E_SHAPE for negative sizes or strides
 * below row_bytes, SEGMLA_E_NULL for missing pointers; nothing is enqueued then). */
segmla_status segmla_prefetch(segmla_prefetcher *pf, const segmla_copy_range *ranges,
                              int32_t n_ranges, void *after_stream);
/* Make `stream` wait for the last prefetch's transfers (SEGMLA_E_STATE before any prefetch). */
segmla_status segmla_prefetch_wait(segmla_prefetcher *pf, void *stream);
/* Milliseconds the last prefetch's transfers took on the prefetch stream (waits for them). */
segmla_status segmla_prefetch_elapsed(segmla_prefetcher *pf, float *ms);
/* Wait for outstanding transfers, then release the stream and events. */
void segmla_prefetcher_destroy(segmla_prefetcher *pf);

/* Compressed-history attention of the DeepSeek-V4 CSA and HCA layers ("Reading notes on
 * DeepSeek-V4 serving in TensorRT-LLM", section 1: the hybrid attention bullets and the
 * dual-pool kernel paragraph) over the relocated segments of a plan. Each request row t attends,
 * with every one of the plan's n_heads heads sharing the keys, in one softmax:
 *  - the raw keys p with max(0, t - window) <= p <= t of the plan's latent pool (128 most recent
 *    tokens: window = 127), and
 *  - compressed entries of a second pool: every entry available at t (HCA, top_k = 0), or the
 *    row's Indexer list (CSA, top_k = K > 0).
 * Entries under relocation (the pages say nothing of it; the plainest reading): compression runs
 * per segment when the segment is stored, so segment i holds floor(len[i] / ratio) entries.
 * Entry j of segment i stands for the segment's rows [ratio j, ratio j + ratio), lies at
 * compressed-pool row cpool_row[i] + j, is encoded in the segment's stored RoPE frame (like its
 * raw rows: documents canonical, prefix and new rows at request positions) and becomes available
 * to row t once offset[i] + ratio (j + 1) - 1 <= t. Entry ids number the request's entries in
 * request order, segment by segment. Both pools are attended in place: the query is rotated by
 * -Delta_i per segment and the output phase restored, as for the layer forward (RedKnot-MLA
 * paper, relocation paragraph, Eq. 5).
 * Supported: plans with kv_dtype and io_dtype BF16 (d_nope = 512, d_rope = 64), any head roles
 * (ignored here: every head attends), contiguous or paged latent pools; else
 * SEGMLA_E_UNSUPPORTED. Requirements (else SEGMLA_E_SHAPE): ratio >= 1, window >= 0,
 * top_k >= 0, 0 <= n_cpool < 2^31; (else SEGMLA_E_GEOMETRY) for every segment
 * 0 <= cpool_row[i] and cpool_row[i] + floor(len[i] / ratio) <= n_cpool. */
typedef struct segmla_dual_pool {
  int32_t ratio;             /* request rows per compressed entry (4 for CSA, 128 for HCA) */
  int32_t window;            /* raw keys t - window .. t */
  int32_t top_k;             /* width K of the per-row lists; 0: every available entry */
  int64_t n_cpool;           /* rows of the compressed pool */
  const int64_t *cpool_row;  /* host [n_seg], read during segmla_dual_create only */
} segmla_dual_pool;

/* Device tensors of one dual-pool forward, row-major, caller-owned, 16-byte aligned (cidx and
 * clen 4-byte aligned), else SEGMLA_E_SHAPE. Rows are the plan's window [q_begin, q_end).
 *  q     [q_end - q_begin][H][576] bf16, stored post-RoPE at request position t
 *  kv    [n_pool][576] bf16, the plan's latent pool
 *  ckv   [n_cpool][576] bf16, the compressed pool
 *  cidx  CSA: int32 [q_end - q_begin][top_k], the row's entry ids; NULL for HCA
 *  clen  CSA: int32 [q_end - q_begin], how many of the row's ids to read (clamped to
 *        [0, top_k]); NULL for HCA
 *  out   [q_end - q_begin][H][d_v] bf16, merged outputs in request phase
 *  lse   optional fp32 [q_end - q_begin][H]: natural-log log-sum-exp of sigma*q.k
 * A list is read in order up to, not including, the first id that is not an entry available at
 * the row (negative, at least the request's entry count, or not yet available), so an Indexer
 * may pad its fixed-width buffer with -1. Ids need not be sorted (sorted lists touch each
 * segment's RoPE frame once); an id listed twice is attended twice. */
typedef struct segmla_dual_tensors {
  const void *q;
  const void *kv;
  const void *ckv;
  const int32_t *cidx;
  const int32_t *clen;
  void *out;
  float *lse;
} segmla_dual_tensors;

typedef struct segmla_dual segmla_dual;

/* Validate the compressed geometry against a plan and size its tables (host only). The plan
 * must outlive the dual-pool object; it need not be built yet. */
segmla_status segmla_dual_create(const segmla_plan *plan, const segmla_dual_pool *dp,
                                 segmla_dual **out_dual);
/* Device workspace bytes segmla_dual_build needs, and the request's entry count (host only;
 * either pointer may be NULL). */
segmla_status segmla_dual_sizes(const segmla_dual *dual, size_t *workspace_bytes,
                                int64_t *n_entries);
/* Copy the entry tables into `workspace` (256-byte aligned, >= segmla_dual_sizes bytes) on
 * `stream`. The workspace must stay allocated and unmodified while the object is used. */
segmla_status segmla_dual_build(segmla_dual *dual, void *workspace, size_t workspace_bytes,
                                void *stream);
/* One dual-pool forward on the rows of the plan's current window (the plan and the object
 * built: else SEGMLA_E_STATE). Enqueues one kernel, no synchronization; capturable in a HIP
 * graph. */
segmla_status segmla_dual_forward(const segmla_dual *dual, const segmla_dual_tensors *t,
                                  void *stream);
void segmla_dual_destroy(segmla_dual *dual);

void segmla_plan_destroy(segmla_plan *plan);
const char *segmla_status_string(int32_t status);
int32_t segmla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGMLA_H */
