// Host side of libsegmla: argument validation, plan sizing, workspace layout and launch
// sequencing on the caller's stream. Every entry point validates before it enqueues anything.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/segmla.h"
#include "internal.h"

using namespace segmla;

struct segmla_plan {
  // geometry
  int32_t n_seg = 0;
  int32_t T = 0;
  int32_t q0 = 0, q1 = 0;  // computed window of request rows [q0, q1)
  int64_t n_pool = 0;
  std::vector<SegDesc> segs;  // logical segments (kinds, edges, relocation)
  // physical runs: maximal stretches of a segment's rows that are contiguous in the pool (one
  // per segment for an unpaged pool); each carries its segment's phase shift and, as `frame`,
  // its segment's index. The attention, the RoPE tables and the row map work on runs.
  std::vector<SegDesc> runs;
  int32_t n_run = 0;
  // layer
  int32_t H = 0, HG = 0, HL = 0, HW = 0, d_nope = 0, d_rope = 0, d_qk = 0, d_v = 0, d_state = 0;
  int32_t v_has_rope = 1, kv_dtype = 0, io_dtype = 0;
  double rope_base = 10000.0;
  float sigma = 1.f;
  // head lists by role: Global (1), Local (0), sink + window (2); the full-context heads
  // (Global and Local, stream F) and the heads computed on every row (Global and sink + window,
  // the epilogue's all-row heads)
  std::vector<int32_t> ghead, lhead, whead, fhead, rowhead;
  int32_t n_sink = 0, window = 0;
  int32_t z_e4m3 = 0;  // grouped state emitted as 1x128 E4M3 codes + fp32 block scales
  int32_t G = 1, n_groups = 0;             // grouped projected state when G >= 2
  std::vector<int32_t> grp_gstart, grp_ghead;  // each group's all-row heads (CSR)
  // protection
  int32_t edge_rows = 0, tail_rows = 0, budget_permille = 0;
  std::vector<int32_t> dirty;  // sorted, unique
  std::vector<char> upload;    // workspace bytes [0, o_segcs): the host-built tables, in place
  int64_t n_forced = 0, n_cand = 0, K = 0, need = 0, nA = 0;
  // prefix counts over request rows: forced rows, and candidate rows not forced (a window's
  // share of A is bounded by them without the Indexer's picks)
  std::vector<int32_t> cum_forced, cum_free_cand;
  int32_t split_req = 0;  // the layer's split_keys request (0: the library decides)
  // work decomposition
  int32_t nF = 0, nG = 0, nW = 0, n_split = 1, split_keys = 0, n_blk = 0;
  int32_t n_cu = 256;  // compute units of the device the plan was sized for
  bool thin = false;   // bf16 projection as matrix-vector products (small windows)
  // workspace layout (byte offsets, 256-aligned)
  size_t o_seg = 0, o_segcs = 0, o_stepcs = 0, o_rowcs = 0, o_seg_of_row = 0, o_flags = 0,
         o_dirty = 0, o_ghead = 0, o_lhead = 0, o_whead = 0, o_fhead = 0, o_rowhead = 0,
         o_alist = 0, o_nalist = 0, o_blk_count = 0,
         o_blk_sum = 0, o_sum_a = 0, o_sel = 0, o_work = 0, o_part_o = 0, o_part_ml = 0, o_wt = 0,
         o_rng = 0, o_lseg = 0, o_grp = 0, o_zpart = 0, o_zbf = 0, ws_bytes = 0;
  // largest number of window rows inside / outside A (the Indexer picks decide the actual)
  int64_t nA_w = 0, nNA_w = 0;
  // profiling (events on the caller's stream)
  bool prof = false, fwd_pending = false, build_pending = false;
  hipEvent_t ev[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  double prof_ms[4] = {0, 0, 0, 0};
  int64_t prof_fwd = 0, prof_build = 0;
  // build state
  bool built = false;
  char* ws = nullptr;
  size_t ws_capacity = 0;  // bytes of the workspace the plan was built into
  size_t o_tail = 0;       // first byte of the window-dependent part of the workspace
  template <typename X>
  X* at(size_t off) const { return reinterpret_cast<X*>(ws + off); }
};

namespace {

// Compute units of the current device: the key-range split spreads short work lists over
// them. A plan can be sized where no device is visible (validation on a host without a GPU);
// it then assumes 256, the MI355X count, and clears the runtime's error state.
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

float elapsed(hipEvent_t a, hipEvent_t b) {
  float ms = 0.f;
  return hipEventElapsedTime(&ms, a, b) == hipSuccess ? ms : 0.f;
}

// Fold the previous profiled forward / build into the totals (waits for their events).
hipError_t flush_profile(segmla_plan* p) {
  if (p->fwd_pending) {
    hipError_t e = hipEventSynchronize(p->ev[3]);
    if (e != hipSuccess) return e;
    p->prof_ms[0] += elapsed(p->ev[0], p->ev[1]);
    p->prof_ms[1] += elapsed(p->ev[1], p->ev[2]);
    p->prof_ms[2] += elapsed(p->ev[2], p->ev[3]);
    p->prof_fwd += 1;
    p->fwd_pending = false;
  }
  if (p->build_pending) {
    hipError_t e = hipEventSynchronize(p->ev[5]);
    if (e != hipSuccess) return e;
    p->prof_ms[3] += elapsed(p->ev[4], p->ev[5]);
    p->prof_build += 1;
    p->build_pending = false;
  }
  return hipSuccess;
}

bool is_dtype(int32_t d) { return d == SEGMLA_F32 || d == SEGMLA_BF16 || d == SEGMLA_E4M3_B128; }

segmla_status check_layer(const segmla_layer* L) {
  if (!L->head_is_global) return SEGMLA_E_NULL;
  if (L->n_heads < 1 || L->d_nope < 0 || L->d_rope < 2 || (L->d_rope & 1) || L->d_state < 1)
    return SEGMLA_E_SHAPE;
  if (L->v_has_rope != 0 && L->v_has_rope != 1) return SEGMLA_E_SHAPE;
  if (!(L->rope_base > 1.0) || !std::isfinite(L->rope_base)) return SEGMLA_E_SHAPE;
  if (!(L->softmax_scale > 0.f) || !std::isfinite(L->softmax_scale)) return SEGMLA_E_SHAPE;
  for (int h = 0; h < L->n_heads; ++h)
    if (L->head_is_global[h] > 2) return SEGMLA_E_SHAPE;
  if (L->n_sink < 0 || L->window < 0) return SEGMLA_E_SHAPE;
  if (!is_dtype(L->kv_dtype) || !is_dtype(L->io_dtype)) return SEGMLA_E_DTYPE;
  if (L->io_dtype == SEGMLA_E4M3_B128) return SEGMLA_E_DTYPE;
  if (L->split_keys < -1 || (L->split_keys > 0 && (L->split_keys % 64) != 0)) return SEGMLA_E_SHAPE;
  if (L->group_heads < 0 || (L->group_heads >= 2 && L->n_heads % L->group_heads != 0))
    return SEGMLA_E_SHAPE;
  if (L->z_e4m3 != 0 && (L->z_e4m3 != 1 || L->io_dtype != SEGMLA_BF16 || L->group_heads < 2 ||
                         L->d_state % 128 != 0))
    return SEGMLA_E_SHAPE;
  const int d_qk = L->d_nope + L->d_rope;
  if (L->kv_dtype == SEGMLA_F32) {
    if (L->io_dtype != SEGMLA_F32) return SEGMLA_E_UNSUPPORTED;
    if (d_qk > 1024 || L->d_state > 1024 || (L->d_nope & 1)) return SEGMLA_E_UNSUPPORTED;
  } else {
    if (L->io_dtype != SEGMLA_BF16) return SEGMLA_E_UNSUPPORTED;
    if (L->d_nope != 512 || L->d_rope != 64 || (L->d_state % 64) != 0 || L->d_state > 4096)
      return SEGMLA_E_UNSUPPORTED;
  }
  return SEGMLA_OK;
}

segmla_status check_geometry(const segmla_geometry* G, const segmla_pages* P, int64_t n_pool,
                             int64_t* T_out) {
  if ((!P && !G->pool_row) || !G->len || !G->offset || !G->kind) return SEGMLA_E_NULL;
  if (G->n_seg < 1 || n_pool < 1) return SEGMLA_E_GEOMETRY;
  int64_t pos = 0;
  for (int i = 0; i < G->n_seg; ++i) {
    if (G->len[i] < 1 || G->kind[i] > 2) return SEGMLA_E_GEOMETRY;
    if (G->offset[i] != pos) return SEGMLA_E_GEOMETRY;
    if (!P && (G->pool_row[i] < 0 || G->pool_row[i] > n_pool - G->len[i])) return SEGMLA_E_GEOMETRY;
    pos += G->len[i];
    if (pos >= ((int64_t)1 << 31)) return SEGMLA_E_GEOMETRY;
  }
  if (P) {  // every page a segment uses: listed, and its used rows inside the pool
    if (!P->page_start || !P->page_table) return SEGMLA_E_NULL;
    if (P->page_rows < 1 || P->n_entries < 0) return SEGMLA_E_GEOMETRY;
    const int64_t pr = P->page_rows;
    for (int i = 0; i < G->n_seg; ++i) {
      const int64_t np = (G->len[i] + pr - 1) / pr, st = P->page_start[i];
      if (st < 0 || st > P->n_entries - np) return SEGMLA_E_GEOMETRY;
      for (int64_t k = 0; k < np; ++k) {
        const int64_t rows = std::min<int64_t>(pr, G->len[i] - k * pr), g = P->page_table[st + k];
        // the page's used rows [g * pr, g * pr + rows) inside [0, n_pool), in int64 without
        // overflow (no division: it would round a negative room up to page 0)
        if (g < 0 || g > (INT64_MAX - rows) / pr || g * pr + rows > n_pool) return SEGMLA_E_GEOMETRY;
      }
    }
  }
  *T_out = pos;
  return SEGMLA_OK;
}

TileMap tile_map(const segmla_plan* p) {
  TileMap m;
  m.alist = p->at<int32_t>(p->o_alist);
  m.nalist = p->at<int32_t>(p->o_nalist);
  m.ghead = p->at<int32_t>(p->o_ghead);
  m.whead = p->at<int32_t>(p->o_whead);
  m.fhead = p->HW > 0 ? p->at<int32_t>(p->o_fhead) : nullptr;  // else heads 0 .. H - 1
  m.rng = p->at<int32_t>(p->o_rng);
  m.H = p->H;
  m.HF = p->H - p->HW;
  m.HG = p->HG;
  m.HW = p->HW;
  m.nW = p->nW;
  m.q0 = p->q0;
  m.nq = p->q1 - p->q0;
  m.nF = p->nF;
  m.nG = p->nG;
  return m;
}

// The window-dependent sizing of a plan: its computed rows [q0, q1), the tile streams, the key
// split, and the workspace tail from o_tail on (the window's RoPE rows, the work list, the split
// partials and the projection's scratch). Fails with SEGMLA_E_WORKSPACE, leaving the plan as it
// was, when the tail would end past `capacity` (fewer key splits are tried first: the split only
// spreads work, it changes no result beyond the summation order).
segmla_status size_window(segmla_plan* p, int32_t q0, int32_t q1, size_t capacity) {
  // window rows of A: its forced rows, plus at most min(need, free candidates) Indexer picks
  const int64_t nf_w = p->cum_forced[q1] - p->cum_forced[q0];
  const int64_t nc_w = p->cum_free_cand[q1] - p->cum_free_cand[q0];
  const int64_t L = (int64_t)q1 - q0;
  const int64_t nA_w = std::min<int64_t>(nf_w + std::min(p->need, nc_w), L);
  const int64_t nNA_w = L - nf_w;
  // Work decomposition: qvec tiles of stream F (window rows of A x the full-context heads),
  // stream G (other window rows x Global heads), optionally split along the key axis, and
  // stream W (every window row x the sink + window heads, never split). For a window smaller
  // than the request, the split between F and G depends on the Indexer picks: both are sized
  // for their largest share.
  const int64_t qF = nA_w * (p->H - p->HW), qG = nNA_w * p->HG, qW = L * p->HW;
  const int64_t nF = (qF + kTileQ - 1) / kTileQ, nG = (qG + kTileQ - 1) / kTileQ;
  const int64_t nW = (qW + kTileQ - 1) / kTileQ;
  if (nF + nG + nW > INT32_MAX / 4) return SEGMLA_E_UNSUPPORTED;
  const int64_t n_tiles = nF + nG;
  const int32_t keys = q1;  // the window's rows see keys [0, q1) at most
  const int64_t ncu = p->n_cu;
  int32_t sk = p->split_req;
  if (sk == 0) {  // few tiles and a long context: spread the key axis over more workgroups
    sk = -1;
    if (n_tiles > 0 && n_tiles < 2 * ncu && keys > 2048) {
      // about four workgroups per CU, each with at least 1024 keys; where that leaves CUs idle
      // (decode: one or two tiles), one workgroup per CU, each with at least 256 keys
      int64_t want = std::min<int64_t>((4 * ncu + n_tiles - 1) / n_tiles, (keys + 1023) / 1024);
      if (want * n_tiles < ncu)
        want = std::min<int64_t>((ncu + n_tiles - 1) / n_tiles, (keys + 255) / 256);
      if (want > 1) sk = (int32_t)((((keys + want - 1) / want) + 63) / 64 * 64);
    }
  }
  const bool thin = p->io_dtype == SEGMLA_BF16 && thin_projection((int)L, p->d_v, p->d_state);
  const size_t half = (size_t)p->d_rope / 2;
  for (;;) {
    const int32_t n_split = (sk > 0 && sk < keys) ? (int32_t)((keys + sk - 1) / sk) : 1;
    size_t o = p->o_tail;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + std::max<size_t>(bytes, 1)); return at; };
    const size_t o_rowcs = take(sizeof(float2) * half * (size_t)L);
    const size_t o_work = take(sizeof(int32_t) * (size_t)n_tiles);
    size_t o_part_o = 0, o_part_ml = 0, o_zpart = 0, o_wt = 0, o_zbf = 0;
    if (n_split > 1) {
      const size_t nvec = (size_t)n_tiles * kTileQ;
      o_part_o = take(sizeof(float) * (size_t)n_split * nvec * p->d_v);
      o_part_ml = take(sizeof(float) * 2 * (size_t)n_split * nvec);
    }
    // bf16 projection: matrix-vector for small windows, else MFMA tiles reading W in their
    // operand order from a per-forward copy (forward scratch); grouped state in a small window
    // (decode): per-head fp32 projections, summed per group
    if (thin && p->G >= 2) o_zpart = take(sizeof(float) * (size_t)L * p->H * p->d_state);
    if (p->io_dtype == SEGMLA_BF16 && !thin) o_wt = take((size_t)p->H * p->d_state * p->d_v * 2);
    // E4M3 output of the grouped state: the bf16 state, quantized block by block afterwards
    if (p->z_e4m3) o_zbf = take((size_t)L * p->n_groups * p->d_state * 2);
    if (o > capacity) {
      if (n_split > 1 && sk < keys) {  // fewer, longer splits
        sk = (int32_t)std::min<int64_t>((int64_t)sk * 2, keys);
        continue;
      }
      return SEGMLA_E_WORKSPACE;
    }
    p->q0 = q0;
    p->q1 = q1;
    p->nA_w = nA_w;
    p->nNA_w = nNA_w;
    p->nF = (int32_t)nF;
    p->nG = (int32_t)nG;
    p->nW = (int32_t)nW;
    p->split_keys = n_split > 1 ? sk : 0;
    p->n_split = n_split;
    p->thin = thin;
    p->o_rowcs = o_rowcs;
    p->o_work = o_work;
    p->o_part_o = o_part_o;
    p->o_part_ml = o_part_ml;
    p->o_zpart = o_zpart;
    p->o_wt = o_wt;
    p->o_zbf = o_zbf;
    p->ws_bytes = o;
    return SEGMLA_OK;
  }
}

// Enqueue the plan build into workspace `ws` (validated by the caller) on stream s.
segmla_status build_impl(segmla_plan* p, char* ws, const uint32_t* indexer_score, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (p->prof) {
    if (flush_profile(p) != hipSuccess || hipEventRecord(p->ev[4], s) != hipSuccess) return SEGMLA_E_HIP;
  }
  p->ws = ws;
  p->built = false;
  p->ws_capacity = p->ws_bytes;
  // the segment, run and head tables: one upload of the image laid out at plan creation
  e = hipMemcpyAsync(p->ws, p->upload.data(), p->upload.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return SEGMLA_E_HIP;
  e = launch_geometry(p->at<SegDesc>(p->o_seg), p->n_run, p->T, p->q0, p->q1, p->d_rope,
                      p->rope_base, p->at<int32_t>(p->o_seg_of_row), p->at<float2>(p->o_segcs),
                      p->at<float2>(p->o_stepcs), p->at<float2>(p->o_rowcs), s);
  if (e != hipSuccess) return SEGMLA_E_HIP;
  e = launch_protect(p->at<SegDesc>(p->o_lseg), p->at<SegDesc>(p->o_seg), p->at<int32_t>(p->o_seg_of_row), p->T,
                     p->edge_rows, p->tail_rows, p->at<int32_t>(p->o_dirty), (int)p->dirty.size(),
                     indexer_score, p->need, p->at<uint8_t>(p->o_flags), p->at<uint32_t>(p->o_sel),
                     p->at<int32_t>(p->o_blk_count), p->at<uint64_t>(p->o_blk_sum), p->n_blk,
                     p->at<int32_t>(p->o_alist), p->at<int32_t>(p->o_nalist), (int)p->nA,
                     p->at<uint64_t>(p->o_sum_a), p->q0, p->q1, p->at<int32_t>(p->o_rng), s);
  if (e != hipSuccess) return SEGMLA_E_HIP;
  e = launch_worklist(tile_map(p), p->at<int32_t>(p->o_work), s);
  if (e != hipSuccess) return SEGMLA_E_HIP;
  if (p->prof) {
    if (hipEventRecord(p->ev[5], s) != hipSuccess) return SEGMLA_E_HIP;
    p->build_pending = true;
  }
  p->built = true;
  return SEGMLA_OK;
}

// Tensor checks of one forward (host only).
segmla_status check_tensors(const segmla_plan* p, const segmla_tensors* t) {
  if (!t->q || !t->kv || !t->w || !t->out || !t->z) return SEGMLA_E_NULL;
  if (p->HL > 0 && !t->z_cached) return SEGMLA_E_NULL;
  if (p->kv_dtype == SEGMLA_E4M3_B128 && (!t->kv_scale || !t->kv_rope)) return SEGMLA_E_NULL;
  if (p->z_e4m3 && !t->z_scale) return SEGMLA_E_NULL;
  for (const void* ptr : {t->q, t->kv, (const void*)t->kv_scale, t->kv_rope, t->w, t->z_cached,
                          (const void*)t->out, (const void*)t->z, (const void*)t->lse,
                          (const void*)t->z_scale})
    if ((uintptr_t)ptr % 16 != 0) return SEGMLA_E_SHAPE;
  return SEGMLA_OK;
}

// Enqueue one forward of a built plan (tensors checked by the caller) on stream s.
segmla_status forward_impl(const segmla_plan* p, const segmla_tensors* t, hipStream_t s) {
  AttnArgs a;
  a.q = t->q;
  a.kv = t->kv;
  a.kv_scale = t->kv_scale;
  a.kv_rope = t->kv_rope;
  a.out = t->out;
  a.lse = t->lse;
  a.part_o = p->n_split > 1 ? p->at<float>(p->o_part_o) : nullptr;
  a.part_ml = p->n_split > 1 ? p->at<float>(p->o_part_ml) : nullptr;
  a.seg = p->at<SegDesc>(p->o_seg);
  a.seg_of_row = p->at<int32_t>(p->o_seg_of_row);
  a.segcs = p->at<float2>(p->o_segcs);
  a.stepcs = p->at<float2>(p->o_stepcs);
  a.work = p->at<int32_t>(p->o_work);
  a.map = tile_map(p);
  a.n_seg = p->n_run;
  a.T = p->T;
  a.d_nope = p->d_nope;
  a.d_rope = p->d_rope;
  a.d_v = p->d_v;
  a.q0 = p->q0;
  a.n_split = p->n_split;
  a.split_keys = p->split_keys;
  a.sigma = p->sigma;
  a.n_sink = p->n_sink;
  a.win = p->window;
  // one-row windows (decode) with a key split: at most 64 query vectors per tile, which the
  // decode kernel runs on all four waves (two sets over alternate key tiles)
  const bool dec = p->kv_dtype == SEGMLA_BF16 && p->n_split > 1 && p->q1 - p->q0 == 1 &&
                   p->H - p->HW <= 64 && p->HG <= 64;
  a.part_bf16 = dec ? 1 : 0;  // the decode kernel writes its partial outputs in bf16
  // the replacement copy rides on the full-context attention grid (bf16 per-head state)
  const int64_t n_wg = (int64_t)(p->nF + p->nG) * p->n_split;
  const bool fuse_rc = !dec && p->io_dtype == SEGMLA_BF16 && p->G < 2 && p->HL > 0 && p->nNA_w > 0 &&
                       n_wg > 0;
  a.z_cached = t->z_cached;
  a.z = t->z;
  a.lhead = p->at<int32_t>(p->o_lhead);
  a.HL = p->HL;
  a.z_chunks = p->d_state * 2 / 16;
  // (a grid too small for the rows keeps the separate copy kernel: at most 64 rows per workgroup)
  const int64_t rc_rows = fuse_rc ? (p->nNA_w + n_wg - 1) / n_wg : 0;
  a.rc_rows = rc_rows <= 64 ? (int32_t)rc_rows : 0;
  hipError_t e = hipSuccess;
  segmla_plan* pm = const_cast<segmla_plan*>(p);  // profiling state only
  if (p->prof) {
    if (flush_profile(pm) != hipSuccess || hipEventRecord(p->ev[0], s) != hipSuccess)
      return SEGMLA_E_HIP;
  }
  if (p->nF + p->nG > 0)
    e = dec ? launch_attn_decode(a, p->v_has_rope, s) : launch_attn(a, p->kv_dtype, p->v_has_rope, s);
  if (e == hipSuccess && p->nW > 0) {  // sink + window heads: their own grid, never split
    AttnArgs aw = a;
    aw.n_split = 1;
    aw.split_keys = 0;
    aw.part_o = aw.part_ml = nullptr;
    aw.rc_rows = 0;
    e = launch_attn_window(aw, p->kv_dtype, p->v_has_rope, s);
  }
  if (e == hipSuccess && p->prof) e = hipEventRecord(p->ev[1], s);
  // decode rows with per-head state: the merge and the projection run as one kernel (the
  // profile's merge stage is then empty and its epilogue stage holds both)
  const bool fuse_dec = dec && p->G < 2 && p->HW == 0 && p->thin && !p->z_e4m3 &&
                        p->io_dtype == SEGMLA_BF16 && dec_merge_project_fits(p->d_v, p->d_state, p->n_split);
  if (e == hipSuccess && p->nF + p->nG > 0 && p->n_split > 1 && !fuse_dec)
    e = launch_merge_tiles(a, p->io_dtype, s);
  if (e == hipSuccess && p->prof) e = hipEventRecord(p->ev[2], s);
  if (e != hipSuccess) return SEGMLA_E_HIP;
  EpiArgs ep;
  ep.out = t->out;
  ep.w = t->w;
  ep.wt = (p->io_dtype == SEGMLA_BF16 && !p->thin) ? p->at<void>(p->o_wt) : nullptr;
  ep.thin = p->thin ? 1 : 0;
  ep.restore_done = a.rc_rows > 0 ? 1 : 0;
  ep.z_cached = t->z_cached;
  ep.z = t->z;
  ep.rowcs = p->at<float2>(p->o_rowcs);
  ep.alist = p->at<int32_t>(p->o_alist);
  ep.nalist = p->at<int32_t>(p->o_nalist);
  ep.rng = p->at<int32_t>(p->o_rng);
  ep.ghead = p->at<int32_t>(p->o_rowhead);  // every-row heads: Global and sink + window
  ep.lhead = p->at<int32_t>(p->o_lhead);
  ep.seg_of_row = p->at<int32_t>(p->o_seg_of_row);
  ep.seg = p->at<SegDesc>(p->o_seg);
  ep.q0 = p->q0;
  ep.nq = p->q1 - p->q0;
  ep.H = p->H;
  ep.HG = p->HG + p->HW;
  ep.HL = p->HL;
  ep.nA = (int32_t)p->nA_w;
  ep.nNA = (int32_t)p->nNA_w;
  ep.d_nope = p->d_nope;
  ep.d_rope = p->d_rope;
  ep.d_v = p->d_v;
  ep.d_state = p->d_state;
  ep.v_has_rope = p->v_has_rope;
  ep.G = p->G;
  ep.n_groups = p->n_groups;
  ep.grp_gstart = p->at<int32_t>(p->o_grp);
  ep.grp_ghead = p->at<int32_t>(p->o_grp) + p->grp_gstart.size();
  ep.zpart = (p->thin && p->G >= 2) ? p->at<float>(p->o_zpart) : nullptr;
  if (p->z_e4m3) ep.z = p->at<void>(p->o_zbf);  // the bf16 state, then its E4M3 blocks
  e = fuse_dec ? launch_dec_merge_project(a, ep, s) : launch_epilogue(ep, p->io_dtype, s);
  if (e == hipSuccess && p->z_e4m3)
    e = launch_quant_e4m3((const __bf16*)ep.z, (uint8_t*)t->z, t->z_scale,
                          (int64_t)(p->q1 - p->q0) * p->n_groups * (p->d_state / 128), s);
  if (e == hipSuccess && p->prof) {
    e = hipEventRecord(p->ev[3], s);
    pm->fwd_pending = e == hipSuccess;
  }
  return e == hipSuccess ? SEGMLA_OK : SEGMLA_E_HIP;
}

}  // namespace

// ------------------------------------------------------------ forward without allocation
// The plan's workspace in a device array of the library's own. Each GPU the library runs on
// holds its copy from the first call there until the process ends; the address of a device's
// copy is taken once, with that device current, and kept per device. Host code uses only these
// addresses: the array's name stands for a host-side shadow, not for device memory.
static __device__ __align__(256) char scratch[SEGMLA_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t segmla_abi_version(void) { return SEGMLA_ABI_VERSION; }

const char* segmla_status_string(int32_t s) {
  switch (s) {
    case SEGMLA_OK: return "ok";
    case SEGMLA_E_NULL: return "required pointer is NULL";
    case SEGMLA_E_GEOMETRY: return "malformed segment geometry";
    case SEGMLA_E_SHAPE: return "invalid layer shape or role mask";
    case SEGMLA_E_DTYPE: return "invalid dtype";
    case SEGMLA_E_PROTECT: return "invalid protection parameters or missing Indexer scores";
    case SEGMLA_E_WORKSPACE: return "workspace missing, too small or misaligned";
    case SEGMLA_E_HIP: return "HIP runtime call or kernel launch failed";
    case SEGMLA_E_UNSUPPORTED: return "shape/dtype combination not implemented";
    case SEGMLA_E_STATE: return "plan not built";
    default: return "unknown status";
  }
}

segmla_status segmla_plan_create(const segmla_geometry* geom, const segmla_layer* layer,
                                 const segmla_protect* prot, int64_t n_pool,
                                 segmla_plan** out_plan) {
  return segmla_plan_create_range(geom, layer, prot, n_pool, 0, -1, out_plan);
}

segmla_status segmla_plan_create_range(const segmla_geometry* geom, const segmla_layer* layer,
                                       const segmla_protect* prot, int64_t n_pool,
                                       int64_t q_begin, int64_t q_end, segmla_plan** out_plan) {
  return segmla_plan_create_paged(geom, nullptr, layer, prot, n_pool, q_begin, q_end, out_plan);
}

// With pages = NULL the pool is unpaged (geom->pool_row places each segment).
segmla_status segmla_plan_create_paged(const segmla_geometry* geom, const segmla_pages* pages,
                                       const segmla_layer* layer, const segmla_protect* prot,
                                       int64_t n_pool, int64_t q_begin, int64_t q_end,
                                       segmla_plan** out_plan) {
  if (!geom || !layer || !prot || !out_plan) return SEGMLA_E_NULL;
  segmla_status st = check_layer(layer);
  if (st != SEGMLA_OK) return st;
  int64_t T64 = 0;
  st = check_geometry(geom, pages, n_pool, &T64);
  if (st != SEGMLA_OK) return st;
  const int32_t T = (int32_t)T64;
  if (q_end == -1) q_end = T;
  if (q_begin < 0 || q_end <= q_begin || q_end > T) return SEGMLA_E_SHAPE;
  if (prot->edge_rows < 0 || prot->tail_rows < 0 || prot->budget_permille < 0 ||
      prot->budget_permille > 1000 || prot->n_dirty < 0)
    return SEGMLA_E_PROTECT;
  if (prot->n_dirty > 0 && !prot->dirty_rows) return SEGMLA_E_NULL;
  for (int i = 0; i < prot->n_dirty; ++i)
    if (prot->dirty_rows[i] < 0 || prot->dirty_rows[i] >= T) return SEGMLA_E_PROTECT;

  segmla_plan* p = new (std::nothrow) segmla_plan();
  if (!p) return SEGMLA_E_UNSUPPORTED;
  p->n_seg = geom->n_seg;
  p->T = T;
  p->q0 = (int32_t)q_begin;
  p->q1 = (int32_t)q_end;
  p->n_pool = n_pool;
  p->segs.resize(geom->n_seg);
  for (int i = 0; i < geom->n_seg; ++i) {
    SegDesc& d = p->segs[i];
    d.pool_row = pages ? -1 : geom->pool_row[i];
    d.offset = (int32_t)geom->offset[i];
    d.len = geom->len[i];
    d.kind = geom->kind[i];
    d.relocated = (geom->kind[i] == SEGMLA_SEG_DOC && geom->offset[i] != 0) ? 1 : 0;
    d.rot = geom->kind[i] == SEGMLA_SEG_DOC ? d.offset : 0;
    d.frame = i;
  }
  // runs: an unpaged segment is one run; a paged one is cut at every page boundary where the
  // next page does not continue the pool rows
  if (!pages) {
    p->runs = p->segs;
  } else {
    const int64_t pr = pages->page_rows;
    for (int i = 0; i < geom->n_seg; ++i) {
      const SegDesc& d = p->segs[i];
      for (int64_t k = 0; k * pr < d.len; ++k) {
        const int64_t prow = pages->page_table[pages->page_start[i] + k] * pr;
        const int32_t rows = (int32_t)std::min<int64_t>(pr, d.len - k * pr);
        if (k > 0 && p->runs.back().pool_row + p->runs.back().len == prow) {
          p->runs.back().len += rows;
          continue;
        }
        SegDesc r = d;
        r.pool_row = prow;
        r.offset = d.offset + (int32_t)(k * pr);
        r.len = rows;
        p->runs.push_back(r);
      }
    }
  }
  p->n_run = (int32_t)p->runs.size();
  p->H = layer->n_heads;
  for (int h = 0; h < p->H; ++h) {
    const int role = layer->head_is_global[h];
    (role == 1 ? p->ghead : role == 2 ? p->whead : p->lhead).push_back(h);
    if (role != 2) p->fhead.push_back(h);
    if (role != 0) p->rowhead.push_back(h);
  }
  p->HG = (int32_t)p->ghead.size();
  p->HL = (int32_t)p->lhead.size();
  p->HW = (int32_t)p->whead.size();
  p->n_sink = layer->n_sink;
  p->window = layer->window;
  p->z_e4m3 = layer->z_e4m3;
  if (layer->group_heads >= 2) {
    p->G = layer->group_heads;
    p->n_groups = p->H / p->G;
    p->grp_gstart.push_back(0);
    for (int g = 0; g < p->n_groups; ++g) {
      for (int h = g * p->G; h < (g + 1) * p->G; ++h)
        if (layer->head_is_global[h] != 0) p->grp_ghead.push_back(h);
      p->grp_gstart.push_back((int32_t)p->grp_ghead.size());
    }
  }
  p->d_nope = layer->d_nope;
  p->d_rope = layer->d_rope;
  p->d_qk = layer->d_nope + layer->d_rope;
  p->d_v = layer->v_has_rope ? p->d_qk : p->d_nope;
  if (p->d_v < 1) { delete p; return SEGMLA_E_SHAPE; }
  p->d_state = layer->d_state;
  p->v_has_rope = layer->v_has_rope;
  p->kv_dtype = layer->kv_dtype;
  p->io_dtype = layer->io_dtype;
  p->rope_base = layer->rope_base;
  p->sigma = layer->softmax_scale;
  p->edge_rows = prot->edge_rows;
  p->tail_rows = prot->tail_rows;
  p->budget_permille = prot->budget_permille;
  p->dirty.assign(prot->dirty_rows, prot->dirty_rows + prot->n_dirty);
  std::sort(p->dirty.begin(), p->dirty.end());
  p->dirty.erase(std::unique(p->dirty.begin(), p->dirty.end()), p->dirty.end());

  // |F|, |C| and |F & C| on the host (the protected-row rule, counted row by row).
  {
    std::vector<uint8_t> forced(T, 0);
    const int b = p->edge_rows;
    for (const SegDesc& d : p->segs) {
      if (d.kind == SEGMLA_SEG_NEW) std::fill(forced.begin() + d.offset, forced.begin() + d.offset + d.len, 1);
      if (d.relocated) {
        int e = std::min(b, d.len);
        std::fill(forced.begin() + d.offset, forced.begin() + d.offset + e, 1);
        std::fill(forced.begin() + d.offset + std::max(0, d.len - b), forced.begin() + d.offset + d.len, 1);
      }
    }
    for (int32_t r : p->dirty) forced[r] = 1;
    for (int64_t t = std::max<int64_t>(0, (int64_t)T - p->tail_rows); t < T; ++t) forced[t] = 1;
    int64_t nf = 0, nc = 0, nfc = 0;
    p->cum_forced.assign((size_t)T + 1, 0);
    p->cum_free_cand.assign((size_t)T + 1, 0);
    for (const SegDesc& d : p->segs) {
      bool cand = d.kind != SEGMLA_SEG_NEW;
      for (int j = 0; j < d.len; ++j) {
        const int64_t t = d.offset + j;
        bool f = forced[t] != 0;
        nf += f;
        nc += cand;
        nfc += (f && cand);
        p->cum_forced[t + 1] = p->cum_forced[t] + (f ? 1 : 0);
        p->cum_free_cand[t + 1] = p->cum_free_cand[t] + ((!f && cand) ? 1 : 0);
      }
    }
    p->n_forced = nf;
    p->n_cand = nc;
    p->K = ((int64_t)p->budget_permille * nc + 999) / 1000;
    p->need = std::max<int64_t>(0, p->K - nfc);
    p->nA = nf + p->need;
  }
  p->n_blk = (T + 1023) / 1024;
  p->n_cu = device_cus();
  p->split_req = layer->split_keys;

  // Workspace layout: the request's part (geometry, tables, row maps, A) first, then the
  // window's part (size_window), so that another window of the same request reuses the first.
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + std::max<size_t>(bytes, 1)); return at; };
  const size_t half = (size_t)p->d_rope / 2;
  // the host-built tables first, contiguous: one upload of a host image per build
  p->o_seg = take(sizeof(SegDesc) * p->n_run);
  p->o_lseg = take(sizeof(SegDesc) * p->n_seg);
  p->o_dirty = take(sizeof(int32_t) * p->dirty.size());
  p->o_ghead = take(sizeof(int32_t) * p->ghead.size());
  p->o_lhead = take(sizeof(int32_t) * p->lhead.size());
  p->o_whead = take(sizeof(int32_t) * p->whead.size());
  p->o_fhead = take(sizeof(int32_t) * p->fhead.size());
  p->o_rowhead = take(sizeof(int32_t) * p->rowhead.size());
  p->o_grp = take(sizeof(int32_t) * (p->grp_gstart.size() + p->grp_ghead.size()));
  p->upload.assign(o, 0);
  auto put = [&](size_t off, const void* src, size_t bytes) {
    if (bytes) std::memcpy(p->upload.data() + off, src, bytes);
  };
  put(p->o_seg, p->runs.data(), sizeof(SegDesc) * p->runs.size());
  put(p->o_lseg, p->segs.data(), sizeof(SegDesc) * p->segs.size());
  put(p->o_dirty, p->dirty.data(), sizeof(int32_t) * p->dirty.size());
  put(p->o_ghead, p->ghead.data(), sizeof(int32_t) * p->ghead.size());
  put(p->o_lhead, p->lhead.data(), sizeof(int32_t) * p->lhead.size());
  put(p->o_whead, p->whead.data(), sizeof(int32_t) * p->whead.size());
  put(p->o_fhead, p->fhead.data(), sizeof(int32_t) * p->fhead.size());
  put(p->o_rowhead, p->rowhead.data(), sizeof(int32_t) * p->rowhead.size());
  put(p->o_grp, p->grp_gstart.data(), sizeof(int32_t) * p->grp_gstart.size());
  put(p->o_grp + sizeof(int32_t) * p->grp_gstart.size(), p->grp_ghead.data(),
      sizeof(int32_t) * p->grp_ghead.size());
  // then what the build computes on the device
  p->o_segcs = take(sizeof(float2) * half * p->n_run);
  p->o_stepcs = take(sizeof(float2) * half * p->n_run);
  p->o_seg_of_row = take(sizeof(int32_t) * (size_t)T);
  p->o_flags = take((size_t)T);
  p->o_alist = take(sizeof(int32_t) * (size_t)p->nA);
  p->o_nalist = take(sizeof(int32_t) * (size_t)(T - p->nA));
  p->o_blk_count = take(sizeof(int32_t) * p->n_blk);
  p->o_blk_sum = take(sizeof(uint64_t) * p->n_blk);
  p->o_sum_a = take(sizeof(uint64_t));
  p->o_sel = take(sizeof(uint32_t) * 4);
  p->o_rng = take(sizeof(int32_t) * 4);
  p->o_tail = o;
  const segmla_status st2 = size_window(p, p->q0, p->q1, ~size_t(0));
  if (st2 != SEGMLA_OK) { delete p; return st2; }
  *out_plan = p;
  return SEGMLA_OK;
}

segmla_status segmla_plan_workspace_bytes(const segmla_plan* p, size_t* bytes) {
  if (!p || !bytes) return SEGMLA_E_NULL;
  *bytes = p->ws_bytes;
  return SEGMLA_OK;
}

segmla_status segmla_plan_rows(const segmla_plan* p, int64_t* n_rows, int64_t* n_protected) {
  if (!p || !n_rows || !n_protected) return SEGMLA_E_NULL;
  *n_rows = p->T;
  *n_protected = p->nA;
  return SEGMLA_OK;
}

segmla_status segmla_plan_get_info(const segmla_plan* p, segmla_plan_info* info) {
  if (!p || !info) return SEGMLA_E_NULL;
  info->T = p->T;
  info->q_begin = p->q0;
  info->q_end = p->q1;
  info->n_pool = p->n_pool;
  info->n_protected = p->nA;
  info->workspace_bytes = (int64_t)p->ws_bytes;
  info->n_heads = p->H;
  info->n_global = p->HG;
  info->n_local = p->HL;
  info->n_window = p->HW;
  info->d_nope = p->d_nope;
  info->d_rope = p->d_rope;
  info->d_v = p->d_v;
  info->d_state = p->d_state;
  info->z_slots = p->G >= 2 ? p->n_groups : p->H;
  info->zc_slots = p->G >= 2 ? p->n_groups : p->HL;
  info->kv_dtype = p->kv_dtype;
  info->io_dtype = p->io_dtype;
  info->n_split = p->n_split;
  info->z_e4m3 = p->z_e4m3;
  return SEGMLA_OK;
}


segmla_status segmla_plan_build(segmla_plan* p, void* workspace, size_t workspace_bytes,
                                const uint32_t* indexer_score, void* stream) {
  if (!p || !workspace) return p ? SEGMLA_E_WORKSPACE : SEGMLA_E_NULL;
  if (workspace_bytes < p->ws_bytes || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return SEGMLA_E_WORKSPACE;
  if (p->need > 0 && !indexer_score) return SEGMLA_E_PROTECT;
  const segmla_status st = build_impl(p, (char*)workspace, indexer_score, (hipStream_t)stream);
  if (st == SEGMLA_OK) p->ws_capacity = workspace_bytes;
  return st;
}

segmla_status segmla_forward(const segmla_plan* p, const segmla_tensors* t, void* stream) {
  if (!p || !t) return SEGMLA_E_NULL;
  if (!p->built) return SEGMLA_E_STATE;
  const segmla_status st = check_tensors(p, t);
  if (st != SEGMLA_OK) return st;
  return forward_impl(p, t, (hipStream_t)stream);
}

segmla_status segmla_forward_noalloc(segmla_plan* p, const uint32_t* indexer_score,
                                     const segmla_tensors* t, void* stream) {
  if (!p || !t) return SEGMLA_E_NULL;
  if (p->ws_bytes > (size_t)SEGMLA_NOALLOC_MAX_BYTES) return SEGMLA_E_WORKSPACE;
  if (p->need > 0 && !indexer_score) return SEGMLA_E_PROTECT;
  segmla_status st = check_tensors(p, t);
  if (st != SEGMLA_OK) return st;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return SEGMLA_E_HIP;
  // build and run into the shared array; the plan's own workspace state (if it was built with
  // segmla_plan_build) and its profiling are left as they were
  char* const own_ws = p->ws;
  const size_t own_capacity = p->ws_capacity;
  const bool own_built = p->built, own_prof = p->prof;
  p->prof = false;
  const hipStream_t s = (hipStream_t)stream;
  st = build_impl(p, (char*)ws, indexer_score, s);
  if (st == SEGMLA_OK) st = forward_impl(p, t, s);
  p->ws = own_ws;
  p->ws_capacity = own_capacity;
  p->built = own_built;
  p->prof = own_prof;
  return st;
}

segmla_status segmla_plan_set_window(segmla_plan* p, int64_t q_begin, int64_t q_end, void* stream) {
  if (!p) return SEGMLA_E_NULL;
  if (!p->built) return SEGMLA_E_STATE;
  if (q_end == -1) q_end = p->T;
  if (q_begin < 0 || q_end <= q_begin || q_end > p->T) return SEGMLA_E_SHAPE;
  const segmla_status st = size_window(p, (int32_t)q_begin, (int32_t)q_end, p->ws_capacity);
  if (st != SEGMLA_OK) return st;  // the plan is unchanged
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if ((int64_t)(p->q1 - p->q0) * (p->d_rope / 2) <= kWindowSmallPairs &&
      p->nF + p->nG <= kWindowSmallTiles) {  // the next decode row: one launch
    e = launch_window_small(p->at<int32_t>(p->o_alist), (int)p->nA, p->d_rope, p->rope_base,
                            p->at<float2>(p->o_rowcs), tile_map(p), p->at<uint64_t>(p->o_sum_a),
                            p->at<int32_t>(p->o_work), s);
  } else {
    e = launch_window(p->at<int32_t>(p->o_alist), (int)p->nA, p->q0, p->q1, p->d_rope,
                      p->rope_base, p->at<float2>(p->o_rowcs), p->at<int32_t>(p->o_rng),
                      p->at<uint64_t>(p->o_sum_a), s);
    if (e == hipSuccess && p->nF + p->nG > 0) e = launch_worklist(tile_map(p), p->at<int32_t>(p->o_work), s);
  }
  if (e != hipSuccess) {
    p->built = false;
    return SEGMLA_E_HIP;
  }
  return SEGMLA_OK;
}

segmla_status segmla_profile_enable(segmla_plan* p, int32_t enable) {
  if (!p) return SEGMLA_E_NULL;
  if (enable) {
    for (hipEvent_t& ev : p->ev)
      if (!ev && hipEventCreate(&ev) != hipSuccess) return SEGMLA_E_HIP;
    p->fwd_pending = p->build_pending = false;
    for (double& x : p->prof_ms) x = 0;
    p->prof_fwd = p->prof_build = 0;
    p->prof = true;
  } else {
    if (flush_profile(p) != hipSuccess) return SEGMLA_E_HIP;
    p->prof = false;
  }
  return SEGMLA_OK;
}

segmla_status segmla_profile_read(segmla_plan* p, double ms[4], int64_t* n_forward,
                                  int64_t* n_build) {
  if (!p || !ms) return SEGMLA_E_NULL;
  if (flush_profile(p) != hipSuccess) return SEGMLA_E_HIP;
  for (int i = 0; i < 4; ++i) ms[i] = p->prof_ms[i];
  if (n_forward) *n_forward = p->prof_fwd;
  if (n_build) *n_build = p->prof_build;
  return SEGMLA_OK;
}

segmla_status segmla_copy_protected(const segmla_plan* p, int32_t* host_rows, int64_t cap,
                                    void* stream) {
  if (!p || !host_rows) return SEGMLA_E_NULL;
  if (!p->built) return SEGMLA_E_STATE;
  if (cap < p->nA) return SEGMLA_E_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (p->nA > 0 && hipMemcpyAsync(host_rows, p->ws + p->o_alist, sizeof(int32_t) * p->nA,
                                  hipMemcpyDeviceToHost, s) != hipSuccess)
    return SEGMLA_E_HIP;
  return hipStreamSynchronize(s) == hipSuccess ? SEGMLA_OK : SEGMLA_E_HIP;
}

segmla_status segmla_copy_geometry(const segmla_plan* p, int32_t* seg_of_row, int64_t* pool_of_row,
                                   int64_t cap, void* stream) {
  if (!p) return SEGMLA_E_NULL;
  if (!p->built) return SEGMLA_E_STATE;
  if (cap < p->T) return SEGMLA_E_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> tmp;
  int32_t* dst = seg_of_row;
  if (!dst && pool_of_row) { tmp.resize(p->T); dst = tmp.data(); }
  if (dst && hipMemcpyAsync(dst, p->ws + p->o_seg_of_row, sizeof(int32_t) * p->T,
                            hipMemcpyDeviceToHost, s) != hipSuccess)
    return SEGMLA_E_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SEGMLA_E_HIP;
  if (!dst) return SEGMLA_OK;
  for (int32_t r = 0; r < p->T; ++r) {  // the device map holds runs
    const int32_t i = dst[r];
    const bool ok = i >= 0 && i < p->n_run;
    if (pool_of_row) pool_of_row[r] = ok ? p->runs[i].pool_row + (r - p->runs[i].offset) : -1;
    dst[r] = ok ? p->runs[i].frame : -1;
  }
  return SEGMLA_OK;
}

segmla_status segmla_plan_pairs(const segmla_plan* p, double out[3], void* stream) {
  if (!p || !out) return SEGMLA_E_NULL;
  if (!p->built) return SEGMLA_E_STATE;
  uint64_t sum_a = 0;
  hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&sum_a, p->ws + p->o_sum_a, sizeof(uint64_t), hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return SEGMLA_E_HIP;
  const double q0 = (double)p->q0, q1 = (double)p->q1;  // window rows t see t + 1 keys
  out[0] = (double)p->HG * (q1 * (q1 + 1.0) - q0 * (q0 + 1.0)) / 2.0;
  out[1] = (double)p->HL * (double)sum_a;
  // a sink + window head sees t + 1 keys while t <= c = window + n_sink, then c + 1
  const double c = (double)p->window + (double)p->n_sink;
  const double t_full = std::min(q1, std::max(q0, c + 1.0));  // rows [q0, t_full) see t + 1
  out[2] = (double)p->HW * ((t_full * (t_full + 1.0) - q0 * (q0 + 1.0)) / 2.0 + (q1 - t_full) * (c + 1.0));
  return SEGMLA_OK;
}

segmla_status segmla_ledger(int32_t f_front, int32_t r, int32_t f_back, int32_t h,
                            int32_t h_local, int64_t T, int64_t n_protected, double global_pairs,
                            double local_pairs, double out[3]) {
  if (!out) return SEGMLA_E_NULL;
  if (f_front < 0 || r < 0 || f_back < 0 || f_front + r + f_back < 1 || h < 1 || h_local < 0 ||
      h_local > h || T < 1 || n_protected < 0 || n_protected > T)
    return SEGMLA_E_SHAPE;
  out[0] = ((double)r / (double)(f_front + r + f_back)) * ((double)h_local / (double)h);
  out[1] = (double)h_local * (double)(T - n_protected) / ((double)h * (double)T);
  const double dense = (double)h * (double)T * ((double)T + 1.0) / 2.0;
  out[2] = local_pairs < 0 ? NAN : 1.0 - (global_pairs + local_pairs) / dense;
  return SEGMLA_OK;
}

segmla_status segmla_lse_merge(const float* partial_o, const float* partial_ml, int32_t n_split,
                               int64_t n_vec, int32_t d, void* out, int32_t out_dtype, float* lse,
                               void* stream) {
  if (!partial_o || !partial_ml || !out) return SEGMLA_E_NULL;
  if (n_split < 1 || n_vec < 0 || d < 1 || d > 4096) return SEGMLA_E_SHAPE;
  if (out_dtype != SEGMLA_F32 && out_dtype != SEGMLA_BF16) return SEGMLA_E_DTYPE;
  if (n_vec == 0) return SEGMLA_OK;
  hipError_t e = launch_lse_merge(partial_o, partial_ml, n_split, n_vec, d, out, out_dtype, lse,
                                  (hipStream_t)stream);
  return e == hipSuccess ? SEGMLA_OK : SEGMLA_E_HIP;
}

// ----------------------------------------------------------- compressed-history layers
struct segmla_dual {
  const segmla_plan* plan = nullptr;
  int32_t ratio = 1, window = 0, top_k = 0;
  int64_t n_cpool = 0, n_entries = 0;
  std::vector<char> upload;  // CSeg per segment, then CEnt per entry (the device tables)
  size_t o_cseg = 0, o_cent = 0, ws_bytes = 0;
  bool built = false;
  char* ws = nullptr;
};

segmla_status segmla_dual_create(const segmla_plan* p, const segmla_dual_pool* dp,
                                 segmla_dual** out) {
  if (!p || !dp || !out || !dp->cpool_row) return SEGMLA_E_NULL;
  if (p->kv_dtype != SEGMLA_BF16 || p->io_dtype != SEGMLA_BF16 || p->d_nope != 512 || p->d_rope != 64)
    return SEGMLA_E_UNSUPPORTED;
  if (dp->ratio < 1 || dp->window < 0 || dp->top_k < 0 || dp->n_cpool < 0 || dp->n_cpool > INT32_MAX)
    return SEGMLA_E_SHAPE;
  const int32_t n = p->n_seg;
  std::vector<CSeg> cs(n);
  int64_t base = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t cnt = p->segs[i].len / dp->ratio;
    const int64_t r0 = dp->cpool_row[i];
    if (r0 < 0 || r0 + cnt > dp->n_cpool) return SEGMLA_E_GEOMETRY;
    cs[i].base = (int32_t)base;
    cs[i].count = (int32_t)cnt;
    cs[i].offset = p->segs[i].offset;
    cs[i].pad = 0;
    base += cnt;
  }
  // a run of each segment: its RoPE frame (every run of a segment has the same phase shift)
  std::vector<int32_t> first_run(n, -1);
  for (int32_t r = p->n_run - 1; r >= 0; --r) first_run[p->runs[r].frame] = r;
  std::vector<CEnt> ce((size_t)base);
  for (int32_t i = 0; i < n; ++i) {
    const CEnt e = {first_run[i], cs[i].base, cs[i].base + cs[i].count,
                    (int32_t)(dp->cpool_row[i] - cs[i].base)};
    for (int32_t j = 0; j < cs[i].count; ++j) ce[(size_t)cs[i].base + j] = e;
  }
  segmla_dual* d = new segmla_dual;
  d->plan = p;
  d->ratio = dp->ratio;
  d->window = dp->window;
  d->top_k = dp->top_k;
  d->n_cpool = dp->n_cpool;
  d->n_entries = base;
  d->o_cseg = 0;
  d->o_cent = align256(sizeof(CSeg) * n);
  d->ws_bytes = align256(d->o_cent + sizeof(CEnt) * ce.size());
  d->upload.assign(d->ws_bytes, 0);
  std::memcpy(d->upload.data() + d->o_cseg, cs.data(), sizeof(CSeg) * n);
  if (!ce.empty()) std::memcpy(d->upload.data() + d->o_cent, ce.data(), sizeof(CEnt) * ce.size());
  *out = d;
  return SEGMLA_OK;
}

segmla_status segmla_dual_sizes(const segmla_dual* d, size_t* workspace_bytes, int64_t* n_entries) {
  if (!d) return SEGMLA_E_NULL;
  if (workspace_bytes) *workspace_bytes = d->ws_bytes;
  if (n_entries) *n_entries = d->n_entries;
  return SEGMLA_OK;
}

segmla_status segmla_dual_build(segmla_dual* d, void* workspace, size_t bytes, void* stream) {
  if (!d || !workspace) return SEGMLA_E_NULL;
  if (bytes < d->ws_bytes || (uintptr_t)workspace % 256 != 0) return SEGMLA_E_WORKSPACE;
  d->built = false;
  if (hipMemcpyAsync(workspace, d->upload.data(), d->ws_bytes, hipMemcpyHostToDevice,
                     (hipStream_t)stream) != hipSuccess)
    return SEGMLA_E_HIP;
  d->ws = (char*)workspace;
  d->built = true;
  return SEGMLA_OK;
}

segmla_status segmla_dual_forward(const segmla_dual* d, const segmla_dual_tensors* t, void* stream) {
  if (!d || !t) return SEGMLA_E_NULL;
  if (!t->q || !t->kv || !t->ckv || !t->out) return SEGMLA_E_NULL;
  if (d->top_k > 0 && (!t->cidx || !t->clen)) return SEGMLA_E_NULL;
  const segmla_plan* p = d->plan;
  if (!p->built || !d->built) return SEGMLA_E_STATE;
  for (const void* ptr : {t->q, t->kv, t->ckv, (const void*)t->out, (const void*)t->lse})
    if ((uintptr_t)ptr % 16 != 0) return SEGMLA_E_SHAPE;
  if ((uintptr_t)t->cidx % 4 != 0 || (uintptr_t)t->clen % 4 != 0) return SEGMLA_E_SHAPE;
  AttnArgs a;
  a.q = t->q;
  a.kv = t->kv;
  a.kv_scale = nullptr;
  a.kv_rope = nullptr;
  a.out = t->out;
  a.lse = t->lse;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.seg = p->at<SegDesc>(p->o_seg);
  a.seg_of_row = p->at<int32_t>(p->o_seg_of_row);
  a.segcs = p->at<float2>(p->o_segcs);
  a.stepcs = p->at<float2>(p->o_stepcs);
  a.work = nullptr;
  a.map = tile_map(p);
  a.n_seg = p->n_run;
  a.T = p->T;
  a.d_nope = p->d_nope;
  a.d_rope = p->d_rope;
  a.d_v = p->d_v;
  a.q0 = p->q0;
  a.n_split = 1;
  a.split_keys = 0;
  a.sigma = p->sigma;
  a.n_sink = 0;
  a.win = 0;
  a.z_cached = nullptr;
  a.z = nullptr;
  a.lhead = nullptr;
  a.HL = 0;
  a.z_chunks = 0;
  a.rc_rows = 0;
  a.ckv = t->ckv;
  a.cidx = d->top_k > 0 ? t->cidx : nullptr;
  a.clen = d->top_k > 0 ? t->clen : nullptr;
  a.cent = reinterpret_cast<const CEnt*>(d->ws + d->o_cent);
  a.cseg = reinterpret_cast<const CSeg*>(d->ws + d->o_cseg);
  a.ratio = d->ratio;
  a.topk = d->top_k;
  a.n_hb = (p->H + 63) / 64;
  a.cwin = d->window;
  const hipError_t e = launch_attn_dual(a, p->v_has_rope, d->top_k > 0, (hipStream_t)stream);
  return e == hipSuccess ? SEGMLA_OK : SEGMLA_E_HIP;
}

void segmla_dual_destroy(segmla_dual* d) { delete d; }

void segmla_plan_destroy(segmla_plan* p) {
  if (!p) return;
  for (hipEvent_t ev : p->ev)
    if (ev) (void)hipEventDestroy(ev);
  delete p;
}

}  // extern "C"
