// Internal declarations shared by the libsegmla HIP sources (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace segmla {

// Device segment descriptor (32 bytes). The attention and the row map walk physical runs:
// stretches of one segment's rows that are contiguous in the latent pool (the whole segment
// for an unpaged pool). A run carries its segment's phase shift, kind and relocation flag,
// and the segment's index as `frame`; the protected-row marking reads the segments.
struct SegDesc {
  int64_t pool_row;  // first latent-pool row
  int32_t offset;    // Delta_i: request position of the segment's first row
  int32_t len;       // n_i
  int32_t rot;       // phase shift the stored latent needs: Delta_i for documents (stored at
                     // canonical 0..n-1), 0 for prefix/new rows (stored at request positions)
  int32_t kind;      // segmla_seg_kind
  int32_t relocated; // document at a nonzero offset
  int32_t frame;     // index of the segment (a run's RoPE frame is its segment's)
};

// Row flag bits written by the protected-row builder.
enum : uint8_t { kFlagForced = 1, kFlagCand = 2, kFlagIndexer = 4 };

// Work decomposition of the attention: (row, head) query vectors ("qvecs") come from three
// streams. Stream F: rows of A with every full-context head (Global and Local), flattened
// (a * HF + f). Stream G: rows outside A with the Global heads only (a * HG + g). Stream W:
// every window row with the sink + window heads (a * HW + w). Each stream is cut into tiles
// of kTileQ consecutive qvecs; tiles [0, nF) are F tiles, [nF, nF + nG) G tiles and
// [nF + nG, nF + nG + nW) W tiles.
constexpr int kTileQ = 128;

// The computed rows are a window [q0, q1) of the request (all of it for a whole prefill).
// Its rows of A are alist[rng[0], rng[1]) and its other rows nalist[rng[2], rng[3]): both lists
// cover the whole request in ascending order, so a window is a contiguous range of each. The
// range ends depend on which rows the Indexer picked, so they live in device memory (written
// by the plan build); nF and nG are sized for the largest share the window can have, and the
// tiles past the actual end are empty.
struct TileMap {
  const int32_t* alist;   // [nA] rows of A, ascending
  const int32_t* nalist;  // [T - nA] rows outside A, ascending
  const int32_t* fhead;   // [HF] full-context head ids (Global and Local); null: heads 0..H-1
  const int32_t* ghead;   // [HG] Global head ids
  const int32_t* whead;   // [HW] sink + window head ids
  const int32_t* rng;     // device {a_lo, a_hi, na_lo, na_hi}
  int32_t H, HF, HG, HW, nF, nG, nW;
  int32_t q0, nq;         // window rows [q0, q0 + nq) (stream W walks them in order)
};

__device__ __forceinline__ bool tile_qvec(const TileMap& m, int tile, int qi, int& t, int& h) {
  if (tile < m.nF) {
    const int a0 = m.rng[0], na = m.rng[1] - a0;
    int64_t f = (int64_t)tile * kTileQ + qi;
    if (f >= (int64_t)na * m.HF) return false;
    int a = (int)(f / m.HF);
    h = (int)(f - (int64_t)a * m.HF);
    if (m.fhead) h = m.fhead[h];
    t = m.alist[a0 + a];
  } else if (tile < m.nF + m.nG) {
    const int b0 = m.rng[2], nb = m.rng[3] - b0;
    int64_t f = (int64_t)(tile - m.nF) * kTileQ + qi;
    if (f >= (int64_t)nb * m.HG) return false;
    int a = (int)(f / m.HG);
    h = m.ghead[(int)(f - (int64_t)a * m.HG)];
    t = m.nalist[b0 + a];
  } else {
    int64_t f = (int64_t)(tile - m.nF - m.nG) * kTileQ + qi;
    if (f >= (int64_t)m.nq * m.HW) return false;
    int a = (int)(f / m.HW);
    h = m.whead[(int)(f - (int64_t)a * m.HW)];
    t = m.q0 + a;
  }
  return true;
}

// Largest request row among a tile's qvecs (lists are ascending); -1 for an empty tile.
__device__ __forceinline__ int tile_max_row(const TileMap& m, int tile) {
  if (tile < m.nF) {
    const int a0 = m.rng[0], na = m.rng[1] - a0;
    const int64_t first = (int64_t)tile * kTileQ, cap = (int64_t)na * m.HF - 1;
    if (first > cap) return -1;
    const int64_t last = first + kTileQ - 1 < cap ? first + kTileQ - 1 : cap;
    return m.alist[a0 + (int)(last / m.HF)];
  }
  if (tile < m.nF + m.nG) {
    const int b0 = m.rng[2], nb = m.rng[3] - b0;
    const int64_t first = (int64_t)(tile - m.nF) * kTileQ, cap = (int64_t)nb * m.HG - 1;
    if (first > cap) return -1;
    const int64_t last = first + kTileQ - 1 < cap ? first + kTileQ - 1 : cap;
    return m.nalist[b0 + (int)(last / m.HG)];
  }
  const int64_t first = (int64_t)(tile - m.nF - m.nG) * kTileQ, cap = (int64_t)m.nq * m.HW - 1;
  if (first > cap) return -1;
  const int64_t last = first + kTileQ - 1 < cap ? first + kTileQ - 1 : cap;
  return m.q0 + (int)(last / m.HW);
}

// Smallest request row of a W tile's qvecs (stream W walks the window rows in order).
__device__ __forceinline__ int wtile_min_row(const TileMap& m, int tile) {
  return m.q0 + (int)((int64_t)(tile - m.nF - m.nG) * kTileQ / m.HW);
}

// Index of the segment containing request row `row` (segments contiguous from 0).
__device__ __forceinline__ int seg_of(const SegDesc* seg, int n_seg, int row) {
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seg[mid].offset <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Compressed entry (16 bytes, read with one scalar load): a run of the entry's segment (its
// RoPE frame), the segment's entry ids [lo, hi), and pool row - id for the segment's entries.
struct CEnt {
  int32_t run, lo, hi, delta;
};
// Per logical segment: id of its entry 0, its entry count, and its request offset.
struct CSeg {
  int32_t base, count, offset, pad;
};

// Arguments of the attention kernels (one struct so every variant shares the launch code).
struct AttnArgs {
  const void* q;          // [q1 - q0][H][d_qk] io dtype (row t at t - q0)
  const void* kv;         // latent pool (f32 / bf16 rows, or E4M3 codes)
  const float* kv_scale;  // E4M3: [n_pool][d_nope/128]
  const void* kv_rope;    // E4M3: [n_pool][d_rope] bf16
  void* out;              // [q1 - q0][H][d_v] io dtype (unsplit)
  float* lse;             // [q1 - q0][H] or null (unsplit)
  float* part_o;          // [n_split][nTiles*kTileQ][d_v] (split); bf16 values when part_bf16
  float* part_ml;         // [n_split][nTiles*kTileQ][2] (split)
  const SegDesc* seg;
  const int32_t* seg_of_row;  // [T] segment of each request row
  const float2* segcs;    // [n_seg][d_rope/2] cos/sin(rot_i * theta_k)
  const float2* stepcs;   // [n_seg][d_rope/2] cos/sin((rot_i - rot_{i+1}) * theta_k)
  const int32_t* work;    // [nF + nG] tile ids in decreasing cost order
  TileMap map;
  int32_t n_seg, T, d_nope, d_rope, d_v;
  int32_t q0;             // first computed row: q, out and lse rows are t - q0
  int32_t n_split, split_keys;
  float sigma;            // softmax scale
  int32_t n_sink, win;    // W tiles: key p visible from row t iff p <= t and (p < n_sink or
                          // p >= t - win)
  // The replacement copy of the rows outside A, done by the full-context attention grid (each
  // workgroup copies rc_rows consecutive rows of the window's complement list before its tile):
  // z[t][lhead[l]] = z_cached[pool_row(t)][l] for the HL Local heads; rc_rows = 0: not here.
  const void* z_cached;   // [n_pool][HL][d_state] bf16
  void* z;                // [q1 - q0][H][d_state] bf16
  const int32_t* lhead;   // [HL]
  int32_t HL, z_chunks, rc_rows;  // z_chunks: 16-byte chunks per head's state vector
  // Compressed-history (dual-pool) launches: one workgroup per (window row, block of 64 heads),
  // raw keys [t - cwin, t] of kv, then entries of ckv (all available ones, or the row's list).
  const void* ckv = nullptr;             // [n_cpool][576] bf16
  const int32_t* cidx = nullptr;         // [nq][topk] entry ids (lists)
  const int32_t* clen = nullptr;         // [nq] list lengths (lists)
  const CEnt* cent = nullptr;     // [n_entries]
  const CSeg* cseg = nullptr;     // [logical segments]
  int32_t ratio = 1, topk = 0, n_hb = 1, cwin = 0;
  int32_t part_bf16 = 0;                 // split partial outputs stored as bf16 (decode kernel)
};


// Launchers (defined in the kernel sources), all on `stream`.
hipError_t launch_geometry(const SegDesc* seg, int n_seg, int T, int q0, int q1, int d_rope,
                           double base, int32_t* seg_of_row, float2* segcs, float2* stepcs,
                           float2* rowcs, hipStream_t stream);
hipError_t launch_protect(const SegDesc* lseg, const SegDesc* runs, const int32_t* seg_of_row, int T,
                          int edge_rows, int tail_rows, const int32_t* dirty, int n_dirty,
                          const uint32_t* score, int64_t need, uint8_t* flags,
                          uint32_t* sel_state, int32_t* blk_count, uint64_t* blk_sum,
                          int n_blk, int32_t* alist, int32_t* nalist, int n_a, uint64_t* sum_a,
                          int q0, int q1, int32_t* rng, hipStream_t stream);
hipError_t launch_worklist(TileMap map, int32_t* work, hipStream_t stream);
// launch_window and launch_worklist in one workgroup, for windows of few rows and tiles
// (kWindowSmallPairs RoPE pairs, kWindowSmallTiles tiles at most)
constexpr int kWindowSmallPairs = 2048, kWindowSmallTiles = 2048;
hipError_t launch_window_small(const int32_t* alist, int nA, int d_rope, double base, float2* rowcs,
                               TileMap map, uint64_t* sum_a, int32_t* work, hipStream_t stream);
hipError_t launch_window(const int32_t* alist, int nA, int q0, int q1, int d_rope, double base,
                         float2* rowcs, int32_t* rng, uint64_t* sum_a, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, int kv_dtype, int v_has_rope, hipStream_t stream);
// the W tiles (sink + window heads): one workgroup per tile, outputs written directly
hipError_t launch_attn_window(const AttnArgs& a, int kv_dtype, int v_has_rope, hipStream_t stream);
// bf16 latent, tiles of at most 64 query vectors (one-row windows), split key ranges: two wave
// sets take alternate key tiles and merge at the end
hipError_t launch_attn_decode(const AttnArgs& a, int v_has_rope, hipStream_t stream);
// the same kernel over two pools (bf16): window rows x blocks of 64 heads, outputs written
// directly; lists = 1 reads per-row entry lists, 0 takes every available entry
hipError_t launch_attn_dual(const AttnArgs& a, int v_has_rope, int lists, hipStream_t stream);
hipError_t launch_merge_tiles(const AttnArgs& a, int io_dtype, hipStream_t stream);
hipError_t launch_lse_merge(const float* part_o, const float* part_ml, int n_split, int64_t n_vec,
                            int d, void* out, int out_dtype, float* lse, hipStream_t stream);

// Matrix-vector projection of small bf16 windows (decode): windows of at most kThinRows rows
// with d_v a multiple of 64, at most kThinMaxDv, and d_state a multiple of kThinCols.
constexpr int kThinRows = 8;
constexpr int kThinCols = 64;
constexpr int kThinMaxDv = 576;
__host__ __device__ inline bool thin_projection(int nq, int d_v, int d_state) {
  return nq <= kThinRows && d_v % 64 == 0 && d_v <= kThinMaxDv && d_state % kThinCols == 0;
}

struct EpiArgs {
  const void* out;        // [nq][H][d_v] merged head outputs (row t at t - q0)
  const void* w;          // [H][d_state][d_v]
  void* wt;               // W in the projection's MFMA operand order (bf16; see k_w_tile)
  const void* z_cached;   // [n_pool][HL][d_state]
  void* z;                // [nq][H][d_state] (row t at t - q0)
  const float2* rowcs;    // [nq][d_rope/2] cos/sin(t theta_k) of window row t at t - q0
  const int32_t* alist;
  const int32_t* nalist;
  const int32_t* rng;     // device {a_lo, a_hi, na_lo, na_hi} (see TileMap)
  const int32_t* ghead;   // [HG] heads computed on every row (Global, sink + window)
  const int32_t* lhead;   // [HL] Local heads
  const int32_t* seg_of_row;
  const SegDesc* seg;
  // grouped state (G >= 2): group g's heads computed on every row are grp_ghead[grp_gstart[g]
  // .. grp_gstart[g + 1]); z and z_cached hold n_groups slots per row
  const int32_t* grp_gstart;
  const int32_t* grp_ghead;
  int32_t G, n_groups;
  float* zpart;  // grouped windows of at most 8 rows: per-head fp32 projections [nq][H][d_state]
  // window [q0, q0 + nq); nA, nNA: the largest number of its rows inside / outside A (grid
  // sizes; the actual numbers are in rng)
  int32_t q0, nq, H, HG, HL, nA, nNA, d_nope, d_rope, d_v, d_state, v_has_rope;
  int32_t thin;  // bf16: the matrix-vector projection (else operand-ordered W copy + MFMA tiles)
  int32_t restore_done;  // the attention grid already copied the rows outside A (bf16)
};
hipError_t launch_epilogue(const EpiArgs& e, int io_dtype, hipStream_t stream);
// One-row windows of the decode kernel (bf16 partials) with per-head state: the split merge
// and the thin projection in one kernel, then the replacement copy of a row outside A. Needs
// d_v a multiple of 64 (at most kThinMaxDv), d_state a multiple of 128 and at most 4096 splits.
__host__ __device__ inline bool dec_merge_project_fits(int d_v, int d_state, int n_split) {
  return d_v % 64 == 0 && d_v <= kThinMaxDv && d_state % 128 == 0 && n_split <= 4096;
}
hipError_t launch_dec_merge_project(const AttnArgs& a, const EpiArgs& e, hipStream_t stream);
// n_blocks blocks of 128 bf16 values -> OCP E4M3 codes + one fp32 scale (amax / 448) each
hipError_t launch_quant_e4m3(const __bf16* src, uint8_t* codes, float* scales, int64_t n_blocks,
                             hipStream_t stream);

}  // namespace segmla
