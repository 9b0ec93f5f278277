// Plan-building kernels: segment geometry / RoPE tables, the protected row set and the
// ordered attention work list. Integer outputs are exact; RoPE tables are computed in
// fp64 and stored as fp32.
#include "internal.h"

namespace segmla {

// ------------------------------------------------------------------------ geometry
// theta_k = base^(-2k/d_rope) in fp64 (RoPE pairs (2k, 2k+1)).
__device__ __forceinline__ double rope_theta(double base, int k, int d_rope) {
  return pow(base, -2.0 * (double)k / (double)d_rope);
}

// Per-row segment map (every request row) and the inverse-output-RoPE table
// cos/sin(t * theta_k) of the computed window's rows t in [q0, q1) (at t - q0).
__global__ void k_geom_rows(const SegDesc* __restrict__ seg, int n_seg, int T, int q0, int q1,
                            int d_rope, double base, int32_t* __restrict__ seg_of_row,
                            float2* __restrict__ rowcs) {
  const int half = d_rope / 2;
  int64_t n = (int64_t)T * half;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    int t = (int)(i / half), k = (int)(i - (int64_t)t * half);
    if (t >= q0 && t < q1) {
      double s, c;
      sincos((double)t * rope_theta(base, k, d_rope), &s, &c);
      rowcs[(int64_t)(t - q0) * half + k] = make_float2((float)c, (float)s);
    }
    if (k == 0) seg_of_row[t] = seg_of(seg, n_seg, t);
  }
}

// Per-segment query-rotation table cos/sin(rot_i * theta_k) and the frame-change table
// cos/sin((rot_i - rot_{i+1}) * theta_k) used when the accumulated output moves from
// segment i's frame to segment i+1's.
__global__ void k_geom_segs(const SegDesc* __restrict__ seg, int n_seg, int d_rope, double base,
                            float2* __restrict__ segcs, float2* __restrict__ stepcs) {
  const int half = d_rope / 2;
  int n = n_seg * half;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    int s = i / half, k = i - s * half;
    double th = rope_theta(base, k, d_rope);
    double sn, cs;
    sincos((double)seg[s].rot * th, &sn, &cs);
    segcs[i] = make_float2((float)cs, (float)sn);
    double step = (s + 1 < n_seg) ? (double)(seg[s].rot - seg[s + 1].rot) : 0.0;
    sincos(step * th, &sn, &cs);
    stepcs[i] = make_float2((float)cs, (float)sn);
  }
}

hipError_t launch_geometry(const SegDesc* seg, int n_seg, int T, int q0, int q1, int d_rope,
                           double base, int32_t* seg_of_row, float2* segcs, float2* stepcs,
                           float2* rowcs, hipStream_t stream) {
  int64_t n = (int64_t)T * (d_rope / 2);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_geom_rows, dim3(blocks), dim3(256), 0, stream, seg, n_seg, T, q0, q1,
                     d_rope, base, seg_of_row, rowcs);
  int ns = n_seg * (d_rope / 2);
  hipLaunchKernelGGL(k_geom_segs, dim3((ns + 255) / 256), dim3(256), 0, stream, seg, n_seg,
                     d_rope, base, segcs, stepcs);
  return hipGetLastError();
}

// ------------------------------------------------------------------ protected rows
// Forced set F (new rows, dirty rows, edges of relocated documents, recent tail) and the
// candidate flag (prefix and document rows). seg_of_row maps rows to runs; a run's frame is
// its segment.
__global__ void k_protect_mark(const SegDesc* __restrict__ seg, const SegDesc* __restrict__ runs,
                               const int32_t* __restrict__ seg_of_row, int T, int b, int tau,
                               const int32_t* __restrict__ dirty, int n_dirty,
                               uint8_t* __restrict__ flags) {
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
    const SegDesc d = seg[runs[seg_of_row[t]].frame];
    int j = t - d.offset;
    bool forced = d.kind == 2 || (d.relocated && (j < b || j >= d.len - b)) || t >= T - tau;
    if (!forced && n_dirty > 0) {  // dirty rows are sorted and unique
      int lo = 0, hi = n_dirty - 1;
      while (lo <= hi) {
        int mid = (lo + hi) >> 1;
        int v = dirty[mid];
        if (v == t) { forced = true; break; }
        if (v < t) lo = mid + 1; else hi = mid - 1;
      }
    }
    flags[t] = (uint8_t)((forced ? kFlagForced : 0) | (d.kind != 2 ? kFlagCand : 0));
  }
}

// Indexer fill: pick the `need` eligible rows (candidate, not forced) with the largest uint32
// score, ties to the smaller row. One workgroup: a 4-pass MSB-first radix select finds the
// need-th largest score thr; rows above thr are taken, and among rows equal to thr the
// smallest ones are taken in row order until `need` is reached.
// Each pass reads four rows per thread and iteration (one 32-bit flag word, one 16-byte score
// load) into per-wave histograms; the crossing bin is found by a parallel suffix sum over the
// 256 bins. When every row equal to thr is taken (the usual case), the final marking is a
// single sweep; otherwise an ordered pass takes the smallest rows among the equal ones.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
__device__ __forceinline__ bool sel_eligible(uint32_t f) {
  return (f & (kFlagCand | kFlagForced)) == kFlagCand;
}
__global__ __launch_bounds__(kSelThreads) void k_protect_select(uint8_t* __restrict__ flags,
                                                                const uint32_t* __restrict__ score,
                                                                int T, uint32_t need) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t wtot[4];
  __shared__ uint32_t s_prefix, s_mask, s_remaining, s_eq;
  __shared__ uint32_t wave_cnt[kSelWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { s_prefix = 0; s_mask = 0; s_remaining = need; s_eq = 0; }
  // vector path over rows [0, T4) when both arrays allow 4-row loads; scalar tail
  const bool vec = ((uintptr_t)score & 15) == 0 && ((uintptr_t)flags & 3) == 0;
  const int T4 = vec ? (T & ~3) : 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    uint32_t* const h = hist[wave];
    auto count = [&](uint32_t f, uint32_t sc) {
      if (sel_eligible(f) && (sc & mask) == prefix) atomicAdd(&h[(sc >> shift) & 255u], 1u);
    };
    for (int t = 4 * tid; t < T4; t += 4 * kSelThreads) {
      const uint32_t f4 = *(const uint32_t*)(flags + t);
      const uint4 s4 = *(const uint4*)(score + t);
      count(f4 & 255u, s4.x);
      count((f4 >> 8) & 255u, s4.y);
      count((f4 >> 16) & 255u, s4.z);
      count(f4 >> 24, s4.w);
    }
    for (int t = T4 + tid; t < T; t += kSelThreads) count(flags[t], score[t]);
    __syncthreads();
    // thread b < 256 owns bin b: its count, and the suffix sums incl(b) = sum over bins >= b
    uint32_t c = 0, suf = 0;
    if (tid < 256) {
      for (int w = 0; w < kSelWaves; ++w) c += hist[w][tid];
      suf = c;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_down(suf, o);
        if (lane + o < 64) suf += v;
      }
      if (lane == 0) wtot[wave] = suf;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t incl = suf;
      for (int w = wave + 1; w < 4; ++w) incl += wtot[w];
      const uint32_t excl = incl - c, rem = s_remaining;
      // the highest bin whose inclusive suffix reaches rem; if even bin 0 does not (fewer
      // eligible rows than rem), bin 0 with everything counted
      const bool cross = incl >= rem && excl < rem;
      const bool short_all = tid == 0 && incl < rem;
      if (cross || short_all) {
        s_prefix = prefix | ((uint32_t)tid << shift);
        s_mask = mask | (255u << shift);
        s_remaining = rem - (cross ? excl : incl);
        s_eq = c;  // after the last pass: eligible rows whose score equals thr
      }
    }
    __syncthreads();
  }
  const uint32_t thr = s_prefix;
  const uint32_t take_eq = s_remaining;  // rows with score == thr to take, smallest rows first
  if (take_eq >= s_eq) {  // every eligible row with score >= thr is taken
    for (int t = 4 * tid; t < T4; t += 4 * kSelThreads) {
      const uint32_t f4 = *(const uint32_t*)(flags + t);
      const uint4 s4 = *(const uint4*)(score + t);
      const uint32_t sv[4] = {s4.x, s4.y, s4.z, s4.w};
      uint32_t add = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t f = (f4 >> (8 * k)) & 255u;
        if (sel_eligible(f) && sv[k] >= thr) add |= (uint32_t)kFlagIndexer << (8 * k);
      }
      if (add) *(uint32_t*)(flags + t) = f4 | add;
    }
    for (int t = T4 + tid; t < T; t += kSelThreads)
      if (sel_eligible(flags[t]) && score[t] >= thr) flags[t] |= kFlagIndexer;
    return;
  }
  uint32_t taken = 0;  // uniform across the workgroup
  for (int base = 0; base < T; base += kSelThreads) {
    int t = base + tid;
    bool elig = false, eq = false;
    uint32_t sc = 0;
    if (t < T) {
      elig = sel_eligible(flags[t]);
      sc = score[t];
      eq = elig && sc == thr;
    }
    uint64_t bal = __ballot(eq);
    uint32_t before_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_cnt[wave] = __popcll(bal);
    __syncthreads();
    uint32_t before = taken + before_in_wave;
    uint32_t blk_total = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      if (w < wave) before += wave_cnt[w];
      blk_total += wave_cnt[w];
    }
    if (elig && (sc > thr || (eq && before < take_eq))) flags[t] |= kFlagIndexer;
    taken += blk_total;
    __syncthreads();
  }
}

// Compaction of A (forced or Indexer rows) and of its complement, both ascending.
constexpr int kScanBlock = 1024;

__device__ __forceinline__ bool in_a(uint8_t f) { return (f & (kFlagForced | kFlagIndexer)) != 0; }

// Per block of rows: how many are in A, and the sum of t + 1 over its rows of A inside the
// computed window [q0, q1) (the Local heads' key count there).
__global__ __launch_bounds__(kScanBlock) void k_count_a(const uint8_t* __restrict__ flags, int T,
                                                        int q0, int q1,
                                                        int32_t* __restrict__ blk_count,
                                                        uint64_t* __restrict__ blk_sum) {
  __shared__ uint32_t c[kScanBlock / 64];
  __shared__ uint64_t sm[kScanBlock / 64];
  int t = blockIdx.x * kScanBlock + threadIdx.x;
  bool a = t < T && in_a(flags[t]);
  uint64_t v = (a && t >= q0 && t < q1) ? (uint64_t)t + 1 : 0;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  uint64_t bal = __ballot(a);
  if ((threadIdx.x & 63) == 0) { c[threadIdx.x >> 6] = __popcll(bal); sm[threadIdx.x >> 6] = v; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tot = 0;
    uint64_t s = 0;
    for (int w = 0; w < kScanBlock / 64; ++w) { tot += c[w]; s += sm[w]; }
    blk_count[blockIdx.x] = (int32_t)tot;
    blk_sum[blockIdx.x] = s;
  }
}

// Exclusive scan of the per-block counts (in place) and the total of the window sums.
__global__ __launch_bounds__(1024) void k_scan_counts(int32_t* __restrict__ blk_count,
                                                      const uint64_t* __restrict__ blk_sum,
                                                      int n_blk, uint64_t* __restrict__ sum_a) {
  __shared__ int32_t part[1024];
  __shared__ uint64_t psum[1024];
  const int tid = threadIdx.x;
  const int per = (n_blk + 1023) / 1024;
  int32_t local = 0;
  uint64_t ls = 0;
  for (int i = 0; i < per; ++i) {
    int k = tid * per + i;
    if (k < n_blk) { local += blk_count[k]; ls += blk_sum[k]; }
  }
  part[tid] = local;
  psum[tid] = ls;
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    uint64_t s = 0;
    for (int i = 0; i < 1024; ++i) { int32_t v = part[i]; part[i] = run; run += v; s += psum[i]; }
    *sum_a = s;
  }
  __syncthreads();
  int32_t run = part[tid];
  for (int i = 0; i < per; ++i) {
    int k = tid * per + i;
    if (k < n_blk) { int32_t v = blk_count[k]; blk_count[k] = run; run += v; }
  }
}

// Scatter of the rows of A and of the other rows into their ascending lists. The window
// [q0, q1) is the range alist[rng[0], rng[1]) and nalist[rng[2], rng[3]): the ranks of q0 and
// q1 in the two lists, written by the threads of rows q0 and q1 (q1 = T: the last row).
__global__ __launch_bounds__(kScanBlock) void k_scatter_a(const uint8_t* __restrict__ flags, int T,
                                                          const int32_t* __restrict__ blk_off,
                                                          int32_t* __restrict__ alist,
                                                          int32_t* __restrict__ nalist, int nA,
                                                          int q0, int q1, int32_t* __restrict__ rng) {
  __shared__ uint32_t c[kScanBlock / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int t = blockIdx.x * kScanBlock + threadIdx.x;
  bool valid = t < T;
  bool a = valid && in_a(flags[t]);
  uint64_t bal = __ballot(a);
  if (lane == 0) c[wave] = __popcll(bal);
  __syncthreads();
  uint32_t before = __popcll(bal & ((1ull << lane) - 1ull));
  for (int w = 0; w < wave; ++w) before += c[w];
  if (valid) {
    int32_t off = blk_off[blockIdx.x];
    const int32_t a_before = off + (int32_t)before;  // rows of A before row t
    if (t == q0) {
      rng[0] = a_before;
      rng[2] = t - a_before;
    }
    if (t == q1) {
      rng[1] = a_before;
      rng[3] = t - a_before;
    } else if (q1 == T && t == T - 1) {
      rng[1] = a_before + (a ? 1 : 0);
      rng[3] = T - rng[1];
    }
    // the host sized both lists from the same rule; the bounds only guard the workspace
    if (a) {
      if (off + (int)before < nA) alist[off + before] = t;
    } else {
      int local_idx = threadIdx.x;
      int32_t na_before = blockIdx.x * kScanBlock - off + (local_idx - (int)before);
      if (na_before >= 0 && na_before < T - nA) nalist[na_before] = t;
    }
  }
}

hipError_t launch_protect(const SegDesc* lseg, const SegDesc* runs, const int32_t* seg_of_row, int T,
                          int edge_rows, int tail_rows, const int32_t* dirty, int n_dirty,
                          const uint32_t* score, int64_t need, uint8_t* flags,
                          uint32_t* sel_state, int32_t* blk_count, uint64_t* blk_sum,
                          int n_blk, int32_t* alist, int32_t* nalist, int n_a, uint64_t* sum_a,
                          int q0, int q1, int32_t* rng, hipStream_t stream) {
  (void)sel_state;
  int blocks = (T + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_protect_mark, dim3(blocks), dim3(256), 0, stream, lseg, runs, seg_of_row, T,
                     edge_rows, tail_rows, dirty, n_dirty, flags);
  if (need > 0)
    hipLaunchKernelGGL(k_protect_select, dim3(1), dim3(kSelThreads), 0, stream, flags, score, T,
                       (uint32_t)need);
  hipLaunchKernelGGL(k_count_a, dim3(n_blk), dim3(kScanBlock), 0, stream, flags, T, q0, q1,
                     blk_count, blk_sum);
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(1024), 0, stream, blk_count, blk_sum, n_blk,
                     sum_a);
  hipLaunchKernelGGL(k_scatter_a, dim3(n_blk), dim3(kScanBlock), 0, stream, flags, T, blk_count,
                     alist, nalist, n_a, q0, q1, rng);
  return hipGetLastError();
}

// --------------------------------------------------------------- another window of a plan
// The inverse-output-RoPE table of the window's rows [q0, q1) (at t - q0), and the window's
// ranges in the ascending list of A and in its complement, with the Local heads' key count
// sum over the window's rows of A of (t + 1). The request's geometry and A are kept.
__global__ void k_geom_window_rows(int q0, int q1, int d_rope, double base, float2* __restrict__ rowcs) {
  const int half = d_rope / 2;
  const int64_t n = (int64_t)(q1 - q0) * half;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / half), k = (int)(i - (int64_t)r * half);
    double s, c;
    sincos((double)(q0 + r) * rope_theta(base, k, d_rope), &s, &c);
    rowcs[i] = make_float2((float)c, (float)s);
  }
}

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// by one workgroup of 256 threads; s_rng receives the four ranges too (shared memory)
__device__ __forceinline__ void window_ranges(const int32_t* __restrict__ alist, int nA, int q0,
                                              int q1, int32_t* __restrict__ rng,
                                              uint64_t* __restrict__ sum_a, int32_t* s_rng) {
  __shared__ uint64_t part[4];
  if (threadIdx.x == 0) {
    const int lo = lower_bound_i32(alist, nA, q0), hi = lower_bound_i32(alist, nA, q1);
    const int32_t r[4] = {lo, hi, q0 - lo, q1 - hi};  // rows outside A before q0, before q1
    for (int k = 0; k < 4; ++k) {
      rng[k] = r[k];
      s_rng[k] = r[k];
    }
  }
  __syncthreads();
  uint64_t v = 0;
  for (int i = s_rng[0] + threadIdx.x; i < s_rng[1]; i += 256) v += (uint64_t)alist[i] + 1;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) *sum_a = part[0] + part[1] + part[2] + part[3];
}

__global__ __launch_bounds__(256) void k_window_ranges(const int32_t* __restrict__ alist, int nA,
                                                       int q0, int q1, int32_t* __restrict__ rng,
                                                       uint64_t* __restrict__ sum_a) {
  __shared__ int32_t s_rng[4];
  window_ranges(alist, nA, q0, q1, rng, sum_a, s_rng);
}

hipError_t launch_window(const int32_t* alist, int nA, int q0, int q1, int d_rope, double base,
                         float2* rowcs, int32_t* rng, uint64_t* sum_a, hipStream_t stream) {
  const int64_t n = (int64_t)(q1 - q0) * (d_rope / 2);
  int blocks = (int)((n + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_geom_window_rows, dim3(blocks), dim3(256), 0, stream, q0, q1, d_rope, base,
                     rowcs);
  hipLaunchKernelGGL(k_window_ranges, dim3(1), dim3(256), 0, stream, alist, nA, q0, q1, rng, sum_a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------ work list
// Tiles sorted by decreasing largest row (their key count), F and G tiles interleaved by a
// merge-by-rank: each tile's rank = its position in its own descending list plus the number
// of tiles of the other list that sort before it (equal costs: F tiles first). Only the first
// nF_act / nG_act tiles of each stream hold rows (a row window can fill less than the host's
// sizing); the empty ones take the last ranks, so `work` stays a permutation of all tiles.
__device__ __forceinline__ void worklist_tiles(const TileMap& m, int32_t* __restrict__ work,
                                               int first, int stride) {
  const int n = m.nF + m.nG;
  const int nF_act = (int)(((int64_t)(m.rng[1] - m.rng[0]) * m.HF + kTileQ - 1) / kTileQ);
  const int nG_act = (int)(((int64_t)(m.rng[3] - m.rng[2]) * m.HG + kTileQ - 1) / kTileQ);
  const int n_act = nF_act + nG_act;
  for (int tile = first; tile < n; tile += stride) {
    int rank;
    if (tile < m.nF) {
      if (tile >= nF_act) {
        rank = n_act + (tile - nF_act);
      } else {
        const int c = tile_max_row(m, tile);
        // G tiles with cost > c: nG_act - (#G tiles with cost <= c)
        int lo = 0, hi = nG_act;  // first G index with cost > c
        while (lo < hi) {
          int mid = (lo + hi) >> 1;
          if (tile_max_row(m, m.nF + mid) > c) hi = mid; else lo = mid + 1;
        }
        rank = (nF_act - 1 - tile) + (nG_act - lo);
      }
    } else {
      const int k = tile - m.nF;
      if (k >= nG_act) {
        rank = n_act + (m.nF - nF_act) + (k - nG_act);
      } else {
        const int c = tile_max_row(m, tile);
        int lo = 0, hi = nF_act;  // first F index with cost >= c
        while (lo < hi) {
          int mid = (lo + hi) >> 1;
          if (tile_max_row(m, mid) >= c) hi = mid; else lo = mid + 1;
        }
        rank = (nG_act - 1 - k) + (nF_act - lo);
      }
    }
    work[rank] = tile;
  }
}

__global__ void k_worklist(TileMap m, int32_t* __restrict__ work) {
  worklist_tiles(m, work, blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}

// A window of a few rows (the next decode row of a plan): its RoPE rows, its ranges and the
// work list in one workgroup, so that moving the plan is one launch instead of three. The
// ranges reach the work list through shared memory.
__global__ __launch_bounds__(256) void k_window_small(const int32_t* __restrict__ alist, int nA,
                                                      int d_rope, double base,
                                                      float2* __restrict__ rowcs, TileMap m,
                                                      uint64_t* __restrict__ sum_a,
                                                      int32_t* __restrict__ work) {
  __shared__ int32_t s_rng[4];
  const int q0 = m.q0, q1 = m.q0 + m.nq, half = d_rope / 2;
  for (int i = threadIdx.x; i < (q1 - q0) * half; i += 256) {
    const int r = i / half, k = i - r * half;
    double s, c;
    sincos((double)(q0 + r) * rope_theta(base, k, d_rope), &s, &c);
    rowcs[i] = make_float2((float)c, (float)s);
  }
  window_ranges(alist, nA, q0, q1, const_cast<int32_t*>(m.rng), sum_a, s_rng);  // ends in a barrier
  TileMap ms = m;
  ms.rng = s_rng;
  worklist_tiles(ms, work, threadIdx.x, 256);
}

hipError_t launch_window_small(const int32_t* alist, int nA, int d_rope, double base, float2* rowcs,
                               TileMap map, uint64_t* sum_a, int32_t* work, hipStream_t stream) {
  hipLaunchKernelGGL(k_window_small, dim3(1), dim3(256), 0, stream, alist, nA, d_rope, base, rowcs,
                     map, sum_a, work);
  return hipGetLastError();
}

hipError_t launch_worklist(TileMap map, int32_t* work, hipStream_t stream) {
  int n = map.nF + map.nG;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_worklist, dim3((n + 255) / 256), dim3(256), 0, stream, map, work);
  return hipGetLastError();
}

}  // namespace segmla
