// Row-replacement epilogue (RedKnot-MLA paper, head-partition paragraph Eq. 2 and the
// protected-row paragraph): for every computed (row t, head h) -- Global heads on all rows,
// Local heads on rows of A -- u = [O^nope, R(-t) O^rope] and Z[t][h] = W_h u with W_h the
// head's slice of the bias-free first output projection. On rows outside A the Local heads'
// slots receive the cached contribution Zc[pool_row(t)] unchanged: replaced, never added to.
#include "internal.h"
#include "lds_tile.h"

namespace segmla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// A tile is a run of rows of one list and an output slot. Per-head state: the slot is a
// head; Global heads walk every row of the window [q0, q0 + nq), Local heads its rows of A
// (alist[rng[0], rng[1])). Grouped state: the slot is a group; on its rows of A the tile sums
// all of the group's heads, on its other rows (nalist[rng[2], rng[3])) the group's Global
// heads plus the cached Local contribution. Lists of rows of A (or outside A) are laid out for
// the largest possible count (e.nA, e.nNA); tiles past the actual count are empty
// (n_rows <= r0).
struct EpiTile {
  int h, r0, n_rows, q0;
  const int32_t* rows;   // null = the window's rows in order (request row q0 + i)
  int nh;                // heads summed into the slot
  const int32_t* heads;  // null = heads h .. h + nh - 1
  int slot;              // output slot: the head, or the group
  bool add_cache;        // add z_cached[pool_row(t)][slot] (grouped state, rows outside A)
};

// grouped = false lays out per-head tiles whatever the state (the per-head fp32 projections
// of a grouped decode window)
__device__ __forceinline__ EpiTile epi_tile(const EpiArgs& e, int b, int rows_per_tile,
                                            bool grouped) {
  EpiTile et;
  et.q0 = e.q0;
  et.nh = 1;
  et.heads = nullptr;
  et.add_cache = false;
  const int ta = (e.nA + rows_per_tile - 1) / rows_per_tile;
  if (grouped) {
    if (b < e.n_groups * ta) {
      const int g = b / ta;
      et.h = g * e.G;
      et.nh = e.G;
      et.slot = g;
      et.r0 = (b % ta) * rows_per_tile;
      et.n_rows = e.rng[1] - e.rng[0];
      et.rows = e.alist + e.rng[0];
    } else {
      b -= e.n_groups * ta;
      const int tn = (e.nNA + rows_per_tile - 1) / rows_per_tile;
      const int g = b / tn;
      et.h = 0;
      et.heads = e.grp_ghead + e.grp_gstart[g];
      et.nh = e.grp_gstart[g + 1] - e.grp_gstart[g];
      et.slot = g;
      et.add_cache = e.HL > 0;
      et.r0 = (b % tn) * rows_per_tile;
      et.n_rows = e.rng[3] - e.rng[2];
      et.rows = e.nalist + e.rng[2];
    }
    return et;
  }
  const int tg = (e.nq + rows_per_tile - 1) / rows_per_tile;
  if (b < e.HG * tg) {
    et.h = e.ghead[b / tg];
    et.r0 = (b % tg) * rows_per_tile;
    et.n_rows = e.nq;
    et.rows = nullptr;
  } else {
    b -= e.HG * tg;
    et.h = e.lhead[b / ta];
    et.r0 = (b % ta) * rows_per_tile;
    et.n_rows = e.rng[1] - e.rng[0];
    et.rows = e.alist + e.rng[0];
  }
  et.slot = et.h;
  return et;
}

// request row of list entry i; head j of the tile
__device__ __forceinline__ int epi_row(const EpiTile& et, int i) { return et.rows ? et.rows[i] : et.q0 + i; }
__device__ __forceinline__ int epi_head(const EpiTile& et, int j) { return et.heads ? et.heads[j] : et.h + j; }
// output slots per row of z, and the pool row of request row t (the cached state's row)
__device__ __forceinline__ int z_slots(const EpiArgs& e) { return e.G >= 2 ? e.n_groups : e.H; }
__device__ __forceinline__ int64_t pool_row_of(const EpiArgs& e, int t) {
  const SegDesc sd = e.seg[e.seg_of_row[t]];
  return sd.pool_row + (t - sd.offset);
}

// ------------------------------------------------------------------------ fp32 path
// One wavefront per (row, slot): for each of the slot's heads u is staged in LDS and each
// lane adds its d_state/64 outputs (per-head state: one head, so z = W_h u exactly).
constexpr int kF32MaxCols = 16;  // d_state <= 64 * 16
__global__ __launch_bounds__(64) void k_project_f32(EpiArgs e) {
  __shared__ float u[1024];
  const int lane = threadIdx.x;
  EpiTile et = epi_tile(e, blockIdx.x, 1, e.G >= 2);
  if (et.r0 >= et.n_rows) return;
  const int t = epi_row(et, et.r0);
  float acc[kF32MaxCols];
#pragma unroll
  for (int k = 0; k < kF32MaxCols; ++k) acc[k] = 0.f;
  for (int j = 0; j < et.nh; ++j) {
    const int h = epi_head(et, j);
    __syncthreads();  // the previous head's u is consumed
    const float* o = (const float*)e.out + ((int64_t)(t - e.q0) * e.H + h) * e.d_v;
    for (int d = lane; d < e.d_v; d += 64) u[d] = o[d];
    __syncthreads();
    if (e.v_has_rope) {
      const int half_r = e.d_rope / 2;
      for (int k = lane; k < half_r; k += 64) {  // u^r <- R(-t) O^r
        float2 cs = e.rowcs[(int64_t)(t - e.q0) * half_r + k];
        float x = o[e.d_nope + 2 * k], y = o[e.d_nope + 2 * k + 1];
        u[e.d_nope + 2 * k] = x * cs.x + y * cs.y;
        u[e.d_nope + 2 * k + 1] = -x * cs.y + y * cs.x;
      }
    }
    __syncthreads();
    const float* w = (const float*)e.w + (int64_t)h * e.d_state * e.d_v;
#pragma unroll
    for (int k = 0; k < kF32MaxCols; ++k) {
      const int c = lane + 64 * k;
      if (c >= e.d_state) continue;
      const float* wr = w + (int64_t)c * e.d_v;
      float dot = 0.f;
      for (int d = 0; d < e.d_v; ++d) dot = fmaf(wr[d], u[d], dot);
      acc[k] += dot;
    }
  }
  const float* zc = et.add_cache
      ? (const float*)e.z_cached + (pool_row_of(e, t) * z_slots(e) + et.slot) * e.d_state : nullptr;
  float* z = (float*)e.z + ((int64_t)(t - e.q0) * z_slots(e) + et.slot) * e.d_state;
#pragma unroll
  for (int k = 0; k < kF32MaxCols; ++k) {
    const int c = lane + 64 * k;
    if (c < e.d_state) z[c] = zc ? acc[k] + zc[c] : acc[k];
  }
}

// ------------------------------------------------------------------------ bf16 path
// W_h in the projection's A-operand order: for head h, k-step ks (16 features) and 32-column
// block b, the 64 lanes' fragments (lane (c, hf) = W[32 b + c][16 ks + 8 hf .. + 7]) are 1 KB
// contiguous, so every operand load of the projection is one contiguous 1 KB read.
// Wt[((h * KS + ks) * NB + b) * 64 + lane] (16-byte chunks), one chunk per thread, read in
// W's own order (coalesced) and written to its operand slot.
__global__ __launch_bounds__(256) void k_w_tile(EpiArgs e) {
  const int ks_n = e.d_v / 16, nb = e.d_state / 32, cpr = e.d_v / 8;  // chunks per W row
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;         // W chunk (h, row, k8)
  if (c >= (int64_t)e.H * e.d_state * cpr) return;
  const int k8 = (int)(c % cpr);
  const int64_t hr = c / cpr;
  const int row = (int)(hr % e.d_state), h = (int)(hr / e.d_state);
  const int ks = k8 >> 1, lane = ((k8 & 1) << 5) | (row & 31), b = row >> 5;
  const uint4 v = ((const uint4*)e.w)[c];
  ((uint4*)e.wt)[(((int64_t)h * ks_n + ks) * nb + b) * 64 + lane] = v;
}

// Workgroup = (head h, 128 rows of its list) x all d_state columns, 4 waves (one per SIMD).
// U (128 x d_v) is staged in LDS in the packed-latent tile layout (lds_tile.h) by
// global->LDS copies, one per nope row and one per 8 RoPE rows, all in flight at once; the
// RoPE part is then de-rotated in place by R(-t) (fp32, rounded to bf16). The product is
// computed transposed, Z^T = W_h U^T, with MFMA 32x32x16 bf16 (fp32 accumulation): the A
// operand (W_h rows) streams from L2 with a two-step register prefetch, the B operand (U^T,
// 16 consecutive rows x one chunk per 16 lanes: conflict-free) comes from LDS. Wave w owns the
// 32-column blocks w, w + 4, ..., four at a time (4 x 4 accumulators of 16 values = the 256
// AGPRs). A lane's accumulator holds 4 consecutive columns of one row, stored as one 8-byte
// write.
constexpr int kEpiRows = 128;
constexpr int kEpiNRow = 1024;                    // LDS bytes per row, nope region
constexpr int kEpiRBase = kEpiRows * kEpiNRow;    // RoPE region (128 rows x 128 bytes)
constexpr int kEpiRowIds = kEpiRBase + kEpiRows * 128;  // request row of each tile row
constexpr int kEpiLds = kEpiRowIds + kEpiRows * 4;      // 147968 bytes
constexpr int kEpiPf = 4;                         // W ring slots, in k-steps (even, divides 32)
static_assert(32 % kEpiPf == 0 && kEpiPf % 2 == 0, "ring slots are compile-time: kEpiPf divides the 32 nope k-steps");

template <bool GROUPED>
__global__ __launch_bounds__(256, 1) void k_project_bf16(EpiArgs e) {
  extern __shared__ __attribute__((aligned(16))) char lds_u[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  EpiTile et = epi_tile(e, blockIdx.x, kEpiRows, e.G >= 2);
  const int n_here = min(kEpiRows, et.n_rows - et.r0);
  if (n_here <= 0) return;  // uniform: a Local tile past the window's rows of A
  const int d_v = e.d_v, half_r = e.d_rope / 2;
  const bool rope = e.v_has_rope != 0;  // d_v = 576 (else 512: nope only)
  const int64_t hstride = (int64_t)d_v * 2;
  // request rows of the tile first (rows past n_here repeat the last row: finite data, outputs
  // not stored), so that no vector load is waited for while copies are in flight
  int* const row_id = (int*)(lds_u + kEpiRowIds);
  if (tid < kEpiRows) row_id[tid] = epi_row(et, et.r0 + min(tid, n_here - 1));
  __syncthreads();
  // stage U of head h (the tile's rows), then de-rotate its RoPE part
  auto stage = [&](int h) __attribute__((always_inline)) {
    const char* outb = (const char*)e.out + (int64_t)h * hstride;
    const uint32_t base = lds_addr(lds_u);
    const int lane = lane_id();
    for (int n = 0; n < kEpiRows / 4; ++n) {
      const int r = wave + 4 * n;
      const int t = __builtin_amdgcn_readfirstlane(row_id[r]);
      dma16(outb + (int64_t)(t - e.q0) * e.H * hstride, (lane * 16) ^ (fn(r) << 4), base + r * kEpiNRow);
    }
    if (rope) {
      for (int m = 0; m < kEpiRows / 32; ++m) {  // 8 RoPE rows per copy
        const int q = wave + 4 * m;
        const int r = 8 * q + (lane >> 3);
        const int t = row_id[r];
        dma16_v(outb + (int64_t)(t - e.q0) * e.H * hstride + kEpiNRow + (((lane & 7) ^ fr(r)) << 4),
                base + kEpiRBase + q * 1024);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (rope) {  // u^r <- R(-t) O^r in place: 128 rows x 8 chunks, 4 chunks per thread
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int idx = n * 256 + tid, r = idx >> 3, c = idx & 7;
        const int t = row_id[r];
        char* p = lds_u + kEpiRBase + r * 128 + ((c ^ fr(r)) << 4);
        uint4 v = *(const uint4*)p;
        const __bf16* x = (const __bf16*)&v;
        __bf16 y[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 cs = e.rowcs[(int64_t)(t - e.q0) * half_r + 4 * c + k];
          const float a0 = (float)(x[2 * k]), a1 = (float)(x[2 * k + 1]);
          y[2 * k] = (__bf16)(a0 * cs.x + a1 * cs.y);
          y[2 * k + 1] = (__bf16)(-a0 * cs.y + a1 * cs.x);
        }
        *(uint4*)p = *(const uint4*)y;
      }
      __syncthreads();
    }
  };
  const int nh = GROUPED ? et.nh : 1;
  if (nh > 0) stage(epi_head(et, 0));
  const int lane = tid & 63;
  const int nblk_all = e.d_state / 32;
  const int64_t wstep = (int64_t)nblk_all * 64 * 8;  // elements per k-step
  const int ksteps = d_v / 16;
  const int nblk = e.d_state / 32;      // 32-column blocks (d_state % 64 == 0)
  const int col = lane & 31, hf = lane >> 5;
  // B operand (U^T, 16 features x 32 rows): lane holds U[row 32 i + col][16 ks + 8 hf .. + 7],
  // nope chunk 2 ks + hf at (2 ks ^ (fn & 14)) | (hf ^ (fn & 1)); RoPE step 32 + j: chunk 2 j + hf
  const int fc = fn(col), rc = fr(col);
  const char* ubn = lds_u + col * kEpiNRow + 16 * (hf ^ (fc & 1));
  const int usw = 16 * (fc & 14);
  const char* ubr = lds_u + kEpiRBase + col * 128 + 16 * (hf ^ (rc & 1));
  const int ursw = 16 * (rc & 6);
  int rows_t[4];                        // request row of each of the lane's 4 output rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * i + col;
    rows_t[i] = r < n_here ? row_id[r] : -1;
  }
  const int zs = z_slots(e);
  // passes over the 32-column blocks: wave w takes blocks b0, b0 + 4, .. < b0 + 16. Grouped,
  // every wave makes the same number of passes (staging the slot's next head is a workgroup
  // barrier); per head, a wave with no block left stops.
  for (int b0 = wave; GROUPED ? b0 - wave < nblk : b0 < nblk; b0 += 16) {
    int nb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) nb += (b0 + 4 * j < nblk) ? 1 : 0;
    floatx16_t acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[j][i][k] = 0.f;
    for (int hj = 0; hj < nh; ++hj) {
      if (GROUPED && nh > 1 && (b0 > wave || hj > 0)) {  // U of the slot's next head
        __syncthreads();
        stage(epi_head(et, hj));
      }
      if (nb == 0) continue;
      const int hh = GROUPED ? epi_head(et, hj) : et.h;
      const __bf16* wt = (const __bf16*)e.wt + (int64_t)hh * (d_v / 16) * nblk_all * 64 * 8;
      // A operand (W_h, 32 columns x 16 features): lane holds W[column][16 ks + 8 hf .. + 7],
      // read from the operand-ordered copy (1 KB contiguous per wave and k-step)
      const __bf16* wr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = min(b0 + 4 * j, nblk - 1);  // clamp: unused blocks read valid data
        wr[j] = wt + ((int64_t)blk * 64 + lane) * 8;
      }
      // W fragments: a ring of kEpiPf k-steps; the loads for k-step ks + kEpiPf - 1 (clamped to
      // the last k-step: no branch, so the wait counts stay exact) are issued at the start of
      // k-step ks, giving each load kEpiPf - 1 k-steps (16 MFMAs each) to arrive. U fragments are
      // read one k-step ahead. The 32 nope k-steps and the 4 RoPE k-steps run as separate loops,
      // so each address form is fixed at compile time.
      bf16x8_t wf[kEpiPf][4];
#pragma unroll
      for (int s = 0; s < kEpiPf - 1; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) wf[s][j] = *(const bf16x8_t*)(wr[j] + wstep * min(s, ksteps - 1));
      auto u_nope = [&](int ks, bf16x8_t* u) __attribute__((always_inline)) {  // ks < 32
        const char* up = ubn + ((32 * (ks & 7)) ^ usw) + 256 * (ks >> 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = *(const bf16x8_t*)(up + i * 32 * kEpiNRow);
      };
      auto u_rope = [&](int j, bf16x8_t* u) __attribute__((always_inline)) {  // k-step 32 + j
        const char* up = ubr + ((32 * j) ^ ursw);
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = *(const bf16x8_t*)(up + i * 32 * 128);
      };
      bf16x8_t ur[2][4];
      auto kstep = [&](int ks, int slot, auto&& read_next) __attribute__((always_inline)) {
        const int kp = min(ks + kEpiPf - 1, ksteps - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) wf[(slot + kEpiPf - 1) % kEpiPf][j] = *(const bf16x8_t*)(wr[j] + wstep * kp);
        read_next();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[slot][j], ur[slot & 1][i], acc[j][i], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      };
      u_nope(0, ur[0]);
      for (int ks0 = 0; ks0 < 32; ks0 += kEpiPf) {
#pragma unroll
        for (int slot = 0; slot < kEpiPf; ++slot)
          kstep(ks0 + slot, slot, [&] { u_nope(min(ks0 + slot + 1, 31), ur[(slot + 1) & 1]); });
      }
      if (rope) {  // k-steps 32..35 (ring slot (32 + j) % kEpiPf; kEpiPf is even)
        u_rope(0, ur[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          kstep(32 + j, (32 + j) % kEpiPf, [&] { u_rope(min(j + 1, 3), ur[(j + 1) & 1]); });
      }
    }
    // C[m][n] = Z^T[column][row]: lane holds row 32 i + col and columns
    // 32 blk + 8 (k >> 2) + 4 hf + (k & 3)
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= nb) continue;
      const int cbase = 32 * (b0 + 4 * j) + 4 * hf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (rows_t[i] < 0) continue;
        __bf16* z = (__bf16*)e.z + ((int64_t)(rows_t[i] - e.q0) * (GROUPED ? zs : e.H) +
                                    (GROUPED ? et.slot : et.h)) * e.d_state + cbase;
        const __bf16* zc = nullptr;
        if (GROUPED && et.add_cache)
          zc = (const __bf16*)e.z_cached + (pool_row_of(e, rows_t[i]) * zs + et.slot) * e.d_state + cbase;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4] = {acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]};
          if (GROUPED && zc) {
            const bf16x4_t c = *(const bf16x4_t*)(zc + 8 * g);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] += (float)c[k];
          }
          const bf16x4_t y = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
          *(bf16x4_t*)(z + 8 * g) = y;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------ thin path
// Windows of at most kThinRows rows (decode): per head the projection is a product of W_h
// with a few vectors, bound by reading W once, so W is read in its own layout (no
// operand-order copy) and no matrix core is used. Workgroup = (slot tile, 64 columns of Z);
// a grouped slot sums its heads one after the other (u restaged per head) and adds the cached
// group vector on rows outside A.
// A team of 8 lanes takes one column: lane j reads the 16-byte chunks j, j + 8, ... of the
// column's W row (each team step reads 128 contiguous bytes) and the team's partial sums meet
// by lane shuffles. The u rows sit in LDS as fp32 holding the values the tile path
// multiplies (nope features as given, RoPE pairs de-rotated by R(-t) and rounded to bf16).
constexpr int kThinMaxK = kThinMaxDv / 64;  // 16-byte chunks per lane and column

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__global__ __launch_bounds__(256) void k_project_thin(EpiArgs e) {
  __shared__ __attribute__((aligned(16))) float us[kThinRows][kThinMaxDv];
  __shared__ int row_id[kThinRows];
  const int ncb = e.d_state / kThinCols;
  const int cb = blockIdx.x % ncb;
  const EpiTile et = epi_tile(e, blockIdx.x / ncb, kThinRows, e.G >= 2 && !e.zpart);
  const int n_here = min(kThinRows, et.n_rows - et.r0);
  if (n_here <= 0) return;  // uniform: a tile past the window's rows of its list
  const int tid = threadIdx.x, d_v = e.d_v;
  const int lane = tid & 63, wave = tid >> 6, team = lane >> 3, j = lane & 7;
  const int nk = d_v / 64;
  // the tile's request rows: loaded first, written to LDS after the first head's W loads are
  // issued (its wait then counts only this load)
  const int rid = tid < kThinRows ? epi_row(et, et.r0 + min(tid, n_here - 1)) : 0;
  float acc[2][kThinRows];
#pragma unroll
  for (int ps = 0; ps < 2; ++ps)
#pragma unroll
    for (int r = 0; r < kThinRows; ++r) acc[ps][r] = 0.f;
  for (int hj = 0; hj < et.nh; ++hj) {  // the slot's heads (grouped state: the group's)
    const int h = epi_head(et, hj);
    // this head's W rows first: they depend on nothing staged, and the u loads below then
    // overlap them instead of following them
    const __bf16* wh = (const __bf16*)e.w + (int64_t)h * e.d_state * d_v;
    uint4 wv[2][kThinMaxK];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const __bf16* wc = wh + (int64_t)(cb * kThinCols + wave * 16 + ps * 8 + team) * d_v + 8 * j;
#pragma unroll
      for (int k = 0; k < kThinMaxK; ++k)
        if (k < nk) wv[ps][k] = *(const uint4*)(wc + 64 * k);
    }
    if (hj == 0 && tid < kThinRows) row_id[tid] = rid;
    __syncthreads();  // first head: the row ids are visible; later heads: every wave is done
                      // with the previous head's u
    {
      const __bf16* outp = (const __bf16*)e.out;
      const int n_pairs = d_v / 2, nope_pairs = e.d_nope / 2, half_r = e.d_rope / 2;
      for (int i = tid; i < n_here * n_pairs; i += 256) {
        const int r = i / n_pairs, k2 = i - r * n_pairs;
        const int t = row_id[r];
        const __bf16* o = outp + ((int64_t)(t - e.q0) * e.H + h) * d_v + 2 * k2;
        float a0 = (float)o[0], a1 = (float)o[1];
        if (k2 >= nope_pairs) {  // v carries the RoPE part (d_v > d_nope)
          const float2 cs = e.rowcs[(int64_t)(t - e.q0) * half_r + (k2 - nope_pairs)];
          const float y0 = (float)(__bf16)(a0 * cs.x + a1 * cs.y);
          const float y1 = (float)(__bf16)(-a0 * cs.y + a1 * cs.x);
          a0 = y0;
          a1 = y1;
        }
        us[r][2 * k2] = a0;
        us[r][2 * k2 + 1] = a1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
      for (int k = 0; k < kThinMaxK; ++k) {
        if (k >= nk) continue;
        const uint4 x = wv[ps][k];
        const float w8[8] = {bf16_lo(x.x), bf16_hi(x.x), bf16_lo(x.y), bf16_hi(x.y),
                             bf16_lo(x.z), bf16_hi(x.z), bf16_lo(x.w), bf16_hi(x.w)};
#pragma unroll
        for (int r = 0; r < kThinRows; ++r) {
          if (r >= n_here) continue;
          const float4 u0 = *(const float4*)&us[r][8 * (j + 8 * k)];
          const float4 u1 = *(const float4*)&us[r][8 * (j + 8 * k) + 4];
          float a = acc[ps][r];
          a = fmaf(w8[0], u0.x, a);
          a = fmaf(w8[1], u0.y, a);
          a = fmaf(w8[2], u0.z, a);
          a = fmaf(w8[3], u0.w, a);
          a = fmaf(w8[4], u1.x, a);
          a = fmaf(w8[5], u1.y, a);
          a = fmaf(w8[6], u1.z, a);
          a = fmaf(w8[7], u1.w, a);
          acc[ps][r] = a;
        }
      }
    }
  }
  const int zs = z_slots(e);
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    // team sums; lane j of the team then stores row j
    float mine = 0.f;
#pragma unroll
    for (int r = 0; r < kThinRows; ++r) {
      float a = acc[ps][r];
      a += __shfl_xor(a, 1);
      a += __shfl_xor(a, 2);
      a += __shfl_xor(a, 4);
      if (r == j) mine = a;
    }
    if (j < n_here) {
      const int col = cb * kThinCols + wave * 16 + ps * 8 + team;
      const int t = row_id[j];
      if (e.zpart) {  // per-head fp32 projection, summed per group by k_group_sum
        e.zpart[((int64_t)(t - e.q0) * e.H + et.h) * e.d_state + col] = mine;
        continue;
      }
      if (et.add_cache)
        mine += (float)((const __bf16*)e.z_cached)[(pool_row_of(e, t) * zs + et.slot) * e.d_state + col];
      ((__bf16*)e.z)[((int64_t)(t - e.q0) * zs + et.slot) * e.d_state + col] = (__bf16)mine;
    }
  }
}

// Grouped decode windows: z[t][g] = the group's computed heads' fp32 projections, summed in
// head order, plus the cached group vector on rows outside A. Workgroup = (window row, group).
__global__ __launch_bounds__(256) void k_group_sum(EpiArgs e) {
  const int i = blockIdx.x / e.n_groups, g = blockIdx.x % e.n_groups;
  const int t = e.q0 + i;
  bool in_a = false;  // the window's rows of A: alist[rng[0], rng[1]), at most 8 of them
  for (int k = e.rng[0]; k < e.rng[1]; ++k) in_a = in_a || e.alist[k] == t;
  const int g0 = e.grp_gstart[g], g1 = e.grp_gstart[g + 1];
  const __bf16* zc = (!in_a && e.HL > 0)
      ? (const __bf16*)e.z_cached + (pool_row_of(e, t) * e.n_groups + g) * e.d_state : nullptr;
  for (int c = threadIdx.x; c < e.d_state; c += 256) {
    float acc = 0.f;
    for (int h = g * e.G; h < (g + 1) * e.G; ++h) {
      bool global = false;
      for (int k = g0; k < g1; ++k) global = global || e.grp_ghead[k] == h;
      if (global || in_a) acc += e.zpart[((int64_t)i * e.H + h) * e.d_state + c];
    }
    if (zc) acc += (float)zc[c];
    ((__bf16*)e.z)[((int64_t)i * e.n_groups + g) * e.d_state + c] = (__bf16)acc;
  }
}

// ------------------------------------------------------------------- restore copy
// Local heads on rows outside A: Z[t][lhead[l]] = Zc[pool_row(t)][l], copied bit for bit.
// One block per window row outside A (nalist[rng[2], rng[3])); the grid is laid out for the
// largest possible count.
template <typename V>
__global__ __launch_bounds__(256) void k_restore_copy(EpiArgs e, int vec_per_head) {
  if ((int)blockIdx.x >= e.rng[3] - e.rng[2]) return;
  const int t = e.nalist[e.rng[2] + blockIdx.x];
  const SegDesc sd = e.seg[e.seg_of_row[t]];
  const int64_t prow = sd.pool_row + (t - sd.offset);
  const V* src = (const V*)e.z_cached + prow * (int64_t)e.HL * vec_per_head;
  V* dst = (V*)e.z + (int64_t)(t - e.q0) * e.H * vec_per_head;
  const int n = e.HL * vec_per_head;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int l = i / vec_per_head, c = i - l * vec_per_head;
    dst[(int64_t)e.lhead[l] * vec_per_head + c] = src[i];
  }
}

// ------------------------------------------------------------------- fused decode path
// One-row windows whose key range the decode kernel split (bf16 partials), per-head state: the
// log-sum-exp merge of the partials (RedKnot-MLA paper, relocation paragraph) and the projection
// of the merged outputs (head-partition paragraph, Eq. 2) in one kernel, so that W streams while
// the partials are merged rather than after them. Workgroup = (query vector v, kDmpCols columns
// of Z), eight waves. Every workgroup of a vector merges all of its channels: thread (slot, g)
// sums channels 8 g .. 8 g + 7 of the splits slot, slot + SS, ... in batches of kDmpLoads
// 16-byte loads, weighted by e^(m_s - M) from an LDS table, and the slots meet in LDS. The
// merged output is rounded to bf16 as stored (the first column block stores it and its lse),
// u = [O^n, R(-t) O^r] is formed from those values as k_project_thin forms it, and the product
// follows k_project_thin lane for lane (the same W chunks per lane, the same summation order).
// A vector's workgroups run on one XCD, so its repeated partial reads meet in one L2 (blocks
// are dispatched round-robin over the 8 XCDs): block b takes vector 8 ((b / 8) / ncb) + b % 8
// and column block (b / 8) % ncb.
constexpr int kDmpThreads = 512;
constexpr int kDmpCols = (kDmpThreads / 64) * 16;  // 8 teams of 8 lanes per wave, two passes
constexpr int kDmpLoads = 18;                      // partial loads in flight per thread
constexpr int kDmpMaxSplits = 4096;                // LDS weight table
static_assert(kDmpCols == 128 && kDmpMaxSplits == 4096, "the limits dec_merge_project_fits states");

__global__ __launch_bounds__(kDmpThreads) void k_dec_merge_project(AttnArgs a, EpiArgs e) {
  __shared__ float sw[kDmpMaxSplits], sl[kDmpMaxSplits];
  __shared__ float red[2][kDmpThreads / 64];
  __shared__ __attribute__((aligned(16))) float us[kThinMaxDv];
  __shared__ __attribute__((aligned(16))) float ps[kDmpThreads * 8];  // [slot][channel]
  const int ncb = e.d_state / kDmpCols;
  const int b = (int)blockIdx.x;
  const int64_t v = (int64_t)((b >> 3) / ncb) * 8 + (b & 7);
  const int cb = (b >> 3) % ncb;
  const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
  if (v >= nvec) return;
  const int tile = (int)(v / kTileQ), qi = (int)(v % kTileQ);
  int t, h;
  if (!tile_qvec(a.map, tile, qi, t, h)) return;  // uniform over the workgroup
  const int n = min(a.n_split, tile_max_row(a.map, tile) / a.split_keys + 1);  // >= 1
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d_v = a.d_v, NG = d_v / 8, SS = kDmpThreads / NG;
  const int slot = tid / NG, g = tid - slot * NG;
  const bool mer = slot < SS;  // the threads past SS * NG take part in the weights only
  const int64_t sstride = nvec * d_v;
  const __bf16* po = (const __bf16*)a.part_o + v * d_v + 8 * g;
  const float* pml = a.part_ml + v * 2;
  // issue order is retire order: the (max, sum) pairs, the first batch of partials, W
  float2 ml0 = make_float2(-INFINITY, 0.f);
  if (tid < n) ml0 = *(const float2*)(pml + (int64_t)tid * nvec * 2);
  uint4 x[kDmpLoads];
  auto load_batch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kDmpLoads; ++k) {  // past the last split: reread it, weight 0
      const int s = min(s0 + slot + SS * k, n - 1);
      x[k] = mer ? *(const uint4*)(po + (int64_t)s * sstride) : make_uint4(0, 0, 0, 0);
    }
  };
  load_batch(0);
  const int team = lane >> 3, j = lane & 7, nk = d_v / 64;
  const __bf16* wh = (const __bf16*)e.w + (int64_t)h * e.d_state * d_v;
  uint4 wv[2][kThinMaxK];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const __bf16* wc = wh + (int64_t)(cb * kDmpCols + wave * 16 + p * 8 + team) * d_v + 8 * j;
#pragma unroll
    for (int k = 0; k < kThinMaxK; ++k)
      if (k < nk) wv[p][k] = *(const uint4*)(wc + 64 * k);
  }
  // split weights e^(m_s - M) and the normaliser
  float m = ml0.x;
  if (tid < n) {
    sw[tid] = ml0.x;
    sl[tid] = ml0.y;
  }
  for (int s = tid + kDmpThreads; s < n; s += kDmpThreads) {  // more than kDmpThreads splits
    const float2 ml = *(const float2*)(pml + (int64_t)s * nvec * 2);
    sw[s] = ml.x;
    sl[s] = ml.y;
    m = fmaxf(m, ml.x);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[0][wave] = m;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < kDmpThreads / 64; ++w) M = fmaxf(M, red[0][w]);
  float den = 0.f;
  for (int s = tid; s < n; s += kDmpThreads) {  // the entries this thread wrote above
    const float ms = sw[s];
    const float w = ms == -INFINITY ? 0.f : expf(ms - M);
    sw[s] = w;
    den += w * sl[s];
  }
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
  if (lane == 0) red[1][wave] = den;
  __syncthreads();
  // weighted sums of the slot's splits
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < n; s0 += SS * kDmpLoads) {
    if (s0 > 0) load_batch(s0);
#pragma unroll
    for (int k = 0; k < kDmpLoads; ++k) {
      const int s = s0 + slot + SS * k;
      const float w = (mer && s < n) ? sw[s] : 0.f;
      const uint32_t xw[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w, bf16_lo(xw[i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, bf16_hi(xw[i]), acc[2 * i + 1]);
      }
    }
  }
  // thread (slot, g) = ps[slot * d_v + 8 g .. + 7] (tid = slot * NG + g)
  *(float4*)&ps[tid * 8] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *(float4*)&ps[tid * 8 + 4] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  float dt = 0.f;
#pragma unroll
  for (int w = 0; w < kDmpThreads / 64; ++w) dt += red[1][w];
  const float inv = dt > 0.f ? 1.f / dt : 0.f;
  const int64_t o = (int64_t)(t - a.q0) * a.map.H + h;
  const int half_r = e.d_rope / 2, nope_pairs = e.d_nope / 2;
  for (int k2 = tid; k2 < d_v / 2; k2 += kDmpThreads) {
    const int c = 2 * k2;
    float s0 = 0.f, s1 = 0.f;
    for (int q = 0; q < SS; ++q) {
      s0 += ps[q * d_v + c];
      s1 += ps[q * d_v + c + 1];
    }
    const __bf16 b0 = (__bf16)(s0 * inv), b1 = (__bf16)(s1 * inv);
    if (cb == 0) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t y = {b0, b1};
      *(bf16x2_t*)((__bf16*)a.out + o * d_v + c) = y;
    }
    float a0 = (float)b0, a1 = (float)b1;
    if (k2 >= nope_pairs) {  // v carries the RoPE part: u^r = R(-t) O^r, rounded as stored
      const float2 cs = e.rowcs[(int64_t)(t - e.q0) * half_r + (k2 - nope_pairs)];
      const float y0 = (float)(__bf16)(a0 * cs.x + a1 * cs.y);
      const float y1 = (float)(__bf16)(-a0 * cs.y + a1 * cs.x);
      a0 = y0;
      a1 = y1;
    }
    us[c] = a0;
    us[c + 1] = a1;
  }
  if (a.lse && cb == 0 && tid == 0) a.lse[o] = dt > 0.f ? M + logf(dt) : -INFINITY;
  __syncthreads();
  // z[t][h][columns] = W_h u: the per-lane chunks and summation order of k_project_thin
  float pacc[2] = {0.f, 0.f};
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int k = 0; k < kThinMaxK; ++k) {
      if (k >= nk) continue;
      const uint4 xv = wv[p][k];
      const float w8[8] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y),
                           bf16_lo(xv.z), bf16_hi(xv.z), bf16_lo(xv.w), bf16_hi(xv.w)};
      const float4 u0 = *(const float4*)&us[8 * (j + 8 * k)];
      const float4 u1 = *(const float4*)&us[8 * (j + 8 * k) + 4];
      float s = pacc[p];
      s = fmaf(w8[0], u0.x, s);
      s = fmaf(w8[1], u0.y, s);
      s = fmaf(w8[2], u0.z, s);
      s = fmaf(w8[3], u0.w, s);
      s = fmaf(w8[4], u1.x, s);
      s = fmaf(w8[5], u1.y, s);
      s = fmaf(w8[6], u1.z, s);
      s = fmaf(w8[7], u1.w, s);
      pacc[p] = s;
    }
  }
  const int zs = z_slots(e);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float s = pacc[p];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (j == 0) {
      const int col = cb * kDmpCols + wave * 16 + p * 8 + team;
      ((__bf16*)e.z)[((int64_t)(t - e.q0) * zs + h) * e.d_state + col] = (__bf16)s;
    }
  }
}

hipError_t launch_dec_merge_project(const AttnArgs& a, const EpiArgs& e, hipStream_t stream) {
  if (!dec_merge_project_fits(a.d_v, e.d_state, a.n_split)) return hipErrorInvalidConfiguration;
  const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
  const int64_t blocks = (nvec + 7) / 8 * 8 * (e.d_state / kDmpCols);
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (blocks > 0)
    hipLaunchKernelGGL(k_dec_merge_project, dim3((unsigned)blocks), dim3(kDmpThreads), 0, stream, a, e);
  if (e.HL > 0 && e.nNA > 0 && !e.restore_done)
    hipLaunchKernelGGL(k_restore_copy<uint4>, dim3(e.nNA), dim3(256), 0, stream, e, e.d_state * 2 / 16);
  return hipGetLastError();
}

// ------------------------------------------------------------------- E4M3 output
// The grouped state for the next projection as 1x128 E4M3 blocks ("Reading notes on
// DeepSeek-V4 serving in TensorRT-LLM", Part I, FP8 dataflow bullet): 16 lanes per block of
// 128 channels, 8 per lane (one 16-byte load, one 8-byte store). scale = amax / 448 in fp32 (1
// for an all-zero block), and the hardware conversion rounds value / scale to the nearest OCP
// E4M3 code (ties to even); every quotient is at most 448 in magnitude up to the rounding of
// the scale, far below the first value that would round past the largest finite code (464).
__global__ __launch_bounds__(256) void k_quant_e4m3(const __bf16* __restrict__ src,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales, int64_t n_blocks) {
  const int64_t b = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  if (b >= n_blocks) return;  // uniform per 16-lane group (the shuffles stay inside it)
  const int j = threadIdx.x & 15;
  const uint4 v = ((const uint4*)(src + b * 128))[j];
  const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(x[k]));
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float scale = m > 0.f ? m / 448.f : 1.f;
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] / scale, x[1] / scale, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] / scale, x[3] / scale, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] / scale, x[5] / scale, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] / scale, x[7] / scale, hi, true);
  ((uint2*)(codes + b * 128))[j] = make_uint2((uint32_t)lo, (uint32_t)hi);
  if (j == 0) scales[b] = scale;
}

hipError_t launch_quant_e4m3(const __bf16* src, uint8_t* codes, float* scales, int64_t n_blocks,
                             hipStream_t stream) {
  const int64_t blocks = (n_blocks + 15) / 16;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_e4m3, dim3((unsigned)blocks), dim3(256), 0, stream, src, codes, scales,
                     n_blocks);
  return hipGetLastError();
}

hipError_t launch_epilogue(const EpiArgs& e, int io_dtype, hipStream_t stream) {
  const bool grouped = e.G >= 2;
  // tiles of `rows` rows: per-head state: Global heads x window rows + Local heads x rows of A
  // (the restore copy takes the Local heads' other rows); grouped: groups x (rows of A + the
  // other rows)
  auto n_tiles = [&](int rows) -> int64_t {
    if (grouped)
      return (int64_t)e.n_groups * ((e.nA + rows - 1) / rows + (e.nNA + rows - 1) / rows);
    return (int64_t)e.HG * ((e.nq + rows - 1) / rows) + (int64_t)e.HL * ((e.nA + rows - 1) / rows);
  };
  if (io_dtype == 0) {
    const int64_t blocks = n_tiles(1);
    if (blocks > 0)
      hipLaunchKernelGGL(k_project_f32, dim3((unsigned)blocks), dim3(64), 0, stream, e);
    if (!grouped && e.HL > 0 && e.nNA > 0)
      hipLaunchKernelGGL(k_restore_copy<float>, dim3(e.nNA), dim3(256), 0, stream, e, e.d_state);
  } else {
    const int64_t blocks = n_tiles(kEpiRows);
    const size_t lds = kEpiLds;
    // once per process (thread-safe initialization of a function-local static)
    static const hipError_t attr = [] {
      for (const void* k : {(const void*)k_project_bf16<false>, (const void*)k_project_bf16<true>}) {
        hipError_t r = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kEpiLds);
        if (r != hipSuccess) return r;
      }
      return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    const bool thin = e.thin != 0;  // decided by the plan (it sizes the W copy only without)
    if (blocks > 0 && thin && e.zpart) {  // grouped: per-head projections, then group sums
      const int64_t tiles = (int64_t)e.HG * ((e.nq + kThinRows - 1) / kThinRows) +
                            (int64_t)e.HL * ((e.nA + kThinRows - 1) / kThinRows);
      hipLaunchKernelGGL(k_project_thin, dim3((unsigned)(tiles * (e.d_state / kThinCols))),
                         dim3(256), 0, stream, e);
      hipLaunchKernelGGL(k_group_sum, dim3((unsigned)(e.nq * e.n_groups)), dim3(256), 0, stream, e);
    } else if (blocks > 0 && thin) {  // one tile per slot and list (nA, nNA <= nq <= kThinRows)
      hipLaunchKernelGGL(k_project_thin, dim3((unsigned)(n_tiles(kThinRows) * (e.d_state / kThinCols))),
                         dim3(256), 0, stream, e);
    } else if (blocks > 0) {
      const int64_t chunks = (int64_t)e.H * e.d_state * e.d_v / 8;
      hipLaunchKernelGGL(k_w_tile, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, e);
      if (grouped)
        hipLaunchKernelGGL(k_project_bf16<true>, dim3((unsigned)blocks), dim3(256), lds, stream, e);
      else
        hipLaunchKernelGGL(k_project_bf16<false>, dim3((unsigned)blocks), dim3(256), lds, stream, e);
    }
    if (!grouped && e.HL > 0 && e.nNA > 0 && !e.restore_done)
      hipLaunchKernelGGL(k_restore_copy<uint4>, dim3(e.nNA), dim3(256), 0, stream, e,
                         e.d_state * 2 / 16);
  }
  return hipGetLastError();
}

}  // namespace segmla
