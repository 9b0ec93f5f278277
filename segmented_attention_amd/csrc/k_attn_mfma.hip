// Segment-relocated MLA attention on CDNA4 matrix cores (bf16 MFMA, fp32 accumulation) for
// the packed 512 + 64 latent (RedKnot-MLA paper: relocation paragraph, Eq. 5, and the fused
// consumer paragraph; DeepSeek-V4 latent shape).
//
// Workgroup = 8 wavefronts (two per SIMD) = one tile of 128 query vectors (row, head); every
// query vector shares the same latent rows, so each 32-key tile of the canonical latent is
// staged once in LDS (a ring of three, loaded two tiles ahead) and read by all eight waves.
// Per wave: 16 query vectors (one per lane column of the 16x16x32 MFMA). The query is the
// MFMA B operand in 18 steps of 32 features: steps 0..11 stay in VGPRs, steps 12..17 live in
// per-lane LDS slots (the last two hold the segment-rotated RoPE part). The output
// accumulator O^T [576 features x 16 query vectors] is 36 16x16 fp32 accumulators.
//
// Per segment i with keys visible from the tile: the query's RoPE part is rotated by
// -rot_i (fp32 from an fp64-built table, rounded to bf16), S^T = K Q^T is computed against
// the stored (canonical) latent rows in place, softmax runs online in the log2 domain with
// a lazy rescale (the running max only moves when it grows by more than 8), and O^T += V^T P^T
// with V^T read straight from the same LDS tile by transposing reads. The accumulator is
// kept in the current segment's RoPE frame and moved by R(rot_i - rot_{i+1}) at each
// segment change; R(rot_last) restores the request phase at the end. The single online
// softmax across segments is the running form of the stable log-sum-exp merge of
// per-segment (max, sum, partial output) statistics; key-range splits write their partials
// for the standalone merge.
//
// LDS tile layout (36 KB): a nope region of 32 rows x 64 16-byte chunks (chunk c of row r at
// r*64 + (c ^ fn(r))) followed by a RoPE region of 32 rows x 8 chunks (chunk c of row r at
// r*8 + (c ^ fr(r))). With 64 banks (16 chunk slots per 256 bytes), the 16 consecutive rows a
// 16-lane group reads for the QK^T operand and the 8 rows x 2 chunks a 32-lane half reads for
// the transposed PV operand each land in 16 distinct slots. Each nope row is one
// global->LDS instruction (64 lanes x 16 bytes), so the loader needs no per-chunk addresses.
#include <cmath>
#include "internal.h"

namespace segmla {

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
// The segment table is read-only for the whole launch: reading it through the constant
// address space lets the compiler use scalar loads (no vector-memory round trip, and no
// wait on the vector-memory counter that also tracks the tile prefetch).
typedef const __attribute__((address_space(4))) SegDesc cseg_t;

constexpr int kD = 576, kDN = 512;
constexpr int kKT = 32;                          // keys per LDS tile
constexpr int kNBuf = 3;                         // LDS tile ring
constexpr int kRowBytes = kD * 2;                // 1152 bytes per bf16 latent row
constexpr int kNRow = 1024;                      // LDS bytes per row, nope region
constexpr int kRRow = 128;                       // LDS bytes per row, RoPE region
constexpr int kRBase = kKT * kNRow;              // 32768
constexpr int kTileBytes = kKT * (kNRow + kRRow);  // 36864
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;            // 512
// per-lane LDS slots for query steps kQReg..17 (16 bytes per lane per step)
constexpr int kQReg = 12;                        // query steps kept in VGPRs
constexpr int kQSlotStep = kThreads * 16;        // 8192 bytes per step
constexpr int kQRBase = kNBuf * kTileBytes;      // 110592
constexpr int kLdsBytes = kQRBase + (18 - kQReg) * kQSlotStep;  // 159744
static_assert(kWaves * 16 == kTileQ, "one 16-vector MFMA column block per wave");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;        // log2 units
#ifndef SEGMLA_QK_DEPTH
#define SEGMLA_QK_DEPTH 2
#endif
#ifndef SEGMLA_PV_DEPTH
#define SEGMLA_PV_DEPTH 3
#endif
constexpr int kQkDepth = SEGMLA_QK_DEPTH;        // K fragments in flight ahead of their MFMA
constexpr int kPvDepth = SEGMLA_PV_DEPTH;        // V^T fragment pairs in flight

__device__ __forceinline__ int bitof(int r, int k) { return (r >> k) & 1; }
// nope-region swizzle: a bijection of row bits 0..3 onto the chunk-slot bits
__device__ __forceinline__ int fn(int r) {
  return bitof(r, 3) | (bitof(r, 0) << 1) | (bitof(r, 1) << 2) | (bitof(r, 2) << 3);
}
// RoPE-region swizzle (row bit 0 already selects the half of the 256-byte bank line)
__device__ __forceinline__ int fr(int r) {
  return bitof(r, 3) | (bitof(r, 1) << 1) | (bitof(r, 2) << 2);
}

__device__ __forceinline__ int wave_max_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
// max / sum over the 4 lanes {l, l^16, l^32, l^48} (the lanes holding one query vector)
__device__ __forceinline__ float max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

// OCP E4M3 (float8_e4m3fn) decoding from the format: bias 7, subnormals m * 2^-9,
// S.1111.111 = NaN, no infinity.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 15u, m = c & 7u;
  if (e == 15u && m == 7u) return __int_as_float(0x7fc00000);
  if (e == 0u) {
    const float v = (float)m * 0.001953125f;  // m * 2^-9
    return s ? -v : v;
  }
  return __int_as_float(s | ((e + 120u) << 23) | (m << 20));
}

struct TileIt {
  int seg;      // segment index
  int j0;       // first canonical row of the tile inside the segment
  int nval;     // rows of the tile that are in range (1..kKT)
  int pos0;     // request position of row j0
  int j_end;    // end of the segment's rows inside the key range
  int64_t row0; // latent-pool row of row j0
};

// One 64-lane global->LDS copy of 16 bytes per lane: lane L's bytes from sbase + voff land
// at LDS byte address lds + 16 L. Issued from inline assembly so that the compiler does not
// see an LDS write in flight: it would otherwise wait for the whole prefetch before every
// later LDS read. The consumer orders it explicitly (s_waitcnt vmcnt, then a barrier).
// M0 needs one wait state after the SALU write before the load reads it.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Stage one bf16 tile of up to 32 latent rows with direct global->LDS 16-byte loads: one
// instruction per nope row (wave w takes rows w, w+8, w+16, w+24) and, for waves 0..3, one
// for 8 RoPE rows. Rows past nval repeat the last in-range row (finite; scores masked).
__device__ __forceinline__ void load_tile_bf16(char* buf, const char* tile_src, int nval, int wave,
                                               int lane) {
  const uint32_t base = lds_addr(buf);
#pragma unroll
  for (int n = 0; n < kKT / kWaves; ++n) {
    const int r = wave + kWaves * n;
    const int rr = min(r, nval - 1);
    dma16(tile_src + rr * kRowBytes, (lane * 16) ^ (fn(r) << 4), base + r * kNRow);
  }
  if (wave < kKT / 8) {
    const int r = 8 * wave + (lane >> 3);
    const int rr = min(r, nval - 1);
    dma16(tile_src, rr * kRowBytes + kNRow + (((lane & 7) ^ fr(r)) << 4), base + kRBase + wave * 1024);
  }
}

// Stage one E4M3 tile: codes * block scale -> bf16, RoPE dims copied, written in the same
// layout as the bf16 tile.
__device__ __forceinline__ void load_tile_e4m3(char* buf, const uint8_t* codes, const float* scales,
                                               const __bf16* rope, int64_t row0, int nval, int tid) {
#pragma unroll
  for (int n = 0; n < (kKT * 72 + kThreads - 1) / kThreads; ++n) {
    const int idx = n * kThreads + tid;    // logical (row, chunk)
    if (idx >= kKT * 72) break;
    const int r = idx / 72, c = idx - r * 72;
    const int64_t row = row0 + min(r, nval - 1);
    uint4 v;
    int dst;
    if (c < kDN / 8) {
      const uint2 raw = *(const uint2*)(codes + row * kDN + 8 * c);
      const float sc = scales[row * (kDN / 128) + (c >> 4)];
      __bf16 y[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = (__bf16)(e4m3_to_f32((raw.x >> (8 * k)) & 255u) * sc);
#pragma unroll
      for (int k = 0; k < 4; ++k) y[4 + k] = (__bf16)(e4m3_to_f32((raw.y >> (8 * k)) & 255u) * sc);
      v = *(const uint4*)y;
      dst = r * kNRow + ((c ^ fn(r)) << 4);
    } else {
      v = *(const uint4*)(rope + row * 64 + 8 * (c - kDN / 8));
      dst = kRBase + r * kRRow + (((c - kDN / 8) ^ fr(r)) << 4);
    }
    *(uint4*)(buf + dst) = v;
  }
}

}  // namespace

template <bool VROPE, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void k_attn_mfma(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_tmax[kWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int rank = blockIdx.x / a.n_split, split = blockIdx.x % a.n_split;
  const int tile = a.work[rank];
  if (tile < 0 || tile >= a.map.nF + a.map.nG) return;  // uniform; the work list is a permutation
  int t = -1, h = 0;
  const bool valid = tile_qvec(a.map, tile, wave * 16 + col, t, h);
  if (!valid) t = -1;
  const int t_wmax = wave_max_i(t);
  if (lane == 0) s_tmax[wave] = t_wmax;
  __syncthreads();
  int t_max = s_tmax[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t_max = max(t_max, s_tmax[w]);
  t_max = __builtin_amdgcn_readfirstlane(t_max);
  cseg_t* const sg = (cseg_t*)a.seg;
  int k_lo = 0, k_hi = t_max + 1;
  if (a.n_split > 1) {
    k_lo = split * a.split_keys;
    k_hi = min(k_hi, k_lo + a.split_keys);
  }
  if (k_lo >= k_hi) return;  // uniform over the workgroup

  const float qk_scale = a.sigma * kLog2e;
  const __bf16* qrow = (const __bf16*)a.q + ((int64_t)(valid ? t : 0) * a.map.H + h) * kD;
  // B operand of S^T = K Q^T: lane holds Q[qvec col][32 s + 8 g + 0..7]
  bf16x8 qf[kQReg];
#pragma unroll
  for (int s = 0; s < kQReg; ++s) {
    uint4 v = *(const uint4*)(qrow + 32 * s + 8 * g);
    if (!valid) v = make_uint4(0, 0, 0, 0);
    qf[s] = *(bf16x8*)&v;
  }
  char* const qslot = lds + kQRBase + tid * 16;  // + (s - kQReg) * kQSlotStep
#pragma unroll
  for (int s = kQReg; s < 16; ++s) {
    uint4 v = *(const uint4*)(qrow + 32 * s + 8 * g);
    if (!valid) v = make_uint4(0, 0, 0, 0);
    *(uint4*)(qslot + (s - kQReg) * kQSlotStep) = v;
  }
  constexpr int NF = VROPE ? 36 : 32;  // 16-feature tiles of O^T
  floatx4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int half_r = a.d_rope / 2;  // 32

  // Per-lane LDS byte offsets within a tile buffer.
  // QK^T A operand, tile tau: row 16 tau + col, chunk 4 s + g. For s < 16 the swizzled
  // chunk is 4 (s ^ (fn>>2)) + (g ^ (fn&3)): base qb[s & 3] + 256 (s >> 2); tau adds 16 rows.
  int qb[4];
  {
    const int f = fn(col);
#pragma unroll
    for (int b = 0; b < 4; ++b) qb[b] = (col * 64 + 4 * (b ^ (f >> 2)) + (g ^ (f & 3))) * 16;
  }
  const int qr0 = kRBase + (col * 8 + ((g) ^ fr(col))) * 16;      // s = 16
  const int qr1 = kRBase + (col * 8 + ((4 + g) ^ fr(col))) * 16;  // s = 17
  // PV A operand (V^T via transposing reads): source lane (g, j) supplies row 4 g + j/4
  // (second read: +16 rows) and features 16 f + 4 (j%4) .. +3 -> chunk 2 f + cofs, half j&1.
  const int pr = 4 * g + (col >> 2);
  const int pcofs = (col & 3) >> 1;
  const int pfn = fn(pr);
  const int pb = (pr * 64 + (pcofs ^ (pfn & 1))) * 16 + 8 * (col & 1);
  const int pfh = pfn >> 1;
  const int pfr = fr(pr);
  const int prb = kRBase + pr * 128 + 8 * (col & 1);

  // ---- tile sequence over the key range [k_lo, k_hi), segment-aligned
  auto first_tile = [&](TileIt& c) {
    int lo = 0, hi = a.n_seg - 1;  // last segment starting at or before k_lo
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sg[mid].offset <= k_lo) lo = mid; else hi = mid - 1;
    }
    c.seg = lo;
    const int off = sg[lo].offset, len = sg[lo].len;
    c.j0 = k_lo - off;
    c.j_end = min(len, k_hi - off);
    c.nval = min(kKT, c.j_end - c.j0);
    c.pos0 = k_lo;
    c.row0 = sg[lo].pool_row + c.j0;
  };
  auto advance = [&](const TileIt& c, TileIt& nx) -> bool {
    if (c.j0 + kKT < c.j_end) {
      nx = c;
      nx.j0 = c.j0 + kKT;
      nx.nval = min(kKT, c.j_end - nx.j0);
      nx.pos0 = c.pos0 + kKT;
      nx.row0 = c.row0 + kKT;
      return true;
    }
    if (c.seg + 1 >= a.n_seg) return false;
    const int off = sg[c.seg + 1].offset;
    if (off >= k_hi) return false;
    nx.seg = c.seg + 1;
    nx.j0 = 0;
    nx.j_end = min(sg[c.seg + 1].len, k_hi - off);
    nx.nval = min(kKT, nx.j_end);
    nx.pos0 = off;
    nx.row0 = sg[c.seg + 1].pool_row;
    return true;
  };
  auto issue = [&](const TileIt& c, int b) {
    char* buf = lds + b * kTileBytes;
    if constexpr (FP8)
      load_tile_e4m3(buf, (const uint8_t*)a.kv, a.kv_scale, (const __bf16*)a.kv_rope, c.row0, c.nval, tid);
    else
      load_tile_bf16(buf, (const char*)a.kv + c.row0 * kRowBytes, c.nval, wave, lane);
  };
  // q^r <- R(-rot_i) q^r from the stored query, into the slots of steps 16, 17
  auto rotate_q = [&](int seg) {
#pragma unroll
    for (int s = 16; s < 18; ++s) {
      uint4 v = *(const uint4*)(qrow + 32 * s + 8 * g);
      if (!valid) v = make_uint4(0, 0, 0, 0);
      const bf16x8 x = *(bf16x8*)&v;
      bf16x8 y;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int k = 16 * (s - 16) + 4 * g + p;
        const float2 cs = a.segcs[seg * half_r + k];
        const float x0 = bf2f(x[2 * p]), x1 = bf2f(x[2 * p + 1]);
        y[2 * p] = (__bf16)(x0 * cs.x + x1 * cs.y);
        y[2 * p + 1] = (__bf16)(-x0 * cs.y + x1 * cs.x);
      }
      *(bf16x8*)(qslot + (s - kQReg) * kQSlotStep) = y;
    }
  };
  auto frame_step = [&](int seg, const float2* table) {  // acc^r <- R(angle of table[seg]) acc^r
#pragma unroll
    for (int f = 32; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int k = 8 * (f - 32) + 2 * g + (i >> 1);
        const float2 cs = table[seg * half_r + k];
        const float x = acc[f][i], y = acc[f][i + 1];
        acc[f][i] = x * cs.x - y * cs.y;
        acc[f][i + 1] = x * cs.y + y * cs.x;
      }
  };

  // ---- prologue: tiles 0 and 1 in flight
  TileIt w0, w1, w2;
  first_tile(w0);
  bool v1 = advance(w0, w1);
  issue(w0, 0);
  if (v1) issue(w1, 1);
  rotate_q(w0.seg);
  int cb = 0;  // buffer of tile b
  for (int b = 0;; ++b) {
    // tile b resident (tile b+1 may still be in flight); every wave is done with tile b-1,
    // whose buffer receives tile b+2
    // (a wave has kKT/kWaves nope-row copies per tile in flight, plus one RoPE copy for the
    // first kKT/8 waves; younger loads only make the wait stricter)
    if (!FP8 && v1) {
      if (wave < kKT / 8) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kKT / kWaves + 1) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kKT / kWaves) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    const bool v2 = v1 && advance(w1, w2);
    if (v2) issue(w2, cb == 0 ? 2 : cb - 1);
    const char* buf = lds + cb * kTileBytes;
    __builtin_amdgcn_sched_barrier(0);
    // ---- S^T = K Q^T for keys 16 tau + m (two 16x16 tiles, one accumulation chain each):
    // 36 MFMAs alternating the tiles, K fragments read kQkDepth steps ahead (the issue order
    // is pinned with scheduling groups so the reads stay ahead of their MFMAs)
    floatx4 sacc[2];
    {
      auto kaddr = [&](int k) -> const char* {   // step k: tau = k & 1, s = k >> 1
        const int tau = k & 1, s = k >> 1;
        return s < 16 ? buf + qb[s & 3] + 256 * (s >> 2) + tau * 16 * kNRow
                      : buf + (s == 16 ? qr0 : qr1) + tau * 16 * kRRow;
      };
      // query steps s >= kQReg come from the per-lane slots, read alongside the K fragment of
      // step 2 s (kQkDepth steps ahead of its first use)
      auto qread = [&](int k) { return (k & 1) == 0 && (k >> 1) >= kQReg; };
      sacc[0] = floatx4{0.f, 0.f, 0.f, 0.f};
      sacc[1] = sacc[0];
      bf16x8 ring[kQkDepth], qring[2];
#pragma unroll
      for (int k = 0; k < kQkDepth; ++k) {
        ring[k] = *(const bf16x8*)kaddr(k);
        if (qread(k)) qring[(k >> 1) & 1] = *(const bf16x8*)(qslot + ((k >> 1) - kQReg) * kQSlotStep);
      }
#pragma unroll
      for (int k = 0; k < 36; ++k) {
        const bf16x8 kf = ring[k % kQkDepth];
        const int s = k >> 1;
        const bf16x8 qv = s < kQReg ? qf[s < kQReg ? s : 0] : qring[s & 1];
        if (k + kQkDepth < 36) {
          const int kn = k + kQkDepth;
          ring[k % kQkDepth] = *(const bf16x8*)kaddr(kn);
          if (qread(kn)) qring[(kn >> 1) & 1] = *(const bf16x8*)(qslot + ((kn >> 1) - kQReg) * kQSlotStep);
        }
        sacc[k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qv, sacc[k & 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kQkDepth, 0);  // first reads (no query step yet)
#pragma unroll
      for (int k = 0; k < 36 - kQkDepth; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (qread(k + kQkDepth)) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // K + Q reads
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      // K read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kQkDepth, 0);
    }
    floatx4 s0 = sacc[0], s1 = sacc[1];
    __builtin_amdgcn_sched_barrier(0);
    // lane (g, col): value (tau, i) = key 16 tau + 4 g + i of this tile, query vector col
    const bool need_mask = (w0.pos0 + 31 > t) || (w0.nval < kKT);
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k0 = 4 * g + i, k1 = 16 + 4 * g + i;
        if (w0.pos0 + k0 > t || k0 >= w0.nval) s0[i] = -INFINITY;
        if (w0.pos0 + k1 > t || k1 >= w0.nval) s1[i] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3]))) * qk_scale;
    mx = max4(mx);
    const float m_new = fmaxf(m_run, mx);
    if (__ballot(m_new > m_run + kRescaleThreshold) != 0ull) {  // wave-uniform rescale
      const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[f] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 pf;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // v_exp_f32 directly: results below 2^-126 flush to zero, irrelevant for probabilities
      const float p0 = __builtin_amdgcn_exp2f(s0[i] * qk_scale - m_use);
      const float p1 = __builtin_amdgcn_exp2f(s1[i] * qk_scale - m_use);
      lsum += p0 + p1;
      pf[i] = (__bf16)p0;
      pf[4 + i] = (__bf16)p1;
    }
    l_run += lsum;
    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T P^T (A operand by two transposing reads: keys 4 g + 0..3, 16 + 4 g + 0..3)
    {
      int vx = pfh;
      asm volatile("" : "+v"(vx));  // addresses computed per use, not hoisted into registers
      auto vaddr = [&](int f) -> const char* {
        if (f < 32) return buf + pb + ((f ^ vx) << 5);
        const int c2 = 2 * (f - 32) + pcofs;
        return buf + prb + ((c2 ^ pfr) << 4);
      };
      auto vtau1 = [&](int f) { return f < 32 ? 16 * kNRow : 16 * kRRow; };
      bf16x4 lo[kPvDepth], hi[kPvDepth];
#pragma unroll
      for (int f = 0; f < kPvDepth; ++f) {
        lo[f] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vaddr(f));
        hi[f] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vaddr(f) + vtau1(f)));
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int r = f % kPvDepth;
        const bf16x8 vt = {lo[r][0], lo[r][1], lo[r][2], lo[r][3], hi[r][0], hi[r][1], hi[r][2], hi[r][3]};
        if (f + kPvDepth < NF) {
          lo[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vaddr(f + kPvDepth));
          hi[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vaddr(f + kPvDepth) + vtau1(f + kPvDepth)));
        }
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pf, acc[f], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvDepth, 1);
#pragma unroll
      for (int f = 0; f < NF - kPvDepth; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kPvDepth, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!v1) break;
    if (w1.seg != w0.seg) {  // next tile starts a new segment
      if (VROPE) frame_step(w0.seg, a.stepcs);
      rotate_q(w1.seg);
    }
    w0 = w1;
    w1 = w2;
    v1 = v2;
    cb = cb == kNBuf - 1 ? 0 : cb + 1;
  }

  // restore the request phase of the RoPE part: R(+rot_last)
  if (VROPE) frame_step(w0.seg, a.segcs);
  const float l_tot = sum4(l_run);
  const int d_v = a.d_v;
  if (a.n_split > 1) {
    const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
    const int64_t v = (int64_t)tile * kTileQ + wave * 16 + col;
    float* po = a.part_o + ((int64_t)split * nvec + v) * d_v;
#pragma unroll
    for (int f = 0; f < NF; ++f)
      *(float4*)(po + 16 * f + 4 * g) = make_float4(acc[f][0], acc[f][1], acc[f][2], acc[f][3]);
    if (g == 0) {
      float* pm = a.part_ml + ((int64_t)split * nvec + v) * 2;
      pm[0] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
      pm[1] = l_tot;
    }
    return;
  }
  if (!valid) return;
  const float inv = 1.f / l_tot;
  __bf16* o = (__bf16*)a.out + ((int64_t)t * a.map.H + h) * d_v;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    bf16x4 y = {(__bf16)(acc[f][0] * inv), (__bf16)(acc[f][1] * inv), (__bf16)(acc[f][2] * inv),
                (__bf16)(acc[f][3] * inv)};
    *(bf16x4*)(o + 16 * f + 4 * g) = y;
  }
  if (a.lse && g == 0) a.lse[(int64_t)t * a.map.H + h] = (m_run + log2f(l_tot)) * kLn2;
}

namespace {
template <bool VROPE, bool FP8>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t stream) {
  static bool attr_set = false;
  const int lds = kLdsBytes;
  if (!attr_set) {
    hipError_t r = hipFuncSetAttribute((const void*)k_attn_mfma<VROPE, FP8>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (r != hipSuccess) return r;
    attr_set = true;
  }
  const int64_t blocks = (int64_t)(a.map.nF + a.map.nG) * a.n_split;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_attn_mfma<VROPE, FP8>), dim3((unsigned)blocks), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn(const AttnArgs& a, int kv_dtype, int v_has_rope, hipStream_t stream) {
  if (kv_dtype == 0) return launch_attn_f32(a, stream);
  const bool fp8 = kv_dtype == 2;
  if (v_has_rope) return fp8 ? launch_mfma<true, true>(a, stream) : launch_mfma<true, false>(a, stream);
  return fp8 ? launch_mfma<false, true>(a, stream) : launch_mfma<false, false>(a, stream);
}

}  // namespace segmla
