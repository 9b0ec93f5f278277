// Segment-relocated MLA attention on CDNA4 matrix cores (bf16 MFMA, fp32 accumulation) for
// the packed 512 + 64 latent (RedKnot-MLA paper: relocation paragraph, Eq. 5, and the fused
// consumer paragraph; DeepSeek-V4 latent shape).
//
// Workgroup = 4 wavefronts (one per SIMD, each with the whole 512-entry register file) = one
// tile of 128 query vectors (row, head). Every query vector of the tile shares the same
// latent rows, so each 32-key tile of the canonical latent is staged once in LDS (a ring of
// three buffers) and read by all four waves. Per wave: 32 query vectors, one per lane column
// of the 32x32x16 MFMA, so every K or V^T fragment read from LDS feeds a 32-wide product
// (32 flops per LDS byte). The query is the MFMA B operand in 36 steps of 16 features: steps
// 0..kQReg-1 stay in registers, the rest (including the four segment-rotated RoPE steps)
// live in per-lane LDS slots. The output accumulator O^T [576 features x 32 query vectors]
// is 18 32x32 fp32 accumulators.
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
// Register files: the 16 nope output tiles (256 values per lane) fill the AGPRs; their MFMAs
// are issued from inline assembly with AGPR accumulators, everything else (query, scores,
// RoPE output tiles) stays in VGPRs with the compiler's MFMAs in VGPR form. Hazards of the
// assembly MFMAs are covered by hand: two wait states before the first of each tile's value
// product (operands written by the vector ALU; the others read LDS results only, which a CPU
// test checks on the generated assembly), twelve before the accumulators are read back after
// the loop.
//
// The key loop is software pipelined: while the softmax of tile i runs on the vector ALU,
// the matrix core computes S^T of tile i+1; then O^T += V^T P^T for tile i. A wave therefore
// holds two key tiles in LDS, and a third is in flight. The loop body runs six times per trip
// (three tile buffers, two score tiles), so buffers and roles are fixed per copy, and the rare
// per-tile work (query rotation and output
// frame step at a segment change, masking of partial tiles, accumulator rescale) is marked
// unlikely, so the common iteration runs straight through: with one wave per SIMD, every
// taken branch is a fetch bubble in front of the matrix core. For the same reason every
// instruction costs the wave an issue slot, and about four fit in the shadow of one score
// MFMA next to its operand read: the softmax is cut into slices of that size, one per score
// step (maxima, rescale test, one exponential per step, then one packed pair per step, the
// row sum last).
//
// LDS tile layout (36 KB): a nope region of 32 rows x 64 16-byte chunks (chunk c of row r at
// r*64 + (c ^ fn(r))) followed by a RoPE region of 32 rows x 8 chunks (chunk c of row r at
// r*8 + (c ^ fr(r))). With 64 banks (16 chunk slots per 256 bytes): the K operand read (16
// consecutive rows, one chunk each, per 16 lanes) and the transposing V^T read (4 rows x 4
// chunks per 32 lanes) both land in 16 distinct slots. Each nope row is one global->LDS
// instruction (64 lanes x 16 bytes), so the loader needs no per-chunk addresses.
#include <cmath>
#include "internal.h"
#include "lds_tile.h"

namespace segmla {

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attn_f32_window(const AttnArgs& a, hipStream_t stream);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
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
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;            // 256
constexpr int kQSteps = kD / 16;                 // 36 query steps of 16 features
#ifndef SEGMLA_QREG
#define SEGMLA_QREG 24
#endif
constexpr int kQReg = SEGMLA_QREG;               // query steps kept in registers
constexpr int kQSlotStep = kThreads * 16;        // 4096 bytes per step
constexpr int kQRBase = kNBuf * kTileBytes;      // 110592
constexpr int kLdsBytes = kQRBase + (kQSteps - kQReg) * kQSlotStep;
constexpr int kLoads = kKT / kWaves + 1;         // global->LDS copies per wave per tile
static_assert(kWaves * 32 == kTileQ, "one 32-vector MFMA column block per wave");
static_assert(kKT / 8 == kWaves, "one RoPE copy (8 rows) per wave");
static_assert(kQReg <= 32, "the RoPE query steps live in LDS slots");
constexpr int kLdsAlloc = kLdsBytes + 16;       // + the per-wave maxima of the prologue
static_assert(kLdsAlloc <= 160 * 1024, "LDS budget");
static_assert(kTileBytes % 256 == 0, "tile buffers keep address bits 0..7 free");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;        // log2 units
#ifndef SEGMLA_QK_DEPTH
#define SEGMLA_QK_DEPTH 3
#endif
#ifndef SEGMLA_PV_DEPTH
#define SEGMLA_PV_DEPTH 4
#endif
constexpr int kQkDepth = SEGMLA_QK_DEPTH;        // K fragments in flight ahead of their MFMA
constexpr int kPvDepth = SEGMLA_PV_DEPTH;        // V^T fragments in flight

__device__ __forceinline__ int wave_max_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
// sum over the lanes l and l ^ 32 (the two lanes holding one query vector): the swap returns
// (own, partner) in the low half and (partner, own) in the high half
__device__ __forceinline__ float pair_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

// max(a, b, c) in one instruction (v_maximum3_f32). fmaxf on values the compiler cannot prove
// canonical (such as MFMA results) costs two extra canonicalising instructions; the IEEE
// maximum propagates NaN instead and needs none (scores are never NaN).
__device__ __forceinline__ float max3r(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
// Two probabilities rounded to bf16 (round to nearest even) and packed, low half first. A
// volatile statement, so that it stays in the score step it is written in (a plain conversion
// is sunk to the value product, after the last score step).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  uint32_t w;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(w) : "v"(lo), "v"(hi));
  return w;
}

// Nope output tiles live in AGPRs ("a" constraints). Inside the key loop only inline
// assembly touches them, so the register allocator keeps them there; vector-ALU work on them
// goes through single-register operands.

// acc += A B (32x32x16 bf16, fp32 accumulation). With kWait, an s_nop gives the two wait
// states an operand written by the vector ALU needs before the MFMA reads it. Without it,
// the caller's operands come from LDS reads and earlier MFMAs only; a CPU test checks on the
// generated assembly that no vector-ALU write of an operand falls within two wait states.
template <bool kWait>
__device__ __forceinline__ void mfma_agpr(floatx16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (kWait)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// acc *= alpha, register by register through one VGPR; the leading s_nops give the twelve
// wait states an MFMA result needs before it is read
__device__ __forceinline__ void rescale_agpr(floatx16& acc, float alpha) {
  float e[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) e[i] = acc[i];
  float tmp;
#define SEGMLA_RS1(n) "v_accvgpr_read_b32 %16, %" #n "\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %" #n ", %16\n\t"
  asm volatile("s_nop 7\n\ts_nop 3\n\t" SEGMLA_RS1(0) SEGMLA_RS1(1) SEGMLA_RS1(2) SEGMLA_RS1(3) SEGMLA_RS1(4)
               SEGMLA_RS1(5) SEGMLA_RS1(6) SEGMLA_RS1(7) SEGMLA_RS1(8) SEGMLA_RS1(9) SEGMLA_RS1(10)
               SEGMLA_RS1(11) SEGMLA_RS1(12) SEGMLA_RS1(13) SEGMLA_RS1(14) SEGMLA_RS1(15)
               : "+a"(e[0]), "+a"(e[1]), "+a"(e[2]), "+a"(e[3]), "+a"(e[4]), "+a"(e[5]), "+a"(e[6]),
                 "+a"(e[7]), "+a"(e[8]), "+a"(e[9]), "+a"(e[10]), "+a"(e[11]), "+a"(e[12]),
                 "+a"(e[13]), "+a"(e[14]), "+a"(e[15]), "=&v"(tmp)
               : "v"(alpha));
#undef SEGMLA_RS1
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = e[i];
}

// twelve wait states after the last MFMA on the tiles, before they are read back
__device__ __forceinline__ void settle_agpr(floatx16* acc) {
  asm volatile("s_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int f = 0; f < 16; ++f) asm volatile("" : "+a"(acc[f]));
}


template <int N>
struct IntC {
  static constexpr int value = N;
};

struct TileIt {  // assigned field by field: a whole-struct copy between the rotating roles
                 // made the compiler keep descriptors in private memory
  int v;        // the tile exists (the key range is not exhausted)
  int seg;      // segment index
  int nval;     // rows of the tile that are in range (1..kKT)
  int pos0;     // request position of the tile's first row
  int pend;     // end (exclusive) of the segment's positions inside the key range
  int64_t src;  // the tile's first row: bf16 latent, byte offset in the pool; E4M3, its row;
                // listed entries: pool row - id of the segment's entries
  int ph;       // decode kernel over two pools: 0 raw keys, 1 compressed entries
  int cur;      // compressed entries: id of the first (all available) or list position (lists)
  int lo;       // listed entries: lane of the first id in the step's id vector
};

// Stage one bf16 tile of up to 32 latent rows with direct global->LDS 16-byte copies: one
// per nope row (wave w takes rows w, w+4, ..., w+28) and one for 8 RoPE rows (rows 8w..8w+7).
// Rows past nval repeat the last in-range row (finite; their scores are masked).
__device__ __forceinline__ void load_tile_bf16(char* buf, const char* tile_src, int nval, int wave) {
  const uint32_t base = lds_addr(buf);
  // lane id recomputed here: per-lane offsets live only as long as the copies that use them,
  // and are never spilled (a spill reload would wait on vmcnt, which also counts these copies)
  const int lane = lane_id();
#pragma unroll
  for (int n = 0; n < kKT / kWaves; ++n) {
    const int r = wave + kWaves * n;
    const int rr = min(r, nval - 1);
    dma16(tile_src + rr * kRowBytes, (lane * 16) ^ (fn(r) << 4), base + r * kNRow);
  }
  const int r = 8 * wave + (lane >> 3);
  const int rr = min(r, nval - 1);
  dma16(tile_src, rr * kRowBytes + kNRow + (((lane & 7) ^ fr(r)) << 4), base + kRBase + wave * 1024);
}

// Full tiles (nval == kKT, every tile but a segment's last) with few instructions per copy:
// with one wave per SIMD each instruction costs the wave an issue slot, and the clamped
// per-row addressing above takes about twelve per row. Wave w copies nope rows r = w + 4 n:
// fn(r) = 4 w + (n & 3), so lane L reads source bytes r * 1152 + 16 (L ^ fn(r)) =
// (lw ^ 16 (n & 3)) + 4608 n with lw = 16 (L ^ 4 w) + 1152 w (1152 w has no bits below 128,
// so adding it commutes with an xor of bits 4 and 5).
// One row: M0 = lds + 4096 N, lane offset vb + 4608 N. The vector add is also the wait state
// the copy needs after the M0 write.
template <int N>
__device__ __forceinline__ void dma16_row(const char* src, uint32_t vb, uint32_t lds) {
  uint32_t t;
  asm volatile("s_add_u32 m0, %2, %3\n\tv_add_u32 %0, %4, %1\n\tglobal_load_lds_dwordx4 %0, %5"
               : "=&v"(t)
               : "v"(vb), "s"(lds), "n"(N * kWaves * kNRow), "n"(N * kWaves * kRowBytes), "s"(src)
               : "memory", "m0", "scc");
}
__device__ __forceinline__ void load_tile_bf16_full(char* buf, const char* tile_src, int wave) {
  const int lane = lane_id();
  const uint32_t lb = lds_addr(buf) + wave * kNRow;
  const uint32_t lw = (uint32_t)(((lane ^ (wave << 2)) << 4) + wave * kRowBytes);
  const uint32_t vb1 = lw ^ 16, vb2 = lw ^ 32, vb3 = lw ^ 48;
  dma16(tile_src, lw, lb);
  dma16_row<1>(tile_src, vb1, lb);
  dma16_row<2>(tile_src, vb2, lb);
  dma16_row<3>(tile_src, vb3, lb);
  dma16_row<4>(tile_src, lw, lb);
  dma16_row<5>(tile_src, vb1, lb);
  dma16_row<6>(tile_src, vb2, lb);
  dma16_row<7>(tile_src, vb3, lb);
  const int r = 8 * wave + (lane >> 3);
  dma16(tile_src, r * kRowBytes + kNRow + (((lane & 7) ^ fr(r)) << 4), lds_addr(buf) + kRBase + wave * 1024);
}
static_assert(kKT / kWaves == 8 && kWaves == 4, "row n of wave w is w + 4 n, n = 0..7");

// E4M3 tiles are staged raw inside their own bf16 buffer and converted in place once per
// tile: the codes (32 rows x 512 bytes) sit where nope rows 16..31 will go, the block scales
// (32 rows x 4 fp32) in the last KB below them, and the RoPE rows (bf16) are copied straight
// to their final place in the RoPE region.
constexpr int kRawCodes = 16 * kNRow;          // 16384
constexpr int kRawScales = kRawCodes - 1024;   // 15360
// Copies of wave `wave`: code row pairs wave + 4 m (m = 0..3, 64 lanes = 2 rows x 512 bytes),
// its 8 RoPE rows, and (wave 0) the scales of all 32 rows (lanes 32..63 write a duplicate).
__device__ __forceinline__ void load_tile_e4m3(char* buf, const uint8_t* codes, const float* scales,
                                               const __bf16* rope, int64_t row0, int nval, int wave) {
  const uint32_t base = lds_addr(buf);
  const int lane = lane_id();
  const char* cbase = (const char*)codes + row0 * kDN;
#pragma unroll
  for (int m = 0; m < kKT / 2 / kWaves; ++m) {
    const int pr = wave + kWaves * m;
    const int rr = min(2 * pr + (lane >> 5), nval - 1);
    dma16(cbase, rr * kDN + 16 * (lane & 31), base + kRawCodes + pr * 1024);
  }
  const int r = 8 * wave + (lane >> 3);
  const int rr = min(r, nval - 1);
  dma16((const char*)rope + row0 * 128, rr * 128 + (((lane & 7) ^ fr(r)) << 4), base + kRBase + wave * 1024);
  if (wave == 0) {
    const int rs = min(lane & 31, nval - 1);
    dma16((const char*)scales + row0 * 16, rs * 16, base + kRawScales);
  }
}
static_assert(kKT / 2 % kWaves == 0, "whole code-row pairs per wave");

// In-place conversion of a staged E4M3 tile to the bf16 tile layout, by all threads: each
// takes 4 chunks of 16 codes (row r, codes 16 j .. 16 j + 15, block scale j / 8), reads them
// all, waits for every thread to have read, then writes 2 bf16 chunks per code chunk.
// Hardware conversion of packed E4M3 pairs to fp32, times the block scale, rounded to bf16.
__device__ __forceinline__ void convert_tile_e4m3(char* buf, int wave) {
  const int tid = wave * 64 + lane_id();  // recomputed here: no offsets kept live across the loop
  uint4 raw[4];
  float sc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int c = tid + kThreads * n, r = c >> 5, j = c & 31;
    raw[n] = *(const uint4*)(buf + kRawCodes + r * kDN + 16 * j);
    sc[n] = *(const float*)(buf + kRawScales + r * 16 + 4 * (j >> 3));
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int c = tid + kThreads * n, r = c >> 5, j = c & 31;
    const uint32_t wds[4] = {raw[n].x, raw[n].y, raw[n].z, raw[n].w};
    bf16x8 y[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      typedef float f2 __attribute__((ext_vector_type(2)));
      const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wds[q], false);
      const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(wds[q], true);
      y[q >> 1][4 * (q & 1) + 0] = (__bf16)(lo[0] * sc[n]);
      y[q >> 1][4 * (q & 1) + 1] = (__bf16)(lo[1] * sc[n]);
      y[q >> 1][4 * (q & 1) + 2] = (__bf16)(hi[0] * sc[n]);
      y[q >> 1][4 * (q & 1) + 3] = (__bf16)(hi[1] * sc[n]);
    }
    const int f = fn(r);
    *(bf16x8*)(buf + r * kNRow + (((2 * j) ^ f) << 4)) = y[0];
    *(bf16x8*)(buf + r * kNRow + (((2 * j + 1) ^ f) << 4)) = y[1];
  }
  __syncthreads();
}
static_assert(kKT * (kDN / 16) == 4 * kThreads, "4 code chunks per thread");

// Replacement of the Local heads' state on the window's rows outside A (RedKnot-MLA paper,
// protected-row paragraph: cached values are replaced, never added to): workgroup `wg` copies
// rows [wg * rc_rows, (wg + 1) * rc_rows) of the window's complement list, z[t][lhead[l]] =
// z_cached[pool_row(t)][l] bit for bit. The attention's registers are still free here; each
// thread keeps kRcBatch 16-byte loads in flight before their stores.
constexpr int kRcBatch = 8;  // loads in flight per thread (v0 .. v7 below)
__device__ __forceinline__ void restore_slice(const AttnArgs& a, int wg) {
  const int na0 = a.map.rng[2], n = a.map.rng[3] - na0;
  const int r0 = wg * a.rc_rows;
  const int r1 = min(n, r0 + a.rc_rows);
  const int per_row = a.HL * a.z_chunks;  // 16-byte chunks of one row's Local state
  const uint4* zc = (const uint4*)a.z_cached;
  uint4* z = (uint4*)a.z;
  for (int r = r0; r < r1; ++r) {
    const int t = a.map.nalist[na0 + r];
    const SegDesc sd = a.seg[a.seg_of_row[t]];
    const uint4* src = zc + (sd.pool_row + (t - sd.offset)) * a.HL * a.z_chunks;
    uint4* dst = z + (int64_t)(t - a.q0) * a.map.H * a.z_chunks;
    // kRcBatch loads in flight per thread (named values: they stay in registers), then stores
    auto ld = [&](int e) __attribute__((always_inline)) { return src[min(e, per_row - 1)]; };
    auto st = [&](int e, const uint4& v) __attribute__((always_inline)) {
      if (e < per_row) {
        const int l = e / a.z_chunks;
        dst[a.lhead[l] * a.z_chunks + (e - l * a.z_chunks)] = v;
      }
    };
    for (int e0 = threadIdx.x; e0 < per_row; e0 += kThreads * kRcBatch) {
      const uint4 v0 = ld(e0), v1 = ld(e0 + kThreads), v2 = ld(e0 + 2 * kThreads),
                  v3 = ld(e0 + 3 * kThreads), v4 = ld(e0 + 4 * kThreads), v5 = ld(e0 + 5 * kThreads),
                  v6 = ld(e0 + 6 * kThreads), v7 = ld(e0 + 7 * kThreads);
      st(e0, v0);
      st(e0 + kThreads, v1);
      st(e0 + 2 * kThreads, v2);
      st(e0 + 3 * kThreads, v3);
      st(e0 + 4 * kThreads, v4);
      st(e0 + 5 * kThreads, v5);
      st(e0 + 6 * kThreads, v6);
      st(e0 + 7 * kThreads, v7);
    }
  }
}

}  // namespace

// WIN: the W tiles (sink + window heads), one workgroup per tile in order: the key walk
// covers the sink [0, min(n_sink, lo)) and the window [lo, t_max] with lo = max(0, t_min - win)
// over the tile's rows, skips the keys between them, and masks per query vector the keys
// below its own window (RedKnot explainer, "Insight 1": W(i) = S_sink U [i - w, i]).
template <bool VROPE, bool FP8, bool WIN>
__global__ __launch_bounds__(kThreads, 1) void k_attn_mfma(AttnArgs a) {
  // The kernel has no static LDS, so the dynamic area, and with it every tile buffer, starts
  // on a 256-byte boundary: the operand addresses below rely on it.
  extern __shared__ __attribute__((aligned(256))) char lds[];
  int* const s_tmax = (int*)(lds + kLdsBytes);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  if (!WIN && a.rc_rows > 0) restore_slice(a, blockIdx.x);  // every workgroup, before any exit
  const int rank = WIN ? (int)blockIdx.x : (int)blockIdx.x / a.n_split;
  const int split = WIN ? 0 : (int)blockIdx.x % a.n_split;
  const int tile = WIN ? a.map.nF + a.map.nG + rank : a.work[rank];
  // uniform; the work list is a permutation of the F and G tiles
  if (tile < 0 || tile >= a.map.nF + a.map.nG + (WIN ? a.map.nW : 0)) return;
  int t = -1, h = 0;
  const bool valid = tile_qvec(a.map, tile, wave * 32 + col, t, h);
  if (!valid) t = -1;
  const int t_wmax = wave_max_i(t);
  if (lane == 0) s_tmax[wave] = t_wmax;
  __syncthreads();
  int t_max = max(max(s_tmax[0], s_tmax[1]), max(s_tmax[2], s_tmax[3]));
  t_max = __builtin_amdgcn_readfirstlane(t_max);
  cseg_t* const sg = (cseg_t*)a.seg;
  int k_lo = 0, k_hi = t_max + 1;
  // WIN: keys [g_lo, g_hi) lie between the sink and the window of every row of the tile
  int g_lo = 0, g_hi = 0;
  if (WIN) {
    const int lo = max(0, wtile_min_row(a.map, tile) - a.win);
    const int sink_end = min(a.n_sink, lo);
    if (sink_end > 0) {
      g_lo = sink_end;
      g_hi = lo;
    } else {
      k_lo = lo;
    }
  } else if (a.n_split > 1) {
    k_lo = split * a.split_keys;
    k_hi = min(k_hi, k_lo + a.split_keys);
  }
  if (k_lo >= k_hi) return;  // uniform over the workgroup

  const float qk_scale = a.sigma * kLog2e;
  const __bf16* qrow = (const __bf16*)a.q + ((int64_t)(valid ? t - a.q0 : 0) * a.map.H + h) * kD;
  // B operand of S^T = K Q^T, step s: lane holds Q[qvec col][16 s + 8 hf + 0..7]; steps below
  // kQReg in registers, the others in per-thread LDS slots (loaded in the prologue)
  bf16x8 qf[kQReg];
  char* const qslot = lds + kQRBase + tid * 16;  // + (s - kQReg) * kQSlotStep
  constexpr int NF = VROPE ? 18 : 16;  // 32-feature tiles of O^T
  constexpr int NR = NF - 16;          // RoPE output tiles (VGPRs)
  floatx16 acc[16], accr[NR > 0 ? NR : 1];  // nope tiles in AGPRs, RoPE tiles in VGPRs
#pragma unroll
  for (int f = 0; f < 16; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[f][i] = 0.f;
#pragma unroll
  for (int f = 0; f < NR; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) accr[f][i] = 0.f;
  // running max (log2 units), the shift the exponentials use (0 while no key is visible) and
  // the threshold of the lazy rescale
  float m_run = -INFINITY, l_run = 0.f, m_use = 0.f, m_thr = -INFINITY;
  const int half_r = a.d_rope / 2;  // 32

  // ---- per-lane LDS offsets inside a tile buffer. Each is a base B plus a swizzle term X ^ C,
  // where C is a per-step constant and B has no bits where X and C live; with the buffer
  // start on a 256-byte boundary, buffer + B + (X ^ C) = (buffer + (B | X)) ^ C, one XOR per
  // read (the remaining per-step term goes into the instruction's offset field).
  // K operand, step s (nope): row col, chunk 2 s + hf -> 2 s ^ (fn & 14) | (hf ^ (fn & 1))
  const int fcol = fn(col), rcol = fr(col);
  const int kx0 = (col * kNRow + 16 * (hf ^ (fcol & 1))) | (16 * (fcol & 14));  // C = 32 (s & 7)
  // K operand, RoPE step 32 + j: row col, RoPE chunk 2 j + hf
  const int krx0 = (kRBase + col * kRRow + 16 * (hf ^ (rcol & 1))) | (16 * (rcol & 6));  // C = 32 j
  // V^T operand (transposing reads): 16-lane group G, source lane j supplies key row
  // 16 u + 4 (G >> 1) + (j >> 2) (+ 8 for the second read) and features
  // 32 f + 16 (G & 1) + 4 (j & 3) .. + 3, i.e. chunk 4 f + cl, half j & 1. C = 64 (f & 3).
  const int G = lane >> 4, jj = lane & 15;
  const int cl = 2 * (G & 1) + ((jj & 3) >> 1);
  const int vrow = 4 * (G >> 1) + (jj >> 2);
  const int vx0 = (vrow * kNRow + 8 * (jj & 1) + 16 * (cl ^ (G >> 1))) | (64 * (jj >> 2));
  const int vx1 = (vrow * kNRow + 8 * (jj & 1) + 16 * (cl ^ ((G >> 1) | 2))) | (64 * (jj >> 2));
  // RoPE features (f = 16, 17): C = 64 (f - 16)
  const int vrx0 = (kRBase + vrow * kRRow + 8 * (jj & 1) + 16 * (cl ^ (G >> 1))) | (64 * ((jj >> 3) & 1));
  const int vrx1 = (kRBase + vrow * kRRow + 8 * (jj & 1) + 16 * (cl ^ ((G >> 1) | 2))) | (64 * ((jj >> 3) & 1));

  // ---- tile sequence over the key range [k_lo, k_hi), segment-aligned
  constexpr int64_t kSrcStride = FP8 ? 1 : kRowBytes;  // TileIt::src units per latent row
  // end of the key range that position `pos` belongs to (WIN: the sink ends at the gap)
  auto range_end = [&](int pos) __attribute__((always_inline)) -> int {
    return (WIN && pos < g_lo && g_lo < g_hi) ? g_lo : k_hi;
  };
  auto first_tile = [&](TileIt& c) __attribute__((always_inline)) {
    const int lo = a.seg_of_row[k_lo];  // k_lo < k_hi <= T
    c.seg = lo;
    const int off = sg[lo].offset, len = sg[lo].len;
    c.pos0 = k_lo;
    c.pend = min(off + len, range_end(k_lo));
    c.nval = min(kKT, c.pend - k_lo);
    c.src = (sg[lo].pool_row + (k_lo - off)) * kSrcStride;
  };
  auto advance = [&](const TileIt& c, TileIt& nx) __attribute__((always_inline)) -> bool {
    if (__builtin_expect(c.pos0 + kKT < c.pend, 1)) {
      nx.seg = c.seg;
      nx.pos0 = c.pos0 + kKT;
      nx.pend = c.pend;
      nx.nval = min(kKT, c.pend - nx.pos0);
      nx.src = c.src + kKT * kSrcStride;
      return true;
    }
    if (WIN && c.pend == g_lo && g_lo < g_hi) {  // the sink is done: jump to the window
      if (g_hi >= k_hi) return false;
      typedef const __attribute__((address_space(4))) int32_t cint_t;
      const int ns = ((cint_t*)a.seg_of_row)[g_hi];  // uniform: a scalar load
      const int off = sg[ns].offset;
      nx.seg = ns;
      nx.pos0 = g_hi;
      nx.pend = min(off + sg[ns].len, k_hi);
      nx.nval = min(kKT, nx.pend - g_hi);
      nx.src = (sg[ns].pool_row + (g_hi - off)) * kSrcStride;
      return true;
    }
    if (c.seg + 1 >= a.n_seg) return false;
    const int off = sg[c.seg + 1].offset;  // the segments are contiguous: off == c.pend
    if (off >= k_hi) return false;
    nx.seg = c.seg + 1;
    nx.pos0 = off;
    nx.pend = min(off + sg[c.seg + 1].len, range_end(off));
    nx.nval = min(kKT, nx.pend - off);
    nx.src = sg[c.seg + 1].pool_row * kSrcStride;
    return true;
  };
  auto issue = [&](const TileIt& c, int b) __attribute__((always_inline)) {
    char* buf = lds + b * kTileBytes;
    if constexpr (FP8)
      load_tile_e4m3(buf, (const uint8_t*)a.kv, a.kv_scale, (const __bf16*)a.kv_rope, c.src, c.nval, wave);
    else if (__builtin_expect(c.nval == kKT, 1))
      load_tile_bf16_full(buf, (const char*)a.kv + c.src, wave);
    else
      load_tile_bf16(buf, (const char*)a.kv + c.src, c.nval, wave);
  };
  // q^r <- R(-rot_i) q^r from the stored query, into the slots of steps 32..35
  auto rotate_q = [&](int seg) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 32; s < 36; ++s) {
      uint4 v = *(const uint4*)(qrow + 16 * s + 8 * hf);
      if (!valid) v = make_uint4(0, 0, 0, 0);
      const bf16x8 x = *(bf16x8*)&v;
      bf16x8 y;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int k = 8 * (s - 32) + 4 * hf + p;
        const float2 cs = a.segcs[seg * half_r + k];
        const float x0 = bf2f(x[2 * p]), x1 = bf2f(x[2 * p + 1]);
        y[2 * p] = (__bf16)(x0 * cs.x + x1 * cs.y);
        y[2 * p + 1] = (__bf16)(-x0 * cs.y + x1 * cs.x);
      }
      *(bf16x8*)(qslot + (s - kQReg) * kQSlotStep) = y;
    }
  };
  // acc^r <- R(angle of table[seg]) acc^r; O^T tile f, register i: feature
  // 32 f + 8 (i >> 2) + 4 hf + (i & 3), so registers i, i + 1 (i even) hold one RoPE pair
  auto frame_step = [&](int seg, const float2* table, float sgn = 1.f) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < NR; ++f) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int k = 16 * f + 4 * (i >> 2) + 2 * hf + ((i & 3) >> 1);
        float2 cs = table[seg * half_r + k];
        cs.y *= sgn;  // -1: the inverse rotation
        const float x = accr[f][i], y = accr[f][i + 1];
        accr[f][i] = fmaf(x, cs.x, -(y * cs.y));  // explicit contraction: fixed rounding
        accr[f][i + 1] = fmaf(x, cs.y, y * cs.x);
      }
      asm volatile("" ::: "memory");  // one tile's table entries at a time (register peak)
    }
  };

  // S^T of one tile (buffer nb) into sacc. With softmax work (sm != nullptr), that work is
  // interleaved with the MFMAs: the matrix core computes the next tile's scores while the
  // vector ALU finishes the current tile's probabilities.
  auto qk_reads = [&](uint32_t kt, uint32_t krt, int k, bf16x8& kf) __attribute__((always_inline)) {
    if (k < 32) {
      const int s8 = k >> 3, sl = k & 7;
      kf = *(const lds_bf16x8*)(size_t)((kt ^ (32 * sl)) + 256 * s8);
    } else {
      kf = *(const lds_bf16x8*)(size_t)(krt ^ (32 * (k - 32)));
    }
  };

  floatx16 S;
  // S^T of one tile (buffer buf) into sacc, one MFMA per 16-feature step; the K fragment of
  // step k + kQkDepth is read before the MFMA of step k, and hook(k) places a slice of
  // vector-ALU work after it (program order is issue order: each step ends in a fence)
  auto qk_tile = [&](const char* buf, floatx16& sacc, auto&& hook) __attribute__((always_inline)) {
    // per-tile bases, opaque to the compiler: the per-step XORs stay XORs of this value (no
    // per-step addresses precomputed and held across the loop)
    uint32_t kt = lds_addr(buf) + kx0, krt = lds_addr(buf) + krx0;
    asm volatile("" : "+v"(kt), "+v"(krt));
    bf16x8 ring[kQkDepth], qring[kQkDepth];
#pragma unroll
    for (int k = 0; k < kQkDepth; ++k) {
      qk_reads(kt, krt, k, ring[k]);
      if (k >= kQReg) qring[k] = *(const bf16x8*)(qslot + (k - kQReg) * kQSlotStep);
    }
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
      const bf16x8 kf = ring[k % kQkDepth];
      const bf16x8 qv = k < kQReg ? qf[k < kQReg ? k : 0] : qring[k % kQkDepth];
      if (k + kQkDepth < kQSteps) {
        const int kn = k + kQkDepth;
        qk_reads(kt, krt, kn, ring[k % kQkDepth]);
        if (kn >= kQReg) qring[k % kQkDepth] = *(const bf16x8*)(qslot + (kn - kQReg) * kQSlotStep);
      }
      if (k == 0) {
        const floatx16 zero = {};
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv, zero, 0, 0, 0);
      } else {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv, sacc, 0, 0, 0);
      }
      hook(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: tiles 0 and 1 in flight, then the query (its loads overlap the copies),
  // scores of tile 0
  TileIt wa, wb, wc;
  first_tile(wa);
  wa.v = 1;
  wb.v = advance(wa, wb);
  issue(wa, 0);
  if (wb.v) issue(wb, 1);
#pragma unroll
  for (int s = 0; s < kQReg; ++s) {
    uint4 v = *(const uint4*)(qrow + 16 * s + 8 * hf);
    if (!valid) v = make_uint4(0, 0, 0, 0);
    qf[s] = *(bf16x8*)&v;
  }
#pragma unroll
  for (int s = kQReg; s < 32; ++s) {
    uint4 v = *(const uint4*)(qrow + 16 * s + 8 * hf);
    if (!valid) v = make_uint4(0, 0, 0, 0);
    *(uint4*)(qslot + (s - kQReg) * kQSlotStep) = v;
  }
  rotate_q(wa.seg);
  if (!FP8 && wb.v) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (FP8) convert_tile_e4m3(lds, wave);
  qk_tile(lds, S, [](int) {});
  __builtin_amdgcn_sched_barrier(0);
  floatx16 Sn;
  int fin_seg = 0;  // segment of the last tile
  // One iteration per key tile i: tile i in buffer CB with descriptor w0 and raw scores Sc,
  // tile i+1 (w1, buffer CB+1) gets its scores into Sx, tile i+2 (w2, buffer CB+2) is staged.
  // The loop below is unrolled six times, so that the buffers (period 3), the descriptor
  // roles (period 3) and the score registers (period 2) are all fixed per copy: no index
  // arithmetic and no descriptor or score copies between iterations.
  auto iteration = [&](auto cbc, floatx16& Sc, floatx16& Sx, const TileIt& w0, const TileIt& w1,
                       TileIt& w2) __attribute__((always_inline)) -> bool {
    constexpr int cb = decltype(cbc)::value;
    constexpr int nb = (cb + 1) % kNBuf, fb = (cb + 2) % kNBuf;
    // every wave is done with tile i-1, whose buffer (fb) receives tile i+2; tile i+1 is
    // resident
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool v1 = w1.v;
    w2.v = v1 && advance(w1, w2);
    const bool v2 = w2.v;
    if constexpr (FP8) {  // tile i+1 arrived raw: convert it in place
      if (v1) convert_tile_e4m3(lds + nb * kTileBytes, wave);
    }
    // a new segment's query rotation reads the stored query and the RoPE table before the next
    // copy is issued: vector loads retire in order, so behind the copy they would wait for the
    // whole tile to land. (E4M3: after the copy. Next to the in-place conversion the earlier
    // rotation made the register allocator spill.)
    if constexpr (!FP8) {
      if (__builtin_expect(v1 && w1.seg != w0.seg, 0) && sg[w1.seg].frame != sg[w0.seg].frame)
        rotate_q(w1.seg);
    }
    if (__builtin_expect(v2, 1)) issue(w2, fb);
    if constexpr (FP8) {
      if (__builtin_expect(v1 && w1.seg != w0.seg, 0) && sg[w1.seg].frame != sg[w0.seg].frame)
        rotate_q(w1.seg);
    }
    // causal / range mask of tile i: register i of lane (hf, col) is key 8 (i >> 2) + 4 hf + (i & 3);
    // WIN: also the keys below the query vector's window that are not sink keys
    if (__builtin_expect(__ballot((w0.pos0 + kKT - 1 > t) || (w0.nval < kKT) ||
                                  (WIN && w0.pos0 < t - a.win)) != 0ull, 0)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = 8 * (i >> 2) + 4 * hf + (i & 3);
        const int p = w0.pos0 + k;
        if (p > t || k >= w0.nval || (WIN && p >= a.n_sink && p < t - a.win)) Sc[i] = -INFINITY;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // softmax of tile i (online, log2 domain, lazy rescale), in slices that ride along the
    // MFMAs of the next tile's scores, a few instructions per step: partial maxima, the pair
    // maximum and the rescale test, the rescale itself (rare, out of line), one probability
    // per step, then one packed pair and its two row-sum terms per step
    constexpr int kSmSteps = 36;
    uint32_t pw[8];
    float alpha, lsum = 0.f, lsum2, mx = 0.f;  // alpha is set and read only when resc
    float pmx[4], p[16];
    bool resc = false;
    auto softmax_step = [&](int k) __attribute__((always_inline)) {
      if (k < 4) {
        pmx[k] = max3r(max3r(Sc[4 * k], Sc[4 * k + 1], Sc[4 * k + 2]), Sc[4 * k + 3], Sc[4 * k + 3]);
      } else if (k == 4) {
        mx = max3r(max3r(pmx[0], pmx[1], pmx[2]), pmx[3], pmx[3]) * qk_scale;
      } else if (k == 5) {
        // the two lanes l, l ^ 32 hold one query vector
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = max3r(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1]));
        // wave-uniform: the running max moves only when some lane's grows by more than 8
        resc = __ballot(mx > m_thr) != 0ull;
      } else if (k == 6) {
        if (__builtin_expect(resc, 0)) {
          const float m_new = fmaxf(m_run, mx);
          alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          m_use = (m_run == -INFINITY) ? 0.f : m_run;
          m_thr = m_run + kRescaleThreshold;
          l_run *= alpha;
        }
      } else if (k < 7 + 16) {
        const int i = k - 7;
        // v_exp_f32 directly: results below 2^-126 flush to zero, irrelevant for probabilities
        p[i] = __builtin_amdgcn_exp2f(fmaf(Sc[i], qk_scale, -m_use));
      } else if (k < 7 + 16 + 8) {
        const int j = k - 23;
        pw[j] = pack_bf16(p[2 * j], p[2 * j + 1]);
        lsum += p[2 * j];
      } else if (k >= kSmSteps - 3) {  // the odd terms of the row sum, three per step
        const int j = k - (kSmSteps - 3);
        if (j == 0) {
          lsum2 = p[1] + p[3];
          lsum2 += p[5];
        } else if (j == 1) {
          lsum2 += p[7];
          lsum2 += p[9];
          lsum2 += p[11];
        } else {
          lsum2 += p[13];
          lsum2 += p[15];
          l_run += lsum + lsum2;
        }
      }
    };
    static_assert(kSmSteps <= kQSteps, "the softmax rides along the score steps");
    if (__builtin_expect(v1, 1)) {
      qk_tile(lds + nb * kTileBytes, Sx, softmax_step);
    } else {
#pragma unroll
      for (int k = 0; k < kSmSteps; ++k) softmax_step(k);
    }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 pw0 = {pw[0], pw[1], pw[2], pw[3]}, pw1 = {pw[4], pw[5], pw[6], pw[7]};
    const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, pw0), __builtin_bit_cast(bf16x8, pw1)};
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_expect(resc, 0)) {
#pragma unroll
      for (int f = 0; f < 16; ++f) rescale_agpr(acc[f], alpha);
#pragma unroll
      for (int f = 0; f < NR; ++f) accr[f] *= alpha;
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T P^T for tile i: 2 key steps x NF feature tiles
    {
      const uint32_t bb = lds_addr(lds + cb * kTileBytes);
      uint32_t vt0 = bb + vx0, vt1 = bb + vx1, vrt0 = bb + vrx0, vrt1 = bb + vrx1;
      asm volatile("" : "+v"(vt0), "+v"(vt1), "+v"(vrt0), "+v"(vrt1));  // as kt above
      auto tr = [](uint32_t addr) __attribute__((always_inline)) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)addr);
      };
      auto vread = [&](int n, bf16x4& lo, bf16x4& hi) __attribute__((always_inline)) {  // n = u * NF + f
        const int u = n / NF, f = n % NF;
        if (f < 16) {
          const int f4 = f >> 2, fl = f & 3;
          lo = tr((vt0 ^ (64 * fl)) + 256 * f4 + 16384 * u);
          hi = tr((vt1 ^ (64 * fl)) + 8192 + 256 * f4 + 16384 * u);
        } else {
          lo = tr((vrt0 ^ (64 * (f - 16))) + 2048 * u);
          hi = tr((vrt1 ^ (64 * (f - 16))) + 1024 + 2048 * u);
        }
      };
      bf16x4 lo[kPvDepth], hi[kPvDepth];
#pragma unroll
      for (int n = 0; n < kPvDepth; ++n) vread(n, lo[n], hi[n]);
#pragma unroll
      for (int n = 0; n < 2 * NF; ++n) {
        const int r = n % kPvDepth;
        const bf16x8 vt = {lo[r][0], lo[r][1], lo[r][2], lo[r][3], hi[r][0], hi[r][1], hi[r][2], hi[r][3]};
        if (n + kPvDepth < 2 * NF) vread(n + kPvDepth, lo[r], hi[r]);
        const int f = n % NF;
        // (program order is issue order: the assembly MFMAs are ordered with the LDS reads)
        if (f < 16) {
          // the first follows the probabilities' conversion and the rescale; the others
          // follow LDS reads
          if (n == 0) mfma_agpr<true>(acc[f], vt, pf[n / NF]);
          else mfma_agpr<false>(acc[f], vt, pf[n / NF]);
        }
        else accr[f - 16] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pf[n / NF], accr[f - 16], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_expect(!v1, 0)) {
      fin_seg = w0.seg;
      return false;
    }
    // next tile starts a new segment (a new run of the same segment keeps the frame)
    if (__builtin_expect(VROPE && w1.seg != w0.seg, 0) && sg[w1.seg].frame != sg[w0.seg].frame) {
      if (!WIN || w1.seg == w0.seg + 1) {
        frame_step(w0.seg, a.stepcs);
      } else {  // past the gap: R(-rot_j) R(rot_i), through the request phase
        frame_step(w0.seg, a.segcs);
        frame_step(w1.seg, a.segcs, -1.f);
      }
    }
    return true;
  };
  for (;;) {
    if (!iteration(IntC<0>{}, S, Sn, wa, wb, wc)) break;
    if (!iteration(IntC<1>{}, Sn, S, wb, wc, wa)) break;
    if (!iteration(IntC<2>{}, S, Sn, wc, wa, wb)) break;
    if (!iteration(IntC<0>{}, Sn, S, wa, wb, wc)) break;
    if (!iteration(IntC<1>{}, S, Sn, wb, wc, wa)) break;
    if (!iteration(IntC<2>{}, Sn, S, wc, wa, wb)) break;
  }
  settle_agpr(acc);
  // whole-tile copies to VGPRs for the stores (element reads of a pinned AGPR tuple are not
  // something the compiler can copy)
  auto tile_vgpr = [&](int f) __attribute__((always_inline)) -> floatx16 {
    floatx16 x = f < 16 ? acc[f < 16 ? f : 0] : accr[f < 16 ? 0 : f - 16];
    asm volatile("" : "+v"(x));
    return x;
  };
  // restore the request phase of the RoPE part: R(+rot_last)
  if (VROPE) frame_step(fin_seg, a.segcs);
  const float l_tot = pair_sum(l_run);
  const int d_v = a.d_v;
  if (a.n_split > 1) {  // partials of the tile's real vectors only: the merge reads no other
    if (!valid) return;
    const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
    const int64_t v = (int64_t)tile * kTileQ + wave * 32 + col;
    float* po = a.part_o + ((int64_t)split * nvec + v) * d_v;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const floatx16 x = tile_vgpr(f);
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *(float4*)(po + 32 * f + 8 * (i >> 2) + 4 * hf) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    }
    if (hf == 0) {
      float* pm = a.part_ml + ((int64_t)split * nvec + v) * 2;
      pm[0] = m_run == -INFINITY ? -INFINITY : m_run * kLn2;
      pm[1] = l_tot;
    }
    return;
  }
  if (!valid) return;
  const float inv = 1.f / l_tot;
  __bf16* o = (__bf16*)a.out + ((int64_t)(t - a.q0) * a.map.H + h) * d_v;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const floatx16 x = tile_vgpr(f);
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      bf16x4 y = {(__bf16)(x[i] * inv), (__bf16)(x[i + 1] * inv), (__bf16)(x[i + 2] * inv),
                  (__bf16)(x[i + 3] * inv)};
      *(bf16x4*)(o + 32 * f + 8 * (i >> 2) + 4 * hf) = y;
    }
  }
  if (a.lse && hf == 0) a.lse[(int64_t)(t - a.q0) * a.map.H + h] = (m_run + log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------- decode tiles
// Split key ranges of tiles that hold at most 64 query vectors (a one-row window: one row x at
// most 64 heads), the same per-key arithmetic as above. In k_attn_mfma such a tile would leave
// two of its four waves without a real query vector. Here the workgroup's four waves form two
// sets over the same 64 vectors (wave & 1 picks the 32-vector group): the key range is walked
// in 32-key tiles as above, set 0 taking the even tiles and set 1 the odd ones, so a step
// consumes two tiles, each in its own LDS buffer, while the next step's two are copied into the
// other two (four buffers, two tiles in flight per workgroup). Each set keeps its own running
// softmax and output, in its own RoPE frame; at the end set 1's (max, sum, output) go through
// LDS and set 0 merges them by the stable log-sum-exp rule (RedKnot-MLA paper, relocation
// paragraph) before the partial or final stores of k_attn_mfma.
//
// The same kernel runs the compressed-history layers of DeepSeek-V4 (CSA / HCA: TensorRT-LLM
// reading notes, section 1, the dual-pool kernel paragraph) under relocation: a workgroup takes
// one request row and 64 heads; its key walk covers the raw window [t - w, t] of the latent
// pool (runs of segments, as above) and then compressed entries of a second pool, one softmax
// over both. Entries come either as every entry available at the row (HCA: consecutive ids,
// contiguous per segment in the pool) or as the row's list (CSA): a tile then holds up to 32
// consecutive list entries of one segment, each gathered row by row (one 64-lane copy per nope
// row from a scalar address, per-lane addresses for the RoPE copy). The list ids of a step are
// read a step ahead, one id per lane, before that step's copies are issued (vector loads retire
// in order), and the run of a segment is cut with a ballot. An entry's RoPE frame is its
// segment's, so the query rotation and output frame steps are the raw keys' ones.
constexpr int kDecSplit = 0, kDecAll = 1, kDecList = 2;  // decode-kernel modes
constexpr int kDecBuf = 4;
#ifndef SEGMLA_DEC_QREG
#define SEGMLA_DEC_QREG 24
#endif
#ifndef SEGMLA_DEC_QK
#define SEGMLA_DEC_QK 3
#endif
#ifndef SEGMLA_DEC_PV
#define SEGMLA_DEC_PV 4
#endif
constexpr int kDecQReg = SEGMLA_DEC_QREG;              // query steps 0..kDecQReg-1 in registers
constexpr int kDecQkDepth = SEGMLA_DEC_QK;
constexpr int kDecPvDepth = SEGMLA_DEC_PV;
constexpr int kDecQSlot = 2 * 64 * 16;                 // steps kDecQReg..31: one slot per vector group
constexpr int kDecQBase = kDecBuf * kTileBytes;        // 147456
constexpr int kDecLds = kDecQBase + (32 - kDecQReg) * kDecQSlot;
constexpr int kDecLdsAlloc = kDecLds;
static_assert(kDecLdsAlloc <= 160 * 1024, "LDS budget");
static_assert(2 * 64 * 18 * 16 * 4 <= kDecQBase, "set 1's outputs fit in the tile buffers");
static_assert(2 * 64 * 8 <= (32 - kDecQReg) * kDecQSlot, "set 1's (max, sum) fit in the slots");

typedef const __attribute__((address_space(4))) CEnt ccent_t;
typedef const __attribute__((address_space(4))) CSeg ccseg_t;

template <bool VROPE, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_attn_dec(AttnArgs a) {
  extern __shared__ __attribute__((aligned(256))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int set = wave >> 1, grp = wave & 1;
  const int col = lane & 31, hf = lane >> 5;
  const int rank = (int)blockIdx.x / a.n_split, split = (int)blockIdx.x % a.n_split;
  // keys up to the window's last row (the row itself for one-row windows): the key range needs
  // no load, so the first copies can go out after two scalar loads (the work-list entry and the
  // split's first segment; scalar loads do not queue behind vector-memory copies)
  const int t_max = a.map.q0 + a.map.nq - 1;
  int k_lo = 0, k_hi = t_max + 1;
  if (MODE == kDecSplit && a.n_split > 1) {
    k_lo = split * a.split_keys;
    k_hi = min(k_hi, k_lo + a.split_keys);
  }
  int t_row = 0, row_i = 0, hb = 0;
  if constexpr (MODE != kDecSplit) {
    // consecutive rows (which share most keys) on one XCD: blocks are dealt to the 8 XCDs in
    // turn, so block b runs on XCD b % 8 and takes the (b / 8)-th item of that XCD's share
    const int nwg = a.map.nq * a.n_hb;
    const int per = (nwg + 7) >> 3;
    const int item = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
    if (item >= nwg) return;
    row_i = item / a.n_hb;
    hb = item - row_i * a.n_hb;
    t_row = a.map.q0 + row_i;
    k_lo = max(0, t_row - a.cwin);
    k_hi = t_row + 1;
  }
  if (k_lo >= k_hi) return;  // uniform over the workgroup
  typedef const __attribute__((address_space(4))) int32_t cint_t;
  const int tile = MODE == kDecSplit ? ((cint_t*)a.work)[rank] : 0;
  const int seg_lo = ((cint_t*)a.seg_of_row)[k_lo];
  if (MODE == kDecSplit && (tile < 0 || tile >= a.map.nF + a.map.nG)) return;  // uniform, before any copy
  cseg_t* const sg = (cseg_t*)a.seg;
  // compressed entries: those with ids below n_avail are available at the row; lists are read
  // up to position n_list
  int n_avail = 0, n_list = 0;
  if constexpr (MODE != kDecSplit) {
    ccseg_t* const cs = (ccseg_t*)a.cseg + sg[((cint_t*)a.seg_of_row)[t_row]].frame;
    n_avail = cs->base + min(cs->count, (t_row - cs->offset + 1) / a.ratio);
    if constexpr (MODE == kDecList) n_list = min(max(((cint_t*)a.clen)[row_i], 0), a.topk);
  }
  // list ids of the step being set up (lane j: position ibase + j), and of the next step
  int idv = 0, idv_n = 0, ibase = 0, ibase_n = 0;
  const int32_t* const clist = MODE == kDecList ? a.cidx + (int64_t)row_i * a.topk : nullptr;
  auto load_ids = [&](int base) __attribute__((always_inline)) -> int {
    return clist[min(base + lane, a.topk - 1)];
  };
  // the tile's query vectors: set after the first copies are issued
  int t = -1, h = 0;
  bool valid = false;
  const __bf16* qrow = nullptr;

  const float qk_scale = a.sigma * kLog2e;
  // B operand of S^T = K Q^T, step s: lane holds Q[qvec col][16 s + 8 hf + 0..7]; steps below
  // kDecQReg and the RoPE steps 32..35 (rotated per segment) in registers, steps kDecQReg..31 in
  // LDS slots shared by the two sets
  bf16x8 qf[kDecQReg], qr[4] = {};
  const char* const qslot = lds + kDecQBase + grp * 1024 + lane * 16;  // + (s - kDecQReg) * kDecQSlot
  constexpr int NF = VROPE ? 18 : 16;
  constexpr int NR = NF - 16;
  floatx16 acc[16], accr[NR > 0 ? NR : 1];
#pragma unroll
  for (int f = 0; f < 16; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[f][i] = 0.f;
#pragma unroll
  for (int f = 0; f < NR; ++f)
#pragma unroll
    for (int i = 0; i < 16; ++i) accr[f][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f, m_use = 0.f, m_thr = -INFINITY;
  const int half_r = a.d_rope / 2;

  // per-lane LDS offsets inside a tile buffer (as in k_attn_mfma)
  const int fcol = fn(col), rcol = fr(col);
  const int kx0 = (col * kNRow + 16 * (hf ^ (fcol & 1))) | (16 * (fcol & 14));
  const int krx0 = (kRBase + col * kRRow + 16 * (hf ^ (rcol & 1))) | (16 * (rcol & 6));
  const int G = lane >> 4, jj = lane & 15;
  const int cl = 2 * (G & 1) + ((jj & 3) >> 1);
  const int vrow = 4 * (G >> 1) + (jj >> 2);
  const int vx0 = (vrow * kNRow + 8 * (jj & 1) + 16 * (cl ^ (G >> 1))) | (64 * (jj >> 2));
  const int vx1 = (vrow * kNRow + 8 * (jj & 1) + 16 * (cl ^ ((G >> 1) | 2))) | (64 * (jj >> 2));
  const int vrx0 = (kRBase + vrow * kRRow + 8 * (jj & 1) + 16 * (cl ^ (G >> 1))) | (64 * ((jj >> 3) & 1));
  const int vrx1 = (kRBase + vrow * kRRow + 8 * (jj & 1) + 16 * (cl ^ ((G >> 1) | 2))) | (64 * ((jj >> 3) & 1));

  // ---- tile sequence over [k_lo, k_hi), segment-aligned (every wave walks all of it)
  auto first_tile = [&](TileIt& c) __attribute__((always_inline)) {
    const int lo = seg_lo;
    c.seg = lo;
    const int off = sg[lo].offset, len = sg[lo].len;
    c.pos0 = k_lo;
    c.pend = min(off + len, k_hi);
    c.nval = min(kKT, c.pend - k_lo);
    c.src = (sg[lo].pool_row + (k_lo - off)) * kRowBytes;
    c.v = 1;
    if constexpr (MODE != kDecSplit) {
      c.ph = 0;
      c.cur = 0;
      c.lo = 0;
    }
  };
  // the compressed tile that starts at id (all entries) or list position `cursor`
  auto comp_at = [&](TileIt& nx, int cursor) __attribute__((always_inline)) {
    if constexpr (MODE == kDecAll) {
      if (cursor >= n_avail) return;
      ccent_t* const e = (ccent_t*)a.cent + cursor;
      const int lim = min(e->hi, n_avail);
      nx.v = 1;
      nx.ph = 1;
      nx.seg = e->run;
      nx.cur = cursor;
      nx.lo = 0;
      nx.pos0 = -kKT;  // no causal mask: every entry of the walk is available
      nx.pend = 0;
      nx.nval = min(kKT, lim - cursor);
      nx.src = (int64_t)(cursor + e->delta) * kRowBytes;
    } else if constexpr (MODE == kDecList) {
      if (cursor >= n_list) return;
      const int o = cursor - ibase;  // 0..32: at most one tile before it in the step
      const int c0 = __builtin_amdgcn_readlane(idv, o);
      if (c0 < 0 || c0 >= n_avail) return;  // the list ends at an id that is not available
      ccent_t* const e = (ccent_t*)a.cent + c0;
      const int lim = min(e->hi, n_avail);
      // the leading run of list entries inside this segment's available ids
      const bool in = lane >= o && lane < o + kKT && ibase + lane < n_list && idv >= e->lo && idv < lim;
      const uint64_t run = __ballot(in) >> o;
      nx.v = 1;
      nx.ph = 1;
      nx.seg = e->run;
      nx.cur = cursor;
      nx.lo = o;
      nx.pos0 = -kKT;
      nx.pend = 0;
      nx.nval = min(kKT, (int)__builtin_ctzll(~run));
      nx.src = e->delta;
    }
  };
  auto advance = [&](const TileIt& c, TileIt& nx) __attribute__((always_inline)) {
    nx.v = 0;  // no next tile: a fully masked dummy (see the step loop)
    nx.seg = c.seg;
    nx.nval = 0;
    nx.pos0 = c.pos0;
    nx.pend = c.pend;
    nx.src = c.src;
    if constexpr (MODE == kDecSplit) {
      if (!c.v) return;
      if (c.pos0 + kKT < c.pend) {
        nx.v = 1;
        nx.seg = c.seg;
        nx.pos0 = c.pos0 + kKT;
        nx.pend = c.pend;
        nx.nval = min(kKT, c.pend - nx.pos0);
        nx.src = c.src + kKT * kRowBytes;
        return;
      }
      if (c.seg + 1 >= a.n_seg) return;
      const int off = sg[c.seg + 1].offset;  // segments are contiguous: off == c.pend
      if (off >= k_hi) return;
      nx.v = 1;
      nx.seg = c.seg + 1;
      nx.pos0 = off;
      nx.pend = min(off + sg[c.seg + 1].len, k_hi);
      nx.nval = min(kKT, nx.pend - off);
      nx.src = sg[c.seg + 1].pool_row * kRowBytes;
    } else {
      nx.ph = c.ph;
      nx.cur = c.cur;
      nx.lo = c.lo;
      if (!c.v) return;
      if (c.ph) {
        comp_at(nx, c.cur + c.nval);
        return;
      }
      if (c.pos0 + kKT < c.pend) {
        nx.v = 1;
        nx.pos0 = c.pos0 + kKT;
        nx.nval = min(kKT, c.pend - nx.pos0);
        nx.src = c.src + kKT * kRowBytes;
        return;
      }
      if (c.seg + 1 < a.n_seg) {
        const int off = sg[c.seg + 1].offset;
        if (off < k_hi) {
          nx.v = 1;
          nx.seg = c.seg + 1;
          nx.pos0 = off;
          nx.pend = min(off + sg[c.seg + 1].len, k_hi);
          nx.nval = min(kKT, nx.pend - off);
          nx.src = sg[c.seg + 1].pool_row * kRowBytes;
          return;
        }
      }
      comp_at(nx, 0);  // the raw window is done: the first compressed tile
    }
  };
  auto issue = [&](const TileIt& c, int b, int ids) __attribute__((always_inline)) {
    char* buf = lds + b * kTileBytes;
    if constexpr (MODE == kDecList) {
      if (c.ph) {  // listed entries, row by row; rows past nval repeat the last one
        const uint32_t lb = lds_addr(buf);
        const int ln = lane_id();
        const char* const cp = (const char*)a.ckv;
#pragma unroll
        for (int n = 0; n < kKT / kWaves; ++n) {
          const int r = wave + kWaves * n;
          const int id = __builtin_amdgcn_readlane(ids, c.lo + min(r, c.nval - 1));
          dma16(cp + (int64_t)(id + (int)c.src) * kRowBytes, (ln * 16) ^ (fn(r) << 4), lb + r * kNRow);
        }
        const int r = 8 * wave + (ln >> 3);
        const int id = __builtin_amdgcn_ds_bpermute(4 * (c.lo + min(r, c.nval - 1)), ids);
        dma16_v(cp + (int64_t)(id + (int)c.src) * kRowBytes + kNRow + (((ln & 7) ^ fr(r)) << 4),
                lb + kRBase + wave * 1024);
        return;
      }
    }
    const char* pool = (const char*)a.kv;
    if constexpr (MODE == kDecAll) pool = c.ph ? (const char*)a.ckv : pool;
    if (__builtin_expect(c.nval == kKT, 1))
      load_tile_bf16_full(buf, pool + c.src, wave);
    else
      load_tile_bf16(buf, pool + c.src, c.nval, wave);
  };
  // q^r <- R(-rot_i) q^r from the stored query (registers)
  auto rotate_q = [&](int seg) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 32; s < 36; ++s) {
      uint4 v = *(const uint4*)(qrow + 16 * s + 8 * hf);
      if (!valid) v = make_uint4(0, 0, 0, 0);
      const bf16x8 x = *(bf16x8*)&v;
      bf16x8 y;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int k = 8 * (s - 32) + 4 * hf + p;
        const float2 cs = a.segcs[seg * half_r + k];
        const float x0 = bf2f(x[2 * p]), x1 = bf2f(x[2 * p + 1]);
        y[2 * p] = (__bf16)(x0 * cs.x + x1 * cs.y);
        y[2 * p + 1] = (__bf16)(-x0 * cs.y + x1 * cs.x);
      }
      qr[s - 32] = y;
    }
  };
  auto frame_step = [&](int seg, float sgn) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < NR; ++f) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int k = 16 * f + 4 * (i >> 2) + 2 * hf + ((i & 3) >> 1);
        float2 cs = a.segcs[seg * half_r + k];
        cs.y *= sgn;
        const float x = accr[f][i], y = accr[f][i + 1];
        accr[f][i] = fmaf(x, cs.x, -(y * cs.y));
        accr[f][i + 1] = fmaf(x, cs.y, y * cs.x);
      }
      asm volatile("" ::: "memory");
    }
  };
  auto qk_reads = [&](uint32_t kt, uint32_t krt, int k, bf16x8& kf) __attribute__((always_inline)) {
    if (k < 32) {
      const int s8 = k >> 3, sl = k & 7;
      kf = *(const lds_bf16x8*)(size_t)((kt ^ (32 * sl)) + 256 * s8);
    } else {
      kf = *(const lds_bf16x8*)(size_t)(krt ^ (32 * (k - 32)));
    }
  };

  // ---- a new segment for this set: the output moves to its RoPE frame, R(-rot_new) R(rot_old)
  // through the request phase (the set may skip the segment the other set took), and the query
  // is rotated. Called before the step's copies are issued: vector loads retire in order, so
  // behind the copies these table and query reads would wait for both tiles to land.
  int cur_seg = -1;  // segment whose RoPE frame the query and the output are in
  auto prepare = [&](const TileIt& w) __attribute__((always_inline)) {
    if (__builtin_expect(w.v && w.seg != cur_seg, 0)) {
      if (cur_seg < 0 || sg[w.seg].frame != sg[cur_seg].frame) {
        if (VROPE && cur_seg >= 0) {
          frame_step(cur_seg, 1.f);
          frame_step(w.seg, -1.f);
        }
        rotate_q(w.seg);
      }
      cur_seg = w.seg;
    }
  };
  // ---- one key tile of this set: scores, mask, online softmax, O^T += V^T P^T
  auto process = [&](const TileIt& w, const char* buf) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    floatx16 S;
    {
      uint32_t kt = lds_addr(buf) + kx0, krt = lds_addr(buf) + krx0;
      asm volatile("" : "+v"(kt), "+v"(krt));
      bf16x8 ring[kDecQkDepth], qring[kDecQkDepth];
#pragma unroll
      for (int k = 0; k < kDecQkDepth; ++k) {
        qk_reads(kt, krt, k, ring[k]);
        if (k >= kDecQReg && k < 32) qring[k] = *(const bf16x8*)(qslot + (k - kDecQReg) * kDecQSlot);
      }
#pragma unroll
      for (int k = 0; k < kQSteps; ++k) {
        const bf16x8 kf = ring[k % kDecQkDepth];
        const bf16x8 qv = k < kDecQReg ? qf[k < kDecQReg ? k : 0]
                                       : (k < 32 ? qring[k % kDecQkDepth] : qr[k < 32 ? 0 : k - 32]);
        if (k + kDecQkDepth < kQSteps) {
          const int kn = k + kDecQkDepth;
          qk_reads(kt, krt, kn, ring[k % kDecQkDepth]);
          if (kn >= kDecQReg && kn < 32)
            qring[k % kDecQkDepth] = *(const bf16x8*)(qslot + (kn - kDecQReg) * kDecQSlot);
        }
        if (k == 0) {
          const floatx16 zero = {};
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv, zero, 0, 0, 0);
        } else {
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv, S, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // causal / range mask: register i of lane (hf, col) is key 8 (i >> 2) + 4 hf + (i & 3)
    const int nval = w.v ? w.nval : 0;  // no tile: every key masked
    if (__builtin_expect(__ballot((w.pos0 + kKT - 1 > t) || (nval < kKT)) != 0ull, 0)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = 8 * (i >> 2) + 4 * hf + (i & 3);
        if (w.pos0 + k > t || k >= nval) S[i] = -INFINITY;
      }
    }
    // online softmax (log2 domain, lazy wave-uniform rescale)
    float mx = max3r(max3r(S[0], S[1], S[2]), S[3], S[4]);
    mx = max3r(max3r(mx, S[5], S[6]), S[7], S[8]);
    mx = max3r(max3r(mx, S[9], S[10]), S[11], S[12]);
    mx = max3r(max3r(mx, S[13], S[14]), S[15], S[15]) * qk_scale;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = max3r(__uint_as_float(sw[0]), __uint_as_float(sw[1]), __uint_as_float(sw[1]));
    }
    float alpha = 1.f;
    const bool resc = __ballot(mx > m_thr) != 0ull;
    if (__builtin_expect(resc, 0)) {
      const float m_new = fmaxf(m_run, mx);
      alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      m_use = (m_run == -INFINITY) ? 0.f : m_run;
      m_thr = m_run + kRescaleThreshold;
      l_run *= alpha;
    }
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(S[i], qk_scale, -m_use));
    uint32_t pw[8];
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pw[j] = pack_bf16(p[2 * j], p[2 * j + 1]);
      lsum += p[2 * j] + p[2 * j + 1];
    }
    l_run += lsum;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 pw0 = {pw[0], pw[1], pw[2], pw[3]}, pw1 = {pw[4], pw[5], pw[6], pw[7]};
    const bf16x8 pf[2] = {__builtin_bit_cast(bf16x8, pw0), __builtin_bit_cast(bf16x8, pw1)};
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_expect(resc, 0)) {
#pragma unroll
      for (int f = 0; f < 16; ++f) rescale_agpr(acc[f], alpha);
#pragma unroll
      for (int f = 0; f < NR; ++f) accr[f] *= alpha;
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      const uint32_t bb = lds_addr(buf);
      uint32_t vt0 = bb + vx0, vt1 = bb + vx1, vrt0 = bb + vrx0, vrt1 = bb + vrx1;
      asm volatile("" : "+v"(vt0), "+v"(vt1), "+v"(vrt0), "+v"(vrt1));
      auto tr = [](uint32_t addr) __attribute__((always_inline)) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)addr);
      };
      auto vread = [&](int n, bf16x4& lo, bf16x4& hi) __attribute__((always_inline)) {
        const int u = n / NF, f = n % NF;
        if (f < 16) {
          const int f4 = f >> 2, fl = f & 3;
          lo = tr((vt0 ^ (64 * fl)) + 256 * f4 + 16384 * u);
          hi = tr((vt1 ^ (64 * fl)) + 8192 + 256 * f4 + 16384 * u);
        } else {
          lo = tr((vrt0 ^ (64 * (f - 16))) + 2048 * u);
          hi = tr((vrt1 ^ (64 * (f - 16))) + 1024 + 2048 * u);
        }
      };
      bf16x4 lo[kDecPvDepth], hi[kDecPvDepth];
#pragma unroll
      for (int n = 0; n < kDecPvDepth; ++n) vread(n, lo[n], hi[n]);
#pragma unroll
      for (int n = 0; n < 2 * NF; ++n) {
        const int r = n % kDecPvDepth;
        const bf16x8 vt = {lo[r][0], lo[r][1], lo[r][2], lo[r][3], hi[r][0], hi[r][1], hi[r][2], hi[r][3]};
        if (n + kDecPvDepth < 2 * NF) vread(n + kDecPvDepth, lo[r], hi[r]);
        const int f = n % NF;
        if (f < 16) {
          if (n == 0) mfma_agpr<true>(acc[f], vt, pf[n / NF]);
          else mfma_agpr<false>(acc[f], vt, pf[n / NF]);
        } else {
          accr[f - 16] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pf[n / NF], accr[f - 16], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: the first step's two tiles in flight, then the query and this set's first
  // segment (their loads retire after the copies), all behind one wait
  TileIt a0, b0, a1, b1;
  first_tile(a0);
  if constexpr (MODE == kDecList) {
    // a one-tile window: the second tile is listed and its ids are needed now (read before any
    // copy is issued; otherwise the first ids are read with the step's copies, below)
    if (__builtin_expect(k_lo + a0.nval >= k_hi, 0)) {
      idv = load_ids(0);
      // a use the compiler sees: its own wait goes here, before any copy, and the load is
      // known complete on every path after it (a wait it cannot see would leave the load
      // pending in its books, and later waits for it would also wait for the copies)
      asm volatile("" ::"v"(idv));
    }
  }
  advance(a0, b0);
  if constexpr (MODE == kDecList) {
    ibase_n = b0.ph ? b0.cur + b0.nval : 0;
    idv_n = load_ids(ibase_n);
  }
  issue(a0, 0, idv);
  if (b0.v) issue(b0, 1, idv);
  if constexpr (MODE == kDecSplit) {
    valid = tile_qvec(a.map, tile, grp * 32 + col, t, h);
  } else {
    t = t_row;
    h = hb * 64 + grp * 32 + col;
    valid = h < a.map.H;
    if (!valid) h = 0;  // a past-the-end head of the last block reads head 0's query (masked)
  }
  if (!valid) t = -1;
  qrow = (const __bf16*)a.q + ((int64_t)(valid ? t - a.q0 : 0) * a.map.H + h) * kD;
#pragma unroll
  for (int s = 0; s < kDecQReg; ++s) {
    uint4 v = *(const uint4*)(qrow + 16 * s + 8 * hf);
    if (!valid) v = make_uint4(0, 0, 0, 0);
    qf[s] = *(bf16x8*)&v;
  }
  if (set == 0) {
#pragma unroll
    for (int s = kDecQReg; s < 32; ++s) {
      uint4 v = *(const uint4*)(qrow + 16 * s + 8 * hf);
      if (!valid) v = make_uint4(0, 0, 0, 0);
      *(uint4*)(lds + kDecQBase + (s - kDecQReg) * kDecQSlot + grp * 1024 + lane * 16) = v;
    }
  }
  {
    TileIt w;
    w.v = set ? b0.v : a0.v;
    w.seg = set ? b0.seg : a0.seg;
    w.nval = w.pos0 = w.pend = 0;
    w.src = 0;
    prepare(w);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (MODE == kDecList) {
    idv = idv_n;
    ibase = ibase_n;
  }
  // One step per pair of tiles: (a0, b0) resident in buffers cb, cb + 1 (set 0 takes a0, set 1
  // b0), (a1, b1) copied into the other two; then the roles swap.
  int cb = 0;
  for (;;) {
    const int ob = 2 - cb;
    TileIt w;  // this set's tile (field by field: no whole-descriptor copies)
    w.v = set ? b0.v : a0.v;
    w.seg = set ? b0.seg : a0.seg;
    w.nval = set ? b0.nval : a0.nval;
    w.pos0 = set ? b0.pos0 : a0.pos0;
    w.pend = 0;
    w.src = 0;
    prepare(w);
    advance(b0, a1);
    advance(a1, b1);
    if constexpr (MODE == kDecList) {  // the next step's ids, ahead of this step's copies
      ibase_n = b1.ph ? b1.cur + b1.nval : 0;
      idv_n = load_ids(ibase_n);
    }
    if (a1.v) issue(a1, ob, idv);
    if (b1.v) issue(b1, ob + 1, idv);
    // a set without a tile in this step (the range's last, odd tile) runs the same code on the
    // other set's buffer with every key masked: no state changes, and the accumulator MFMAs
    // stay unconditional (a conditional call made the register allocator shuffle them)
    process(w, lds + (cb + (w.v ? set : 0)) * kTileBytes);
    // next step's tiles have landed, and every wave is done with this step's buffers
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!a1.v) break;
    a0.v = a1.v; a0.seg = a1.seg; a0.nval = a1.nval; a0.pos0 = a1.pos0; a0.pend = a1.pend; a0.src = a1.src;
    b0.v = b1.v; b0.seg = b1.seg; b0.nval = b1.nval; b0.pos0 = b1.pos0; b0.pend = b1.pend; b0.src = b1.src;
    if constexpr (MODE != kDecSplit) {
      a0.ph = a1.ph; a0.cur = a1.cur; a0.lo = a1.lo;
      b0.ph = b1.ph; b0.cur = b1.cur; b0.lo = b1.lo;
    }
    if constexpr (MODE == kDecList) {
      idv = idv_n;
      ibase = ibase_n;
    }
    cb = ob;
  }
  settle_agpr(acc);
  auto tile_vgpr = [&](int f) __attribute__((always_inline)) -> floatx16 {
    floatx16 x = f < 16 ? acc[f < 16 ? f : 0] : accr[f < 16 ? 0 : f - 16];
    asm volatile("" : "+v"(x));
    return x;
  };
  if (VROPE && cur_seg >= 0) frame_step(cur_seg, 1.f);  // restore the request phase
  // ---- set 1 hands (max, sum, output) to set 0 through LDS (the tile buffers are free)
  float* const xo = (float*)lds + grp * (64 * 18 * 16) + lane * 4;  // + f * 1024 + q * 256 floats
  float* const xml = (float*)(lds + kDecQBase) + (grp * 64 + lane) * 2;
  if (set == 1) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const floatx16 x = tile_vgpr(f);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4*)(xo + f * 1024 + q * 256) = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
    }
    xml[0] = m_run;
    xml[1] = l_run;
  }
  __syncthreads();
  if (set == 1) return;
  const float m1 = xml[0], l1 = xml[1];
  const float mm = fmaxf(m_run, m1);
  const float w0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mm);
  const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
  const float l_tot = pair_sum(l_run * w0 + l1 * w1);
  auto merged = [&](int f) __attribute__((always_inline)) -> floatx16 {
    floatx16 x = tile_vgpr(f);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 y = *(const float4*)(xo + f * 1024 + q * 256);
      x[4 * q] = fmaf(x[4 * q], w0, y.x * w1);
      x[4 * q + 1] = fmaf(x[4 * q + 1], w0, y.y * w1);
      x[4 * q + 2] = fmaf(x[4 * q + 2], w0, y.z * w1);
      x[4 * q + 3] = fmaf(x[4 * q + 3], w0, y.w * w1);
    }
    return x;
  };
  const int d_v = a.d_v;
  if (!valid) return;
  if (MODE == kDecSplit && a.n_split > 1) {
    // partial outputs in bf16 (half the bytes written here and read by the merge); the
    // statistics (max, sum) stay fp32
    const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
    const int64_t v = (int64_t)tile * kTileQ + grp * 32 + col;
    __bf16* po = (__bf16*)a.part_o + ((int64_t)split * nvec + v) * d_v;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const floatx16 x = merged(f);
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const bf16x4 y = {(__bf16)x[i], (__bf16)x[i + 1], (__bf16)x[i + 2], (__bf16)x[i + 3]};
        *(bf16x4*)(po + 32 * f + 8 * (i >> 2) + 4 * hf) = y;
      }
    }
    if (hf == 0) {
      float* pm = a.part_ml + ((int64_t)split * nvec + v) * 2;
      pm[0] = mm == -INFINITY ? -INFINITY : mm * kLn2;
      pm[1] = l_tot;
    }
    return;
  }
  const float inv = 1.f / l_tot;
  __bf16* o = (__bf16*)a.out + ((int64_t)(t - a.q0) * a.map.H + h) * d_v;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const floatx16 x = merged(f);
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      bf16x4 y = {(__bf16)(x[i] * inv), (__bf16)(x[i + 1] * inv), (__bf16)(x[i + 2] * inv),
                  (__bf16)(x[i + 3] * inv)};
      *(bf16x4*)(o + 32 * f + 8 * (i >> 2) + 4 * hf) = y;
    }
  }
  if (a.lse && hf == 0) a.lse[(int64_t)(t - a.q0) * a.map.H + h] = (mm + log2f(l_tot)) * kLn2;
}

namespace {
template <bool VROPE, bool FP8, bool WIN>
hipError_t launch_mfma(const AttnArgs& a, hipStream_t stream) {
  const int lds = kLdsAlloc;
  // once per process and instantiation; a function-local static is initialized exactly once
  // even when several host threads launch at the same time
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_attn_mfma<VROPE, FP8, WIN>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = WIN ? (int64_t)a.map.nW : (int64_t)(a.map.nF + a.map.nG) * a.n_split;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((k_attn_mfma<VROPE, FP8, WIN>), dim3((unsigned)blocks), dim3(kThreads), lds,
                     stream, a);
  return hipGetLastError();
}

template <bool WIN>
hipError_t launch_any(const AttnArgs& a, int kv_dtype, int v_has_rope, hipStream_t stream) {
  const bool fp8 = kv_dtype == 2;
  if (v_has_rope)
    return fp8 ? launch_mfma<true, true, WIN>(a, stream) : launch_mfma<true, false, WIN>(a, stream);
  return fp8 ? launch_mfma<false, true, WIN>(a, stream) : launch_mfma<false, false, WIN>(a, stream);
}
}  // namespace

namespace {
template <bool VROPE, int MODE>
hipError_t launch_dec(const AttnArgs& a, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_attn_dec<VROPE, MODE>, hipFuncAttributeMaxDynamicSharedMemorySize, kDecLdsAlloc);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = MODE == kDecSplit ? (int64_t)(a.map.nF + a.map.nG) * a.n_split
                                           : 8 * (((int64_t)a.map.nq * a.n_hb + 7) / 8);
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((k_attn_dec<VROPE, MODE>), dim3((unsigned)blocks), dim3(kThreads), kDecLdsAlloc,
                     stream, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_decode(const AttnArgs& a, int v_has_rope, hipStream_t stream) {
  return v_has_rope ? launch_dec<true, kDecSplit>(a, stream) : launch_dec<false, kDecSplit>(a, stream);
}

hipError_t launch_attn_dual(const AttnArgs& a, int v_has_rope, int lists, hipStream_t stream) {
  if (lists)
    return v_has_rope ? launch_dec<true, kDecList>(a, stream) : launch_dec<false, kDecList>(a, stream);
  return v_has_rope ? launch_dec<true, kDecAll>(a, stream) : launch_dec<false, kDecAll>(a, stream);
}

hipError_t launch_attn(const AttnArgs& a, int kv_dtype, int v_has_rope, hipStream_t stream) {
  if (kv_dtype == 0) return launch_attn_f32(a, stream);
  return launch_any<false>(a, kv_dtype, v_has_rope, stream);
}

hipError_t launch_attn_window(const AttnArgs& a, int kv_dtype, int v_has_rope, hipStream_t stream) {
  if (kv_dtype == 0) return launch_attn_f32_window(a, stream);
  return launch_any<true>(a, kv_dtype, v_has_rope, stream);
}

}  // namespace segmla
