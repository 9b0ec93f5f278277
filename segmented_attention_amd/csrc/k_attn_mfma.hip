// Segment-relocated MLA attention on CDNA4 matrix cores (bf16 MFMA, fp32 accumulation) for
// the packed 512 + 64 latent (RedKnot-MLA paper: relocation paragraph, Eq. 5, and the fused
// consumer paragraph; DeepSeek-V4 latent shape).
//
// Workgroup = 8 wavefronts (two per SIMD) = one tile of 128 query vectors (row, head); every
// query vector shares the same latent rows, so one 64-key tile of the canonical latent is
// staged once in LDS and read by all eight waves. Per wave: 16 query vectors (one per lane
// column of the 16x16x32 MFMA), the query kept in VGPRs as the B operand (18 steps of 32
// features) and the output accumulator O^T [576 features x 16 query vectors] in 36 16x16
// accumulators.
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
// LDS tile layout (72 KB): a nope region of 64 rows x 64 16-byte chunks (chunk c of row r at
// r*64 + (c ^ fn(r))) followed by a RoPE region of 64 rows x 8 chunks (chunk c of row r at
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

constexpr int kD = 576, kDN = 512;
constexpr int kKT = 64;                          // keys per LDS tile
constexpr int kRowBytes = kD * 2;                // 1152 bytes per bf16 latent row
constexpr int kNRow = 1024;                      // LDS bytes per row, nope region
constexpr int kRRow = 128;                       // LDS bytes per row, RoPE region
constexpr int kRBase = kKT * kNRow;              // 65536
constexpr int kTileBytes = kKT * (kNRow + kRRow);  // 73728
constexpr int kWaves = 8;
// per-lane slots for the segment-rotated RoPE query fragments (2 x 16 bytes per lane)
constexpr int kQRBase = 2 * kTileBytes;          // 147456
constexpr int kQRBytes = kWaves * 2 * 64 * 16;   // 16384
constexpr int kLdsBytes = kQRBase + kQRBytes;    // 163840 = all of a CU's LDS
constexpr int kThreads = 64 * kWaves;            // 512
static_assert(kWaves * 16 == kTileQ, "one 16-vector MFMA column block per wave");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;        // log2 units

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
  int seg;   // segment index
  int j0;    // first canonical row of the tile inside the segment
  int nval;  // rows of the tile that are in range (1..64)
  int pos0;  // request position of row j0
};

// Stage one bf16 tile of up to 64 latent rows with direct global->LDS 16-byte loads: one
// instruction per nope row (wave w takes rows w, w+8, ...) and one for 8 RoPE rows per wave.
// Rows past nval repeat the last in-range row (finite data; their scores are masked).
__device__ __forceinline__ void load_tile_bf16(char* buf, const char* tile_src, int nval, int wave,
                                               int lane) {
  int lane16 = lane * 16;
  asm volatile("" : "+v"(lane16));  // keep the per-row XORs in the loop (no hoisted copies)
#pragma unroll
  for (int n = 0; n < kKT / kWaves; ++n) {
    const int r = wave + kWaves * n;
    const int rr = min(r, nval - 1);
    const char* src = tile_src + rr * kRowBytes + (lane16 ^ (fn(r) << 4));
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(buf + r * kNRow), 16, 0, 0);
  }
  const int r = 8 * wave + (lane >> 3);
  const int rr = min(r, nval - 1);
  const char* src = tile_src + rr * kRowBytes + kNRow + (((lane & 7) ^ fr(r)) << 4);
  __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(buf + kRBase + wave * 1024), 16, 0, 0);
}

// Stage one E4M3 tile: codes * block scale -> bf16, RoPE dims copied, written in the same
// layout as the bf16 tile.
__device__ __forceinline__ void load_tile_e4m3(char* buf, const uint8_t* codes, const float* scales,
                                               const __bf16* rope, int64_t row0, int nval, int tid) {
#pragma unroll 3
  for (int n = 0; n < kKT * 72 / kThreads; ++n) {
    const int idx = n * kThreads + tid;    // logical (row, chunk)
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
  // the per-wave row maxima use the RoPE-query slots before any fragment is written there
  int* s_tmax = (int*)(lds + kQRBase);
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
  int k_lo = 0, k_hi = t_max + 1;
  if (a.n_split > 1) {
    k_lo = split * a.split_keys;
    k_hi = min(k_hi, k_lo + a.split_keys);
  }
  if (k_lo >= k_hi) return;  // uniform over the workgroup

  const float qk_scale = a.sigma * kLog2e;
  const __bf16* qrow = (const __bf16*)a.q + ((int64_t)(valid ? t : 0) * a.map.H + h) * kD;
  // B operand of S^T = K Q^T: lane holds Q[qvec col][32 s + 8 g + 0..7]; the two RoPE
  // steps (s = 16, 17) are rotated per segment and kept in this lane's LDS slots
  bf16x8 qf[16];
  char* const qslot = lds + kQRBase + wave * 2048 + lane * 16;
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    uint4 v = *(const uint4*)(qrow + 32 * s + 8 * g);
    if (!valid) v = make_uint4(0, 0, 0, 0);
    qf[s] = *(bf16x8*)&v;
  }
  constexpr int NF = VROPE ? 36 : 32;  // 16-feature tiles of O^T
  floatx4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS byte offsets (first 32-key block, tile buffer 0).
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

  // tile iterator over the key range [k_lo, k_hi), segment-aligned
  TileIt cur;
  {
    cur.seg = seg_of(a.seg, a.n_seg, k_lo);
    const SegDesc sd = a.seg[cur.seg];
    cur.j0 = k_lo - sd.offset;
    cur.nval = min(kKT, min(sd.len, k_hi - sd.offset) - cur.j0);
    cur.pos0 = sd.offset + cur.j0;
  }
  auto advance = [&](const TileIt& c, TileIt& nx) -> bool {
    const SegDesc sd = a.seg[c.seg];
    const int j_end = min(sd.len, k_hi - sd.offset);
    if (c.j0 + kKT < j_end) {
      nx.seg = c.seg;
      nx.j0 = c.j0 + kKT;
      nx.nval = min(kKT, j_end - nx.j0);
      nx.pos0 = sd.offset + nx.j0;
      return true;
    }
    if (c.seg + 1 >= a.n_seg) return false;
    const SegDesc sn = a.seg[c.seg + 1];
    if (sn.offset >= k_hi) return false;
    nx.seg = c.seg + 1;
    nx.j0 = 0;
    nx.nval = min(kKT, min(sn.len, k_hi - sn.offset));
    nx.pos0 = sn.offset;
    return true;
  };
  auto issue = [&](const TileIt& c, int b) {
    char* buf = lds + b * kTileBytes;
    const int64_t row0 = a.seg[c.seg].pool_row + c.j0;
    if constexpr (FP8)
      load_tile_e4m3(buf, (const uint8_t*)a.kv, a.kv_scale, (const __bf16*)a.kv_rope, row0, c.nval, tid);
    else
      load_tile_bf16(buf, (const char*)a.kv + row0 * kRowBytes, c.nval, wave, lane);
  };

  const int half_r = a.d_rope / 2;  // 32
  issue(cur, 0);
  int prev_seg = -1;
  for (int it = 0;; ++it) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    TileIt nxt;
    const bool has_next = advance(cur, nxt);
    if (has_next) issue(nxt, (it + 1) & 1);
    if (cur.seg != prev_seg) {
      if (VROPE && prev_seg >= 0) {
        // move the accumulated output from segment prev_seg's RoPE frame to cur.seg's:
        // lane holds features 16 f + 4 g + i, pairs (i, i+1) for even i
#pragma unroll
        for (int f = 32; f < NF; ++f)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const int k = 8 * (f - 32) + 2 * g + (i >> 1);
            const float2 cs = a.stepcs[prev_seg * half_r + k];
            const float x = acc[f][i], y = acc[f][i + 1];
            acc[f][i] = x * cs.x - y * cs.y;
            acc[f][i + 1] = x * cs.y + y * cs.x;
          }
      }
      // q^r <- R(-rot_i) q^r, from the stored query (features 512 + 32 (s-16) + 8 g + 0..7)
#pragma unroll
      for (int s = 16; s < 18; ++s) {
        uint4 v = *(const uint4*)(qrow + 32 * s + 8 * g);
        if (!valid) v = make_uint4(0, 0, 0, 0);
        const bf16x8 x = *(bf16x8*)&v;
        bf16x8 y;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int k = 16 * (s - 16) + 4 * g + p;
          const float2 cs = a.segcs[cur.seg * half_r + k];
          const float x0 = bf2f(x[2 * p]), x1 = bf2f(x[2 * p + 1]);
          y[2 * p] = (__bf16)(x0 * cs.x + x1 * cs.y);
          y[2 * p + 1] = (__bf16)(-x0 * cs.y + x1 * cs.x);
        }
        *(bf16x8*)(qslot + (s - 16) * 1024) = y;
      }
      prev_seg = cur.seg;
    }

    const char* buf = lds + (it & 1) * kTileBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int pos_b = cur.pos0 + 32 * kb;
      if (32 * kb >= cur.nval || pos_b > t_wmax) continue;  // uniform per wave
      const char* kbuf = buf + kb * 32 * kNRow;          // nope rows of this 32-key block
      const char* rbuf = buf + kb * 32 * kRRow;          // RoPE rows (offset by kRBase)
      __builtin_amdgcn_sched_barrier(0);
      // ---- S^T = K Q^T for keys 16 tau + m (two 16x16 tiles, one accumulation chain each)
      const bf16x8 qr16 = *(const bf16x8*)qslot;
      const bf16x8 qr17 = *(const bf16x8*)(qslot + 1024);
      floatx4 sacc[2];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const char* kt = kbuf + tau * 16 * kNRow;
        const char* rt = rbuf + tau * 16 * kRRow;
        auto kaddr = [&](int s) -> const char* {
          return s < 16 ? kt + qb[s & 3] + 256 * (s >> 2) : rt + (s == 16 ? qr0 : qr1);
        };
        floatx4 acc_s = floatx4{0.f, 0.f, 0.f, 0.f};
        bf16x8 ka = *(const bf16x8*)kaddr(0);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          bf16x8 na = ka;
          if (s + 1 < 18) na = *(const bf16x8*)kaddr(s + 1);
          const bf16x8 qv = s < 16 ? qf[s] : (s == 16 ? qr16 : qr17);
          acc_s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qv, acc_s, 0, 0, 0);
          ka = na;
        }
        sacc[tau] = acc_s;
      }
      floatx4 s0 = sacc[0], s1 = sacc[1];
      __builtin_amdgcn_sched_barrier(0);
      // lane (g, col): value (tau, i) = key 16 tau + 4 g + i of this block, query vector col
      const bool need_mask = (pos_b + 31 > t) || (32 * kb + 32 > cur.nval);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k0 = 4 * g + i, k1 = 16 + 4 * g + i;
          if (pos_b + k0 > t || 32 * kb + k0 >= cur.nval) s0[i] = -INFINITY;
          if (pos_b + k1 > t || 32 * kb + k1 >= cur.nval) s1[i] = -INFINITY;
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
        const float p0 = exp2f(s0[i] * qk_scale - m_use);
        const float p1 = exp2f(s1[i] * qk_scale - m_use);
        lsum += p0 + p1;
        pf[i] = (__bf16)p0;
        pf[4 + i] = (__bf16)p1;
      }
      l_run += lsum;
      __builtin_amdgcn_sched_barrier(0);
      // ---- O^T += V^T P^T (A operand by two transposing reads: keys 4 g + 0..3, 16 + 4 g + 0..3)
      const char* vbuf = buf + kb * 32 * kNRow;
      int vx = pfh;
      asm volatile("" : "+v"(vx));  // addresses computed per use, not hoisted into registers
      auto vaddr = [&](int f) -> const char* {
        if (f < 32) return vbuf + pb + ((f ^ vx) << 5);
        const int c2 = 2 * (f - 32) + pcofs;
        return rbuf + prb + ((c2 ^ pfr) << 4);
      };
      auto vtau1 = [&](int f) { return f < 32 ? 16 * kNRow : 16 * kRRow; };
      bf16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vaddr(0));
      bf16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vaddr(0) + vtau1(0)));
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        bf16x4 nlo = vlo, nhi = vhi;
        if (f + 1 < NF) {
          nlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)vaddr(f + 1));
          nhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vaddr(f + 1) + vtau1(f + 1)));
        }
        const bf16x8 vt = {vlo[0], vlo[1], vlo[2], vlo[3], vhi[0], vhi[1], vhi[2], vhi[3]};
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pf, acc[f], 0, 0, 0);
        vlo = nlo;
        vhi = nhi;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!has_next) break;
    cur = nxt;
  }

  // restore the request phase of the RoPE part: R(+rot_last)
  if (VROPE && prev_seg >= 0) {
#pragma unroll
    for (int f = 32; f < NF; ++f)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const int k = 8 * (f - 32) + 2 * g + (i >> 1);
        const float2 cs = a.segcs[prev_seg * half_r + k];
        const float x = acc[f][i], y = acc[f][i + 1];
        acc[f][i] = x * cs.x - y * cs.y;
        acc[f][i + 1] = x * cs.y + y * cs.x;
      }
  }
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
