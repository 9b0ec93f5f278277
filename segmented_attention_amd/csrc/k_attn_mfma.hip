// Segment-relocated MLA attention on CDNA4 matrix cores (bf16 MFMA, fp32 accumulation) for
// the packed 512 + 64 latent (RedKnot-MLA paper: relocation paragraph, Eq. 5, and the fused
// consumer paragraph; DeepSeek-V4 latent shape).
//
// Workgroup = 4 wavefronts (one per SIMD) = one tile of 64 query vectors (row, head); every
// query vector shares the same latent rows, so one 64-key tile of the canonical latent is
// staged once in LDS and read by all four waves. Per wave: 16 query vectors (one per lane column of the
// 16x16x32 MFMA), the query kept in VGPRs as the B operand (18 steps of 32 features) and
// the output accumulator O^T [576 features x 16 query vectors] in 36 16x16 accumulators.
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
// LDS tile layout: 64 key rows x 72 16-byte chunks, chunk c of row r stored at
// r*72 + (c ^ x(r)). With 64 banks (16 chunk slots per 256 bytes) the 16 rows a 16-lane
// group reads for the QK^T operand land in 16 distinct slots, and the 8 rows x 2 chunks a
// 32-lane half reads for the transposed PV operand do too.
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
constexpr int kRowChunks = kD / 8;               // 72
constexpr int kTileChunks = kKT * kRowChunks;    // 4608
constexpr int kTileBytes = kTileChunks * 16;     // 73728
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;            // 512
constexpr int kLoadsPerThread = kTileChunks / kThreads;  // 18
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;        // log2 units

__device__ __forceinline__ int swz(int r) {
  return ((r >> 4) & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2);
}
__device__ __forceinline__ int phys_chunk(int r, int c) { return r * kRowChunks + (c ^ swz(r)); }

__device__ __forceinline__ int wave_max_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
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

// Stage one bf16 tile of up to 64 latent rows with direct global->LDS 16-byte loads. Rows
// past nval repeat the last in-range row (finite data; their scores are masked).
__device__ __forceinline__ void load_tile_bf16(char* buf, const __bf16* kv, int64_t row0, int nval,
                                               int wave, int lane) {
#pragma unroll
  for (int n = 0; n < kLoadsPerThread; ++n) {
    const int blk = n * kWaves + wave;     // 64 consecutive physical chunks per wave instruction
    const int p = blk * 64 + lane;
    const int r = p / kRowChunks;
    const int c = (p - r * kRowChunks) ^ swz(r);
    const int rr = min(r, nval - 1);
    const __bf16* src = kv + (row0 + rr) * (int64_t)kD + 8 * c;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(buf + blk * 64 * 16), 16, 0, 0);
  }
}

// Stage one E4M3 tile: codes * block scale -> bf16, RoPE dims copied, written in the same
// swizzled layout as the bf16 tile.
__device__ __forceinline__ void load_tile_e4m3(char* buf, const uint8_t* codes, const float* scales,
                                               const __bf16* rope, int64_t row0, int nval, int tid) {
#pragma unroll 2
  for (int n = 0; n < kLoadsPerThread; ++n) {
    const int idx = n * kThreads + tid;    // logical (row, chunk)
    const int r = idx / kRowChunks, c = idx - r * kRowChunks;
    const int64_t row = row0 + min(r, nval - 1);
    uint4 v;
    if (c < kDN / 8) {
      const uint2 raw = *(const uint2*)(codes + row * kDN + 8 * c);
      const float sc = scales[row * (kDN / 128) + (c >> 4)];
      __bf16 y[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = (__bf16)(e4m3_to_f32((raw.x >> (8 * k)) & 255u) * sc);
#pragma unroll
      for (int k = 0; k < 4; ++k) y[4 + k] = (__bf16)(e4m3_to_f32((raw.y >> (8 * k)) & 255u) * sc);
      v = *(const uint4*)y;
    } else {
      v = *(const uint4*)(rope + row * 64 + 8 * (c - kDN / 8));
    }
    *(uint4*)(buf + phys_chunk(r, c) * 16) = v;
  }
}

}  // namespace

template <bool VROPE, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void k_attn_mfma(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int s_tmax[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  // B operand of S^T = K Q^T: lane holds Q[qvec col][32 s + 8 g + 0..7]
  bf16x8 qf[18];
#pragma unroll
  for (int s = 0; s < 18; ++s) {
    uint4 v = *(const uint4*)(qrow + 32 * s + 8 * g);
    if (!valid) v = make_uint4(0, 0, 0, 0);
    qf[s] = *(bf16x8*)&v;
  }
  // per-lane LDS byte offsets (within a tile buffer, first 32-key block)
  int kaddr_base[2], kaddr_flip[2];
#pragma unroll
  for (int tau = 0; tau < 2; ++tau) {
    const int krow = 8 * ((lane >> 2) & 3) + 4 * tau + (lane & 3);
    const int x = swz(krow);
    kaddr_base[tau] = (krow * kRowChunks + (g ^ (x & 3))) * 16;
    kaddr_flip[tau] = ((x >> 2) & 1) * 64;  // s ^ x2 = s + x2 (s even), s - x2 (s odd)
  }
  int vaddr_base[4];
  {
    const int j = lane & 15;
    const int r0 = 8 * g + (j >> 2);
    const int x = swz(r0);
    const int xp = (x >> 1) & 3, cofs = ((j & 3) >> 1) ^ (x & 1);
#pragma unroll
    for (int b = 0; b < 4; ++b) vaddr_base[b] = (r0 * kRowChunks + 2 * (b ^ xp) + cofs) * 16 + 8 * (j & 1);
  }
  constexpr int NF = VROPE ? 36 : 32;  // 16-feature tiles of O^T
  floatx4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

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
      load_tile_bf16(buf, (const __bf16*)a.kv, row0, c.nval, wave, lane);
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
        qf[s] = y;
      }
      prev_seg = cur.seg;
    }

    const char* buf = lds + (it & 1) * kTileBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int pos_b = cur.pos0 + 32 * kb;
      if (32 * kb >= cur.nval || pos_b > t_wmax) continue;  // uniform per wave
      // S^T for 32 keys as two 16-key tiles; tile tau row m reads key 8 (m/4) + 4 tau + m%4
      // so lane (g, col) ends up with keys 8 g + 0..7 in k-slot order of the PV B operand.
      floatx4 sacc[2];
      sacc[0] = floatx4{0.f, 0.f, 0.f, 0.f};
      sacc[1] = sacc[0];
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        // chunk 4 s + g of row krow sits at krow*72 + 4 (s ^ x2) + (g ^ (x & 3)), x = swz(krow):
        // an even/odd base plus an immediate 64-byte step per s
        const char* kb_even = buf + kaddr_base[tau] + 32 * kb * kRowChunks * 16;
        const char* kb_odd = kb_even - kaddr_flip[tau];
        kb_even += kaddr_flip[tau];
#pragma unroll
        for (int s = 0; s < 18; ++s) {
          const char* p = ((s & 1) ? kb_odd : kb_even) + 64 * s;
          const bf16x8 kf = *(const bf16x8*)p;
          sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sacc[tau], 0, 0, 0);
        }
      }
      // this lane: value (tau, i) = key 8 g + 4 tau + i of the 32-key block, qvec col
      const bool need_mask = (pos_b + 31 > t) || (32 * kb + 32 > cur.nval);
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kp = 8 * g + e;
        float v = sacc[e >> 2][e & 3] * qk_scale;
        if (need_mask && (pos_b + kp > t || 32 * kb + kp >= cur.nval)) v = -INFINITY;
        x[e] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const bool grow = m_new > m_run + kRescaleThreshold;
      if (__ballot(grow) != 0ull) {  // wave-uniform rescale
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
      for (int e = 0; e < 8; ++e) {
        const float p = exp2f(x[e] - m_use);
        lsum += p;
        pf[e] = (__bf16)p;
      }
      l_run += lsum;
      // O^T += V^T P^T: A operand = V^T (16 features x 32 keys) by transposing reads; source
      // lane j of group g supplies key 8 g + j/4 (+4) and features 16 f + 4 (j%4) .. +3.
      // chunk 2 f + cofs of row r0 sits at r0*72 + 2 (f ^ x') + (cofs ^ x0), x' = (x>>1)&3:
      // four bases (f mod 4) plus an immediate 128-byte step per 4 f; row r0 + 4 has the same x
      const char* vb = buf + 32 * kb * kRowChunks * 16;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const char* p = vb + vaddr_base[f & 3] + 128 * (f >> 2);
        const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(p + 4 * kRowChunks * 16));
        const bf16x8 vt = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pf, acc[f], 0, 0, 0);
      }
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
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
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
  const int lds = 2 * kTileBytes;
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
