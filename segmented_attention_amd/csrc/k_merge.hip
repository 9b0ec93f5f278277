// Stable log-sum-exp merge of split attention partials (RedKnot-MLA paper, relocation
// paragraph): M = max_s m_s, O = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s,
// lse = M + log(sum_s e^(m_s - M) l_s). One wavefront per vector, channels across lanes.
#include <cmath>
#include "internal.h"

namespace segmla {

namespace {
__device__ __forceinline__ void store(float* p, float v) { *p = v; }
__device__ __forceinline__ void store(__bf16* p, float v) { *p = (__bf16)v; }

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const __bf16* p) { return (float)*p; }

// Merge one vector: partial index base_v in split-major arrays of n_vec vectors.
template <typename OutT, typename PartT = float>
__device__ __forceinline__ void merge_vec(const PartT* __restrict__ part_o,
                                          const float* __restrict__ part_ml, int n_split,
                                          int64_t n_vec, int64_t v, int d, OutT* __restrict__ dst,
                                          float* __restrict__ lse_dst, int lane) {
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[((int64_t)s * n_vec + v) * 2]);
  float den = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float* ml = part_ml + ((int64_t)s * n_vec + v) * 2;
    if (ml[0] != -INFINITY) den += expf(ml[0] - M) * ml[1];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int c = lane; c < d; c += 64) {
    float num = 0.f;
    for (int s = 0; s < n_split; ++s) {
      float ms = part_ml[((int64_t)s * n_vec + v) * 2];
      if (ms != -INFINITY) num += expf(ms - M) * ld(part_o + ((int64_t)s * n_vec + v) * d + c);
    }
    store(dst + c, num * inv);
  }
  if (lse_dst && lane == 0) *lse_dst = den > 0.f ? M + logf(den) : -INFINITY;
}
}  // namespace

template <typename OutT>
__global__ __launch_bounds__(256) void k_lse_merge(const float* __restrict__ part_o,
                                                   const float* __restrict__ part_ml, int n_split,
                                                   int64_t n_vec, int d, OutT* __restrict__ out,
                                                   float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= n_vec) return;
  merge_vec(part_o, part_ml, n_split, n_vec, v, d, out + v * d, lse ? lse + v : nullptr, lane);
}

constexpr int kWideMergeSplits = 16;   // from this many splits on, the wide merge
constexpr int kWideMaxSplits = 4096;   // its LDS weight table
constexpr int kWideChunk = 64;         // channels per workgroup
constexpr int kWideLoads = 8;          // 16-byte partial loads in flight per thread and pass

// Forward's merge: vector v = tile * kTileQ + qi goes to out[t][h]; only the splits the
// attention wrote (split start <= the tile's largest row) are read. Partials are fp32, or bf16
// from the decode kernel.
template <typename OutT, typename PartT>
__global__ __launch_bounds__(256) void k_merge_tiles(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= nvec) return;
  const int tile = (int)(v / kTileQ), qi = (int)(v % kTileQ);
  int t, h;
  if (!tile_qvec(a.map, tile, qi, t, h)) return;
  const int n_valid = min(a.n_split, tile_max_row(a.map, tile) / a.split_keys + 1);
  const int64_t o = (int64_t)(t - a.q0) * a.map.H + h;
  merge_vec((const PartT*)a.part_o, a.part_ml, n_valid, nvec, v, a.d_v, (OutT*)a.out + o * a.d_v,
            a.lse ? a.lse + o : nullptr, lane);
}

// The same merge for many splits of few vectors (decode: a few rows against a long context),
// laid out so that a workgroup's loads are all in flight at once. Workgroup = (vector, 64
// channels); thread (slot, g) owns CPL channels (one 16-byte load: 8 bf16 or 4 fp32 partial
// values) and the splits slot, slot + SS, ... of each pass, kWideLoads of them, loaded before
// anything waits on them. The split weights e^(m_s - M) are computed into LDS while the first
// pass is in flight (its (m, l) loads are issued first and retire first). A split past the
// vector's last rereads the last one with weight 0. The slots' sums meet by lane shuffles,
// then across the four waves in LDS.

// the CPL partial values of one 16-byte load, as fp32
__device__ __forceinline__ void unpack16(const uint4& x, float* f, const float*) {
  f[0] = __uint_as_float(x.x);
  f[1] = __uint_as_float(x.y);
  f[2] = __uint_as_float(x.z);
  f[3] = __uint_as_float(x.w);
}
__device__ __forceinline__ void unpack16(const uint4& x, float* f, const __bf16*) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename OutT, typename PartT>
__global__ __launch_bounds__(256) void k_merge_tiles_wide(AttnArgs a) {
  constexpr int CPL = 16 / (int)sizeof(PartT);  // channels per thread: 8 (bf16) or 4 (fp32)
  constexpr int CG = kWideChunk / CPL;          // channel groups per chunk: 8 or 16
  constexpr int SS = 256 / CG;                  // split slots: 32 or 16
  constexpr int PASS = SS * kWideLoads;         // splits per pass: 256 or 128
  static_assert(CG <= 64 && 64 % CG == 0, "a wave holds whole split slots");
  __shared__ float sw[kWideMaxSplits], sl[kWideMaxSplits];
  __shared__ float red[2][4];
  __shared__ float accs[4][kWideChunk];
  const int nchunk = (a.d_v + kWideChunk - 1) / kWideChunk;
  const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
  const int64_t v = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const int tile = (int)(v / kTileQ), qi = (int)(v % kTileQ);
  int t, h;
  if (!tile_qvec(a.map, tile, qi, t, h)) return;  // uniform over the workgroup
  const int n = min(a.n_split, tile_max_row(a.map, tile) / a.split_keys + 1);  // >= 1
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = tid / CG, g = tid % CG;
  const int c = chunk * kWideChunk + g * CPL;
  const bool on = c < a.d_v;  // d_v is a multiple of CPL: a group is wholly in or out
  const int64_t sstride = nvec * a.d_v;
  const PartT* po = (const PartT*)a.part_o + v * a.d_v + (on ? c : 0);
  const float* pml = a.part_ml + v * 2;
  // (m, l) of the first 256 splits, then the first pass of partials
  float2 ml0 = make_float2(-INFINITY, 0.f);
  if (tid < n) ml0 = *(const float2*)(pml + (int64_t)tid * nvec * 2);
  uint4 x[kWideLoads];
  auto load_pass = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kWideLoads; ++k) {
      const int s = min(s0 + slot + SS * k, n - 1);
      x[k] = *(const uint4*)(po + (int64_t)s * sstride);
    }
  };
  load_pass(0);
  float m = ml0.x;
  if (tid < n) {
    sw[tid] = ml0.x;
    sl[tid] = ml0.y;
  }
  for (int s = tid + 256; s < n; s += 256) {  // more than 256 splits
    const float2 ml = *(const float2*)(pml + (int64_t)s * nvec * 2);
    sw[s] = ml.x;
    sl[s] = ml.y;
    m = fmaxf(m, ml.x);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[0][wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float den = 0.f;
  for (int s = tid; s < n; s += 256) {  // the entries this thread wrote above
    const float ms = sw[s];
    const float w = ms == -INFINITY ? 0.f : expf(ms - M);
    sw[s] = w;
    den += w * sl[s];
  }
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
  if (lane == 0) red[1][wave] = den;
  __syncthreads();
  float acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < n; s0 += PASS) {
    if (s0 > 0) load_pass(s0);
#pragma unroll
    for (int k = 0; k < kWideLoads; ++k) {
      const int s = s0 + slot + SS * k;
      const float w = s < n ? sw[s] : 0.f;
      float f[CPL];
      unpack16(x[k], f, (const PartT*)nullptr);
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] = fmaf(w, f[i], acc[i]);
    }
  }
  // sum over the split slots of the wave (lanes g, g + CG, ...), then over the waves
#pragma unroll
  for (int i = 0; i < CPL; ++i)
    for (int o = CG; o < 64; o <<= 1) acc[i] += __shfl_xor(acc[i], o);
  if (lane < CG) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) accs[wave][lane * CPL + i] = acc[i];
  }
  __syncthreads();
  const float dt = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const float inv = dt > 0.f ? 1.f / dt : 0.f;
  const int64_t o = (int64_t)(t - a.q0) * a.map.H + h;
  const int ch = chunk * kWideChunk + tid;
  if (tid < kWideChunk && ch < a.d_v)
    store((OutT*)a.out + o * a.d_v + ch, (accs[0][tid] + accs[1][tid] + accs[2][tid] + accs[3][tid]) * inv);
  if (a.lse && chunk == 0 && tid == 0) a.lse[o] = dt > 0.f ? M + logf(dt) : -INFINITY;
}

hipError_t launch_lse_merge(const float* part_o, const float* part_ml, int n_split, int64_t n_vec,
                            int d, void* out, int out_dtype, float* lse, hipStream_t stream) {
  const int64_t blocks = (n_vec + 3) / 4;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (out_dtype == 0)
    hipLaunchKernelGGL(k_lse_merge<float>, dim3((unsigned)blocks), dim3(256), 0, stream, part_o,
                       part_ml, n_split, n_vec, d, (float*)out, lse);
  else
    hipLaunchKernelGGL(k_lse_merge<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       part_o, part_ml, n_split, n_vec, d, (__bf16*)out, lse);
  return hipGetLastError();
}

hipError_t launch_merge_tiles(const AttnArgs& a, int io_dtype, hipStream_t stream) {
  const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
  if (a.n_split >= kWideMergeSplits && a.n_split <= kWideMaxSplits &&
      a.d_v % (a.part_bf16 && io_dtype != 0 ? 8 : 4) == 0) {
    const int64_t blocks = nvec * ((a.d_v + kWideChunk - 1) / kWideChunk);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    if (a.part_bf16 && io_dtype != 0)
      hipLaunchKernelGGL((k_merge_tiles_wide<__bf16, __bf16>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (io_dtype == 0)
      hipLaunchKernelGGL((k_merge_tiles_wide<float, float>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_merge_tiles_wide<__bf16, float>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t blocks = (nvec + 3) / 4;
  if (a.part_bf16 && io_dtype != 0)
    hipLaunchKernelGGL((k_merge_tiles<__bf16, __bf16>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else if (io_dtype == 0)
    hipLaunchKernelGGL((k_merge_tiles<float, float>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_merge_tiles<__bf16, float>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace segmla
