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
constexpr int kWideChunk = 256;        // channels per workgroup (4 per lane)
constexpr int kWideBatch = 16;         // splits whose loads a lane has in flight at once

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

// The same merge for many splits (decode: a few rows against a long context), laid out for
// bandwidth: workgroup = (vector, 256 channels). The split weights e^(m_s - M) are computed
// once into LDS; then wave w sums splits w, w + 4, ... with each lane holding 4 channels and
// kWideBatch splits' loads in flight per batch, no branch between them (a split that saw no
// key of the vector has weight 0 and a zero partial). The four waves' sums meet in LDS.
__device__ __forceinline__ void store4(float* p, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ void store4(__bf16* p, float4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 y = {(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w};
  *(bf16x4*)p = y;
}
__device__ __forceinline__ void fma4(float4& acc, float w, const float4& x) {
  acc.x = fmaf(w, x.x, acc.x);
  acc.y = fmaf(w, x.y, acc.y);
  acc.z = fmaf(w, x.z, acc.z);
  acc.w = fmaf(w, x.w, acc.w);
}

// partials of four channels: fp32, or bf16 (the decode kernel's)
__device__ __forceinline__ float4 load4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load4(const __bf16* p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 y = *(const bf16x4*)p;
  return make_float4((float)y[0], (float)y[1], (float)y[2], (float)y[3]);
}

template <typename OutT, typename PartT>
__global__ __launch_bounds__(256) void k_merge_tiles_wide(AttnArgs a) {
  __shared__ float sw[kWideMaxSplits], sl[kWideMaxSplits];
  __shared__ float red[4], dens[4];
  __shared__ float4 accs[3][64];
  const int nchunk = (a.d_v + kWideChunk - 1) / kWideChunk;
  const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
  const int64_t v = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const int tile = (int)(v / kTileQ), qi = (int)(v % kTileQ);
  int t, h;
  if (!tile_qvec(a.map, tile, qi, t, h)) return;  // uniform over the workgroup
  const int n = min(a.n_split, tile_max_row(a.map, tile) / a.split_keys + 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // every split's (m, l) first, then this wave's first batch of partials: the batch is in
  // flight while the weights are computed (loads retire in order, so the (m, l) wait does not
  // include the batch)
  float m = -INFINITY;
  for (int s = tid; s < n; s += 256) {
    const float2 ml = *(const float2*)(a.part_ml + ((int64_t)s * nvec + v) * 2);
    sw[s] = ml.x;
    sl[s] = ml.y;
    m = fmaxf(m, ml.x);
  }
  const int c = chunk * kWideChunk + 4 * lane;
  const bool on = c < a.d_v;
  const int64_t sstride = nvec * a.d_v;
  const PartT* po = (const PartT*)a.part_o + v * a.d_v + (on ? c : 0);
  float4 x[kWideBatch];
  auto load_batch = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kWideBatch; ++k) {  // past the last split: reread split s, weight 0
      const int sk = s + 4 * k < n ? s + 4 * k : s;
      x[k] = load4(po + (int64_t)sk * sstride);
    }
  };
  if (wave < n) load_batch(wave);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float den = 0.f;
  for (int s = tid; s < n; s += 256) {  // the same entries this thread wrote above
    const float ms = sw[s];
    const float w = ms == -INFINITY ? 0.f : expf(ms - M);
    sw[s] = w;
    den += w * sl[s];
  }
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
  if (lane == 0) dens[wave] = den;
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = wave; s < n; s += 4 * kWideBatch) {
    if (s != wave) load_batch(s);
#pragma unroll
    for (int k = 0; k < kWideBatch; ++k) fma4(acc, s + 4 * k < n ? sw[s + 4 * k] : 0.f, x[k]);
  }
  if (wave > 0) accs[wave - 1][lane] = acc;
  __syncthreads();
  if (wave > 0) return;
  const float dt = dens[0] + dens[1] + dens[2] + dens[3];
  const float inv = dt > 0.f ? 1.f / dt : 0.f;
  const int64_t o = (int64_t)(t - a.q0) * a.map.H + h;
  if (on) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      acc.x += accs[w][lane].x;
      acc.y += accs[w][lane].y;
      acc.z += accs[w][lane].z;
      acc.w += accs[w][lane].w;
    }
    store4((OutT*)a.out + o * a.d_v + c, make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
  }
  if (a.lse && chunk == 0 && lane == 0) a.lse[o] = dt > 0.f ? M + logf(dt) : -INFINITY;
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
  if (a.n_split >= kWideMergeSplits && a.n_split <= kWideMaxSplits && a.d_v % 4 == 0) {
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
