// Stable log-sum-exp merge of split attention partials (RedKnot-MLA paper, relocation
// paragraph): M = max_s m_s, O = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s,
// lse = M + log(sum_s e^(m_s - M) l_s). One wavefront per vector, channels across lanes.
#include <cmath>
#include "internal.h"

namespace segmla {

namespace {
__device__ __forceinline__ void store(float* p, float v) { *p = v; }
__device__ __forceinline__ void store(__bf16* p, float v) { *p = (__bf16)v; }

// Merge one vector: partial index base_v in split-major arrays of n_vec vectors.
template <typename OutT>
__device__ __forceinline__ void merge_vec(const float* __restrict__ part_o,
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
      if (ms != -INFINITY) num += expf(ms - M) * part_o[((int64_t)s * n_vec + v) * d + c];
    }
    store(dst + c, num * inv);
  }
  if (lse_dst && lane == 0) *lse_dst = den > 0.f ? M + logf(den) : -INFINITY;
}
// The same merge of one vector by a whole workgroup, for many splits (decode: a few rows
// against a long context): wave w takes splits w, w + 4, ...; each lane accumulates all of its
// channels (lane + 64 k) for a split at once, so that those loads are in flight together; the
// waves' partial sums meet in LDS. d <= 64 * kWideCh.
constexpr int kWideCh = 9;
template <typename OutT>
__device__ __forceinline__ void merge_vec_wide(const float* __restrict__ part_o,
                                               const float* __restrict__ part_ml, int n_split,
                                               int64_t n_vec, int64_t v, int d,
                                               OutT* __restrict__ dst, float* __restrict__ lse_dst) {
  __shared__ float red[4], dens[4];
  __shared__ float accs[4][64 * kWideCh];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float m = -INFINITY;
  for (int s = tid; s < n_split; s += 256) m = fmaxf(m, part_ml[((int64_t)s * n_vec + v) * 2]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float den = 0.f, acc[kWideCh];
#pragma unroll
  for (int k = 0; k < kWideCh; ++k) acc[k] = 0.f;
#pragma unroll 2
  for (int s = wave; s < n_split; s += 4) {
    const float* ml = part_ml + ((int64_t)s * n_vec + v) * 2;
    const float ms = ml[0];
    if (ms == -INFINITY) continue;  // the split saw no key of this vector
    const float w = expf(ms - M);
    den += w * ml[1];
    const float* o = part_o + ((int64_t)s * n_vec + v) * d;
#pragma unroll
    for (int k = 0; k < kWideCh; ++k) {
      const int c = lane + 64 * k;
      if (c < d) acc[k] += w * o[c];
    }
  }
#pragma unroll
  for (int k = 0; k < kWideCh; ++k) accs[wave][lane + 64 * k] = acc[k];
  if (lane == 0) dens[wave] = den;
  __syncthreads();
  const float dt = dens[0] + dens[1] + dens[2] + dens[3];
  const float inv = dt > 0.f ? 1.f / dt : 0.f;
  for (int c = tid; c < d; c += 256)
    store(dst + c, (accs[0][c] + accs[1][c] + accs[2][c] + accs[3][c]) * inv);
  if (lse_dst && tid == 0) *lse_dst = dt > 0.f ? M + logf(dt) : -INFINITY;
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

constexpr int kWideMergeSplits = 16;  // from this many splits on, a workgroup per vector

// Forward's merge: vector v = tile * kTileQ + qi goes to out[t][h]; only the splits the
// attention wrote (split start <= the tile's largest row) are read.
template <typename OutT>
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
  merge_vec(a.part_o, a.part_ml, n_valid, nvec, v, a.d_v, (OutT*)a.out + o * a.d_v,
            a.lse ? a.lse + o : nullptr, lane);
}

// One workgroup per vector (merge_vec_wide), for many splits.
template <typename OutT>
__global__ __launch_bounds__(256) void k_merge_tiles_wide(AttnArgs a) {
  const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
  const int64_t v = blockIdx.x;
  const int tile = (int)(v / kTileQ), qi = (int)(v % kTileQ);
  int t, h;
  if (!tile_qvec(a.map, tile, qi, t, h)) return;  // uniform over the workgroup
  const int n_valid = min(a.n_split, tile_max_row(a.map, tile) / a.split_keys + 1);
  const int64_t o = (int64_t)(t - a.q0) * a.map.H + h;
  merge_vec_wide(a.part_o, a.part_ml, n_valid, nvec, v, a.d_v, (OutT*)a.out + o * a.d_v,
                 a.lse ? a.lse + o : nullptr);
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
  if (a.n_split >= kWideMergeSplits && a.d_v <= 64 * kWideCh) {
    if (nvec > INT32_MAX) return hipErrorInvalidConfiguration;
    if (io_dtype == 0)
      hipLaunchKernelGGL(k_merge_tiles_wide<float>, dim3((unsigned)nvec), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(k_merge_tiles_wide<__bf16>, dim3((unsigned)nvec), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t blocks = (nvec + 3) / 4;
  if (io_dtype == 0)
    hipLaunchKernelGGL(k_merge_tiles<float>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_merge_tiles<__bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace segmla
