// fp32 segment-relocated attention (any even d_rope, d_nope + d_rope <= 1024).
//
// One wavefront per query vector (row t, head h). For every segment with keys visible from
// t, the query's RoPE part is rotated by -rot_i, the stored latent rows are attended in
// place (keys 64 at a time, one key per lane, wave-shuffle max/sum), and the running output
// accumulator, kept in the current segment's RoPE frame, is moved to the next segment's
// frame by R(rot_i - rot_{i+1}); at the end R(rot_last) restores the request phase. The
// single online softmax across segments is the running form of the log-sum-exp merge of
// per-segment (max, sum, partial) statistics (RedKnot-MLA paper, relocation paragraph).
#include <cmath>
#include "internal.h"

namespace segmla {

namespace {
constexpr int kMaxPairsPerLane = 8;  // d_v <= 1024 -> <= 512 pairs -> 8 per lane

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
}  // namespace

// WIN: the W tiles (sink + window heads), in order, never split: key p is visible from row t
// iff p <= t and (p < n_sink or p >= t - win) (RedKnot explainer, "Insight 1"); 64-key chunks
// with no visible key are skipped (they would leave the running state unchanged).
template <bool WIN>
__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
  __shared__ float qs[1024];   // query, RoPE part rotated for the current segment
  __shared__ float q0[1024];   // query as stored
  const int lane = threadIdx.x;
  const int qi = blockIdx.x % kTileQ;
  const int item = blockIdx.x / kTileQ;
  const int rank = WIN ? item : item / a.n_split, split = WIN ? 0 : item % a.n_split;
  const int tile = WIN ? a.map.nF + a.map.nG + rank : a.work[rank];
  if (tile < 0 || tile >= a.map.nF + a.map.nG + (WIN ? a.map.nW : 0)) return;
  int t, h;
  if (!tile_qvec(a.map, tile, qi, t, h)) return;
  const int d_qk = a.d_nope + a.d_rope, d_v = a.d_v, half_r = a.d_rope / 2;
  const int S = a.split_keys;
  int k_lo = 0, k_hi = t + 1;
  if (!WIN && a.n_split > 1) {
    k_lo = split * S;
    if (k_lo > tile_max_row(a.map, tile)) return;  // this split is not read by the merge
    k_hi = min(k_hi, k_lo + S);
  }
  const float* q = (const float*)a.q + ((int64_t)(t - a.q0) * a.map.H + h) * d_qk;
  for (int d = lane; d < d_qk; d += 64) q0[d] = q[d];
  const float* kv = (const float*)a.kv;

  float acc[2 * kMaxPairsPerLane];
  for (int i = 0; i < 2 * kMaxPairsPerLane; ++i) acc[i] = 0.f;
  const int n_pairs = (d_v + 1) / 2;
  float m = -INFINITY, l = 0.f;
  int prev_seg = -1;
  if (k_lo < k_hi) {
    int si = seg_of(a.seg, a.n_seg, k_lo);
    for (; si < a.n_seg && a.seg[si].offset < k_hi; ++si) {
      const SegDesc sd = a.seg[si];
      if (prev_seg >= 0) {  // move the accumulated output into this segment's RoPE frame
        for (int r = 0; r < kMaxPairsPerLane; ++r) {
          int p = lane + 64 * r, d0 = 2 * p;
          if (p < n_pairs && d0 >= a.d_nope && d0 + 1 < d_v) {
            float2 cs = a.stepcs[prev_seg * half_r + (d0 - a.d_nope) / 2];
            float x = acc[2 * r], y = acc[2 * r + 1];
            acc[2 * r] = x * cs.x - y * cs.y;
            acc[2 * r + 1] = x * cs.y + y * cs.x;
          }
        }
      }
      prev_seg = si;
      __syncthreads();
      for (int d = lane; d < d_qk; d += 64) qs[d] = q0[d];
      for (int k = lane; k < half_r; k += 64) {  // q^r <- R(-rot_i) q^r
        float2 cs = a.segcs[si * half_r + k];
        float x = q0[a.d_nope + 2 * k], y = q0[a.d_nope + 2 * k + 1];
        qs[a.d_nope + 2 * k] = x * cs.x + y * cs.y;
        qs[a.d_nope + 2 * k + 1] = -x * cs.y + y * cs.x;
      }
      __syncthreads();
      const int j_lo = max(0, k_lo - sd.offset), j_hi = min(sd.len, k_hi - sd.offset);
      for (int j0 = j_lo; j0 < j_hi; j0 += 64) {
        const int j = j0 + lane;
        if (WIN) {  // uniform: no key of the chunk in the sink or the window
          const int p_lo = sd.offset + j0, p_hi = sd.offset + min(j0 + 64, j_hi) - 1;
          if (p_lo >= a.n_sink && p_hi < t - a.win) continue;
        }
        const int pos = sd.offset + j;
        const bool valid = j < j_hi && (!WIN || pos < a.n_sink || pos >= t - a.win);
        const float* krow = kv + (sd.pool_row + (valid ? j : j0)) * (int64_t)d_qk;
        float s = -INFINITY;
        if (valid) {
          float dot = 0.f;
          for (int d = 0; d < d_qk; ++d) dot = fmaf(qs[d], krow[d], dot);
          s = a.sigma * dot;
        }
        const float m_new = fmaxf(m, wave_max(s));
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
        const float p = valid ? expf(s - m_new) : 0.f;
        l = l * alpha + wave_sum(p);
        m = m_new;
        for (int i = 0; i < 2 * kMaxPairsPerLane; ++i) acc[i] *= alpha;
        const int nk = min(64, j_hi - j0);
        for (int k = 0; k < nk; ++k) {
          const float pk = __shfl(p, k);
          if (WIN && pk == 0.f) continue;  // a masked key (uniform: the value is shuffled)
          const float* vrow = kv + (sd.pool_row + j0 + k) * (int64_t)d_qk;
          for (int r = 0; r < kMaxPairsPerLane; ++r) {
            int d0 = 2 * (lane + 64 * r);
            if (d0 < d_v) acc[2 * r] = fmaf(pk, vrow[d0], acc[2 * r]);
            if (d0 + 1 < d_v) acc[2 * r + 1] = fmaf(pk, vrow[d0 + 1], acc[2 * r + 1]);
          }
        }
      }
    }
  }
  if (prev_seg >= 0) {  // restore the request phase: R(+rot_last)
    for (int r = 0; r < kMaxPairsPerLane; ++r) {
      int p = lane + 64 * r, d0 = 2 * p;
      if (p < n_pairs && d0 >= a.d_nope && d0 + 1 < d_v) {
        float2 cs = a.segcs[prev_seg * half_r + (d0 - a.d_nope) / 2];
        float x = acc[2 * r], y = acc[2 * r + 1];
        acc[2 * r] = x * cs.x - y * cs.y;
        acc[2 * r + 1] = x * cs.y + y * cs.x;
      }
    }
  }
  if (a.n_split > 1) {
    const int64_t nvec = (int64_t)(a.map.nF + a.map.nG) * kTileQ;
    const int64_t v = (int64_t)tile * kTileQ + qi;
    float* po = a.part_o + ((int64_t)split * nvec + v) * d_v;
    for (int r = 0; r < kMaxPairsPerLane; ++r) {
      int d0 = 2 * (lane + 64 * r);
      if (d0 < d_v) po[d0] = acc[2 * r];
      if (d0 + 1 < d_v) po[d0 + 1] = acc[2 * r + 1];
    }
    if (lane == 0) {
      float* pm = a.part_ml + ((int64_t)split * nvec + v) * 2;
      pm[0] = m;
      pm[1] = l;
    }
    return;
  }
  const float inv = 1.f / l;
  float* o = (float*)a.out + ((int64_t)(t - a.q0) * a.map.H + h) * d_v;
  for (int r = 0; r < kMaxPairsPerLane; ++r) {
    int d0 = 2 * (lane + 64 * r);
    if (d0 < d_v) o[d0] = acc[2 * r] * inv;
    if (d0 + 1 < d_v) o[d0 + 1] = acc[2 * r + 1] * inv;
  }
  if (a.lse && lane == 0) a.lse[(int64_t)(t - a.q0) * a.map.H + h] = m + logf(l);
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)(a.map.nF + a.map.nG) * a.n_split;
  const int64_t blocks = items * kTileQ;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_f32<false>, dim3((unsigned)blocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_f32_window(const AttnArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.map.nW * kTileQ;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_f32<true>, dim3((unsigned)blocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace segmla
