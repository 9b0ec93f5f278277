// Row-replacement epilogue (RedKnot-MLA paper, head-partition paragraph Eq. 2 and the
// protected-row paragraph): for every computed (row t, head h) -- Global heads on all rows,
// Local heads on rows of A -- u = [O^nope, R(-t) O^rope] and Z[t][h] = W_h u with W_h the
// head's slice of the bias-free first output projection. On rows outside A the Local heads'
// slots receive the cached contribution Zc[pool_row(t)] unchanged: replaced, never added to.
#include "internal.h"

namespace segmla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// Row t of head h's list: Global heads walk every request row, Local heads walk A.
struct EpiTile {
  int h, r0, n_rows;
  const int32_t* rows;  // null = identity (row index = request row)
};

__device__ __forceinline__ EpiTile epi_tile(const EpiArgs& e, int b, int rows_per_tile) {
  EpiTile et;
  const int tg = (e.T + rows_per_tile - 1) / rows_per_tile;
  if (b < e.HG * tg) {
    et.h = e.ghead[b / tg];
    et.r0 = (b % tg) * rows_per_tile;
    et.n_rows = e.T;
    et.rows = nullptr;
  } else {
    b -= e.HG * tg;
    const int ta = (e.nA + rows_per_tile - 1) / rows_per_tile;
    et.h = e.lhead[b / ta];
    et.r0 = (b % ta) * rows_per_tile;
    et.n_rows = e.nA;
    et.rows = e.alist;
  }
  return et;
}

__device__ __forceinline__ int epi_row(const EpiTile& et, int i) { return et.rows ? et.rows[i] : i; }

// ------------------------------------------------------------------------ fp32 path
// One wavefront per (row, head): u staged in LDS, each lane produces d_state/64 outputs.
__global__ __launch_bounds__(64) void k_project_f32(EpiArgs e) {
  __shared__ float u[1024];
  const int lane = threadIdx.x;
  EpiTile et = epi_tile(e, blockIdx.x, 1);
  if (et.r0 >= et.n_rows) return;
  const int t = epi_row(et, et.r0), h = et.h;
  const float* o = (const float*)e.out + ((int64_t)t * e.H + h) * e.d_v;
  for (int d = lane; d < e.d_v; d += 64) u[d] = o[d];
  __syncthreads();
  if (e.v_has_rope) {
    const int half_r = e.d_rope / 2;
    for (int k = lane; k < half_r; k += 64) {  // u^r <- R(-t) O^r
      float2 cs = e.rowcs[(int64_t)t * half_r + k];
      float x = o[e.d_nope + 2 * k], y = o[e.d_nope + 2 * k + 1];
      u[e.d_nope + 2 * k] = x * cs.x + y * cs.y;
      u[e.d_nope + 2 * k + 1] = -x * cs.y + y * cs.x;
    }
  }
  __syncthreads();
  const float* w = (const float*)e.w + (int64_t)h * e.d_state * e.d_v;
  float* z = (float*)e.z + ((int64_t)t * e.H + h) * e.d_state;
  for (int c = lane; c < e.d_state; c += 64) {
    const float* wr = w + (int64_t)c * e.d_v;
    float acc = 0.f;
    for (int d = 0; d < e.d_v; ++d) acc = fmaf(wr[d], u[d], acc);
    z[c] = acc;
  }
}

// ------------------------------------------------------------------------ bf16 path
// Workgroup = (head, 64 rows of its list) x all d_state columns. U (64 x d_v, RoPE part
// de-rotated in fp32, rounded to bf16) is staged in LDS with a 16-byte row pad so the
// MFMA A-operand reads of 32 rows hit distinct banks; W_h fragments stream from global
// (the slice is shared by all row tiles of the head and stays in L2). 4 waves, each owns
// d_state/4 columns; MFMA 32x32x16 bf16 with fp32 accumulation.
constexpr int kEpiRows = 64;
constexpr int kEpiDv = 576;
constexpr int kEpiChunks = kEpiDv / 8;       // 16-byte chunks per U row
constexpr int kEpiStride = kEpiChunks + 1;   // padded row stride in chunks

__global__ __launch_bounds__(256, 1) void k_project_bf16(EpiArgs e) {
  extern __shared__ __attribute__((aligned(16))) uint4 lds_u[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  EpiTile et = epi_tile(e, blockIdx.x, kEpiRows);
  const int h = et.h;
  const int n_here = min(kEpiRows, et.n_rows - et.r0);
  const int d_v = e.d_v, chunks = d_v / 8, half_r = e.d_rope / 2;
  // stage U
  for (int i = tid; i < kEpiRows * chunks; i += 256) {
    const int r = i / chunks, c = i - r * chunks;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < n_here) {
      const int t = epi_row(et, et.r0 + r);
      const __bf16* src = (const __bf16*)e.out + ((int64_t)t * e.H + h) * d_v + 8 * c;
      v = *(const uint4*)src;
      if (e.v_has_rope && 8 * c >= e.d_nope) {
        const __bf16* x = (const __bf16*)&v;
        __bf16 y[8];
        const int k0 = (8 * c - e.d_nope) / 2;
        for (int p = 0; p < 4; ++p) {
          float2 cs = e.rowcs[(int64_t)t * half_r + k0 + p];
          float a0 = (float)(x[2 * p]), a1 = (float)(x[2 * p + 1]);
          y[2 * p] = (__bf16)(a0 * cs.x + a1 * cs.y);
          y[2 * p + 1] = (__bf16)(-a0 * cs.y + a1 * cs.x);
        }
        v = *(const uint4*)y;
      }
    }
    lds_u[r * kEpiStride + c] = v;
  }
  __syncthreads();
  const int cols_per_wave = e.d_state / 4;      // multiple of 16 (d_state % 64 == 0)
  const int col0 = wave * cols_per_wave;
  const __bf16* w = (const __bf16*)e.w + (int64_t)h * e.d_state * d_v;
  const int ksteps = d_v / 16;
  for (int cb = 0; cb < cols_per_wave; cb += 64) {  // 64 columns x 64 rows per pass
    floatx16_t acc[2][2];
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j)
        for (int k = 0; k < 16; ++k) acc[i][j][k] = 0.f;
    const int ncol = min(64, cols_per_wave - cb);
    for (int ks = 0; ks < ksteps; ++ks) {
      const int chunk = 2 * ks + (lane >> 5);
      bf16x8_t af[2], bfr[2];
      for (int i = 0; i < 2; ++i) {
        uint4 v = lds_u[(32 * i + (lane & 31)) * kEpiStride + chunk];
        af[i] = *(bf16x8_t*)&v;
      }
      for (int j = 0; j < 2; ++j) {
        const int cw = cb + 32 * j + (lane & 31);  // column within this wave's share
        uint4 v = make_uint4(0, 0, 0, 0);
        if (cw < cols_per_wave) v = *(const uint4*)(w + (int64_t)(col0 + cw) * d_v + 8 * chunk);
        bfr[j] = *(bf16x8_t*)&v;
      }
      for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    // C layout: lane holds column lane%32, rows 8*(k/4) + 4*(lane/32) + k%4
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 2; ++j) {
        if (32 * j >= ncol) continue;
        const int cw = cb + 32 * j + (lane & 31);
        const int col = col0 + cw;
        for (int k = 0; k < 16; ++k) {
          const int r = 32 * i + 8 * (k / 4) + 4 * (lane >> 5) + (k % 4);
          if (r < n_here && cw < cols_per_wave) {
            const int t = epi_row(et, et.r0 + r);
            __bf16* z = (__bf16*)e.z + ((int64_t)t * e.H + h) * e.d_state;
            z[col] = (__bf16)(acc[i][j][k]);
          }
        }
      }
  }
}

// ------------------------------------------------------------------- restore copy
// Local heads on rows outside A: Z[t][lhead[l]] = Zc[pool_row(t)][l], copied bit for bit.
template <typename V>
__global__ __launch_bounds__(256) void k_restore_copy(EpiArgs e, int vec_per_head) {
  const int t = e.nalist[blockIdx.x];
  const SegDesc sd = e.seg[e.seg_of_row[t]];
  const int64_t prow = sd.pool_row + (t - sd.offset);
  const V* src = (const V*)e.z_cached + prow * (int64_t)e.HL * vec_per_head;
  V* dst = (V*)e.z + (int64_t)t * e.H * vec_per_head;
  const int n = e.HL * vec_per_head;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int l = i / vec_per_head, c = i - l * vec_per_head;
    dst[(int64_t)e.lhead[l] * vec_per_head + c] = src[i];
  }
}

hipError_t launch_epilogue(const EpiArgs& e, int io_dtype, hipStream_t stream) {
  if (io_dtype == 0) {
    const int64_t blocks = (int64_t)e.HG * e.T + (int64_t)e.HL * e.nA;
    if (blocks > 0)
      hipLaunchKernelGGL(k_project_f32, dim3((unsigned)blocks), dim3(64), 0, stream, e);
    if (e.HL > 0 && e.nNA > 0)
      hipLaunchKernelGGL(k_restore_copy<float>, dim3(e.nNA), dim3(256), 0, stream, e, e.d_state);
  } else {
    const int64_t blocks = (int64_t)e.HG * ((e.T + kEpiRows - 1) / kEpiRows) +
                           (int64_t)e.HL * ((e.nA + kEpiRows - 1) / kEpiRows);
    const size_t lds = sizeof(uint4) * kEpiRows * kEpiStride;
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t r = hipFuncSetAttribute((const void*)k_project_bf16,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (r != hipSuccess) return r;
      attr_set = true;
    }
    if (blocks > 0)
      hipLaunchKernelGGL(k_project_bf16, dim3((unsigned)blocks), dim3(256), lds, stream, e);
    if (e.HL > 0 && e.nNA > 0)
      hipLaunchKernelGGL(k_restore_copy<uint4>, dim3(e.nNA), dim3(256), 0, stream, e,
                         e.d_state * 2 / 16);
  }
  return hipGetLastError();
}

}  // namespace segmla
