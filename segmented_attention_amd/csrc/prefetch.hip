// Artifact prefetch on a stream of the library's own (RedKnot-MLA paper, TP8 fast-path
// paragraph): while one layer runs on the caller's stream, the cached rows a later layer will
// read (latent rows, the cached projected state) are staged into device buffers by copy-engine
// transfers on a dedicated stream; device events order the transfers after the earlier users
// of the destination buffers and the consumer after the transfers, so the host never polls.
#include <hip/hip_runtime.h>

#include <new>

#include "../../include/segmla.h"

struct segmla_prefetcher {
  hipStream_t side = nullptr;
  hipEvent_t free_ev = nullptr;   // caller's stream: work enqueued before the prefetch is done
  hipEvent_t start_ev = nullptr;  // side stream: the transfers begin
  hipEvent_t ready_ev = nullptr;  // side stream: the transfers are done
  bool issued = false;
};

namespace {
void release(segmla_prefetcher* pf) {
  if (pf->side) (void)hipStreamSynchronize(pf->side);
  for (hipEvent_t ev : {pf->free_ev, pf->start_ev, pf->ready_ev})
    if (ev) (void)hipEventDestroy(ev);
  if (pf->side) (void)hipStreamDestroy(pf->side);
  delete pf;
}
}  // namespace

extern "C" {

segmla_status segmla_prefetcher_create(segmla_prefetcher** out) {
  if (!out) return SEGMLA_E_NULL;
  segmla_prefetcher* pf = new (std::nothrow) segmla_prefetcher();
  if (!pf) return SEGMLA_E_UNSUPPORTED;
  // default priority, not synchronizing with the null stream
  if (hipStreamCreateWithFlags(&pf->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&pf->free_ev, hipEventDisableTiming) != hipSuccess ||
      hipEventCreate(&pf->start_ev) != hipSuccess || hipEventCreate(&pf->ready_ev) != hipSuccess) {
    release(pf);
    return SEGMLA_E_HIP;
  }
  *out = pf;
  return SEGMLA_OK;
}

segmla_status segmla_prefetch(segmla_prefetcher* pf, const segmla_copy_range* ranges,
                              int32_t n_ranges, void* after_stream) {
  if (!pf || (!ranges && n_ranges > 0)) return SEGMLA_E_NULL;
  if (n_ranges < 0) return SEGMLA_E_SHAPE;
  for (int32_t i = 0; i < n_ranges; ++i) {
    const segmla_copy_range& r = ranges[i];
    if (r.rows < 0 || r.row_bytes < 1 || r.src_stride < r.row_bytes || r.dst_stride < r.row_bytes)
      return SEGMLA_E_SHAPE;
    if (r.rows > 0 && (!r.src || !r.dst)) return SEGMLA_E_NULL;
  }
  hipError_t e = hipEventRecord(pf->free_ev, (hipStream_t)after_stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(pf->side, pf->free_ev, 0);
  if (e == hipSuccess) e = hipEventRecord(pf->start_ev, pf->side);
  for (int32_t i = 0; i < n_ranges && e == hipSuccess; ++i) {
    const segmla_copy_range& r = ranges[i];
    if (r.rows == 0) continue;
    e = hipMemcpy2DAsync(r.dst, (size_t)r.dst_stride, r.src, (size_t)r.src_stride,
                         (size_t)r.row_bytes, (size_t)r.rows, hipMemcpyDefault, pf->side);
  }
  if (e == hipSuccess) e = hipEventRecord(pf->ready_ev, pf->side);
  pf->issued = e == hipSuccess;
  return e == hipSuccess ? SEGMLA_OK : SEGMLA_E_HIP;
}

segmla_status segmla_prefetch_wait(segmla_prefetcher* pf, void* stream) {
  if (!pf) return SEGMLA_E_NULL;
  if (!pf->issued) return SEGMLA_E_STATE;
  return hipStreamWaitEvent((hipStream_t)stream, pf->ready_ev, 0) == hipSuccess ? SEGMLA_OK
                                                                               : SEGMLA_E_HIP;
}

segmla_status segmla_prefetch_elapsed(segmla_prefetcher* pf, float* ms) {
  if (!pf || !ms) return SEGMLA_E_NULL;
  if (!pf->issued) return SEGMLA_E_STATE;
  if (hipEventSynchronize(pf->ready_ev) != hipSuccess) return SEGMLA_E_HIP;
  return hipEventElapsedTime(ms, pf->start_ev, pf->ready_ev) == hipSuccess ? SEGMLA_OK
                                                                           : SEGMLA_E_HIP;
}

void segmla_prefetcher_destroy(segmla_prefetcher* pf) {
  if (pf) release(pf);
}

}  // extern "C"
