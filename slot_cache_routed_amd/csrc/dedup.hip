// Distinct experts as a sorted, fixed-length list (no host sync).
//
// The chunk's distinct experts form a sorted list whose length the host
// knows in advance (FreeToken PR #676, Solution, second bullet); each route
// maps back to its entry (same page, gdevenyi's comment).  One workgroup
// marks present ids in LDS, scans the marks and scatters: a counting sort
// over expert ids.
#include "small_blocks.h"

namespace scr {


__global__ __launch_bounds__(kPlanThreads) void dedup_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                          int lmax, int32_t* __restrict__ distinct,
                                                          int32_t* __restrict__ n_distinct,
                                                          int32_t* __restrict__ inverse) {
  __shared__ int pos[kDedupMaxE];
  __shared__ int wave_tot[kWave + 1];
  dedup_block(ids, n, E, lmax, distinct, n_distinct, inverse, pos, wave_tot);
}

}  // namespace scr

extern "C" int scr_dedup(const int32_t* ids, int n, int E, int32_t* distinct, int32_t* n_distinct,
                         int32_t* inverse, hipStream_t stream) {
  SCR_CHECK_ARG(n >= 0, "dedup: n must be >= 0");
  SCR_CHECK_ARG(E >= 1 && E <= scr::kDedupMaxE, "dedup: E must be in [1, %d] (got %d)", scr::kDedupMaxE, E);
  SCR_CHECK_ARG(n_distinct != nullptr, "dedup: n_distinct is null");
  SCR_CHECK_ARG(n == 0 || (ids && distinct), "dedup: null pointer");
  const int lmax = n < E ? n : E;
  hipLaunchKernelGGL(scr::dedup_kernel, dim3(1), dim3(scr::kPlanThreads), 0, stream, ids, n, E,
                     lmax, distinct, n_distinct, inverse);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}
