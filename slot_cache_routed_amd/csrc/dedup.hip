// Distinct experts as a sorted, fixed-length list (no host sync).
//
// The chunk's distinct experts form a sorted list whose length the host
// knows in advance (FreeToken PR #676, Solution, second bullet); each route
// maps back to its entry (same page, gdevenyi's comment).  One workgroup
// marks present ids in LDS, scans the marks and scatters: a counting sort
// over expert ids.
#include "common.h"

namespace scr {

constexpr int kDedupThreads = 1024;
constexpr int kDedupMaxE = 8192;

// inclusive scan of one int per thread across the block; returns the block total
__device__ int block_inclusive_scan(int v, int* wave_tot) {
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) wave_tot[wv] = v;
  __syncthreads();
  if (wv == 0) {
    int t = lane < nw ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(t, off, kWave);
      if (lane >= off) t += o;
    }
    if (lane < nw) wave_tot[lane] = t;
  }
  __syncthreads();
  const int before = wv > 0 ? wave_tot[wv - 1] : 0;
  const int total = wave_tot[nw - 1];
  __syncthreads();
  wave_tot[kWave] = total;
  return v + before;
}

__global__ __launch_bounds__(kDedupThreads) void dedup_kernel(const int32_t* __restrict__ ids, int n,
                                                            int E, int lmax,
                                                            int32_t* __restrict__ distinct,
                                                            int32_t* __restrict__ n_distinct,
                                                            int32_t* __restrict__ inverse) {
  __shared__ int pos[kDedupMaxE];
  __shared__ int wave_tot[kWave + 1];
  for (int e = threadIdx.x; e < E; e += blockDim.x) pos[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ids[i];
    if (e >= 0 && e < E) pos[e] = 1;
  }
  __syncthreads();
  // each thread owns a contiguous run of ids [e0, e1)
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = min(E, (int)threadIdx.x * per), e1 = min(E, e0 + per);
  int cnt = 0;
  for (int e = e0; e < e1; ++e) cnt += pos[e];
  const int incl = block_inclusive_scan(cnt, wave_tot);
  const int total = wave_tot[kWave];
  int p = incl - cnt;
  for (int e = e0; e < e1; ++e) {
    const int present = pos[e];
    if (present) distinct[p] = e;
    pos[e] = present ? p : -1;
    p += present;
  }
  for (int i = total + threadIdx.x; i < lmax; i += blockDim.x) distinct[i] = E;
  if (threadIdx.x == 0) *n_distinct = total;
  if (inverse) {
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int e = ids[i];
      inverse[i] = (e >= 0 && e < E) ? pos[e] : -1;
    }
  }
}

}  // namespace scr

extern "C" int scr_dedup(const int32_t* ids, int n, int E, int32_t* distinct, int32_t* n_distinct,
                         int32_t* inverse, hipStream_t stream) {
  SCR_CHECK_ARG(n >= 0, "dedup: n must be >= 0");
  SCR_CHECK_ARG(E >= 1 && E <= scr::kDedupMaxE, "dedup: E must be in [1, %d] (got %d)", scr::kDedupMaxE, E);
  SCR_CHECK_ARG(n_distinct != nullptr, "dedup: n_distinct is null");
  SCR_CHECK_ARG(n == 0 || (ids && distinct), "dedup: null pointer");
  const int lmax = n < E ? n : E;
  hipLaunchKernelGGL(scr::dedup_kernel, dim3(1), dim3(scr::kDedupThreads), 0, stream, ids, n, E,
                     lmax, distinct, n_distinct, inverse);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}
