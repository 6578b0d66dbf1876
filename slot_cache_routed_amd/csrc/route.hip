// Top-k softmax routing: one wavefront per token.
//
// Each token is routed to its k largest logits before any expert is loaded
// (FreeToken PR #676, Known limits; FreeToken PR #68, first commit).  The
// weights are the softmax of the k selected logits; they are formed in fp64
// and rounded once to fp32, so they do not depend on the order of lanes.
#include "common.h"

#include <math.h>

namespace scr {

// Lane l holds logits l, l+64, l+128, ... (VPL of them, E <= 64*VPL).  Each of
// the k rounds takes every lane's best untaken value, then a butterfly over
// the wave keeps the larger value (lower id on ties); the owning lane marks
// it taken.  Lane j keeps the j-th selection.
template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? row[e] : 0.0f;
  }
  uint64_t taken = 0;
  float my_val = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      const bool ok = e < E && !((taken >> i) & 1ull);
      if (ok && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, kWave);
      const int oi = __shfl_xor(bi, off, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1ull << (bi / kWave);
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
  }
  // softmax over the selection, in fp64, summed in rank order
  const double top = (double)__shfl(my_val, 0, kWave);
  const double ex = lane < k ? exp((double)my_val - top) : 0.0;
  double s = 0.0;
  for (int j = 0; j < k; ++j) s += __shfl(ex, j, kWave);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = (float)(ex / s);
  }
}

template <int VPL>
static int launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block);
  hipLaunchKernelGGL(route_kernel<VPL>, grid, dim3(waves_per_block * kWave), 0, s, logits, T, E, k,
                     ids, w);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

}  // namespace scr

extern "C" int scr_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                         hipStream_t stream) {
  SCR_CHECK_ARG(T >= 0, "route: T must be >= 0 (got %d)", T);
  SCR_CHECK_ARG(E >= 1 && E <= SCR_MAX_EXPERTS, "route: E must be in [1, %d] (got %d)",
                SCR_MAX_EXPERTS, E);
  SCR_CHECK_ARG(k >= 1 && k <= E && k <= SCR_MAX_TOPK, "route: k must be in [1, min(E, %d)] (got %d)",
                SCR_MAX_TOPK, k);
  if (T == 0) return SCR_OK;
  SCR_CHECK_ARG(logits && topk_ids && topk_w, "route: null pointer");
  const int vpl = (E + 63) / 64;
  if (vpl <= 1) return scr::launch_route<1>(logits, T, E, k, topk_ids, topk_w, stream);
  if (vpl <= 2) return scr::launch_route<2>(logits, T, E, k, topk_ids, topk_w, stream);
  if (vpl <= 4) return scr::launch_route<4>(logits, T, E, k, topk_ids, topk_w, stream);
  if (vpl <= 8) return scr::launch_route<8>(logits, T, E, k, topk_ids, topk_w, stream);
  if (vpl <= 16) return scr::launch_route<16>(logits, T, E, k, topk_ids, topk_w, stream);
  if (vpl <= 32) return scr::launch_route<32>(logits, T, E, k, topk_ids, topk_w, stream);
  return scr::launch_route<64>(logits, T, E, k, topk_ids, topk_w, stream);
}
