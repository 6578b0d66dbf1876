// Top-k softmax routing: one wavefront per token.
//
// Each token is routed to its k largest logits before any expert is loaded
// (FreeToken PR #676, Known limits; FreeToken PR #68, first commit).  The
// weights are the softmax of the k selected logits; they are formed in fp64
// and rounded once to fp32, so they do not depend on the order of lanes.
#include "common.h"

#include <math.h>

#include <type_traits>

namespace scr {

// float -> u32 with the same order (non-NaN inputs; -0 is first made +0, so
// that equal logits compare equal) and back
__device__ __forceinline__ unsigned ordered_key(float f) {
  const unsigned u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One DPP move of x; lanes whose source lies outside the pattern, or whose
// row is masked off, get IDENT, the identity of the reduction (so that the
// compiler folds the move into the max or min itself).
template <int CTRL, int ROW_MASK, unsigned IDENT>
__device__ __forceinline__ unsigned dpp_mov(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)IDENT, (int)x, CTRL, ROW_MASK, 0xf, false);
}

// Wave-wide max / min of an unsigned value by DPP: a shift-right ladder of
// 1, 2, 4 and 8 lanes leaves each 16-lane row's result in its lane 15; a
// broadcast of lane 15 into rows 1 and 3, then of lane 31 into rows 2 and 3,
// folds the four rows into lane 63, which is read back to every lane.
template <bool MAX>
__device__ __forceinline__ unsigned wave_reduce_u32(unsigned x) {
  auto op = [](unsigned a, unsigned b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  constexpr unsigned I = MAX ? 0u : 0xFFFFFFFFu;  // the identity
  x = op(x, dpp_mov<0x111, 0xf, I>(x));  // row_shr:1
  x = op(x, dpp_mov<0x112, 0xf, I>(x));  // row_shr:2
  x = op(x, dpp_mov<0x114, 0xf, I>(x));  // row_shr:4
  x = op(x, dpp_mov<0x118, 0xf, I>(x));  // row_shr:8
  x = op(x, dpp_mov<0x142, 0xa, I>(x));  // row_bcast:15
  x = op(x, dpp_mov<0x143, 0xc, I>(x));  // row_bcast:31
  return (unsigned)__builtin_amdgcn_readlane((int)x, 63);
}

// Lane l holds logits l, l+64, l+128, ... (VPL of them, E <= 64*VPL) as
// ordered keys (every finite or infinite key is above 0, the "taken" mark).
// Each of the k rounds takes every lane's best untaken key (lowest id on
// ties: a tree of maxima, then the lowest slot holding the maximum), the
// wave's largest key by a DPP reduction (wave_reduce_u32), then the lowest id among the lanes
// holding it: a ballot of those lanes, and when there is more than one (equal
// logits), a second reduction.  The owning lane marks the key taken.  Lane j
// keeps the j-th selection.
template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  // every load is issued (lanes past E read the last logit and drop it), so
  // that all VPL of them are in flight together
  unsigned key[VPL];
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = row[e < E ? e : E - 1];
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) key[i] = lane + kWave * i < E ? ordered_key(v[i]) : 0u;
  unsigned my_key = 0u;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    unsigned bk[VPL];  // tree of maxima over the slots
#pragma unroll
    for (int i = 0; i < VPL; ++i) bk[i] = key[i];
#pragma unroll
    for (int st = 1; st < VPL; st *= 2)
#pragma unroll
      for (int m = 0; m + st < VPL; m += 2 * st) bk[m] = bk[m] > bk[m + st] ? bk[m] : bk[m + st];
    const unsigned lk = bk[0];
    // the lowest slot holding it (the lowest id of the lane)
    typedef typename std::conditional<(VPL > 32), unsigned long long, unsigned>::type SlotMask;
    SlotMask held = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) held |= key[i] == lk ? (SlotMask)1 << i : (SlotMask)0;
    const int slot = VPL > 32 ? __builtin_ctzll((unsigned long long)held) : __builtin_ctz((unsigned)held);
    const unsigned li = lk ? (unsigned)lane + (unsigned)kWave * (unsigned)slot : 0xffffffffu;
    const unsigned gk = wave_reduce_u32<true>(lk);
    const uint64_t holders = __ballot(lk == gk);
    unsigned gi;
    if (__popcll(holders) == 1)
      gi = (unsigned)__builtin_amdgcn_readlane((int)li, __builtin_ctzll(holders));
    else
      gi = wave_reduce_u32<false>(lk == gk ? li : 0xffffffffu);
    const bool mine = (int)(gi & (kWave - 1)) == lane;  // the owner marks it taken (no branch)
#pragma unroll
    for (int i = 0; i < VPL; ++i) key[i] = (mine && (int)(gi / kWave) == i) ? 0u : key[i];
    if (lane == j) {
      my_key = gk;
      my_id = (int)gi;
    }
  }
  // softmax over the selection, in fp64, summed in rank order
  const float my_val = key_value(my_key);
  const double top = (double)key_value((unsigned)__builtin_amdgcn_readlane((int)my_key, 0));
  const double ex = lane < k ? exp((double)my_val - top) : 0.0;
  const unsigned long long exb = __double_as_longlong(ex);
  double s = 0.0;
  for (int j = 0; j < k; ++j) {
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)exb, j);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(exb >> 32), j);
    s += __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  }
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
