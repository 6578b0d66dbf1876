// Align routes into fixed-size per-bucket blocks, for any bucket count.
//
// A demand chunk aligns against the slot count, which is past the 1023 that
// a one-block aligner can count (FreeToken PR #676, Solution third bullet
// and Tests; gdevenyi's comment there: valid at 2100 and 4096).  Routes are
// split into chunks; each chunk's per-bucket counts go to a bucket-major
// matrix, a column scan turns them into per-chunk starting ranks, one
// workgroup lays the buckets out, and a stable scatter places every route in
// ascending route order inside its bucket (wave ballots give the rank among
// equal buckets of one 64-route batch).
#include "small_blocks.h"

namespace scr {

constexpr int kAlignMatrixBudget = 1 << 18;  // entries of the chunk x bucket count matrix

struct AlignPlan {
  int nchunks, chunk;
};

static AlignPlan align_plan(int n, int nb) {
  AlignPlan p;
  long long by_budget = kAlignMatrixBudget / nb;
  if (by_budget < 1) by_budget = 1;
  long long by_n = (n + 63) / 64;
  if (by_n < 1) by_n = 1;
  p.nchunks = (int)(by_budget < by_n ? by_budget : by_n);
  p.chunk = (int)(((long long)n + p.nchunks - 1) / p.nchunks);
  if (p.chunk < 1) p.chunk = 1;
  p.nchunks = (int)(((long long)n + p.chunk - 1) / p.chunk);
  if (p.nchunks < 1) p.nchunks = 1;
  return p;
}


// one wave per chunk: per-bucket counts of the chunk, written bucket-major
__global__ __launch_bounds__(64) void align_count_kernel(const int32_t* __restrict__ ids, int n,
                                                         const int32_t* __restrict__ map, int num_ids,
                                                         int nb, int chunk, int nchunks,
                                                         int32_t* __restrict__ cnt) {
  extern __shared__ int hist[];
  const int c = blockIdx.x;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) hist[b] = 0;
  __syncthreads();
  const int r0 = c * chunk, r1 = min(n, r0 + chunk);
  for (int r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
    const int b = bucket_of(ids, map, num_ids, nb, r);
    if (b >= 0) atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x) cnt[(size_t)b * nchunks + c] = hist[b];
}

// one wave per bucket: exclusive scan over chunks in place, bucket total out
__global__ __launch_bounds__(256) void align_colscan_kernel(int32_t* __restrict__ cnt, int nb, int nchunks,
                                                            int32_t* __restrict__ total) {
  const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (b >= nb) return;
  const int lane = lane_id();
  int32_t* col = cnt + (size_t)b * nchunks;
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += kWave) {
    const int c = c0 + lane;
    const int v = c < nchunks ? col[c] : 0;
    int s = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(s, off, kWave);
      if (lane >= off) s += o;
    }
    if (c < nchunks) col[c] = carry + s - v;
    carry += __shfl(s, kWave - 1, kWave);
  }
  if (lane == 0) total[b] = carry;
}

// one workgroup: padded bucket offsets, active list, padded total
__global__ __launch_bounds__(1024) void align_layout_kernel(const int32_t* __restrict__ total, int nb, int B,
                                                            int32_t* __restrict__ bucket_off,
                                                            int32_t* __restrict__ active_buckets,
                                                            int32_t* __restrict__ active_block_begin,
                                                            int32_t* __restrict__ n_active,
                                                            int32_t* __restrict__ n_post_pad) {
  __shared__ int wave_tot[2][kWave];
  __shared__ int carry[2];
  if (threadIdx.x == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  const int lane = lane_id(), wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
  for (int b0 = 0; b0 < nb; b0 += blockDim.x) {
    const int b = b0 + threadIdx.x;
    const int c = b < nb ? total[b] : 0;
    const int padded = (c + B - 1) / B * B;
    const int act = c > 0;
    int s0 = padded, s1 = act;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o0 = __shfl_up(s0, off, kWave), o1 = __shfl_up(s1, off, kWave);
      if (lane >= off) {
        s0 += o0;
        s1 += o1;
      }
    }
    if (lane == kWave - 1) {
      wave_tot[0][wv] = s0;
      wave_tot[1][wv] = s1;
    }
    __syncthreads();
    int before0 = carry[0], before1 = carry[1];
    for (int w = 0; w < wv; ++w) {
      before0 += wave_tot[0][w];
      before1 += wave_tot[1][w];
    }
    const int off_b = before0 + s0 - padded;  // exclusive
    const int idx = before1 + s1 - act;
    if (b < nb) {
      bucket_off[b] = off_b;
      if (act) {
        active_buckets[idx] = b;
        active_block_begin[idx] = off_b / B;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int t0 = 0, t1 = 0;
      for (int w = 0; w < nw; ++w) {
        t0 += wave_tot[0][w];
        t1 += wave_tot[1][w];
      }
      carry[0] += t0;
      carry[1] += t1;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *n_post_pad = carry[0];
    *n_active = carry[1];
    active_block_begin[carry[1]] = carry[0] / B;
  }
}

// one wave per chunk: stable scatter of the chunk's routes, 64 at a time
__global__ __launch_bounds__(64) void align_scatter_kernel(const int32_t* __restrict__ ids, int n,
                                                           const int32_t* __restrict__ map, int num_ids,
                                                           int nb, int chunk, int nchunks,
                                                           const int32_t* __restrict__ cnt,
                                                           const int32_t* __restrict__ bucket_off,
                                                           int32_t* __restrict__ sorted_routes) {
  extern __shared__ int base[];
  const int c = blockIdx.x;
  const int lane = lane_id();
  for (int b = lane; b < nb; b += kWave) base[b] = bucket_off[b] + cnt[(size_t)b * nchunks + c];
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < nb) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int r0 = c * chunk, r1 = min(n, r0 + chunk);
  for (int rb = r0; rb < r1; rb += kWave) {
    const int r = rb + lane;
    const int b = r < r1 ? bucket_of(ids, map, num_ids, nb, r) : -1;
    uint64_t peers = __ballot(b >= 0);
    for (int bit = 0; bit < nbits; ++bit) {
      const uint64_t ones = __ballot(b >= 0 && ((b >> bit) & 1));
      peers &= ((b >> bit) & 1) ? ones : ~ones;
    }
    int pos = 0;
    if (b >= 0) pos = base[b] + __popcll(peers & lt_mask);
    __syncthreads();  // every lane has read base[] before it moves
    if (b >= 0) {
      sorted_routes[pos] = r;
      if ((peers & lt_mask) == 0) base[b] += __popcll(peers);  // lowest peer advances the bucket
    }
    __syncthreads();
  }
}

// grid-stride over blocks: block bucket ids and the sentinel in every padding entry
__global__ __launch_bounds__(256) void align_fill_kernel(int n, int B, int nblocks,
                                                         const int32_t* __restrict__ total,
                                                         const int32_t* __restrict__ bucket_off,
                                                         const int32_t* __restrict__ active_buckets,
                                                         const int32_t* __restrict__ active_block_begin,
                                                         const int32_t* __restrict__ n_active_p,
                                                         int32_t* __restrict__ block_bucket,
                                                         int32_t* __restrict__ sorted_routes) {
  const int n_active = *n_active_p;
  const int end_block = active_block_begin[n_active];
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < nblocks; j += gridDim.x * blockDim.x) {
    if (j >= end_block) {
      block_bucket[j] = -1;
      for (int q = 0; q < B; ++q) sorted_routes[(size_t)j * B + q] = n;
      continue;
    }
    // last active entry whose first block is <= j
    int lo = 0, hi = n_active - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (active_block_begin[mid] <= j) lo = mid;
      else hi = mid - 1;
    }
    const int b = active_buckets[lo];
    block_bucket[j] = b;
    const int fill_from = bucket_off[b] + total[b];  // first padding position of the bucket
    for (int q = 0; q < B; ++q) {
      const int pos = j * B + q;
      if (pos >= fill_from) sorted_routes[pos] = n;
    }
  }
}

__global__ __launch_bounds__(kPlanThreads) void align_small_kernel(const int32_t* __restrict__ ids, int n,
                                                                   const int32_t* __restrict__ map, int num_ids,
                                                                   int nb, int B, int cap,
                                                                   int32_t* __restrict__ sorted_routes,
                                                                   int32_t* __restrict__ block_bucket,
                                                                   int32_t* __restrict__ n_post_pad,
                                                                   int32_t* __restrict__ active_buckets,
                                                                   int32_t* __restrict__ active_block_begin,
                                                                   int32_t* __restrict__ n_active) {
  __shared__ int cnt[kSmallBuckets];  // counts, then running scatter positions
  __shared__ int rb[kSmallRoutes];    // bucket of each route (-1 dropped)
  __shared__ int wave_tot[2 * kWave];
  align_small_block(ids, n, map, num_ids, nb, B, cap, sorted_routes, block_bucket, n_post_pad, active_buckets,
                    active_block_begin, n_active, cnt, rb, wave_tot);
}

}  // namespace scr

extern "C" size_t scr_align_capacity(int n, int num_buckets, int block_size) {
  if (n < 0 || num_buckets < 1 || block_size < 1) return 0;
  const long long m = n < num_buckets ? n : num_buckets;
  const long long cap = (long long)n + m * (block_size - 1);
  return (size_t)((cap + block_size - 1) / block_size * block_size);
}

extern "C" int scr_align_workspace(int n, int num_buckets, size_t* bytes) {
  SCR_CHECK_ARG(bytes && n >= 0 && num_buckets >= 1 && num_buckets <= SCR_MAX_BUCKETS,
                "align_workspace: bad arguments");
  const scr::AlignPlan p = scr::align_plan(n, num_buckets);
  const size_t cnt = (size_t)p.nchunks * num_buckets;
  *bytes = (cnt + 2 * (size_t)num_buckets) * sizeof(int32_t) + 256;
  return SCR_OK;
}

extern "C" int scr_align_blocks(const int32_t* ids, int n, const int32_t* id_to_bucket, int num_ids,
                                int num_buckets, int block_size, int32_t* sorted_routes,
                                int32_t* block_bucket, int32_t* n_post_pad, int32_t* active_buckets,
                                int32_t* active_block_begin, int32_t* n_active, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  SCR_CHECK_ARG(n >= 0 && n < (1 << 30), "align: n out of range");
  SCR_CHECK_ARG(num_buckets >= 1 && num_buckets <= SCR_MAX_BUCKETS, "align: num_buckets must be in [1, %d]",
                SCR_MAX_BUCKETS);
  SCR_CHECK_ARG(block_size == 16 || block_size == 32 || block_size == 64, "align: block_size must be 16, 32 or 64");
  SCR_CHECK_ARG(!id_to_bucket || num_ids >= 1, "align: num_ids must be >= 1 with a map");
  SCR_CHECK_ARG(sorted_routes && block_bucket && n_post_pad && active_buckets && active_block_begin &&
                    n_active && ws,
                "align: null pointer");
  SCR_CHECK_ARG(n == 0 || ids, "align: ids is null");
  size_t need = 0;
  scr_align_workspace(n, num_buckets, &need);
  SCR_CHECK_ARG(ws_bytes >= need, "align: workspace of %zu bytes, %zu needed", ws_bytes, need);
  if (n <= scr::kSmallRoutes && num_buckets <= scr::kSmallBuckets) {
    const int cap = (int)scr_align_capacity(n, num_buckets, block_size);
    hipLaunchKernelGGL(scr::align_small_kernel, dim3(1), dim3(scr::kPlanThreads), 0, stream, ids, n, id_to_bucket, num_ids,
                       num_buckets, block_size, cap, sorted_routes, block_bucket, n_post_pad, active_buckets,
                       active_block_begin, n_active);
    SCR_CHECK_LAUNCH();
    return SCR_OK;
  }
  const scr::AlignPlan p = scr::align_plan(n, num_buckets);
  int32_t* cnt = static_cast<int32_t*>(ws);
  int32_t* total = cnt + (size_t)p.nchunks * num_buckets;
  int32_t* bucket_off = total + num_buckets;
  const size_t lds = (size_t)num_buckets * sizeof(int);
  hipLaunchKernelGGL(scr::align_count_kernel, dim3(p.nchunks), dim3(64), lds, stream, ids, n, id_to_bucket,
                     num_ids, num_buckets, p.chunk, p.nchunks, cnt);
  SCR_CHECK_LAUNCH();
  hipLaunchKernelGGL(scr::align_colscan_kernel, dim3((num_buckets + 3) / 4), dim3(256), 0, stream, cnt,
                     num_buckets, p.nchunks, total);
  SCR_CHECK_LAUNCH();
  hipLaunchKernelGGL(scr::align_layout_kernel, dim3(1), dim3(1024), 0, stream, total, num_buckets, block_size,
                     bucket_off, active_buckets, active_block_begin, n_active, n_post_pad);
  SCR_CHECK_LAUNCH();
  hipLaunchKernelGGL(scr::align_scatter_kernel, dim3(p.nchunks), dim3(64), lds, stream, ids, n, id_to_bucket,
                     num_ids, num_buckets, p.chunk, p.nchunks, cnt, bucket_off, sorted_routes);
  SCR_CHECK_LAUNCH();
  const int nblocks = (int)(scr_align_capacity(n, num_buckets, block_size) / block_size);
  if (nblocks > 0) {
    int grid = (nblocks + 255) / 256;
    if (grid > 1024) grid = 1024;
    hipLaunchKernelGGL(scr::align_fill_kernel, dim3(grid), dim3(256), 0, stream, n, block_size, nblocks, total,
                       bucket_off, active_buckets, active_block_begin, n_active, block_bucket, sorted_routes);
    SCR_CHECK_LAUNCH();
  }
  return SCR_OK;
}
