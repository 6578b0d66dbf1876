// Align routes into fixed-size per-bucket blocks, for any bucket count.
//
// A demand chunk aligns against the slot count, which is past the 1023 that
// a one-block aligner can count (FreeToken PR #676, Solution third bullet
// and Tests; gdevenyi's comment there: valid at 2100 and 4096).  Routes are
// split into chunks of 512-4K routes; each chunk's per-bucket counts go to a
// chunk-major matrix, a column scan turns them into per-chunk starting
// ranks, one workgroup lays the buckets out, and a stable scatter places
// every route in ascending route order inside its bucket.  In the scatter
// each wave of a chunk's workgroup owns a contiguous run of the chunk's
// routes with its own LDS histogram, so the 64-route batches of one wave
// need no workgroup barrier (wave ballots rank equal buckets of a batch).
#include "small_blocks.h"

#include <mutex>

namespace scr {

constexpr int kAlignMatrixBudget = 1 << 20;  // entries of the chunk x bucket count matrix (4 MiB)
constexpr int kAlignLdsInts = 36864;         // per-wave histograms and stash of the scatter: at most 144 KiB of LDS
constexpr int kAlignMaxWaves = 16;           // waves of a scatter workgroup
constexpr int kAlignLoads = 8;               // independent global loads a thread keeps in flight

struct AlignPlan {
  int nchunks, chunk, waves;
};

static AlignPlan align_plan(int n, int nb) {
  AlignPlan p;
  // as many waves (each with its own histogram) as the LDS holds beside the
  // chunk's stash: the scatter walks each wave's run in series, so more waves
  // mean shorter runs
  p.waves = 1;
  // about 256 chunks for a large input, each of 512..4096 routes (a chunk
  // well past the bucket count keeps the per-bucket work of a workgroup
  // small against its routes), fewer and longer if the matrix would pass its
  // budget
  long long chunk = ((long long)n + 255) / 256;
  chunk = (chunk + 255) / 256 * 256;
  if (chunk < 512) chunk = 512;
  if (chunk > 4096) chunk = 4096;
  long long nchunks = ((long long)n + chunk - 1) / chunk;
  if (nchunks < 1) nchunks = 1;
  long long by_budget = kAlignMatrixBudget / nb;
  if (by_budget < 1) by_budget = 1;
  if (nchunks > by_budget) {
    nchunks = by_budget;
    chunk = ((long long)n + nchunks - 1) / nchunks;
    nchunks = ((long long)n + chunk - 1) / chunk;
  }
  p.chunk = (int)chunk;
  p.nchunks = (int)nchunks;
  for (int w = kAlignMaxWaves; w >= 1; w /= 2)
    if ((long long)w * nb + chunk <= kAlignLdsInts || w == 1) {
      p.waves = w;
      break;
    }
  return p;
}

__device__ __forceinline__ void chunk_range(int n, int chunk, int c, int& r0, int& r1) {
  const long long a = (long long)c * chunk;
  r0 = (int)(a < n ? a : n);
  r1 = (int)(a + chunk < n ? a + chunk : n);
}

// one workgroup per chunk: per-bucket counts of the chunk, one matrix row
__global__ __launch_bounds__(256) void align_count_kernel(const int32_t* __restrict__ ids, int n,
                                                          const int32_t* __restrict__ map, int num_ids,
                                                          int nb, int chunk, int32_t* __restrict__ cnt) {
  extern __shared__ int hist[];
  const int c = blockIdx.x;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) hist[b] = 0;
  __syncthreads();
  int r0, r1;
  chunk_range(n, chunk, c, r0, r1);
  for (int rb = r0; rb < r1; rb += kAlignLoads * (int)blockDim.x) {  // loads in flight per thread
    int bk[kAlignLoads];
#pragma unroll
    for (int u = 0; u < kAlignLoads; ++u) {
      const int r = rb + u * (int)blockDim.x + (int)threadIdx.x;
      bk[u] = r < r1 ? bucket_of(ids, map, num_ids, nb, r) : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignLoads; ++u)
      if (bk[u] >= 0) atomicAdd(&hist[bk[u]], 1);
  }
  __syncthreads();
  int32_t* row = cnt + (size_t)c * nb;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) row[b] = hist[b];
}

// 64 buckets per workgroup, one lane per bucket; the 16 waves split the
// chunks into contiguous runs: exclusive scan down each column in place,
// bucket total out
constexpr int kColRun = 16;  // chunks per wave held in registers

__global__ __launch_bounds__(1024) void align_colscan_kernel(int32_t* __restrict__ cnt, int nb, int nchunks,
                                                             int32_t* __restrict__ total) {
  __shared__ int part[1024 / kWave][kWave];
  const int lane = lane_id(), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const int b = blockIdx.x * kWave + lane;
  const int q = (nchunks + nw - 1) / nw;
  const int c0 = min(nchunks, w * q), c1 = min(nchunks, c0 + q);
  int run = 0;
  if (q <= kColRun) {  // the usual case: one load per chunk, all in flight at once
    int v[kColRun];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kColRun; ++i) {
      v[i] = (b < nb && c0 + i < c1) ? cnt[(size_t)(c0 + i) * nb + b] : 0;
      sum += v[i];
    }
    part[w][lane] = sum;
    __syncthreads();
    for (int u = 0; u < w; ++u) run += part[u][lane];
#pragma unroll
    for (int i = 0; i < kColRun; ++i) {
      if (b < nb && c0 + i < c1) cnt[(size_t)(c0 + i) * nb + b] = run;
      run += v[i];
    }
  } else {
    int sum = 0;
    if (b < nb) {
#pragma unroll 8
      for (int c = c0; c < c1; ++c) sum += cnt[(size_t)c * nb + b];
    }
    part[w][lane] = sum;
    __syncthreads();
    for (int u = 0; u < w; ++u) run += part[u][lane];
    if (b < nb) {
#pragma unroll 8
      for (int c = c0; c < c1; ++c) {
        const int v = cnt[(size_t)c * nb + b];
        cnt[(size_t)c * nb + b] = run;
        run += v;
      }
    }
  }
  if (w == nw - 1 && b < nb) total[b] = run;  // the last run ends at the last chunk
}

// one workgroup: padded bucket offsets, active list, padded total.  Each
// thread owns a contiguous run of at most 16 buckets.
constexpr int kLayoutThreads = 1024;
constexpr int kLayoutRun = SCR_MAX_BUCKETS / kLayoutThreads;
static_assert(kLayoutRun * kLayoutThreads == SCR_MAX_BUCKETS, "layout runs cover every bucket");

__global__ __launch_bounds__(kLayoutThreads) void align_layout_kernel(const int32_t* __restrict__ total, int nb,
                                                                      int B, int32_t* __restrict__ bucket_off,
                                                                      int32_t* __restrict__ active_buckets,
                                                                      int32_t* __restrict__ active_block_begin,
                                                                      int32_t* __restrict__ n_active,
                                                                      int32_t* __restrict__ n_post_pad) {
  __shared__ int wave_tot[2][kLayoutThreads / kWave];
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int per = (nb + kLayoutThreads - 1) / kLayoutThreads;
  const int b0 = min(nb, (int)threadIdx.x * per), b1 = min(nb, b0 + per);
  int cnt[kLayoutRun];
  int pad_sum = 0, act_sum = 0;
#pragma unroll
  for (int i = 0; i < kLayoutRun; ++i) {
    cnt[i] = b0 + i < b1 ? total[b0 + i] : 0;
    pad_sum += (cnt[i] + B - 1) / B * B;
    act_sum += cnt[i] > 0;
  }
  const int s0 = wave_incl_sum(pad_sum), s1 = wave_incl_sum(act_sum);  // inclusive scans over the wave
  if (lane == kWave - 1) {
    wave_tot[0][wv] = s0;
    wave_tot[1][wv] = s1;
  }
  __syncthreads();
  int off = s0 - pad_sum, idx = s1 - act_sum;  // exclusive, then past the earlier waves
  for (int u = 0; u < wv; ++u) {
    off += wave_tot[0][u];
    idx += wave_tot[1][u];
  }
#pragma unroll
  for (int i = 0; i < kLayoutRun; ++i) {
    if (b0 + i < b1) {
      bucket_off[b0 + i] = off;
      if (cnt[i] > 0) {
        active_buckets[idx] = b0 + i;
        active_block_begin[idx] = off / B;
        ++idx;
      }
      off += (cnt[i] + B - 1) / B * B;
    }
  }
  if (threadIdx.x == kLayoutThreads - 1) {  // the last run ends at the last bucket
    *n_post_pad = off;
    *n_active = idx;
    active_block_begin[idx] = off / B;
  }
}

// One workgroup per chunk, one contiguous run of it per wave: the wave's
// histogram, per-wave starting positions of every bucket, then a stable
// scatter of the run 64 routes at a time.  The same launch writes the block
// table and the padding: every nchunks-th bucket (from the chunk index on)
// gets its block ids and the sentinel in its padding, and the blocks past the
// last bucket are split over the workgroups.
__global__ __launch_bounds__(64 * kAlignMaxWaves) void align_scatter_kernel(const int32_t* __restrict__ ids, int n,
                                                            const int32_t* __restrict__ map, int num_ids,
                                                            int nb, int B, int chunk, int stash_ok,
                                                            const int32_t* __restrict__ cnt,
                                                            const int32_t* __restrict__ total,
                                                            const int32_t* __restrict__ bucket_off,
                                                            const int32_t* __restrict__ n_post_pad, int nblocks,
                                                            int32_t* __restrict__ block_bucket,
                                                            int32_t* __restrict__ sorted_routes) {
  extern __shared__ int lds[];
  const int c = blockIdx.x, nchunks = gridDim.x;
  const int lane = lane_id(), w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  int* base = lds;             // [waves][nb]: counts of each wave's run, then its running positions
  int* stash = lds + nw * nb;  // [chunk] when stash_ok: the bucket of every route of the chunk
  for (int i = threadIdx.x; i < nw * nb; i += blockDim.x) base[i] = 0;
  __syncthreads();
  int r0, r1;
  chunk_range(n, chunk, c, r0, r1);
  const int per = ((r1 - r0 + nw - 1) / nw + kWave - 1) / kWave * kWave;
  const int s0 = min(r1, r0 + w * per), s1 = min(r1, s0 + per);
  int* mine = base + w * nb;
  for (int rb = s0; rb < s1; rb += kAlignLoads * kWave) {
    int bk[kAlignLoads];
#pragma unroll
    for (int u = 0; u < kAlignLoads; ++u) {
      const int r = rb + u * kWave + lane;
      bk[u] = r < s1 ? bucket_of(ids, map, num_ids, nb, r) : -1;
    }
#pragma unroll
    for (int u = 0; u < kAlignLoads; ++u) {
      const int r = rb + u * kWave + lane;
      if (r < s1) {
        if (stash_ok) stash[r - r0] = bk[u];
        if (bk[u] >= 0) atomicAdd(&mine[bk[u]], 1);
      }
    }
  }
  __syncthreads();
  const int32_t* row = cnt + (size_t)c * nb;
  for (int b0 = threadIdx.x; b0 < nb; b0 += kAlignLoads * (int)blockDim.x) {
    int start[kAlignLoads];
#pragma unroll
    for (int u = 0; u < kAlignLoads; ++u) {
      const int b = b0 + u * (int)blockDim.x;
      start[u] = b < nb ? bucket_off[b] + row[b] : 0;
    }
#pragma unroll
    for (int u = 0; u < kAlignLoads; ++u) {
      const int b = b0 + u * (int)blockDim.x;
      if (b < nb) {
        int run = start[u];
        for (int v = 0; v < nw; ++v) {
          const int t = base[v * nb + b];
          base[v * nb + b] = run;
          run += t;
        }
      }
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < nb) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int rb = s0; rb < s1; rb += kWave) {  // the same trip count on every lane of the wave
    const int r = rb + lane;
    int b = -1;
    if (r < s1) b = stash_ok ? stash[r - r0] : bucket_of(ids, map, num_ids, nb, r);
    const uint64_t peers = bucket_peers(b, nbits);
    const uint64_t below = peers & lt_mask;
    int pos = 0;
    if (b >= 0) pos = mine[b] + __popcll(below);
    __builtin_amdgcn_wave_barrier();  // the wave's reads of its histogram precede the update below
    if (b >= 0) {
      sorted_routes[pos] = r;
      if (below == 0) mine[b] += __popcll(peers);  // lowest peer advances the bucket
    }
    __builtin_amdgcn_wave_barrier();
  }
  // block ids and padding of this workgroup's buckets
  for (long long bl = c + (long long)threadIdx.x * nchunks; bl < nb; bl += (long long)blockDim.x * nchunks) {
    const int b = (int)bl;
    const int t = total[b];
    if (t == 0) continue;
    const int off = bucket_off[b];
    const int end = off + (t + B - 1) / B * B;
    for (int j = off / B; j < end / B; ++j) block_bucket[j] = b;
    for (int q = off + t; q < end; ++q) sorted_routes[q] = n;
  }
  // this workgroup's share of the unused blocks
  const int end_block = *n_post_pad / B;
  const long long tail = (long long)(nblocks - end_block) * B;
  for (long long e = (long long)c * blockDim.x + threadIdx.x; e < tail; e += (long long)nchunks * blockDim.x) {
    sorted_routes[(size_t)end_block * B + e] = n;
    if (e % B == 0) block_bucket[end_block + e / B] = -1;
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
  __shared__ uint16_t tab[kAlignTab];  // per-(bucket, batch) counts of the scatter
  align_small_block(ids, n, map, num_ids, nb, B, cap, sorted_routes, block_bucket, n_post_pad, active_buckets,
                    active_block_begin, n_active, cnt, rb, wave_tot, tab);
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

namespace scr {

static int align_blocks_impl(const int32_t* ids, int n, const int32_t* id_to_bucket, int num_ids, int num_buckets,
                             int block_size, int32_t* sorted_routes, int32_t* block_bucket, int32_t* n_post_pad,
                             int32_t* active_buckets, int32_t* active_block_begin, int32_t* n_active, void* ws,
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
  hipLaunchKernelGGL(scr::align_count_kernel, dim3(p.nchunks), dim3(256), lds, stream, ids, n, id_to_bucket,
                     num_ids, num_buckets, p.chunk, cnt);
  SCR_CHECK_LAUNCH();
  hipLaunchKernelGGL(scr::align_colscan_kernel, dim3((num_buckets + scr::kWave - 1) / scr::kWave), dim3(1024), 0,
                     stream, cnt, num_buckets, p.nchunks, total);
  SCR_CHECK_LAUNCH();
  hipLaunchKernelGGL(scr::align_layout_kernel, dim3(1), dim3(scr::kLayoutThreads), 0, stream, total, num_buckets,
                     block_size, bucket_off, active_buckets, active_block_begin, n_active, n_post_pad);
  SCR_CHECK_LAUNCH();
  const int nblocks = (int)(scr_align_capacity(n, num_buckets, block_size) / block_size);
  const int hist_ints = p.waves * num_buckets;
  const int stash_ok = hist_ints + p.chunk <= scr::kAlignLdsInts;
  const size_t scatter_lds = (size_t)(hist_ints + (stash_ok ? p.chunk : 0)) * sizeof(int);
  hipLaunchKernelGGL(scr::align_scatter_kernel, dim3(p.nchunks), dim3(scr::kWave * p.waves), scatter_lds, stream,
                     ids, n, id_to_bucket, num_ids, num_buckets, block_size, p.chunk, stash_ok, cnt, total,
                     bucket_off, n_post_pad, nblocks, block_bucket, sorted_routes);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

// Scratch of the entry point that allocates nothing: the largest workspace an
// align call can need (the count matrix is capped at kAlignMatrixBudget
// entries, plus two ints per bucket), resident on every GPU the library runs
// on until the process ends.  Host code never uses the array's name as an
// address: each device's copy is looked up once with hipGetSymbolAddress (on
// the first call made with that device current) and that address is what
// the kernels receive.  Every entry of it that an align call reads is written
// by the same call first (counts, then totals and offsets), so nothing needs
// clearing between calls.
constexpr size_t kAlignScratchBytes = ((size_t)kAlignMatrixBudget + 2 * (size_t)SCR_MAX_BUCKETS) * sizeof(int32_t) + 256;
static __device__ __align__(256) unsigned char scratch[kAlignScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_for_current_device(void** out) {
  int dev = -1;
  SCR_CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("align_blocks_noalloc: device %d beyond the %d the library tracks", dev, kMaxDevices);
    return SCR_ENOTSUP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    SCR_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) {
      set_error("align_blocks_noalloc: no device address for the scratch array on device %d", dev);
      return SCR_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SCR_OK;
}

}  // namespace scr

extern "C" int scr_align_blocks(const int32_t* ids, int n, const int32_t* id_to_bucket, int num_ids,
                                int num_buckets, int block_size, int32_t* sorted_routes,
                                int32_t* block_bucket, int32_t* n_post_pad, int32_t* active_buckets,
                                int32_t* active_block_begin, int32_t* n_active, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  return scr::align_blocks_impl(ids, n, id_to_bucket, num_ids, num_buckets, block_size, sorted_routes, block_bucket,
                                n_post_pad, active_buckets, active_block_begin, n_active, ws, ws_bytes, stream);
}

extern "C" int scr_align_blocks_noalloc(const int32_t* ids, int n, const int32_t* id_to_bucket, int num_ids,
                                        int num_buckets, int block_size, int32_t* sorted_routes,
                                        int32_t* block_bucket, int32_t* n_post_pad, int32_t* active_buckets,
                                        int32_t* active_block_begin, int32_t* n_active, hipStream_t stream) {
  SCR_CHECK_ARG(n >= 0 && n < (1 << 30), "align_noalloc: n out of range");
  SCR_CHECK_ARG(num_buckets >= 1 && num_buckets <= SCR_MAX_BUCKETS, "align_noalloc: num_buckets must be in [1, %d]",
                SCR_MAX_BUCKETS);
  size_t need = 0;
  int rc = scr_align_workspace(n, num_buckets, &need);
  if (rc) return rc;
  if (need > scr::kAlignScratchBytes) {
    scr::set_error("align_noalloc: %zu bytes of scratch needed, the library holds %zu", need,
                   scr::kAlignScratchBytes);
    return SCR_ECAPACITY;
  }
  void* ws = nullptr;
  rc = scr::scratch_for_current_device(&ws);
  if (rc) return rc;
  return scr::align_blocks_impl(ids, n, id_to_bucket, num_ids, num_buckets, block_size, sorted_routes, block_bucket,
                                n_post_pad, active_buckets, active_block_begin, n_active, ws, scr::kAlignScratchBytes,
                                stream);
}
