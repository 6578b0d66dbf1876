// Single-workgroup bodies shared by the stand-alone kernels (dedup, the small
// align) and the fused chunk planner: each is called by all threads of one
// workgroup of kPlanThreads threads with its LDS passed in.
#pragma once
#include "common.h"

namespace scr {

constexpr int kPlanThreads = 1024;
constexpr int kDedupMaxE = 8192;
constexpr int kSmallRoutes = 4096;   // routes the one-workgroup align takes
constexpr int kSmallBuckets = 8192;  // buckets the one-workgroup align takes
constexpr int kAlignTab = 20480;     // entries of its (bucket, 64-route batch) count table

// inclusive scan of one int per thread across the block; returns the block total
__device__ __forceinline__ int block_inclusive_scan(int v, int* wave_tot) {
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  v = wave_incl_sum(v);
  if (lane == kWave - 1) wave_tot[wv] = v;
  __syncthreads();
  if (wv == 0) {
    const int t = wave_incl_sum(lane < nw ? wave_tot[lane] : 0);
    if (lane < nw) wave_tot[lane] = t;
  }
  __syncthreads();
  const int before = wv > 0 ? wave_tot[wv - 1] : 0;
  const int total = wave_tot[nw - 1];
  __syncthreads();
  wave_tot[kWave] = total;
  return v + before;
}


__device__ __forceinline__ int bucket_of(const int32_t* __restrict__ ids, const int32_t* __restrict__ map,
                                         int num_ids, int nb, int r) {
  int b = ids[r];
  if (map) b = (b >= 0 && b < num_ids) ? map[b] : -1;
  return (b >= 0 && b < nb) ? b : -1;
}

// Lanes of the wave whose bucket equals this lane's, from one ballot per
// bucket bit (every lane of the wave calls it; nbits = bits of the largest
// bucket, at most 14).  Dropped lanes (b < 0) are in no lane's mask; a
// dropped lane's own result is meaningless.
__device__ __forceinline__ uint64_t bucket_peers(int b, int nbits) {
  uint64_t peers = __ballot(b >= 0);
#pragma unroll
  for (int bit = 0; bit < 14; ++bit) {
    if (bit < nbits) {  // the same on every lane
      const int set = (b >> bit) & 1;
      const uint64_t ones = __ballot(set);
      peers &= ones ^ ((uint64_t)set - 1);  // ones where the bit is set, ~ones where it is clear
    }
  }
  return peers;
}

// Distinct ids as a sorted fixed-length list: marks in LDS, a scan, a
// scatter (a counting sort over ids).  pos: LDS [kDedupMaxE]; wave_tot: LDS
// [kWave + 1].  With lds_e / lds_s (LDS [lmax], the chunk planner's copy for
// its LRU queries) the list is also written there with each id's slot
// slot_of[id] (-1 for the sentinels), so that the queries need no loads.
__device__ __forceinline__ void dedup_block(const int32_t* __restrict__ ids, int n, int E, int lmax,
                                            int32_t* __restrict__ distinct, int32_t* __restrict__ n_distinct,
                                            int32_t* __restrict__ inverse, int* pos, int* wave_tot,
                                            int* lds_e = nullptr, int* lds_s = nullptr,
                                            const int32_t* __restrict__ slot_of = nullptr) {
  // each thread owns a contiguous run of ids [e0, e1), at most
  // kDedupMaxE / kPlanThreads of them; with lds_e their slots are read first,
  // so that those loads overlap the marking
  constexpr int kRun = kDedupMaxE / kPlanThreads;
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = min(E, (int)threadIdx.x * per), e1 = min(E, e0 + per);
  int slot_pre[kRun];
  if (lds_e) {
#pragma unroll
    for (int u = 0; u < kRun; ++u) slot_pre[u] = e0 + u < e1 ? slot_of[e0 + u] : -1;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) pos[e] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = ids[i];
    if (e >= 0 && e < E) pos[e] = 1;
  }
  __syncthreads();
  int cnt = 0;
  for (int e = e0; e < e1; ++e) cnt += pos[e];
  const int incl = block_inclusive_scan(cnt, wave_tot);
  const int total = wave_tot[kWave];
  int p = incl - cnt;
#pragma unroll
  for (int u = 0; u < kRun; ++u) {
    const int e = e0 + u;
    if (e >= e1) break;
    const int present = pos[e];
    if (present) {
      distinct[p] = e;
      if (lds_e) {
        lds_e[p] = e;
        lds_s[p] = slot_pre[u];
      }
    }
    pos[e] = present ? p : -1;
    p += present;
  }
  for (int i = total + threadIdx.x; i < lmax; i += blockDim.x) {
    distinct[i] = E;
    if (lds_e) {
      lds_e[i] = E;
      lds_s[i] = -1;
    }
  }
  if (threadIdx.x == 0) *n_distinct = total;
  if (inverse) {
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int e = ids[i];
      inverse[i] = (e >= 0 && e < E) ? pos[e] : -1;
    }
  }
}

// Small inputs (n <= kSmallRoutes, nb <= kSmallBuckets): the whole align in
// one workgroup.  All waves count and lay the buckets out; one wave scatters
// the routes in ascending order (64 at a time, ballot ranks) while the other
// waves write the padding and block ids.  cnt: LDS [kSmallBuckets]; rb: LDS
// [kSmallRoutes]; wave_tot: LDS [2 * kWave].
__device__ __forceinline__ void align_small_block(const int32_t* __restrict__ ids, int n,
                                                  const int32_t* __restrict__ map, int num_ids, int nb, int B,
                                                  int cap, int32_t* __restrict__ sorted_routes,
                                                  int32_t* __restrict__ block_bucket, int32_t* __restrict__ n_post_pad,
                                                  int32_t* __restrict__ active_buckets,
                                                  int32_t* __restrict__ active_block_begin,
                                                  int32_t* __restrict__ n_active, int* cnt, int* rb, int* wave_tot,
                                                  uint16_t* tab) {
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave, nw = blockDim.x / kWave;
  const int nchunks = (n + kWave - 1) / kWave;
  // the scatter ranks across 64-route batches through a table of per-(bucket,
  // batch) counts when it fits, else by one wave walking the batches in order
  const bool use_tab = (long long)nb * nchunks <= kAlignTab;
  for (int b = tid; b < nb; b += blockDim.x) cnt[b] = 0;
  // every position a sentinel and every block unused, in coalesced passes;
  // the layout and the scatter below overwrite the used ones (the barriers in
  // between order the stores)
  if ((reinterpret_cast<uintptr_t>(sorted_routes) & 15) == 0 && cap % 4 == 0) {  // 16-byte stores
    const int4 sv = make_int4(n, n, n, n);
    for (int q = tid; q < cap / 4; q += blockDim.x) reinterpret_cast<int4*>(sorted_routes)[q] = sv;
  } else {
    for (int q = tid; q < cap; q += blockDim.x) sorted_routes[q] = n;
  }
  for (int j = tid; j < cap / B; j += blockDim.x) block_bucket[j] = -1;
  __syncthreads();
  for (int r = tid; r < n; r += blockDim.x) {
    const int b = bucket_of(ids, map, num_ids, nb, r);
    rb[r] = b;
    if (b >= 0) atomicAdd(&cnt[b], 1);
  }
  __syncthreads();
  // exclusive scans of padded counts and of the active flags; thread owns a
  // contiguous run of buckets
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
  int pad_sum = 0, act_sum = 0;
  for (int b = b0; b < b1; ++b) {
    const int c = cnt[b];
    pad_sum += (c + B - 1) / B * B;
    act_sum += c > 0;
  }
  const int s0 = wave_incl_sum(pad_sum), s1 = wave_incl_sum(act_sum);
  if (lane == kWave - 1) {
    wave_tot[wv] = s0;
    wave_tot[kWave + wv] = s1;
  }
  __syncthreads();
  // the waves' totals, all loads in flight at once (a workgroup has at most
  // kPlanThreads / kWave waves)
  int before0 = 0, before1 = 0, total0 = 0, total1 = 0;
#pragma unroll
  for (int w = 0; w < kPlanThreads / kWave; ++w) {
    const int t0 = w < nw ? wave_tot[w] : 0, t1 = w < nw ? wave_tot[kWave + w] : 0;
    if (w < wv) {
      before0 += t0;
      before1 += t1;
    }
    total0 += t0;
    total1 += t1;
  }
  int off = before0 + s0 - pad_sum, idx = before1 + s1 - act_sum;
  for (int b = b0; b < b1; ++b) {
    const int c = cnt[b];
    const int padded = (c + B - 1) / B * B;
    if (c > 0) {
      if (use_tab)  // only the rows of active buckets are ever read
        for (int j = 0; j < nchunks; ++j) tab[b * nchunks + j] = 0;
      active_buckets[idx] = b;
      active_block_begin[idx] = off / B;
      ++idx;
      for (int j = off / B; j < (off + padded) / B; ++j) block_bucket[j] = b;
    }
    cnt[b] = off;  // scatter position of the bucket's first route
    off += padded;
  }
  if (tid == 0) {
    *n_post_pad = total0;
    *n_active = total1;
    active_block_begin[total1] = total0 / B;
  }
  __syncthreads();
  // Stable scatter.  First every wave takes 64-route batches and finds, by
  // ballots over the bucket bits, each route's rank among the routes of its
  // bucket in the batch, packed into rb as bucket | rank << 14 (buckets <
  // 2^13), and at the first of them their count.  With the table: each count
  // goes to tab[bucket][batch], one thread per bucket turns its row into
  // running counts, and every route lands at offset + running count + rank.
  // Without it the count rides in rb (<< 20) and one wave walks the batches in
  // order: position = the bucket's running offset + rank, and the first route
  // of each bucket advances the offset.
  int nbits = 0;
  while ((1 << nbits) < nb) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c = wv; c < nchunks; c += nw) {
    const int r = c * kWave + lane;
    const int b = r < n ? rb[r] : -1;
    const uint64_t peers = bucket_peers(b, nbits);
    const int rank = __popcll(peers & lt_mask);
    if (b >= 0) {
      if (use_tab) {
        rb[r] = b | (rank << 14);
        if (rank == 0) tab[b * nchunks + c] = (uint16_t)__popcll(peers);
      } else {
        rb[r] = b | (rank << 14) | ((rank == 0 ? __popcll(peers) : 0) << 20);
      }
    }
  }
  __syncthreads();
  if (use_tab) {
    for (int b = tid; b < nb; b += blockDim.x) {
      // a bucket is active when its first position differs from the next's
      if ((b + 1 < nb ? cnt[b + 1] : total0) == cnt[b]) continue;
      uint16_t* row = tab + b * nchunks;
      int run = 0;
      for (int c0 = 0; c0 < nchunks; c0 += 16) {  // 16 reads in flight, then the running counts
        int v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = c0 + u < nchunks ? row[c0 + u] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (c0 + u < nchunks) row[c0 + u] = (uint16_t)run;
          run += v[u];
        }
      }
    }
    __syncthreads();
    for (int r = tid; r < n; r += blockDim.x) {
      const int v = rb[r];
      if (v >= 0) {
        const int b = v & 0x3fff, rank = v >> 14;
        sorted_routes[cnt[b] + tab[b * nchunks + r / kWave] + rank] = r;
      }
    }
  } else if (wv == 0) {
    // the next chunk's packed value is read one iteration ahead
    int vn = lane < n ? rb[lane] : -1;
    for (int c = 0; c < nchunks; ++c) {
      const int r = c * kWave + lane;
      const int v = vn;
      vn = r + kWave < n ? rb[r + kWave] : -1;
      const int b = v & 0x3fff, rank = (v >> 14) & 63;
      if (v >= 0) sorted_routes[cnt[b] + rank] = r;
      __builtin_amdgcn_wave_barrier();  // every lane has read the offsets before the leaders move them
      if (v >= 0 && rank == 0) cnt[b] += v >> 20;
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace scr
