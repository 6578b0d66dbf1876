// Device-side LRU planner over a bank keyed by (layer, expert).
//
// A query of distinct expert ids is admitted in one workgroup (FreeToken PR
// #676, Solution second bullet and the author's reply: LRU only, earlier
// queries evicted last; vLLM fork PR #48, What: a device-side planner over one
// bank shared by all layers).  Recency is one stamp per query; candidates for
// eviction are ordered by the 64-bit key (stamp << 20 | slot), found by an
// 8-bit radix select in LDS instead of sorting the bank.  Under the scored
// policy (LRFU; FreeToken PR #676 run notes and Solution: earlier pieces of a
// chunk pinned against the later ones) the key is (decayed value << 20 |
// slot) over the slots the chunk has not touched; include/scr.h gives the
// integer definition.
#include "small_blocks.h"

#include <vector>

namespace scr {

constexpr int kLruThreads = kPlanThreads;
constexpr int kSlotBits = 20;  // SCR_MAX_SLOTS <= 2^18 < 2^20
// a batched call reads every query entry's slot once, up front, when the
// chunk has at most kEnsPrefetch entries and the bank at most kPrefetchSlots
constexpr int kEnsPrefetch = 4096;
constexpr int kPrefetchSlots = 65536;

__device__ __forceinline__ uint64_t cand_key(uint64_t stamp, int slot) {
  return (stamp << kSlotBits) | (uint64_t)slot;
}

struct EnsureShared {
  uint32_t hit_bits[SCR_MAX_SLOTS / 32];
  int q_key[SCR_MAX_QUERY_WIDTH];
  int q_miss_rank[SCR_MAX_QUERY_WIDTH];  // -1: not a miss
  uint64_t sel_key[SCR_MAX_QUERY_WIDTH];
  int victim[SCR_MAX_QUERY_WIDTH];
  unsigned hist[256];
  int wave_tot[kWave + 1];
  int nhit, nsel, evict, npinned;
  uint64_t prefix;
  unsigned rank;
  // batched calls: the chunk's query entries and their slots at its start,
  // and the slots its earlier queries gave to misses
  int pf_e[kEnsPrefetch];
  int pf_s[kEnsPrefetch];
  uint32_t taken[kPrefetchSlots / 32];
};

struct BankRefs {
  int S, E, layer;
  int32_t* slot_key;
  uint64_t* slot_stamp;
  int32_t* key_to_slot;
  uint64_t* stats;
  uint32_t* decode_freq;
  uint32_t* err;
  int policy;
  uint32_t decay;         // LRFU per-tick factor, Q0.32
  uint32_t* slot_crf;     // LRFU value at the slot's stamp, Q8.24
  uint64_t* chunk_start;  // clock of the chunk's first query
};

constexpr uint32_t kCrfOne = 1u << 24;

// D^n in Q0.32 by right-to-left binary exponentiation, truncating each product
__device__ __forceinline__ uint64_t pow_q32(uint64_t D, uint64_t n) {
  uint64_t r = 1ull << 32, b = D;
  while (n != 0 && r != 0) {
    if (n & 1) r = (r * b) >> 32;
    b = (b * b) >> 32;
    n >>= 1;
  }
  return r;
}

// an LRFU value (Q8.24) decayed over n ticks
__device__ __forceinline__ uint64_t crf_decay(uint32_t c, uint64_t n, uint32_t D) {
  return ((uint64_t)c * pow_q32(D, n)) >> 32;
}

// eviction order key of an untouched slot at time now
__device__ __forceinline__ uint64_t victim_key(const BankRefs& bk, int s, uint64_t now) {
  const uint64_t stamp = bk.slot_stamp[s];
  if (bk.policy == SCR_POLICY_LRFU) return cand_key(crf_decay(bk.slot_crf[s], now - stamp, bk.decay), s);
  return cand_key(stamp, s);
}

// One query with clock `now`; the admitted misses are written in query order
// to miss_slot/miss_key[0 ..) and their number returned (in every thread).
// `pin`: under LRFU only slots stamped before it are candidates (the chunk's
// first query's clock).  Called by all threads of the workgroup.
// pfe, pfs, taken (all null, or all set by a batched call): this query's
// entries and their slots read at the chunk's start, and the bitmap of slots
// that the chunk's earlier queries gave to misses.  A key's slot changes only
// when an earlier query of the chunk takes it for a miss (keys are distinct
// across the chunk's queries), so a prefetched slot is exact unless taken.
__device__ int ensure_query(EnsureShared& sh, const BankRefs& bk, uint64_t now, uint64_t pin,
                            const int32_t* __restrict__ query, int width, int record_stats,
                            int32_t* __restrict__ miss_slot, int32_t* __restrict__ miss_key,
                            const int* pfe = nullptr, const int* pfs = nullptr, uint32_t* taken = nullptr) {
  const bool lrfu = bk.policy == SCR_POLICY_LRFU;
  const int tid = threadIdx.x;
  const int S = bk.S, E = bk.E;
  const int nwords = (S + 31) / 32;
  for (int i = tid; i < nwords; i += blockDim.x) sh.hit_bits[i] = 0;
  if (tid == 0) {
    sh.nhit = 0;
    sh.evict = 0;
    sh.nsel = 0;
    sh.npinned = 0;
  }
  // a query holding only sentinels (the tail of a chunk's padded distinct
  // list) changes nothing but the clock (the caller's) and the query count
  const int qe = tid < width ? (pfe ? pfe[tid] : query[tid]) : -1;
  const int any_valid = __syncthreads_or(qe >= 0 && qe < E);
  if (!any_valid) {
    if (tid == 0 && record_stats) bk.stats[3] += 1;
    __syncthreads();
    return 0;
  }

  // lookup: one query entry per thread (width <= blockDim)
  int my_key = -1, is_miss = 0, is_hit = 0;
  if (tid < width) {
    const int e = qe;
    if (e >= 0 && e < E) {
      my_key = bk.layer * E + e;
      int s = pfs ? pfs[tid] : bk.key_to_slot[my_key];
      if (pfs && s >= 0 && ((taken[s >> 5] >> (s & 31)) & 1u)) s = -1;  // evicted by an earlier query
      if (s >= 0) {
        if (lrfu) {  // the hit's value decayed to now, plus this reference
          const uint64_t c = crf_decay(bk.slot_crf[s], now - bk.slot_stamp[s], bk.decay) + kCrfOne;
          bk.slot_crf[s] = c > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)c;
        }
        bk.slot_stamp[s] = now;  // touch the hit
        atomicOr(&sh.hit_bits[s >> 5], 1u << (s & 31));
        is_hit = 1;
      } else {
        is_miss = 1;
      }
    }
  }
  {  // the hits counted per wave: one LDS atomic per wave instead of one per hit
    const uint64_t hits = __ballot(is_hit);
    if (lane_id() == 0 && hits) atomicAdd(&sh.nhit, (int)__popcll(hits));
  }
  const int m = __syncthreads_count(is_miss);
  // misses keep query order: exclusive scan of the miss flags
  if (m > 0) {
    const int lane = lane_id(), wv = tid / kWave, nw = blockDim.x / kWave;
    const int v = wave_incl_sum(is_miss);
    if (lane == kWave - 1) sh.wave_tot[wv] = v;
    __syncthreads();
    if (wv == 0) {
      const int t = wave_incl_sum(lane < nw ? sh.wave_tot[lane] : 0);
      if (lane < nw) sh.wave_tot[lane] = t;
    }
    __syncthreads();
    const int before = wv > 0 ? sh.wave_tot[wv - 1] : 0;
    if (tid < SCR_MAX_QUERY_WIDTH) {
      sh.q_key[tid] = my_key;
      sh.q_miss_rank[tid] = is_miss ? before + v - 1 : -1;
    }
    __syncthreads();
  }
  // LRFU: untouched slots stamped at or after the pin (earlier queries of the
  // chunk) are no candidates either
  if (lrfu) {
    int np = 0;
    for (int s = tid; s < S; s += blockDim.x)
      if (!((sh.hit_bits[s >> 5] >> (s & 31)) & 1u) && bk.slot_stamp[s] >= pin) ++np;
    if (np) atomicAdd(&sh.npinned, np);
    __syncthreads();
  }

  const int n_cand = S - sh.nhit - sh.npinned;
  const int m_adm = m < n_cand ? m : n_cand;

  if (m_adm > 0) {
    // radix select: the m_adm-th smallest candidate key, 8 bits at a time
    if (tid == 0) {
      sh.prefix = 0;
      sh.rank = (unsigned)m_adm;
    }
    __syncthreads();
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += blockDim.x) sh.hist[i] = 0;
      __syncthreads();
      const uint64_t prefix = sh.prefix;
      for (int s = tid; s < S; s += blockDim.x) {
        if ((sh.hit_bits[s >> 5] >> (s & 31)) & 1u) continue;
        if (lrfu && bk.slot_stamp[s] >= pin) continue;
        const uint64_t key = victim_key(bk, s, now);
        const bool match = (shift == 56) ? true : ((key >> (shift + 8)) == prefix);
        if (match) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        unsigned r = sh.rank, acc = 0;
        int d = 0;
        for (; d < 256; ++d) {
          if (acc + sh.hist[d] >= r) break;
          acc += sh.hist[d];
        }
        sh.rank = r - acc;
        sh.prefix = (prefix << 8) | (uint64_t)d;
      }
      __syncthreads();
    }
    const uint64_t thresh = sh.prefix;
    // collect the selected candidates (exactly m_adm distinct keys <= thresh)
    for (int s = tid; s < S; s += blockDim.x) {
      if ((sh.hit_bits[s >> 5] >> (s & 31)) & 1u) continue;
      if (lrfu && bk.slot_stamp[s] >= pin) continue;
      const uint64_t key = victim_key(bk, s, now);
      if (key <= thresh) {
        const int idx = atomicAdd(&sh.nsel, 1);
        if (idx < SCR_MAX_QUERY_WIDTH) sh.sel_key[idx] = key;
      }
    }
    __syncthreads();
    // order the selection ascending: rank = number of smaller selected keys
    const int nsel = sh.nsel < m_adm ? sh.nsel : m_adm;
    for (int i = tid; i < nsel; i += blockDim.x) {
      const uint64_t ki = sh.sel_key[i];
      int rank = 0;
      for (int j = 0; j < nsel; ++j) rank += sh.sel_key[j] < ki;
      sh.victim[rank] = (int)(ki & ((1ull << kSlotBits) - 1));
    }
    __syncthreads();
    // the i-th miss takes the i-th victim
    if (tid < width) {
      const int r = sh.q_miss_rank[tid];
      if (r >= 0 && r < nsel) {
        const int v = sh.victim[r];
        const int key = sh.q_key[tid];
        const int old = bk.slot_key[v];
        if (old >= 0) {
          bk.key_to_slot[old] = -1;
          atomicAdd(&sh.evict, 1);
        }
        bk.slot_key[v] = key;
        bk.key_to_slot[key] = v;
        bk.slot_stamp[v] = now;
        if (lrfu) bk.slot_crf[v] = kCrfOne;
        if (taken) atomicOr(&taken[v >> 5], 1u << (v & 31));
        miss_slot[r] = v;
        miss_key[r] = key;
      }
    }
    __syncthreads();
  }

  if (tid == 0) {
    if (m > m_adm) atomicOr(bk.err, SCR_ERR_CAPACITY);
    if (record_stats) {
      bk.stats[0] += (uint64_t)sh.nhit;
      bk.stats[1] += (uint64_t)m_adm;
      bk.stats[2] += (uint64_t)sh.evict;
      bk.stats[3] += 1;
    }
  }
  if (record_stats && my_key >= 0) bk.decode_freq[my_key] += 1u;
  __syncthreads();
  return m_adm;
}

__global__ __launch_bounds__(kLruThreads) void ensure_slots_kernel(BankRefs bk, uint64_t* __restrict__ clock,
                                                                  const int32_t* __restrict__ query, int width,
                                                                  int record_stats, int32_t* __restrict__ miss_slot,
                                                                  int32_t* __restrict__ miss_key,
                                                                  int32_t* __restrict__ n_miss, int chunk_first) {
  __shared__ EnsureShared sh;
  const uint64_t now = *clock + 1;
  // a chunk starts at q_begin = 0; its later queries pin from that clock
  uint64_t pin = now;
  if (bk.chunk_start) {
    if (!chunk_first) pin = *bk.chunk_start;
    else if (threadIdx.x == 0) *bk.chunk_start = now;
  }
  const int m = ensure_query(sh, bk, now, pin, query, width, record_stats, miss_slot, miss_key);
  if (threadIdx.x == 0) {
    *n_miss = m;
    *clock = now;
  }
}

// Several consecutive queries in one launch, each with its own clock tick.
// Their admitted misses are appended to one list; an entry whose slot was
// taken again by a later query of the same call is marked superseded (slot -1)
// so that one copy over the list moves only each slot's final record.
// prefilled: the chunk planner's dedup already wrote the entries and their
// slots into sh.pf_e / sh.pf_s (only when they fit, see ensure_prefetches).
// Queries from valid_queries on hold only sentinels (the tail of a dedup'd
// list): each is one clock tick and one counted query, as ensure_query would
// make it, without its barriers.
__device__ __forceinline__ bool ensure_prefetches(int entries, int S) {
  return entries <= kEnsPrefetch && S <= kPrefetchSlots;
}

__device__ __forceinline__ void ensure_batched_block(EnsureShared& sh, const BankRefs& bk, uint64_t* __restrict__ clock,
                                                     const int32_t* __restrict__ distinct, int width, int n_queries,
                                                     int last_width, int record_stats, int32_t* __restrict__ miss_slot,
                                                     int32_t* __restrict__ miss_key, int32_t* __restrict__ n_miss,
                                                     int32_t* __restrict__ n_total, bool prefilled = false,
                                                     int valid_queries = 1 << 30) {
  uint64_t now = *clock;
  const uint64_t pin = now + 1;  // the call is one chunk: its first query's clock
  if (bk.chunk_start && threadIdx.x == 0) *bk.chunk_start = pin;
  const int entries = (n_queries - 1) * width + last_width;
  const bool pf = ensure_prefetches(entries, bk.S);
  if (pf) {  // every entry's slot in one round of loads
    if (!prefilled)
      for (int i = threadIdx.x; i < entries; i += blockDim.x) {
        const int e = distinct[i];
        sh.pf_e[i] = e;
        sh.pf_s[i] = (e >= 0 && e < bk.E) ? bk.key_to_slot[(size_t)bk.layer * bk.E + e] : -1;
      }
    for (int i = threadIdx.x; i < (bk.S + 31) / 32; i += blockDim.x) sh.taken[i] = 0;
    __syncthreads();
    // A chunk whose every valid entry is resident admits nothing, so its
    // queries need no candidate selection: each hit is touched at its own
    // query's clock (keys are distinct, so no slot twice), and the counts are
    // those the per-query path would add.  One barrier for the whole call.
    int valid = 0, miss = 0;
    for (int i = threadIdx.x; i < entries; i += blockDim.x) {
      const int e = sh.pf_e[i];
      if (e >= 0 && e < bk.E) {
        ++valid;
        miss |= sh.pf_s[i] < 0;
      }
    }
    const int wvalid = wave_incl_sum(valid);
    if (lane_id() == kWave - 1) sh.wave_tot[threadIdx.x / kWave] = wvalid;
    if (!__syncthreads_or(miss)) {
      const bool lrfu = bk.policy == SCR_POLICY_LRFU;
      for (int i = threadIdx.x; i < entries; i += blockDim.x) {
        const int e = sh.pf_e[i];
        if (e < 0 || e >= bk.E) continue;
        const int s = sh.pf_s[i];
        const uint64_t tq = now + 1 + (uint64_t)(i / width);
        if (lrfu) {
          const uint64_t c = crf_decay(bk.slot_crf[s], tq - bk.slot_stamp[s], bk.decay) + kCrfOne;
          bk.slot_crf[s] = c > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)c;
        }
        bk.slot_stamp[s] = tq;
        if (record_stats) bk.decode_freq[(size_t)bk.layer * bk.E + e] += 1u;
      }
      if (threadIdx.x == 0) {
        if (record_stats) {
          int hits = 0;
          for (int w = 0; w < (int)blockDim.x / kWave; ++w) hits += sh.wave_tot[w];
          bk.stats[0] += (uint64_t)hits;
          bk.stats[3] += (uint64_t)n_queries;
        }
        for (int q = 0; q < n_queries; ++q) n_miss[q] = 0;
        *clock = now + (uint64_t)n_queries;
        *n_total = 0;
      }
      return;
    }
  }
  int total = 0;
  for (int q = 0; q < n_queries; ++q) {
    now += 1;
    if (q >= valid_queries) {  // sentinels only
      if (threadIdx.x == 0) {
        if (record_stats) bk.stats[3] += 1;
        n_miss[q] = 0;
      }
      continue;
    }
    const int w = q + 1 < n_queries ? width : last_width;
    const int m = ensure_query(sh, bk, now, pin, distinct + (size_t)q * width, w, record_stats, miss_slot + total,
                               miss_key + total, pf ? sh.pf_e + q * width : nullptr,
                               pf ? sh.pf_s + q * width : nullptr, pf ? sh.taken : nullptr);
    if (threadIdx.x == 0) n_miss[q] = m;
    total += m;
  }
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int v = miss_slot[i];
    if (v >= 0 && bk.slot_key[v] != miss_key[i]) miss_slot[i] = -1;
  }
  if (threadIdx.x == 0) {
    *clock = now;
    *n_total = total;
  }
}

__global__ __launch_bounds__(kLruThreads) void ensure_slots_batched_kernel(
    BankRefs bk, uint64_t* __restrict__ clock, const int32_t* __restrict__ distinct, int width, int n_queries,
    int last_width, int record_stats, int32_t* __restrict__ miss_slot, int32_t* __restrict__ miss_key,
    int32_t* __restrict__ n_miss, int32_t* __restrict__ n_total) {
  __shared__ EnsureShared sh;
  ensure_batched_block(sh, bk, clock, distinct, width, n_queries, last_width, record_stats, miss_slot, miss_key,
                       n_miss, n_total);
}

// The chunk's planning in one workgroup and one launch: dedup of the routed
// ids, the LRU queries over the distinct list, then the align of the routes by
// their (new) slots.  The phases share one LDS area; each phase's global
// writes are visible to the next after the barrier between them.
union PlanShared {
  EnsureShared ens;
  struct {
    int pos[kDedupMaxE];
    int wave_tot[kWave + 1];
  } dd;
  struct {
    int cnt[kSmallBuckets];
    int rb[kSmallRoutes];
    int wave_tot[2 * kWave];
    uint16_t tab[kAlignTab];
  } al;
};

static_assert(offsetof(EnsureShared, pf_e) >= sizeof(PlanShared::dd) &&
                  offsetof(EnsureShared, pf_s) >= sizeof(PlanShared::dd),
              "the dedup's LDS must not overlap the LRU copy it fills");

__global__ __launch_bounds__(kPlanThreads) void plan_chunk_kernel(
    BankRefs bk, uint64_t* __restrict__ clock, const int32_t* __restrict__ ids, int n, int lmax,
    int32_t* __restrict__ distinct, int32_t* __restrict__ n_distinct, int width, int n_queries, int last_width,
    int record_stats, int32_t* __restrict__ miss_slot, int32_t* __restrict__ miss_key, int32_t* __restrict__ n_miss,
    int32_t* __restrict__ n_total, int B, int cap, int32_t* __restrict__ sorted_routes,
    int32_t* __restrict__ block_bucket, int32_t* __restrict__ n_post_pad, int32_t* __restrict__ active_buckets,
    int32_t* __restrict__ active_block_begin, int32_t* __restrict__ n_active) {
  __shared__ PlanShared sh;
  // the dedup writes the distinct list and its slots straight into the LRU's
  // LDS copy (those arrays lie past the dedup's own)
  const bool pf = ensure_prefetches(lmax, bk.S);
  dedup_block(ids, n, bk.E, lmax, distinct, n_distinct, nullptr, sh.dd.pos, sh.dd.wave_tot, pf ? sh.ens.pf_e : nullptr,
              pf ? sh.ens.pf_s : nullptr, bk.key_to_slot + (size_t)bk.layer * bk.E);
  const int n_dist = sh.dd.wave_tot[kWave];  // valid entries fill the list's head
  __syncthreads();
  ensure_batched_block(sh.ens, bk, clock, distinct, width, n_queries, last_width, record_stats, miss_slot, miss_key,
                       n_miss, n_total, pf, (n_dist + width - 1) / width);
  __syncthreads();
  align_small_block(ids, n, bk.key_to_slot + (size_t)bk.layer * bk.E, bk.E, bk.S, B, cap, sorted_routes,
                    block_bucket, n_post_pad, active_buckets, active_block_begin, n_active, sh.al.cnt, sh.al.rb,
                    sh.al.wave_tot, sh.al.tab);
}

__global__ void rebuild_map_clear(int32_t* __restrict__ key_to_slot, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    key_to_slot[i] = -1;
}

__global__ void rebuild_map_fill(const int32_t* __restrict__ slot_key, int S, int n_keys,
                                 int32_t* __restrict__ key_to_slot) {
  for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < S; s += gridDim.x * blockDim.x) {
    const int key = slot_key[s];
    if (key >= 0 && key < n_keys) key_to_slot[key] = s;
  }
}

int check_bank(const scr_bank_desc* b) {
  SCR_CHECK_ARG(b != nullptr, "bank is null");
  SCR_CHECK_ARG(b->S >= 1 && b->S <= SCR_MAX_SLOTS, "bank: S must be in [1, %d] (got %d)", SCR_MAX_SLOTS, b->S);
  SCR_CHECK_ARG(b->L >= 1 && b->E >= 1 && (long long)b->L * b->E < (1ll << 31), "bank: bad L or E");
  SCR_CHECK_ARG(b->slot_key && b->slot_stamp && b->key_to_slot && b->clock && b->stats &&
                    b->decode_freq && b->err,
                "bank: null state pointer");
  SCR_CHECK_ARG(b->policy == SCR_POLICY_LRU || b->policy == SCR_POLICY_LRFU, "bank: unknown policy %d", b->policy);
  SCR_CHECK_ARG(b->policy != SCR_POLICY_LRFU || (b->slot_crf && b->chunk_start && b->lrfu_decay > 0),
                "bank: LRFU needs slot_crf, chunk_start and a decay factor in (0, 2^32)");
  return SCR_OK;
}

static BankRefs bank_refs(const scr_bank_desc* b, int layer) {
  BankRefs r;
  r.S = b->S;
  r.E = b->E;
  r.layer = layer;
  r.slot_key = b->slot_key;
  r.slot_stamp = b->slot_stamp;
  r.key_to_slot = b->key_to_slot;
  r.stats = b->stats;
  r.decode_freq = b->decode_freq;
  r.err = b->err;
  r.policy = b->policy;
  r.decay = b->lrfu_decay;
  r.slot_crf = b->slot_crf;
  r.chunk_start = b->chunk_start;
  return r;
}

}  // namespace scr

extern "C" int scr_ensure_slots(const scr_bank_desc* bank, int layer, const int32_t* distinct, int q_begin,
                                int width, int record_stats, int32_t* miss_slot, int32_t* miss_key,
                                int32_t* n_miss, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  SCR_CHECK_ARG(layer >= 0 && layer < bank->L, "ensure_slots: layer %d out of [0, %d)", layer, bank->L);
  SCR_CHECK_ARG(width >= 1 && width <= SCR_MAX_QUERY_WIDTH, "ensure_slots: width must be in [1, %d]",
                SCR_MAX_QUERY_WIDTH);
  SCR_CHECK_ARG(q_begin >= 0, "ensure_slots: q_begin must be >= 0");
  SCR_CHECK_ARG(distinct && miss_slot && miss_key && n_miss, "ensure_slots: null pointer");
  hipLaunchKernelGGL(scr::ensure_slots_kernel, dim3(1), dim3(scr::kLruThreads), 0, stream,
                     scr::bank_refs(bank, layer), bank->clock, distinct + q_begin, width, record_stats ? 1 : 0,
                     miss_slot, miss_key, n_miss, q_begin == 0 ? 1 : 0);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

extern "C" int scr_ensure_slots_batched(const scr_bank_desc* bank, int layer, const int32_t* distinct, int n,
                                        int width, int record_stats, int32_t* miss_slot, int32_t* miss_key,
                                        int32_t* n_miss, int32_t* n_total, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  SCR_CHECK_ARG(layer >= 0 && layer < bank->L, "ensure_slots_batched: layer %d out of [0, %d)", layer, bank->L);
  SCR_CHECK_ARG(width >= 1 && width <= SCR_MAX_QUERY_WIDTH, "ensure_slots_batched: width must be in [1, %d]",
                SCR_MAX_QUERY_WIDTH);
  SCR_CHECK_ARG(n >= 1, "ensure_slots_batched: n must be >= 1");
  SCR_CHECK_ARG(distinct && miss_slot && miss_key && n_miss && n_total, "ensure_slots_batched: null pointer");
  const int n_queries = (n + width - 1) / width;
  const int last_width = n - (n_queries - 1) * width;
  hipLaunchKernelGGL(scr::ensure_slots_batched_kernel, dim3(1), dim3(scr::kLruThreads), 0, stream,
                     scr::bank_refs(bank, layer), bank->clock, distinct, width, n_queries, last_width,
                     record_stats ? 1 : 0, miss_slot, miss_key, n_miss, n_total);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

extern "C" int scr_plan_chunk(const scr_bank_desc* bank, int layer, const int32_t* ids, int n, int32_t* distinct,
                              int32_t* n_distinct, int width, int record_stats, int32_t* miss_slot,
                              int32_t* miss_key, int32_t* n_miss, int32_t* n_total, int block_size,
                              int32_t* sorted_routes, int32_t* block_bucket, int32_t* n_post_pad,
                              int32_t* active_buckets, int32_t* active_block_begin, int32_t* n_active,
                              hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  SCR_CHECK_ARG(layer >= 0 && layer < bank->L, "plan_chunk: layer %d out of [0, %d)", layer, bank->L);
  SCR_CHECK_ARG(width >= 1 && width <= SCR_MAX_QUERY_WIDTH, "plan_chunk: width must be in [1, %d]",
                SCR_MAX_QUERY_WIDTH);
  SCR_CHECK_ARG(n >= 1, "plan_chunk: n must be >= 1");
  SCR_CHECK_ARG(block_size == 16 || block_size == 32 || block_size == 64,
                "plan_chunk: block_size must be 16, 32 or 64");
  SCR_CHECK_ARG(ids && distinct && n_distinct && miss_slot && miss_key && n_miss && n_total && sorted_routes &&
                    block_bucket && n_post_pad && active_buckets && active_block_begin && n_active,
                "plan_chunk: null pointer");
  if (n > scr::kSmallRoutes || bank->E > scr::kDedupMaxE || bank->S > scr::kSmallBuckets) {
    scr::set_error("plan_chunk: n %d, E %d or S %d beyond one workgroup (%d, %d, %d)", n, bank->E, bank->S,
                   scr::kSmallRoutes, scr::kDedupMaxE, scr::kSmallBuckets);
    return SCR_ENOTSUP;
  }
  const int lmax = n < bank->E ? n : bank->E;
  const int n_queries = (lmax + width - 1) / width;
  const int last_width = lmax - (n_queries - 1) * width;
  const int cap = (int)scr_align_capacity(n, bank->S, block_size);
  hipLaunchKernelGGL(scr::plan_chunk_kernel, dim3(1), dim3(scr::kPlanThreads), 0, stream, scr::bank_refs(bank, layer),
                     bank->clock, ids, n, lmax, distinct, n_distinct, width, n_queries, last_width,
                     record_stats ? 1 : 0, miss_slot, miss_key, n_miss, n_total, block_size, cap, sorted_routes,
                     block_bucket, n_post_pad, active_buckets, active_block_begin, n_active);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

extern "C" int scr_bank_rebuild_map(const scr_bank_desc* bank, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  const int n_keys = bank->L * bank->E;
  hipLaunchKernelGGL(scr::rebuild_map_clear, dim3((n_keys + 255) / 256 < 1024 ? (n_keys + 255) / 256 : 1024),
                     dim3(256), 0, stream, bank->key_to_slot, n_keys);
  SCR_CHECK_LAUNCH();
  hipLaunchKernelGGL(scr::rebuild_map_fill, dim3((bank->S + 255) / 256), dim3(256), 0, stream,
                     bank->slot_key, bank->S, n_keys, bank->key_to_slot);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

extern "C" int scr_bank_init(const scr_bank_desc* bank, const int32_t* host_slot_keys, const uint64_t* host_stamps,
                             uint64_t clock, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  SCR_CHECK_ARG(host_slot_keys && host_stamps, "bank_init: null host array");
  const int S = bank->S;
  const long long n_keys = (long long)bank->L * bank->E;
  // the state must be one the planners can continue from: keys in range and
  // each held by at most one slot, no stamp ahead of the clock, empty slots
  // never stamped
  std::vector<unsigned char> seen((size_t)n_keys, 0);
  for (int s = 0; s < S; ++s) {
    const int32_t key = host_slot_keys[s];
    SCR_CHECK_ARG(key >= -1 && key < n_keys, "bank_init: slot %d holds key %d outside [-1, %lld)", s, key, n_keys);
    SCR_CHECK_ARG(host_stamps[s] <= clock, "bank_init: slot %d is stamped after the clock", s);
    if (key < 0) {
      SCR_CHECK_ARG(host_stamps[s] == 0, "bank_init: empty slot %d has a non-zero stamp", s);
      continue;
    }
    SCR_CHECK_ARG(!seen[key], "bank_init: key %d is held by more than one slot", key);
    seen[key] = 1;
  }
  SCR_CHECK_HIP(hipMemcpyAsync(bank->slot_key, host_slot_keys, (size_t)S * sizeof(int32_t), hipMemcpyHostToDevice,
                               stream));
  SCR_CHECK_HIP(hipMemcpyAsync(bank->slot_stamp, host_stamps, (size_t)S * sizeof(uint64_t), hipMemcpyHostToDevice,
                               stream));
  SCR_CHECK_HIP(hipMemcpyAsync(bank->clock, &clock, sizeof(uint64_t), hipMemcpyHostToDevice, stream));
  SCR_CHECK_HIP(hipMemsetAsync(bank->stats, 0, 4 * sizeof(uint64_t), stream));
  SCR_CHECK_HIP(hipMemsetAsync(bank->decode_freq, 0, (size_t)n_keys * sizeof(uint32_t), stream));
  SCR_CHECK_HIP(hipMemsetAsync(bank->err, 0, sizeof(uint32_t), stream));
  if (bank->slot_crf) SCR_CHECK_HIP(hipMemsetAsync(bank->slot_crf, 0, (size_t)S * sizeof(uint32_t), stream));
  if (bank->chunk_start) SCR_CHECK_HIP(hipMemsetAsync(bank->chunk_start, 0, sizeof(uint64_t), stream));
  rc = scr_bank_rebuild_map(bank, stream);
  if (rc) return rc;
  // the host arrays (and `clock`, a local) are read by the copies above
  SCR_CHECK_HIP(hipStreamSynchronize(stream));
  return SCR_OK;
}
