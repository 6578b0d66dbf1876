// Device-side LRU planner over a bank keyed by (layer, expert).
//
// A query of distinct expert ids is admitted in one workgroup (FreeToken PR
// #676, Solution second bullet and the author's reply: LRU only, earlier
// queries evicted last; vLLM fork PR #48, What: a device-side planner over one
// bank shared by all layers).  Recency is one stamp per query; candidates for
// eviction are ordered by the 64-bit key (stamp << 20 | slot), found by an
// 8-bit radix select in LDS instead of sorting the bank.
#include "common.h"

namespace scr {

constexpr int kLruThreads = 1024;
constexpr int kSlotBits = 20;  // SCR_MAX_SLOTS <= 2^18 < 2^20

__device__ __forceinline__ uint64_t cand_key(uint64_t stamp, int slot) {
  return (stamp << kSlotBits) | (uint64_t)slot;
}

__global__ __launch_bounds__(kLruThreads) void ensure_slots_kernel(
    int S, int E, int layer, int32_t* __restrict__ slot_key, uint64_t* __restrict__ slot_stamp,
    int32_t* __restrict__ key_to_slot, uint64_t* __restrict__ clock, uint64_t* __restrict__ stats,
    uint32_t* __restrict__ decode_freq, uint32_t* __restrict__ err, const int32_t* __restrict__ query,
    int width, int record_stats, int32_t* __restrict__ miss_slot, int32_t* __restrict__ miss_key,
    int32_t* __restrict__ n_miss) {
  __shared__ uint32_t hit_bits[SCR_MAX_SLOTS / 32];
  __shared__ int q_key[SCR_MAX_QUERY_WIDTH];
  __shared__ int q_miss_rank[SCR_MAX_QUERY_WIDTH];  // -1: not a miss
  __shared__ uint64_t sel_key[SCR_MAX_QUERY_WIDTH];
  __shared__ int victim[SCR_MAX_QUERY_WIDTH];
  __shared__ unsigned hist[256];
  __shared__ int wave_tot[kWave + 1];
  __shared__ int s_nhit, s_nmiss, s_nsel, s_evict;
  __shared__ uint64_t s_prefix;
  __shared__ unsigned s_rank;

  const int tid = threadIdx.x;
  const uint64_t now = *clock + 1;
  const int nwords = (S + 31) / 32;
  for (int i = tid; i < nwords; i += blockDim.x) hit_bits[i] = 0;
  if (tid == 0) {
    s_nhit = 0;
    s_evict = 0;
    s_nsel = 0;
  }
  __syncthreads();

  // lookup: one query entry per thread (width <= blockDim)
  int my_key = -1, is_miss = 0;
  if (tid < width) {
    const int e = query[tid];
    if (e >= 0 && e < E) {
      my_key = layer * E + e;
      const int s = key_to_slot[my_key];
      if (s >= 0) {
        slot_stamp[s] = now;  // touch the hit
        atomicOr(&hit_bits[s >> 5], 1u << (s & 31));
        atomicAdd(&s_nhit, 1);
      } else {
        is_miss = 1;
      }
    }
  }
  // misses keep query order: exclusive scan of the miss flags
  {
    const int lane = lane_id(), wv = tid / kWave, nw = blockDim.x / kWave;
    int v = is_miss;
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
    if (tid < SCR_MAX_QUERY_WIDTH) {
      q_key[tid] = my_key;
      q_miss_rank[tid] = is_miss ? before + v - 1 : -1;
    }
    if (tid == 0) s_nmiss = wave_tot[nw - 1];
  }
  __syncthreads();

  const int m = s_nmiss;
  const int n_cand = S - s_nhit;
  const int m_adm = m < n_cand ? m : n_cand;

  if (m_adm > 0) {
    // radix select: the m_adm-th smallest candidate key, 8 bits at a time
    if (tid == 0) {
      s_prefix = 0;
      s_rank = (unsigned)m_adm;
    }
    __syncthreads();
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
      __syncthreads();
      const uint64_t prefix = s_prefix;
      for (int s = tid; s < S; s += blockDim.x) {
        if ((hit_bits[s >> 5] >> (s & 31)) & 1u) continue;
        const uint64_t key = cand_key(slot_stamp[s], s);
        const bool match = (shift == 56) ? true : ((key >> (shift + 8)) == prefix);
        if (match) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        unsigned r = s_rank, acc = 0;
        int d = 0;
        for (; d < 256; ++d) {
          if (acc + hist[d] >= r) break;
          acc += hist[d];
        }
        s_rank = r - acc;
        s_prefix = (prefix << 8) | (uint64_t)d;
      }
      __syncthreads();
    }
    const uint64_t thresh = s_prefix;
    // collect the selected candidates (exactly m_adm distinct keys <= thresh)
    for (int s = tid; s < S; s += blockDim.x) {
      if ((hit_bits[s >> 5] >> (s & 31)) & 1u) continue;
      const uint64_t key = cand_key(slot_stamp[s], s);
      if (key <= thresh) {
        const int idx = atomicAdd(&s_nsel, 1);
        if (idx < SCR_MAX_QUERY_WIDTH) sel_key[idx] = key;
      }
    }
    __syncthreads();
    // order the selection ascending: rank = number of smaller selected keys
    const int nsel = s_nsel < m_adm ? s_nsel : m_adm;
    for (int i = tid; i < nsel; i += blockDim.x) {
      const uint64_t ki = sel_key[i];
      int rank = 0;
      for (int j = 0; j < nsel; ++j) rank += sel_key[j] < ki;
      victim[rank] = (int)(ki & ((1ull << kSlotBits) - 1));
    }
    __syncthreads();
    // the i-th miss takes the i-th victim
    if (tid < width) {
      const int r = q_miss_rank[tid];
      if (r >= 0 && r < nsel) {
        const int v = victim[r];
        const int key = q_key[tid];
        const int old = slot_key[v];
        if (old >= 0) {
          key_to_slot[old] = -1;
          atomicAdd(&s_evict, 1);
        }
        slot_key[v] = key;
        key_to_slot[key] = v;
        slot_stamp[v] = now;
        miss_slot[r] = v;
        miss_key[r] = key;
      }
    }
    __syncthreads();
  }

  if (tid == 0) {
    *n_miss = m_adm;
    *clock = now;
    if (m > m_adm) atomicOr(err, SCR_ERR_CAPACITY);
    if (record_stats) {
      stats[0] += (uint64_t)s_nhit;
      stats[1] += (uint64_t)m_adm;
      stats[2] += (uint64_t)s_evict;
      stats[3] += 1;
    }
  }
  if (record_stats && my_key >= 0) decode_freq[my_key] += 1u;
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
  return SCR_OK;
}

}  // namespace scr

extern "C" int scr_ensure_slots(const scr_bank_desc* bank, int layer, const int32_t* distinct,
                                int q_begin, int width, int record_stats, int32_t* miss_slot,
                                int32_t* miss_key, int32_t* n_miss, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  SCR_CHECK_ARG(layer >= 0 && layer < bank->L, "ensure_slots: layer %d out of [0, %d)", layer, bank->L);
  SCR_CHECK_ARG(width >= 1 && width <= SCR_MAX_QUERY_WIDTH, "ensure_slots: width must be in [1, %d]",
                SCR_MAX_QUERY_WIDTH);
  SCR_CHECK_ARG(q_begin >= 0, "ensure_slots: q_begin must be >= 0");
  SCR_CHECK_ARG(distinct && miss_slot && miss_key && n_miss, "ensure_slots: null pointer");
  hipLaunchKernelGGL(scr::ensure_slots_kernel, dim3(1), dim3(scr::kLruThreads), 0, stream, bank->S,
                     bank->E, layer, bank->slot_key, bank->slot_stamp, bank->key_to_slot, bank->clock,
                     bank->stats, bank->decode_freq, bank->err, distinct + q_begin, width,
                     record_stats ? 1 : 0, miss_slot, miss_key, n_miss);
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
