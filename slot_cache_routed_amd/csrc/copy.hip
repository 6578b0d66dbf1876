// Host-to-bank row movement: fixed-grid miss copies, whole-layer streaming,
// and prefill staging.
//
// Misses are copied by a kernel that reads the pinned host pool through its
// device-mapped view, with a grid that does not depend on the miss count, so
// the demand path needs no host sync (FreeToken PR #676, Solution; vLLM fork
// PR #48, What: fixed-grid row copies from the host source's accelerator
// view).  Whole layers and staging runs are copied the same way, by a
// kernel over record ranges whose descriptors travel as a kernel argument
// (the host link sustains about 57 GB/s this way against about 50 GB/s for
// one DMA per run); staging runs on a side stream ordered by events (vLLM
// fork PR #51, Prefill staging) with a small fixed grid, so that the GEMMs
// on the compute stream keep most of the chip.
#include "common.h"

#include <vector>

namespace scr {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr uint64_t kCopyChunk = 64 * 1024;  // bytes per work item
constexpr int kCopyUnroll = kCopyChunk / (kCopyThreads * 16);  // 16-byte loads per thread
constexpr uint64_t kMissGrid = 256;  // workgroups of a miss copy

// Work item w = (miss i, chunk c).  Each thread issues all of its 16-byte
// loads before its stores so many PCIe reads are in flight.
__global__ __launch_bounds__(kCopyThreads) void copy_misses_kernel(
    uint8_t* __restrict__ bank_rows, uint64_t rec, const void* const* __restrict__ key_rows,
    const int32_t* __restrict__ miss_slot, const int32_t* __restrict__ miss_key,
    const int32_t* __restrict__ n_miss_p, int max_miss, int n_keys, int n_slots) {
  const int n_miss = min(*n_miss_p, max_miss);
  const uint64_t chunks = (rec + kCopyChunk - 1) / kCopyChunk;
  const uint64_t items = (uint64_t)n_miss * chunks;
  for (uint64_t w = blockIdx.x; w < items; w += gridDim.x) {
    const int i = (int)(w / chunks);
    const uint64_t c = w % chunks;
    const int slot = miss_slot[i];
    const int key = miss_key[i];
    if (slot < 0 || slot >= n_slots || key < 0 || key >= n_keys) continue;
    const u32x4* src = reinterpret_cast<const u32x4*>(
        static_cast<const uint8_t*>(key_rows[key]) + c * kCopyChunk);
    u32x4* dst = reinterpret_cast<u32x4*>(bank_rows + (uint64_t)slot * rec + c * kCopyChunk);
    const uint64_t bytes = min(kCopyChunk, rec - c * kCopyChunk);
    const int n16 = (int)(bytes / 16);
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int j = u * kCopyThreads + threadIdx.x;
      if (j < n16) v[u] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int j = u * kCopyThreads + threadIdx.x;
      if (j < n16) dst[j] = v[u];
    }
  }
}

__global__ void fill_row_table_kernel(const uint8_t* base, int n, uint64_t stride, const void** rows) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    rows[i] = base + (uint64_t)i * stride;
}

__global__ void fill_staged_rows_kernel(const int32_t* __restrict__ key_to_slot, int layer, int E,
                                        const uint8_t* bank_rows, const uint8_t* staging,
                                        uint64_t rec, const void** rows) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x) {
    const int s = key_to_slot[layer * E + e];
    rows[e] = s >= 0 ? bank_rows + (uint64_t)s * rec : staging + (uint64_t)e * rec;
  }
}

int check_pool(const scr_host_pool* p) {
  SCR_CHECK_ARG(p != nullptr, "pool is null");
  SCR_CHECK_ARG(p->L >= 1 && p->E >= 1, "pool: bad L or E");
  SCR_CHECK_ARG(p->record_bytes > 0 && p->record_bytes % 16 == 0,
                "pool: record_bytes must be a positive multiple of 16");
  return SCR_OK;
}
int check_bank(const scr_bank_desc* b);

// Record ranges of one layer, passed by value: expert range i is
// [e_begin[i], e_begin[i] + count[i]), copied to dst + e * record_bytes.
constexpr int kRangesPerLaunch = 240;
struct RecordRanges {
  int n;
  int32_t e_begin[kRangesPerLaunch];
  int32_t count[kRangesPerLaunch];
};
constexpr int kRangeGridWide = 2048;  // whole layers: as many reads in flight as the chip takes
constexpr int kRangeGridSide = 64;    // staging beside the GEMMs: enough for the host link

// Work item w = (record of the ranges, 64 KiB chunk of it); every record is
// read through its own device-mapped pool pointer (no adjacency assumed).
__global__ __launch_bounds__(kCopyThreads) void copy_ranges_kernel(const void* const* __restrict__ key_rows,
                                                                   int layer, int E, uint64_t rec,
                                                                   uint8_t* __restrict__ dst, RecordRanges rg) {
  const uint64_t chunks = (rec + kCopyChunk - 1) / kCopyChunk;
  int total = 0;
  for (int i = 0; i < rg.n; ++i) total += rg.count[i];
  const uint64_t items = (uint64_t)total * chunks;
  for (uint64_t w = blockIdx.x; w < items; w += gridDim.x) {
    int j = (int)(w / chunks);  // record index over the ranges
    const uint64_t c = w % chunks;
    int i = 0;
    while (j >= rg.count[i]) j -= rg.count[i++];
    const int e = rg.e_begin[i] + j;
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(key_rows[(size_t)layer * E + e]) +
                                                      c * kCopyChunk);
    u32x4* out = reinterpret_cast<u32x4*>(dst + (uint64_t)e * rec + c * kCopyChunk);
    const uint64_t bytes = min(kCopyChunk, rec - c * kCopyChunk);
    const int n16 = (int)(bytes / 16);
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int q = u * kCopyThreads + threadIdx.x;
      if (q < n16) v[u] = __builtin_nontemporal_load(src + q);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int q = u * kCopyThreads + threadIdx.x;
      if (q < n16) out[q] = v[u];
    }
  }
}

// launches the copy of ranges (e_begin, count) of `layer`, kRangesPerLaunch at a time
int copy_record_ranges(const scr_host_pool* pool, int layer, const int32_t* e_begin, const int32_t* count, int n,
                       uint8_t* dst, int grid_cap, hipStream_t stream) {
  const uint64_t chunks = (pool->record_bytes + kCopyChunk - 1) / kCopyChunk;
  for (int i0 = 0; i0 < n; i0 += kRangesPerLaunch) {
    RecordRanges rg;
    rg.n = n - i0 < kRangesPerLaunch ? n - i0 : kRangesPerLaunch;
    uint64_t recs = 0;
    for (int i = 0; i < rg.n; ++i) {
      rg.e_begin[i] = e_begin[i0 + i];
      rg.count[i] = count[i0 + i];
      recs += (uint64_t)count[i0 + i];
    }
    uint64_t grid = recs * chunks;
    if (grid > (uint64_t)grid_cap) grid = (uint64_t)grid_cap;
    if (grid == 0) continue;
    hipLaunchKernelGGL(copy_ranges_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, stream, pool->key_rows_dev,
                       layer, pool->E, pool->record_bytes, dst, rg);
    SCR_CHECK_LAUNCH();
  }
  return SCR_OK;
}

}  // namespace scr

extern "C" int scr_copy_misses(const scr_bank_desc* bank, const scr_host_pool* pool,
                               const int32_t* miss_slot, const int32_t* miss_key,
                               const int32_t* n_miss, int max_miss, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  rc = scr::check_pool(pool);
  if (rc) return rc;
  SCR_CHECK_ARG(bank->rows != nullptr, "copy_misses: bank rows are null");
  SCR_CHECK_ARG(pool->key_rows_dev != nullptr, "copy_misses: pool has no device-mapped table");
  SCR_CHECK_ARG(pool->record_bytes == bank->record_bytes, "copy_misses: record sizes differ");
  SCR_CHECK_ARG(pool->L == bank->L && pool->E == bank->E, "copy_misses: pool and bank key spaces differ");
  SCR_CHECK_ARG(max_miss >= 0 && max_miss <= 65536, "copy_misses: max_miss out of range");
  SCR_CHECK_ARG(miss_slot && miss_key && n_miss, "copy_misses: null pointer");
  if (max_miss == 0) return SCR_OK;
  const uint64_t chunks = (pool->record_bytes + scr::kCopyChunk - 1) / scr::kCopyChunk;
  // 256 workgroups keep 16 MB of host reads in flight, several times what the
  // host link needs; a launch with nothing to copy (a warm chunk) stays short
  uint64_t grid = (uint64_t)max_miss * chunks;
  if (grid > scr::kMissGrid) grid = scr::kMissGrid;
  hipLaunchKernelGGL(scr::copy_misses_kernel, dim3((unsigned)grid), dim3(scr::kCopyThreads), 0, stream,
                     bank->rows, pool->record_bytes, pool->key_rows_dev, miss_slot, miss_key, n_miss,
                     max_miss, bank->L * bank->E, bank->S);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

extern "C" int scr_stream_layer_async(const scr_host_pool* pool, int layer, void* dst, hipStream_t stream) {
  int rc = scr::check_pool(pool);
  if (rc) return rc;
  SCR_CHECK_ARG(pool->key_rows_dev != nullptr && dst != nullptr, "stream_layer: null pointer");
  SCR_CHECK_ARG(layer >= 0 && layer < pool->L, "stream_layer: layer out of range");
  const int32_t begin = 0, count = pool->E;
  return scr::copy_record_ranges(pool, layer, &begin, &count, 1, static_cast<uint8_t*>(dst), scr::kRangeGridWide,
                                 stream);
}

extern "C" int scr_stage_plan(const scr_bank_desc* bank, const scr_host_pool* pool, int layer_begin,
                              int n_layers, int32_t* host_map, scr_run* runs, int max_runs,
                              int* n_runs, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  rc = scr::check_pool(pool);
  if (rc) return rc;
  SCR_CHECK_ARG(host_map && runs && n_runs && pool->key_rows_host, "stage_plan: null pointer");
  SCR_CHECK_ARG(layer_begin >= 0 && n_layers >= 1 && layer_begin + n_layers <= bank->L,
                "stage_plan: layer range out of the bank");
  SCR_CHECK_ARG(pool->E == bank->E && pool->L == bank->L, "stage_plan: pool and bank key spaces differ");
  const int E = bank->E;
  SCR_CHECK_HIP(hipMemcpyAsync(host_map, bank->key_to_slot + (size_t)layer_begin * E,
                               (size_t)n_layers * E * sizeof(int32_t), hipMemcpyDeviceToHost, stream));
  SCR_CHECK_HIP(hipStreamSynchronize(stream));
  const uint64_t rec = pool->record_bytes;
  int n = 0;
  for (int li = 0; li < n_layers; ++li) {
    const int layer = layer_begin + li;
    int e = 0;
    while (e < E) {
      if (host_map[(size_t)li * E + e] >= 0) {
        ++e;
        continue;
      }
      const uint8_t* src0 = static_cast<const uint8_t*>(pool->key_rows_host[(size_t)layer * E + e]);
      int run = 1;
      while (e + run < E && host_map[(size_t)li * E + e + run] < 0 &&
             static_cast<const uint8_t*>(pool->key_rows_host[(size_t)layer * E + e + run]) ==
                 src0 + (uint64_t)run * rec)
        ++run;
      if (n >= max_runs) {
        scr::set_error("stage_plan: more than %d runs", max_runs);
        *n_runs = n;
        return SCR_ECAPACITY;
      }
      runs[n].layer = layer;
      runs[n].e_begin = e;
      runs[n].count = run;
      ++n;
      e += run;
    }
  }
  *n_runs = n;
  return SCR_OK;
}

extern "C" int scr_stage_rows_async(const scr_host_pool* pool, const scr_run* runs, int n_runs, int layer,
                                    void* dst_layer_buf, hipStream_t side, hipEvent_t wait_on,
                                    hipEvent_t done) {
  int rc = scr::check_pool(pool);
  if (rc) return rc;
  SCR_CHECK_ARG(n_runs >= 0 && (n_runs == 0 || runs), "stage_rows: bad runs");
  SCR_CHECK_ARG(dst_layer_buf && pool->key_rows_dev, "stage_rows: null pointer");
  SCR_CHECK_ARG(layer >= 0 && layer < pool->L, "stage_rows: layer out of range");
  for (int i = 0; i < n_runs; ++i)
    SCR_CHECK_ARG(runs[i].e_begin >= 0 && runs[i].count >= 1 && runs[i].e_begin + runs[i].count <= pool->E,
                  "stage_rows: run %d out of the layer", i);
  std::vector<int32_t> begin, count;
  for (int i = 0; i < n_runs; ++i)
    if (runs[i].layer == layer) {
      begin.push_back(runs[i].e_begin);
      count.push_back(runs[i].count);
    }
  if (wait_on) SCR_CHECK_HIP(hipStreamWaitEvent(side, wait_on, 0));
  rc = scr::copy_record_ranges(pool, layer, begin.data(), count.data(), (int)begin.size(),
                               static_cast<uint8_t*>(dst_layer_buf), scr::kRangeGridSide, side);
  if (rc) return rc;
  if (done) SCR_CHECK_HIP(hipEventRecord(done, side));
  return SCR_OK;
}

extern "C" int scr_stage_rows_dma_async(const scr_host_pool* pool, const scr_run* runs, int n_runs, int layer,
                                        void* dst_layer_buf, hipStream_t side, hipEvent_t wait_on,
                                        hipEvent_t done) {
  int rc = scr::check_pool(pool);
  if (rc) return rc;
  SCR_CHECK_ARG(n_runs >= 0 && (n_runs == 0 || runs), "stage_rows_dma: bad runs");
  SCR_CHECK_ARG(dst_layer_buf && pool->key_rows_host, "stage_rows_dma: null pointer");
  SCR_CHECK_ARG(layer >= 0 && layer < pool->L, "stage_rows_dma: layer out of range");
  for (int i = 0; i < n_runs; ++i)
    SCR_CHECK_ARG(runs[i].e_begin >= 0 && runs[i].count >= 1 && runs[i].e_begin + runs[i].count <= pool->E,
                  "stage_rows_dma: run %d out of the layer", i);
  const uint64_t rec = pool->record_bytes;
  for (int i = 0; i < n_runs; ++i) {  // a run's host records are adjacent (scr_stage_plan builds them so)
    if (runs[i].layer != layer) continue;
    const uint8_t* src0 = static_cast<const uint8_t*>(pool->key_rows_host[(size_t)layer * pool->E + runs[i].e_begin]);
    for (int j = 1; j < runs[i].count; ++j)
      SCR_CHECK_ARG(static_cast<const uint8_t*>(pool->key_rows_host[(size_t)layer * pool->E + runs[i].e_begin + j]) ==
                        src0 + (uint64_t)j * rec,
                    "stage_rows_dma: run %d is not contiguous in host memory", i);
  }
  if (wait_on) SCR_CHECK_HIP(hipStreamWaitEvent(side, wait_on, 0));
  uint8_t* dst = static_cast<uint8_t*>(dst_layer_buf);
  for (int i = 0; i < n_runs; ++i) {
    if (runs[i].layer != layer) continue;
    const uint8_t* src = static_cast<const uint8_t*>(pool->key_rows_host[(size_t)layer * pool->E + runs[i].e_begin]);
    SCR_CHECK_HIP(hipMemcpyAsync(dst + (uint64_t)runs[i].e_begin * rec, src, (uint64_t)runs[i].count * rec,
                                 hipMemcpyHostToDevice, side));
  }
  if (done) SCR_CHECK_HIP(hipEventRecord(done, side));
  return SCR_OK;
}

extern "C" int scr_fill_row_table(const void* base, int n, uint64_t stride, const void** bucket_rows,
                                  hipStream_t stream) {
  SCR_CHECK_ARG(base && bucket_rows && n >= 1, "fill_row_table: bad arguments");
  hipLaunchKernelGGL(scr::fill_row_table_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(base), n, stride, bucket_rows);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

extern "C" int scr_fill_staged_rows(const scr_bank_desc* bank, int layer, const void* staging,
                                    const void** bucket_rows, hipStream_t stream) {
  int rc = scr::check_bank(bank);
  if (rc) return rc;
  SCR_CHECK_ARG(staging && bucket_rows && bank->rows, "fill_staged_rows: null pointer");
  SCR_CHECK_ARG(layer >= 0 && layer < bank->L, "fill_staged_rows: layer out of range");
  hipLaunchKernelGGL(scr::fill_staged_rows_kernel, dim3((bank->E + 255) / 256), dim3(256), 0, stream,
                     bank->key_to_slot, layer, bank->E, bank->rows, static_cast<const uint8_t*>(staging),
                     bank->record_bytes, bucket_rows);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

extern "C" int scr_host_device_alias(const void* host_ptr, void** dev_ptr) {
  SCR_CHECK_ARG(host_ptr && dev_ptr, "host_device_alias: null pointer");
  SCR_CHECK_HIP(hipHostGetDevicePointer(dev_ptr, const_cast<void*>(host_ptr), 0));
  return SCR_OK;
}
