// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdarg.h>

#include "../../include/scr.h"

namespace scr {

// thread-local text of the last error returned by an entry point
void set_error(const char* fmt, ...);

#define SCR_CHECK_ARG(cond, ...)            \
  do {                                      \
    if (!(cond)) {                          \
      ::scr::set_error(__VA_ARGS__);        \
      return SCR_EINVAL;                    \
    }                                       \
  } while (0)

#define SCR_CHECK_HIP(expr)                                                        \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess) {                                                        \
      ::scr::set_error("%s: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__,   \
                       __LINE__);                                                  \
      return SCR_EHIP;                                                             \
    }                                                                              \
  } while (0)

// checks the launch that was just enqueued
#define SCR_CHECK_LAUNCH() SCR_CHECK_HIP(hipGetLastError())

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Inclusive prefix sum of one int per lane over the wave by DPP moves: row
// shifts of 1, 2, 4 and 8 lanes sum each 16-lane row (a lane whose source
// falls outside its row adds 0), then lane 15's total joins rows 1 and 3 and
// lane 31's total rows 2 and 3.  Every lane of the wave must call it.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

}  // namespace scr
