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

}  // namespace scr
