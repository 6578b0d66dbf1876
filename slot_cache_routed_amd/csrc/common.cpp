// Error text and small host-side entry points of libscr.
#include "common.h"

#include <string.h>

namespace scr {
static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
}  // namespace scr

extern "C" const char* scr_last_error(void) { return scr::g_err; }

extern "C" const char* scr_version(void) { return "scr 0.1 gfx950"; }

extern "C" int scr_prefill_on_demand(int T, int threshold) { return threshold > 0 && T > 0 && T <= threshold; }

extern "C" int scr_demand_capacity_ok(int T, int k, int E, int S, int half) {
  long long need = (long long)T * k;
  if (need > E) need = E;
  long long cap = half ? S / 2 : S;
  return need <= cap;
}

extern "C" int scr_record_layout_of(int wdtype, int H, int I, scr_record_layout* out) {
  SCR_CHECK_ARG(out != nullptr, "record_layout: out is null");
  SCR_CHECK_ARG(H >= 128 && I >= 128 && H % 128 == 0 && I % 128 == 0,
                "record_layout: H and I must be positive multiples of 128 (tile-major records)");
  memset(out, 0, sizeof(*out));
  const uint64_t h = (uint64_t)H, i = (uint64_t)I;
  if (wdtype == SCR_W_BF16) {
    out->w13_off = 0;
    out->w2_off = 2 * i * h * 2;
    out->record_bytes = out->w2_off + h * i * 2;
    out->w13_scale_off = out->w2_scale_off = out->g13_off = out->g2_off = 0;
    SCR_CHECK_ARG(out->record_bytes % 16 == 0, "record_layout: bf16 record not 16-byte sized");
    return SCR_OK;
  }
  if (wdtype == SCR_W_NVFP4 || wdtype == SCR_W_NVFP4_A4) {
    out->w13_off = 0;
    out->w13_scale_off = out->w13_off + 2 * i * h / 2;
    out->w2_off = out->w13_scale_off + 2 * i * h / 16;
    out->w2_scale_off = out->w2_off + h * i / 2;
    out->g13_off = out->w2_scale_off + h * i / 16;
    out->g2_off = out->g13_off + 4;
    out->record_bytes = (out->g2_off + 4 + 255) / 256 * 256;
    return SCR_OK;
  }
  if (wdtype == SCR_W_FP8) {
    out->w13_off = 0;
    out->w2_off = 2 * i * h;
    out->g13_off = out->w2_off + h * i;
    out->g2_off = out->g13_off + 4;
    out->w13_scale_off = out->w2_scale_off = 0;
    out->record_bytes = (out->g2_off + 4 + 255) / 256 * 256;
    return SCR_OK;
  }
  if (wdtype == SCR_W_MXFP4 || wdtype == SCR_W_MXFP4_A8) {
    out->w13_off = 0;
    out->w13_scale_off = out->w13_off + 2 * i * h / 2;
    out->w2_off = out->w13_scale_off + 2 * i * h / 32;
    out->w2_scale_off = out->w2_off + h * i / 2;
    out->g13_off = out->g2_off = 0;  // no global scales
    out->record_bytes = (out->w2_scale_off + h * i / 32 + 255) / 256 * 256;
    return SCR_OK;
  }
  scr::set_error("record_layout: unknown wdtype %d", wdtype);
  return SCR_ENOTSUP;
}

extern "C" int scr_timer_create(hipEvent_t* ev) {
  SCR_CHECK_ARG(ev != nullptr, "timer_create: null pointer");
  SCR_CHECK_HIP(hipEventCreateWithFlags(ev, hipEventDisableSystemFence));
  return SCR_OK;
}

extern "C" int scr_timer_record(hipEvent_t ev, hipStream_t stream) {
  SCR_CHECK_ARG(ev != nullptr, "timer_record: null event");
  SCR_CHECK_HIP(hipEventRecord(ev, stream));
  return SCR_OK;
}

extern "C" int scr_timer_elapsed_ms(hipEvent_t start, hipEvent_t stop, float* ms) {
  SCR_CHECK_ARG(start && stop && ms, "timer_elapsed: null argument");
  SCR_CHECK_HIP(hipEventSynchronize(stop));
  SCR_CHECK_HIP(hipEventElapsedTime(ms, start, stop));
  return SCR_OK;
}

extern "C" int scr_timer_destroy(hipEvent_t ev) {
  SCR_CHECK_ARG(ev != nullptr, "timer_destroy: null event");
  SCR_CHECK_HIP(hipEventDestroy(ev));
  return SCR_OK;
}
