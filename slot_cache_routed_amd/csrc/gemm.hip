// Grouped SwiGLU expert GEMMs over the active buckets, and the weighted
// top-k combine.
//
// The demand chunk runs the same grouped GEMM over its layer's slots as the
// streamed layer does (FreeToken PR #676, Solution), sized by the routed
// layer's expert count, never the bank's (same page, fourth bullet; Tests).
// Each workgroup owns one (active bucket, N tile) and walks every row of its
// bucket, so each weight tile is read from HBM once per slot rather than once
// per M block (vLLM fork PR #51, the host-view root cause: a consumer that
// re-reads B per M block moved each expert about five times).
//
// MFMA: v_mfma_f32_16x16x32_bf16 (gfx950).  Operand layout per lane l:
//   A (16 x 32): row l % 16, k = 8 * (l / 16) .. + 7
//   B (32 x 16): col l % 16, k = 8 * (l / 16) .. + 7
//   C (16 x 16): col l % 16, rows 4 * (l / 16) .. + 3
// A rows are routes (tokens gathered through sorted_routes), B columns are
// weight rows (output features), K runs along the weight row.
#include "common.h"

#include <math.h>

namespace scr {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kGemmThreads = 256;  // 4 waves, each owns 16 output columns
constexpr int kNTile = 64;         // output columns per workgroup

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ NVFP4 decode
// e2m1 code -> bf16 bits (exact): 0, 0.5, 1, 1.5, 2, 3, 4, 6 with sign in bit 3.
__device__ __forceinline__ unsigned e2m1_bf16_bits(unsigned c) {
  const unsigned m = c & 7u;
  unsigned mag;
  if (m == 0u) mag = 0u;
  else if (m == 1u) mag = 0x3F00u;  // 0.5
  else mag = ((126u + (m >> 1)) << 7) | ((m & 1u) << 6);
  return mag | ((c & 8u) << 12);
}

// e4m3 (OCP E4M3FN) code -> float (finite codes only)
__device__ __forceinline__ float e4m3_to_f32(unsigned c) {
  const unsigned e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0u ? (float)m * 0.001953125f  // m/8 * 2^-6
                      : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// 8 consecutive codes (one uint32) times one block scale, as exact bf16
__device__ __forceinline__ bf16x8 dequant8(unsigned packed, float scale) {
  u16x8 out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned code = (packed >> (4 * i)) & 0xFu;
    const float v = __uint_as_float(e2m1_bf16_bits(code) << 16) * scale;  // exact product
    out[i] = (unsigned short)(__float_as_uint(v) >> 16);                   // exact: truncation
  }
  return __builtin_bit_cast(bf16x8, out);
}

// B fragment loader: 8 consecutive weights of one row starting at column kk
template <int WDT>
struct WRow;

template <>
struct WRow<SCR_W_BF16> {
  const bf16* p;
  __device__ __forceinline__ void init(const uint8_t* tensor, const uint8_t*, int row, int cols) {
    p = reinterpret_cast<const bf16*>(tensor) + (size_t)row * cols;
  }
  __device__ __forceinline__ bf16x8 load(int kk) const {
    return *reinterpret_cast<const bf16x8*>(p + kk);
  }
};

template <>
struct WRow<SCR_W_NVFP4> {
  const uint8_t* q;
  const uint8_t* s;
  __device__ __forceinline__ void init(const uint8_t* tensor, const uint8_t* scales, int row, int cols) {
    q = tensor + (size_t)row * (cols / 2);
    s = scales + (size_t)row * (cols / 16);
  }
  __device__ __forceinline__ bf16x8 load(int kk) const {
    const unsigned packed = *reinterpret_cast<const unsigned*>(q + kk / 2);
    return dequant8(packed, e4m3_to_f32(s[kk / 16]));
  }
};

struct GemmArgs {
  const void* const* bucket_rows;
  scr_record_layout lay;
  const bf16* x;        // [T][H]
  const float* topk_w;  // [R]
  const int32_t* sorted_routes;
  const int32_t* active_buckets;
  const int32_t* active_block_begin;
  const int32_t* n_active;
  bf16* h;              // [h_rows][I]
  float* o;             // [R][H]
  int32_t* flags;       // [R]
  int T, k, R, H, I, B, h_rows;
};

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// gate/up: h[pos][n] = silu(g * G[n] . x) * (g * U[n] . x) for the bucket's rows
template <int WDT, int MT>
__global__ __launch_bounds__(kGemmThreads) void gateup_kernel(GemmArgs a) {
  const int j = blockIdx.y;
  if (j >= *a.n_active) return;
  const int b = a.active_buckets[j];
  const int p0 = a.active_block_begin[j] * a.B, p1 = a.active_block_begin[j + 1] * a.B;
  if (p1 > a.h_rows || p0 >= p1) return;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 15, kgrp = (lane >> 4) * 8;
  const int n = blockIdx.x * kNTile + wave * 16 + col;  // h column of this lane's B fragment
  const uint8_t* rec = static_cast<const uint8_t*>(a.bucket_rows[b]);
  WRow<WDT> wg, wu;
  wg.init(rec + a.lay.w13_off, rec + a.lay.w13_scale_off, n, a.H);
  wu.init(rec + a.lay.w13_off, rec + a.lay.w13_scale_off, a.I + n, a.H);
  const float gs = WDT == SCR_W_NVFP4 ? *reinterpret_cast<const float*>(rec + a.lay.g13_off) : 1.0f;

  for (int m0 = p0; m0 < p1; m0 += MT * 16) {
    const int mt_count = min(MT, (p1 - m0) / 16);
    const bf16* xa[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      xa[mt] = nullptr;
      if (mt < mt_count) {
        const int r = a.sorted_routes[m0 + mt * 16 + col];
        if (r >= 0 && r < a.R) xa[mt] = a.x + (size_t)(r / a.k) * a.H + kgrp;
      }
    }
    f32x4 accg[MT], accu[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bf16x8 zero = {};
    for (int k0 = 0; k0 < a.H; k0 += 32) {
      const bf16x8 bg = wg.load(k0 + kgrp);
      const bf16x8 bu = wu.load(k0 + kgrp);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < mt_count) {
          const bf16x8 av = xa[mt] ? *reinterpret_cast<const bf16x8*>(xa[mt] + k0) : zero;
          accg[mt] = mfma16(av, bg, accg[mt]);
          accu[mt] = mfma16(av, bu, accu[mt]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = m0 + mt * 16 + (lane >> 4) * 4 + i;
          const float hv = silu_mul(gs * accg[mt][i], gs * accu[mt][i]);
          a.h[(size_t)pos * a.I + n] = static_cast<bf16>(hv);
        }
      }
    }
  }
}

// down: o[r][n] = w_r * (g * W2[n] . h[pos]) for the bucket's rows
template <int WDT, int MT>
__global__ __launch_bounds__(kGemmThreads) void down_kernel(GemmArgs a) {
  const int j = blockIdx.y;
  if (j >= *a.n_active) return;
  const int b = a.active_buckets[j];
  const int p0 = a.active_block_begin[j] * a.B, p1 = a.active_block_begin[j + 1] * a.B;
  if (p1 > a.h_rows || p0 >= p1) return;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 15, kgrp = (lane >> 4) * 8;
  const int n = blockIdx.x * kNTile + wave * 16 + col;  // output feature of this lane's B fragment
  const uint8_t* rec = static_cast<const uint8_t*>(a.bucket_rows[b]);
  WRow<WDT> w2;
  w2.init(rec + a.lay.w2_off, rec + a.lay.w2_scale_off, n, a.I);
  const float gs = WDT == SCR_W_NVFP4 ? *reinterpret_cast<const float*>(rec + a.lay.g2_off) : 1.0f;

  for (int m0 = p0; m0 < p1; m0 += MT * 16) {
    const int mt_count = min(MT, (p1 - m0) / 16);
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < a.I; k0 += 32) {
      const bf16x8 bw = w2.load(k0 + kgrp);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < mt_count) {
          const bf16x8 av =
              *reinterpret_cast<const bf16x8*>(a.h + (size_t)(m0 + mt * 16 + col) * a.I + k0 + kgrp);
          acc[mt] = mfma16(av, bw, acc[mt]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = m0 + mt * 16 + (lane >> 4) * 4 + i;
          const int r = a.sorted_routes[pos];
          if (r >= 0 && r < a.R) {
            a.o[(size_t)r * a.H + n] = a.topk_w[r] * (gs * acc[mt][i]);
            if (n == 0) a.flags[r] = 1;
          }
        }
      }
    }
  }
}

// clears the per-route written flags and reports the layer's activation scale
__global__ __launch_bounds__(256) void prologue_kernel(int32_t* __restrict__ flags, int R,
                                                       const float* __restrict__ input_scale, int E,
                                                       float* __restrict__ a_scale_out) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < R; r += gridDim.x * blockDim.x) flags[r] = 0;
  if (a_scale_out && blockIdx.x == 0) {
    __shared__ float red[256];
    float m = -INFINITY;
    for (int e = threadIdx.x; e < E; e += blockDim.x) m = fmaxf(m, input_scale[e]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
      __syncthreads();
    }
    if (threadIdx.x == 0) *a_scale_out = red[0];
  }
}

// y[t][c] = sum_j o[t*k + j][c] in rank order (unwritten routes count as zero)
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ flags, int T, int k,
                                                      int H, void* __restrict__ y) {
  const int h4 = H / 4;
  const size_t total = (size_t)T * h4;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / h4), c4 = (int)(i % h4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int r = t * k + j;
      if (!flags[r]) continue;
      const float4 v = reinterpret_cast<const float4*>(o + (size_t)r * H)[c4];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    if (BF16_OUT) {
      bf16* yp = static_cast<bf16*>(y) + (size_t)t * H + 4 * c4;
      yp[0] = static_cast<bf16>(acc.x);
      yp[1] = static_cast<bf16>(acc.y);
      yp[2] = static_cast<bf16>(acc.z);
      yp[3] = static_cast<bf16>(acc.w);
    } else {
      reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * H)[c4] = acc;
    }
  }
}

struct WsLayout {
  size_t h_off, o_off, flags_off, bytes;
  int h_rows;
};

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

static WsLayout ws_layout(int T, int k, int E_layer, int H, int I, int B) {
  WsLayout w;
  const long long R = (long long)T * k;
  const long long m = R < E_layer ? R : E_layer;
  long long rows = R + m * (B - 1);
  rows = (rows + B - 1) / B * B;
  w.h_rows = (int)rows;
  w.h_off = 0;
  w.o_off = align256(w.h_off + (size_t)rows * I * sizeof(uint16_t));
  w.flags_off = align256(w.o_off + (size_t)R * H * sizeof(float));
  w.bytes = align256(w.flags_off + (size_t)R * sizeof(int32_t));
  return w;
}

template <int WDT, int MT>
static int launch_gemms(const GemmArgs& a, int max_active, hipEvent_t* marks, hipStream_t s) {
  dim3 gu(a.I / kNTile, max_active), dn(a.H / kNTile, max_active);
  hipLaunchKernelGGL((gateup_kernel<WDT, MT>), gu, dim3(kGemmThreads), 0, s, a);
  SCR_CHECK_LAUNCH();
  if (marks && marks[2]) SCR_CHECK_HIP(hipEventRecord(marks[2], s));
  hipLaunchKernelGGL((down_kernel<WDT, MT>), dn, dim3(kGemmThreads), 0, s, a);
  SCR_CHECK_LAUNCH();
  if (marks && marks[3]) SCR_CHECK_HIP(hipEventRecord(marks[3], s));
  return SCR_OK;
}

}  // namespace scr

extern "C" int scr_tile_config(int T, int k, int E_layer, int wdtype, scr_tile_cfg* cfg) {
  SCR_CHECK_ARG(cfg != nullptr, "tile_config: cfg is null");
  SCR_CHECK_ARG(T >= 0 && k >= 1 && E_layer >= 1, "tile_config: bad T, k or E");
  SCR_CHECK_ARG(wdtype == SCR_W_BF16 || wdtype == SCR_W_NVFP4, "tile_config: unknown wdtype");
  // rows per expert of the routed layer (never of the bank)
  const long long per_expert = ((long long)T * k + E_layer - 1) / E_layer;
  cfg->block_m = 16;
  cfg->m_chunk = per_expert <= 32 ? 64 : 128;
  cfg->n_tile_gu = scr::kNTile;
  cfg->n_tile_dn = scr::kNTile;
  cfg->wdtype = wdtype;
  return SCR_OK;
}

extern "C" int scr_moe_workspace(int T, int k, int E_layer, int H, int I, const scr_tile_cfg* cfg, size_t* bytes) {
  SCR_CHECK_ARG(cfg && bytes && T >= 0 && k >= 1 && E_layer >= 1 && H >= 1 && I >= 1,
                "moe_workspace: bad arguments");
  *bytes = scr::ws_layout(T, k, E_layer, H, I, cfg->block_m).bytes;
  return SCR_OK;
}

extern "C" int scr_grouped_moe_forward(const scr_routed_experts* view, const void* x, int T,
                                       const float* topk_w, const int32_t* sorted_routes,
                                       const int32_t* active_buckets, const int32_t* active_block_begin,
                                       const int32_t* n_active, void* y, int y_dtype, void* ws,
                                       size_t ws_bytes, scr_tile_cfg* cfg_out, float* a_scale_out,
                                       hipEvent_t* marks, hipStream_t stream) {
  SCR_CHECK_ARG(view != nullptr, "forward: view is null");
  const int E = view->num_experts, k = view->k, H = view->H, I = view->I;
  SCR_CHECK_ARG(E >= 1 && k >= 1 && k <= E && k <= SCR_MAX_TOPK, "forward: bad num_experts or k");
  SCR_CHECK_ARG(H >= 64 && H % 64 == 0 && H <= 16384, "forward: H must be a multiple of 64 in [64, 16384]");
  SCR_CHECK_ARG(I >= 64 && I % 64 == 0 && I <= 16384, "forward: I must be a multiple of 64 in [64, 16384]");
  SCR_CHECK_ARG(view->num_buckets >= 1 && view->bucket_rows && view->input_scale, "forward: bad view");
  SCR_CHECK_ARG(view->wdtype == SCR_W_BF16 || view->wdtype == SCR_W_NVFP4, "forward: unknown wdtype");
  SCR_CHECK_ARG(y_dtype == SCR_Y_F32 || y_dtype == SCR_Y_BF16, "forward: unknown y dtype");
  SCR_CHECK_ARG(T >= 0 && (long long)T * k < (1ll << 30), "forward: T out of range");
  if (T == 0) return SCR_OK;
  SCR_CHECK_ARG(x && topk_w && sorted_routes && active_buckets && active_block_begin && n_active && y && ws,
                "forward: null pointer");
  scr_tile_cfg cfg;
  int rc = scr_tile_config(T, k, E, view->wdtype, &cfg);
  if (rc) return rc;
  if (cfg_out) *cfg_out = cfg;
  scr_record_layout lay;
  rc = scr_record_layout_of(view->wdtype, H, I, &lay);
  if (rc) return rc;
  const scr::WsLayout wl = scr::ws_layout(T, k, E, H, I, cfg.block_m);
  SCR_CHECK_ARG(ws_bytes >= wl.bytes, "forward: workspace of %zu bytes, %zu needed", ws_bytes, wl.bytes);

  const int R = T * k;
  scr::GemmArgs a;
  a.bucket_rows = view->bucket_rows;
  a.lay = lay;
  a.x = static_cast<const scr::bf16*>(x);
  a.topk_w = topk_w;
  a.sorted_routes = sorted_routes;
  a.active_buckets = active_buckets;
  a.active_block_begin = active_block_begin;
  a.n_active = n_active;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  a.h = reinterpret_cast<scr::bf16*>(wsb + wl.h_off);
  a.o = reinterpret_cast<float*>(wsb + wl.o_off);
  a.flags = reinterpret_cast<int32_t*>(wsb + wl.flags_off);
  a.T = T;
  a.k = k;
  a.R = R;
  a.H = H;
  a.I = I;
  a.B = cfg.block_m;
  a.h_rows = wl.h_rows;

  if (marks && marks[0]) SCR_CHECK_HIP(hipEventRecord(marks[0], stream));
  int pgrid = (R + 255) / 256;
  if (pgrid > 256) pgrid = 256;
  hipLaunchKernelGGL(scr::prologue_kernel, dim3(pgrid), dim3(256), 0, stream, a.flags, R, view->input_scale, E,
                     a_scale_out);
  SCR_CHECK_LAUNCH();
  if (marks && marks[1]) SCR_CHECK_HIP(hipEventRecord(marks[1], stream));

  // the grid covers at most min(R, E_layer) active buckets: a layer size
  const int max_active = R < E ? R : E;
  if (view->wdtype == SCR_W_BF16) {
    rc = cfg.m_chunk == 64 ? scr::launch_gemms<SCR_W_BF16, 4>(a, max_active, marks, stream)
                           : scr::launch_gemms<SCR_W_BF16, 8>(a, max_active, marks, stream);
  } else {
    rc = cfg.m_chunk == 64 ? scr::launch_gemms<SCR_W_NVFP4, 4>(a, max_active, marks, stream)
                           : scr::launch_gemms<SCR_W_NVFP4, 8>(a, max_active, marks, stream);
  }
  if (rc) return rc;

  const size_t total = (size_t)T * (H / 4);
  int cgrid = (int)((total + 255) / 256);
  if (cgrid > 4096) cgrid = 4096;
  if (y_dtype == SCR_Y_BF16)
    hipLaunchKernelGGL(scr::combine_kernel<true>, dim3(cgrid), dim3(256), 0, stream, a.o, a.flags, T, k, H, y);
  else
    hipLaunchKernelGGL(scr::combine_kernel<false>, dim3(cgrid), dim3(256), 0, stream, a.o, a.flags, T, k, H, y);
  SCR_CHECK_LAUNCH();
  if (marks && marks[4]) SCR_CHECK_HIP(hipEventRecord(marks[4], stream));
  return SCR_OK;
}
