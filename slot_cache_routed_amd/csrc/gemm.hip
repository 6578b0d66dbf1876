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

constexpr int kGemmThreads = 256;  // 4 waves per workgroup

// Load through a global-address-space pointer.  Pointers read from tables
// (bucket_rows) are generic; a generic load compiles to a FLAT instruction,
// which also counts on the LDS counter, so every wait for an LDS read would
// wait for the in-flight weight stream as well.
template <typename T>
__device__ __forceinline__ T ldg(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
// the same as a nontemporal (streaming) load
template <typename T>
__device__ __forceinline__ T ldg_nt(const void* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)(p));
}
template <bool NT, typename T>
__device__ __forceinline__ T ldg_w(const void* p) {
  if constexpr (NT) return ldg_nt<T>(p);
  else return ldg<T>(p);
}

// cache policy of the buffer loads of weights: nontemporal (each weight byte
// is read once per pass; keeping it out of the caches' way measured faster)
constexpr int kNonTemporal = 2;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// the same product on fp16 operands (carried in the same 16-byte registers)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16_f16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}

// ------------------------------------------------------------ NVFP4 decode
// e4m3 (OCP E4M3FN) code -> float (finite codes only), without branches:
// |v| = (m + 8 [e > 0]) * 2^(max(e, 1) - 10), exact in fp32 (the subnormal
// case e = 0 is m/8 * 2^-6)
__device__ __forceinline__ float e4m3_to_f32(unsigned c) {
  const unsigned e = (c >> 3) & 0xFu, m = c & 7u;
  const unsigned mant = m | (min(e, 1u) << 3);
  const float mag = __builtin_amdgcn_ldexpf((float)mant, (int)max(e, 1u) - 10);
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// ------------------------------------------- activation codes (A8 / A4)
// OCP E4M3FN code of v, rounded to nearest even, saturated to +-448 (the
// hardware conversion rounds to nearest even; the clamp makes it saturate)
__device__ __forceinline__ unsigned e4m3_code_sat(float v) {
  const float c = fminf(fmaxf(v, -448.0f), 448.0f);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}
// NVFP4 activation block under the layer scale s: the block scale code of a
// block whose largest magnitude is amax (fp32 product and IEEE division)
__device__ __forceinline__ unsigned nvfp4_block_code(float amax, float s) {
  return e4m3_code_sat(amax / (6.0f * s));
}
// the reciprocal an NVFP4 block's elements are multiplied by: 1 / (block
// scale value * layer scale), an IEEE division once per block (0 for a zero
// block scale, whose elements all get zero codes)
__device__ __forceinline__ float nvfp4_block_rcp(float bv, float s) {
  return bv > 0.0f ? 1.0f / (bv * s) : 0.0f;
}
// E2M1 codes of two values times their block's reciprocal, v0 in the low
// nibble: the magnitudes from the gfx950 conversion (nearest of 0, 0.5, 1,
// 1.5, 2, 3, 4, 6, ties to the even code, saturated to 6: the rule, checked
// on every midpoint and its neighbours), the sign bit from the input (set
// for every negative v, also where the magnitude rounds to 0)
__device__ __forceinline__ unsigned nvfp4_pair_codes(float v0, float v1, float rcp) {
  const unsigned m = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, fabsf(v0 * rcp), fabsf(v1 * rcp), 1.0f, 0) & 0xFFu;
  return m | (v0 < 0.0f ? 0x8u : 0u) | (v1 < 0.0f ? 0x80u : 0u);
}
// the pair's decoded values without the layer scale, e2m1 * block, as two
// fp16 (exact: at most 5 significant bits, magnitude in [2^-10, 2688])
__device__ __forceinline__ unsigned nvfp4_pair_f16(unsigned codes, float bv) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  const _Float16 b = (_Float16)bv;
  const h2 bb = {b, b};
  return __builtin_bit_cast(unsigned, e * bb);
}

// Weight formats: bytes of one tile-block (16 rows x 128 columns) of codes
// and of its block scales, whether the record carries a per-tensor scale,
// and the few-rows kernels' per-route row type: fp32 for bf16 weights (their
// output tolerance is tighter); for the narrow formats fp16 bits scaled per 32
// columns (half the bytes of fp32, with 11 significant bits where bf16 rows
// kept 8; see scaled_row16).  The wide kernels write the fp16 rows for every
// format (rows_f32).
template <int WDT>
struct WFmt;
template <>
struct WFmt<SCR_W_BF16> {
  static constexpr int tile = 4096, stile = 0;
  static constexpr bool gscale = false;
  typedef float row_t;
};
template <>
struct WFmt<SCR_W_NVFP4> {
  static constexpr int tile = 1024, stile = 128;
  static constexpr bool gscale = true;
  typedef uint16_t row_t;
};
template <>
struct WFmt<SCR_W_FP8> {
  static constexpr int tile = 2048, stile = 0;
  static constexpr bool gscale = true;
  typedef uint16_t row_t;
};
template <>
struct WFmt<SCR_W_MXFP4> {
  static constexpr int tile = 1024, stile = 64;
  static constexpr bool gscale = false;
  typedef uint16_t row_t;
};
// W4A4 reads NVFP4 records
template <>
struct WFmt<SCR_W_NVFP4_A4> : WFmt<SCR_W_NVFP4> {};
template <int WDT>
struct RowT {
  typedef typename WFmt<WDT>::row_t type;
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
  void* o;              // [R][H] per-route weighted expert outputs (fp32 or fp16 rows: rows_f32)
  int8_t* oe;           // narrow formats: [R][H / kRowGroup] the rows' group exponents
  int32_t* flags;       // [R]
  const float* input_scale;       // [E] the layer's scales of the gate/up input
  const float* down_input_scale;  // [E] the layer's scales of the down input, or null
  float* a_scale_out;             // nullable, device [2]
  // A8 / A4 formats: the layer's activation scales (max of each array),
  // written by the activation quantisation before the GEMMs
  const float* act_scale;  // [2]
  // W4A8 only: E4M3 codes of x / a1 and of h / a2
  const uint8_t* xq;  // [T][H]
  uint8_t* hq;        // [h_rows][I]
  // NVFP4 wide gate/up: x as fp16, row t scaled by 2^xe[t]; W4A4: the decoded
  // NVFP4 values of x (xe unused)
  const uint16_t* x16;  // [T][H]
  const int32_t* xe;    // [T]
  int T, k, R, H, I, B, h_rows, E;
};

// maxima of the layer's two scale arrays (n >= 1 each; s2 may be null, its
// maximum then 0) over one wave, every lane getting them.  Loads go out in
// rounds of 8 per lane per array, clamped to the last entry (a repeat cannot
// change a maximum), so a round costs one memory latency.
__device__ __forceinline__ void wave_scale_max2(const float* s1, const float* s2, int n, int lane, float& m1,
                                                float& m2) {
  float a = -INFINITY, b = s2 ? -INFINITY : 0.0f;
  for (int e0 = 0; e0 < n; e0 += 64 * 8) {
    float v[8], w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = min(e0 + 64 * u + lane, n - 1);
      v[u] = s1[e];
      w[u] = s2 ? s2[e] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a = fmaxf(a, v[u]);
      b = fmaxf(b, w[u]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a = fmaxf(a, __shfl_xor(a, off, 64));
    b = fmaxf(b, __shfl_xor(b, off, 64));
  }
  m1 = a;
  m2 = b;
}

// Work that must precede the down GEMM, done by the gate/up workgroups before
// anything else (so that it costs no launch of its own): clear the per-route
// written flags that down sets, and report the layer's activation scales
// (the max of each array of its input scales) from the first wave of
// workgroup 0.  (The A8/A4 formats report them from their quantisation.)
__device__ __forceinline__ void gateup_prologue(const GemmArgs& a) {
  const int nthreads = gridDim.x * blockDim.x;
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < a.R; r += nthreads) a.flags[r] = 0;
  if (a.a_scale_out && !a.act_scale && blockIdx.x == 0 && threadIdx.x < 64) {
    float m1, m2;
    wave_scale_max2(a.input_scale, a.down_input_scale, a.E, threadIdx.x, m1, m2);
    if (threadIdx.x == 0) {
      a.a_scale_out[0] = m1;
      a.a_scale_out[1] = m2;
    }
  }
}

// silu(g) * u with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// ------------------------------------------------------------ grouped GEMM
//
// One workgroup = one (active bucket, N tile, pass slice).  A bucket's rows
// are walked in passes of up to MT*16 rows (a workgroup takes every pslices-th
// pass); per pass the K dimension is consumed in blocks of 128.  Activation
// rows (x, or for NVFP4 its fp16 copy, gathered through sorted_routes for
// gate/up; contiguous h rows for down) are staged once per block in LDS and
// shared by the 4 waves; each wave streams its own weight rows straight into
// registers ahead of use and decodes the narrow formats there, so every
// weight byte is fetched and decoded once per pass.
//
// K order inside a 128-wide block (A and B use the same one, so the sum is the
// full dot product; it is fixed, so every path that runs this kernel gets the
// same bits).  MFMA step s (0..3) gives lane group g = lane / 16 eight columns:
//   bf16 : 32 s + 8 g   (the natural layout: one load = 64 B of a row)
//   NVFP4: 32 g + 8 s   (lane group g owns 32 consecutive codes = 16 B and
//                        their two e4m3 scales, so one load covers them;
//                        MXFP4 and FP8 the same: 16 B of codes and one e8m0
//                        scale, or 32 B of fp8 codes in two loads)
constexpr int kKB = 128;               // K block
constexpr int kAStride = kKB + 8;      // LDS row stride (bf16): conflict-free b128 reads

template <int WDT>
__device__ __forceinline__ int kcol(int g, int s) {
  return WDT == SCR_W_BF16 ? 32 * s + 8 * g : 32 * g + 8 * s;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// exact codes (unit scale), then the full e4m3 scale in fp32; the product has
// at most 5 significant bits, so the bf16 conversion is exact
__device__ __forceinline__ unsigned dq_pair(f32x2 v, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {static_cast<__bf16>(v[0] * scale), static_cast<__bf16>(v[1] * scale)};
  return __builtin_bit_cast(unsigned, r);
}

// two floats as a bf16 pair (round to nearest even), a in the low half.  The
// empty asm keeps the compiler from splitting the pair back into two single
// conversions when the halves are stored separately.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  unsigned p = __builtin_bit_cast(unsigned, r);
  asm("" : "+v"(p));
  return p;
}

// Per-route output rows of the narrow formats: fp16 values times 2^e, one e
// per kRowGroup columns of a row (an int8 beside the row).  e comes from the
// exponent field f of the group's largest magnitude M: e = 141 - f, capped at
// 127, puts a normal M in [2^14, 2^15), so every value keeps 11 significant
// bits relative to the largest of its group.  e lies in [-114, 127]: a zero
// or tiny group (M < 2^-113) keeps 127, one holding an infinity -114 (inf and
// NaN values stay what they are).  Magnitudes are compared as their fp32 bit
// patterns, which order non-negative floats as unsigned integers.
constexpr int kRowGroup = 32;
__device__ __forceinline__ int row_group_exp(unsigned mbits) { return min(141 - (int)(mbits >> 23), 127); }
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
// the largest m over the 16 lanes of a lane group (lanes 16 g .. 16 g + 15,
// one DPP row): rotations of the row by 1, 2, 4 and 8 lanes leave the row's
// maximum in every lane (DPP moves, no LDS round trip per step)
__device__ __forceinline__ unsigned group16_max(unsigned m) {
  m = max(m, dpp_u32<0x121>(m));  // row_ror:1
  m = max(m, dpp_u32<0x122>(m));  // row_ror:2
  m = max(m, dpp_u32<0x124>(m));  // row_ror:4
  m = max(m, dpp_u32<0x128>(m));  // row_ror:8
  return m;
}
// the largest m over an aligned quad of lanes (two quad_perm DPP steps)
__device__ __forceinline__ unsigned quad_max(unsigned m) {
  m = max(m, dpp_u32<0xB1>(m));  // quad_perm [1, 0, 3, 2]
  m = max(m, dpp_u32<0x4E>(m));  // quad_perm [2, 3, 0, 1]
  return m;
}
// v * 2^e as fp16 bits (nearest even)
__device__ __forceinline__ uint16_t scaled_row16(float v, float scale) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v * scale));
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// a and b times 2^e as one packed fp16 pair (a low)
__device__ __forceinline__ unsigned scaled_pair16(float a, float b, float scale) {
  const f16x2_t h = {static_cast<_Float16>(a * scale), static_cast<_Float16>(b * scale)};
  return __builtin_bit_cast(unsigned, h);
}

// A wave's 16 x OC block of down output (fp32, row-major in LDS) written as
// fp16 rows scaled per 32 columns: each lane takes 8 consecutive values of a
// row, so four neighbouring lanes hold one group and share its largest
// magnitude over two quad DPP steps; the group's first lane writes the
// exponent.  routes[r] is the route of tile row r (or -1 for padding);
// c_base the wave's first output column.
template <int OC>
__device__ __forceinline__ void store_rows_f16(const float* sf, const int* routes, int lane, uint16_t* o, int8_t* oe,
                                               int32_t* flags, int H, int c_base, bool set_flag) {
  static_assert(OC % kRowGroup == 0 && kRowGroup == 32, "four 8-value pieces per group");
  constexpr int PPR = OC / 8;  // 8-value pieces per row
  static_assert((16 * PPR) % 64 == 0, "whole rounds of 64 lanes");
#pragma unroll
  for (int rd = 0; rd < 16 * PPR / 64; ++rd) {
    const int q = rd * 64 + lane, rr = q / PPR, pc = q % PPR;
    const float4 a0 = *reinterpret_cast<const float4*>(sf + rr * OC + pc * 8);
    const float4 a1 = *reinterpret_cast<const float4*>(sf + rr * OC + pc * 8 + 4);
    const float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(v[c]));
    const int e = row_group_exp(quad_max(__float_as_uint(m)));
    const float sc = __builtin_ldexpf(1.0f, e);
    u32x4 out;
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = scaled_pair16(v[2 * c], v[2 * c + 1], sc);
    const int rt = routes[rr];
    if (rt >= 0) {
      const int c0 = c_base + pc * 8;
      *reinterpret_cast<u32x4*>(o + (size_t)rt * H + c0) = out;
      if ((pc & 3) == 0) oe[(size_t)rt * (H / kRowGroup) + c0 / kRowGroup] = (int8_t)e;
      if (set_flag && pc == 0) flags[rt] = 1;
    }
  }
}

// 8 e2m1 codes (one dword, low nibble first) times a block scale, as bf16
__device__ __forceinline__ bf16x8 dequant8_hw(unsigned packed, float scale) {
  u32x4 out;
  out[0] = dq_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 0), scale);
  out[1] = dq_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 1), scale);
  out[2] = dq_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 2), scale);
  out[3] = dq_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, 3), scale);
  return __builtin_bit_cast(bf16x8, out);
}

// Weight fragments of one wave for one K block: NT tiles x 4 MFMA steps.
// Records are tile-major (see scr.h): tile-block (t, kb) of a tensor holds its
// 16 rows x 128 columns in the order the lanes load them, so each load below
// is one contiguous 1 KB (codes, bf16 steps) or 128 B (scales) range.
// tile[i] points at tile-block (t_i, 0); consecutive K blocks follow it.
template <int WDT, int NT>
struct BFrag;

template <int NT>
struct BFrag<SCR_W_BF16, NT> {
  u32x4 raw[NT][4];
  template <bool STREAM = false>
  __device__ __forceinline__ void load(const uint8_t* const* tile, const uint8_t* const*, int kb, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        raw[t][st] = ldg_w<STREAM, u32x4>(tile[t] + (size_t)kb * 4096 + st * 1024 + lane * 16);
  }
  // through a buffer resource: the wave-uniform tile offsets go in scalar
  // registers, the per-lane part is the constant lane * 16
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, const int* toff, const int*, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        raw[t][st] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, toff[t] + st * 1024, kNonTemporal);
  }
  __device__ __forceinline__ bf16x8 get(int t, int st) const { return __builtin_bit_cast(bf16x8, raw[t][st]); }
  __device__ __forceinline__ bf16x8 get_hw(int t, int st) const { return get(t, st); }
};

template <int NT>
struct BFrag<SCR_W_NVFP4, NT> {
  u32x4 codes[NT];  // 32 codes: step s uses dword s
  unsigned sc[NT];  // two scale codes: low byte for codes 0..15, next for 16..31
  template <bool STREAM = false>
  __device__ __forceinline__ void load(const uint8_t* const* tile, const uint8_t* const* stile, int kb, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      codes[t] = ldg_w<STREAM, u32x4>(tile[t] + (size_t)kb * 1024 + lane * 16);
      sc[t] = ldg_w<STREAM, unsigned short>(stile[t] + (size_t)kb * 128 + lane * 2);
    }
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, const int* toff, const int* soff, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      codes[t] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, toff[t], kNonTemporal);
      sc[t] = __builtin_amdgcn_raw_buffer_load_b16(r, lane * 2, soff[t], kNonTemporal);
    }
  }
  __device__ __forceinline__ bf16x8 get(int t, int st) const {
    return dequant8_hw(codes[t][st], e4m3_to_f32((sc[t] >> (8 * (st >> 1))) & 0xFFu));
  }
  // the same with the scale decoded by the hardware OCP E4M3 conversion
  __device__ __forceinline__ bf16x8 get_hw(int t, int st) const {
    const float scale = (st >> 1) ? __builtin_amdgcn_cvt_f32_fp8((int)sc[t], 1) : __builtin_amdgcn_cvt_f32_fp8((int)sc[t], 0);
    return dequant8_hw(codes[t][st], scale);
  }
  // as fp16: e2m1 codes and the e4m3 scale both convert exactly, and their
  // product (at most 6 significant bits, magnitude in [2^-10, 2688]) is exact
  // in fp16, so one packed fp16 multiply per pair finishes the decode
  __device__ __forceinline__ bf16x8 get_f16(int t, int st) const {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)sc[t], 1.0f, false);
    const _Float16 sv = (st >> 1) ? s2[1] : s2[0];
    const h2 sa = {sv, sv};
    const unsigned c = codes[t][st];
    u32x4 o;
    o[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * sa);
    o[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * sa);
    o[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * sa);
    o[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * sa);
    return __builtin_bit_cast(bf16x8, o);
  }
};

template <int NT>
struct BFrag<SCR_W_FP8, NT> {
  u32x4 raw[NT][2];  // 32 codes: columns 0..15 of the lane's group, then 16..31
  template <bool STREAM = false>
  __device__ __forceinline__ void load(const uint8_t* const* tile, const uint8_t* const*, int kb, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      raw[t][0] = ldg_w<STREAM, u32x4>(tile[t] + (size_t)kb * 2048 + lane * 16);
      raw[t][1] = ldg_w<STREAM, u32x4>(tile[t] + (size_t)kb * 2048 + 1024 + lane * 16);
    }
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, const int* toff, const int*, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      raw[t][0] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, toff[t], kNonTemporal);
      raw[t][1] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, toff[t] + 1024, kNonTemporal);
    }
  }
  // step s: codes 8 s .. 8 s + 7, exact in bf16 (the tensor scale is applied
  // to the accumulator)
  __device__ __forceinline__ bf16x8 get(int t, int st) const {
    const unsigned d0 = raw[t][st >> 1][2 * (st & 1)], d1 = raw[t][st >> 1][2 * (st & 1) + 1];
    u32x4 out;
    out[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
    out[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
    out[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
    out[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
    return __builtin_bit_cast(bf16x8, out);
  }
  __device__ __forceinline__ bf16x8 get_hw(int t, int st) const { return get(t, st); }
};

template <int NT>
struct BFrag<SCR_W_MXFP4, NT> {
  u32x4 codes[NT];  // 32 codes: step s uses dword s
  unsigned sc[NT];  // the group's e8m0 scale code
  template <bool STREAM = false>
  __device__ __forceinline__ void load(const uint8_t* const* tile, const uint8_t* const* stile, int kb, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      codes[t] = ldg_w<STREAM, u32x4>(tile[t] + (size_t)kb * 1024 + lane * 16);
      sc[t] = ldg_w<STREAM, uint8_t>(stile[t] + (size_t)kb * 64 + lane);
    }
  }
  __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, const int* toff, const int* soff, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      codes[t] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, toff[t], kNonTemporal);
      sc[t] = __builtin_amdgcn_raw_buffer_load_b8(r, lane, soff[t], kNonTemporal);
    }
  }
  // the conversion's scale operand contributes its exponent field only, which
  // is exactly the e8m0 code: value = e2m1 * 2^(code - 127), rounded to bf16
  // (exact for scale codes 2..252)
  __device__ __forceinline__ bf16x8 get(int t, int st) const {
    const float scale = __builtin_bit_cast(float, (sc[t] & 0xFFu) << 23);
    const unsigned c = codes[t][st];
    u32x4 out;
    out[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 0));
    out[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 1));
    out[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 2));
    out[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, scale, 3));
    return __builtin_bit_cast(bf16x8, out);
  }
  __device__ __forceinline__ bf16x8 get_hw(int t, int st) const { return get(t, st); }
};

// W4A4 reads NVFP4 records
template <int NT>
struct BFrag<SCR_W_NVFP4_A4, NT> : BFrag<SCR_W_NVFP4, NT> {};

// Gate/up operands as fp16 (NVFP4 weights and x's fp16 copy with its row
// scales; the W4A4 format's exact fp16 values): one packed fp16 multiply
// finishes each pair of weights, where the bf16 MFMA would need the products
// rounded through fp32
template <int WDT, bool GATEUP>
struct WideF16A {
  static constexpr bool value = (WDT == SCR_W_NVFP4 && GATEUP) || WDT == SCR_W_NVFP4_A4;
};

struct PassCtx {
  int tid, lane, wave, col, grp, rows, m0, nkb, ncol0, tx;
  bool active;
  float gs;
};

// One pass over exactly MTC*16 rows of a bucket: the whole K loop and the
// epilogue.  Every load in the loop is unconditional (clamped to valid
// addresses, padding rows zeroed by a select), because a load under a branch
// makes the compiler wait for all outstanding loads at the join, which would
// defeat the prefetch.
template <int WDT, int MT, int NT, bool GATEUP, int MTC>
__device__ __forceinline__ void gemm_pass(const GemmArgs& a, const PassCtx& c, const uint8_t* const* rowp,
                                          const uint8_t* const* scp, bf16 (*As)[MT * 16][kAStride],
                                          const int* src_row, const float* row_rs) {
  // NVFP4 gate/up: x's fp16 copy (row t scaled by 2^xe[t]) on the fp16 MFMA
  constexpr bool F16A = WideF16A<WDT, GATEUP>::value;
  const bf16* abase = GATEUP ? (F16A ? reinterpret_cast<const bf16*>(a.x16) : a.x) : a.h;
  const int tid = c.tid, col = c.col, grp = c.grp, nkb = c.nkb;
  constexpr int kRowChunks = kKB / 8;                      // 16-byte chunks per row and block
  constexpr int kChunks = MTC * 16 * kRowChunks;
  static_assert(kChunks % kGemmThreads == 0, "staging covers the tile exactly");
  constexpr int kPerThread = kChunks / kGemmThreads;
  // this thread's staged chunks: row offsets (element index, row-valid flag)
  // and LDS destinations, fixed for the pass
  const bf16* asrc[kPerThread];
  bool avalid[kPerThread];
  int adst[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int ci = u * kGemmThreads + tid;
    const int r = ci / kRowChunks, ch = ci % kRowChunks;
    const int off = src_row[r];
    avalid[u] = off >= 0;
    asrc[u] = abase + (off >= 0 ? off : 0) + ch * 8;
    adst[u] = r * kAStride + ch * 8;
  }
  struct AStage {
    u32x4 v[kPerThread];
  };
  auto load_a = [&](AStage& st, int kb) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) st.v[u] = ldg<u32x4>(asrc[u] + kb * kKB);
  };
  auto store_a = [&](const AStage& st, int buf) {
    bf16* base = &As[buf][0][0];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(base + adst[u]) = avalid[u] ? st.v[u] : z;
    }
  };
  // gate/up streams its weights with nontemporal loads (measured faster);
  // down, with fewer rows per weight byte, measured slower that way
  auto load_b = [&](BFrag<WDT, NT>& f, int kb) { f.template load<GATEUP>(rowp, scp, kb, c.lane); };

  f32x4 acc[MTC][NT];
#pragma unroll
  for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const BFrag<WDT, NT>& bc, int buf) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 bf[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (F16A) bf[t] = bc.get_f16(t, st);
        else bf[t] = bc.get_hw(t, st);
      }
#pragma unroll
      for (int mt = 0; mt < MTC; ++mt) {
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(&As[buf][mt * 16 + col][kcol<WDT>(grp, st)]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (F16A) acc[mt][t] = mfma16_f16(av, bf[t], acc[mt][t]);
          else acc[mt][t] = mfma16(av, bf[t], acc[mt][t]);
        }
      }
    }
  };

  // Pipeline: the weights of block kb+D-1 are requested at step kb into a
  // ring of D register slots (weights stream from HBM and need many bytes in
  // flight); the activations (mostly L2 hits) go one block ahead through
  // registers into the other LDS buffer, and are requested first so that the
  // LDS store does not wait behind the weight loads (the load counter is in
  // order).  Past the last block the loads are clamped to it (redundant, in
  // bounds).  The ring is indexed by compile-time constants.
  constexpr int D = (WDT == SCR_W_BF16 || NT == 4) ? 2 : 4;  // four 4-bit tiles per wave: two blocks
  BFrag<WDT, NT> ring[D];
  AStage A0;
  // down: the route and top-k weight of each output row of this lane, read
  // before the K loop (their latency overlaps the first weight loads instead
  // of following the last MFMA); clamped indices keep the loads unconditional
  int out_route[GATEUP ? 1 : MTC][4];
  float out_w[GATEUP ? 1 : MTC][4];
  if (!GATEUP) {
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) out_route[mt][i] = a.sorted_routes[c.m0 + mt * 16 + grp * 4 + i];
  }
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load_b(ring[i], min(i, nkb - 1));
  load_a(A0, 0);
  if (!GATEUP) {
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = out_route[mt][i];
        out_w[mt][i] = a.topk_w[(r >= 0 && r < a.R) ? r : 0];
      }
  }
  store_a(A0, 0);
  __syncthreads();
  auto step = [&](int kb, const BFrag<WDT, NT>& bc, BFrag<WDT, NT>& bl) {
    load_a(A0, min(kb + 1, nkb - 1));
    load_b(bl, min(kb + D - 1, nkb - 1));
    // the narrow formats' weight loads stay ahead of the block's decode and
    // products (left to itself the compiler sinks them to the block's end,
    // so fewer bytes are in flight: measured 3-10 % slower)
    if constexpr (WDT != SCR_W_BF16) __builtin_amdgcn_sched_barrier(0);
    compute(bc, kb & 1);
    store_a(A0, (kb + 1) & 1);
    __syncthreads();
  };
  int kb0 = 0;
  for (; kb0 + D <= nkb; kb0 += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) step(kb0 + i, ring[i], ring[(i + D - 1) % D]);
  }
#pragma unroll
  for (int i = 0; i < D - 1; ++i)
    if (kb0 + i < nkb) step(kb0 + i, ring[i], ring[(i + D - 1) % D]);

  if (!c.active) return;
#pragma unroll
  for (int mt = 0; mt < MTC; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = c.m0 + mt * 16 + grp * 4 + i;
      if (GATEUP) {
        // F16A: the row's power of two comes off after the global scale
        const float rs = F16A ? row_rs[mt * 16 + grp * 4 + i] : 1.0f;
#pragma unroll
        for (int t = 0; t < NT / 2; ++t) {
          const int hc = c.ncol0 + 16 * t + col;
          const float hv = silu_mul(c.gs * acc[mt][t][i] * rs, c.gs * acc[mt][t + NT / 2][i] * rs);
          a.h[(size_t)pos * a.I + hc] = static_cast<bf16>(hv);
        }
      } else {
        const int r = out_route[mt][i];
        const float w = out_w[mt][i];
        typedef typename RowT<WDT>::type OT;
        float v[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = w * (c.gs * acc[mt][t][i]);
        if constexpr (sizeof(OT) == 4) {
          if (r >= 0 && r < a.R) {
            OT* orow = static_cast<OT*>(a.o) + (size_t)r * a.H + c.ncol0 + col;
#pragma unroll
            for (int t = 0; t < NT; ++t) orow[16 * t] = v[t];
          }
        } else {
          // the wave's 16 NT columns of this row are NT / 2 groups of 32 (two
          // tiles each), spread over the 16 lanes of the lane group; every
          // lane takes part in the reductions, also those of padding rows
          static_assert((16 * NT) % kRowGroup == 0, "whole row groups per wave");
          int e[NT / 2];
#pragma unroll
          for (int g = 0; g < NT / 2; ++g)
            e[g] = row_group_exp(group16_max(__float_as_uint(fmaxf(fabsf(v[2 * g]), fabsf(v[2 * g + 1])))));
          if (r >= 0 && r < a.R) {
            OT* orow = static_cast<OT*>(a.o) + (size_t)r * a.H + c.ncol0 + col;
#pragma unroll
            for (int t = 0; t < NT; ++t) orow[16 * t] = scaled_row16(v[t], __builtin_ldexpf(1.0f, e[t / 2]));
            if (col == 0) {
#pragma unroll
              for (int g = 0; g < NT / 2; ++g)
                a.oe[(size_t)r * (a.H / kRowGroup) + c.ncol0 / kRowGroup + g] = (int8_t)e[g];
            }
          }
        }
        if (r >= 0 && r < a.R && c.tx == 0 && c.wave == 0 && col == 0) a.flags[r] = 1;
      }
    }
  }
}

template <int WDT, int MT, int NT, bool GATEUP>
__global__ __launch_bounds__(kGemmThreads, 2) void moe_gemm_kernel(GemmArgs a, int ntx, int pslices) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][MT * 16][kAStride];
  __shared__ int src_row[MT * 16];  // element offset of each staged row, -1 = zero row
  // F16A gate/up: 2^-xe of each pass row's token, undoing its fp16 scaling
  __shared__ float row_rs[WideF16A<WDT, GATEUP>::value ? MT * 16 : 1];

  // XCD-aware order: consecutive workgroups go to different XCDs, so bucket j
  // and all its N tiles and pass slices land on XCD (j mod 8) and share its L2
  if (GATEUP) gateup_prologue(a);
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int per_bucket = ntx * pslices;
  const int j = 8 * (q / per_bucket) + xcd;
  const int tx = q % ntx, ps = (q % per_bucket) / ntx;
  if (j >= *a.n_active) return;
  const int b = a.active_buckets[j];
  const int p0 = a.active_block_begin[j] * a.B, p1 = a.active_block_begin[j + 1] * a.B;
  if (p1 > a.h_rows || p0 >= p1) return;

  PassCtx c;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  c.wave = c.tid >> 6;
  c.col = c.lane & 15;
  c.grp = c.lane >> 4;
  c.tx = tx;
  const int K = GATEUP ? a.H : a.I;
  c.nkb = K / kKB;
  const uint8_t* rec = static_cast<const uint8_t*>(a.bucket_rows[b]);

  // this wave's weight tiles: tile-block (t, 0) of each of its NT row tiles
  const uint8_t* rowp[NT];
  const uint8_t* scp[NT];
  const int K_blocks = K / kKB;
  const size_t tile_bytes = WFmt<WDT>::tile;   // per tile-block
  const size_t stile_bytes = WFmt<WDT>::stile;
  if (GATEUP) {
    // tiles 0..NT/2-1: gate rows; NT/2..NT-1: the matching up rows
    c.ncol0 = tx * (4 * 8 * NT) + c.wave * (8 * NT);
    c.active = c.ncol0 < a.I;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row0 = (t < NT / 2 ? 0 : a.I) + (c.active ? c.ncol0 + 16 * (t % (NT / 2)) : 0);
      const size_t tb = (size_t)(row0 / 16) * K_blocks;
      rowp[t] = rec + a.lay.w13_off + tb * tile_bytes;
      scp[t] = rec + a.lay.w13_scale_off + tb * stile_bytes;
    }
  } else {
    c.ncol0 = tx * (4 * 16 * NT) + c.wave * (16 * NT);
    c.active = c.ncol0 < a.H;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row0 = c.active ? c.ncol0 + 16 * t : 0;
      const size_t tb = (size_t)(row0 / 16) * K_blocks;
      rowp[t] = rec + a.lay.w2_off + tb * tile_bytes;
      scp[t] = rec + a.lay.w2_scale_off + tb * stile_bytes;
    }
  }
  c.gs = WFmt<WDT>::gscale ? *reinterpret_cast<const float*>(rec + (GATEUP ? a.lay.g13_off : a.lay.g2_off))
                           : 1.0f;
  const int arow_len = K;  // elements per activation row

  // this workgroup's passes: slice ps of every pslices-th
  for (int m0 = p0 + ps * (MT * 16); m0 < p1; m0 += pslices * (MT * 16)) {
    c.m0 = m0;
    c.rows = min(MT * 16, p1 - m0);
    for (int i = c.tid; i < MT * 16; i += kGemmThreads) {
      int off = -1;
      float rs = 1.0f;
      if (i < c.rows) {
        if (GATEUP) {
          const int r = a.sorted_routes[m0 + i];
          if (r >= 0 && r < a.R) {
            off = (r / a.k) * arow_len;
            if constexpr (WideF16A<WDT, GATEUP>::value) rs = __builtin_ldexpf(1.0f, -a.xe[r / a.k]);
          }
        } else {
          off = (m0 + i) * arow_len;
        }
      }
      src_row[i] = off;
      if constexpr (WideF16A<WDT, GATEUP>::value) row_rs[i] = rs;
    }
    __syncthreads();
    switch (c.rows / 16) {
      case 1: gemm_pass<WDT, MT, NT, GATEUP, 1>(a, c, rowp, scp, As, src_row, row_rs); break;
      case 2: if constexpr (MT >= 2) gemm_pass<WDT, MT, NT, GATEUP, 2>(a, c, rowp, scp, As, src_row, row_rs); break;
      case 3: if constexpr (MT >= 3) gemm_pass<WDT, MT, NT, GATEUP, 3>(a, c, rowp, scp, As, src_row, row_rs); break;
      case 4: if constexpr (MT >= 4) gemm_pass<WDT, MT, NT, GATEUP, 4>(a, c, rowp, scp, As, src_row, row_rs); break;
      case 5: if constexpr (MT >= 5) gemm_pass<WDT, MT, NT, GATEUP, 5>(a, c, rowp, scp, As, src_row, row_rs); break;
      case 6: if constexpr (MT >= 6) gemm_pass<WDT, MT, NT, GATEUP, 6>(a, c, rowp, scp, As, src_row, row_rs); break;
      case 7: if constexpr (MT >= 7) gemm_pass<WDT, MT, NT, GATEUP, 7>(a, c, rowp, scp, As, src_row, row_rs); break;
      case 8: if constexpr (MT >= 8) gemm_pass<WDT, MT, NT, GATEUP, 8>(a, c, rowp, scp, As, src_row, row_rs); break;
      default: break;
    }
    __syncthreads();  // src_row and As are reused by the next pass
  }
}

// ------------------------------------------------------- wide-tile GEMM
//
// For chunks with many rows per expert (the MFMA-bound shapes).  One
// workgroup of EW = 8 waves (two per SIMD, 256 registers each, one workgroup
// per CU) owns one active bucket, a contiguous range of its N chunks and a
// slice of its row passes; within a pass the weight stream never restarts
// (the prefetch ring runs across chunk boundaries).  Each wave owns NTW row
// tiles of 16 weight rows per chunk (gate/up: NTW/2 gate tiles and the
// matching up tiles; down: NTW tiles of output columns), so every activation
// fragment read from LDS feeds NTW MFMAs, and the two waves of a SIMD
// overlap one another's decode, waits and barriers with their MFMAs.
//
// Activations reach LDS by direct global-to-LDS loads (no register staging):
// K-block buffers, each a [rows][128] bf16 tile whose 16-byte chunks are
// XOR-swizzled by a function of (row mod 16) (wide_swz), so the fragment
// reads hit distinct banks.
// The buffers are separate arrays so that the compiler can tell a read of one
// from the direct loads still in flight into the other.
// activation K-block buffers in LDS (loaded NBUF - 1 blocks ahead): four
// where the K blocks of a GEMM come in fours, else two (K a multiple of 256)
constexpr int kWideBufs = 4;
constexpr int kWideRing = 2;  // NVFP4 weight ring depth in K blocks (deeper measured slower)
constexpr int kWideStage = 4096;  // bytes of LDS per wave for the epilogue tile (16 rows x 64 fp32)

// The chunk swizzle of activation row r: physical chunk = logical ^ wide_swz(r).
// A 16-lane group of a fragment read takes 16 rows; the bf16 order (lane
// group g reads logical chunk 4 s + g) is conflict-free with r mod 16 itself,
// while the block-scaled formats' order (chunk 4 g + s) needs the two 2-bit
// halves of r mod 16 swapped: with r mod 16 every 128-bit read of the
// latter took a two-way bank conflict on gfx950 (measured with the LDS
// conflict counter), with the swap none, for every step and row tile.
template <int WDT>
__device__ __forceinline__ int wide_swz(int r) {
  return WDT == SCR_W_BF16 ? (r & 15) : (((r & 3) << 2) | ((r >> 2) & 3));
}

// s_waitcnt immediate that waits until at most n vector memory operations are
// outstanding (gfx9 encoding; the LDS and export counters are left alone)
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// the NVFP4 wide gate/up runs on fp16 (half the decode work of bf16: see
// BFrag<SCR_W_NVFP4>::get_f16); every other wide pass on bf16
// (W4A4: both GEMMs, whose activations are exact fp16 values)

// x as fp16 for the F16A gate/up, one wave per token: the row is scaled by
// 2^e, e = 15 - (the exponent of its largest magnitude in frexp form), which
// puts that magnitude in [2^14, 2^15).  Every bf16 value of the row at or
// above 2^-28 of it is then exact in fp16, so the products and fp32 sums are
// those of the bf16 values times 2^e (smaller values round as fp16
// subnormals).  An all-zero or non-finite row keeps e = 0.  NC > 0: the row
// is H = 512 * NC wide and stays in registers between the two steps; NC = 0:
// any multiple of 512, read twice.
__device__ __forceinline__ float bf16_lo(unsigned v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(unsigned v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ u32x4 scaled_f16x8(const u32x4& v, int e) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const h2 p = {(_Float16)__builtin_ldexpf(bf16_lo(v[i]), e), (_Float16)__builtin_ldexpf(bf16_hi(v[i]), e)};
    o[i] = __builtin_bit_cast(unsigned, p);
  }
  return o;
}

template <int NC>
__global__ __launch_bounds__(256) void x_to_f16_kernel(const bf16* __restrict__ x, int T, int H,
                                                       uint16_t* __restrict__ x16, int32_t* __restrict__ xe) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (t >= T) return;
  const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
  u32x4* out = reinterpret_cast<u32x4*>(x16 + (size_t)t * H);
  const int n8 = H / 8;
  float m = 0.0f;
  u32x4 v[NC > 0 ? NC : 1];
  if constexpr (NC > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) v[c] = row[c * 64 + lane];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(v[c][i])), fabsf(bf16_hi(v[c][i]))));
  } else {
    for (int c = lane; c < n8; c += 64) {
      const u32x4 w = row[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  int e = 0;
  if (m > 0.0f && m <= 3.4028235e38f) {
    int ex;
    (void)__builtin_frexpf(m, &ex);
    e = 15 - ex;
  }
  if constexpr (NC > 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) out[c * 64 + lane] = scaled_f16x8(v[c], e);
  } else {
    for (int c = lane; c < n8; c += 64) out[c] = scaled_f16x8(row[c], e);
  }
  if (lane == 0) xe[t] = e;
}

static int launch_x_to_f16(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((a.T + 3) / 4), block(256);
  uint16_t* x16 = const_cast<uint16_t*>(a.x16);
  int32_t* xe = const_cast<int32_t*>(a.xe);
  // rows of exactly 512, 1024, 2048 or 4096 values are held in registers;
  // every other row length (any multiple of 8) takes the strided loop
  switch (a.H % 512 == 0 ? a.H / 512 : 0) {
    case 1: hipLaunchKernelGGL(x_to_f16_kernel<1>, grid, block, 0, s, a.x, a.T, a.H, x16, xe); break;
    case 2: hipLaunchKernelGGL(x_to_f16_kernel<2>, grid, block, 0, s, a.x, a.T, a.H, x16, xe); break;
    case 4: hipLaunchKernelGGL(x_to_f16_kernel<4>, grid, block, 0, s, a.x, a.T, a.H, x16, xe); break;
    case 8: hipLaunchKernelGGL(x_to_f16_kernel<8>, grid, block, 0, s, a.x, a.T, a.H, x16, xe); break;
    default: hipLaunchKernelGGL(x_to_f16_kernel<0>, grid, block, 0, s, a.x, a.T, a.H, x16, xe); break;
  }
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

template <int WDT, int NTW>
struct BLoads {  // vector memory instructions per wave for one K block of weights
  static constexpr int value = WDT == SCR_W_BF16 ? 4 * NTW : 2 * NTW;  // fp8: two code loads; fp4: codes + scales
};

template <int WDT, int MT, bool GATEUP, int EW, int NTW, int MTC, int NBUF>
__device__ __forceinline__ void wide_pass(const GemmArgs& a, const int* src_row, const int* row_route,
                                          const float* row_w, const float* row_rs, bf16* As0, bf16* As1, bf16* As2,
                                          bf16* As3, uint32_t* stg, int m0, __amdgpu_buffer_rsrc_t wrsrc,
                                          const int* toff0, const int* soff0, float gs, int nkb, int c_begin,
                                          int c_end) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  constexpr int CT = GATEUP ? EW * NTW / 2 : EW * NTW;  // row tiles per chunk and tensor half
  constexpr int tile_bytes = WFmt<WDT>::tile;
  constexpr int stile_bytes = WFmt<WDT>::stile;
  constexpr bool F16A = WideF16A<WDT, GATEUP>::value;  // fp16 activations and weights
  static_assert(NBUF == 2 || NBUF == 4, "two or four activation buffers");
  bf16* const bufs[kWideBufs] = {As0, As1, As2, As3};

  // activations through a buffer resource over x (gate/up; its fp16 copy
  // for F16A) or h (down)
  const void* const abase = GATEUP ? (F16A ? (const void*)a.x16 : (const void*)a.x) : (const void*)a.h;
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)abase, (short)0, (int)(2u * (unsigned)(GATEUP ? a.T * a.H : a.h_rows * a.I)), 0x00020000);
  // direct-load sources of this lane: the 4 * MTC wave instructions of a K
  // block (each fills 64 16-byte chunks = 4 rows) are dealt round-robin to the
  // EW waves; every wave issues the same count NA (a wave past the end repeats
  // the last instruction: the same bytes to the same place), so that the
  // waits below can count them.  Instruction j fills LDS chunk q = 64 j +
  // lane of a buffer, i.e. row q / 16, physical chunk q % 16, which holds
  // logical chunk (q % 16) ^ wide_swz(row).
  constexpr int NA = (4 * MTC + EW - 1) / EW;
  unsigned aoff[NA];  // byte offsets (below 2^32: the host bounds T * H and h_rows * I by 2^31)
  int adst[NA];       // LDS element offsets of the wave's 1 KB destinations
#pragma unroll
  for (int u = 0; u < NA; ++u) {
    const int j = min(u * EW + wave, 4 * MTC - 1);
    const int q = j * 64 + lane;
    const int r = q >> 4, c = (q & 15) ^ wide_swz<WDT>(r);
    const int off = src_row[r];
    aoff[u] = 2u * (unsigned)(off >= 0 ? off : 0) + 16u * c;  // padding rows read row 0 (outputs dropped)
    adst[u] = j * 512;
  }
  auto load_a = [&](bf16* buf, int kb) {
#pragma unroll
    for (int u = 0; u < NA; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (__attribute__((address_space(3))) void*)(buf + adst[u]), 16,
                                               (int)aoff[u], kb * (2 * kKB), 0, 0);
  };
  // weights of flat step s = chunk * nkb + kb
  auto load_b = [&](BFrag<WDT, NTW>& f, int s) {
    const int ch = s / nkb, kb = s - ch * nkb;
    const int blk = ch * CT * nkb + kb;
    int tp[NTW], sp[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      tp[t] = toff0[t] + blk * tile_bytes;
      sp[t] = soff0[t] + blk * stile_bytes;
    }
    f.load_buf(wrsrc, tp, sp, lane);
  };
  auto read_a = [&](bf16x8 (&af)[MTC], const bf16* buf, int st) {
    const int c = kcol<WDT>(grp, st) >> 3;
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt)
      af[mt] = *reinterpret_cast<const bf16x8*>(buf + (mt * 16 + col) * kKB + ((c ^ wide_swz<WDT>(col)) << 3));
  };


  f32x4 acc[MTC][NTW];

  // Epilogue through a per-wave LDS tile: the outputs of one 16-row tile are
  // written to LDS in the MFMA layout and read back as 16-byte row pieces,
  // so that each global store writes whole row segments (gate/up: 64 bytes
  // of h per row and wave; down: a row's 64 output columns, one or two cache
  // lines) instead of scattered 2- and 4-byte values.
  uint32_t* const wst = stg + wave * (kWideStage / 4);
  auto epilogue = [&](int ch) {
    if (GATEUP) {
      constexpr int HC = 8 * NTW;                  // h columns per wave
      constexpr int PPR = HC / 8;                  // 16-byte pieces per row
      constexpr int ROUNDS = (16 * PPR + 63) / 64;  // store rounds for 16 rows
      bf16* sh = reinterpret_cast<bf16*>(wst);
#pragma unroll
      for (int mt = 0; mt < MTC; ++mt) {
        // rows i and i + 1 of a lane converted as one bf16 pair, stored as halves
        uint16_t* sh16 = reinterpret_cast<uint16_t*>(sh);
        if constexpr (WDT == SCR_W_NVFP4_A4) {
          // W4A4: h quantised to NVFP4 under the layer's down scale a2, per
          // row and 16 columns.  The wave's 16 x HC block of h goes through
          // its LDS tile as fp32; then lane l takes row l / 4, the 8 columns
          // 8 (l % 4) .. + 7 (half of one NVFP4 block: lanes l and l ^ 1
          // share a block and its largest magnitude), and writes them as the
          // exact fp16 values e2m1 * block (the down GEMM's fp16 operand; a2
          // goes to its accumulators)
          static_assert(HC == 32, "one wave's h row holds two NVFP4 blocks");
          float* shf = reinterpret_cast<float*>(wst);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int t = 0; t < NTW / 2; ++t)
              shf[(grp * 4 + i) * HC + 16 * t + col] = silu_mul(gs * acc[mt][t][i], gs * acc[mt][t + NTW / 2][i]);
          {
            const float a2 = a.act_scale[1];
            const float4* src = reinterpret_cast<const float4*>(shf + (lane >> 2) * HC + 8 * (lane & 3));
            const float4 q0 = src[0], q1 = src[1];
            const float v[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            float amax = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(v[c]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            const float bv = __builtin_amdgcn_cvt_f32_fp8((int)nvfp4_block_code(amax, a2), 0);
            const float rcp = nvfp4_block_rcp(bv, a2);
            u32x4 out;
#pragma unroll
            for (int c = 0; c < 4; ++c) out[c] = nvfp4_pair_f16(nvfp4_pair_codes(v[2 * c], v[2 * c + 1], rcp), bv);
            const int pos = m0 + mt * 16 + (lane >> 2);
            const int hc = ch * (HC * EW) + wave * HC + 8 * (lane & 3);
            *reinterpret_cast<u32x4*>(a.h + (size_t)pos * a.I + hc) = out;
          }
          // one row tile at a time (interleaving the tiles' divisions would
          // hold more registers than the accumulators leave)
          __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int i = 0; i < 4; i += 2)
#pragma unroll
            for (int t = 0; t < NTW / 2; ++t) {
              unsigned p;
              if constexpr (F16A) {
                // the row's power of two comes off after the global scale, as
                // exact multiplies (gs * acc is then the bf16 path's value)
                const float s0 = row_rs[mt * 16 + grp * 4 + i], s1 = row_rs[mt * 16 + grp * 4 + i + 1];
                p = pack_bf16(silu_mul(gs * acc[mt][t][i] * s0, gs * acc[mt][t + NTW / 2][i] * s0),
                              silu_mul(gs * acc[mt][t][i + 1] * s1, gs * acc[mt][t + NTW / 2][i + 1] * s1));
              } else {
                p = pack_bf16(silu_mul(gs * acc[mt][t][i], gs * acc[mt][t + NTW / 2][i]),
                              silu_mul(gs * acc[mt][t][i + 1], gs * acc[mt][t + NTW / 2][i + 1]));
              }
              sh16[(grp * 4 + i) * HC + 16 * t + col] = (uint16_t)p;
              sh16[(grp * 4 + i + 1) * HC + 16 * t + col] = (uint16_t)(p >> 16);
            }
        }
        if constexpr (WDT != SCR_W_NVFP4_A4) {
#pragma unroll
          for (int rd = 0; rd < ROUNDS; ++rd) {
            const int q = rd * 64 + lane, rr = q / PPR, pc = q % PPR;
            if (q < 16 * PPR) {
              const u32x4 v = *reinterpret_cast<const u32x4*>(sh + rr * HC + pc * 8);
              const int pos = m0 + mt * 16 + rr;
              const int hc = ch * (HC * EW) + wave * HC + pc * 8;
              *reinterpret_cast<u32x4*>(a.h + (size_t)pos * a.I + hc) = v;
            }
          }
        }
      }
    } else {
      // fp16 rows scaled per 32 columns (every format here), through the
      // wave's tile as fp32; row weights carry the global scale
      constexpr int OC = 16 * NTW;  // output columns per wave
      static_assert(16 * OC * 4 <= kWideStage, "the fp32 tile fits the wave's stage");
      float* sf = reinterpret_cast<float*>(wst);
#pragma unroll
      for (int mt = 0; mt < MTC; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w0 = row_w[mt * 16 + grp * 4 + i];
#pragma unroll
          for (int t = 0; t < NTW; ++t) sf[(grp * 4 + i) * OC + 16 * t + col] = w0 * acc[mt][t][i];
        }
        store_rows_f16<OC>(sf, row_route + mt * 16, lane, static_cast<uint16_t*>(a.o), a.oe, a.flags, a.H,
                           ch * (OC * EW) + wave * OC, ch == 0 && wave == 0);
      }
    }
  };

  // weight ring depth (blocks): HBM latency under load is about two blocks
  // of compute, so the weights of block s are requested at block s - D + 1
  constexpr int D = WDT == SCR_W_BF16 ? 2 : kWideRing;
  constexpr int U = D > NBUF ? D : NBUF;  // unroll: ring and buffers indexed statically
  constexpr int NB = BLoads<WDT, NTW>::value;
  const int s0 = c_begin * nkb, s1 = c_end * nkb;  // flat steps s = chunk * nkb + kb
  constexpr int LA = NBUF - 1;  // activation blocks loaded ahead
  BFrag<WDT, NTW> ring[D];
  // Down (K = I = NBUF blocks) keeps the bucket's whole h block resident
  // for all of its chunks: loaded once, no further activation loads or
  // barriers.  Gate/up streams x blocks LA ahead through the buffers.
  const bool resident = !GATEUP && nkb == NBUF;
  // blocks s0 .. s0+LA-1 of the activations (all of them when resident),
  // then the weights of blocks s0 .. s0+D-2
#pragma unroll
  for (int i = 0; i < LA; ++i) load_a(bufs[i], i % nkb);
  if (resident) load_a(bufs[LA], LA);
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load_b(ring[i], min(s0 + i, s1 - 1));
  if (resident)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 1) * NB));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((LA - 1) * NA + (D - 1) * NB));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  bf16x8 af[MTC];
  for (int ch = c_begin; ch < c_end; ++ch) {
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb0 = 0; kb0 < nkb; kb0 += U) {
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int kb = kb0 + i, s = ch * nkb + kb;
        const BFrag<WDT, NTW>& bc = ring[i % D];
        const bf16* buf = bufs[i % NBUF];
        // the activations of block kb + LA into the buffer block kb - 1 used
        // (every wave has finished it), then the weights of block s + D - 1
        // into the ring slot block s - 1 used
        if (!resident) load_a(bufs[(i + LA) % NBUF], (kb + LA) % nkb);
        load_b(ring[(i + D - 1) % D], min(s + D - 1, s1 - 1));
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          read_a(af, buf, st);
          // one weight tile at a time: its decode, then its MTC products
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            if constexpr (F16A) {
              const bf16x8 bt = bc.get_f16(t, st);
#pragma unroll
              for (int mt = 0; mt < MTC; ++mt) acc[mt][t] = mfma16_f16(af[mt], bt, acc[mt][t]);
            } else {
              const bf16x8 bt = bc.get_hw(t, st);
#pragma unroll
              for (int mt = 0; mt < MTC; ++mt) acc[mt][t] = mfma16(af[mt], bt, acc[mt][t]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!resident) {
          // the next block's activations (issued LA - 1 blocks ago) are in
          // LDS once at most the loads issued after them are pending: in
          // steady state weights of LA blocks and activations of LA - 1;
          // right after the prologue (which issued D - 1 weight blocks behind
          // the activations) possibly fewer weights, so the smaller count
          __builtin_amdgcn_s_waitcnt(vmcnt_imm((LA - 1) * NA + (D < LA ? D : LA) * NB));
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    epilogue(ch);
  }
  // no direct load may still target the buffers when the next pass refills them
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
}

template <int WDT, int MT, bool GATEUP, int EW, int NTW, int NBUF>
__global__ __launch_bounds__(64 * EW) void moe_wide_kernel(GemmArgs a, int groups, int pslices) {
  __shared__ __attribute__((aligned(1024))) bf16 As0[MT * 16 * kKB];
  __shared__ __attribute__((aligned(1024))) bf16 As1[MT * 16 * kKB];
  __shared__ __attribute__((aligned(1024))) bf16 As2[NBUF > 2 ? MT * 16 * kKB : 8];
  __shared__ __attribute__((aligned(1024))) bf16 As3[NBUF > 3 ? MT * 16 * kKB : 8];
  __shared__ int src_row[MT * 16];
  // down: the route of each pass row (-1 for padding) and its top-k weight,
  // read once per pass so that the epilogue does no dependent global loads
  __shared__ int row_route[GATEUP ? 1 : MT * 16];
  __shared__ float row_w[GATEUP ? 1 : MT * 16];
  // F16A gate/up: 2^-xe of each pass row's token, undoing its fp16 scaling
  __shared__ float row_rs[WideF16A<WDT, GATEUP>::value ? MT * 16 : 1];
  __shared__ __attribute__((aligned(256))) uint32_t stg[EW * kWideStage / 4];  // per-wave epilogue tiles
  if (GATEUP) gateup_prologue(a);
  // XCD-aware order: all groups and pass slices of bucket j run on XCD j mod 8
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int per_bucket = groups * pslices;
  const int j = 8 * (q / per_bucket) + xcd, g = q % groups, ps = (q % per_bucket) / groups;
  if (j >= *a.n_active) return;
  const int b = a.active_buckets[j];
  const int p0 = a.active_block_begin[j] * a.B, p1 = a.active_block_begin[j + 1] * a.B;
  if (p1 > a.h_rows || p0 >= p1) return;
  constexpr int kThreads = 64 * EW;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int K = GATEUP ? a.H : a.I;
  const int nkb = K / kKB;
  const int nchunks = GATEUP ? a.I / (8 * NTW * EW) : a.H / (16 * NTW * EW);
  const int c_begin = g * nchunks / groups, c_end = (g + 1) * nchunks / groups;
  if (c_begin >= c_end) return;
  const uint8_t* rec = static_cast<const uint8_t*>(a.bucket_rows[b]);
  // the record as a buffer (every weight load is range-checked against it)
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, (int)a.lay.record_bytes, 0x00020000);
  constexpr int tile_bytes = WFmt<WDT>::tile;
  constexpr int stile_bytes = WFmt<WDT>::stile;
  // byte offsets of tile-block (t, 0) of this wave's tiles in chunk 0 (wave-uniform)
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int toff0[NTW], soff0[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int row0 = GATEUP ? (t < NTW / 2 ? 0 : a.I) + wv * 8 * NTW + 16 * (t % (NTW / 2)) : wv * 16 * NTW + 16 * t;
    const int tb = (row0 / 16) * nkb;
    toff0[t] = (int)(GATEUP ? a.lay.w13_off : a.lay.w2_off) + tb * tile_bytes;
    soff0[t] = (int)(GATEUP ? a.lay.w13_scale_off : a.lay.w2_scale_off) + tb * stile_bytes;
  }
  float gs = WFmt<WDT>::gscale ? *reinterpret_cast<const float*>(rec + (GATEUP ? a.lay.g13_off : a.lay.g2_off))
                               : 1.0f;
  // W4A4: the layer's activation scale joins the record's global scale
  if constexpr (WDT == SCR_W_NVFP4_A4) gs *= a.act_scale[GATEUP ? 0 : 1];
  // this workgroup's passes: slice ps of every pslices-th
  for (int m0 = p0 + ps * (MT * 16); m0 < p1; m0 += pslices * (MT * 16)) {
    const int rows = min(MT * 16, p1 - m0);
    for (int i = tid; i < MT * 16; i += kThreads) {
      int off = -1;
      if (i < rows) {
        if (GATEUP) {
          const int r = a.sorted_routes[m0 + i];
          if (r >= 0 && r < a.R) off = (r / a.k) * K;
        } else {
          off = (m0 + i) * K;
        }
      }
      src_row[i] = off;
      if constexpr (WideF16A<WDT, GATEUP>::value && WDT == SCR_W_NVFP4) {
        const int r = i < rows ? a.sorted_routes[m0 + i] : -1;
        row_rs[i] = (r >= 0 && r < a.R) ? __builtin_ldexpf(1.0f, -a.xe[r / a.k]) : 1.0f;
      } else if constexpr (WideF16A<WDT, GATEUP>::value) {
        row_rs[i] = 1.0f;
      }
      if (!GATEUP) {
        const int r = i < rows ? a.sorted_routes[m0 + i] : -1;
        const bool valid = r >= 0 && r < a.R;
        row_route[i] = valid ? r : -1;
        row_w[i] = valid ? a.topk_w[r] * gs : 0.0f;  // the expert's global scale folded in
      }
    }
    __syncthreads();
#define SCR_WIDE_PASS(n)                                                                                   \
  case n:                                                                                                  \
    if constexpr (MT >= n)                                                                                 \
      wide_pass<WDT, MT, GATEUP, EW, NTW, n, NBUF>(a, src_row, row_route, row_w, row_rs, As0, As1, As2, As3, stg, m0, \
                                             wrsrc, toff0, soff0, gs, nkb, c_begin, c_end);                     \
    break;
    switch (rows / 16) {
      SCR_WIDE_PASS(1)
      SCR_WIDE_PASS(2)
      SCR_WIDE_PASS(3)
      SCR_WIDE_PASS(4)
      SCR_WIDE_PASS(5)
      SCR_WIDE_PASS(6)
      SCR_WIDE_PASS(7)
      SCR_WIDE_PASS(8)
      default: break;
    }
#undef SCR_WIDE_PASS
    __syncthreads();  // src_row is reused by the next pass
  }
}

// y[t][c] = sum_j o[t*k + j][c] in rank order j, in fp32 (unwritten routes
// count as zero); 8 columns per thread
__device__ __forceinline__ void load_row8(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
// fp16 rows (their group's 2^-e applied by the caller).  Each dword is split
// by shifts: a bit_cast of a vector element to a half2 compiled to one dword
// load whose halves every pair then repeated.
__device__ __forceinline__ void load_row8(const uint16_t* p, float* v) {
  const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned u = q[i];
    v[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu)));
    v[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)));
  }
}

template <typename OT, bool BF16_OUT, int G>
__global__ __launch_bounds__(256) void combine_kernel(const OT* __restrict__ o, const int8_t* __restrict__ oe,
                                                      const int32_t* __restrict__ flags, int T, int k,
                                                      int H, void* __restrict__ y) {
  const int h8 = H / 8;
  const size_t total = (size_t)T * h8;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / h8), c8 = (int)(i % h8);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // ranks in groups of G (G >= k up to 16: one round of loads): every flag
    // and row of a group is loaded unconditionally (clamped to the last rank),
    // so the loads overlap; an unwritten route leaves the sum untouched (a
    // select, not a branch)
    for (int j0 = 0; j0 < k; j0 += G) {
      int fl[G];
      float v[G][8];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int r = t * k + min(j0 + u, k - 1);
        const int f = flags[r];
        fl[u] = j0 + u < k ? f : 0;
        load_row8(o + (size_t)r * H + 8 * c8, v[u]);
        if constexpr (sizeof(OT) == 2) {  // the group's exponent (8 c8 .. + 7 lie in one group)
          const float sc = __builtin_ldexpf(1.0f, -(int)oe[(size_t)r * (H / kRowGroup) + (8 * c8) / kRowGroup]);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[u][q] *= sc;
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fl[u] ? acc[q] + v[u][q] : acc[q];
    }
    if (BF16_OUT) {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      u32x4 out;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t pr = {static_cast<bf16>(acc[2 * q]), static_cast<bf16>(acc[2 * q + 1])};
        out[q] = __builtin_bit_cast(unsigned, pr);
      }
      reinterpret_cast<u32x4*>(static_cast<bf16*>(y) + (size_t)t * H)[c8] = out;
    } else {
      float4* yp = reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * H + 8 * c8);
      yp[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      yp[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

// ------------------------------------- activations under the layer's scales
//
// The A8 and A4 formats quantise each GEMM's input under the largest of the
// routed layer's input scales for that GEMM (FreeToken PR #676, Solution,
// fourth bullet): a1 = max(input_scale), a2 = max(down_input_scale).  x is
// quantised here, before the GEMMs, one thread per 16 consecutive elements of
// a row; h in the gate/up epilogue.  MODE:
//   kActFp8      E4M3 codes of x / a1 (W4A8, and scr_quantize_fp8)
//   kActNvfp4    NVFP4 codes (packed, low nibble = even column) and block
//                scale codes (scr_quantize_nvfp4)
//   kActNvfp4F16 the decoded NVFP4 values e2m1 * block as fp16 (the W4A4
//                GEMM's operand; a1 goes to its accumulators)
// Every workgroup reduces the scale arrays itself (at most 4096 floats);
// workgroup 0 also stores a1, a2 for the GEMMs and for the caller.
constexpr int kActFp8 = 0, kActNvfp4 = 1, kActNvfp4F16 = 2;
constexpr int kActMaxGrid = 1024;

template <int MODE>
__global__ __launch_bounds__(256) void act_quant_kernel(const bf16* __restrict__ x, long long nblk,
                                                        const float* __restrict__ s1, const float* __restrict__ s2,
                                                        int n_scales, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ bs, uint16_t* __restrict__ f16,
                                                        float* __restrict__ act_scale, float* __restrict__ a_out) {
  __shared__ float sm;
  if (threadIdx.x < 64) {
    float m1, m2;
    wave_scale_max2(s1, s2, n_scales, threadIdx.x, m1, m2);
    if (threadIdx.x == 0) {
      sm = m1;
      if (blockIdx.x == 0) {
        if (act_scale) {
          act_scale[0] = m1;
          act_scale[1] = m2;
        }
        if (a_out) {
          a_out[0] = m1;
          a_out[1] = m2;
        }
      }
    }
  }
  __syncthreads();
  const float a1 = sm;
  const float r1 = 1.0f / a1;  // FP8: codes of x times the reciprocal of the layer scale
  for (long long b = blockIdx.x * 256ll + threadIdx.x; b < nblk; b += (long long)gridDim.x * 256) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 16);
    const u32x4 v0 = ldg<u32x4>(src), v1 = ldg<u32x4>(src + 1);
    float f[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(v0[i]);
      f[2 * i + 1] = bf16_hi(v0[i]);
      f[8 + 2 * i] = bf16_lo(v1[i]);
      f[8 + 2 * i + 1] = bf16_hi(v1[i]);
    }
    if constexpr (MODE == kActFp8) {
      u32x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[i] = e4m3_code_sat(f[4 * i] * r1) | (e4m3_code_sat(f[4 * i + 1] * r1) << 8) |
                 (e4m3_code_sat(f[4 * i + 2] * r1) << 16) | (e4m3_code_sat(f[4 * i + 3] * r1) << 24);
      reinterpret_cast<u32x4*>(q + b * 16)[0] = out;
    } else {
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
      const unsigned bc = nvfp4_block_code(amax, a1);
      const float bv = __builtin_amdgcn_cvt_f32_fp8((int)bc, 0);
      const float rcp = nvfp4_block_rcp(bv, a1);
      unsigned c[8];  // code pairs, the even element in the low nibble
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = nvfp4_pair_codes(f[2 * i], f[2 * i + 1], rcp);
      if constexpr (MODE == kActNvfp4) {
        u32x2 out;
#pragma unroll
        for (int w = 0; w < 2; ++w) out[w] = c[4 * w] | (c[4 * w + 1] << 8) | (c[4 * w + 2] << 16) | (c[4 * w + 3] << 24);
        reinterpret_cast<u32x2*>(q + b * 8)[0] = out;
        bs[b] = (uint8_t)bc;
      } else {
        u32x4 out[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i / 4][i % 4] = nvfp4_pair_f16(c[i], bv);
        u32x4* dst = reinterpret_cast<u32x4*>(f16 + b * 16);
        dst[0] = out[0];
        dst[1] = out[1];
      }
    }
  }
}

template <int MODE>
static int launch_act_quant(const bf16* x, long long rows, int cols, const float* s1, const float* s2, int n_scales,
                            uint8_t* q, uint8_t* bs, uint16_t* f16, float* act_scale, float* a_out, hipStream_t s) {
  const long long nblk = rows * (cols / 16);
  long long grid = (nblk + 255) / 256;
  if (grid > kActMaxGrid) grid = kActMaxGrid;
  if (grid < 1) grid = 1;  // the scales are still reduced and reported
  hipLaunchKernelGGL((act_quant_kernel<MODE>), dim3((unsigned)grid), dim3(256), 0, s, x, nblk, s1, s2, n_scales, q,
                     bs, f16, act_scale, a_out);
  SCR_CHECK_LAUNCH();
  return SCR_OK;
}

// ------------------------------------------------ W4A8: MXFP4 x FP8
//
// FP8 activations (E4M3 codes of x / a1, h / a2) against MXFP4 weights,
// multiplied by the gfx950 block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4
// (A fp8, B fp4): one instruction per 16x16 output tile and 128-wide K block,
// the weights' e8m0 scales applied inside the instruction, the activations'
// scale 1 (code 127) there and the layer scale applied to the fp32
// accumulators.  No dequantisation.  Operand layout per lane l, g = l / 16
// (measured on the device with one-hot operands):
//   A (16 x 128 fp8): row l % 16; bytes 0..15 hold k = 16 g .. 16 g + 15,
//                     bytes 16..31 hold k = 64 + 16 g .. 64 + 16 g + 15
//   B (128 x 16 fp4): column l % 16; nibbles 0..31 (low first) hold
//                     k = 32 g .. 32 g + 31: exactly one MXFP4 tile-block load
//   scales: lane l gives the e8m0 code of row (A) / column (B) l % 16 for the
//           32-column block l / 16: the MXFP4 tile-block's scale byte `lane`
// h is quantised in the gate/up epilogue and read by down the way gate/up
// reads x.
constexpr int kUnitScale = 127;  // e8m0 code of 2^0

typedef int i32x8 __attribute__((ext_vector_type(8)));

// RES: down with K = I = NBUF blocks keeps the bucket's whole h block
// resident in LDS (a compile-time choice: the run-time one spills registers)
template <int MT, bool GATEUP, int EW, int NTW, int MTC, bool RES, int NBUF>
__device__ __forceinline__ void w4a8_pass(const GemmArgs& a, const int* src_row, const int* row_route, const float* row_w, uint8_t* As0, uint8_t* As1,
                                          uint8_t* As2, uint8_t* As3, uint32_t* stg, int m0,
                                          __amdgpu_buffer_rsrc_t wrsrc, const int* toff0, const int* soff0,
                                          int nkb, int c_begin, int c_end) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  constexpr int CT = GATEUP ? EW * NTW / 2 : EW * NTW;  // row tiles per chunk and tensor half
  static_assert(NBUF == 2 || NBUF == 4, "two or four activation buffers");
  uint8_t* const bufs[kWideBufs] = {As0, As1, As2, As3};

  // MXFP8 activations through a buffer resource over x's codes (gate/up) or h's (down)
  const __amdgpu_buffer_rsrc_t arsrc =
      GATEUP ? __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, (short)0, a.T * a.H, 0x00020000)
             : __builtin_amdgcn_make_buffer_rsrc((void*)a.hq, (short)0, a.h_rows * a.I, 0x00020000);
  // direct loads of a K block: rows of 128 bytes = 8 chunks of 16; 2 * MTC
  // wave instructions dealt round-robin to the waves (a wave past the end
  // repeats the last one), instruction j filling LDS chunk q = 64 j + lane,
  // i.e. row q / 8, physical chunk q % 8 = logical chunk (q % 8) ^ (row % 8)
  constexpr int NA = (2 * MTC + EW - 1) / EW;
  int aoff[NA];
  int adst[NA];
#pragma unroll
  for (int u = 0; u < NA; ++u) {
    const int j = min(u * EW + wave, 2 * MTC - 1);
    const int q = j * 64 + lane;
    const int r = q >> 3, c = (q & 7) ^ (r & 7);
    const int off = src_row[r];
    aoff[u] = (off >= 0 ? off : 0) + 16 * c;  // padding rows read row 0 (their outputs are dropped)
    adst[u] = j * 1024;
  }
  auto load_a = [&](uint8_t* buf, int kb) {
#pragma unroll
    for (int u = 0; u < NA; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (__attribute__((address_space(3))) void*)(buf + adst[u]), 16,
                                               aoff[u], kb * kKB, 0, 0);
  };
  auto load_b = [&](BFrag<SCR_W_MXFP4, NTW>& f, int s) {
    const int ch = s / nkb, kb = s - ch * nkb;
    const int blk = ch * CT * nkb + kb;
    int tp[NTW], sp[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      tp[t] = toff0[t] + blk * 1024;
      sp[t] = soff0[t] + blk * 64;
    }
    f.load_buf(wrsrc, tp, sp, lane);
  };
  // A operand of row tile mt: row mt * 16 + col, logical chunks grp and 4 + grp
  auto read_a = [&](const uint8_t* buf, int mt) {
    const int row = mt * 16 + col;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(buf + row * 128 + 16 * (grp ^ (row & 7)));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(buf + row * 128 + 16 * ((4 + grp) ^ (row & 7)));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  f32x4 acc[MTC][NTW];

  uint32_t* const wst = stg + wave * (kWideStage / 4);
  auto epilogue = [&](int ch) {
    if (GATEUP) {
      // h = silu(g) * u for this wave's 32 h columns, g and u the accumulators
      // times a1, as E4M3 codes of h times the reciprocal of a2
      const float a1 = a.act_scale[0], r2 = 1.0f / a.act_scale[1];
      uint8_t* sh = reinterpret_cast<uint8_t*>(wst);
#pragma unroll
      for (int mt = 0; mt < MTC; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float h0 = silu_mul(a1 * acc[mt][0][i], a1 * acc[mt][NTW / 2][i]);
          const float h1 = silu_mul(a1 * acc[mt][1][i], a1 * acc[mt][NTW / 2 + 1][i]);
          sh[(grp * 4 + i) * 32 + col] = (uint8_t)e4m3_code_sat(h0 * r2);
          sh[(grp * 4 + i) * 32 + 16 + col] = (uint8_t)e4m3_code_sat(h1 * r2);
        }
        // 16 rows x 32 bytes = 32 lanes x 16 bytes
        if (lane < 32) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(sh + (lane >> 1) * 32 + (lane & 1) * 16);
          const int pos = m0 + mt * 16 + (lane >> 1);
          *reinterpret_cast<u32x4*>(a.hq + (size_t)pos * a.I + ch * (32 * EW) + wave * 32 + (lane & 1) * 16) = v;
        }
      }
    } else {
      constexpr int OC = 16 * NTW;   // output columns per wave
      static_assert(16 * OC * 4 <= kWideStage, "the fp32 tile fits the wave's stage");
      float* sf = reinterpret_cast<float*>(wst);
#pragma unroll
      for (int mt = 0; mt < MTC; ++mt) {
        // fp16 rows scaled per 32 columns, through the wave's tile as fp32
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w0 = row_w[mt * 16 + grp * 4 + i];
#pragma unroll
          for (int t = 0; t < NTW; ++t) sf[(grp * 4 + i) * OC + 16 * t + col] = w0 * acc[mt][t][i];
        }
        store_rows_f16<OC>(sf, row_route + mt * 16, lane, static_cast<uint16_t*>(a.o), a.oe, a.flags, a.H,
                           ch * (OC * EW) + wave * OC, ch == 0 && wave == 0);
      }
    }
  };

  constexpr int D = kWideRing;
  constexpr int U = D > NBUF ? D : NBUF;
  constexpr int NB = 2 * NTW;  // codes + scale per tile
  const int s0 = c_begin * nkb, s1 = c_end * nkb;
  constexpr int LA = NBUF - 1;
  BFrag<SCR_W_MXFP4, NTW> ring[D];
  constexpr bool resident = RES;
#pragma unroll
  for (int i = 0; i < LA; ++i) load_a(bufs[i], i % nkb);
  if (resident) load_a(bufs[LA], LA);
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load_b(ring[i], min(s0 + i, s1 - 1));
  if (resident)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 1) * NB));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((LA - 1) * NA + (D - 1) * NB));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  for (int ch = c_begin; ch < c_end; ++ch) {
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb0 = 0; kb0 < nkb; kb0 += U) {
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int kb = kb0 + i, s = ch * nkb + kb;
        const BFrag<SCR_W_MXFP4, NTW>& bc = ring[i % D];
        const uint8_t* buf = bufs[i % NBUF];
        if (!resident) load_a(bufs[(i + LA) % NBUF], (kb + LA) % nkb);
        load_b(ring[(i + D - 1) % D], min(s + D - 1, s1 - 1));
#pragma unroll
        for (int mt = 0; mt < MTC; ++mt) {
          const i32x8 af = read_a(buf, mt);
#pragma unroll
          for (int t = 0; t < NTW; ++t) {
            const u32x4 c4 = bc.codes[t];
            const i32x8 bf = {(int)c4[0], (int)c4[1], (int)c4[2], (int)c4[3], 0, 0, 0, 0};
            acc[mt][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf, acc[mt][t], 0, 4, 0, kUnitScale, 0,
                                                                            (int)(bc.sc[t] & 0xFFu));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!resident) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm((LA - 1) * NA + (D < LA ? D : LA) * NB));
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    epilogue(ch);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
}

template <int MT, bool GATEUP, int EW, int NTW, bool RES, int NBUF>
__global__ __launch_bounds__(64 * EW) void moe_w4a8_kernel(GemmArgs a, int groups, int pslices) {
  __shared__ __attribute__((aligned(1024))) uint8_t As0[MT * 16 * kKB];
  __shared__ __attribute__((aligned(1024))) uint8_t As1[MT * 16 * kKB];
  __shared__ __attribute__((aligned(1024))) uint8_t As2[NBUF > 2 ? MT * 16 * kKB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t As3[NBUF > 3 ? MT * 16 * kKB : 16];
  __shared__ int src_row[MT * 16];
  __shared__ int row_route[GATEUP ? 1 : MT * 16];
  __shared__ float row_w[GATEUP ? 1 : MT * 16];
  __shared__ __attribute__((aligned(256))) uint32_t stg[EW * kWideStage / 4];
  if (GATEUP) gateup_prologue(a);
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int per_bucket = groups * pslices;
  const int j = 8 * (q / per_bucket) + xcd, g = q % groups, ps = (q % per_bucket) / groups;
  if (j >= *a.n_active) return;
  const int b = a.active_buckets[j];
  const int p0 = a.active_block_begin[j] * a.B, p1 = a.active_block_begin[j + 1] * a.B;
  if (p1 > a.h_rows || p0 >= p1) return;
  constexpr int kThreads = 64 * EW;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int K = GATEUP ? a.H : a.I;
  const int nkb = K / kKB;
  const int nchunks = GATEUP ? a.I / (8 * NTW * EW) : a.H / (16 * NTW * EW);
  const int c_begin = g * nchunks / groups, c_end = (g + 1) * nchunks / groups;
  if (c_begin >= c_end) return;
  const uint8_t* rec = static_cast<const uint8_t*>(a.bucket_rows[b]);
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, (int)a.lay.record_bytes, 0x00020000);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int toff0[NTW], soff0[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int row0 = GATEUP ? (t < NTW / 2 ? 0 : a.I) + wv * 8 * NTW + 16 * (t % (NTW / 2)) : wv * 16 * NTW + 16 * t;
    const int tb = (row0 / 16) * nkb;
    toff0[t] = (int)(GATEUP ? a.lay.w13_off : a.lay.w2_off) + tb * 1024;
    soff0[t] = (int)(GATEUP ? a.lay.w13_scale_off : a.lay.w2_scale_off) + tb * 64;
  }
  for (int m0 = p0 + ps * (MT * 16); m0 < p1; m0 += pslices * (MT * 16)) {
    const int rows = min(MT * 16, p1 - m0);
    for (int i = tid; i < MT * 16; i += kThreads) {
      int off = -1;
      int r = -1;
      if (i < rows) {
        if (GATEUP) {
          r = a.sorted_routes[m0 + i];
          if (r >= 0 && r < a.R) off = (r / a.k) * K;
        } else {
          off = (m0 + i) * K;
          r = a.sorted_routes[m0 + i];
        }
      }
      src_row[i] = off;
      if (!GATEUP) {
        const bool valid = r >= 0 && r < a.R;
        row_route[i] = valid ? r : -1;
        row_w[i] = valid ? a.topk_w[r] * a.act_scale[1] : 0.0f;  // the layer's h scale folded in
      }
    }
    __syncthreads();
#define SCR_W4A8_PASS(n)                                                                                     \
  case n:                                                                                                    \
    if constexpr (MT >= n)                                                                                   \
      w4a8_pass<MT, GATEUP, EW, NTW, n, RES, NBUF>(a, src_row, row_route, row_w, As0, As1, As2, As3, stg, m0,   \
                                             wrsrc, toff0, soff0, nkb, c_begin, c_end);                        \
    break;
    switch (rows / 16) {
      SCR_W4A8_PASS(1)
      SCR_W4A8_PASS(2)
      SCR_W4A8_PASS(3)
      SCR_W4A8_PASS(4)
      SCR_W4A8_PASS(5)
      SCR_W4A8_PASS(6)
      SCR_W4A8_PASS(7)
      default: break;
    }
#undef SCR_W4A8_PASS
    __syncthreads();
  }
}

struct WsLayout {
  size_t h_off, o_off, oe_off, flags_off, act_off, bytes;
  size_t xq_off;          // W4A8: E4M3 codes of x (h_off then holds those of h)
  size_t x16_off, xe_off;  // NVFP4: x as fp16 and its row exponents; W4A4: x's decoded NVFP4 values
  int h_rows;
};

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

constexpr int kWideWaves = 8;  // two waves per SIMD in one workgroup per CU
static_assert(kWideRing == 2, "the ring steps with either buffer count");
// activation buffers of a wide GEMM over nkb K blocks: four where they come
// in fours, two where they come in pairs, 0 (the wide kernels do not fit)
static int wide_nbuf(int nkb) { return nkb % 4 == 0 ? 4 : nkb % 2 == 0 ? 2 : 0; }
template <int WDT>
struct WideNT {  // row tiles per wave: the bf16 weight ring holds four times the registers
  static constexpr int value = WDT == SCR_W_BF16 ? 2 : 4;
};

template <int WDT>
static bool wide_gemms_fit(int H, int I) {
  constexpr int NTW = WideNT<WDT>::value;
  // K blocks cycle through the LDS buffers and the two-block weight ring in
  // steps of the buffer count (four, or two): an even count of K blocks
  return wide_nbuf(H / kKB) > 0 && wide_nbuf(I / kKB) > 0 && I % (8 * NTW * kWideWaves) == 0 &&
         H % (16 * NTW * kWideWaves) == 0;
}

// Per-route rows are fp32 for bf16 weights in the few-rows kernels (the
// 96-token chunk's distance to the oracle is 1.08e-2 with them and, by CPU
// emulation, 1.19e-2 with fp16 rows, which would save 4 MB of its 1 GB) and
// the scaled fp16 rows everywhere else: every narrow format, and bf16 in the
// wide kernels, where the rows' write and the combine's read are a large share
// of a long chunk's traffic
static bool rows_f32(int wdtype, int m_chunk, int H, int I) {
  return wdtype == SCR_W_BF16 && (m_chunk == 32 || !wide_gemms_fit<SCR_W_BF16>(H, I));
}

static WsLayout ws_layout(int T, int k, int E_layer, int H, int I, int B, int m_chunk, int wdtype) {
  WsLayout w;
  const long long R = (long long)T * k;
  const long long m = R < E_layer ? R : E_layer;
  long long rows = R + m * (B - 1);
  rows = (rows + B - 1) / B * B;
  w.h_rows = (int)rows;
  w.xq_off = 0;
  w.h_off = 0;
  size_t end;
  if (wdtype == SCR_W_MXFP4_A8) {
    w.xq_off = 0;
    w.h_off = align256((size_t)T * H);
    end = w.h_off + (size_t)rows * I;
  } else {
    end = w.h_off + (size_t)rows * I * sizeof(uint16_t);
  }
  w.o_off = align256(end);
  const bool f32 = rows_f32(wdtype, m_chunk, H, I);
  const size_t row_bytes = f32 ? sizeof(float) : sizeof(uint16_t);
  // fp16 rows carry one exponent byte per kRowGroup columns
  w.oe_off = align256(w.o_off + (size_t)R * H * row_bytes);
  const size_t oe_bytes = f32 ? 0 : (size_t)R * (H / kRowGroup);
  w.flags_off = align256(w.oe_off + oe_bytes);
  w.act_off = align256(w.flags_off + (size_t)R * sizeof(int32_t));
  w.bytes = align256(w.act_off + 2 * sizeof(float));
  w.x16_off = w.xe_off = 0;
  if (wdtype == SCR_W_NVFP4 || wdtype == SCR_W_NVFP4_A4) {
    w.x16_off = w.bytes;
    w.xe_off = align256(w.x16_off + (size_t)T * H * sizeof(uint16_t));
    w.bytes = align256(w.xe_off + (size_t)T * sizeof(int32_t));
  }
  return w;
}

// Pass slices: a bucket walks its rows in passes of pass_rows, and with few
// buckets and many rows each (a small layer over a long chunk) one workgroup
// per bucket would leave most CUs idle.  The passes of a bucket are then dealt
// to pslices workgroups (slice i takes passes i, i + pslices, ...): as many as
// bring the launch to about kFillWorkgroups, at most the passes of a bucket of
// average size.  The weights are streamed once per pass either way, so the
// slices add no weight traffic; a slice past a bucket's last pass exits at
// once.
constexpr int kFillWorkgroups = 1024;
// below this many buckets one workgroup per bucket cannot fill the chip
constexpr int kFewBuckets = 256;
constexpr int kCUs = 256;  // compute units of the chip
static int pass_slices(const GemmArgs& a, int max_active, int pass_rows, int base_wgs) {
  const long long avg_rows = ((long long)a.R + max_active - 1) / max_active + a.B - 1;  // padded
  const long long avg_passes = (avg_rows + pass_rows - 1) / pass_rows;
  const long long want = (kFillWorkgroups + base_wgs - 1) / base_wgs;
  const long long ps = want < avg_passes ? want : avg_passes;
  return ps < 1 ? 1 : (int)ps;
}

// many rows per expert: both GEMMs as wide-tile workgroups, each walking a
// contiguous range of one bucket's N chunks (gate/up: one chunk of 128 h
// columns; down: two chunks of 256 output columns)
template <int WDT, int MT>
static int launch_wide_gemms(const GemmArgs& a, int max_active, hipEvent_t* marks, hipStream_t s) {
  constexpr int NTW = WideNT<WDT>::value;
  const int rows8 = (max_active + 7) / 8;  // buckets per XCD (rounded up)
  const int g_gu = a.I / (8 * NTW * kWideWaves);
  const int nch_dn = a.H / (16 * NTW * kWideWaves);
  // down: one workgroup per bucket walks all of its N chunks (its h block
  // made resident once) at many rows per expert; measured 6-14 % faster for
  // bf16, FP8 and MXFP4 at 80 rows per expert, no faster for NVFP4 (its bf16
  // weight decode dominates), which keeps two chunks per workgroup.  When
  // those workgroups (with their pass slices) could not fill the chip, the
  // chunks go to workgroups of their own instead (bf16 at 8 experts 72 ->
  // 47 us; at 64 experts the merged grid fills the chip and stays)
  const bool one_dn = WDT != SCR_W_NVFP4 && (long long)a.R >= 32ll * a.E &&
                      8 * rows8 * pass_slices(a, max_active, MT * 16, 8 * rows8) >= kCUs;
  const bool split_dn = WDT != SCR_W_NVFP4 && (long long)a.R >= 32ll * a.E && !one_dn;
  const int g_dn = one_dn ? 1 : split_dn ? nch_dn : (nch_dn >= 2 ? nch_dn / 2 : 1);
  if constexpr (WDT == SCR_W_NVFP4) {
    const int rc = launch_x_to_f16(a, s);
    if (rc) return rc;
  }
  const int ps_gu = pass_slices(a, max_active, MT * 16, 8 * rows8 * g_gu);
  const int ps_dn = pass_slices(a, max_active, MT * 16, 8 * rows8 * g_dn);
  const dim3 grid_gu(8 * rows8 * g_gu * ps_gu), grid_dn(8 * rows8 * g_dn * ps_dn), block(64 * kWideWaves);
  if (wide_nbuf(a.H / kKB) == 4)
    hipLaunchKernelGGL((moe_wide_kernel<WDT, MT, true, kWideWaves, NTW, 4>), grid_gu, block, 0, s, a, g_gu, ps_gu);
  else
    hipLaunchKernelGGL((moe_wide_kernel<WDT, MT, true, kWideWaves, NTW, 2>), grid_gu, block, 0, s, a, g_gu, ps_gu);
  SCR_CHECK_LAUNCH();
  if (marks && marks[2]) SCR_CHECK_HIP(hipEventRecord(marks[2], s));
  if (wide_nbuf(a.I / kKB) == 4)
    hipLaunchKernelGGL((moe_wide_kernel<WDT, MT, false, kWideWaves, NTW, 4>), grid_dn, block, 0, s, a, g_dn, ps_dn);
  else
    hipLaunchKernelGGL((moe_wide_kernel<WDT, MT, false, kWideWaves, NTW, 2>), grid_dn, block, 0, s, a, g_dn, ps_dn);
  SCR_CHECK_LAUNCH();
  if (marks && marks[3]) SCR_CHECK_HIP(hipEventRecord(marks[3], s));
  return SCR_OK;
}

// NTG / NTD: row tiles of 16 weight rows per wave in gate/up and in down
template <int WDT, int MT, int NTG, int NTD>
static int launch_gemms(const GemmArgs& a, int max_active, hipEvent_t* marks, hipStream_t s) {
  const int rows8 = (max_active + 7) / 8;     // buckets per XCD (rounded up)
  const int ntx_gu = (a.I + 4 * 8 * NTG - 1) / (4 * 8 * NTG);
  const int ntx_dn = (a.H + 4 * 16 * NTD - 1) / (4 * 16 * NTD);
  const int ps_gu = pass_slices(a, max_active, MT * 16, 8 * rows8 * ntx_gu);
  const int ps_dn = pass_slices(a, max_active, MT * 16, 8 * rows8 * ntx_dn);
  if constexpr (WDT == SCR_W_NVFP4) {  // x's fp16 copy for the fp16 gate/up
    const int rc = launch_x_to_f16(a, s);
    if (rc) return rc;
  }
  hipLaunchKernelGGL((moe_gemm_kernel<WDT, MT, NTG, true>), dim3(8 * rows8 * ntx_gu * ps_gu), dim3(kGemmThreads), 0,
                     s, a, ntx_gu, ps_gu);
  SCR_CHECK_LAUNCH();
  if (marks && marks[2]) SCR_CHECK_HIP(hipEventRecord(marks[2], s));
  hipLaunchKernelGGL((moe_gemm_kernel<WDT, MT, NTD, false>), dim3(8 * rows8 * ntx_dn * ps_dn), dim3(kGemmThreads), 0,
                     s, a, ntx_dn, ps_dn);
  SCR_CHECK_LAUNCH();
  if (marks && marks[3]) SCR_CHECK_HIP(hipEventRecord(marks[3], s));
  return SCR_OK;
}

// W4A8 and W4A4: the wide kernels for every row count (their 16-row passes
// serve few rows per expert as well); the shape must fit the wide tiling
static bool act_quant_fits(const GemmArgs& a, int wdtype) {
  return wdtype == SCR_W_MXFP4_A8 ? wide_gemms_fit<SCR_W_MXFP4>(a.H, a.I) : wide_gemms_fit<SCR_W_NVFP4_A4>(a.H, a.I);
}

static int launch_w4a8(const GemmArgs& a, int max_active, hipEvent_t* marks, hipStream_t s) {
  constexpr int NTW = 4;
  const int rows8 = (max_active + 7) / 8;
  // Many rows per expert: one workgroup per bucket in both GEMMs, walking all
  // of its N chunks, so the bucket's fp8 activation rows are gathered
  // (gate/up) or its h block made resident (down) once, not once per
  // workgroup (measured 3 % and 5 % faster at 80 rows per expert; the NVFP4
  // wide kernel, with its weight decode, gained nothing from it).  Few rows:
  // the chunks split over workgroups, for parallelism; and with fewer buckets
  // than CUs, every chunk a workgroup of its own (8 experts: 98 -> 69 us).
  const bool few_buckets = max_active < kFewBuckets;
  const bool many_rows = (long long)a.R >= 32ll * a.E && !few_buckets;
  const int nch_dn = a.H / (16 * NTW * kWideWaves);
  const int g_gu = many_rows ? 1 : a.I / (8 * NTW * kWideWaves);
  const int g_dn = many_rows ? 1 : few_buckets ? nch_dn : (nch_dn >= 2 ? nch_dn / 2 : 1);
  const int ps_gu = pass_slices(a, max_active, 7 * 16, 8 * rows8 * g_gu);
  const int ps_dn = pass_slices(a, max_active, 7 * 16, 8 * rows8 * g_dn);
  const dim3 grid_gu(8 * rows8 * g_gu * ps_gu), grid_dn(8 * rows8 * g_dn * ps_dn), block(64 * kWideWaves);
  if (wide_nbuf(a.H / kKB) == 4)
    hipLaunchKernelGGL((moe_w4a8_kernel<7, true, kWideWaves, NTW, false, 4>), grid_gu, block, 0, s, a, g_gu, ps_gu);
  else
    hipLaunchKernelGGL((moe_w4a8_kernel<7, true, kWideWaves, NTW, false, 2>), grid_gu, block, 0, s, a, g_gu, ps_gu);
  SCR_CHECK_LAUNCH();
  if (marks && marks[2]) SCR_CHECK_HIP(hipEventRecord(marks[2], s));
  // down: the bucket's whole h block resident in the buffers when it fits them
  const int nkb_dn = a.I / kKB, nbuf_dn = wide_nbuf(nkb_dn);
  if (nbuf_dn == 4 && nkb_dn == 4)
    hipLaunchKernelGGL((moe_w4a8_kernel<7, false, kWideWaves, NTW, true, 4>), grid_dn, block, 0, s, a, g_dn, ps_dn);
  else if (nbuf_dn == 4)
    hipLaunchKernelGGL((moe_w4a8_kernel<7, false, kWideWaves, NTW, false, 4>), grid_dn, block, 0, s, a, g_dn, ps_dn);
  else if (nkb_dn == 2)
    hipLaunchKernelGGL((moe_w4a8_kernel<7, false, kWideWaves, NTW, true, 2>), grid_dn, block, 0, s, a, g_dn, ps_dn);
  else
    hipLaunchKernelGGL((moe_w4a8_kernel<7, false, kWideWaves, NTW, false, 2>), grid_dn, block, 0, s, a, g_dn, ps_dn);
  SCR_CHECK_LAUNCH();
  if (marks && marks[3]) SCR_CHECK_HIP(hipEventRecord(marks[3], s));
  return SCR_OK;
}

// few rows per expert: the small-M kernels; many: the wide-tile kernels when
// the shape fits them, else the small-M kernels with 112-row passes
template <int WDT>
static int run_gemms(const scr_tile_cfg& cfg, const GemmArgs& a, int max_active, hipEvent_t* marks,
                     hipStream_t s) {
  // few rows: the 4-bit gate/up streams four tiles per wave (twice the weight
  // bytes per block and barrier of two; measured 13-17 % faster for NVFP4 at
  // 2-10 rows per expert, where the down measured slower that way)
  constexpr int NTG = (WDT == SCR_W_NVFP4 || WDT == SCR_W_MXFP4) ? 4 : 2;
  if (cfg.m_chunk == 32) return launch_gemms<WDT, 2, NTG, 2>(a, max_active, marks, s);
  if (wide_gemms_fit<WDT>(a.H, a.I)) return launch_wide_gemms<WDT, 7>(a, max_active, marks, s);
  return launch_gemms<WDT, 7, 2, 2>(a, max_active, marks, s);
}

// the combine, its rank group the smallest of 4, 8, 12, 16 that holds k
template <typename OT>
static void launch_combine(const OT* o, const int8_t* oe, const int32_t* flags, int T, int k, int H, void* y,
                           bool bf16_out, int grid, hipStream_t s) {
#define SCR_COMBINE(G)                                                                                          \
  if (bf16_out)                                                                                                 \
    hipLaunchKernelGGL((combine_kernel<OT, true, G>), dim3(grid), dim3(256), 0, s, o, oe, flags, T, k, H, y);  \
  else                                                                                                          \
    hipLaunchKernelGGL((combine_kernel<OT, false, G>), dim3(grid), dim3(256), 0, s, o, oe, flags, T, k, H, y);
  if (k <= 4) {
    SCR_COMBINE(4)
  } else if (k <= 8) {
    SCR_COMBINE(8)
  } else if (k <= 12) {
    SCR_COMBINE(12)
  } else {
    SCR_COMBINE(16)
  }
#undef SCR_COMBINE
}

}  // namespace scr

extern "C" int scr_tile_config(int T, int k, int E_layer, int wdtype, scr_tile_cfg* cfg) {
  SCR_CHECK_ARG(cfg != nullptr, "tile_config: cfg is null");
  SCR_CHECK_ARG(T >= 0 && k >= 1 && E_layer >= 1, "tile_config: bad T, k or E");
  SCR_CHECK_ARG(wdtype == SCR_W_BF16 || wdtype == SCR_W_NVFP4 || wdtype == SCR_W_FP8 || wdtype == SCR_W_MXFP4 ||
                    wdtype == SCR_W_MXFP4_A8 || wdtype == SCR_W_NVFP4_A4,
                "tile_config: unknown wdtype");
  // rows per expert of the routed layer (never of the bank)
  const long long per_expert = ((long long)T * k + E_layer - 1) / E_layer;
  cfg->block_m = 16;
  // few rows per expert: 32-row passes and narrow N tiles (more workgroups to
  // stream weights); many rows: 112-row passes (seven 16-row tiles, every
  // weight format) and wide N tiles (MFMA reuse)
  const bool small = per_expert <= 16;
  cfg->m_chunk = small ? 32 : 112;
  const bool four_bit = wdtype == SCR_W_NVFP4 || wdtype == SCR_W_MXFP4;
  if (small) {
    // four waves; gate/up 8 h columns per weight tile pair, down 16 columns per tile
    cfg->n_tile_gu = 4 * 8 * (four_bit ? 4 : 2);
    cfg->n_tile_dn = 4 * 16 * 2;
  } else {
    // the wide kernels' N chunk (eight waves of two or four tiles), where the
    // layer's H and I fit their tiling
    const int ntw = wdtype == SCR_W_BF16 ? 2 : 4;
    cfg->n_tile_gu = scr::kWideWaves * 8 * ntw;
    cfg->n_tile_dn = scr::kWideWaves * 16 * ntw;
  }
  cfg->wdtype = wdtype;
  return SCR_OK;
}

extern "C" int scr_moe_workspace(int T, int k, int E_layer, int H, int I, const scr_tile_cfg* cfg, size_t* bytes) {
  SCR_CHECK_ARG(cfg && bytes && T >= 0 && k >= 1 && E_layer >= 1 && H >= 1 && I >= 1,
                "moe_workspace: bad arguments");
  *bytes = scr::ws_layout(T, k, E_layer, H, I, cfg->block_m, cfg->m_chunk, cfg->wdtype).bytes;
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
  SCR_CHECK_ARG(H >= 128 && H % 128 == 0 && H <= 16384, "forward: H must be a multiple of 128 in [128, 16384]");
  SCR_CHECK_ARG(I >= 128 && I % 128 == 0 && I <= 16384, "forward: I must be a multiple of 128 in [128, 16384]");
  SCR_CHECK_ARG(view->num_buckets >= 1 && view->bucket_rows && view->input_scale, "forward: bad view");
  SCR_CHECK_ARG(view->wdtype == SCR_W_BF16 || view->wdtype == SCR_W_NVFP4 || view->wdtype == SCR_W_FP8 ||
                    view->wdtype == SCR_W_MXFP4 || view->wdtype == SCR_W_MXFP4_A8 || view->wdtype == SCR_W_NVFP4_A4,
                "forward: unknown wdtype");
  const bool act_quant = view->wdtype == SCR_W_MXFP4_A8 || view->wdtype == SCR_W_NVFP4_A4;
  SCR_CHECK_ARG(!act_quant || view->down_input_scale,
                "forward: the activation-quantising formats need the layer's down input scales");
  SCR_CHECK_ARG(y_dtype == SCR_Y_F32 || y_dtype == SCR_Y_BF16, "forward: unknown y dtype");
  SCR_CHECK_ARG(T >= 0 && (long long)T * k < (1ll << 30) && (long long)T * H < (1ll << 31),
                "forward: T out of range");
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
  const scr::WsLayout wl = scr::ws_layout(T, k, E, H, I, cfg.block_m, cfg.m_chunk, view->wdtype);
  SCR_CHECK_ARG((long long)wl.h_rows * I < (1ll << 31), "forward: T out of range");
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
  a.xq = wsb + wl.xq_off;
  a.hq = wsb + wl.h_off;
  a.x16 = reinterpret_cast<const uint16_t*>(wsb + wl.x16_off);
  a.xe = reinterpret_cast<const int32_t*>(wsb + wl.xe_off);
  a.o = wsb + wl.o_off;
  a.oe = reinterpret_cast<int8_t*>(wsb + wl.oe_off);
  a.flags = reinterpret_cast<int32_t*>(wsb + wl.flags_off);
  a.T = T;
  a.k = k;
  a.R = R;
  a.H = H;
  a.I = I;
  a.B = cfg.block_m;
  a.h_rows = wl.h_rows;

  a.input_scale = view->input_scale;
  a.down_input_scale = view->down_input_scale;
  a.a_scale_out = a_scale_out;
  a.act_scale = act_quant ? reinterpret_cast<const float*>(wsb + wl.act_off) : nullptr;
  a.E = E;
  // marks[0] and marks[1] bracket the prologue (the activation quantisation
  // of the A8/A4 formats; otherwise empty: the gate/up kernel clears the
  // flags and reports the activation scales itself)
  if (act_quant && !scr::act_quant_fits(a, view->wdtype)) {
    scr::set_error("forward: W4A8 and W4A4 need H a multiple of 512 and I of 256 (H=%d I=%d)", H, I);
    return SCR_ENOTSUP;
  }
  if (marks && marks[0]) SCR_CHECK_HIP(hipEventRecord(marks[0], stream));
  if (view->wdtype == SCR_W_MXFP4_A8) {
    rc = scr::launch_act_quant<scr::kActFp8>(a.x, T, H, view->input_scale, view->down_input_scale, E,
                                             wsb + wl.xq_off, nullptr, nullptr,
                                             reinterpret_cast<float*>(wsb + wl.act_off), a_scale_out, stream);
    if (rc) return rc;
  } else if (view->wdtype == SCR_W_NVFP4_A4) {
    rc = scr::launch_act_quant<scr::kActNvfp4F16>(a.x, T, H, view->input_scale, view->down_input_scale, E, nullptr,
                                                  nullptr, reinterpret_cast<uint16_t*>(wsb + wl.x16_off),
                                                  reinterpret_cast<float*>(wsb + wl.act_off), a_scale_out, stream);
    if (rc) return rc;
  }
  if (marks && marks[1]) SCR_CHECK_HIP(hipEventRecord(marks[1], stream));

  // the grid covers at most min(R, E_layer) active buckets: a layer size
  const int max_active = R < E ? R : E;
  switch (view->wdtype) {
    case SCR_W_BF16: rc = scr::run_gemms<SCR_W_BF16>(cfg, a, max_active, marks, stream); break;
    case SCR_W_NVFP4: rc = scr::run_gemms<SCR_W_NVFP4>(cfg, a, max_active, marks, stream); break;
    case SCR_W_FP8: rc = scr::run_gemms<SCR_W_FP8>(cfg, a, max_active, marks, stream); break;
    case SCR_W_MXFP4: rc = scr::run_gemms<SCR_W_MXFP4>(cfg, a, max_active, marks, stream); break;
    case SCR_W_NVFP4_A4: rc = scr::launch_wide_gemms<SCR_W_NVFP4_A4, 7>(a, max_active, marks, stream); break;
    default: rc = scr::launch_w4a8(a, max_active, marks, stream); break;
  }
  if (rc) return rc;

  const size_t total = (size_t)T * (H / 8);
  int cgrid = (int)((total + 255) / 256);
  if (cgrid > 4096) cgrid = 4096;
  if (!scr::rows_f32(view->wdtype, cfg.m_chunk, H, I))
    scr::launch_combine(static_cast<const uint16_t*>(a.o), a.oe, a.flags, T, k, H, y, y_dtype == SCR_Y_BF16, cgrid,
                        stream);
  else
    scr::launch_combine(static_cast<const float*>(a.o), a.oe, a.flags, T, k, H, y, y_dtype == SCR_Y_BF16, cgrid,
                        stream);
  SCR_CHECK_LAUNCH();
  if (marks && marks[4]) SCR_CHECK_HIP(hipEventRecord(marks[4], stream));
  return SCR_OK;
}

extern "C" int scr_quantize_fp8(const void* x, long long rows, int cols, const float* scales, int n_scales,
                                uint8_t* codes, hipStream_t stream) {
  SCR_CHECK_ARG(rows >= 0 && cols >= 16 && cols % 16 == 0, "quantize_fp8: cols must be a positive multiple of 16");
  SCR_CHECK_ARG(n_scales >= 1 && n_scales <= SCR_MAX_EXPERTS, "quantize_fp8: n_scales must be in [1, %d]",
                SCR_MAX_EXPERTS);
  if (rows == 0) return SCR_OK;
  SCR_CHECK_ARG(x && codes && scales, "quantize_fp8: null pointer");
  return scr::launch_act_quant<scr::kActFp8>(static_cast<const scr::bf16*>(x), rows, cols, scales, nullptr, n_scales,
                                             codes, nullptr, nullptr, nullptr, nullptr, stream);
}

extern "C" int scr_quantize_nvfp4(const void* x, long long rows, int cols, const float* scales, int n_scales,
                                  uint8_t* codes, uint8_t* block_scales, hipStream_t stream) {
  SCR_CHECK_ARG(rows >= 0 && cols >= 16 && cols % 16 == 0, "quantize_nvfp4: cols must be a positive multiple of 16");
  SCR_CHECK_ARG(n_scales >= 1 && n_scales <= SCR_MAX_EXPERTS, "quantize_nvfp4: n_scales must be in [1, %d]",
                SCR_MAX_EXPERTS);
  if (rows == 0) return SCR_OK;
  SCR_CHECK_ARG(x && codes && block_scales && scales, "quantize_nvfp4: null pointer");
  return scr::launch_act_quant<scr::kActNvfp4>(static_cast<const scr::bf16*>(x), rows, cols, scales, nullptr,
                                               n_scales, codes, block_scales, nullptr, nullptr, nullptr, stream);
}
