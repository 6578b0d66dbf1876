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

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------ NVFP4 decode
// e4m3 (OCP E4M3FN) code -> float (finite codes only)
__device__ __forceinline__ float e4m3_to_f32(unsigned c) {
  const unsigned e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0u ? (float)m * 0.001953125f  // m/8 * 2^-6
                      : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// per-route rows: fp32 for bf16 weights (their output tolerance is tighter),
// bf16 for NVFP4 weights (half the bytes at the large-chunk shapes)
template <int WDT>
struct RowT {
  typedef float type;
};
template <>
struct RowT<SCR_W_NVFP4> {
  typedef __bf16 type;
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
  void* o;              // [R][H] per-route weighted expert outputs (RowT<WDT>)
  int32_t* flags;       // [R]
  int T, k, R, H, I, B, h_rows;
};

// silu(g) * u with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// ------------------------------------------------------------ grouped GEMM
//
// One workgroup = one (active bucket, N tile).  It walks every row of its
// bucket in passes of up to MT*16 rows; per pass the K dimension is consumed
// in blocks of 128.  Activation rows (x gathered through sorted_routes for
// gate/up, contiguous h rows for down) are staged once per block in LDS and
// shared by the 4 waves; each wave streams its own weight rows straight into
// registers one block ahead and decodes NVFP4 there, so every weight byte is
// fetched and decoded once per pass.
//
// K order inside a 128-wide block (A and B use the same one, so the sum is the
// full dot product; it is fixed, so every path that runs this kernel gets the
// same bits).  MFMA step s (0..3) gives lane group g = lane / 16 eight columns:
//   bf16 : 32 s + 8 g   (the natural layout: one load = 64 B of a row)
//   NVFP4: 32 g + 8 s   (lane group g owns 32 consecutive codes = 16 B and
//                        their two e4m3 scales, so one load covers them)
constexpr int kKB = 128;               // K block
constexpr int kAStride = kKB + 8;      // LDS row stride (bf16): conflict-free b128 reads

template <int WDT>
__device__ __forceinline__ int kcol(int g, int s) {
  return WDT == SCR_W_NVFP4 ? 32 * g + 8 * s : 32 * s + 8 * g;
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
  __device__ __forceinline__ void load(const uint8_t* const* tile, const uint8_t* const*, int kb, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        raw[t][st] = ldg<u32x4>(tile[t] + (size_t)kb * 4096 + st * 1024 + lane * 16);
  }
  __device__ __forceinline__ bf16x8 get(int t, int st) const { return __builtin_bit_cast(bf16x8, raw[t][st]); }
};

template <int NT>
struct BFrag<SCR_W_NVFP4, NT> {
  u32x4 codes[NT];  // 32 codes: step s uses dword s
  unsigned sc[NT];  // two scale codes: low byte for codes 0..15, next for 16..31
  __device__ __forceinline__ void load(const uint8_t* const* tile, const uint8_t* const* stile, int kb, int lane) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      codes[t] = ldg<u32x4>(tile[t] + (size_t)kb * 1024 + lane * 16);
      sc[t] = ldg<unsigned short>(stile[t] + (size_t)kb * 128 + lane * 2);
    }
  }
  __device__ __forceinline__ bf16x8 get(int t, int st) const {
    return dequant8_hw(codes[t][st], e4m3_to_f32((sc[t] >> (8 * (st >> 1))) & 0xFFu));
  }
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
                                          const int* src_row) {
  const bf16* abase = GATEUP ? a.x : a.h;
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
  auto load_b = [&](BFrag<WDT, NT>& f, int kb) { f.load(rowp, scp, kb, c.lane); };

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
      for (int t = 0; t < NT; ++t) bf[t] = bc.get(t, st);
#pragma unroll
      for (int mt = 0; mt < MTC; ++mt) {
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(&As[buf][mt * 16 + col][kcol<WDT>(grp, st)]);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = mfma16(av, bf[t], acc[mt][t]);
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
  constexpr int D = WDT == SCR_W_NVFP4 ? 4 : 2;
  BFrag<WDT, NT> ring[D];
  AStage A0;
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load_b(ring[i], min(i, nkb - 1));
  load_a(A0, 0);
  store_a(A0, 0);
  __syncthreads();
  auto step = [&](int kb, const BFrag<WDT, NT>& bc, BFrag<WDT, NT>& bl) {
    load_a(A0, min(kb + 1, nkb - 1));
    load_b(bl, min(kb + D - 1, nkb - 1));
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
#pragma unroll
        for (int t = 0; t < NT / 2; ++t) {
          const int hc = c.ncol0 + 16 * t + col;
          const float hv = silu_mul(c.gs * acc[mt][t][i], c.gs * acc[mt][t + NT / 2][i]);
          a.h[(size_t)pos * a.I + hc] = static_cast<bf16>(hv);
        }
      } else {
        const int r = a.sorted_routes[pos];
        if (r >= 0 && r < a.R) {
          const float w = a.topk_w[r];
          typedef typename RowT<WDT>::type OT;
          OT* orow = static_cast<OT*>(a.o) + (size_t)r * a.H + c.ncol0 + col;
#pragma unroll
          for (int t = 0; t < NT; ++t) orow[16 * t] = static_cast<OT>(w * (c.gs * acc[mt][t][i]));
          if (c.tx == 0 && c.wave == 0 && col == 0) a.flags[r] = 1;
        }
      }
    }
  }
}

template <int WDT, int MT, int NT, bool GATEUP>
__global__ __launch_bounds__(kGemmThreads, 2) void moe_gemm_kernel(GemmArgs a, int ntx) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][MT * 16][kAStride];
  __shared__ int src_row[MT * 16];  // element offset of each staged row, -1 = zero row

  // XCD-aware order: consecutive workgroups go to different XCDs, so bucket j
  // and all its N tiles land on XCD (j mod 8) and share its L2
  const int bid = blockIdx.x, xcd = bid & 7, q = bid >> 3;
  const int j = 8 * (q / ntx) + xcd;
  const int tx = q % ntx;
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
  const size_t tile_bytes = WDT == SCR_W_NVFP4 ? 1024 : 4096;  // per tile-block
  if (GATEUP) {
    // tiles 0..NT/2-1: gate rows; NT/2..NT-1: the matching up rows
    c.ncol0 = tx * (4 * 8 * NT) + c.wave * (8 * NT);
    c.active = c.ncol0 < a.I;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row0 = (t < NT / 2 ? 0 : a.I) + (c.active ? c.ncol0 + 16 * (t % (NT / 2)) : 0);
      const size_t tb = (size_t)(row0 / 16) * K_blocks;
      rowp[t] = rec + a.lay.w13_off + tb * tile_bytes;
      scp[t] = rec + a.lay.w13_scale_off + tb * 128;
    }
  } else {
    c.ncol0 = tx * (4 * 16 * NT) + c.wave * (16 * NT);
    c.active = c.ncol0 < a.H;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int row0 = c.active ? c.ncol0 + 16 * t : 0;
      const size_t tb = (size_t)(row0 / 16) * K_blocks;
      rowp[t] = rec + a.lay.w2_off + tb * tile_bytes;
      scp[t] = rec + a.lay.w2_scale_off + tb * 128;
    }
  }
  c.gs = WDT == SCR_W_NVFP4 ? *reinterpret_cast<const float*>(rec + (GATEUP ? a.lay.g13_off : a.lay.g2_off))
                            : 1.0f;
  const int arow_len = K;  // elements per activation row

  for (int m0 = p0; m0 < p1; m0 += MT * 16) {
    c.m0 = m0;
    c.rows = min(MT * 16, p1 - m0);
    for (int i = c.tid; i < MT * 16; i += kGemmThreads) {
      int off = -1;
      if (i < c.rows) {
        if (GATEUP) {
          const int r = a.sorted_routes[m0 + i];
          if (r >= 0 && r < a.R) off = (r / a.k) * arow_len;
        } else {
          off = (m0 + i) * arow_len;
        }
      }
      src_row[i] = off;
    }
    __syncthreads();
    switch (c.rows / 16) {
      case 1: gemm_pass<WDT, MT, NT, GATEUP, 1>(a, c, rowp, scp, As, src_row); break;
      case 2: if constexpr (MT >= 2) gemm_pass<WDT, MT, NT, GATEUP, 2>(a, c, rowp, scp, As, src_row); break;
      case 3: if constexpr (MT >= 3) gemm_pass<WDT, MT, NT, GATEUP, 3>(a, c, rowp, scp, As, src_row); break;
      case 4: if constexpr (MT >= 4) gemm_pass<WDT, MT, NT, GATEUP, 4>(a, c, rowp, scp, As, src_row); break;
      case 5: if constexpr (MT >= 5) gemm_pass<WDT, MT, NT, GATEUP, 5>(a, c, rowp, scp, As, src_row); break;
      case 6: if constexpr (MT >= 6) gemm_pass<WDT, MT, NT, GATEUP, 6>(a, c, rowp, scp, As, src_row); break;
      case 7: if constexpr (MT >= 7) gemm_pass<WDT, MT, NT, GATEUP, 7>(a, c, rowp, scp, As, src_row); break;
      case 8: if constexpr (MT >= 8) gemm_pass<WDT, MT, NT, GATEUP, 8>(a, c, rowp, scp, As, src_row); break;
      default: break;
    }
    __syncthreads();  // src_row and As are reused by the next pass
  }
}

// ------------------------------------------------- expert-persistent GEMM
//
// For chunks with many rows per expert: one workgroup of 8 waves owns one
// active bucket and walks all of its N chunks, so the weight stream of the
// expert never restarts (the prefetch ring runs across chunk boundaries) and
// no other workgroup re-reads the bucket's activation rows for it.  A chunk
// is 256 weight rows: each wave owns NTW = 2 tiles of 16 rows (gate/up: one
// gate tile and the matching up tile, 16 h columns; down: 32 output columns).
// Down keeps the bucket's whole h block (K = I <= 512) resident in LDS for
// all chunks; gate/up stages x blocks of 128 columns double-buffered.
constexpr int kExpWaves = 8;
constexpr int kExpThreads = 64 * kExpWaves;
constexpr int kNTW = 2;
constexpr int kResMaxKB = 4;  // resident activation blocks (K <= 512)

template <int WDT, int MT, bool GATEUP, bool ARES>
struct ExpSmem {
  static constexpr int kBufs = ARES ? kResMaxKB : 2;
  bf16 As[kBufs][MT * 16 + 1][kAStride];  // the extra row takes the stores of unused staging lanes
  int src_row[MT * 16];
};

template <int WDT, int MT, bool GATEUP, bool ARES, int MTC>
__device__ __forceinline__ void expert_pass(const GemmArgs& a, ExpSmem<WDT, MT, GATEUP, ARES>& sm, int m0,
                                            const uint8_t* const* tile0, const uint8_t* const* stile0,
                                            float gs, int nkb, int nchunks) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const bf16* abase = GATEUP ? a.x : a.h;
  constexpr int kRowChunks = kKB / 8;
  constexpr int kChunks = MTC * 16 * kRowChunks;
  constexpr int kPerThread = (kChunks + kExpThreads - 1) / kExpThreads;
  constexpr int CT = GATEUP ? kExpWaves * kNTW / 2 : kExpWaves * kNTW;  // row tiles per chunk and tensor half
  constexpr size_t tile_bytes = WDT == SCR_W_NVFP4 ? 1024 : 4096;

  // staging addresses of this thread (fixed for the pass)
  const bf16* asrc[kPerThread];
  bool avalid[kPerThread];
  int adst[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int ci = u * kExpThreads + tid;
    const bool in = ci < kChunks;
    const int r = in ? ci / kRowChunks : 0, ch = ci % kRowChunks;
    const int off = sm.src_row[r];
    avalid[u] = in && off >= 0;
    asrc[u] = abase + (off >= 0 ? off : 0) + ch * 8;
    adst[u] = (in ? r : MT * 16) * kAStride + ch * 8;
  }
  struct AStage {
    u32x4 v[kPerThread];
  };
  auto load_a = [&](AStage& st, int kb) {
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) st.v[u] = ldg<u32x4>(asrc[u] + kb * kKB);
  };
  auto store_a = [&](const AStage& st, int buf) {
    bf16* base = &sm.As[buf][0][0];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(base + adst[u]) = avalid[u] ? st.v[u] : z;
    }
  };
  // weights of flat step s = chunk * nkb + kb
  auto load_b = [&](BFrag<WDT, kNTW>& f, int s) {
    const int ch = s / nkb, kb = s - ch * nkb;
    const size_t blk = (size_t)ch * CT * nkb + kb;
    const uint8_t* tp[kNTW];
    const uint8_t* sp[kNTW];
#pragma unroll
    for (int t = 0; t < kNTW; ++t) {
      tp[t] = tile0[t] + blk * tile_bytes;
      sp[t] = stile0[t] + blk * 128;
    }
    f.load(tp, sp, 0, lane);
  };

  f32x4 acc[MTC][kNTW];
  auto zero_acc = [&]() {  // (defined before use below)
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt)
#pragma unroll
      for (int t = 0; t < kNTW; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto compute = [&](const BFrag<WDT, kNTW>& bc, int buf) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 bf[kNTW];
#pragma unroll
      for (int t = 0; t < kNTW; ++t) bf[t] = bc.get(t, st);
#pragma unroll
      for (int mt = 0; mt < MTC; ++mt) {
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(&sm.As[buf][mt * 16 + col][kcol<WDT>(grp, st)]);
#pragma unroll
        for (int t = 0; t < kNTW; ++t) acc[mt][t] = mfma16(av, bf[t], acc[mt][t]);
      }
    }
  };
  auto epilogue = [&](int ch) {
#pragma unroll
    for (int mt = 0; mt < MTC; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = m0 + mt * 16 + grp * 4 + i;
        if (GATEUP) {
          constexpr int HW = 8 * kNTW;  // h columns per wave
#pragma unroll
          for (int t = 0; t < kNTW / 2; ++t) {
            const int hc = ch * (HW * kExpWaves) + wave * HW + 16 * t + col;
            const float hv = silu_mul(gs * acc[mt][t][i], gs * acc[mt][t + kNTW / 2][i]);
            a.h[(size_t)pos * a.I + hc] = static_cast<bf16>(hv);
          }
        } else {
          const int r = a.sorted_routes[pos];
          if (r >= 0 && r < a.R) {
            const float w = a.topk_w[r];
            typedef typename RowT<WDT>::type OT;
            OT* orow = static_cast<OT*>(a.o) + (size_t)r * a.H + ch * (16 * kNTW * kExpWaves) + wave * 16 * kNTW + col;
#pragma unroll
            for (int t = 0; t < kNTW; ++t) orow[16 * t] = static_cast<OT>(w * (gs * acc[mt][t][i]));
            if (ch == 0 && wave == 0 && col == 0) a.flags[r] = 1;
          }
        }
      }
    }
  };

  const int S = nchunks * nkb;  // flat steps s = chunk * nkb + kb
  constexpr int D = WDT == SCR_W_NVFP4 ? 4 : 2;  // the launcher guarantees nkb % D == 0
  BFrag<WDT, kNTW> ring[D];
#pragma unroll
  for (int i = 0; i < D - 1; ++i) load_b(ring[i], min(i, S - 1));
  AStage A0;
  if (ARES) {
    // the whole K of the bucket's rows, once for all chunks (two blocks in flight)
    AStage A1;
    for (int b = 0; b < nkb; b += 2) {
      load_a(A0, b);
      if (b + 1 < nkb) load_a(A1, b + 1);
      store_a(A0, b);
      if (b + 1 < nkb) store_a(A1, b + 1);
    }
  } else {
    load_a(A0, 0);
    store_a(A0, 0);
  }
  __syncthreads();
  auto step = [&](int s, int kb, const BFrag<WDT, kNTW>& bc, BFrag<WDT, kNTW>& bl) {
    if (!ARES) load_a(A0, (s + 1) % nkb);  // next step's activation block
    load_b(bl, min(s + D - 1, S - 1));
    compute(bc, ARES ? kb : (s & 1));
    if (!ARES) {
      store_a(A0, (s + 1) & 1);
      __syncthreads();
    }
  };
  for (int ch = 0; ch < nchunks; ++ch) {
    zero_acc();
    for (int kb0 = 0; kb0 < nkb; kb0 += D) {
#pragma unroll
      for (int i = 0; i < D; ++i) step(ch * nkb + kb0 + i, kb0 + i, ring[i], ring[(i + D - 1) % D]);
    }
    epilogue(ch);
  }
}

template <int WDT, int MT, bool GATEUP, bool ARES>
__global__ __launch_bounds__(kExpThreads) void moe_expert_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) ExpSmem<WDT, MT, GATEUP, ARES> sm;
  // XCD-aware order: bucket j runs on XCD j mod 8
  const int bid = blockIdx.x, j = 8 * (bid >> 3) + (bid & 7);
  if (j >= *a.n_active) return;
  const int b = a.active_buckets[j];
  const int p0 = a.active_block_begin[j] * a.B, p1 = a.active_block_begin[j + 1] * a.B;
  if (p1 > a.h_rows || p0 >= p1) return;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int K = GATEUP ? a.H : a.I;
  const int nkb = K / kKB;
  const int nchunks = GATEUP ? a.I / (8 * kNTW * kExpWaves) : a.H / (16 * kNTW * kExpWaves);
  const uint8_t* rec = static_cast<const uint8_t*>(a.bucket_rows[b]);
  constexpr size_t tile_bytes = WDT == SCR_W_NVFP4 ? 1024 : 4096;
  // tile-block (t, 0) of this wave's tiles in chunk 0
  const uint8_t* tile0[kNTW];
  const uint8_t* stile0[kNTW];
#pragma unroll
  for (int t = 0; t < kNTW; ++t) {
    const int row0 = GATEUP ? (t < kNTW / 2 ? 0 : a.I) + wave * 8 * kNTW + 16 * (t % (kNTW / 2))
                            : wave * 16 * kNTW + 16 * t;
    const size_t tb = (size_t)(row0 / 16) * nkb;
    tile0[t] = rec + (GATEUP ? a.lay.w13_off : a.lay.w2_off) + tb * tile_bytes;
    stile0[t] = rec + (GATEUP ? a.lay.w13_scale_off : a.lay.w2_scale_off) + tb * 128;
  }
  const float gs = WDT == SCR_W_NVFP4
                       ? *reinterpret_cast<const float*>(rec + (GATEUP ? a.lay.g13_off : a.lay.g2_off))
                       : 1.0f;
  for (int m0 = p0; m0 < p1; m0 += MT * 16) {
    const int rows = min(MT * 16, p1 - m0);
    for (int i = tid; i < MT * 16; i += kExpThreads) {
      int off = -1;
      if (i < rows) {
        if (GATEUP) {
          const int r = a.sorted_routes[m0 + i];
          if (r >= 0 && r < a.R) off = (r / a.k) * K;
        } else {
          off = (m0 + i) * K;
        }
      }
      sm.src_row[i] = off;
    }
    __syncthreads();
    switch (rows / 16) {
      case 1: expert_pass<WDT, MT, GATEUP, ARES, 1>(a, sm, m0, tile0, stile0, gs, nkb, nchunks); break;
      case 2: if constexpr (MT >= 2) expert_pass<WDT, MT, GATEUP, ARES, 2>(a, sm, m0, tile0, stile0, gs, nkb, nchunks); break;
      case 3: if constexpr (MT >= 3) expert_pass<WDT, MT, GATEUP, ARES, 3>(a, sm, m0, tile0, stile0, gs, nkb, nchunks); break;
      case 4: if constexpr (MT >= 4) expert_pass<WDT, MT, GATEUP, ARES, 4>(a, sm, m0, tile0, stile0, gs, nkb, nchunks); break;
      case 5: if constexpr (MT >= 5) expert_pass<WDT, MT, GATEUP, ARES, 5>(a, sm, m0, tile0, stile0, gs, nkb, nchunks); break;
      case 6: if constexpr (MT >= 6) expert_pass<WDT, MT, GATEUP, ARES, 6>(a, sm, m0, tile0, stile0, gs, nkb, nchunks); break;
      default: break;
    }
    __syncthreads();  // src_row and As are reused by the next pass
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
// y[t][c] = sum_j o[t*k + j][c] in rank order j, in fp32 (unwritten routes
// count as zero); 8 columns per thread
__device__ __forceinline__ void load_row8(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load_row8(const bf16* p, float* v) {
  const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
  }
}

template <typename OT, bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const OT* __restrict__ o,
                                                      const int32_t* __restrict__ flags, int T, int k,
                                                      int H, void* __restrict__ y) {
  const int h8 = H / 8;
  const size_t total = (size_t)T * h8;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / h8), c8 = (int)(i % h8);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = t * k + j;
      if (!flags[r]) continue;
      float v[8];
      load_row8(o + (size_t)r * H + 8 * c8, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
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

struct WsLayout {
  size_t h_off, o_off, flags_off, bytes;
  int h_rows;
};

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

static WsLayout ws_layout(int T, int k, int E_layer, int H, int I, int B, int wdtype) {
  WsLayout w;
  const long long R = (long long)T * k;
  const long long m = R < E_layer ? R : E_layer;
  long long rows = R + m * (B - 1);
  rows = (rows + B - 1) / B * B;
  w.h_rows = (int)rows;
  w.h_off = 0;
  w.o_off = align256(w.h_off + (size_t)rows * I * sizeof(uint16_t));
  const size_t row_bytes = wdtype == SCR_W_NVFP4 ? sizeof(uint16_t) : sizeof(float);
  w.flags_off = align256(w.o_off + (size_t)R * H * row_bytes);
  w.bytes = align256(w.flags_off + (size_t)R * sizeof(int32_t));
  return w;
}

template <int WDT, int MT>
static bool expert_gemms_fit(const GemmArgs& a) {
  constexpr int D = WDT == SCR_W_NVFP4 ? 4 : 2;
  return (a.H / kKB) % D == 0 && (a.I / kKB) % D == 0 && a.I % (8 * kNTW * kExpWaves) == 0 &&
         a.H % (16 * kNTW * kExpWaves) == 0;
}

// many rows per expert: gate/up as (bucket, N tile) workgroups (measured
// faster for the long K = H loop), down as one expert-persistent workgroup per
// bucket with its h rows resident in LDS
template <int WDT, int MT>
static int launch_expert_gemms(const GemmArgs& a, int max_active, hipEvent_t* marks, hipStream_t s) {
  const int grid = 8 * ((max_active + 7) / 8);
  const int ntx_gu = (a.I + 4 * 8 * 2 - 1) / (4 * 8 * 2);
  hipLaunchKernelGGL((moe_gemm_kernel<WDT, MT, 2, true>), dim3(grid * ntx_gu), dim3(kGemmThreads), 0, s, a, ntx_gu);
  SCR_CHECK_LAUNCH();
  if (marks && marks[2]) SCR_CHECK_HIP(hipEventRecord(marks[2], s));
  if (a.I / kKB <= kResMaxKB)
    hipLaunchKernelGGL((moe_expert_kernel<WDT, MT, false, true>), dim3(grid), dim3(kExpThreads), 0, s, a);
  else
    hipLaunchKernelGGL((moe_expert_kernel<WDT, MT, false, false>), dim3(grid), dim3(kExpThreads), 0, s, a);
  SCR_CHECK_LAUNCH();
  if (marks && marks[3]) SCR_CHECK_HIP(hipEventRecord(marks[3], s));
  return SCR_OK;
}

template <int WDT, int MT, int NT>
static int launch_gemms(const GemmArgs& a, int max_active, hipEvent_t* marks, hipStream_t s) {
  const int rows8 = (max_active + 7) / 8;     // buckets per XCD (rounded up)
  const int ntx_gu = (a.I + 4 * 8 * NT - 1) / (4 * 8 * NT);
  const int ntx_dn = (a.H + 4 * 16 * NT - 1) / (4 * 16 * NT);
  hipLaunchKernelGGL((moe_gemm_kernel<WDT, MT, NT, true>), dim3(8 * rows8 * ntx_gu), dim3(kGemmThreads), 0, s, a,
                     ntx_gu);
  SCR_CHECK_LAUNCH();
  if (marks && marks[2]) SCR_CHECK_HIP(hipEventRecord(marks[2], s));
  hipLaunchKernelGGL((moe_gemm_kernel<WDT, MT, NT, false>), dim3(8 * rows8 * ntx_dn), dim3(kGemmThreads), 0, s, a,
                     ntx_dn);
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
  // few rows per expert: small M passes and narrow N tiles (more workgroups to
  // stream weights); many rows: 128-row passes and wide N tiles (MFMA reuse)
  const bool small = per_expert <= 16;
  cfg->m_chunk = small ? 32 : 96;
  cfg->n_tile_gu = 4 * 8 * 2;    // h columns per workgroup
  cfg->n_tile_dn = 4 * 16 * 2;   // output columns per workgroup
  cfg->wdtype = wdtype;
  return SCR_OK;
}

extern "C" int scr_moe_workspace(int T, int k, int E_layer, int H, int I, const scr_tile_cfg* cfg, size_t* bytes) {
  SCR_CHECK_ARG(cfg && bytes && T >= 0 && k >= 1 && E_layer >= 1 && H >= 1 && I >= 1,
                "moe_workspace: bad arguments");
  *bytes = scr::ws_layout(T, k, E_layer, H, I, cfg->block_m, cfg->wdtype).bytes;
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
  SCR_CHECK_ARG(view->wdtype == SCR_W_BF16 || view->wdtype == SCR_W_NVFP4, "forward: unknown wdtype");
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
  const scr::WsLayout wl = scr::ws_layout(T, k, E, H, I, cfg.block_m, view->wdtype);
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
  a.o = wsb + wl.o_off;
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
    rc = cfg.m_chunk == 32                              ? scr::launch_gemms<SCR_W_BF16, 2, 2>(a, max_active, marks, stream)
         : scr::expert_gemms_fit<SCR_W_BF16, 6>(a) ? scr::launch_expert_gemms<SCR_W_BF16, 6>(a, max_active, marks, stream)
                                                    : scr::launch_gemms<SCR_W_BF16, 6, 2>(a, max_active, marks, stream);
  } else {
    rc = cfg.m_chunk == 32                               ? scr::launch_gemms<SCR_W_NVFP4, 2, 2>(a, max_active, marks, stream)
         : scr::expert_gemms_fit<SCR_W_NVFP4, 6>(a) ? scr::launch_expert_gemms<SCR_W_NVFP4, 6>(a, max_active, marks, stream)
                                                     : scr::launch_gemms<SCR_W_NVFP4, 6, 2>(a, max_active, marks, stream);
  }
  if (rc) return rc;

  const size_t total = (size_t)T * (H / 8);
  int cgrid = (int)((total + 255) / 256);
  if (cgrid > 4096) cgrid = 4096;
  if (view->wdtype == SCR_W_NVFP4) {
    const scr::bf16* o = static_cast<const scr::bf16*>(a.o);
    if (y_dtype == SCR_Y_BF16)
      hipLaunchKernelGGL((scr::combine_kernel<scr::bf16, true>), dim3(cgrid), dim3(256), 0, stream, o, a.flags, T, k, H, y);
    else
      hipLaunchKernelGGL((scr::combine_kernel<scr::bf16, false>), dim3(cgrid), dim3(256), 0, stream, o, a.flags, T, k, H, y);
  } else {
    const float* o = static_cast<const float*>(a.o);
    if (y_dtype == SCR_Y_BF16)
      hipLaunchKernelGGL((scr::combine_kernel<float, true>), dim3(cgrid), dim3(256), 0, stream, o, a.flags, T, k, H, y);
    else
      hipLaunchKernelGGL((scr::combine_kernel<float, false>), dim3(cgrid), dim3(256), 0, stream, o, a.flags, T, k, H, y);
  }
  SCR_CHECK_LAUNCH();
  if (marks && marks[4]) SCR_CHECK_HIP(hipEventRecord(marks[4], stream));
  return SCR_OK;
}
