// Common device helpers for libdgstep (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dgstep.h"

namespace dg {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even, as the storage rounding of a bf16 tensor.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = (u >> 16) | 0x40u;                       // NaN stays a (quiet) NaN
  return static_cast<bf16_t>((u & 0x7fffffffu) > 0x7f800000u ? qnan : rne);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// ------------------------------------------------------------ MFMA fragments
//
// One 16x16x32 step.  Lane l supplies row (A) / column (B) l % 16 and eight
// consecutive k values [8*(l/16), 8*(l/16)+8) of the 32-wide k slice.  A and B
// use the same k assignment, so the product is the plain sum over k.  The
// fp32 accumulator of lane l holds C[4*(l/16) + i][l % 16], i = 0..3.

template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16_t *p) { v = *reinterpret_cast<const bf16x8 *>(p); }
  __device__ __forceinline__ void zero() {
    uint4 z = make_uint4(0, 0, 0, 0);
    v = *reinterpret_cast<bf16x8 *>(&z);
  }
  // keep the fragment (mask all ones) or zero it (mask 0) without a branch
  __device__ __forceinline__ void mask(uint32_t m) {
    uint4 u = *reinterpret_cast<uint4 *>(&v);
    u.x &= m; u.y &= m; u.z &= m; u.w &= m;
    v = *reinterpret_cast<bf16x8 *>(&u);
  }
  __device__ __forceinline__ void from_floats(const float *f) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = static_cast<uint32_t>(f32_to_bf16(f[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(f[2 * j + 1])) << 16);
    v = *reinterpret_cast<bf16x8 *>(w);
  }
};

template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void load(const float *p) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.f;
  }
  __device__ __forceinline__ void mask(uint32_t m) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) & m);
  }
  __device__ __forceinline__ void from_floats(const float *f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = f[j];
  }
};

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

// fp32 path: eight 16x16x4 steps, step j taking element j of every lane, so the
// k assignment matches the bf16 path.
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// ------------------------------------------------ row-contiguous fragments
//
// A 16-row x 64-deep bf16 block (two 32-wide k slices) loaded with whole
// 128-byte row segments instead of the fragment order: with lane l = 16g + r,
// load 0 takes row r%8 and load 1 row 8 + r%8, both at 16-byte chunk
// 4*(r/8) + g.  Each load then covers 8 full rows (8 cache lines instead of
// 16 half lines).  Fragment 0 (chunks 0-3) needs row r, chunk g at lane l:
// lanes r < 8 of load 0 hold it, lanes r >= 8 take load 1 from lane l-8;
// fragment 1 (chunks 4-7) keeps load 1 in lanes r >= 8 and takes load 0
// from lane l+8 in lanes r < 8.  Both moves are DPP row shifts by 8 inside
// each 16-lane row, restricted to half the row by the bank mask.

// lane offsets of the two loads inside a 16-row block: row (r%8) [+8], byte chunk
__device__ __forceinline__ int contig_row(int lane) { return (lane & 15) & 7; }
__device__ __forceinline__ int contig_chunk(int lane) { return ((lane & 15) >> 3) * 4 + (lane >> 4); }

__device__ __forceinline__ void contig_to_frags(const bf16x8 &x0, const bf16x8 &x1, bf16x8 &f0, bf16x8 &f1) {
  int a[4], b[4], o0[4], o1[4];
  __builtin_memcpy(a, &x0, 16);
  __builtin_memcpy(b, &x1, 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o0[j] = __builtin_amdgcn_update_dpp(a[j], b[j], 0x118 /* row_shr:8 */, 0xF, 0xC, false);
    o1[j] = __builtin_amdgcn_update_dpp(b[j], a[j], 0x108 /* row_shl:8 */, 0xF, 0x3, false);
  }
  __builtin_memcpy(&f0, o0, 16);
  __builtin_memcpy(&f1, o1, 16);
}

// 1: the XCD-aware tile numbering for grids of any size (0: multiples of 8 only)
#ifndef DG_XCD_ANY_GRID
#define DG_XCD_ANY_GRID 1
#endif
// Workgroup b of a grid of `total` runs on XCD b % 8.  Logical tile numbers
// that keep neighbours on one XCD (one L2): XCD x takes the contiguous block
// [x*q + min(x, r), ...) of q + (x < r) numbers, q = total / 8, r = total % 8
// (a permutation of [0, total) for any total).
__device__ __forceinline__ int xcd_tile(int b, int total) {
  if (!DG_XCD_ANY_GRID && (total & 7)) return b;
  const int q = total >> 3, r = total & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// 16-byte vector of T elements.
template <typename T> struct Vec16 { static constexpr int n = 16 / sizeof(T); };

__device__ __forceinline__ void load8(const bf16_t *p, float *f) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float *p, float *f) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void store8(bf16_t *p, const float *f) {
  uint4 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(f[0])) | (static_cast<uint32_t>(f32_to_bf16(f[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(f[2])) | (static_cast<uint32_t>(f32_to_bf16(f[3])) << 16);
  u.z = static_cast<uint32_t>(f32_to_bf16(f[4])) | (static_cast<uint32_t>(f32_to_bf16(f[5])) << 16);
  u.w = static_cast<uint32_t>(f32_to_bf16(f[6])) | (static_cast<uint32_t>(f32_to_bf16(f[7])) << 16);
  *reinterpret_cast<uint4 *>(p) = u;
}
__device__ __forceinline__ void store8(float *p, const float *f) {
  reinterpret_cast<float4 *>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4 *>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}


// Online softmax statistics of a set of values x (x = logit / t): m = max x,
// Z = sum exp(x - m), S = sum exp(x - m) (x - m).  merge_row_stats folds
// (m2, Z2, S2) into (m, Z, S); a side whose m is -inf holds no value yet.
__device__ __forceinline__ void merge_row_stats(float &m, float &Z, float &S, float m2, float Z2, float S2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    Z = Z2;
    S = S2;
    return;
  }
  if (m2 > m) {
    const float sc = __expf(m - m2);
    S = sc * (S + (m - m2) * Z) + S2;
    Z = sc * Z + Z2;
    m = m2;
  } else {
    const float sc = __expf(m2 - m);
    S = S + sc * (S2 + (m2 - m) * Z2);
    Z = Z + sc * Z2;
  }
}

// Keep the larger value, the lower index on ties (a NaN is never taken).
__device__ __forceinline__ void better_of(float &bv, int &bi, float v, int i) {
  const bool take = v > bv || (v == bv && i < bi);
  bv = take ? v : bv;
  bi = take ? i : bi;
}

}  // namespace dg

// ------------------------------------------------------------ host launchers
// Implemented in the kernel translation units; all return hipError_t.
namespace dg {

enum EpiMode {
  EPI_STORE = 0,       // C (T)   = acc
  EPI_STORE_F32 = 1,   // C (f32) = acc
  EPI_ADD = 2,         // C (T)   = T(C + acc)          (residual add)
  EPI_SWIGLU = 3,      // C (T)   = T(silu(acc0) * acc1) (dual B)
  EPI_ROWSCALE_F32 = 4,// C (f32) = acc * rowscale[row]
  EPI_PARTIAL_F32 = 5  // C (f32)[split][row][col] = acc  (split-K partials)
};

struct GemmArgs {
  // A operand: logical row r reads physical row a_rows ? a_rows[r] : r.
  const void *A;
  long long lda;
  const int *a_rows;
  // B operand ([N][K] rows, i.e. y = x B^T).  Dense: up to 4 column segments
  // (seg_start ascending, seg_start[nseg] = N), each with its own matrix.
  int nseg;
  int seg_start[5];
  const void *seg_B0[4];
  const void *seg_B1[4];  // second matrix for the dual (SwiGLU) mode
  long long ldb;
  // Grouped mode (g_off != nullptr): groups 0..n_xgroups-1 (row chunks of the
  // shared expert) use (Bx0, Bx1, N_x); groups n_xgroups..n_groups-1 use
  // B0 + (g-n_xgroups)*b_gstride (and B1) with N columns.  Rows of group g
  // are logical rows [g_off[g], g_off[g+1]).
  const int *g_off;
  int n_groups;
  int n_xgroups;
  const void *Bx0, *Bx1;
  int N_x, K_x;           // group 0 columns and depth
  long long ldb_x;        // group 0 weight row stride
  long long b_gstride;
  // sizes
  int M, N, K;
  int k_splits;     // split-K count (dense only); K % (64 * k_splits) == 0
  // output
  void *C;
  long long ldc;
  const float *rowscale;
  int tile_order;   // 0: consecutive tiles share B columns (m fastest), 1: share A rows (n fastest)
  // fp8 weights (launch_gemm_f8_grouped): one fp32 scale per weight row;
  // routed expert e's rows scale by bs0/bs1 + e*N, the shared expert's by bxs0/bxs1
  const float *bs0, *bs1, *bxs0, *bxs1;
};

template <typename T>
hipError_t launch_gemm(const GemmArgs &a, int mode, int bm, int bn, hipStream_t s);
// Grouped expert product with OCP E4M3 weights ([N][K] bytes per expert) and
// bf16 activations; mode EPI_SWIGLU or EPI_ROWSCALE_F32, mt = 2 or 4.
hipError_t launch_gemm_f8_grouped(const GemmArgs &a, int mode, int mt, hipStream_t s);
// The expert gate/up product (SwiGLU epilogue) with fp8 weights in the
// wide-tile form: 16*DG_WMOE_MT rows x 64 columns of both matrices, four
// waves sharing each activation stage through LDS.  Returns
// hipErrorNotSupported unless K and K_x are multiples of 128, the weight
// rows 16-byte aligned and every scale pointer given.
hipError_t launch_gemm_wide_f8_gu(const GemmArgs &a, hipStream_t s);
#ifndef DG_WIDE_F8_GU
#define DG_WIDE_F8_GU 1
#endif
#ifndef DG_F8_NT_GU
#define DG_F8_NT_GU 2
#endif
#ifndef DG_F8_NT_DN
#define DG_F8_NT_DN 4
#endif
#ifndef DG_F8_S
#define DG_F8_S 2
#endif
// Tile shapes of the streaming products (in 16x16 MFMA tiles) and ring depth.
#ifndef DG_DENSE_MT
#define DG_DENSE_MT 4
#endif
#ifndef DG_DENSE_NT
#define DG_DENSE_NT 4
#endif
#ifndef DG_DENSE_S
#define DG_DENSE_S 3
#endif
#ifndef DG_MOE_MT
#define DG_MOE_MT 2
#endif
#ifndef DG_MOE_NT_GU
#define DG_MOE_NT_GU 2
#endif
#ifndef DG_MOE_NT_DN
#define DG_MOE_NT_DN 4
#endif
#ifndef DG_CONTIG
#define DG_CONTIG 1
#endif
#ifndef DG_DN_MT
#define DG_DN_MT DG_MOE_MT
#endif
#ifndef DG_GU_S
#define DG_GU_S 3
#endif
#ifndef DG_MOE_S
#define DG_MOE_S 4
#endif

// Expert down product with several (group, column tile, row block) items per
// workgroup and the load ring carried across items: bf16 weights (5..12
// stages of 64) or E4M3 weights with per-row scales (fp8: 5..8 stages of
// 128, the last one possibly 64 deep), grouped mode, mt == DG_DN_MT,
// K == K_x.  Returns hipErrorNotSupported for other shapes (the caller then
// uses the streaming kernel).  DG_DN_RING_WG resident workgroups stride
// through the items.
hipError_t launch_gemm_down_ring(const GemmArgs &a, int mt, bool fp8, hipStream_t s);
#ifndef DG_DN_RING
#define DG_DN_RING 1
#endif
#ifndef DG_DN_RING_WG
#define DG_DN_RING_WG 512
#endif
// streaming variant: tile (16*mt) x (16*nt), waves split k (K per split a multiple of 32)
template <typename T>
hipError_t launch_gemm_stream(const GemmArgs &a, int mode, int mt, int nt, hipStream_t s);
// Wide-tile bf16 products (A shared through LDS by the workgroup's waves).
enum WideCfg {
  WIDE_ROWS256_N256 = 0,  // 256 x 256 tile, 8 waves x 32 columns
  WIDE_ROWS256_N128 = 1,  // 256 x 128 tile, 8 waves x 16 columns
  WIDE_EXPERT_GU = 2,     // expert gate/up: 16*DG_WMOE_MT rows x 64 columns (x2 matrices), 4 waves
  WIDE_EXPERT_DN = 3,     // expert down: 16*DG_WMOE_MT rows x 128 columns, 4 waves
  WIDE_EXPERT_GU_L = 4,   // expert gate/up, long groups: 256 rows x 128 columns (x2 matrices), 8 waves
  WIDE_EXPERT_DN_L = 5,   // expert down, long groups: 256 rows x 128 columns, 8 waves
  WIDE_ROWS256_N128_OP = 6,  // the 256 x 128 form with DG_OPROJ_P weight stages ahead (output projection)
  // every configuration walks k in stages of 64
};
// 1: the wide-tile loops issue each stage's global loads ahead of its MFMAs
// (a scheduling barrier after the loads)
#ifndef DG_LOAD_FENCE
#define DG_LOAD_FENCE 1
#endif
#ifndef DG_WIDE_P
#define DG_WIDE_P 3
#endif
#ifndef DG_WIDE_PA
#define DG_WIDE_PA 1
#endif
// weight stages in flight for the output projection (deeper rings measured
// faster for Q|K|V, slower for O-proj)
#ifndef DG_OPROJ_P
#define DG_OPROJ_P 2
#endif
#ifndef DG_WIDE256_P
#define DG_WIDE256_P 2
#endif
#ifndef DG_HEAD_CFG
#define DG_HEAD_CFG WIDE_ROWS256_N256
#endif
#ifndef DG_SOFT_CFG
#define DG_SOFT_CFG WIDE_ROWS256_N256
#endif
#ifndef DG_PROJ_WIDE
#define DG_PROJ_WIDE 1
#endif
#ifndef DG_PROJ_CFG
#define DG_PROJ_CFG WIDE_ROWS256_N128
#endif
#ifndef DG_PROJ_TARGET
#define DG_PROJ_TARGET 256
#endif
#ifndef DG_WIDE_EXPERTS
#define DG_WIDE_EXPERTS 0
#endif
#ifndef DG_WIDE_EXPERTS_GU
#define DG_WIDE_EXPERTS_GU 1
#endif
#ifndef DG_WMOE_MT
#define DG_WMOE_MT 2
#endif
// 1: the grouped wide-tile products with 32-row tiles number their (group,
// column tile) items so that each XCD takes a contiguous run of them
#ifndef DG_GROUPED_XCD
#define DG_GROUPED_XCD 1
#endif
// expert groups averaging more rows than this use the 256-row configurations
// router product: split-K partials, summed in split order by the top-k pass
#ifndef DG_ROUTER_KS
#define DG_ROUTER_KS 4
#endif
#ifndef DG_WIDE_EXPERTS_L
#define DG_WIDE_EXPERTS_L 48
#endif
#ifndef DG_WMOE_P
#define DG_WMOE_P 3
#endif
// activation prefetch depth (stages) of the expert gate/up configuration
#ifndef DG_WMOE_PA
#define DG_WMOE_PA 2
#endif
// column tile width and k-stage depth of each wide configuration
inline int wide_bn(int cfg) { return cfg == WIDE_ROWS256_N256 ? 256 : (cfg == WIDE_EXPERT_GU ? 64 : 128); }
inline int wide_bm(int cfg) {
  return (cfg <= WIDE_ROWS256_N128 || cfg >= WIDE_EXPERT_GU_L) ? 256 : 16 * DG_WMOE_MT;   // _N128_OP too
}
inline int wide_kstage(int) { return 64; }
hipError_t launch_gemm_wide(const GemmArgs &a, int mode, int cfg, hipStream_t s);

template <typename T>
hipError_t launch_splitk_reduce(const float *part, int splits, int M, int N, long long ldc,
                                void *C, int mode, hipStream_t s);

}  // namespace dg
