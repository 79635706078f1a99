// Matrix products y = x W^T on bf16/fp32 MFMA (gfx950).
//
// Every product of the step has a weight operand W [N][K] that is streamed
// from HBM exactly once per output tile, and a narrow activation operand
// (256 canvas rows, or the few rows routed to one expert).  The kernel stages
// the activation tile (A) through LDS, where the four waves of a workgroup
// share it, and streams each wave's own weight columns (B) from global memory
// straight into MFMA fragment registers, one 64-wide k stage ahead of use.
//
// Modes: dense (tiles over M x N, optional split-K, up to four weight
// segments side by side, e.g. the Q|K|V projections) and grouped (one group
// per expert: rows gathered by token index, one weight matrix per group,
// workgroup loops over the group's row tiles).  Epilogues: store, residual
// add, SwiGLU of two products (expert gate/up), per-row scale (routing
// weight) and split-K partials.
#include "dg_common.h"

namespace dg {

namespace {

constexpr int kBK = 64;  // k elements per LDS stage (two 32-wide MFMA steps)

#ifndef DG_RING_MASKED
#define DG_RING_MASKED 0
#endif

template <typename T, int BM, int BN, int NB, int MODE>
struct GemmTile {
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDS_ROW = kBK + PAD;  // elements per LDS row (16 B pad vs bank conflicts)
  static constexpr int MT = BM / 16;
  static constexpr int WN = BN / 4;          // columns per wave
  static constexpr int NT = WN / 16;
  static constexpr int VEC = 16 / sizeof(T); // elements per 16-byte chunk
  static constexpr int CPR = kBK / VEC;      // chunks per A row per stage
  static constexpr int A_CHUNKS = BM * CPR;
  static constexpr int A_ITERS = (A_CHUNKS + 255) / 256;
  static_assert(BN % 64 == 0, "BN must give each of the four waves a multiple of 16 columns");
  static_assert(BM % 16 == 0, "BM must be a multiple of 16");
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

// One BM x BN output tile over k in [kb, ke).
//   row_begin/rows: logical rows of the tile (rows <= BM valid)
//   Bp[nb]: pointer to row n0 of weight nb; ncols: valid columns from n0
template <typename T, int BM, int BN, int NB, int MODE>
__device__ __forceinline__ void gemm_tile(const GemmArgs &a, T *sA0, T *sA1, int row_begin, int rows,
                                          const T *const *Bp, int n0, int ncols, int kb, int ke,
                                          int split) {
  using G = GemmTile<T, BM, BN, NB, MODE>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const T *A = static_cast<const T *>(a.A);

  // physical A rows of the chunks this thread stages (fixed over k)
  long long arow[G::A_ITERS];
  int acol[G::A_ITERS];
  bool aval[G::A_ITERS];
#pragma unroll
  for (int it = 0; it < G::A_ITERS; ++it) {
    const int c = tid + it * 256;
    const int r = c / G::CPR;
    acol[it] = (c % G::CPR) * G::VEC;
    aval[it] = (c < G::A_CHUNKS) && (r < rows);
    int pr = row_begin + r;
    if (aval[it] && a.a_rows) pr = a.a_rows[pr];
    arow[it] = aval[it] ? static_cast<long long>(pr) * a.lda : 0;
  }
  // per-lane column validity (N need not be a multiple of 16)
  bool bval[G::NT];
#pragma unroll
  for (int nt = 0; nt < G::NT; ++nt) bval[nt] = (wave * G::WN + nt * 16 + l16) < ncols;

  f32x4 acc[NB][G::MT][G::NT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) acc[nb][mt][nt] = zero4();

  uint4 ra[G::A_ITERS];
  auto loadA = [&](int k0) {
#pragma unroll
    for (int it = 0; it < G::A_ITERS; ++it) {
      if (aval[it]) ra[it] = *reinterpret_cast<const uint4 *>(A + arow[it] + k0 + acol[it]);
      else ra[it] = make_uint4(0, 0, 0, 0);
    }
  };
  auto storeA = [&](T *s) {
#pragma unroll
    for (int it = 0; it < G::A_ITERS; ++it) {
      const int c = tid + it * 256;
      if (c < G::A_CHUNKS)
        *reinterpret_cast<uint4 *>(s + (c / G::CPR) * G::LDS_ROW + acol[it]) = ra[it];
    }
  };
  auto loadB = [&](Frag<T>(&fb)[NB][G::NT][2], int k0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < G::NT; ++nt) {
        const T *p = Bp[nb] + static_cast<long long>(wave * G::WN + nt * 16 + l16) * a.ldb + k0 + lg * 8;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (bval[nt]) fb[nb][nt][s].load(p + s * 32);
          else fb[nb][nt][s].zero();
        }
      }
  };
  auto compute = [&](const T *s, const Frag<T>(&fb)[NB][G::NT][2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mt = 0; mt < G::MT; ++mt) {
        Frag<T> fa;
        fa.load(s + (mt * 16 + l16) * G::LDS_ROW + ks * 32 + lg * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int nt = 0; nt < G::NT; ++nt) mma(acc[nb][mt][nt], fa, fb[nb][nt][ks]);
      }
    }
  };

  Frag<T> fb0[NB][G::NT][2], fb1[NB][G::NT][2];
  const int nst = (ke - kb) / kBK;
  loadA(kb);
  loadB(fb0, kb);
  storeA(sA0);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    const bool more1 = st + 1 < nst;
    if (more1) {
      loadA(kb + (st + 1) * kBK);
      loadB(fb1, kb + (st + 1) * kBK);
    }
    compute(sA0, fb0);
    if (more1) storeA(sA1);
    __syncthreads();
    if (!more1) break;
    const bool more2 = st + 2 < nst;
    if (more2) {
      loadA(kb + (st + 2) * kBK);
      loadB(fb0, kb + (st + 2) * kBK);
    }
    compute(sA1, fb1);
    if (more2) storeA(sA0);
    __syncthreads();
  }

  // epilogue: lane holds rows 4*lg + i, column l16 of each 16x16 sub-tile
#pragma unroll
  for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < G::NT; ++nt) {
      if (!bval[nt]) continue;
      const int col = n0 + wave * G::WN + nt * 16 + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + lg * 4 + i;
        if (r >= rows) continue;
        const long long row = row_begin + r;
        const float v = acc[0][mt][nt][i];
        if constexpr (MODE == EPI_STORE) {
          static_cast<T *>(a.C)[row * a.ldc + col] = from_f32<T>(v);
        } else if constexpr (MODE == EPI_STORE_F32) {
          static_cast<float *>(a.C)[row * a.ldc + col] = v;
        } else if constexpr (MODE == EPI_ADD) {
          T *c = static_cast<T *>(a.C) + row * a.ldc + col;
          *c = from_f32<T>(to_f32<T>(*c) + v);
        } else if constexpr (MODE == EPI_SWIGLU) {
          const float u = acc[NB - 1][mt][nt][i];
          static_cast<T *>(a.C)[row * a.ldc + col] = from_f32<T>(silu_f(v) * u);
        } else if constexpr (MODE == EPI_ROWSCALE_F32) {
          static_cast<float *>(a.C)[row * a.ldc + col] = v * a.rowscale[row];
        } else if constexpr (MODE == EPI_PARTIAL_F32) {
          static_cast<float *>(a.C)[(static_cast<long long>(split) * a.M + row) * a.ldc + col] = v;
        }
      }
    }
}

template <typename T, int BM, int BN, int NB, int MODE>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const GemmArgs a) {
  using G = GemmTile<T, BM, BN, NB, MODE>;
  __shared__ __attribute__((aligned(16))) T sA0[BM * G::LDS_ROW];
  __shared__ __attribute__((aligned(16))) T sA1[BM * G::LDS_ROW];

  if (a.g_off == nullptr) {
    // dense: one tile per workgroup; consecutive workgroup ids are spread
    // over the 8 XCDs, so renumber tiles to keep neighbours on one XCD (L2)
    const int L = xcd_tile(blockIdx.x, gridDim.x);
    const int m_tiles = (a.M + BM - 1) / BM;
    const int n_tiles = (a.N + BN - 1) / BN;
    int m_tile, n_tile, split;
    if (a.tile_order == 0) {
      m_tile = L % m_tiles;
      const int r = L / m_tiles;
      n_tile = r % n_tiles;
      split = r / n_tiles;
    } else {
      n_tile = L % n_tiles;
      const int r = L / n_tiles;
      m_tile = r % m_tiles;
      split = r / m_tiles;
    }
    const int n0 = n_tile * BN;
    int s = 0;
    while (s + 1 < a.nseg && n0 >= a.seg_start[s + 1]) ++s;
    const T *Bp[NB];
    Bp[0] = static_cast<const T *>(a.seg_B0[s]) + static_cast<long long>(n0 - a.seg_start[s]) * a.ldb;
    if (NB > 1) Bp[NB - 1] = static_cast<const T *>(a.seg_B1[s]) + static_cast<long long>(n0 - a.seg_start[s]) * a.ldb;
    const int kper = a.K / a.k_splits;
    const int row0 = m_tile * BM;
    gemm_tile<T, BM, BN, NB, MODE>(a, sA0, sA1, row0, min(BM, a.M - row0), Bp, n0,
                                   a.seg_start[s + 1] - n0, split * kper, (split + 1) * kper, split);
  } else {
    const int g = blockIdx.y;
    const int n0 = blockIdx.x * BN;
    const int Ng = (g < a.n_xgroups) ? a.N_x : a.N;
    if (n0 >= Ng) return;
    const T *Bp[NB];
    GemmArgs ga = a;   // group 0 (shared expert) may have its own depth and row stride
    if (g < a.n_xgroups) {
      ga.K = a.K_x;
      ga.ldb = a.ldb_x;
      Bp[0] = static_cast<const T *>(a.Bx0) + static_cast<long long>(n0) * a.ldb_x;
      if (NB > 1) Bp[NB - 1] = static_cast<const T *>(a.Bx1) + static_cast<long long>(n0) * a.ldb_x;
    } else {
      const long long off = static_cast<long long>(g - a.n_xgroups) * a.b_gstride + static_cast<long long>(n0) * a.ldb;
      Bp[0] = static_cast<const T *>(a.seg_B0[0]) + off;
      if (NB > 1) Bp[NB - 1] = static_cast<const T *>(a.seg_B1[0]) + off;
    }
    const int r0 = a.g_off[g], r1 = a.g_off[g + 1];
    for (int rb = r0; rb < r1; rb += BM)
      gemm_tile<T, BM, BN, NB, MODE>(ga, sA0, sA1, rb, min(BM, r1 - rb), Bp, n0, Ng - n0, 0, ga.K, 0);
  }
}

template <typename T, int BM, int BN, int NB, int MODE>
hipError_t launch_one(const GemmArgs &a, hipStream_t s) {
  dim3 grid;
  if (a.g_off) {
    const int nmax = a.N > a.N_x ? a.N : a.N_x;
    grid = dim3((nmax + BN - 1) / BN, a.n_groups);
  } else {
    const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
    grid = dim3(mt * nt * a.k_splits, 1);
  }
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, NB, MODE>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *part, int splits, int M, int N,
                                                            long long ldc, void *C, int mode) {
  const long long i8 = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i8 >= static_cast<long long>(M) * N) return;
  const int row = static_cast<int>(i8 / N), col = static_cast<int>(i8 % N);
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int z = 0; z < splits; ++z) {
    float v[8];
    load8(part + (static_cast<long long>(z) * M + row) * N + col, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] += v[j];
  }
  if (mode == EPI_STORE_F32) {
    store8(static_cast<float *>(C) + row * ldc + col, s);
  } else {
    T *c = static_cast<T *>(C) + row * ldc + col;
    if (mode == EPI_ADD) {
      float o[8];
      load8(c, o);
#pragma unroll
      for (int j = 0; j < 8; ++j) s[j] += o[j];
    }
    store8(c, s);
  }
}

// ----------------------------------------------------------------------------
// Streaming variant for the weight-bound products (few activation rows per
// weight tile).  The four waves of a workgroup split the k range of the
// whole BM x BN tile between them (wave w takes k steps w, w+4, w+8, ...,
// so together they walk each weight row's bytes in order), load both
// operands straight from global memory into MFMA fragments through a ring
// of S k steps -- S-1 steps of loads stay in flight behind the MFMAs -- and
// meet only once, at the end, to add their partial tiles through LDS.  No
// barrier sits in the main loop.

template <typename T, int MT, int NT, int NB, int MODE, int S>
__device__ __forceinline__ void stream_tile(const GemmArgs &a, float *red, int row_begin, int rows,
                                            const T *const *Bp, int n0, int ncols, int kb, int ke, int split) {
  constexpr int EL = NB * MT * NT * 4;   // accumulator floats per lane
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
  const int l16 = lane & 15, lg = lane >> 4;
  const T *A = static_cast<const T *>(a.A);

  // Wave-uniform bases + 32-bit per-lane byte offsets, so loads take the
  // scalar-base form.  Rows past `rows` and columns past `ncols` are
  // clamped onto row 0 of the tile and loaded anyway: an MFMA output element
  // depends only on its own A row and B column, and those outputs are never
  // stored, so no lane needs a branch around its loads.
  uint32_t ao[MT];
  bool av[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = mt * 16 + l16;
    av[mt] = r < rows;
    int pr = row_begin + (av[mt] ? r : 0);
    if (a.a_rows) pr = a.a_rows[pr];
    ao[mt] = (static_cast<uint32_t>(pr) * static_cast<uint32_t>(a.lda) + lg * 8) * sizeof(T);
  }
  uint32_t bo[NT];
  bool bv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = nt * 16 + l16;
    bv[nt] = c < ncols;
    bo[nt] = (static_cast<uint32_t>(bv[nt] ? c : 0) * static_cast<uint32_t>(a.ldb) + lg * 8) * sizeof(T);
  }
  const char *Ab = reinterpret_cast<const char *>(A);
  const char *B0 = reinterpret_cast<const char *>(Bp[0]);
  const char *B1 = reinterpret_cast<const char *>(Bp[NB - 1]);

  f32x4 acc[NB][MT][NT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nb][mt][nt] = zero4();

  const int nsteps = (ke - kb) / 32;
  const int my = nsteps > wave ? (nsteps - wave + 3) / 4 : 0;
  const int last = my > 0 ? my - 1 : 0;

  Frag<T> fa[S][MT];
  Frag<T> fb[S][NB][NT];

#if DG_RING_MASKED
  // Variant: no branch in the loop body.  Steps past the wave's last one
  // re-read that last step (in-bounds, cached) and get an all-zero A
  // fragment at use, so their MFMAs add exactly nothing.
  auto load = [&](int it, Frag<T>(&xa)[MT], Frag<T>(&xb)[NB][NT]) {
    const int st = it < last ? it : last;
    const uint32_t kbyte = static_cast<uint32_t>(kb + (wave + 4 * st) * 32) * sizeof(T);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        xb[nb][nt].load(reinterpret_cast<const T *>((nb == 0 ? B0 : B1) + (bo[nt] + kbyte)));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xa[mt].load(reinterpret_cast<const T *>(Ab + (ao[mt] + kbyte)));
  };
#pragma unroll
  for (int r = 0; r < S - 1; ++r) load(r, fa[r], fb[r]);
  for (int i = 0; i < my; i += S) {
#pragma unroll
    for (int r = 0; r < S; ++r) {
      load(i + r + S - 1, fa[(r + S - 1) % S], fb[(r + S - 1) % S]);
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t keep = (i + r) < my ? 0xffffffffu : 0u;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Frag<T> am = fa[r][mt];
        am.mask(keep);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(acc[nb][mt][nt], am, fb[r][nb][nt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#else
  // The prefetch of step it+S-1 and the MFMAs of step it are both skipped
  // past the wave's last step (wave-uniform branches).
  auto load = [&](int it, Frag<T>(&xa)[MT], Frag<T>(&xb)[NB][NT]) {
    const uint32_t kbyte = static_cast<uint32_t>(kb + (wave + 4 * it) * 32) * sizeof(T);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        xb[nb][nt].load(reinterpret_cast<const T *>((nb == 0 ? B0 : B1) + (bo[nt] + kbyte)));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) xa[mt].load(reinterpret_cast<const T *>(Ab + (ao[mt] + kbyte)));
  };
#pragma unroll
  for (int r = 0; r < S - 1; ++r)
    if (r < my) load(r, fa[r], fb[r]);
  for (int i = 0; i < my; i += S) {
#pragma unroll
    for (int r = 0; r < S; ++r) {
      const int it = i + r;
      if (it < my) {
        if (it + S - 1 < my) load(it + S - 1, fa[(r + S - 1) % S], fb[(r + S - 1) % S]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) mma(acc[nb][mt][nt], fa[r][mt], fb[r][nb][nt]);
      }
    }
  }
#endif

  // cross-wave reduction: every wave parks its partial tile in LDS, then all
  // 256 threads each add up and store a slice of the tile
  __syncthreads();   // LDS may still be read by the previous tile's epilogue
  {
    float *dst = red + wave * EL * 64;
    int e = 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i, ++e) dst[e * 64 + lane] = acc[nb][mt][nt][i];
  }
  __syncthreads();
  constexpr int EH = EL / NB;   // elements per lane of one product
  for (int q = tid; q < EH * 64; q += 256) {
    const int ln = q & 63, e = q >> 6;
    const int i = e & 3, nt = (e >> 2) % NT, mt = (e >> 2) / NT;
    const int r = mt * 16 + (ln >> 4) * 4 + i;
    const int c = nt * 16 + (ln & 15);
    if (r >= rows || c >= ncols) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) v += red[(w * EL + e) * 64 + ln];
    const long long row = row_begin + r;
    const int col = n0 + c;
    if constexpr (MODE == EPI_STORE) {
      static_cast<T *>(a.C)[row * a.ldc + col] = from_f32<T>(v);
    } else if constexpr (MODE == EPI_STORE_F32) {
      static_cast<float *>(a.C)[row * a.ldc + col] = v;
    } else if constexpr (MODE == EPI_ADD) {
      T *cp = static_cast<T *>(a.C) + row * a.ldc + col;
      *cp = from_f32<T>(to_f32<T>(*cp) + v);
    } else if constexpr (MODE == EPI_SWIGLU) {
      float u = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) u += red[(w * EL + EH + e) * 64 + ln];
      static_cast<T *>(a.C)[row * a.ldc + col] = from_f32<T>(silu_f(v) * u);
    } else if constexpr (MODE == EPI_ROWSCALE_F32) {
      static_cast<float *>(a.C)[row * a.ldc + col] = v * a.rowscale[row];
    } else if constexpr (MODE == EPI_PARTIAL_F32) {
      static_cast<float *>(a.C)[(static_cast<long long>(split) * a.M + row) * a.ldc + col] = v;
    }
  }
}

// Epilogue of the streaming tiles: the four waves' partial accumulators
// (each over its own k stages) are summed through LDS in wave order, so the
// result does not depend on timing.  SCALED multiplies column c of the first
// (and second) product by sc0[c] (sc1[c]) before the mode's operation: the
// per-row scales of fp8 weight matrices, sc0/sc1 pointing at the tile's
// first column.
template <int MT, int NT, int NB, int MODE, bool SCALED>
__device__ __forceinline__ void stream_epilogue(const GemmArgs &a, float *red, const f32x4 (&acc)[NB][MT][NT],
                                                int row_begin, int rows, int n0, int ncols, int split,
                                                const float *sc0, const float *sc1) {
  constexpr int EL = NB * MT * NT * 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __syncthreads();   // LDS may still be read by the previous tile's epilogue
  {
    float *dst = red + wave * EL * 64;
    int e = 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i, ++e) dst[e * 64 + lane] = acc[nb][mt][nt][i];
  }
  __syncthreads();
  // Each thread adds up and stores 4 neighbouring lanes of one accumulator
  // element: 4 consecutive columns of one row (float4 LDS reads, 16- or
  // 8-byte stores).
  constexpr int EH = EL / NB;
  for (int q = tid; q < EH * 16; q += 256) {
    const int l4 = (q & 15) * 4, e = q >> 4;
    const int i = e & 3, nt = (e >> 2) % NT, mt = (e >> 2) / NT;
    const int r = mt * 16 + (l4 >> 4) * 4 + i;
    const int c = nt * 16 + (l4 & 15);
    if (r >= rows || c >= ncols) continue;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 t = *reinterpret_cast<const float4 *>(red + (w * EL + e) * 64 + l4);
      v[0] += t.x; v[1] += t.y; v[2] += t.z; v[3] += t.w;
    }
    if constexpr (SCALED) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] *= sc0[c + (j < ncols - c ? j : 0)];
    }
    if constexpr (MODE == EPI_SWIGLU) {
      float u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float4 t = *reinterpret_cast<const float4 *>(red + (w * EL + EH + e) * 64 + l4);
        u[0] += t.x; u[1] += t.y; u[2] += t.z; u[3] += t.w;
      }
      if constexpr (SCALED) {
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] *= sc1[c + (j < ncols - c ? j : 0)];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = silu_f(v[j]) * u[j];
    }
    const long long row = row_begin + r;
    const int col = n0 + c;
    const int nv = ncols - c < 4 ? ncols - c : 4;   // valid columns of the four
    if constexpr (MODE == EPI_STORE_F32 || MODE == EPI_ROWSCALE_F32 || MODE == EPI_PARTIAL_F32) {
      if constexpr (MODE == EPI_ROWSCALE_F32) {
        const float rs = a.rowscale[row];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] *= rs;
      }
      const long long off = (MODE == EPI_PARTIAL_F32 ? (static_cast<long long>(split) * a.M + row) : row) * a.ldc + col;
      float *cp = static_cast<float *>(a.C) + off;
      if (nv == 4 && (off & 3) == 0) {
        *reinterpret_cast<float4 *>(cp) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        for (int j = 0; j < nv; ++j) cp[j] = v[j];
      }
    } else {
      bf16_t *cp = static_cast<bf16_t *>(a.C) + row * a.ldc + col;
      const bool vec = nv == 4 && ((row * a.ldc + col) & 3) == 0;
      if constexpr (MODE == EPI_ADD) {
        if (vec) {
          const uint2 o = *reinterpret_cast<const uint2 *>(cp);
          v[0] += __uint_as_float(o.x << 16);
          v[1] += __uint_as_float(o.x & 0xffff0000u);
          v[2] += __uint_as_float(o.y << 16);
          v[3] += __uint_as_float(o.y & 0xffff0000u);
        } else {
          for (int j = 0; j < nv; ++j) v[j] += bf16_to_f32(cp[j]);
        }
      }
      if (vec) {
        uint2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
        *reinterpret_cast<uint2 *>(cp) = o;
      } else {
        for (int j = 0; j < nv; ++j) cp[j] = f32_to_bf16(v[j]);
      }
    }
  }
}

// Weight (streamed) operand loads are non-temporal: each weight byte is read
// once per product, and marking it so keeps the L2 for the activation rows
// that every column tile of the product re-reads (measured on the expert
// gate/up product: HBM fetch 1.085x -> 1.026x of the algorithmic bytes).
__device__ __forceinline__ bf16x8 ld_stream(const char *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
}

// bf16 form with row-contiguous loads: 64-deep k stages (wave w takes
// stages w, w+4, ...), each 16-row block of A and B fetched as two loads of
// 8 whole rows and turned into the two fragments of the stage with DPP row
// shifts (contig_to_frags).  Same ring, same epilogue as stream_tile.
template <int MT, int NT, int NB, int MODE, int S>
__device__ __forceinline__ void stream_tile_c(const GemmArgs &a, float *red, int row_begin, int rows,
                                              const bf16_t *const *Bp, int n0, int ncols, int kb, int ke,
                                              int split) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cr = contig_row(lane), cc = contig_chunk(lane);

  // rows past `rows` / columns past `ncols` are clamped onto row 0 of the
  // tile (loaded, never stored), as in stream_tile
  uint32_t ao[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = mt * 16 + h * 8 + cr;
      int pr = row_begin + (r < rows ? r : 0);
      if (a.a_rows) pr = a.a_rows[pr];
      ao[mt][h] = (static_cast<uint32_t>(pr) * static_cast<uint32_t>(a.lda) + cc * 8) * 2u;
    }
  uint32_t bo[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = nt * 16 + h * 8 + cr;
      bo[nt][h] = (static_cast<uint32_t>(c < ncols ? c : 0) * static_cast<uint32_t>(a.ldb) + cc * 8) * 2u;
    }
  const char *Ab = static_cast<const char *>(a.A);
  const char *B0 = reinterpret_cast<const char *>(Bp[0]);
  const char *B1 = reinterpret_cast<const char *>(Bp[NB - 1]);

  f32x4 acc[NB][MT][NT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nb][mt][nt] = zero4();

  const int nsteps = (ke - kb) / 64;
  const int my = nsteps > wave ? (nsteps - wave + 3) / 4 : 0;

  bf16x8 xa[S][MT][2];
  bf16x8 xb[S][NB][NT][2];
  auto load = [&](int it, bf16x8(&ya)[MT][2], bf16x8(&yb)[NB][NT][2]) {
    const uint32_t kbyte = static_cast<uint32_t>(kb + (wave + 4 * it) * 64) * 2u;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          yb[nb][nt][h] = ld_stream((nb == 0 ? B0 : B1) + (bo[nt][h] + kbyte));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) ya[mt][h] = *reinterpret_cast<const bf16x8 *>(Ab + (ao[mt][h] + kbyte));
  };
  auto compute = [&](const bf16x8(&ya)[MT][2], const bf16x8(&yb)[NB][NT][2]) {
    Frag<bf16_t> fb[NB][NT][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) contig_to_frags(yb[nb][nt][0], yb[nb][nt][1], fb[nb][nt][0].v, fb[nb][nt][1].v);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      Frag<bf16_t> fa[2];
      contig_to_frags(ya[mt][0], ya[mt][1], fa[0].v, fa[1].v);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(acc[nb][mt][nt], fa[ks], fb[nb][nt][ks]);
    }
  };
#pragma unroll
  for (int r = 0; r < S - 1; ++r)
    if (r < my) load(r, xa[r], xb[r]);
  for (int i = 0; i < my; i += S) {
#pragma unroll
    for (int r = 0; r < S; ++r) {
      const int it = i + r;
      if (it < my) {
        if (it + S - 1 < my) load(it + S - 1, xa[(r + S - 1) % S], xb[(r + S - 1) % S]);
        compute(xa[r], xb[r]);
      }
    }
  }

  stream_epilogue<MT, NT, NB, MODE, false>(a, red, acc, row_begin, rows, n0, ncols, split, nullptr, nullptr);
}

// ----------------------------------------------------------------------------
// Expert products with OCP E4M3 weights (one fp32 scale per weight row) and
// bf16 activations.  The kernel is bound by streaming the weights, so the
// bytes are what fp8 saves; each weight byte is widened to bf16 in registers
// (exact: every E4M3 value is a bf16 value) and the products run on the
// bf16 MFMA, with the row scales applied in the epilogue.
//
// k stages are 128 deep (128 weight bytes per row, one whole cache line).
// A 16-row weight block of a stage is two row-contiguous loads (8 rows x
// 128 bytes each), turned by contig_to_frags into two 16-byte pieces per
// lane: row l16, bytes 16*lg.. (f0) and 64 + 16*lg.. (f1).  Each piece
// widens to two bf16 fragments.  The MFMA k order inside the stage is
// therefore: step ks, lane group lg, element i  <->  depth
// 64*(ks/2) + 16*lg + 8*(ks%2) + i; the activation fragments are loaded in
// the same order (per 64-deep half, lane group lg takes the 8-element
// chunks 2*lg and 2*lg+1 of its rows, again as 8 rows x 128 bytes).
// With k % 128 == 64 the last stage is 64 deep: its second-half loads
// re-read the first half (in bounds) and the second-half activation
// fragments are zeroed, so those products add exactly 0.

__device__ __forceinline__ void e4m3x16_to_bf16(const bf16x8 &raw, bf16x8 &lo, bf16x8 &hi) {
  uint32_t w[4], o[8];
  __builtin_memcpy(w, &raw, 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, false);   // bytes 0, 1
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.0f, true);    // bytes 2, 3
    __builtin_memcpy(&o[2 * j], &p0, 4);
    __builtin_memcpy(&o[2 * j + 1], &p1, 4);
  }
  __builtin_memcpy(&lo, &o[0], 16);
  __builtin_memcpy(&hi, &o[4], 16);
}

template <int MT, int NT, int NB, int MODE, int S>
__device__ __forceinline__ void stream_tile_f8(const GemmArgs &a, float *red, int row_begin, int rows,
                                               const uint8_t *const *Bp, const float *const *Sp, int n0,
                                               int ncols, int K) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cr = contig_row(lane), cb = contig_chunk(lane);
  const int hb = (lane & 15) >> 3, lg = lane >> 4;
  const int ca = 2 * lg + hb;   // activation chunk (8 elements) inside a 64-deep half

  uint32_t ao[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = mt * 16 + h * 8 + cr;
      int pr = row_begin + (r < rows ? r : 0);
      if (a.a_rows) pr = a.a_rows[pr];
      ao[mt][h] = (static_cast<uint32_t>(pr) * static_cast<uint32_t>(a.lda) + ca * 8) * 2u;
    }
  uint32_t bo[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = nt * 16 + h * 8 + cr;
      bo[nt][h] = static_cast<uint32_t>(c < ncols ? c : 0) * static_cast<uint32_t>(a.ldb) + cb * 16;
    }
  const char *Ab = static_cast<const char *>(a.A);
  const char *B0 = reinterpret_cast<const char *>(Bp[0]);
  const char *B1 = reinterpret_cast<const char *>(Bp[NB - 1]);

  f32x4 acc[NB][MT][NT];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nb][mt][nt] = zero4();

  const int nst = (K + 127) >> 7;
  const int my = nst > wave ? (nst - wave + 3) / 4 : 0;

  bf16x8 xa[S][MT][2][2];   // [slot][mt][64-deep half][8-row load]
  bf16x8 xb[S][NB][NT][2];
  auto load = [&](int it, bf16x8(&ya)[MT][2][2], bf16x8(&yb)[NB][NT][2]) {
    const int st = wave + 4 * it;
    const bool half = (st + 1) * 128 > K;
    const uint32_t kb = static_cast<uint32_t>(st) * 128u - ((half && hb) ? 64u : 0u);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          yb[nb][nt][h] = ld_stream((nb == 0 ? B0 : B1) + (bo[nt][h] + kb));
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
      const uint32_t ka = (static_cast<uint32_t>(st) * 128u + (half ? 0u : 64u * jh)) * 2u;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) ya[mt][jh][h] = *reinterpret_cast<const bf16x8 *>(Ab + (ao[mt][h] + ka));
    }
  };
  auto compute = [&](int it, const bf16x8(&ya)[MT][2][2], const bf16x8(&yb)[NB][NT][2]) {
    const bool half = (wave + 4 * it + 1) * 128 > K;
    Frag<bf16_t> fa[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      contig_to_frags(ya[mt][0][0], ya[mt][0][1], fa[mt][0].v, fa[mt][1].v);
      contig_to_frags(ya[mt][1][0], ya[mt][1][1], fa[mt][2].v, fa[mt][3].v);
      if (half) {
        fa[mt][2].v = bf16x8{};
        fa[mt][3].v = bf16x8{};
      }
    }
    // weight fragments are widened one 16-column block at a time
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 f0, f1;
        contig_to_frags(yb[nb][nt][0], yb[nb][nt][1], f0, f1);
        Frag<bf16_t> fb[4];
        e4m3x16_to_bf16(f0, fb[0].v, fb[1].v);
        e4m3x16_to_bf16(f1, fb[2].v, fb[3].v);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) mma(acc[nb][mt][nt], fa[mt][ks], fb[ks]);
      }
  };
#pragma unroll
  for (int r = 0; r < S - 1; ++r)
    if (r < my) load(r, xa[r], xb[r]);
  for (int i = 0; i < my; i += S) {
#pragma unroll
    for (int r = 0; r < S; ++r) {
      const int it = i + r;
      if (it < my) {
        if (it + S - 1 < my) load(it + S - 1, xa[(r + S - 1) % S], xb[(r + S - 1) % S]);
        compute(it, xa[r], xb[r]);
      }
    }
  }
  stream_epilogue<MT, NT, NB, MODE, true>(a, red, acc, row_begin, rows, n0, ncols, 0, Sp[0], Sp[NB - 1]);
}

// (group, column tile) of a grouped launch over a grid of (column tiles,
// groups).  Consecutive workgroups go to the eight XCDs in turn, so with
// `xcd` each XCD takes a contiguous run of items instead: the column tiles
// of one group then share that XCD's L2 for the group's activation rows.
// Measured on the 32-row expert tiles (gate/up: HBM fetch 1.078x -> 1.040x
// of the algorithmic bytes, 176.7-182.8 -> 174.3 us per launch); the
// 256-row tiles of long groups ran slower with it (8 canvases per forward:
// 160.0 against 162.1 canvas-steps/s), so they keep the plain order.
__device__ __forceinline__ void grouped_item(int &g, int &n0, int BN, bool xcd) {
  g = blockIdx.y;
  n0 = blockIdx.x * BN;
  if (xcd) {
    const int gx = gridDim.x, total = gx * gridDim.y;
    int L = blockIdx.y * gx + blockIdx.x;
    const int full = total & ~7;
    if (L < full) L = (L & 7) * (full >> 3) + (L >> 3);   // a permutation of [0, full)
    g = L / gx;
    n0 = (L - g * gx) * BN;
  }
}

// Grouped expert product with fp8 weights: blockIdx.y = group (shared-expert
// row chunks first, then the routed experts), blockIdx.x = column tile.
// Weight rows are K bytes apart (ldb, ldb_x in bytes); routed expert e's
// scales start at bs0 + e*N, the shared expert's at bxs0.
template <int MT, int NT, int NB, int MODE, int S>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MT <= 2 ? 2 : 1, 2))) void gemm_f8_grouped_kernel(const GemmArgs a) {
  constexpr int BM = MT * 16, BN = NT * 16;
  __shared__ __attribute__((aligned(16))) float red[4 * NB * MT * NT * 4 * 64];
  int g, n0;
  grouped_item(g, n0, BN, false);
  const bool sh = g < a.n_xgroups;
  const int Ng = sh ? a.N_x : a.N;
  if (n0 >= Ng) return;
  GemmArgs ga = a;
  const uint8_t *Bp[NB];
  const float *Sp[NB];
  if (sh) {
    ga.K = a.K_x;
    ga.ldb = a.ldb_x;
    Bp[0] = static_cast<const uint8_t *>(a.Bx0) + static_cast<long long>(n0) * a.ldb_x;
    Sp[0] = a.bxs0 + n0;
    if (NB > 1) {
      Bp[NB - 1] = static_cast<const uint8_t *>(a.Bx1) + static_cast<long long>(n0) * a.ldb_x;
      Sp[NB - 1] = a.bxs1 + n0;
    }
  } else {
    const int e = g - a.n_xgroups;
    const long long off = static_cast<long long>(e) * a.b_gstride + static_cast<long long>(n0) * a.ldb;
    Bp[0] = static_cast<const uint8_t *>(a.seg_B0[0]) + off;
    Sp[0] = a.bs0 + static_cast<long long>(e) * a.N + n0;
    if (NB > 1) {
      Bp[NB - 1] = static_cast<const uint8_t *>(a.seg_B1[0]) + off;
      Sp[NB - 1] = a.bs1 + static_cast<long long>(e) * a.N + n0;
    }
  }
  const int r0 = a.g_off[g], r1 = a.g_off[g + 1];
  for (int rb = r0; rb < r1; rb += BM)
    stream_tile_f8<MT, NT, NB, MODE, S>(ga, red, rb, min(BM, r1 - rb), Bp, Sp, n0, Ng - n0, ga.K);
}

template <int MT, int NT, int NB, int MODE, int S>
hipError_t launch_f8_one(const GemmArgs &a, hipStream_t s) {
  constexpr int BN = NT * 16;
  const int nmax = a.N > a.N_x ? a.N : a.N_x;
  const dim3 grid((nmax + BN - 1) / BN, a.n_groups);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f8_grouped_kernel<MT, NT, NB, MODE, S>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Tile body of the streaming kernel: the row-contiguous bf16 form when every
// k range of the launch is a whole number of 64-deep stages (CONTIG).
template <typename T, int MT, int NT, int NB, int MODE, int S, bool CONTIG>
__device__ __forceinline__ void stream_any(const GemmArgs &a, float *red, int row_begin, int rows,
                                           const T *const *Bp, int n0, int ncols, int kb, int ke, int split) {
  if constexpr (CONTIG && sizeof(T) == 2)
    stream_tile_c<MT, NT, NB, MODE, (S + 1) / 2>(a, red, row_begin, rows, reinterpret_cast<const bf16_t *const *>(Bp),
                                                 n0, ncols, kb, ke, split);
  else
    stream_tile<T, MT, NT, NB, MODE, S>(a, red, row_begin, rows, Bp, n0, ncols, kb, ke, split);
}

template <typename T, int MT, int NT, int NB, int MODE, int S, bool CONTIG>
__global__ __launch_bounds__(256) void gemm_stream_kernel(const GemmArgs a) {
  constexpr int BM = MT * 16, BN = NT * 16;
  __shared__ __attribute__((aligned(16))) float red[4 * NB * MT * NT * 4 * 64];
  if (a.g_off == nullptr) {
    const int L = xcd_tile(blockIdx.x, gridDim.x);
    const int m_tiles = (a.M + BM - 1) / BM;
    const int n_tiles = (a.N + BN - 1) / BN;
    int m_tile, n_tile, split;
    if (a.tile_order == 0) {
      m_tile = L % m_tiles;
      const int r = L / m_tiles;
      n_tile = r % n_tiles;
      split = r / n_tiles;
    } else {
      n_tile = L % n_tiles;
      const int r = L / n_tiles;
      m_tile = r % m_tiles;
      split = r / m_tiles;
    }
    const int n0 = n_tile * BN;
    int s = 0;
    while (s + 1 < a.nseg && n0 >= a.seg_start[s + 1]) ++s;
    const T *Bp[NB];
    Bp[0] = static_cast<const T *>(a.seg_B0[s]) + static_cast<long long>(n0 - a.seg_start[s]) * a.ldb;
    if (NB > 1) Bp[NB - 1] = static_cast<const T *>(a.seg_B1[s]) + static_cast<long long>(n0 - a.seg_start[s]) * a.ldb;
    const int kper = a.K / a.k_splits;
    const int row0 = m_tile * BM;
    stream_any<T, MT, NT, NB, MODE, S, CONTIG>(a, red, row0, min(BM, a.M - row0), Bp, n0, a.seg_start[s + 1] - n0,
                                               split * kper, (split + 1) * kper, split);
  } else {
    const int g = blockIdx.y;
    const int n0 = blockIdx.x * BN;
    const int Ng = (g < a.n_xgroups) ? a.N_x : a.N;
    if (n0 >= Ng) return;
    const T *Bp[NB];
    GemmArgs ga = a;
    if (g < a.n_xgroups) {
      ga.K = a.K_x;
      ga.ldb = a.ldb_x;
      Bp[0] = static_cast<const T *>(a.Bx0) + static_cast<long long>(n0) * a.ldb_x;
      if (NB > 1) Bp[NB - 1] = static_cast<const T *>(a.Bx1) + static_cast<long long>(n0) * a.ldb_x;
    } else {
      const long long off = static_cast<long long>(g - a.n_xgroups) * a.b_gstride + static_cast<long long>(n0) * a.ldb;
      Bp[0] = static_cast<const T *>(a.seg_B0[0]) + off;
      if (NB > 1) Bp[NB - 1] = static_cast<const T *>(a.seg_B1[0]) + off;
    }
    const int r0 = a.g_off[g], r1 = a.g_off[g + 1];
    for (int rb = r0; rb < r1; rb += BM)
      stream_any<T, MT, NT, NB, MODE, S, CONTIG>(ga, red, rb, min(BM, r1 - rb), Bp, n0, Ng - n0, 0, ga.K, 0);
  }
}

template <typename T, int MT, int NT, int NB, int MODE, int S>
hipError_t launch_stream_one(const GemmArgs &a, hipStream_t s) {
  constexpr int BM = MT * 16, BN = NT * 16;
  dim3 grid;
  if (a.g_off) {
    const int nmax = a.N > a.N_x ? a.N : a.N_x;
    grid = dim3((nmax + BN - 1) / BN, a.n_groups);
  } else {
    const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
    grid = dim3(mt * nt * a.k_splits, 1);
  }
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  // row-contiguous bf16 form when every k range is whole 64-deep stages
  const bool contig = DG_CONTIG && sizeof(T) == 2 &&
                      (a.g_off ? (a.K % 64 == 0 && a.K_x % 64 == 0) : ((a.K / a.k_splits) % 64 == 0));
  if (contig)
    hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NT, NB, MODE, S, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<T, MT, NT, NB, MODE, S, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Wide-tile variant (bfloat16) for products whose activation operand is
// re-read by many weight tiles: the 256-row canvas products (LM head, the
// soft embedding P.E, projections) and the expert products.  A workgroup of
// NW waves owns a (16*MT) x (NW*NTW*16) output tile and walks k in stages of
// 64.  The A slice of a stage is fetched once per workgroup with row-
// contiguous loads (8 rows x 128 bytes per wave instruction: whole cache
// lines, the cheap pattern for the load units) and written to an LDS tile,
// where every wave reads its MFMA fragments.  Each wave streams its own
// weight rows (B) with the same row-contiguous loads, P stages ahead, and
// turns them into fragments through a private LDS region (no barrier).
//
// Order inside stage it: load A(it+1) into registers, then issue B(it+P), run
// the MFMAs of stage it, write A(it+1) to the other LDS buffer, barrier.  A is
// issued before B, so waiting for A never waits for the younger B loads; the
// barrier waits only for LDS traffic (lgkmcnt), leaving the B loads in flight.
//
// LDS tile: BM rows x 128 bytes; 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7), which keeps both the row-contiguous writes and the
// 16-row fragment reads free of bank conflicts.

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int MT, int NTW, int NB, int NW, int KSUB, int P, int MODE>
__device__ __forceinline__ void wide_tile(const GemmArgs &a, bf16_t *lds, bf16_t *ldsb, int row_begin, int rows,
                                          const bf16_t *const *Bp, int n0, int ncols, int kb, int ke,
                                          int split) {
  static_assert(KSUB == 2, "stages are 64 deep (128 bytes per A row)");
  // A is fetched PA stages ahead (ring of PA register slots); PA = 2 needs
  // an even ring length R so slot parity is fixed inside the unrolled body.
  // The expert gate/up configuration (two products, short row tiles) takes
  // its own depth: two stages measured faster there, slower for the
  // 256-row projections.
  constexpr int PA_WANT = (NB == 2 && MT <= 4) ? DG_WMOE_PA : DG_WIDE_PA;
  constexpr int PA = ((P + 1) % 2 == 0) ? PA_WANT : 1;
  constexpr int BM = MT * 16;
  constexpr int D = BM / 8 / NW;         // A load instructions per wave per stage
  static_assert(D * 8 * NW == BM, "A rows must split evenly over the waves");
  constexpr int DB = NTW * 2;            // B load instructions per weight matrix per stage
  constexpr int R = P + 1;               // B ring slots
  constexpr int STAGE = BM * 64;         // bf16 elements per LDS buffer of A
  constexpr int WB = NB * NTW * 16 * 64; // bf16 elements of one wave's B region
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;   // row-contiguous pattern: 8 rows x 8 chunks

  // A: instruction j of this wave covers rows 8*(wave + NW*j) + lane/8, chunk lane%8
  uint32_t ao[D];
  int aw[D];   // LDS element offset of this lane's chunk
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int r = (wave + NW * j) * 8 + lr;
    int pr = row_begin + (r < rows ? r : 0);
    if (a.a_rows) pr = a.a_rows[pr];
    ao[j] = (static_cast<uint32_t>(pr) * static_cast<uint32_t>(a.lda) + lc * 8) * 2u;
    aw[j] = r * 64 + ((lc ^ ((r >> 1) & 7)) * 8);
  }
  // fragment read offsets inside a swizzled 16-row block (A and B alike)
  int fo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) fo[ks] = l16 * 64 + (((4 * ks + lg) ^ (l16 >> 1)) * 8);
  // B: the wave's NTW*16 weight rows, 8 per instruction, columns past ncols
  // re-read column 0 of the tile
  uint32_t bo[DB];
  int bw[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    const int r = j * 8 + lr;                       // row inside the wave's block
    const int c = wave * (NTW * 16) + r;
    bo[j] = (static_cast<uint32_t>(c < ncols ? c : 0) * static_cast<uint32_t>(a.ldb) + lc * 8) * 2u;
    bw[j] = r * 64 + ((lc ^ ((r >> 1) & 7)) * 8);
  }
  bf16_t *myb = ldsb + wave * WB;
  const char *Ab = static_cast<const char *>(a.A);
  const char *Bb[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) Bb[nb] = reinterpret_cast<const char *>(Bp[nb]);

  f32x4 acc[NB][MT][NTW];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[nb][mi][nt] = zero4();

  Frag<bf16_t> ra[PA][D];                // native vectors: must stay in registers
  Frag<bf16_t> rb[R][NB][DB];

  auto load_a = [&](int st, Frag<bf16_t>(&xa)[D]) {
    const uint32_t kbyte = static_cast<uint32_t>(kb + st * 64) * 2u;
#pragma unroll
    for (int j = 0; j < D; ++j) xa[j].load(reinterpret_cast<const bf16_t *>(Ab + (ao[j] + kbyte)));
  };
  auto load_b = [&](int st, Frag<bf16_t>(&xb)[NB][DB]) {
    const uint32_t kbyte = static_cast<uint32_t>(kb + st * 64) * 2u;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < DB; ++j) xb[nb][j].v = ld_stream(Bb[nb] + (bo[j] + kbyte));
  };
  auto stage_a = [&](int buf, const Frag<bf16_t>(&xa)[D]) {
#pragma unroll
    for (int j = 0; j < D; ++j) *reinterpret_cast<bf16x8 *>(lds + buf * STAGE + aw[j]) = xa[j].v;
  };
  auto compute = [&](int buf, const Frag<bf16_t>(&xb)[NB][DB]) {
    // this wave's B slice: rows to its own LDS region, back as fragments
    // (wave-local: LDS operations of one wave complete in order)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < DB; ++j) *reinterpret_cast<bf16x8 *>(myb + nb * (NTW * 16 * 64) + bw[j]) = xb[nb][j].v;
    Frag<bf16_t> fb[NB][NTW][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) fb[nb][nt][ks].load(myb + nb * (NTW * 16 * 64) + nt * 16 * 64 + fo[ks]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        Frag<bf16_t> fa;
        fa.load(lds + buf * STAGE + mi * 16 * 64 + fo[ks]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) mma(acc[nb][mi][nt], fa, fb[nb][nt][ks]);
      }
  };

  // No memory operation of the loop body sits under a branch, so the
  // compiler's count of loads in flight stays exact: stages past the last
  // re-load the last one (in bounds) and only their MFMAs are skipped.
  const int nst = (ke - kb) / 64;
  const int lastst = nst > 0 ? nst - 1 : 0;
  if (nst > 0) {
    load_a(0, ra[0]);
    if constexpr (PA == 2) load_a(1 < lastst ? 1 : lastst, ra[1]);
#pragma unroll
    for (int r = 0; r < P; ++r) load_b(r < lastst ? r : lastst, rb[r]);
    stage_a(0, ra[0]);
  }
  lds_barrier();
  for (int i = 0; i < nst; i += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int it = i + r;
      // A slot of stage s is s % PA (R is even when PA == 2, so r's parity is it's)
      if constexpr (PA == 2) load_a(it + 2 < lastst ? it + 2 : lastst, ra[r & 1]);
      else load_a(it + 1 < lastst ? it + 1 : lastst, ra[0]);
      load_b(it + P < lastst ? it + P : lastst, rb[(r + P) % R]);
      // the loads go out before the stage's MFMAs: left to itself the
      // scheduler sinks them to the end of the body, next to the LDS write
      // that waits for A, and every stage then waits a whole memory round trip
      if constexpr (DG_LOAD_FENCE) __builtin_amdgcn_sched_barrier(0);
      if (it < nst) compute(it & 1, rb[r]);
      stage_a((it + 1) & 1, ra[PA == 2 ? ((r + 1) & 1) : 0]);
      lds_barrier();
    }
  }

  // epilogue straight from the accumulators: lane holds rows 4*lg+i, column l16
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int c = wave * (NTW * 16) + nt * 16 + l16;
    if (c >= ncols) continue;
    const int col = n0 + c;
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mi * 16 + lg * 4 + i;
        if (r >= rows) continue;
        const long long row = row_begin + r;
        const float v = acc[0][mi][nt][i];
        if constexpr (MODE == EPI_STORE) {
          static_cast<bf16_t *>(a.C)[row * a.ldc + col] = f32_to_bf16(v);
        } else if constexpr (MODE == EPI_STORE_F32) {
          static_cast<float *>(a.C)[row * a.ldc + col] = v;
        } else if constexpr (MODE == EPI_ADD) {
          bf16_t *cp = static_cast<bf16_t *>(a.C) + row * a.ldc + col;
          *cp = f32_to_bf16(bf16_to_f32(*cp) + v);
        } else if constexpr (MODE == EPI_SWIGLU) {
          static_cast<bf16_t *>(a.C)[row * a.ldc + col] = f32_to_bf16(silu_f(v) * acc[NB - 1][mi][nt][i]);
        } else if constexpr (MODE == EPI_ROWSCALE_F32) {
          static_cast<float *>(a.C)[row * a.ldc + col] = v * a.rowscale[row];
        } else if constexpr (MODE == EPI_PARTIAL_F32) {
          static_cast<float *>(a.C)[(static_cast<long long>(split) * a.M + row) * a.ldc + col] = v;
        }
      }
  }
}

template <int MT, int NTW, int NB, int NW, int KSUB, int P, int MODE>
__global__ __launch_bounds__(64 * NW) void gemm_wide_kernel(const GemmArgs a) {
  constexpr int BM = MT * 16, BN = NW * NTW * 16, KS = 64;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * MT * 16 * 64];
  __shared__ __attribute__((aligned(16))) bf16_t ldsb[NW * NB * NTW * 16 * 64];
  if (a.g_off == nullptr) {
    const int L = xcd_tile(blockIdx.x, gridDim.x);
    const int m_tiles = (a.M + BM - 1) / BM;
    const int n_tiles = (a.N + BN - 1) / BN;
    int m_tile, n_tile, split;
    if (a.tile_order == 0) {
      m_tile = L % m_tiles;
      const int r = L / m_tiles;
      n_tile = r % n_tiles;
      split = r / n_tiles;
    } else {
      n_tile = L % n_tiles;
      const int r = L / n_tiles;
      m_tile = r % m_tiles;
      split = r / m_tiles;
    }
    const int n0 = n_tile * BN;
    int s = 0;
    while (s + 1 < a.nseg && n0 >= a.seg_start[s + 1]) ++s;
    const bf16_t *Bp[NB];
    Bp[0] = static_cast<const bf16_t *>(a.seg_B0[s]) + static_cast<long long>(n0 - a.seg_start[s]) * a.ldb;
    if (NB > 1)
      Bp[NB - 1] = static_cast<const bf16_t *>(a.seg_B1[s]) + static_cast<long long>(n0 - a.seg_start[s]) * a.ldb;
    // split s covers [s*kper, min(K, (s+1)*kper)), kper a multiple of the stage depth
    const int kper = ((a.K + a.k_splits - 1) / a.k_splits + KS - 1) / KS * KS;
    const int kb = split * kper, ke = min(a.K, kb + kper);
    const int row0 = m_tile * BM;
    wide_tile<MT, NTW, NB, NW, KSUB, P, MODE>(a, lds, ldsb, row0, min(BM, a.M - row0), Bp, n0,
                                              min(BN, a.seg_start[s + 1] - n0), kb, ke > kb ? ke : kb, split);
  } else {
    int g, n0;
    grouped_item(g, n0, BN, DG_GROUPED_XCD && MT <= 2);
    const int Ng = (g < a.n_xgroups) ? a.N_x : a.N;
    if (n0 >= Ng) return;
    const bf16_t *Bp[NB];
    GemmArgs ga = a;
    if (g < a.n_xgroups) {
      ga.K = a.K_x;
      ga.ldb = a.ldb_x;
      Bp[0] = static_cast<const bf16_t *>(a.Bx0) + static_cast<long long>(n0) * a.ldb_x;
      if (NB > 1) Bp[NB - 1] = static_cast<const bf16_t *>(a.Bx1) + static_cast<long long>(n0) * a.ldb_x;
    } else {
      const long long off = static_cast<long long>(g - a.n_xgroups) * a.b_gstride + static_cast<long long>(n0) * a.ldb;
      Bp[0] = static_cast<const bf16_t *>(a.seg_B0[0]) + off;
      if (NB > 1) Bp[NB - 1] = static_cast<const bf16_t *>(a.seg_B1[0]) + off;
    }
    const int r0 = a.g_off[g], r1 = a.g_off[g + 1];
    for (int rb = r0; rb < r1; rb += BM)
      wide_tile<MT, NTW, NB, NW, KSUB, P, MODE>(ga, lds, ldsb, rb, min(BM, r1 - rb), Bp, n0, min(BN, Ng - n0), 0,
                                                ga.K, 0);
  }
}

// ----------------------------------------------------------------------------
// Wide-tile expert gate/up with OCP E4M3 weights (one fp32 scale per weight
// row).  The bf16 wide tile with two changes: a stage is 128 deep, so each
// weight row still arrives as a 128-byte segment (the same loads and private
// LDS layout as bf16), while an activation stage is two 64-deep halves (two
// LDS sub-tiles in the bf16 layout); each fragment read takes the 8 bytes of
// a 32-deep k slice from the private region and widens them to bf16 with the
// hardware conversion.  The scales multiply the gate and up columns in the
// epilogue, before the SwiGLU.  K must be a multiple of 128.
template <int MT, int NTW, int NW, int P>
__device__ __forceinline__ void wide_tile_f8(const GemmArgs &a, bf16_t *lds, uint8_t *ldsb, int row_begin, int rows,
                                             const uint8_t *const *Bp, const float *const *Sp, int n0, int ncols,
                                             int K) {
  constexpr int NB = 2;
  constexpr int BM = MT * 16;
  constexpr int D = BM / 8 / NW;         // A load instructions per wave per 64-deep half
  static_assert(D * 8 * NW == BM, "A rows must split evenly over the waves");
  constexpr int DB = NTW * 2;            // B load instructions per weight matrix per stage
  constexpr int R = P + 1;               // B ring slots (A: one stage ahead)
  constexpr int HALF = BM * 64;          // bf16 elements of one 64-deep A sub-tile
  constexpr int STAGE = 2 * HALF;
  constexpr int WB = NB * NTW * 16 * 128; // bytes of one wave's B region
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;

  uint32_t ao[D];
  int aw[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int r = (wave + NW * j) * 8 + lr;
    int pr = row_begin + (r < rows ? r : 0);
    if (a.a_rows) pr = a.a_rows[pr];
    ao[j] = (static_cast<uint32_t>(pr) * static_cast<uint32_t>(a.lda) + lc * 8) * 2u;
    aw[j] = r * 64 + ((lc ^ ((r >> 1) & 7)) * 8);
  }
  int fo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) fo[ks] = l16 * 64 + (((4 * ks + lg) ^ (l16 >> 1)) * 8);
  // B fragment of 32-deep slice ks: bytes [32 ks + 8 lg, +8) of row l16
  int fbo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c16 = 2 * ks + (lg >> 1);
    fbo[ks] = l16 * 128 + ((c16 ^ ((l16 >> 1) & 7)) * 16) + (lg & 1) * 8;
  }
  uint32_t bo[DB];
  int bw[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    const int r = j * 8 + lr;
    const int c = wave * (NTW * 16) + r;
    bo[j] = static_cast<uint32_t>(c < ncols ? c : 0) * static_cast<uint32_t>(a.ldb) + lc * 16;
    bw[j] = r * 128 + ((lc ^ ((r >> 1) & 7)) * 16);
  }
  uint8_t *myb = ldsb + wave * WB;
  const char *Ab = static_cast<const char *>(a.A);

  f32x4 acc[NB][MT][NTW];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[nb][mi][nt] = zero4();

  Frag<bf16_t> ra[2][D];                 // the next stage's activation halves
  Frag<bf16_t> rb[R][NB][DB];
  auto load_a = [&](int st, Frag<bf16_t>(&xa)[2][D]) {
    const uint32_t kbyte = static_cast<uint32_t>(st) * 256u;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < D; ++j) xa[h][j].load(reinterpret_cast<const bf16_t *>(Ab + (ao[j] + kbyte + h * 128u)));
  };
  auto load_b = [&](int st, Frag<bf16_t>(&xb)[NB][DB]) {
    const uint32_t kbyte = static_cast<uint32_t>(st) * 128u;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < DB; ++j) xb[nb][j].v = ld_stream(reinterpret_cast<const char *>(Bp[nb]) + (bo[j] + kbyte));
  };
  auto stage_a = [&](int buf, const Frag<bf16_t>(&xa)[2][D]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < D; ++j) *reinterpret_cast<bf16x8 *>(lds + buf * STAGE + h * HALF + aw[j]) = xa[h][j].v;
  };
  auto compute = [&](int buf, const Frag<bf16_t>(&xb)[NB][DB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < DB; ++j) *reinterpret_cast<bf16x8 *>(myb + nb * (NTW * 16 * 128) + bw[j]) = xb[nb][j].v;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      Frag<bf16_t> fb[NB][NTW];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const uint2 q = *reinterpret_cast<const uint2 *>(myb + nb * (NTW * 16 * 128) + nt * 16 * 128 + fbo[ks]);
          const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false);
          const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true);
          const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false);
          const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true);
          uint32_t o[4];
          __builtin_memcpy(&o[0], &p0, 4);
          __builtin_memcpy(&o[1], &p1, 4);
          __builtin_memcpy(&o[2], &p2, 4);
          __builtin_memcpy(&o[3], &p3, 4);
          __builtin_memcpy(&fb[nb][nt].v, o, 16);
        }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        Frag<bf16_t> fa;
        fa.load(lds + buf * STAGE + (ks >> 1) * HALF + mi * 16 * 64 + fo[ks & 1]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) mma(acc[nb][mi][nt], fa, fb[nb][nt]);
      }
    }
  };

  // as in wide_tile: no memory operation of the loop body under a branch;
  // stages past the last re-load the last one and skip their MFMAs
  const int nst = K / 128;
  const int lastst = nst > 0 ? nst - 1 : 0;
  if (nst > 0) {
    load_a(0, ra);
#pragma unroll
    for (int r = 0; r < P; ++r) load_b(r < lastst ? r : lastst, rb[r]);
    stage_a(0, ra);
  }
  lds_barrier();
  for (int i = 0; i < nst; i += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int it = i + r;
      load_a(it + 1 < lastst ? it + 1 : lastst, ra);
      load_b(it + P < lastst ? it + P : lastst, rb[(r + P) % R]);
      if constexpr (DG_LOAD_FENCE) __builtin_amdgcn_sched_barrier(0);   // as in wide_tile
      if (it < nst) compute(it & 1, rb[r]);
      stage_a((it + 1) & 1, ra);
      lds_barrier();
    }
  }

#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int c = wave * (NTW * 16) + nt * 16 + l16;
    if (c >= ncols) continue;
    const int col = n0 + c;
    const float sg = Sp[0][c], su = Sp[1][c];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mi * 16 + lg * 4 + i;
        if (r >= rows) continue;
        const long long row = row_begin + r;
        const float v = acc[0][mi][nt][i] * sg, u = acc[1][mi][nt][i] * su;
        static_cast<bf16_t *>(a.C)[row * a.ldc + col] = f32_to_bf16(silu_f(v) * u);
      }
  }
}

template <int MT, int NTW, int NW, int P>
__global__ __launch_bounds__(64 * NW) void gemm_wide_f8_kernel(const GemmArgs a) {
  constexpr int BM = MT * 16, BN = NW * NTW * 16;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb[NW * 2 * NTW * 16 * 128];
  int g, n0;
  grouped_item(g, n0, BN, DG_GROUPED_XCD && MT <= 2);
  const bool sh = g < a.n_xgroups;
  const int Ng = sh ? a.N_x : a.N;
  if (n0 >= Ng) return;
  GemmArgs ga = a;
  const uint8_t *Bp[2];
  const float *Sp[2];
  if (sh) {
    ga.K = a.K_x;
    ga.ldb = a.ldb_x;
    Bp[0] = static_cast<const uint8_t *>(a.Bx0) + static_cast<long long>(n0) * a.ldb_x;
    Bp[1] = static_cast<const uint8_t *>(a.Bx1) + static_cast<long long>(n0) * a.ldb_x;
    Sp[0] = a.bxs0 + n0;
    Sp[1] = a.bxs1 + n0;
  } else {
    const int e = g - a.n_xgroups;
    const long long off = static_cast<long long>(e) * a.b_gstride + static_cast<long long>(n0) * a.ldb;
    Bp[0] = static_cast<const uint8_t *>(a.seg_B0[0]) + off;
    Bp[1] = static_cast<const uint8_t *>(a.seg_B1[0]) + off;
    Sp[0] = a.bs0 + static_cast<long long>(e) * a.N + n0;
    Sp[1] = a.bs1 + static_cast<long long>(e) * a.N + n0;
  }
  const int r0 = a.g_off[g], r1 = a.g_off[g + 1];
  for (int rb = r0; rb < r1; rb += BM)
    wide_tile_f8<MT, NTW, NW, P>(ga, lds, ldsb, rb, min(BM, r1 - rb), Bp, Sp, n0, min(BN, Ng - n0), ga.K);
}

template <int MT, int NTW, int NB, int NW, int KSUB, int P, int MODE>
hipError_t launch_wide_one(const GemmArgs &a, hipStream_t s) {
  constexpr int BM = MT * 16, BN = NW * NTW * 16;
  dim3 grid;
  if (a.g_off) {
    const int nmax = a.N > a.N_x ? a.N : a.N_x;
    grid = dim3((nmax + BN - 1) / BN, a.n_groups);
  } else {
    const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
    grid = dim3(mt * nt * a.k_splits, 1);
  }
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_wide_kernel<MT, NTW, NB, NW, KSUB, P, MODE>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Grouped product of short depth (the expert down projection, k = F) with
// several work items per workgroup and each wave's load ring carried from one
// item to the next.
//
// A work item is one 16*NT-column tile of one group for one block of 16*MT
// rows.  At k = 704 a wave owns only three 64-deep stages of an item, so with
// one item per workgroup every wave first waits a whole HBM latency for its
// first stage and has no loads in flight while the workgroup reduces and
// stores.  Here the G workgroups stay resident and workgroup b takes items
// b, b + G, b + 2G, ... (items ordered by group, column tile, row block), so
// the live workgroups sweep the weights together through a narrow window;
// a wave issues the loads of the next item's stage s as soon as it has
// consumed stage s of the current one: the next item's weights stream in
// during the rest of the current item, its reduction and its stores.
//
// Wave w owns stages w, w+4, ...  Its ring holds exactly its stages of one
// item, so ring slots are compile-time constants.  Every load is issued
// unconditionally (after the last item they re-read one 16-byte chunk of the
// activation rows), and the routing weights of an item are loaded before the
// next item's stages, so the compiler's wait counts never drain the ring.
// The cross-wave reduction alternates between two LDS buffers behind one
// LDS-only barrier per item.
constexpr int kDnMaxGroups = 1024;
// LDS pitch (floats) of one accumulator element's 64 lanes in the reduction
// buffer: 4 extra floats spread the row-major reads over the banks
constexpr int kDnPitch = 68;

struct DnItem {
  const char *B;    // first weight row of the column tile
  const float *S;   // its per-row weight scales (fp8 weights only)
  long long ldb;    // weight row stride (elements)
  int row0, rows;   // logical rows [row0, row0 + rows)
  int n0, ncols;    // output columns [n0, n0 + ncols)
};

// ESZ: bytes per weight element (2: bf16, 1: fp8 e4m3 with per-row scales)
template <int BM, int BN, int ESZ>
__device__ __forceinline__ DnItem dn_decode(const GemmArgs &a, const int *pre, const int *goff, int ng, int item) {
  // group g with pre[g] <= item < pre[g + 1] (groups without items have pre[g] == pre[g + 1])
  int lo = 0, hi = ng;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (__builtin_amdgcn_readfirstlane(pre[mid]) <= item) lo = mid;
    else hi = mid;
  }
  const int g = lo;
  const int r0 = __builtin_amdgcn_readfirstlane(goff[g]);
  const int r1 = __builtin_amdgcn_readfirstlane(goff[g + 1]);
  const int nrb = (r1 - r0 + BM - 1) / BM;
  const int local = item - __builtin_amdgcn_readfirstlane(pre[g]);
  const int ct = local / nrb, rb = local - ct * nrb;
  DnItem it;
  it.n0 = ct * BN;
  it.row0 = r0 + rb * BM;
  it.rows = min(BM, r1 - it.row0);
  if (g < a.n_xgroups) {
    it.ncols = min(BN, a.N_x - it.n0);
    it.ldb = a.ldb_x;
    it.B = static_cast<const char *>(a.Bx0) + static_cast<long long>(it.n0) * a.ldb_x * ESZ;
    it.S = ESZ == 1 ? a.bxs0 + it.n0 : nullptr;
  } else {
    const int e = g - a.n_xgroups;
    it.ncols = min(BN, a.N - it.n0);
    it.ldb = a.ldb;
    it.B = static_cast<const char *>(a.seg_B0[0]) +
           (static_cast<long long>(e) * a.b_gstride + static_cast<long long>(it.n0) * a.ldb) * ESZ;
    it.S = ESZ == 1 ? a.bs0 + static_cast<long long>(e) * a.N + it.n0 : nullptr;
  }
  return it;
}

// F8: OCP E4M3 weights with one fp32 scale per weight row, widened to bf16
// in registers.  A stage is then 128 deep (128 weight bytes per row, as in
// stream_tile_f8): its activation rows are two 64-deep halves, and with
// k % 128 == 64 the last stage is 64 deep (its second-half weight loads
// re-read the first half and the second-half activation fragments are
// zeroed).  The scales are applied per column in the epilogue, before the
// routing weight.
template <int MT, int NT, int SW, int MODE, bool F8>
__device__ __forceinline__ void dn_walk(const GemmArgs &a, float *red, const int *pre, const int *goff, int ng,
                                        int total) {
  constexpr int BM = MT * 16, BN = NT * 16, EL = MT * NT * 4;
  constexpr int JH = F8 ? 2 : 1;         // activation halves per stage
  constexpr int ESZ = F8 ? 1 : 2;        // weight bytes per element
  constexpr int NQ = EL * 16 / 256;   // epilogue quads per thread
  static_assert(EL * 16 % 256 == 0, "epilogue quads must divide among the workgroup");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cr = contig_row(lane), cc = contig_chunk(lane);
  const int hb = (lane & 15) >> 3, lg = lane >> 4;
  const int ca = F8 ? 2 * lg + hb : cc;   // activation chunk (8 elements) inside a 64-deep block
  const char *Ab = static_cast<const char *>(a.A);

  uint32_t ao[MT][2], bo[NT][2];
  const char *Bn;
  auto point_at = [&](const DnItem &it) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = mt * 16 + h * 8 + cr;
        ao[mt][h] = (static_cast<uint32_t>(it.row0 + (r < it.rows ? r : 0)) * static_cast<uint32_t>(a.lda) + ca * 8) * 2u;
      }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = nt * 16 + h * 8 + cr;
        bo[nt][h] = F8 ? static_cast<uint32_t>(c < it.ncols ? c : 0) * static_cast<uint32_t>(it.ldb) + cc * 16
                       : (static_cast<uint32_t>(c < it.ncols ? c : 0) * static_cast<uint32_t>(it.ldb) + cc * 8) * 2u;
      }
    Bn = it.B;
  };
  auto point_idle = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ao[mt][0] = ao[mt][1] = 0u;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bo[nt][0] = bo[nt][1] = 0u;
    Bn = Ab;
  };

  bf16x8 xa[SW][MT][JH][2];
  bf16x8 xb[SW][NT][2];
  auto load = [&](int st, bf16x8(&ya)[MT][JH][2], bf16x8(&yb)[NT][2]) {
    const int sg = wave + 4 * st;   // stage of the item
    if constexpr (F8) {
      const bool half = (sg + 1) * 128 > a.K;
      const uint32_t kb = static_cast<uint32_t>(sg) * 128u - ((half && hb) ? 64u : 0u);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h) yb[nt][h] = ld_stream(Bn + (bo[nt][h] + kb));
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        const uint32_t ka = (static_cast<uint32_t>(sg) * 128u + (half ? 0u : 64u * jh)) * 2u;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int h = 0; h < 2; ++h) ya[mt][jh][h] = *reinterpret_cast<const bf16x8 *>(Ab + (ao[mt][h] + ka));
      }
    } else {
      const uint32_t kbyte = static_cast<uint32_t>(sg) * 128u;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h) yb[nt][h] = ld_stream(Bn + (bo[nt][h] + kbyte));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) ya[mt][0][h] = *reinterpret_cast<const bf16x8 *>(Ab + (ao[mt][h] + kbyte));
    }
  };
  f32x4 acc[MT][NT];
  auto compute = [&](int st, const bf16x8(&ya)[MT][JH][2], const bf16x8(&yb)[NT][2]) {
    if constexpr (F8) {
      const bool half = (wave + 4 * st + 1) * 128 > a.K;
      Frag<bf16_t> fa[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        contig_to_frags(ya[mt][0][0], ya[mt][0][1], fa[mt][0].v, fa[mt][1].v);
        contig_to_frags(ya[mt][1][0], ya[mt][1][1], fa[mt][2].v, fa[mt][3].v);
        if (half) {
          fa[mt][2].v = bf16x8{};
          fa[mt][3].v = bf16x8{};
        }
      }
      // weight fragments are widened one 16-column block at a time
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 f0, f1;
        contig_to_frags(yb[nt][0], yb[nt][1], f0, f1);
        Frag<bf16_t> fb[4];
        e4m3x16_to_bf16(f0, fb[0].v, fb[1].v);
        e4m3x16_to_bf16(f1, fb[2].v, fb[3].v);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) mma(acc[mt][nt], fa[mt][ks], fb[ks]);
      }
    } else {
      Frag<bf16_t> fb[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) contig_to_frags(yb[nt][0], yb[nt][1], fb[nt][0].v, fb[nt][1].v);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Frag<bf16_t> fa[2];
        contig_to_frags(ya[mt][0][0], ya[mt][0][1], fa[0].v, fa[1].v);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(acc[mt][nt], fa[ks], fb[nt][ks]);
      }
    }
  };

  // item j of this workgroup: b + j G (the live workgroups sweep the weights
  // together; contiguous item ranges per workgroup measured 13% slower)
  auto item_of = [&](int j) { return static_cast<int>(blockIdx.x) + j * static_cast<int>(gridDim.x); };
  DnItem cur = dn_decode<BM, BN, ESZ>(a, pre, goff, ng, item_of(0));
  point_at(cur);
#pragma unroll
  for (int st = 0; st < SW; ++st) {
    load(st, xa[st], xb[st]);
    __builtin_amdgcn_sched_barrier(0);   // stages in order: the loop waits on them oldest first
  }

  for (int j = 0, buf = 0; item_of(j) < total; ++j, buf ^= 1) {
    // rows this thread stores in the epilogue, and their routing weights
    // (loaded ahead of the next item's stages; see above)
    float rs[NQ];
    float4 sc[NQ];   // weight scales of the 4 columns (fp8)
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int r = (tid + 256 * j) / (BN / 4);
      if constexpr (F8) {
        const int c = ((tid + 256 * j) % (BN / 4)) * 4;
        sc[j] = *reinterpret_cast<const float4 *>(cur.S + (c + 4 <= cur.ncols ? c : 0));
      }
      rs[j] = MODE == EPI_ROWSCALE_F32 ? a.rowscale[cur.row0 + (r < cur.rows ? r : 0)] : 1.f;
    }
    // keep these loads ahead of the stage loads below, and each stage's
    // fragment moves after the wait for that stage only
    __builtin_amdgcn_sched_barrier(0);
    DnItem nxt = cur;
    if (item_of(j + 1) < total) {
      nxt = dn_decode<BM, BN, ESZ>(a, pre, goff, ng, item_of(j + 1));
      point_at(nxt);
    } else {
      point_idle();
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = zero4();
#pragma unroll
    for (int st = 0; st < SW; ++st) {
      compute(st, xa[st], xb[st]);
      load(st, xa[st], xb[st]);
      __builtin_amdgcn_sched_barrier(0);
    }

    float *rbuf = red + buf * (4 * EL * kDnPitch);
    {
      float *dst = rbuf + wave * EL * kDnPitch;
      int e = 0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int k = 0; k < 4; ++k, ++e) dst[e * kDnPitch + lane] = acc[mt][nt][k];
    }
    lds_barrier();
    // each thread adds up, over the 4 waves, 4 consecutive columns of one row
    // (4 neighbouring lanes of one accumulator element); a wave covers whole
    // rows of the tile, so each store instruction writes whole cache lines
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = tid + 256 * j, r = q / (BN / 4), c = (q % (BN / 4)) * 4;
      const int e = ((r >> 4) * NT + (c >> 4)) * 4 + (r & 3);
      const int l4 = ((r & 15) >> 2) * 16 + (c & 15);
      float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float4 t = *reinterpret_cast<const float4 *>(rbuf + (w * EL + e) * kDnPitch + l4);
        v[0] += t.x; v[1] += t.y; v[2] += t.z; v[3] += t.w;
      }
      if (r < cur.rows && c < cur.ncols) {
        const long long off = static_cast<long long>(cur.row0 + r) * a.ldc + cur.n0 + c;
        float *cp = static_cast<float *>(a.C) + off;
        const int nv = cur.ncols - c < 4 ? cur.ncols - c : 4;
        if constexpr (F8) {
          v[0] *= sc[j].x;
          v[1] *= sc[j].y;
          v[2] *= sc[j].z;
          v[3] *= sc[j].w;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] *= rs[j];
        if (nv == 4 && (off & 3) == 0) {
          // non-temporal: the rows are read once, by the combine pass
          const f32x4 q4 = {v[0], v[1], v[2], v[3]};
          __builtin_nontemporal_store(q4, reinterpret_cast<f32x4 *>(cp));
        } else {
          for (int u = 0; u < nv; ++u) cp[u] = v[u];
        }
      }
    }
    cur = nxt;
  }
}

template <int MT, int NT, int SPW, int MODE, bool F8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_down_ring_kernel(const GemmArgs a) {
  constexpr int BM = MT * 16, BN = NT * 16, EL = MT * NT * 4;
  __shared__ __attribute__((aligned(16))) float red[2 * 4 * EL * kDnPitch];
  __shared__ int pre[kDnMaxGroups + 1], goff[kDnMaxGroups + 1];
  const int ng = a.n_groups, tid = threadIdx.x;
  for (int g = tid; g <= ng; g += 256) goff[g] = a.g_off[g];
  __syncthreads();
  // items per group, then their running sum (wave 0, 64 groups at a time)
  for (int g = tid; g < ng; g += 256) {
    const int Ng = g < a.n_xgroups ? a.N_x : a.N;
    pre[g + 1] = ((goff[g + 1] - goff[g] + BM - 1) / BM) * ((Ng + BN - 1) / BN);
  }
  __syncthreads();
  if (tid < 64) {
    int carry = 0;
    for (int base = 1; base <= ng; base += 64) {
      const int idx = base + tid;
      int v = idx <= ng ? pre[idx] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(v, off, 64);
        if (tid >= off) v += t;
      }
      if (idx <= ng) pre[idx] = v + carry;
      carry += __shfl(v, 63, 64);
    }
    if (tid == 0) pre[0] = 0;
  }
  __syncthreads();
  const int total = pre[ng];
  if (static_cast<int>(blockIdx.x) >= total) return;
  // a wave owns (nsteps - wave + 3) / 4 stages: SPW or SPW - 1 (checked on the host)
  const int nsteps = F8 ? (a.K + 127) / 128 : a.K / 64;
  const int wave = tid >> 6;
  if ((nsteps - wave + 3) / 4 == SPW) dn_walk<MT, NT, SPW, MODE, F8>(a, red, pre, goff, ng, total);
  else dn_walk<MT, NT, SPW - 1, MODE, F8>(a, red, pre, goff, ng, total);
}

}  // namespace

template <typename T>
hipError_t launch_gemm(const GemmArgs &a, int mode, int bm, int bn, hipStream_t s) {
#define DG_GEMM_CASE(BM_, BN_, NB_, MODE_) \
  if (bm == BM_ && bn == BN_ && mode == MODE_) return launch_one<T, BM_, BN_, NB_, MODE_>(a, s);
  DG_GEMM_CASE(64, 128, 1, EPI_STORE)
  DG_GEMM_CASE(64, 128, 1, EPI_STORE_F32)
  DG_GEMM_CASE(64, 128, 1, EPI_ADD)
  DG_GEMM_CASE(64, 128, 1, EPI_PARTIAL_F32)
  DG_GEMM_CASE(64, 64, 2, EPI_SWIGLU)
  DG_GEMM_CASE(32, 64, 2, EPI_SWIGLU)
  DG_GEMM_CASE(32, 64, 1, EPI_ROWSCALE_F32)
  if constexpr (sizeof(T) == 2) {
    DG_GEMM_CASE(128, 64, 2, EPI_SWIGLU)
    DG_GEMM_CASE(128, 64, 1, EPI_ROWSCALE_F32)
  }
#undef DG_GEMM_CASE
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_gemm_stream(const GemmArgs &a, int mode, int mt, int nt, hipStream_t s) {
#define DG_STREAM_CASE(MT_, NT_, NB_, MODE_, S_) \
  if (mt == MT_ && nt == NT_ && mode == MODE_) return launch_stream_one<T, MT_, NT_, NB_, MODE_, S_>(a, s);
  DG_STREAM_CASE(DG_DENSE_MT, DG_DENSE_NT, 1, EPI_STORE, DG_DENSE_S)
  DG_STREAM_CASE(DG_DENSE_MT, DG_DENSE_NT, 1, EPI_STORE_F32, DG_DENSE_S)
  DG_STREAM_CASE(DG_DENSE_MT, DG_DENSE_NT, 1, EPI_ADD, DG_DENSE_S)
  DG_STREAM_CASE(DG_DENSE_MT, DG_DENSE_NT, 1, EPI_PARTIAL_F32, DG_DENSE_S)
  DG_STREAM_CASE(1, 1, 1, EPI_STORE_F32, 3)     // router logits: 16 x 16 tiles, whole depth
  DG_STREAM_CASE(1, 1, 1, EPI_PARTIAL_F32, 3)   // router logits as split-K partials
  DG_STREAM_CASE(DG_MOE_MT, DG_MOE_NT_GU, 2, EPI_SWIGLU, DG_GU_S)
  DG_STREAM_CASE(DG_DN_MT, DG_MOE_NT_DN, 1, EPI_ROWSCALE_F32, DG_MOE_S)
  DG_STREAM_CASE(DG_MOE_MT, DG_MOE_NT_DN, 1, EPI_ROWSCALE_F32, DG_MOE_S)
  DG_STREAM_CASE(4, DG_MOE_NT_GU, 2, EPI_SWIGLU, 3)
  DG_STREAM_CASE(4, DG_MOE_NT_DN, 1, EPI_ROWSCALE_F32, 3)
#undef DG_STREAM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f8_grouped(const GemmArgs &a, int mode, int mt, hipStream_t s) {
  if (!a.g_off || a.K % 64 || a.K_x % 64 || a.ldb % 16 || a.ldb_x % 16 || a.lda % 8) return hipErrorInvalidValue;
#define DG_F8_CASE(MODE_, MT_, NT_, NB_, S_) \
  if (mode == MODE_ && mt == MT_) return launch_f8_one<MT_, NT_, NB_, MODE_, S_>(a, s);
  DG_F8_CASE(EPI_SWIGLU, DG_MOE_MT, DG_F8_NT_GU, 2, DG_F8_S)
  DG_F8_CASE(EPI_ROWSCALE_F32, DG_MOE_MT, DG_F8_NT_DN, 1, DG_F8_S)
  DG_F8_CASE(EPI_SWIGLU, 4, DG_F8_NT_GU, 2, DG_F8_S)
  DG_F8_CASE(EPI_ROWSCALE_F32, 4, DG_F8_NT_DN, 1, DG_F8_S)
#undef DG_F8_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_wide_f8_gu(const GemmArgs &a, hipStream_t s) {
  constexpr int MT = DG_WMOE_MT, NTW = 1, NW = 4, BN = NW * NTW * 16;
  if (!a.g_off || a.K % 128 || a.K_x % 128 || a.ldb % 16 || a.ldb_x % 16 || a.lda % 8 || !a.bs0 || !a.bs1 ||
      !a.bxs0 || !a.bxs1)
    return hipErrorNotSupported;
  // 32-bit byte offsets: every activation row and every weight tile
  if (static_cast<long long>(a.M) * a.lda * 2 >= (1ll << 31) ||
      static_cast<long long>(a.N > a.N_x ? a.N : a.N_x) * (a.ldb > a.ldb_x ? a.ldb : a.ldb_x) >= (1ll << 31))
    return hipErrorNotSupported;
  const int nmax = a.N > a.N_x ? a.N : a.N_x;
  const dim3 grid((nmax + BN - 1) / BN, a.n_groups);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_wide_f8_kernel<MT, NTW, NW, DG_WMOE_P>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_wide(const GemmArgs &a, int mode, int cfg, hipStream_t s) {
#define DG_WIDE_CASE(CFG_, MT_, NTW_, NB_, NW_, KSUB_, P_, MODE_) \
  if (cfg == CFG_ && mode == MODE_) return launch_wide_one<MT_, NTW_, NB_, NW_, KSUB_, P_, MODE_>(a, s);
  DG_WIDE_CASE(WIDE_ROWS256_N256, 16, 2, 1, 8, 2, DG_WIDE256_P, EPI_STORE_F32)
  DG_WIDE_CASE(WIDE_ROWS256_N256, 16, 2, 1, 8, 2, DG_WIDE256_P, EPI_PARTIAL_F32)
  DG_WIDE_CASE(WIDE_ROWS256_N256, 16, 2, 1, 8, 2, DG_WIDE256_P, EPI_STORE)
  DG_WIDE_CASE(WIDE_ROWS256_N256, 16, 2, 1, 8, 2, DG_WIDE256_P, EPI_ADD)
  DG_WIDE_CASE(WIDE_ROWS256_N128, 16, 1, 1, 8, 2, DG_WIDE_P, EPI_STORE)
  DG_WIDE_CASE(WIDE_ROWS256_N128, 16, 1, 1, 8, 2, DG_WIDE_P, EPI_PARTIAL_F32)
  DG_WIDE_CASE(WIDE_ROWS256_N128, 16, 1, 1, 8, 2, DG_WIDE_P, EPI_STORE_F32)
  DG_WIDE_CASE(WIDE_ROWS256_N128, 16, 1, 1, 8, 2, DG_WIDE_P, EPI_ADD)
  DG_WIDE_CASE(WIDE_ROWS256_N128_OP, 16, 1, 1, 8, 2, DG_OPROJ_P, EPI_PARTIAL_F32)
  DG_WIDE_CASE(WIDE_ROWS256_N128_OP, 16, 1, 1, 8, 2, DG_OPROJ_P, EPI_ADD)
  DG_WIDE_CASE(WIDE_EXPERT_GU, DG_WMOE_MT, 1, 2, 4, 2, DG_WMOE_P, EPI_SWIGLU)
  DG_WIDE_CASE(WIDE_EXPERT_DN, DG_WMOE_MT, 2, 1, 4, 2, DG_WMOE_P, EPI_ROWSCALE_F32)
  DG_WIDE_CASE(WIDE_EXPERT_GU_L, 16, 1, 2, 8, 2, DG_WIDE_P, EPI_SWIGLU)
  DG_WIDE_CASE(WIDE_EXPERT_DN_L, 16, 1, 1, 8, 2, DG_WIDE_P, EPI_ROWSCALE_F32)
#undef DG_WIDE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_down_ring(const GemmArgs &a, int mt, bool fp8, hipStream_t s) {
  constexpr int MT = DG_DN_MT, NT = DG_MOE_NT_DN;
  if (mt != MT || !a.g_off || a.a_rows || a.K != a.K_x || a.K % 64 || a.n_groups < 1 || a.n_groups > kDnMaxGroups ||
      a.lda % 8 || a.ldb % 8 || a.ldb_x % 8 || a.ldc % 4 || !a.rowscale)
    return hipErrorNotSupported;
  // fp8 rows are read 16 bytes at a time and scaled per row
  if (fp8 && (a.ldb % 16 || a.ldb_x % 16 || !a.bs0 || !a.bxs0)) return hipErrorNotSupported;
  // 32-bit lane offsets: every activation row and every weight tile
  if (static_cast<long long>(a.M) * a.lda * 2 >= (1ll << 31) || 16ll * NT * (a.ldb > a.ldb_x ? a.ldb : a.ldb_x) * 2 >= (1ll << 31))
    return hipErrorNotSupported;
  const int nsteps = fp8 ? (a.K + 127) / 128 : a.K / 64, spw = (nsteps + 3) / 4;
  const dim3 grid(DG_DN_RING_WG);
  // (the fp8 form with three stages per wave does not fit the registers)
  if (spw == 3 && nsteps > 8 && !fp8) {
    hipLaunchKernelGGL((gemm_down_ring_kernel<MT, NT, 3, EPI_ROWSCALE_F32, false>), grid, dim3(256), 0, s, a);
  } else if (spw == 2 && nsteps > 4) {
    if (fp8) hipLaunchKernelGGL((gemm_down_ring_kernel<MT, NT, 2, EPI_ROWSCALE_F32, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gemm_down_ring_kernel<MT, NT, 2, EPI_ROWSCALE_F32, false>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_splitk_reduce(const float *part, int splits, int M, int N, long long ldc, void *C,
                                int mode, hipStream_t s) {
  const long long n8 = static_cast<long long>(M) * N / 8;
  if (n8 == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, s,
                     part, splits, M, N, ldc, C, mode);
  return hipGetLastError();
}

template hipError_t launch_gemm<bf16_t>(const GemmArgs &, int, int, int, hipStream_t);
template hipError_t launch_gemm<float>(const GemmArgs &, int, int, int, hipStream_t);
template hipError_t launch_gemm_stream<bf16_t>(const GemmArgs &, int, int, int, hipStream_t);
template hipError_t launch_gemm_stream<float>(const GemmArgs &, int, int, int, hipStream_t);
template hipError_t launch_splitk_reduce<bf16_t>(const float *, int, int, int, long long, void *, int, hipStream_t);
template hipError_t launch_splitk_reduce<float>(const float *, int, int, int, long long, void *, int, hipStream_t);

}  // namespace dg
