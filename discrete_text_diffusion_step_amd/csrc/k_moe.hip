// MoE routing for the canvas step (gfx950): top-k router, expert batching,
// deterministic combine (aitrends notebook summary, glossary "MoE":
// exp(router key . x) scores, renormalised over the chosen experts and
// scaled; tokens routed to one expert are processed together; the shared
// expert is always added).
//
// Group layout produced by moe_permute (consumed by the grouped GEMM):
//   groups 0..X-1    : the shared expert, rows [0, n_tok) in token order, cut
//                      into X chunks of `chunk` rows (parallel workgroups)
//   group X + e      : routed expert e, rows sorted by (token, slot)
// so g_off has X + n_experts + 1 entries.  row_token[r] is the token of row r,
// row_weight[r] its mixing weight (1 for the shared expert) and pair_row[t*k+j]
// the row holding token t's j-th expert.
#include "dg_launch.h"

namespace dg {

namespace {

// Order-preserving 32-bit key of a float (larger float -> larger key); NaN
// sorts below every number.
__device__ __forceinline__ uint32_t float_key(float v) {
  const uint32_t u = __float_as_uint(v);
  if (v != v) return 1u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One step of the 64-bit wave maximum: compare with the DPP-moved pair.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void max64_step(uint32_t &hi, uint32_t &lo) {
  const uint32_t oh = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(hi), static_cast<int>(hi), CTRL, ROW_MASK, 0xF, false));
  const uint32_t ol = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(lo), static_cast<int>(lo), CTRL, ROW_MASK, 0xF, false));
  const bool take = oh > hi || (oh == hi && ol > lo);
  hi = take ? oh : hi;
  lo = take ? ol : lo;
}

// Largest (hi, lo) pair over the wave, returned to every lane: DPP row shifts
// accumulate each 16-lane row's maximum into its lane 15, row broadcasts
// carry it to lanes 31 and 63, and lane 63 is read out.
__device__ __forceinline__ void wave_max64(uint32_t &hi, uint32_t &lo) {
  max64_step<0x111, 0xF>(hi, lo);   // row_shr:1
  max64_step<0x112, 0xF>(hi, lo);   // row_shr:2
  max64_step<0x114, 0xF>(hi, lo);   // row_shr:4
  max64_step<0x118, 0xF>(hi, lo);   // row_shr:8
  max64_step<0x142, 0xA>(hi, lo);   // row_bcast:15 into rows 1 and 3
  max64_step<0x143, 0xC>(hi, lo);   // row_bcast:31 into rows 2 and 3
  hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), 63));
  lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), 63));
}

// One wave per token.  Top-k by logit, ties to the lower expert id: each
// (logit, expert) is one 64-bit key (order-preserving logit, then the
// complemented expert id), so k rounds of a wave maximum pick the experts in
// order.  Weights are the softmax restricted to the chosen experts (the
// full-softmax denominator cancels in the renormalisation) times route_scale.
__global__ __launch_bounds__(256) void router_topk_kernel(const float *logits, int n_parts, int n_tok, int E,
                                                          int k, float scale, int32_t *idx_out, float *w_out) {
  const int lane = threadIdx.x & 63;
  // wave-uniform token: the row base lives in scalar registers, so each load
  // needs only a per-lane offset
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (t >= n_tok) return;
  const long long part_stride = static_cast<long long>(n_tok) * E;
  const float *r = logits + static_cast<long long>(t) * E;
  // the logit is the sum of the split-K partials, in split order; the first
  // kMaxParts partials of all four experts are loaded before any is added,
  // so the wave waits for memory once
  constexpr int kMaxParts = 8;
  float pv[4][kMaxParts];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p)
      if (e < E && p < n_parts)
        pv[i][p] = logits[static_cast<uint32_t>(p * part_stride + static_cast<long long>(t) * E + e)];
  }
  uint32_t kh[4], kl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    float v = 0.f;
    if (e < E) {
      v = pv[i][0];
#pragma unroll
      for (int p = 1; p < kMaxParts; ++p)
        if (p < n_parts) v += pv[i][p];
      for (int p = kMaxParts; p < n_parts; ++p) v += r[p * part_stride + e];
    }
    kh[i] = e < E ? float_key(v) : 0u;
    kl[i] = e < E ? 0xffffffffu - static_cast<uint32_t>(e) : 0u;
  }
  float chosen_v[8];
  int chosen_e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    chosen_v[j] = 0.f;
    chosen_e[j] = 0;
    if (j < k) {
      uint32_t bh = kh[0], bl = kl[0];
#pragma unroll
      for (int i = 1; i < 4; ++i)
        if (kh[i] > bh || (kh[i] == bh && kl[i] > bl)) {
          bh = kh[i];
          bl = kl[i];
        }
      wave_max64(bh, bl);
      chosen_v[j] = key_float(bh);
      chosen_e[j] = static_cast<int>(0xffffffffu - bl);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (kh[i] == bh && kl[i] == bl) kh[i] = kl[i] = 0u;   // taken
    }
  }
  float p[8], sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = j < k ? __expf(chosen_v[j] - chosen_v[0]) : 0.f;
    sum += p[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k && lane == j) {
      idx_out[static_cast<long long>(t) * k + j] = chosen_e[j];
      w_out[static_cast<long long>(t) * k + j] = p[j] / sum * scale;
    }
}

// One workgroup of 16 waves: counts (LDS integer atomics), an exclusive wave
// scan over the experts, then a stable scatter.  Pairs are staged in LDS in
// chunks; each wave takes a contiguous run of 64-pair blocks and ranks every
// pair among the earlier pairs of the same expert in its run (ballots over
// the bits of the expert id, per-wave running counts); a prefix over the
// waves, in wave order, turns the per-wave counts into row bases.  Rows of
// an expert thus come out sorted by (token, slot).  Integer work only:
// bit-exact and independent of scheduling.
constexpr int kPermWaves = 16;
constexpr int kPermChunk = 4096;

__global__ __launch_bounds__(64 * kPermWaves) void moe_permute_kernel(const int32_t *idx, const float *w, int n_tok,
                                                                      int k, int E, int chunk, int *g_off,
                                                                      int *row_token, float *row_weight,
                                                                      int *pair_row) {
  __shared__ int cnt[256];
  __shared__ int start[256];   // next free row of each expert
  __shared__ int hist[kPermWaves][256];
  __shared__ int s_e[kPermChunk];
  __shared__ float s_w[kPermChunk];
  __shared__ int s_rank[kPermChunk];
  constexpr int NT = 64 * kPermWaves;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < 256; e += NT) cnt[e] = 0;
  __syncthreads();
  const int n_pairs = n_tok * k;
  for (int p = tid; p < n_pairs; p += NT) {
    int e = idx[p];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (wave == 0) {
    // lane l holds experts 4l..4l+3; routed rows start after the n_tok shared rows
    int c[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? cnt[e] : 0;
      local += c[i];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int X = (n_tok + chunk - 1) / chunk;   // shared-expert row chunks
    int run = n_tok + incl - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        start[e] = run;
        g_off[X + 1 + e] = run + c[i];
      }
      run += c[i];
    }
    for (int x = lane; x <= X; x += 64) g_off[x] = min(x * chunk, n_tok);
  }
  for (int t = tid; t < n_tok; t += NT) {
    row_token[t] = t;
    row_weight[t] = 1.0f;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n_pairs; base += kPermChunk) {
    const int len = min(kPermChunk, n_pairs - base);
    __syncthreads();   // previous chunk consumed; start[] visible
    for (int p = tid; p < len; p += NT) {
      int e = idx[base + p];
      s_e[p] = e < 0 ? 0 : (e >= E ? E - 1 : e);
      s_w[p] = w[base + p];
    }
    for (int i = tid; i < kPermWaves * 256; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();
    const int nblk = (len + 63) / 64;
    const int per = (nblk + kPermWaves - 1) / kPermWaves;
    const int b0 = wave * per, b1 = min(nblk, b0 + per);
    for (int b = b0; b < b1; ++b) {
      const int q = b * 64 + lane;
      const bool valid = q < len;
      const int e = valid ? s_e[q] : -1;
      const unsigned key = static_cast<unsigned>(e + 1);   // 0 = no pair
      uint64_t peers = __ballot(1);
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) {
        const bool on = (key >> bit) & 1u;
        const uint64_t m = __ballot(on);
        peers &= on ? m : ~m;
      }
      const int rank = __popcll(peers & lt_mask);
      const int old = valid ? hist[wave][e] : 0;   // all lanes read before the leaders write
      if (valid && rank == 0) hist[wave][e] = old + __popcll(peers);
      if (valid) s_rank[q] = old + rank;
    }
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
      int run = start[e];
      for (int v = 0; v < kPermWaves; ++v) {
        const int c = hist[v][e];
        hist[v][e] = run;
        run += c;
      }
      start[e] = run;
    }
    __syncthreads();
    for (int b = b0; b < b1; ++b) {
      const int q = b * 64 + lane;
      if (q < len) {
        const int row = hist[wave][s_e[q]] + s_rank[q];
        const int p = base + q;
        row_token[row] = p / k;
        row_weight[row] = s_w[q];
        pair_row[p] = row;
      }
    }
  }
}

// x[t] <- layer_scalar * (x[t] + Y[shared row t] + sum_j Y[pair_row[t*k+j]])
// Y rows already carry their routing weight.  Fixed summation order.
template <typename T>
__global__ __launch_bounds__(256) void moe_combine_kernel(T *x, const float *Y, const int *pair_row, int n_tok,
                                                          int k, int D, float ls) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= D) return;
  float y[8];
  load8(Y + static_cast<long long>(t) * D + c, y);
  for (int j = 0; j < k; ++j) {
    float v[8];
    load8(Y + static_cast<long long>(pair_row[t * k + j]) * D + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] += v[i];
  }
  T *xp = x + static_cast<long long>(t) * D + c;
  float xv[8];
  load8(xp, xv);
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = ls * (xv[i] + y[i]);
  store8(xp, xv);
}

}  // namespace

hipError_t launch_router_topk(const float *logits, int n_parts, int n_tok, int E, int k, float scale, int32_t *idx,
                              float *w, hipStream_t s) {
  if (n_tok <= 0) return hipSuccess;
  hipLaunchKernelGGL(router_topk_kernel, dim3((n_tok + 3) / 4), dim3(256), 0, s, logits, n_parts, n_tok, E, k, scale,
                     idx, w);
  return hipGetLastError();
}

hipError_t launch_moe_permute(const int32_t *idx, const float *w, int n_tok, int k, int E, int chunk, int *g_off,
                              int *row_token, float *row_weight, int *pair_row, hipStream_t s) {
  if (chunk <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_permute_kernel, dim3(1), dim3(64 * kPermWaves), 0, s, idx, w, n_tok, k, E, chunk, g_off,
                     row_token, row_weight, pair_row);
  return hipGetLastError();
}

hipError_t launch_moe_combine(int dtype, void *x, const float *Y, const int *pair_row, int n_tok, int k, int D,
                              float layer_scalar, hipStream_t s) {
  if (n_tok <= 0) return hipSuccess;
  dim3 grid((D / 8 + 255) / 256, n_tok);
  if (dtype == DG_BF16)
    hipLaunchKernelGGL(moe_combine_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<bf16_t *>(x), Y, pair_row,
                       n_tok, k, D, layer_scalar);
  else
    hipLaunchKernelGGL(moe_combine_kernel<float>, grid, dim3(256), 0, s, static_cast<float *>(x), Y, pair_row,
                       n_tok, k, D, layer_scalar);
  return hipGetLastError();
}

}  // namespace dg
