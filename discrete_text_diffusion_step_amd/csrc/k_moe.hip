// MoE routing for the canvas step (gfx950): top-k router, expert batching,
// deterministic combine (aitrends notebook summary, glossary "MoE":
// exp(router key . x) scores, renormalised over the chosen experts and
// scaled; tokens routed to one expert are processed together; the shared
// expert is always added).
//
// Group layout produced by moe_permute (consumed by the grouped GEMM):
//   group 0          : the shared expert, rows [0, n_tok) in token order
//   group 1 + e      : routed expert e, rows sorted by (token, slot)
// so g_off has n_experts + 2 entries.  row_token[r] is the token of row r,
// row_weight[r] its mixing weight (1 for the shared expert) and pair_row[t*k+j]
// the row holding token t's j-th expert.
#include "dg_launch.h"

namespace dg {

namespace {

// One wave per token.  Top-k by logit, ties to the lower expert id; weights
// are softmax restricted to the chosen experts (the full-softmax denominator
// cancels in the renormalisation) times route_scale.
__global__ __launch_bounds__(256) void router_topk_kernel(const float *logits, int n_tok, int E, int k,
                                                          float scale, int32_t *idx_out, float *w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= n_tok) return;
  const float *r = logits + static_cast<long long>(t) * E;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? r[e] : -INFINITY;
  }
  float chosen_v[8];
  int chosen_e[8];
  for (int j = 0; j < k; ++j) {
    // lane-local best (lower id wins ties: ids grow with i)
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    chosen_v[j] = bv;
    chosen_e[j] = be;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == be) v[i] = -INFINITY;
  }
  if (lane == 0) {
    const float mx = chosen_v[0];
    float p[8], sum = 0.f;
    for (int j = 0; j < k; ++j) {
      p[j] = __expf(chosen_v[j] - mx);
      sum += p[j];
    }
    for (int j = 0; j < k; ++j) {
      idx_out[static_cast<long long>(t) * k + j] = chosen_e[j];
      w_out[static_cast<long long>(t) * k + j] = p[j] / sum * scale;
    }
  }
}

// One workgroup: counts (LDS integer atomics, all threads), exclusive scan,
// then a stable scatter.  The pairs are staged in LDS in chunks; one wave
// walks each chunk 64 pairs at a time in order, ranking a pair among the
// pairs of the same expert in its 64 with ballots over the bits of the
// expert id, so rows of an expert come out sorted by (token, slot).
// Integer work only: bit-exact and independent of scheduling.
constexpr int kPermChunk = 4096;

__global__ __launch_bounds__(256) void moe_permute_kernel(const int32_t *idx, const float *w, int n_tok, int k,
                                                          int E, int *g_off, int *row_token, float *row_weight,
                                                          int *pair_row) {
  __shared__ int cnt[258];
  __shared__ int cur[258];
  __shared__ int s_e[kPermChunk];
  __shared__ float s_w[kPermChunk];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E + 2; e += 256) cnt[e] = 0;
  __syncthreads();
  const int n_pairs = n_tok * k;
  for (int p = tid; p < n_pairs; p += 256) {
    int e = idx[p];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = n_tok;
    g_off[0] = 0;
    g_off[1] = n_tok;
    for (int e = 0; e < E; ++e) {
      cur[e] = acc;
      acc += cnt[e];
      g_off[e + 2] = acc;
    }
  }
  for (int t = tid; t < n_tok; t += 256) {
    row_token[t] = t;
    row_weight[t] = 1.0f;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n_pairs; base += kPermChunk) {
    const int len = min(kPermChunk, n_pairs - base);
    __syncthreads();   // previous chunk consumed; scan visible
    for (int p = tid; p < len; p += 256) {
      int e = idx[base + p];
      s_e[p] = e < 0 ? 0 : (e >= E ? E - 1 : e);
      s_w[p] = w[base + p];
    }
    __syncthreads();
    if (wave != 0) continue;
    for (int b = 0; b < len; b += 64) {
      const int q = b + lane;
      const bool valid = q < len;
      const int e = valid ? s_e[q] : -1;
      const unsigned key = static_cast<unsigned>(e + 1);  // 0 = no pair
      uint64_t peers = __ballot(1);
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) {
        const bool on = (key >> bit) & 1u;
        const uint64_t m = __ballot(on);
        peers &= on ? m : ~m;
      }
      const int rank = __popcll(peers & lt_mask);
      const int start = valid ? cur[e] : 0;   // all lanes read before the leaders write
      if (valid && rank == 0) cur[e] = start + __popcll(peers);
      if (valid) {
        const int p = base + q;
        const int row = start + rank;
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

hipError_t launch_router_topk(const float *logits, int n_tok, int E, int k, float scale, int32_t *idx,
                              float *w, hipStream_t s) {
  if (n_tok <= 0) return hipSuccess;
  hipLaunchKernelGGL(router_topk_kernel, dim3((n_tok + 3) / 4), dim3(256), 0, s, logits, n_tok, E, k, scale, idx, w);
  return hipGetLastError();
}

hipError_t launch_moe_permute(const int32_t *idx, const float *w, int n_tok, int k, int E, int *g_off,
                              int *row_token, float *row_weight, int *pair_row, hipStream_t s) {
  hipLaunchKernelGGL(moe_permute_kernel, dim3(1), dim3(256), 0, s, idx, w, n_tok, k, E, g_off, row_token,
                     row_weight, pair_row);
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
