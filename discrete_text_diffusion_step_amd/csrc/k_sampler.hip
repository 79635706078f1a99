// Entropy-bound sampler, uniform re-noise and tempered probabilities (gfx950).
//
// aitrends notebook summary, sampler paragraph: per position, the entropy of
// the tempered distribution decides whether the position is fixed or
// re-noised with a uniform random token (aibars news, self-correction).
//
// rowstats_partial: each workgroup streams one slice of one logits row once
//   and keeps, per thread, the online statistics of d = l/t - m:
//   m (running max), Z = sum e^d, S = sum e^d * d, and the argmax of l
//   (first index on ties).  Slices are merged in a fixed order.
// sample_finalize: merges the slices of every row, H = ln Z - S/Z, commit iff
//   H < tau (or on the final step), token = argmax or a Philox4x32-10 draw,
//   and counts the re-noised positions with a block reduction (no atomics).
// Variants: the Gumbel-max proposal argmax_v (l_v/t + g_v) in place of the
//   argmax (the slice pass draws g from Philox as it streams the row), the
//   sorted cumulative commit rule (ranks by entropy inside the one-workgroup
//   finalize), and the count of proposals changed since the previous step.
// probs: p = exp(l/t - m) / Z stored in the model dtype (input of P.E).
#include "dg_launch.h"

namespace dg {

namespace {

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// 4x32 bijection with multipliers 0xD2511F53 / 0xCD9E8D57, key advanced by
// the Weyl constants 0x9E3779B9 / 0xBB67AE85 between rounds.
__device__ __forceinline__ uint4 philox4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                         uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ uint32_t philox_x0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1) {
  return philox4(c0, c1, c2, c3, k0, k1).x;
}

// Gumbel(0,1) value of one 32-bit word: k = word >> 9, u = (k + 1/2) 2^-23
// (exact), E = -ln u (through log1p(-(1-u)) for u >= 1/2, where 1-u is exact
// and ln u is small), g = -ln E.
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  const uint32_t k = x >> 9;
  const float u = (static_cast<float>(k) + 0.5f) * 0x1p-23f;
  const float w = (static_cast<float>(0x7FFFFFu - k) + 0.5f) * 0x1p-23f;
  const float e = k < 0x400000u ? -logf(u) : -log1pf(-w);
  return -logf(e);
}

__device__ __forceinline__ int32_t uniform_token(uint32_t x0, int vocab) {
  return static_cast<int32_t>((static_cast<uint64_t>(x0) * static_cast<uint64_t>(vocab)) >> 32);
}

__device__ __forceinline__ void better(float &bv, int &bi, float v, int i) { better_of(bv, bi, v, i); }

__device__ __forceinline__ void load_logits8(const void *p, int bf16, long long off, float *f) {
  if (bf16) load8(static_cast<const bf16_t *>(p) + off, f);
  else load8(static_cast<const float *>(p) + off, f);
}

template <bool GUMBEL>
__global__ __launch_bounds__(256) void rowstats_partial_kernel(const SampleArgs a) {
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int clen = a.vocab / a.n_chunks;
  const long long base = static_cast<long long>(row) * a.vocab + static_cast<long long>(chunk) * clen;
  float m = -INFINITY, Z = 0.f, S = 0.f, bv = -INFINITY;
  int bi = 0x7fffffff, nf = 0;
  for (int c = threadIdx.x * 8; c < clen; c += 256 * 8) {
    float l[8];
    load_logits8(a.logits, a.logits_bf16, base + c, l);
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) nf += !isfinite(l[j]);
    if constexpr (GUMBEL) {
      // proposal score l/t + g, noise words for v = v0 .. v0+7 (v0 % 8 == 0)
      const uint32_t v0 = static_cast<uint32_t>(chunk * clen + c);
      const uint4 r0 = philox4(static_cast<uint32_t>(row), a.step, a.canvas_idx, 1u + (v0 >> 2), a.key0, a.key1);
      const uint4 r1 = philox4(static_cast<uint32_t>(row), a.step, a.canvas_idx, 2u + (v0 >> 2), a.key0, a.key1);
      const uint32_t wd[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        better(bv, bi, l[j] * a.inv_t + gumbel_of(wd[j]), chunk * clen + c + j);
        mx = fmaxf(mx, l[j] * a.inv_t);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        better(bv, bi, l[j], chunk * clen + c + j);
        mx = fmaxf(mx, l[j] * a.inv_t);
      }
    }
    if (mx > m) {
      if (m != -INFINITY) {
        const float sc = __expf(m - mx);
        S = sc * (S + (m - mx) * Z);
        Z = sc * Z;
      }
      m = mx;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float d = l[j] * a.inv_t - m;
      const float e = __expf(d);
      Z += e;
      S += e * d;
    }
  }
  // block merge in a fixed order: wave butterfly, then the four waves
  __shared__ float sm[4][4];
  __shared__ int si[4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), Z2 = __shfl_xor(Z, o, 64), S2 = __shfl_xor(S, o, 64);
    const float bv2 = __shfl_xor(bv, o, 64);
    const int bi2 = __shfl_xor(bi, o, 64);
    merge_row_stats(m, Z, S, m2, Z2, S2);
    better(bv, bi, bv2, bi2);
    nf += __shfl_xor(nf, o, 64);
  }
  __shared__ int snf[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm[wave][0] = m;
    sm[wave][1] = Z;
    sm[wave][2] = S;
    sm[wave][3] = bv;
    si[wave] = bi;
    snf[wave] = nf;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0][0], ZZ = sm[0][1], SS = sm[0][2], BV = sm[0][3];
    int BI = si[0];
    for (int w = 1; w < 4; ++w) {
      merge_row_stats(M, ZZ, SS, sm[w][0], sm[w][1], sm[w][2]);
      better(BV, BI, sm[w][3], si[w]);
    }
    float *p = a.part + (static_cast<long long>(row) * a.n_chunks + chunk) * 4;
    p[0] = M;
    p[1] = ZZ;
    p[2] = SS;
    p[3] = BV;
    a.part_idx[static_cast<long long>(row) * a.n_chunks + chunk] = BI;
    a.part_nf[static_cast<long long>(row) * a.n_chunks + chunk] = snf[0] + snf[1] + snf[2] + snf[3];
  }
}

__device__ __forceinline__ int block_sum(int v, int *red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const int r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void sample_finalize_kernel(const SampleArgs a) {
  __shared__ int red[256];
  __shared__ float sH[kSortedMaxRows];
  __shared__ int sP[kSortedMaxRows];
  const bool sorted = a.commit_rule == 1;
  int renoised = 0, changed = 0, nonfinite = 0;
  for (int row = threadIdx.x; row < a.n_pos; row += 256) {
    const float *p = a.part + static_cast<long long>(row) * a.n_chunks * 4;
    const int *pi = a.part_idx + static_cast<long long>(row) * a.n_chunks;
    const int *pnf = a.part_nf + static_cast<long long>(row) * a.n_chunks;
    float M = p[0], Z = p[1], S = p[2], bv = p[3];
    int bi = pi[0], nf = pnf[0];
    for (int c = 1; c < a.n_chunks; ++c) {
      merge_row_stats(M, Z, S, p[c * 4], p[c * 4 + 1], p[c * 4 + 2]);
      better(bv, bi, p[c * 4 + 3], pi[c]);
      nf += pnf[c];
    }
    nonfinite += nf > 0;
    // NaN logits are never a candidate; a row of NaN only proposes token 0
    if (bi < 0 || bi >= a.vocab) bi = 0;
    // a row holding a NaN or +-inf has no defined entropy (never committed on its own)
    const float H = nf > 0 ? NAN : __logf(Z) - S / Z;
    if (a.pred) {
      changed += a.pred[row] != bi;
      a.pred[row] = bi;
    }
    a.entropy[row] = H;
    if (a.rowstats) {
      a.rowstats[2 * row] = M;
      a.rowstats[2 * row + 1] = Z;
    }
    if (sorted) {
      sH[row] = H;
      sP[row] = bi;
      continue;
    }
    const bool commit = a.final_step || (H < a.tau);
    int32_t tok = bi;
    if (!commit) {
      const uint32_t x0 = philox_x0(static_cast<uint32_t>(row), a.step, a.canvas_idx, 0u, a.key0, a.key1);
      tok = uniform_token(x0, a.vocab);
      ++renoised;
    }
    a.tokens[row] = tok;
    a.commit[row] = commit ? 1 : 0;
  }
  if (sorted) {
    __syncthreads();
    // rank by (H, position); a position commits iff the entropy summed over
    // the positions ranked before it (added in position order) is <= tau
    for (int row = threadIdx.x; row < a.n_pos; row += 256) {
      const float H = sH[row];
      float prior = 0.f;
      for (int i = 0; i < a.n_pos; ++i) {
        const float Hi = sH[i];
        if (Hi < H || (Hi == H && i < row)) prior += Hi;
      }
      const bool commit = a.final_step || prior <= a.tau;
      int32_t tok = sP[row];
      if (!commit) {
        const uint32_t x0 = philox_x0(static_cast<uint32_t>(row), a.step, a.canvas_idx, 0u, a.key0, a.key1);
        tok = uniform_token(x0, a.vocab);
        ++renoised;
      }
      a.tokens[row] = tok;
      a.commit[row] = commit ? 1 : 0;
    }
  }
  const int nre = block_sum(renoised, red);
  if (a.pred && a.n_changed) {
    const int nch = block_sum(changed, red);
    if (threadIdx.x == 0) *a.n_changed = nch;
  }
  if (a.n_nonfinite) {
    const int nnf = block_sum(nonfinite, red);
    if (threadIdx.x == 0) *a.n_nonfinite = nnf;
  }
  if (threadIdx.x == 0) *a.n_renoised = nre;
}

__global__ __launch_bounds__(256) void canvas_noise_kernel(int n_pos, int vocab, uint32_t k0, uint32_t k1,
                                                           uint32_t canvas_idx, int32_t *tokens) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n_pos) return;
  tokens[j] = uniform_token(philox_x0(static_cast<uint32_t>(j), 0xFFFFFFFFu, canvas_idx, 0u, k0, k1), vocab);
}

template <typename T>
__global__ __launch_bounds__(256) void probs_kernel(const float *logits, const float *rowstats, int vocab,
                                                    float inv_t, T *P) {
  const int row = blockIdx.y;
  const long long c = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (c >= vocab) return;
  const float m = rowstats[2 * row], invZ = 1.0f / rowstats[2 * row + 1];
  float l[8];
  load8(logits + static_cast<long long>(row) * vocab + c, l);
#pragma unroll
  for (int j = 0; j < 8; ++j) l[j] = __expf(l[j] * inv_t - m) * invZ;
  store8(P + static_cast<long long>(row) * vocab + c, l);
}

}  // namespace

hipError_t launch_sampler(const SampleArgs &a, hipStream_t s) {
  if (a.n_pos <= 0) return hipSuccess;
  if (a.commit_rule == 1 && a.n_pos > kSortedMaxRows) return hipErrorInvalidValue;
  if (a.token_rule == 1)
    hipLaunchKernelGGL(rowstats_partial_kernel<true>, dim3(a.n_chunks, a.n_pos), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rowstats_partial_kernel<false>, dim3(a.n_chunks, a.n_pos), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_finalize_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_canvas_noise(int n_pos, int vocab, uint32_t key0, uint32_t key1, uint32_t canvas_idx,
                               int32_t *tokens, hipStream_t s) {
  if (n_pos <= 0) return hipSuccess;
  hipLaunchKernelGGL(canvas_noise_kernel, dim3((n_pos + 255) / 256), dim3(256), 0, s, n_pos, vocab, key0, key1,
                     canvas_idx, tokens);
  return hipGetLastError();
}

hipError_t launch_probs(int dtype, const float *logits, const float *rowstats, int n_pos, int vocab, float inv_t,
                        void *P, hipStream_t s) {
  if (n_pos <= 0) return hipSuccess;
  dim3 grid((vocab / 8 + 255) / 256, n_pos);
  if (dtype == DG_BF16)
    hipLaunchKernelGGL(probs_kernel<bf16_t>, grid, dim3(256), 0, s, logits, rowstats, vocab, inv_t,
                       static_cast<bf16_t *>(P));
  else
    hipLaunchKernelGGL(probs_kernel<float>, grid, dim3(256), 0, s, logits, rowstats, vocab, inv_t,
                       static_cast<float *>(P));
  return hipGetLastError();
}

}  // namespace dg
