// Row kernels (gfx950): RMSNorm, embedding gather, embedding transpose.
#include "dg_launch.h"

namespace dg {

namespace {

// aitrends notebook summary, rms code: y = w * x * sqrt(D) / (||x||_2 + eps)
// with the norm reduced in fp32.  One wave per row, 16-byte vector accesses.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(int n, int D, float eps, float sqrt_d, const T *x,
                                                      const T *w, T *y) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const T *xr = x + static_cast<long long>(row) * D;
  float ss = 0.f;
  for (int c = lane * 8; c < D; c += 64 * 8) {
    float v[8];
    load8(xr + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
  }
  ss = wave_allsum(ss);
  const float scale = sqrt_d / (sqrtf(ss) + eps);
  T *yr = y + static_cast<long long>(row) * D;
  for (int c = lane * 8; c < D; c += 64 * 8) {
    float v[8], g[8];
    load8(xr + c, v);
    load8(w + c, g);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = g[j] * v[j] * scale;
    store8(yr + c, v);
  }
}

// Residual update fused with the next block's RMSNorm, one workgroup of 512
// threads per row (rows up to 512 * 8 wide): each thread owns 8 consecutive
// elements and issues the loads of every extra row at once (up to 16 at a
// time), so a row costs one round of memory latency instead of one per batch.
// The stored row is rounded to T first and the norm is taken over the stored
// values (fp32 sum of squares, block reduction).
//   reduce_add: x <- T(x + sum_s part[s])      (split-K partials, s ascending)
//   combine:    x <- T(ls * (x + Y[t] + sum_j Y[pair_row[t*k+j]]))
//   then        h <- T(w * x * sqrt(D) / (||x||_2 + eps))
constexpr int kResThreads = 512;
template <typename T, bool COMBINE>
__global__ __launch_bounds__(kResThreads) void residual_rmsnorm_kernel(const float *part, int splits,
                                                                       const int *pair_row, int k, float ls, int n,
                                                                       int D, T *x, const T *w, float eps,
                                                                       float sqrt_d, T *h) {
  __shared__ float red[kResThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  T *xr = x + static_cast<long long>(row) * D;
  const int c = tid * 8;
  const bool active = c < D;
  constexpr int KX = 16;
  const int nx = COMBINE ? k : splits;
  float v[8], g[8];
  float ss = 0.f;
  if (active) {
    float a[8], o[8];
    load8(w + c, g);
    if constexpr (COMBINE) {
      // the shared expert's row is the token's own, then its k experts
      load8(part + static_cast<long long>(row) * D + c, a);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = 0.f;
    }
    load8(xr + c, o);
    for (int z0 = 0; z0 < nx; z0 += KX) {
      float t[KX][8];
#pragma unroll
      for (int j = 0; j < KX; ++j)
        if (z0 + j < nx) {
          const long long r = COMBINE ? pair_row[row * k + z0 + j] : static_cast<long long>(z0 + j) * n + row;
          load8(part + r * D + c, t[j]);
        }
#pragma unroll
      for (int j = 0; j < KX; ++j)
        if (z0 + j < nx) {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] += t[j][e];
        }
    }
    if constexpr (COMBINE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = ls * (o[e] + a[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += o[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = to_f32<T>(from_f32<T>(a[e]));
      ss += v[e] * v[e];
    }
    store8(xr + c, v);
  }
  ss = wave_allsum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  ss = 0.f;
#pragma unroll
  for (int i = 0; i < kResThreads / 64; ++i) ss += red[i];
  const float scale = sqrt_d / (sqrtf(ss) + eps);
  if (active) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = g[e] * v[e] * scale;
    store8(h + static_cast<long long>(row) * D + c, o);
  }
}

// x[j] = E[tokens[j]]; ids outside [0, vocab) are clamped into range.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t *tokens, int n, int D, int vocab, const T *E,
                                                    T *x) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  int t = tokens[row];
  t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
  const uint4 *src = reinterpret_cast<const uint4 *>(E + static_cast<long long>(t) * D);
  uint4 *dst = reinterpret_cast<uint4 *>(x + static_cast<long long>(row) * D);
  const int nv = D * static_cast<int>(sizeof(T)) / 16;
  for (int c = lane; c < nv; c += 64) dst[c] = src[c];
}

// out[c][r] = in[r][c] through a 64x64 LDS tile.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(int rows, int cols, const T *in, T *out) {
  __shared__ T tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = in[static_cast<long long>(r) * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) out[static_cast<long long>(c) * rows + r] = tile[tx][i];
  }
}

// fp32 -> OCP E4M3 code: round to nearest, ties to even, magnitudes above
// 448 saturate to 448 (S.1111.110).  Subnormals are steps of 2^-9 below
// 2^-6; normals round the fp32 mantissa to 3 bits (a carry moves into the
// exponent) and rebias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0x1p-6f) {
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t u = __float_as_uint(a);
    code = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return (code > 0x7Eu ? 0x7Eu : code) | sign;
}

// Row-wise E4M3 quantisation, one workgroup per row:
//   scale = max|w| / 448 (fp32, correctly rounded; 1 for a zero row)
//   q     = E4M3(w / scale)  (fp32 division, correctly rounded)
template <typename T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T *w, int cols, uint8_t *q, float *scale) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long row = blockIdx.x;
  const T *wr = w + row * cols;
  float m = 0.f;
  for (int c = tid; c < cols; c += 256) m = fmaxf(m, fabsf(to_f32<T>(wr[c])));
  m = wave_allmax(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = m > 0.f ? __fdiv_rn(m, 448.0f) : 1.0f;
  uint8_t *qr = q + row * cols;
  for (int c = tid; c < cols; c += 256) qr[c] = static_cast<uint8_t>(e4m3_code(__fdiv_rn(to_f32<T>(wr[c]), sc)));
  if (tid == 0) scale[row] = sc;
}

}  // namespace

hipError_t launch_rmsnorm(int dtype, int n, int D, float eps, const void *x, const void *w, void *y,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const float sqrt_d = static_cast<float>(__builtin_sqrt(static_cast<double>(D)));
  if (dtype == DG_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3((n + 3) / 4), dim3(256), 0, s, n, D, eps, sqrt_d,
                       static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(w), static_cast<bf16_t *>(y));
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3((n + 3) / 4), dim3(256), 0, s, n, D, eps, sqrt_d,
                       static_cast<const float *>(x), static_cast<const float *>(w), static_cast<float *>(y));
  return hipGetLastError();
}

hipError_t launch_embed(int dtype, const int32_t *tokens, int n, int D, int vocab, const void *E, void *x,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == DG_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3((n + 3) / 4), dim3(256), 0, s, tokens, n, D, vocab,
                       static_cast<const bf16_t *>(E), static_cast<bf16_t *>(x));
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3((n + 3) / 4), dim3(256), 0, s, tokens, n, D, vocab,
                       static_cast<const float *>(E), static_cast<float *>(x));
  return hipGetLastError();
}

hipError_t launch_transpose(int dtype, int rows, int cols, const void *in, void *out, hipStream_t s) {
  dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  if (dtype == DG_BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, s, rows, cols, static_cast<const bf16_t *>(in),
                       static_cast<bf16_t *>(out));
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, rows, cols, static_cast<const float *>(in),
                       static_cast<float *>(out));
  return hipGetLastError();
}


int residual_norm_max_width() { return kResThreads * 8; }

hipError_t launch_reduce_add_rmsnorm(int dtype, const float *part, int splits, int n, int D, void *x, const void *w,
                                     float eps, void *h, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (D > residual_norm_max_width() || D % 8) return hipErrorInvalidValue;
  const float sq = static_cast<float>(__builtin_sqrt(static_cast<double>(D)));   // as launch_rmsnorm
  const dim3 grid(n);
  if (dtype == DG_BF16)
    hipLaunchKernelGGL((residual_rmsnorm_kernel<bf16_t, false>), grid, dim3(kResThreads), 0, s, part, splits, nullptr, 0,
                       1.0f, n, D, static_cast<bf16_t *>(x), static_cast<const bf16_t *>(w), eps, sq,
                       static_cast<bf16_t *>(h));
  else
    hipLaunchKernelGGL((residual_rmsnorm_kernel<float, false>), grid, dim3(kResThreads), 0, s, part, splits, nullptr, 0,
                       1.0f, n, D, static_cast<float *>(x), static_cast<const float *>(w), eps, sq,
                       static_cast<float *>(h));
  return hipGetLastError();
}

hipError_t launch_combine_rmsnorm(int dtype, void *x, const float *Y, const int *pair_row, int n, int k, int D,
                                  float layer_scalar, const void *w, float eps, void *h, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (D > residual_norm_max_width() || D % 8) return hipErrorInvalidValue;
  const float sq = static_cast<float>(__builtin_sqrt(static_cast<double>(D)));   // as launch_rmsnorm
  const dim3 grid(n);
  if (dtype == DG_BF16)
    hipLaunchKernelGGL((residual_rmsnorm_kernel<bf16_t, true>), grid, dim3(kResThreads), 0, s, Y, 0, pair_row, k,
                       layer_scalar, n, D, static_cast<bf16_t *>(x), static_cast<const bf16_t *>(w), eps, sq,
                       static_cast<bf16_t *>(h));
  else
    hipLaunchKernelGGL((residual_rmsnorm_kernel<float, true>), grid, dim3(kResThreads), 0, s, Y, 0, pair_row, k,
                       layer_scalar, n, D, static_cast<float *>(x), static_cast<const float *>(w), eps, sq,
                       static_cast<float *>(h));
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(int dtype, const void *w, long long rows, int cols, uint8_t *q, float *scale,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(rows));
  if (dtype == DG_BF16)
    hipLaunchKernelGGL(quantize_fp8_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t *>(w), cols, q,
                       scale);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<float>, grid, dim3(256), 0, s, static_cast<const float *>(w), cols, q,
                       scale);
  return hipGetLastError();
}

}  // namespace dg
