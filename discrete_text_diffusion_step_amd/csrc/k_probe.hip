// Roof probes (gfx950): the attainable HBM read rate and bf16 MFMA rate on
// the device at hand, against which the kernels' roofline fractions are also
// reported (the datasheet figures being the other reference).  Neither is an
// operation of the denoising step; both produce results the caller can check
// exactly, so no load or MFMA can be optimised away unnoticed.
#include "dg_common.h"

namespace dg {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kReadUnroll = 16;   // 16-byte loads in flight per thread
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Read-only stream: workgroup b reads its own contiguous span of the buffer
// (ceil(n_chunks / gridDim) 16-byte chunks), 256 threads side by side,
// kReadUnroll loads issued before any is used; each thread adds the four
// 32-bit words of every chunk it reads (wrapping), and the workgroup's sum
// goes to sink[b].  Non-temporal loads, as the weight streams of the
// products use.  Of the shapes measured (grid-strided sweeps with 4..16
// loads in flight and 1,024..16,384 workgroups: 5.3-6.5 TB/s; spans: up to
// 7.0 TB/s), contiguous spans over 1,024 workgroups read fastest, so this
// is the strictest read roof.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4 *buf, long long n_chunks,
                                                                   uint32_t *sink) {
  __shared__ uint32_t part[kProbeThreads / 64];
  const long long per = (n_chunks + gridDim.x - 1) / gridDim.x;
  const long long b0 = static_cast<long long>(blockIdx.x) * per;
  const long long b1 = b0 + per < n_chunks ? b0 + per : n_chunks;
  long long i = b0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * kProbeThreads < b1; i += kReadUnroll * kProbeThreads) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; i < b1; i += kProbeThreads) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    acc += v.x + v.y + v.z + v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o, 64));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) s += part[w];
    sink[blockIdx.x] = s;
  }
}

// MFMA loop: every wave runs `iters` rounds (a multiple of kUnroll) of kAcc
// independent 16x16x32 bf16 MFMAs whose A elements all equal a and B
// elements all equal b, so each round adds 32*a*b to every accumulator
// element.  Wave w of workgroup g stores the sum of element 0 of its
// accumulators (lane 0) to sink[4g + w]: kAcc * iters * 32 * a * b, exact
// when that and every partial sum are representable (powers of two, say).
// The rounds are unrolled kUnroll deep: the compiler moves loop-carried
// accumulators between AGPRs at each trip of the loop (about 100 moves), so a
// deep body keeps those moves small beside the 256 MFMAs.
constexpr int kAcc = 16;
constexpr int kUnroll = 16;

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, float a, float b, float *sink) {
  Frag<bf16_t> fa, fb;
  {
    const uint32_t ua = static_cast<uint32_t>(f32_to_bf16(a)) * 0x10001u;
    const uint32_t ub = static_cast<uint32_t>(f32_to_bf16(b)) * 0x10001u;
    uint4 va = make_uint4(ua, ua, ua, ua), vb = make_uint4(ub, ub, ub, ub);
    fa.v = *reinterpret_cast<bf16x8 *>(&va);
    fb.v = *reinterpret_cast<bf16x8 *>(&vb);
  }
  f32x4 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = zero4();
  for (int it = 0; it < iters; it += kUnroll) {
#pragma unroll
    for (int r = 0; r < kUnroll; ++r)
#pragma unroll
      for (int j = 0; j < kAcc; ++j) mma(acc[j], fa, fb);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kAcc; ++j) s += acc[j][0];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

}  // namespace dg

extern "C" {

int dg_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, int n_groups, void *stream) {
  if (!buf || !sink) return DG_ERR_NULL;
  if (n_groups <= 0 || n_groups > 65536 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16) return DG_ERR_SHAPE;
  if (bytes == 0) return DG_OK;
  hipLaunchKernelGGL(dg::probe_read_kernel, dim3(n_groups), dim3(dg::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const dg::u32x4 *>(buf),
                     static_cast<long long>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

int dg_probe_mfma_bf16(int iters, float a, float b, float *sink, int n_groups, void *stream) {
  if (!sink) return DG_ERR_NULL;
  if (iters < 0 || iters % dg::kUnroll || n_groups <= 0 || n_groups > 65536) return DG_ERR_SHAPE;
  hipLaunchKernelGGL(dg::probe_mfma_kernel, dim3(n_groups), dim3(dg::kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), iters, a, b, sink);
  return hipGetLastError() == hipSuccess ? DG_OK : DG_ERR_HIP;
}

long long dg_probe_mfma_flops(int iters, int n_groups) {
  if (iters < 0 || iters % dg::kUnroll || n_groups <= 0) return 0;
  return static_cast<long long>(n_groups) * (dg::kProbeThreads / 64) * iters * dg::kAcc * (2LL * 16 * 16 * 32);
}

}  // extern "C"
