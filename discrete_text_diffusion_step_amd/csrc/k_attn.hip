// Attention for the canvas step (gfx950).
//
//  * qkv_norm_rope: per-head QK-RMSNorm with the gamma vectors, unit-RMS V in
//    shared-K/V layers, split-half RoPE (pair t with t + d/2) with angles
//    computed in fp64 from the absolute position (aitrends notebook summary,
//    QK-norm and RoPE paragraphs with their code; glossary "Partial RoPE").
//    Writes q in place and the layer's k/v rows to their destination: the
//    workspace in decode mode, the KV cache in encode (commit) mode.
//  * attn_fwd: flash-style softmax(q K^T) V with scale 1 (scalar QK-norm
//    fixes the temperature).  One workgroup takes one kv head, a block of
//    query rows of all q heads that share it (GQA rows packed as
//    head-major x canvas position), and one slice of the keys.  K and a
//    transposed V tile go through LDS; the score tile is computed transposed
//    (S^T = K Q^T) so that each lane owns one query column and the
//    probabilities sit in registers in exactly the B-operand layout of the
//    P V MFMA -- no LDS round trip for P.  Online softmax in fp32.
//  * attn_combine: merges the per-slice (max, sum, O) partials.
#include "dg_launch.h"

namespace dg {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void norm_rope_kernel(const NormRopeArgs a) {
  __shared__ float cs[256], sn[256];
  const int j = blockIdx.x;
  const int half = a.dh >> 1;
  for (int t = threadIdx.x; t < half; t += blockDim.x) {
    if (t < a.n_rot) {
      const double f = pow(a.rope_base, -2.0 * static_cast<double>(t) / static_cast<double>(a.dh));
      const double th = static_cast<double>(a.pos0 + j) * f;
      cs[t] = static_cast<float>(cos(th));
      sn[t] = static_cast<float>(sin(th));
    } else {
      cs[t] = 1.0f;
      sn[t] = 0.0f;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T *row = static_cast<T *>(a.qkv) + static_cast<long long>(j) * a.ld;
  const int items = a.Hq + 2 * a.Hkv;
  for (int it = wave; it < items; it += 4) {
    const T *src;
    const T *w = nullptr;
    T *dst;
    bool rope = true, norm = true;
    if (it < a.Hq) {
      src = row + a.q_off + it * a.dh;
      dst = row + a.q_off + it * a.dh;
      w = static_cast<const T *>(a.q_norm);
    } else if (it < a.Hq + a.Hkv) {
      const int h = it - a.Hq;
      src = row + a.k_off + h * a.dh;
      dst = static_cast<T *>(a.k_dst) + h * a.dst_head_stride + static_cast<long long>(a.dst_row0 + j) * a.dh;
      w = static_cast<const T *>(a.k_norm);
    } else {
      const int h = it - a.Hq - a.Hkv;
      src = row + a.v_off + h * a.dh;
      dst = static_cast<T *>(a.v_dst) + h * a.dst_head_stride + static_cast<long long>(a.dst_row0 + j) * a.dh;
      rope = false;
      norm = a.v_unit_rms != 0;
    }
    float x0[4], x1[4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = lane + 64 * i;
      if (t < half) {
        x0[i] = to_f32<T>(src[t]);
        x1[i] = to_f32<T>(src[t + half]);
      } else {
        x0[i] = 0.f;
        x1[i] = 0.f;
      }
      ss += x0[i] * x0[i] + x1[i] * x1[i];
    }
    float scale = 1.0f;
    if (norm) {
      ss = wave_sum(ss);
      scale = a.sqrt_dh / (sqrtf(ss) + a.eps);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = lane + 64 * i;
      if (t >= half) continue;
      float p = x0[i] * scale, q = x1[i] * scale;
      if (w) {
        p *= to_f32<T>(w[t]);
        q *= to_f32<T>(w[t + half]);
      }
      if (rope) {
        const float c = cs[t], s = sn[t];
        const float o0 = p * c - q * s;
        const float o1 = q * c + p * s;
        p = o0;
        q = o1;
      }
      dst[t] = from_f32<T>(p);
      dst[t + half] = from_f32<T>(q);
    }
  }
}

constexpr int kBKV = 32;  // keys per tile

template <typename T, int DH>
struct AttnCfg {
  static constexpr int QT = DH >= 512 ? 1 : 2;      // 16-query tiles per wave
  static constexpr int BQ = 4 * 16 * QT;            // query rows per workgroup
  static constexpr int PADK = 16 / sizeof(T);
  static constexpr int KROW = DH + PADK;            // sK row (elements)
  static constexpr int PADV = 4;                    // keeps bf16 rows 8-B and fp32 rows 16-B aligned
  static constexpr int VROW = kBKV + PADV;          // sVt row (elements)
  static constexpr int DS = DH / 32;                // 32-wide d steps
  static constexpr int DT = DH / 16;                // 16-wide d tiles
};

__device__ __forceinline__ void store_pair(bf16_t *p, float a, float b) {
  *reinterpret_cast<uint32_t *>(p) = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}
__device__ __forceinline__ void store_pair(float *p, float a, float b) {
  *reinterpret_cast<float2 *>(p) = make_float2(a, b);
}

__device__ __forceinline__ void load_vt_frag(Frag<bf16_t> &f, const bf16_t *row, int lg) {
  const uint2 a = *reinterpret_cast<const uint2 *>(row + lg * 4);
  const uint2 b = *reinterpret_cast<const uint2 *>(row + 16 + lg * 4);
  uint4 u = make_uint4(a.x, a.y, b.x, b.y);
  f.v = *reinterpret_cast<bf16x8 *>(&u);
}
__device__ __forceinline__ void load_vt_frag(Frag<float> &f, const float *row, int lg) {
  const float4 a = *reinterpret_cast<const float4 *>(row + lg * 4);
  const float4 b = *reinterpret_cast<const float4 *>(row + 16 + lg * 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const AttnArgs a) {
  using C = AttnCfg<T, DH>;
  __shared__ __attribute__((aligned(16))) T sK[kBKV * C::KROW];
  __shared__ __attribute__((aligned(16))) T sVt[DH * C::VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = a.n_rep * a.n_tok;
  const int qblocks = (R + C::BQ - 1) / C::BQ;
  const int g = blockIdx.x / qblocks;
  const int qb = blockIdx.x % qblocks;
  const int split = blockIdx.y;
  const int r0 = qb * C::BQ;
  const int r1 = min(R, r0 + C::BQ);

  // key range of this block: decode sees [key_lo, kv_len + n_tok); encode
  // narrows it to what the block's queries can see
  int lo = a.key_lo, hi = a.kv_len + a.n_tok;
  if (a.causal) {
    int jmin = r0 % a.n_tok, jmax = (r1 - 1) % a.n_tok;
    if (r0 / a.n_tok != (r1 - 1) / a.n_tok) {
      jmin = 0;
      jmax = a.n_tok - 1;
    }
    hi = a.kv_len + jmax + 1;
    lo = a.sliding ? max(0, a.kv_len + jmin - a.window + 1) : 0;
  }
  const int span = max(0, hi - lo);
  int chunk = (span + a.n_split - 1) / a.n_split;
  chunk = (chunk + kBKV - 1) / kBKV * kBKV;
  const int k_lo = lo + split * chunk;
  const int k_hi = min(hi, k_lo + chunk);

  // this lane's query rows (one per 16-query tile) and their q fragments
  int qrow[C::QT], qpos[C::QT];
  bool qval[C::QT];
  Frag<T> qf[C::QT][C::DS];
  const T *Q = static_cast<const T *>(a.q);
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    const int r = r0 + wave * 16 * C::QT + qt * 16 + l16;
    qval[qt] = r < r1;
    const int rr = qval[qt] ? r : r0;
    const int h = g * a.n_rep + rr / a.n_tok;
    const int j = rr % a.n_tok;
    qrow[qt] = rr;
    qpos[qt] = a.kv_len + j;
    const T *qp = Q + static_cast<long long>(j) * a.q_ld + h * DH;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      if (qval[qt]) qf[qt][s].load(qp + s * 32 + lg * 8);
      else qf[qt][s].zero();
    }
  }

  f32x4 o[C::DT][C::QT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) o[dt][qt] = zero4();
  float m_run[C::QT], l_run[C::QT];
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    m_run[qt] = -1e30f;
    l_run[qt] = 0.f;
  }

  const T *Kc = static_cast<const T *>(a.k_cache) + g * a.cache_hs;
  const T *Vc = static_cast<const T *>(a.v_cache) + g * a.cache_hs;
  const T *Kn = static_cast<const T *>(a.k_new) + g * a.new_hs;
  const T *Vn = static_cast<const T *>(a.v_new) + g * a.new_hs;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int KCH = kBKV * DH / VEC;   // 16-byte chunks of a K tile
  constexpr int VPAIRS = (kBKV / 2) * (DH / 8);

  for (int t0 = k_lo; t0 < k_hi; t0 += kBKV) {
    // ---- stage K tile [key][d] and V^T tile [d][key] in LDS
    for (int c = tid; c < KCH; c += 256) {
      const int kk = c / (DH / VEC), d0 = (c % (DH / VEC)) * VEC;
      const int m = t0 + kk;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < k_hi) {
        const T *src = (m < a.kv_len) ? Kc + static_cast<long long>(m) * DH : Kn + static_cast<long long>(m - a.kv_len) * DH;
        v = *reinterpret_cast<const uint4 *>(src + d0);
      }
      *reinterpret_cast<uint4 *>(sK + kk * C::KROW + d0) = v;
    }
    for (int c = tid; c < VPAIRS; c += 256) {
      const int kp = c % (kBKV / 2), d0 = (c / (kBKV / 2)) * 8;
      float va[8], vb[8];
      const int m0 = t0 + 2 * kp, m1 = m0 + 1;
      if (m0 < k_hi) {
        const T *src = (m0 < a.kv_len) ? Vc + static_cast<long long>(m0) * DH : Vn + static_cast<long long>(m0 - a.kv_len) * DH;
        load8(src + d0, va);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) va[e] = 0.f;
      }
      if (m1 < k_hi) {
        const T *src = (m1 < a.kv_len) ? Vc + static_cast<long long>(m1) * DH : Vn + static_cast<long long>(m1 - a.kv_len) * DH;
        load8(src + d0, vb);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vb[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) store_pair(sVt + (d0 + e) * C::VROW + 2 * kp, va[e], vb[e]);
    }
    __syncthreads();

    // ---- S^T = K Q^T for 32 keys x (16*QT) queries of this wave
    f32x4 st[2][C::QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt) st[kt][qt] = zero4();
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        Frag<T> kf;
        kf.load(sK + (kt * 16 + l16) * C::KROW + s * 32 + lg * 8);
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) mma(st[kt][qt], kf, qf[qt][s]);
      }
    }

    // ---- mask, online softmax (lane owns one query per tile)
    Frag<T> pf[C::QT];
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      float sv[8];
      float mt = -1e30f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = t0 + kt * 16 + lg * 4 + i;
          bool ok = m < k_hi;
          if (a.causal) {
            const int p = qpos[qt];
            ok = ok && (m <= p) && (!a.sliding || m > p - a.window);
          }
          const float v = ok ? st[kt][qt][i] : -INFINITY;
          sv[kt * 4 + i] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run[qt], mt);
      const float corr = __expf(m_run[qt] - m_new);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[e] = __expf(sv[e] - m_new);
        psum += sv[e];
      }
      l_run[qt] = l_run[qt] * corr + psum;
      m_run[qt] = m_new;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        o[dt][qt][0] *= corr;
        o[dt][qt][1] *= corr;
        o[dt][qt][2] *= corr;
        o[dt][qt][3] *= corr;
      }
      pf[qt].from_floats(sv);
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      Frag<T> vf;
      load_vt_frag(vf, sVt + (dt * 16 + l16) * C::VROW, lg);
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt) mma(o[dt][qt], vf, pf[qt]);
    }
    __syncthreads();
  }

  // ---- finish: lanes sharing a query (same l16) hold partial sums of l
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    float l = l_run[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!qval[qt]) continue;
    const int rr = qrow[qt];
    if (a.n_split == 1) {
      const int h = g * a.n_rep + rr / a.n_tok;
      const int j = rr % a.n_tok;
      T *op = static_cast<T *>(a.out) + static_cast<long long>(j) * a.out_ld + h * DH;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) op[dt * 16 + lg * 4 + i] = from_f32<T>(o[dt][qt][i] * inv);
    } else {
      const long long prow = static_cast<long long>(split) * a.Hkv * R + static_cast<long long>(g) * R + rr;
      float *op = a.o_part + prow * DH;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        *reinterpret_cast<float4 *>(op + dt * 16 + lg * 4) =
            make_float4(o[dt][qt][0], o[dt][qt][1], o[dt][qt][2], o[dt][qt][3]);
      if (lg == 0) {
        a.ml_part[prow * 2] = m_run[qt];
        a.ml_part[prow * 2 + 1] = l;
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a, int dh) {
  const int R = a.n_rep * a.n_tok;
  const int idx = blockIdx.x;  // g * R + rr
  const int g = idx / R, rr = idx % R;
  const long long rows = static_cast<long long>(a.Hkv) * R;
  float M = -1e30f;
  for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, a.ml_part[(s * rows + idx) * 2]);
  float L = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float* ml = a.ml_part + (s * rows + idx) * 2;
    L += ml[1] * __expf(ml[0] - M);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  const int h = g * a.n_rep + rr / a.n_tok;
  const int j = rr % a.n_tok;
  T *op = static_cast<T *>(a.out) + static_cast<long long>(j) * a.out_ld + h * dh;
  for (int d = threadIdx.x; d < dh; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
      const float w = __expf(a.ml_part[(s * rows + idx) * 2] - M);
      acc += w * a.o_part[(s * rows + idx) * dh + d];
    }
    op[d] = from_f32<T>(acc * inv);
  }
}

template <typename T, int DH>
hipError_t launch_attn_t(const AttnArgs &a, hipStream_t s) {
  using C = AttnCfg<T, DH>;
  const int R = a.n_rep * a.n_tok;
  const int qblocks = (R + C::BQ - 1) / C::BQ;
  hipLaunchKernelGGL((attn_fwd_kernel<T, DH>), dim3(a.Hkv * qblocks, a.n_split), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  hipLaunchKernelGGL(attn_combine_kernel<T>, dim3(a.Hkv * R), dim3(DH < 256 ? DH : 256), 0, s, a, DH);
  return hipGetLastError();
}

}  // namespace

int attn_block_rows(int dtype, int dh) {
  if (dtype == DG_BF16) {
    switch (dh) {
      case 64: return AttnCfg<bf16_t, 64>::BQ;
      case 128: return AttnCfg<bf16_t, 128>::BQ;
      case 256: return AttnCfg<bf16_t, 256>::BQ;
      case 512: return AttnCfg<bf16_t, 512>::BQ;
    }
  } else {
    switch (dh) {
      case 64: return AttnCfg<float, 64>::BQ;
      case 128: return AttnCfg<float, 128>::BQ;
      case 256: return AttnCfg<float, 256>::BQ;
    }
  }
  return 0;
}

hipError_t launch_attention(const AttnArgs &a, int dtype, int dh, hipStream_t s) {
  if (a.n_tok <= 0) return hipSuccess;
  if (dtype == DG_BF16) {
    switch (dh) {
      case 64: return launch_attn_t<bf16_t, 64>(a, s);
      case 128: return launch_attn_t<bf16_t, 128>(a, s);
      case 256: return launch_attn_t<bf16_t, 256>(a, s);
      case 512: return launch_attn_t<bf16_t, 512>(a, s);
    }
  } else {
    switch (dh) {
      case 64: return launch_attn_t<float, 64>(a, s);
      case 128: return launch_attn_t<float, 128>(a, s);
      case 256: return launch_attn_t<float, 256>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_norm_rope(const NormRopeArgs &a, int dtype, hipStream_t s) {
  if (a.n_tok <= 0) return hipSuccess;
  if (dtype == DG_BF16) hipLaunchKernelGGL(norm_rope_kernel<bf16_t>, dim3(a.n_tok), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(norm_rope_kernel<float>, dim3(a.n_tok), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dg
