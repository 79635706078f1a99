// Attention for the canvas step (gfx950).
//
//  * qkv_norm_rope: per-head QK-RMSNorm with the gamma vectors, unit-RMS V in
//    shared-K/V layers, split-half RoPE (pair t with t + d/2) with angles
//    computed in fp64 from the absolute position (aitrends notebook summary,
//    QK-norm and RoPE paragraphs with their code; glossary "Partial RoPE").
//    Writes q in place, the layer's k rows to the key cache and its v rows
//    into the transposed value cache (cache rows / columns [kv_len,
//    kv_len + n): scratch in decode mode, kept in encode (commit) mode).
//  * attn_fwd: flash-style softmax(q K^T) V with scale 1 (scalar QK-norm
//    fixes the temperature).  One workgroup takes one kv head, a block of
//    query rows of all q heads that share it (GQA rows packed as
//    head-major x canvas position), and one slice of the keys.  K and a
//    transposed V tile go through LDS; the score tile is computed transposed
//    (S^T = K Q^T) so that each lane owns one query column and the
//    probabilities sit in registers in exactly the B-operand layout of the
//    P V MFMA -- no LDS round trip for P.  Online softmax in fp32.
//    bf16 forms: attn_pair (d_h 512; two waves split the head dimension of
//    each query tile) and attn_solo (d_h 256; each wave owns whole query
//    tiles).
//  * attn_combine: merges the per-slice (max, sum, O) partials (bf16 rows
//    divided by their slice's sum for the bf16 forms, fp32 otherwise).
#include "dg_launch.h"

namespace dg {

namespace {

// cos/sin of the rotation angle of position pos and frequency t (fp64 angle).
__device__ __forceinline__ float2 rope_angle(int pos, int t, int dh, double base, int n_rot) {
  if (t >= n_rot) return make_float2(1.0f, 0.0f);
  const double f = pow(base, -2.0 * static_cast<double>(t) / static_cast<double>(dh));
  const double th = static_cast<double>(pos) * f;
  return make_float2(static_cast<float>(cos(th)), static_cast<float>(sin(th)));
}

// tab[j][t] = (cos, sin) of the angle of position pos0 + j, frequency t
__global__ __launch_bounds__(256) void rope_table_kernel(int pos0, int n_tok, int dh, double base, int n_rot,
                                                         float2 *tab) {
  const int half = dh >> 1;
  const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long long>(n_tok) * half) return;
  const int j = static_cast<int>(i / half), t = static_cast<int>(i - static_cast<long long>(j) * half);
  tab[i] = rope_angle(pos0 + j, t, dh, base, n_rot);
}

// One wave per (token, head item): items are the q heads, then the k heads
// (normed, rotated, written to the cache), then the v heads (unit-RMS in
// global layers, written to the row buffer v_dst; the fused launch below
// writes them to the cache itself and stops at the k heads).  Angles come
// from the table.  Items at or past `items` are left alone.
template <typename T>
__device__ __forceinline__ void norm_rope_item(const NormRopeArgs &a, int j, int it, int items, int lane) {
  const int half = a.dh >> 1;
  T *row = static_cast<T *>(a.qkv) + static_cast<long long>(j) * a.ld;
  const float2 *tab = a.rope_tab + static_cast<long long>(j) * half;
  if (it < items) {
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
      const int kr = a.k_ring ? (a.k_row0 + j) % a.k_ring : a.k_row0 + j;
      dst = static_cast<T *>(a.k_dst) + h * a.k_head_stride + static_cast<long long>(kr) * a.dh;
      w = static_cast<const T *>(a.k_norm);
    } else {
      const int h = it - a.Hq - a.Hkv;
      src = row + a.v_off + h * a.dh;
      dst = static_cast<T *>(a.v_dst) + h * a.v_head_stride + static_cast<long long>(j) * a.dh;
      rope = false;
      norm = a.v_unit_rms != 0;
    }
    // lane handles the 4 consecutive pair indices t0 = 4*lane + 256*i (t0 < half)
    // and their partners t0 + half.  Every load is issued before any value is
    // unpacked, so the wave waits for memory once.
    using Raw = typename std::conditional<sizeof(T) == 2, uint2, float4>::type;
    auto unpack = [](const Raw &r, float *o) {
      if constexpr (sizeof(T) == 2) {
        o[0] = __uint_as_float(r.x << 16);
        o[1] = __uint_as_float(r.x & 0xffff0000u);
        o[2] = __uint_as_float(r.y << 16);
        o[3] = __uint_as_float(r.y & 0xffff0000u);
      } else {
        o[0] = r.x; o[1] = r.y; o[2] = r.z; o[3] = r.w;
      }
    };
    Raw rx0[2], rx1[2], rw0[2], rw1[2];
    float4 rcs[2][2];   // (cos, sin) of pairs t0, t0+1 and t0+2, t0+3
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t0 = 4 * lane + 256 * i;
      if (t0 < half) {
        rx0[i] = *reinterpret_cast<const Raw *>(src + t0);
        rx1[i] = *reinterpret_cast<const Raw *>(src + t0 + half);
        if (w) {
          rw0[i] = *reinterpret_cast<const Raw *>(w + t0);
          rw1[i] = *reinterpret_cast<const Raw *>(w + t0 + half);
        }
        if (rope) {
          rcs[i][0] = *reinterpret_cast<const float4 *>(tab + t0);
          rcs[i][1] = *reinterpret_cast<const float4 *>(tab + t0 + 2);
        }
      }
    }
    float x0[2][4], x1[2][4], wp[2][4], wq[2][4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t0 = 4 * lane + 256 * i;
      if (t0 < half) {
        unpack(rx0[i], x0[i]);
        unpack(rx1[i], x1[i]);
        if (w) {
          unpack(rw0[i], wp[i]);
          unpack(rw1[i], wq[i]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += x0[i][e] * x0[i][e] + x1[i][e] * x1[i][e];
      }
    }
    float scale = 1.0f;
    if (norm) {
      ss = wave_allsum(ss);
      scale = a.sqrt_dh / (sqrtf(ss) + a.eps);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t0 = 4 * lane + 256 * i;
      if (t0 >= half) continue;
      float po[4], qo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
        float p = x0[i][e] * scale, q = x1[i][e] * scale;
        if (w) {
          p *= wp[i][e];
          q *= wq[i][e];
        }
        if (rope) {
          const float4 cs = rcs[i][e >> 1];
          const float c = (e & 1) ? cs.z : cs.x, sv = (e & 1) ? cs.w : cs.y;
          const float o0 = p * c - q * sv;
          const float o1 = q * c + p * sv;
          p = o0;
          q = o1;
        }
        po[e] = p;
        qo[e] = q;
      }
      if constexpr (sizeof(T) == 2) {
        uint2 u, v;
        u.x = static_cast<uint32_t>(f32_to_bf16(po[0])) | (static_cast<uint32_t>(f32_to_bf16(po[1])) << 16);
        u.y = static_cast<uint32_t>(f32_to_bf16(po[2])) | (static_cast<uint32_t>(f32_to_bf16(po[3])) << 16);
        v.x = static_cast<uint32_t>(f32_to_bf16(qo[0])) | (static_cast<uint32_t>(f32_to_bf16(qo[1])) << 16);
        v.y = static_cast<uint32_t>(f32_to_bf16(qo[2])) | (static_cast<uint32_t>(f32_to_bf16(qo[3])) << 16);
        *reinterpret_cast<uint2 *>(dst + t0) = u;
        *reinterpret_cast<uint2 *>(dst + t0 + half) = v;
      } else {
        *reinterpret_cast<float4 *>(dst + t0) = make_float4(po[0], po[1], po[2], po[3]);
        *reinterpret_cast<float4 *>(dst + t0 + half) = make_float4(qo[0], qo[1], qo[2], qo[3]);
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void norm_rope_kernel(const NormRopeArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  norm_rope_item<T>(a, blockIdx.x, blockIdx.y * 4 + wave, a.Hq + 2 * a.Hkv, threadIdx.x & 63);
}

// V heads straight to the transposed cache: one workgroup per (kv head,
// token tile of 32*RH tokens).  All DH/64 column blocks of the tile's rows
// are loaded first (8 lanes per 128-byte row segment, rows t/8 + 32r), the
// unit-RMS scale of each row (global layers) comes from an 8-lane sum, and
// each 64-wide column block is turned around in an LDS tile (two buffers,
// one barrier per block) and stored as 64 dimension rows of 32*RH tokens
// (16-byte stores).  RH * NQ = 8 keeps the rows in 32 registers a thread.
// vt_col0, vt_ld, vt_hs and vt_ring are multiples of 8, so an 8-token chunk
// never wraps the ring.
template <int NQ, int RH>
__device__ __forceinline__ void v_tile_to_cache(const NormRopeArgs &a, int h, int j0, bf16_t (*tile)[64][72]) {
  constexpr int DH = 64 * NQ, TJ = 32 * RH, CH = TJ / 8;   // tokens per tile, 8-token chunks per dimension row
  const int tid = threadIdx.x;
  const int lr = tid >> 3, lc = tid & 7;     // row lr (+32r), 16-byte chunk lc of each 64-wide block
  const bf16_t *base = static_cast<const bf16_t *>(a.qkv) + a.v_off + h * DH;
  uint4 x[RH][NQ];
#pragma unroll
  for (int r = 0; r < RH; ++r) {
    const int j = j0 + lr + 32 * r;
    const bf16_t *src = base + static_cast<long long>(j < a.n_tok ? j : j0) * a.ld + lc * 8;
#pragma unroll
    for (int q = 0; q < NQ; ++q) x[r][q] = *reinterpret_cast<const uint4 *>(src + 64 * q);
  }
  float scale[RH];
#pragma unroll
  for (int r = 0; r < RH; ++r) scale[r] = 1.0f;
  if (a.v_unit_rms) {
#pragma unroll
    for (int r = 0; r < RH; ++r) {
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const uint32_t u[4] = {x[r][q].x, x[r][q].y, x[r][q].z, x[r][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xffff0000u);
          ss += lo * lo + hi * hi;
        }
      }
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 4, 64);
      scale[r] = a.sqrt_dh / (sqrtf(ss) + a.eps);
    }
  }
  bf16_t *o = static_cast<bf16_t *>(a.vt_dst) + h * a.vt_hs;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    bf16_t (*tl)[72] = tile[q & 1];
#pragma unroll
    for (int r = 0; r < RH; ++r) {
      uint4 v = x[r][q];
      if (a.v_unit_rms) {
        uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(u[e] << 16) * scale[r];
          const float hi = __uint_as_float(u[e] & 0xffff0000u) * scale[r];
          u[e] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
        }
        v = make_uint4(u[0], u[1], u[2], u[3]);
      }
      *reinterpret_cast<uint4 *>(&tl[lr + 32 * r][lc * 8]) = v;
    }
    __syncthreads();   // this block's tile written; the block before last (other buffer) is read out
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      const int c = tid + 256 * i;          // 64 * CH chunks: 64 d rows x CH chunks of 8 tokens
      const int dd = c / CH, jc = (c % CH) * 8;
      const int j = j0 + jc;
      if (j >= a.n_tok) continue;
      const long long orow = static_cast<long long>(64 * q + dd) * a.vt_ld;
      if (j + 8 <= a.n_tok) {
        const int col = a.vt_ring ? (a.vt_col0 + j) % a.vt_ring : a.vt_col0 + j;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = static_cast<uint32_t>(tl[jc + 2 * e][dd]) | (static_cast<uint32_t>(tl[jc + 2 * e + 1][dd]) << 16);
        *reinterpret_cast<uint4 *>(o + orow + col) = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        for (int e = 0; j + e < a.n_tok; ++e) {
          const int col = a.vt_ring ? (a.vt_col0 + j + e) % a.vt_ring : a.vt_col0 + j + e;
          o[orow + col] = tl[jc + e][dd];
        }
      }
    }
  }
}

// q and k items of norm_rope_item, with the V heads of the same call handled
// by v_tile_to_cache: the first Hkv * ceil(n_tok / (32 * RH)) workgroups take
// the V tiles, the rest (n_tok per group of four q/k items) one wave per item.
template <int NQ, int RH>
__global__ __launch_bounds__(256) void norm_rope_vt_kernel(const NormRopeArgs a, int n_vt) {
  __shared__ __attribute__((aligned(16))) bf16_t tile[2][64][72];
  const int b = blockIdx.x;
  if (b < n_vt) {
    const int ntj = (a.n_tok + 32 * RH - 1) / (32 * RH);
    v_tile_to_cache<NQ, RH>(a, b / ntj, (b % ntj) * 32 * RH, tile);
    return;
  }
  const int bq = b - n_vt;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  norm_rope_item<bf16_t>(a, bq % a.n_tok, (bq / a.n_tok) * 4 + wave, a.Hq + a.Hkv, threadIdx.x & 63);
}

constexpr int kBKV = 32;  // keys per tile

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Tiles go from global memory straight into LDS (global_load_lds_dwordx4:
// each instruction writes 64 lanes x 16 B = 1 KB contiguous at a wave-
// uniform LDS address), so the layouts are unpadded and the 16-byte chunks
// of a row are XOR-swizzled by the row index to spread MFMA operand reads
// over the LDS banks.
template <typename T, int DH>
struct AttnCfg {
  static constexpr int QT = DH >= 512 ? 1 : 2;      // 16-query tiles per wave
  static constexpr int BQ = 4 * 16 * QT;            // query rows per workgroup
  static constexpr int VEC = 16 / sizeof(T);        // elements per 16-B chunk
  static constexpr int KCPR = DH / VEC;             // K tile: chunks per key row
  static constexpr int VCPR = kBKV / VEC;           // V^T tile: chunks per d row
  static constexpr int KCH = kBKV * KCPR;           // chunks per K tile
  static constexpr int VCH = DH * VCPR;             // chunks per V^T tile
  static constexpr int KINS = KCH / 64;             // 1-KB loads per K tile
  static constexpr int VINS = VCH / 64;
  static constexpr int KSW = KCPR >= 16 ? 15 : KCPR - 1;
  static constexpr int VSW = VCPR - 1;
  // chunk swizzles: K rows by a hash that is distinct over the 16 rows one
  // MFMA reads (keys 8q + {0..3} (+4): see key_row), V^T rows by d / 4 for
  // 16-byte chunks (rows are 64 bytes, four to a bank period)
  __device__ static int kswz(int r) { return ((((r >> 3) << 2) | (r & 3)) & KSW); }
  __device__ static int vswz(int d) { return sizeof(T) == 2 ? ((d >> 2) & VSW) : (d & VSW); }
  static constexpr int DS = DH / 32;                // 32-wide d steps
  static constexpr int DT = DH / 16;                // 16-wide d tiles
  static_assert(KINS % 4 == 0 && VINS % 4 == 0, "each wave issues an equal share of a tile");
};

// K fragment: elements [e0, e0+8) of key row r of a swizzled K tile
template <typename T, int DH>
__device__ __forceinline__ void load_k_frag(Frag<T> &f, const T *tile, int r, int e0) {
  using C = AttnCfg<T, DH>;
  if constexpr (sizeof(T) == 2) {
    const int c = e0 / 8;
    f.load(tile + (r * C::KCPR + (c ^ C::kswz(r))) * 8);
  } else {
    const int c = e0 / 4;
    const float4 a = *reinterpret_cast<const float4 *>(tile + (r * C::KCPR + (c ^ C::kswz(r))) * 4);
    const float4 b = *reinterpret_cast<const float4 *>(tile + (r * C::KCPR + ((c + 1) ^ C::kswz(r))) * 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  }
}

// V^T fragment of row d holding keys 8g..8g+7 (g = lane/16): the key order of
// the P^T fragment built from the S^T accumulators (see key_row).
template <typename T, int DH>
__device__ __forceinline__ void load_v_frag(Frag<T> &f, const T *tile, int d, int lg) {
  using C = AttnCfg<T, DH>;
  if constexpr (sizeof(T) == 2) {
    f.load(tile + (d * C::VCPR + (lg ^ C::vswz(d))) * 8);
  } else {
    const float *row = tile + d * C::VCPR * 4;
    const float4 a = *reinterpret_cast<const float4 *>(row + ((2 * lg) ^ C::vswz(d)) * 4);
    const float4 b = *reinterpret_cast<const float4 *>(row + ((2 * lg + 1) ^ C::vswz(d)) * 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  }
}

// Key order of the score tiles: MFMA row q (0..15) of key tile kt holds key
// 8*(q/4) + 4*kt + q%4 of the 32-key tile, so the accumulator element i of
// lane group g is key 8g + 4kt + i and a lane's eight probabilities are the
// consecutive keys 8g..8g+7.
__device__ __forceinline__ int key_row(int q, int kt) { return ((q >> 2) << 3) | (kt << 2) | (q & 3); }

__device__ __forceinline__ void mask_frag(Frag<bf16_t> &f, const uint32_t *m) {
  uint4 u = *reinterpret_cast<uint4 *>(&f.v);
  u.x &= m[0]; u.y &= m[1]; u.z &= m[2]; u.w &= m[3];
  f.v = *reinterpret_cast<bf16x8 *>(&u);
}
__device__ __forceinline__ void mask_frag(Frag<float> &f, const uint32_t *m) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = __uint_as_float(__float_as_uint(f.v[j]) & m[j]);
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one score column of
// an MFMA tile).  gfx950's row swaps do it in the VALU: swapping a register
// with itself by v_permlane16_swap leaves each lane holding its own value and
// that of lane l ^ 16 in the two results (v_permlane32_swap: lane l ^ 32), so
// no LDS round trip (ds_bpermute) sits in the softmax.
__device__ __forceinline__ float col_max4(float v) {
  if (DG_ATTN_PERMLANE) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}

// One workgroup: kv head g, query rows [r0, r1) of the heads sharing it,
// keys [k_lo, k_hi), all read from the cache (this call's rows sit at
// [kv_len, kv_len + n_tok)).  32-key tiles start at multiples of 32; two
// LDS buffers alternate: tile t+1 streams in while tile t is computed.
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const AttnArgs a) {
  using C = AttnCfg<T, DH>;
  __shared__ __attribute__((aligned(16))) T sK0[C::KCH * C::VEC];
  __shared__ __attribute__((aligned(16))) T sK1[C::KCH * C::VEC];
  __shared__ __attribute__((aligned(16))) T sV0[C::VCH * C::VEC];
  __shared__ __attribute__((aligned(16))) T sV1[C::VCH * C::VEC];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = a.n_rep * a.n_tok;
  const int qblocks = (R + C::BQ - 1) / C::BQ;
  // Consecutive workgroups are dealt round-robin to the 8 XCDs.  Renumber
  // them so that each XCD receives whole runs of query blocks reading the
  // same (kv head, key slice): that slice then stays in the XCD's L2.
  int L = blockIdx.y * gridDim.x + blockIdx.x;
  const int total = gridDim.x * gridDim.y;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int qb = L % qblocks;
  const int split = (L / qblocks) % a.n_split;
  const int g = L / (qblocks * a.n_split);
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
  const int t_first = (k_lo / kBKV) * kBKV;
  const int n_tiles = k_hi > k_lo ? (k_hi - t_first + kBKV - 1) / kBKV : 0;

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

  const T *Kg = static_cast<const T *>(a.k_cache) + g * a.cache_hs;    // [cap][DH]
  const T *Vg = static_cast<const T *>(a.v_cache) + g * a.vcache_hs;   // [DH][cap]
  const int vld = a.vcache_ld;

  // Stream one tile into LDS.  Keys outside [k_lo, k_hi) read a valid row
  // instead (their scores are masked and their values zeroed at use).
  auto issue = [&](int t0, T *kb, T *vb) {
#pragma unroll
    for (int j = 0; j < C::KINS / 4; ++j) {
      const int blk = wave + 4 * j;
      const int p = blk * 64 + lane;
      const int r = p / C::KCPR, c = (p % C::KCPR) ^ C::kswz(r);
      int m = t0 + r;
      m = m < k_lo ? k_lo : (m >= k_hi ? k_hi - 1 : m);
      if (a.ring) m %= a.ring;
      const T *src = Kg + static_cast<long long>(m) * DH + c * C::VEC;
      __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)(kb + blk * 64 * C::VEC), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::VINS / 4; ++j) {
      const int blk = wave + 4 * j;
      const int p = blk * 64 + lane;
      const int d = p / C::VCPR, c = (p % C::VCPR) ^ C::vswz(d);
      int k0 = t0 + c * C::VEC;
      // ring: 32-key tiles start at multiples of 32 and the ring length is a
      // multiple of 32, so a chunk of 8 keys never wraps
      k0 = a.ring ? k0 % a.ring : (k0 > vld - C::VEC ? vld - C::VEC : k0);
      const T *src = Vg + static_cast<long long>(d) * vld + k0;
      __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)(vb + blk * 64 * C::VEC), 16, 0, 0);
    }
  };

  auto compute = [&](int t0, const T *kb, const T *vb) {
    // ---- S^T = K Q^T for 32 keys x (16*QT) queries of this wave
    f32x4 st[2][C::QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt) st[kt][qt] = zero4();
    // K fragments double-buffered in registers: step s+1 is read from LDS
    // while the MFMAs of step s run
    Frag<T> kf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) load_k_frag<T, DH>(kf[0][kt], kb, key_row(l16, kt), lg * 8);
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      if (s + 1 < C::DS) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) load_k_frag<T, DH>(kf[(s + 1) & 1][kt], kb, key_row(l16, kt), (s + 1) * 32 + lg * 8);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt) mma(st[kt][qt], kf[s & 1][kt], qf[qt][s]);
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
          const int m = t0 + lg * 8 + kt * 4 + i;
          bool ok = m >= k_lo && m < k_hi;
          if (a.causal) {
            const int pq = qpos[qt];
            ok = ok && (m <= pq) && (!a.sliding || m > pq - a.window);
          }
          const float v = ok ? st[kt][qt][i] : -INFINITY;
          sv[kt * 4 + i] = v;
          mt = fmaxf(mt, v);
        }
      mt = col_max4(mt);
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
      // rescale the output accumulators only when some lane's running max
      // grew (corr == 1 exactly otherwise): after the first tiles this is rare
      if (__ballot(corr != 1.0f) != 0ull) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          o[dt][qt][0] *= corr;
          o[dt][qt][1] *= corr;
          o[dt][qt][2] *= corr;
          o[dt][qt][3] *= corr;
        }
      }
      pf[qt].from_floats(sv);
    }
    // ---- O^T += V^T P^T; on edge tiles values of keys outside the range
    // are zeroed (their rows may hold anything, e.g. never-written memory)
    const bool edge = (t0 < k_lo) || (t0 + kBKV > k_hi);
    constexpr int NW = sizeof(T) == 2 ? 4 : 8;
    uint32_t vm[NW];
    if (edge) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = t0 + lg * 8 + e;
        const bool ok = m >= k_lo && m < k_hi;
        if constexpr (sizeof(T) == 2) {
          if ((e & 1) == 0) vm[e >> 1] = 0;
          vm[e >> 1] |= ok ? ((e & 1) ? 0xffff0000u : 0x0000ffffu) : 0u;
        } else {
          vm[e] = ok ? 0xffffffffu : 0u;
        }
      }
    }
    Frag<T> vf[2];
    load_v_frag<T, DH>(vf[0], vb, l16, lg);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      if (dt + 1 < C::DT) load_v_frag<T, DH>(vf[(dt + 1) & 1], vb, (dt + 1) * 16 + l16, lg);
      Frag<T> v = vf[dt & 1];
      if (edge) mask_frag(v, vm);
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt) mma(o[dt][qt], v, pf[qt]);
    }
  };

  if (n_tiles > 0) issue(t_first, sK0, sV0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int it = 0; it < n_tiles; it += 2) {
    const int t0 = t_first + it * kBKV;
    if (it + 1 < n_tiles) issue(t0 + kBKV, sK1, sV1);
    compute(t0, sK0, sV0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 >= n_tiles) break;
    if (it + 2 < n_tiles) issue(t0 + 2 * kBKV, sK0, sV0);
    compute(t0 + kBKV, sK1, sV1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

// Split-head form (bf16, d_h 256 / 512): eight waves in four pairs.  The two
// waves of a pair take the same 16*QT query rows and one half of the head
// dimension each, so a wave holds Q and the O accumulator of its half only
// (half the registers: two waves per SIMD instead of one).  Per 32-key tile
// each wave computes the partial scores S^T over its half, the pair swaps
// them through LDS and adds (IEEE addition commutes: both waves hold the
// same scores), both run the same online softmax, and each wave computes
// P V for its half of the output.  Grid, query blocks, key slices and the
// split partials are those of attn_fwd_kernel.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;   // nats a score may exceed the reference max by


// P to bf16: gfx950 packs two floats with round-to-nearest-even in one
// instruction (the same rounding as f32_to_bf16 on the finite values P holds)
__device__ __forceinline__ void p_to_bf16(Frag<bf16_t> &f, const float *s) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f2_t x = {s[2 * j], s[2 * j + 1]};
    w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf2_t));
  }
  f.v = *reinterpret_cast<bf16x8 *>(w);
}

__device__ __forceinline__ void store4(bf16_t *p, const float *f) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(f[0])) | (static_cast<uint32_t>(f32_to_bf16(f[1])) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(f[2])) | (static_cast<uint32_t>(f32_to_bf16(f[3])) << 16);
  *reinterpret_cast<uint2 *>(p) = u;
}
__device__ __forceinline__ void store4(float *p, const float *f) {
  *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
}
// four floats to bf16 by the packed conversion (round to nearest even, as
// f32_to_bf16 on finite values), one 8-byte store
__device__ __forceinline__ void store4_pk(bf16_t *p, const float *f) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  const f2_t a = {f[0], f[1]}, b = {f[2], f[3]};
  uint2 u;
  u.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf2_t));
  u.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf2_t));
  *reinterpret_cast<uint2 *>(p) = u;
}

// Raw buffer resource (gfx9 layout: 48-bit base, stride 0, byte extent,
// word 3 = 32-bit data format), wave-uniform.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t buffer_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p)));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from (resource + soff + voff) into LDS at lds + 16*lane
// (lds wave-uniform).  Issued through inline asm, so the compiler sees no
// LDS write and adds no waits of its own for it (it cannot tell these tiles
// from the other LDS data and would wait for every transfer in flight): the
// caller waits with vmcnt and synchronises before any wave reads the data.
// The instruction writes no register; M0 carries the LDS address (one wait
// state between writing M0 and the load) and is declared clobbered.
__device__ __forceinline__ void dma16(const i32x4_t &rsrc, uint32_t voff, int soff, const void *lds) {
  const uint32_t m0 = static_cast<uint32_t>((uintptr_t)((lds_void_t *)(const_cast<void *>(lds))));
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(soff), "s"(__builtin_amdgcn_readfirstlane(static_cast<int>(m0)))
               : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory loads are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DH>
__global__ __launch_bounds__(512) void attn_pair_kernel(const AttnArgs a) {
  using T = bf16_t;
  using C = AttnCfg<T, DH>;
  constexpr int QT = C::QT;
  constexpr int HALF = DH / 2, DSH = HALF / 32, DTH = HALF / 16;
  static_assert(C::KINS % 8 == 0 && C::VINS % 8 == 0, "eight waves share each tile");
  constexpr int kNK = C::KINS / 8, kNV = C::VINS / 8;   // loads per wave per K / V^T tile
  __shared__ __attribute__((aligned(16))) T sK0[C::KCH * C::VEC];
  __shared__ __attribute__((aligned(16))) T sK1[C::KCH * C::VEC];
  __shared__ __attribute__((aligned(16))) T sV0[C::VCH * C::VEC];
  __shared__ __attribute__((aligned(16))) T sV1[C::VCH * C::VEC];
  __shared__ __attribute__((aligned(16))) float xs[8][2 * QT * 4][64];   // partial scores per wave

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1, hf = wave & 1;
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = a.n_rep * a.n_tok;
  const int qblocks = (R + C::BQ - 1) / C::BQ;
  int L = blockIdx.y * gridDim.x + blockIdx.x;
  const int total = gridDim.x * gridDim.y;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int qb = L % qblocks;
  const int split = (L / qblocks) % a.n_split;
  const int g = L / (qblocks * a.n_split);
  const int r0 = qb * C::BQ;
  const int r1 = min(R, r0 + C::BQ);

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
  const int t_first = (k_lo / kBKV) * kBKV;
  const int n_tiles = k_hi > k_lo ? (k_hi - t_first + kBKV - 1) / kBKV : 0;

  int qrow[QT], qpos[QT];
  bool qval[QT];
  Frag<T> qf[QT][DSH];
  const T *Q = static_cast<const T *>(a.q);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = r0 + pair * 16 * QT + qt * 16 + l16;
    qval[qt] = r < r1;
    const int rr = qval[qt] ? r : r0;
    const int h = g * a.n_rep + rr / a.n_tok;
    const int j = rr % a.n_tok;
    qrow[qt] = rr;
    qpos[qt] = a.kv_len + j;
    const T *qp = Q + static_cast<long long>(j) * a.q_ld + h * DH + hf * HALF;
#pragma unroll
    for (int s = 0; s < DSH; ++s) {
      if (qval[qt]) qf[qt][s].load(qp + s * 32 + lg * 8);
      else qf[qt][s].zero();
    }
  }
  // Consume the Q fragments here, so the compiler waits for their loads once
  // before the tile loop; otherwise it waits (vmcnt(0): every K/V DMA in
  // flight as well) at their first use inside the loop, on every tile.
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int s = 0; s < DSH; ++s) asm volatile("" ::"v"(qf[qt][s].v));

  f32x4 o[DTH][QT];
#pragma unroll
  for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) o[dt][qt] = zero4();
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -1e30f;
    l_run[qt] = 0.f;
  }

  const T *Kg = static_cast<const T *>(a.k_cache) + g * a.cache_hs;
  const T *Vg = static_cast<const T *>(a.v_cache) + g * a.vcache_hs;
  const int vld = a.vcache_ld;

  // Tiles move by buffer loads into LDS (dma16) over resources spanning this
  // kv head's K rows / V^T columns.  A tile that lies wholly inside
  // [k_lo, k_hi) uses a 32-bit per-lane offset inside the tile plus a scalar
  // tile offset; a tile never wraps the ring (tiles start at multiples of 32
  // and the ring length is a multiple of 32).  Other tiles take the general
  // path, whose per-lane offsets clamp each key.
  static_assert(C::VCPR == 4, "V^T chunk swizzle below assumes four 16-byte chunks per row");
  // K: with 64 chunks per row (d_h 512) load j of a wave covers row
  // wave + 8j, so its lane offset is (lane ^ swizzle) * 16, formed in the
  // loop from the lane index rather than held in registers (the d_h 512
  // kernel has none to spare); narrower rows keep precomputed offsets.
  constexpr bool kRowPerLoad = C::KCPR == 64;
  uint32_t koff[kRowPerLoad ? 1 : kNK] = {};
  if constexpr (!kRowPerLoad) {
#pragma unroll
    for (int j = 0; j < kNK; ++j) {
      const int p = (wave + 8 * j) * 64 + lane;
      const int r = p / C::KCPR, c = (p % C::KCPR) ^ C::kswz(r);
      koff[j] = static_cast<uint32_t>((r * DH + c * C::VEC) * sizeof(T));
    }
  }
  // V^T chunk (wave + 8j)*64 + lane is row d = (wave + 8j)*16 + lane/4; its
  // swizzle (d/4) % 4 = (lane/16) % 4 is the same for every j
  const uint32_t voff = static_cast<uint32_t>(
      ((lane >> 2) * vld + (((lane & 3) ^ ((lane >> 4) & 3)) * C::VEC)) * sizeof(T));
  // byte extents below 2^31 (the launcher sends larger caches to attn_fwd_kernel)
  const i32x4_t k_rsrc = buffer_rsrc(Kg, static_cast<uint32_t>((a.ring ? a.ring : k_hi) * DH * sizeof(T)));
  const i32x4_t v_rsrc = buffer_rsrc(Vg, static_cast<uint32_t>(DH * vld * sizeof(T)));

  auto issue_k = [&](int t0, T *kb) {
    if (t0 >= k_lo && t0 + kBKV <= k_hi) {
      const int row0 = a.ring ? t0 % a.ring : t0;
      const int soff = row0 * DH * static_cast<int>(sizeof(T));
      if constexpr (kRowPerLoad) {
        uint32_t ln;   // lane index, recomputed here (not hoisted, not spilled)
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const uint32_t l16 = ln << 4;
#pragma unroll
        for (int j = 0; j < kNK; ++j) {
          const int r = wave + 8 * j;
          dma16(k_rsrc, l16 ^ static_cast<uint32_t>(C::kswz(r) * 16), soff + r * DH * static_cast<int>(sizeof(T)),
                kb + r * 64 * C::VEC);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kNK; ++j) dma16(k_rsrc, koff[j], soff, kb + (wave + 8 * j) * 64 * C::VEC);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < kNK; ++j) {
      const int blk = wave + 8 * j;
      const int p = blk * 64 + lane;
      const int r = p / C::KCPR, c = (p % C::KCPR) ^ C::kswz(r);
      int m = t0 + r;
      m = m < k_lo ? k_lo : (m >= k_hi ? k_hi - 1 : m);
      if (a.ring) m %= a.ring;
      dma16(k_rsrc, static_cast<uint32_t>((m * DH + c * C::VEC) * sizeof(T)), 0, kb + blk * 64 * C::VEC);
    }
  };
  auto issue_v = [&](int t0, T *vb) {
    if (a.ring || t0 + kBKV <= vld) {
      const int col0 = a.ring ? t0 % a.ring : t0;
#pragma unroll
      for (int j = 0; j < kNV; ++j)
        dma16(v_rsrc, voff, (col0 + (wave + 8 * j) * 16 * vld) * static_cast<int>(sizeof(T)),
              vb + (wave + 8 * j) * 64 * C::VEC);
      return;
    }
#pragma unroll
    for (int j = 0; j < kNV; ++j) {
      const int blk = wave + 8 * j;
      const int p = blk * 64 + lane;
      const int d = p / C::VCPR, c = (p % C::VCPR) ^ C::vswz(d);
      int k0 = t0 + c * C::VEC;
      // ring: a chunk of 8 keys never wraps (see above)
      k0 = a.ring ? k0 % a.ring : (k0 > vld - C::VEC ? vld - C::VEC : k0);
      dma16(v_rsrc, static_cast<uint32_t>((d * vld + k0) * sizeof(T)), 0, vb + blk * 64 * C::VEC);
    }
  };

  // Wave-uniform bounds of this wave's query positions: a tile needs no
  // per-score mask when every key in it is visible to every query here.
  int pq_min = qpos[0], pq_max = qpos[0];
#pragma unroll
  for (int qt = 1; qt < QT; ++qt) {
    pq_min = min(pq_min, qpos[qt]);
    pq_max = max(pq_max, qpos[qt]);
  }
  if (a.causal) {   // the bounds serve only the causal masks
    pq_min = wave_allreduce_i(pq_min, [](int x, int y) { return min(x, y); });
    pq_max = wave_allreduce_i(pq_max, [](int x, int y) { return max(x, y); });
  }
  pq_min = __builtin_amdgcn_readfirstlane(pq_min);
  pq_max = __builtin_amdgcn_readfirstlane(pq_max);

  // One 32-key tile.  Loads run two deep per operand: K(i+2) is issued once
  // every wave has read K(i) (after the score exchange), V(i+1) once every
  // wave has finished P V on tile i-1 (after the barrier that opens tile i).
  // The DMA queue per wave is therefore K0 V0 K1 V1 K2 ..., and the waits
  // count loads issued after the one needed: K(i) is followed by V(i) and
  // K(i+1); V(i), waited for before the exchange barrier, by K(i+1) and
  // V(i+1) (and K(i+2) too where a third barrier before P V carries it),
  // each present if that tile is.
  auto tile = [&](int ti, T *kb, const T *vb, T *vb_next) {
    const int t0 = t_first + ti * kBKV;
    const bool in_range = t0 >= k_lo && t0 + kBKV <= k_hi;
    const bool unmasked = in_range && (!a.causal || (t0 + kBKV - 1 <= pq_min &&
                                                     (!a.sliding || t0 > pq_max - a.window)));
    if (ti + 1 < n_tiles) wait_vm<kNV + kNK>();
    else wait_vm<kNV>();
    lds_sync();   // not __syncthreads(): its fence would wait for every DMA in flight
    if (ti + 1 < n_tiles) issue_v(t0 + kBKV, vb_next);
    // ---- partial S^T = K Q^T over this wave's half of the head dimension
    f32x4 st[2][QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) st[kt][qt] = zero4();
    Frag<T> kf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) load_k_frag<T, DH>(kf[0][kt], kb, key_row(l16, kt), hf * HALF + lg * 8);
#pragma unroll
    for (int s = 0; s < DSH; ++s) {
      if (s + 1 < DSH) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          load_k_frag<T, DH>(kf[(s + 1) & 1][kt], kb, key_row(l16, kt), hf * HALF + (s + 1) * 32 + lg * 8);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(st[kt][qt], kf[s & 1][kt], qf[qt][s]);
    }
    // ---- swap halves with the partner wave and add
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) xs[wave][(kt * QT + qt) * 4 + i][lane] = st[kt][qt][i];
    if (DG_PAIR_V_AT_EXCHANGE) {
      // V(i) was issued a tile and a half ago; waiting for it here lets the
      // exchange barrier publish it too (loads in flight after it: K(i+1)
      // and V(i+1), if that tile exists)
      if (ti + 1 < n_tiles) wait_vm<kNK + kNV>();
      else wait_vm<0>();
    }
    lds_sync();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[kt][qt][i] += xs[wave ^ 1][(kt * QT + qt) * 4 + i][lane];
    if (ti + 2 < n_tiles) issue_k(t0 + 2 * kBKV, kb);
    // ---- mask (tiles cut by the key range, the causal diagonal or the
    // window only), online softmax (identical in both waves of the pair)
    if (!unmasked) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = t0 + lg * 8 + kt * 4 + i;
            bool ok = m >= k_lo && m < k_hi;
            if (a.causal) {
              const int pq = qpos[qt];
              ok = ok && (m <= pq) && (!a.sliding || m > pq - a.window);
            }
            if (!ok) st[kt][qt][i] = -INFINITY;
          }
    }
    Frag<T> pf[QT];
    float corr[QT];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mt = -1e30f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) mt = fmaxf(mt, fmaxf(fmaxf(st[kt][qt][0], st[kt][qt][1]),
                                                          fmaxf(st[kt][qt][2], st[kt][qt][3])));
      mt = col_max4(mt);
      corr[qt] = mt;
      grow = grow || mt > m_run[qt] + kRescaleSlack;
    }
    // The reference maximum moves only when a score exceeds it by more than
    // kRescaleSlack (then for every query of the wave, so the O rescale is
    // one uniform branch); until then exp(s - m) <= e^kRescaleSlack, and
    // O / l is the same quotient.
    if (__ballot(grow) != 0ull) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float m_new = fmaxf(m_run[qt], corr[qt]);
        const float c = __builtin_amdgcn_exp2f((m_run[qt] - m_new) * kLog2e);
        m_run[qt] = m_new;
        l_run[qt] *= c;
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) {
          o[dt][qt][0] *= c;
          o[dt][qt][1] *= c;
          o[dt][qt][2] *= c;
          o[dt][qt][3] *= c;
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float nm = -m_run[qt] * kLog2e;
      float sv[8];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(st[kt][qt][i], kLog2e, nm));
          sv[kt * 4 + i] = e;
          psum += e;
        }
      l_run[qt] += psum;
      p_to_bf16(pf[qt], sv);
    }
    // ---- O^T += V^T P^T over this wave's half (tiles cut by the key range:
    // values of keys outside it are zeroed, as the cache holds anything there)
    if (!DG_PAIR_V_AT_EXCHANGE) {
      if (ti + 2 < n_tiles) wait_vm<2 * kNK + kNV>();
      else if (ti + 1 < n_tiles) wait_vm<kNK + kNV>();
      else wait_vm<0>();
      lds_sync();
    }
    Frag<T> vf[2];
    load_v_frag<T, DH>(vf[0], vb, hf * HALF + l16, lg);
    if (in_range) {
#pragma unroll
      for (int dt = 0; dt < DTH; ++dt) {
        if (dt + 1 < DTH) load_v_frag<T, DH>(vf[(dt + 1) & 1], vb, hf * HALF + (dt + 1) * 16 + l16, lg);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(o[dt][qt], vf[dt & 1], pf[qt]);
      }
    } else {
      uint32_t vm[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = t0 + lg * 8 + e;
        const bool ok = m >= k_lo && m < k_hi;
        if ((e & 1) == 0) vm[e >> 1] = 0;
        vm[e >> 1] |= ok ? ((e & 1) ? 0xffff0000u : 0x0000ffffu) : 0u;
      }
#pragma unroll
      for (int dt = 0; dt < DTH; ++dt) {
        if (dt + 1 < DTH) load_v_frag<T, DH>(vf[(dt + 1) & 1], vb, hf * HALF + (dt + 1) * 16 + l16, lg);
        Frag<T> v = vf[dt & 1];
        mask_frag(v, vm);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(o[dt][qt], v, pf[qt]);
      }
    }
  };

  if (n_tiles > 0) {
    issue_k(t_first, sK0);
    issue_v(t_first, sV0);
  }
  if (n_tiles > 1) issue_k(t_first + kBKV, sK1);
  for (int it = 0; it < n_tiles; it += 2) {
    tile(it, sK0, sV0, sV1);
    if (it + 1 >= n_tiles) break;
    tile(it + 1, sK1, sV1, sV0);
  }

  // ---- finish: lanes sharing a query (same l16) hold partial sums of l
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l = l_run[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (!qval[qt]) continue;
    const int rr = qrow[qt];
    if (a.n_split == 1) {
      const int h = g * a.n_rep + rr / a.n_tok;
      const int j = rr % a.n_tok;
      T *op = static_cast<T *>(a.out) + static_cast<long long>(j) * a.out_ld + h * DH + hf * HALF;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) op[dt * 16 + lg * 4 + i] = f32_to_bf16(o[dt][qt][i] * inv);
    } else {
      // split partials as in the solo form: rows divided by this split's l, bf16
      const long long prow = static_cast<long long>(split) * a.Hkv * R + static_cast<long long>(g) * R + rr;
      T *op = reinterpret_cast<T *>(a.o_part) + prow * DH + hf * HALF;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DTH; ++dt) {
        const float f[4] = {o[dt][qt][0] * inv, o[dt][qt][1] * inv, o[dt][qt][2] * inv, o[dt][qt][3] * inv};
        store4_pk(op + dt * 16 + lg * 4, f);
      }
      if (lg == 0 && hf == 0) {
        a.ml_part[prow * 2] = m_run[qt];
        a.ml_part[prow * 2 + 1] = l;
      }
    }
  }
}


// Solo form of the bf16 attention: each wave owns QT 16-query tiles over the
// whole head dimension, so its scores need no exchange with another wave and
// every softmax runs once.  NW waves share each K / V^T tile.  NBUF tile
// buffers form a ring: the loads of tile i + NBUF - 1 are issued at the start
// of tile i, into the buffers tile i - 1 used, and one workgroup barrier per
// tile hands them over (after it every wave has finished tile i - 1).
// Tile loads, key order, masking and the online softmax are those of the
// pair form above.
// Split partials: each split stores its rows divided by its own normaliser
// (O_s / l_s, a convex combination of value rows) rounded to bf16, beside
// fp32 (m_s, l_s); the merge weights split s by l_s exp(m_s - M) / sum.
template <int DH, int QT, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void attn_solo_kernel(const AttnArgs a) {
  using T = bf16_t;
  using C = AttnCfg<T, DH>;
  constexpr int BQ = NW * 16 * QT;
  constexpr int DS = DH / 32, DT = DH / 16;
  static_assert(C::KINS % NW == 0 && C::VINS % NW == 0, "the waves share each tile's loads equally");
  constexpr int kNK = C::KINS / NW, kNV = C::VINS / NW;   // loads per wave per K / V^T tile
  static_assert(NBUF >= 2 && NBUF <= 3, "two or three tile buffers");
  __shared__ __attribute__((aligned(16))) T sK[NBUF][C::KCH * C::VEC];
  __shared__ __attribute__((aligned(16))) T sV[NBUF][C::VCH * C::VEC];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = a.n_rep * a.n_tok;
  const int qblocks = (R + BQ - 1) / BQ;
  int L = blockIdx.y * gridDim.x + blockIdx.x;
  const int total = gridDim.x * gridDim.y;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int qb = L % qblocks;
  const int split = (L / qblocks) % a.n_split;
  const int g = L / (qblocks * a.n_split);
  const int r0 = qb * BQ;
  const int r1 = min(R, r0 + BQ);

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
  const int t_first = (k_lo / kBKV) * kBKV;
  const int n_tiles = k_hi > k_lo ? (k_hi - t_first + kBKV - 1) / kBKV : 0;

  // This wave's queries: positions first (the tile masks need them), the
  // fragments after the first tiles' loads are issued, so the two latencies
  // overlap; they are consumed before the loop, so their wait (which also
  // covers those tile loads) is not repeated on every tile.
  int qrow[QT], qpos[QT];
  bool qval[QT];
  const T *qptr[QT];
  Frag<T> qf[QT][DS];
  const T *Q = static_cast<const T *>(a.q);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = r0 + wave * 16 * QT + qt * 16 + l16;
    qval[qt] = r < r1;
    const int rr = qval[qt] ? r : r0;
    const int h = g * a.n_rep + rr / a.n_tok;
    const int j = rr % a.n_tok;
    qrow[qt] = rr;
    qpos[qt] = a.kv_len + j;
    qptr[qt] = Q + static_cast<long long>(j) * a.q_ld + h * DH;
  }
  auto qload = [&]() {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        if (qval[qt]) qf[qt][s].load(qptr[qt] + s * 32 + lg * 8);
        else qf[qt][s].zero();
      }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int s = 0; s < DS; ++s) asm volatile("" ::"v"(qf[qt][s].v));
  };

  f32x4 o[DT][QT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) o[dt][qt] = zero4();
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -1e30f;
    l_run[qt] = 0.f;
  }

  const T *Kg = static_cast<const T *>(a.k_cache) + g * a.cache_hs;
  const T *Vg = static_cast<const T *>(a.v_cache) + g * a.vcache_hs;
  const int vld = a.vcache_ld;
  static_assert(C::VCPR == 4, "V^T chunk swizzle below assumes four 16-byte chunks per row");
  constexpr bool kRowPerLoad = C::KCPR == 64;
  uint32_t koff[kRowPerLoad ? 1 : kNK] = {};
  if constexpr (!kRowPerLoad) {
#pragma unroll
    for (int j = 0; j < kNK; ++j) {
      const int p = (wave + NW * j) * 64 + lane;
      const int r = p / C::KCPR, c = (p % C::KCPR) ^ C::kswz(r);
      koff[j] = static_cast<uint32_t>((r * DH + c * C::VEC) * sizeof(T));
    }
  }
  // V^T chunk (wave + NW j)*64 + lane is row d = (wave + NW j)*16 + lane/4;
  // its swizzle (d/4) % 4 = (lane/16) % 4 is the same for every j
  const uint32_t voff = static_cast<uint32_t>(
      ((lane >> 2) * vld + (((lane & 3) ^ ((lane >> 4) & 3)) * C::VEC)) * sizeof(T));
  const i32x4_t k_rsrc = buffer_rsrc(Kg, static_cast<uint32_t>((a.ring ? a.ring : k_hi) * DH * sizeof(T)));
  const i32x4_t v_rsrc = buffer_rsrc(Vg, static_cast<uint32_t>(DH * vld * sizeof(T)));

  auto issue_k = [&](int t0, T *kb) {
    if (t0 >= k_lo && t0 + kBKV <= k_hi) {
      const int row0 = a.ring ? t0 % a.ring : t0;
      const int soff = row0 * DH * static_cast<int>(sizeof(T));
      if constexpr (kRowPerLoad) {
        uint32_t ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const uint32_t l16b = ln << 4;
#pragma unroll
        for (int j = 0; j < kNK; ++j) {
          const int r = wave + NW * j;
          dma16(k_rsrc, l16b ^ static_cast<uint32_t>(C::kswz(r) * 16), soff + r * DH * static_cast<int>(sizeof(T)),
                kb + r * 64 * C::VEC);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kNK; ++j) dma16(k_rsrc, koff[j], soff, kb + (wave + NW * j) * 64 * C::VEC);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < kNK; ++j) {
      const int blk = wave + NW * j;
      const int p = blk * 64 + lane;
      const int r = p / C::KCPR, c = (p % C::KCPR) ^ C::kswz(r);
      int m = t0 + r;
      m = m < k_lo ? k_lo : (m >= k_hi ? k_hi - 1 : m);
      if (a.ring) m %= a.ring;
      dma16(k_rsrc, static_cast<uint32_t>((m * DH + c * C::VEC) * sizeof(T)), 0, kb + blk * 64 * C::VEC);
    }
  };
  auto issue_v = [&](int t0, T *vb) {
    if (a.ring || t0 + kBKV <= vld) {
      const int col0 = a.ring ? t0 % a.ring : t0;
#pragma unroll
      for (int j = 0; j < kNV; ++j)
        dma16(v_rsrc, voff, (col0 + (wave + NW * j) * 16 * vld) * static_cast<int>(sizeof(T)),
              vb + (wave + NW * j) * 64 * C::VEC);
      return;
    }
#pragma unroll
    for (int j = 0; j < kNV; ++j) {
      const int blk = wave + NW * j;
      const int p = blk * 64 + lane;
      const int d = p / C::VCPR, c = (p % C::VCPR) ^ C::vswz(d);
      int k0 = t0 + c * C::VEC;
      k0 = a.ring ? k0 % a.ring : (k0 > vld - C::VEC ? vld - C::VEC : k0);
      dma16(v_rsrc, static_cast<uint32_t>((d * vld + k0) * sizeof(T)), 0, vb + blk * 64 * C::VEC);
    }
  };

  int pq_min = qpos[0], pq_max = qpos[0];
#pragma unroll
  for (int qt = 1; qt < QT; ++qt) {
    pq_min = min(pq_min, qpos[qt]);
    pq_max = max(pq_max, qpos[qt]);
  }
  if (a.causal) {   // the bounds serve only the causal masks
    pq_min = wave_allreduce_i(pq_min, [](int x, int y) { return min(x, y); });
    pq_max = wave_allreduce_i(pq_max, [](int x, int y) { return max(x, y); });
  }
  pq_min = __builtin_amdgcn_readfirstlane(pq_min);
  pq_max = __builtin_amdgcn_readfirstlane(pq_max);

  // One 32-key tile.  This wave's loads in flight at its start are those of
  // this tile and, with three buffers, of the next one if it exists (loads
  // complete in issue order).
  auto tile = [&](int ti, const T *kb, const T *vb, T *kb_next, T *vb_next) {
    const int t0 = t_first + ti * kBKV;
    const bool in_range = t0 >= k_lo && t0 + kBKV <= k_hi;
    const bool unmasked = in_range && (!a.causal || (t0 + kBKV - 1 <= pq_min &&
                                                     (!a.sliding || t0 > pq_max - a.window)));
    if (NBUF == 3 && ti + 1 < n_tiles) wait_vm<kNK + kNV>();
    else wait_vm<0>();
    lds_sync();   // every wave's share of this tile has landed; tile ti - 1's buffers are free
    if (ti + NBUF - 1 < n_tiles) {
      issue_k(t0 + (NBUF - 1) * kBKV, kb_next);
      issue_v(t0 + (NBUF - 1) * kBKV, vb_next);
    }
    // ---- S^T = K Q^T over the whole head dimension: every K fragment of
    // the tile is read from LDS before the first product, so one LDS latency
    // is exposed per tile rather than one per step
    f32x4 st[2][QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) st[kt][qt] = zero4();
    {
      Frag<T> kf[DS][2];
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) load_k_frag<T, DH>(kf[s][kt], kb, key_row(l16, kt), s * 32 + lg * 8);
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) mma(st[kt][qt], kf[s][kt], qf[qt][s]);
    }
    // the first VD V^T fragments are read now, so their latency hides behind
    // the softmax; the rest run VD steps ahead of their products
    constexpr int VD = DT < DG_SOLO_VDEPTH ? DT : DG_SOLO_VDEPTH;
    Frag<T> vf[VD];
#pragma unroll
    for (int dt = 0; dt < VD; ++dt) load_v_frag<T, DH>(vf[dt], vb, dt * 16 + l16, lg);
    // ---- mask (tiles cut by the key range, the causal diagonal or the window)
    if (!unmasked) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = t0 + lg * 8 + kt * 4 + i;
            bool ok = m >= k_lo && m < k_hi;
            if (a.causal) {
              const int pq = qpos[qt];
              ok = ok && (m <= pq) && (!a.sliding || m > pq - a.window);
            }
            if (!ok) st[kt][qt][i] = -INFINITY;
          }
    }
    // ---- online softmax (reference maximum moved past kRescaleSlack only)
    Frag<T> pf[QT];
    float corr[QT];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mt = -1e30f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) mt = fmaxf(mt, fmaxf(fmaxf(st[kt][qt][0], st[kt][qt][1]),
                                                          fmaxf(st[kt][qt][2], st[kt][qt][3])));
      mt = col_max4(mt);
      corr[qt] = mt;
      grow = grow || mt > m_run[qt] + kRescaleSlack;
    }
    if (__ballot(grow) != 0ull) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float m_new = fmaxf(m_run[qt], corr[qt]);
        const float c = __builtin_amdgcn_exp2f((m_run[qt] - m_new) * kLog2e);
        m_run[qt] = m_new;
        l_run[qt] *= c;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          o[dt][qt][0] *= c;
          o[dt][qt][1] *= c;
          o[dt][qt][2] *= c;
          o[dt][qt][3] *= c;
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float nm = -m_run[qt] * kLog2e;
      float sv[8];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(st[kt][qt][i], kLog2e, nm));
          sv[kt * 4 + i] = e;
          psum += e;
        }
      l_run[qt] += psum;
      p_to_bf16(pf[qt], sv);
    }
    // ---- O^T += V^T P^T (tiles cut by the key range: values of keys
    // outside it are zeroed, as the cache holds anything there)
    if (in_range) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(o[dt][qt], vf[dt % VD], pf[qt]);
        if (dt + VD < DT) load_v_frag<T, DH>(vf[dt % VD], vb, (dt + VD) * 16 + l16, lg);
      }
    } else {
      uint32_t vm[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = t0 + lg * 8 + e;
        const bool ok = m >= k_lo && m < k_hi;
        if ((e & 1) == 0) vm[e >> 1] = 0;
        vm[e >> 1] |= ok ? ((e & 1) ? 0xffff0000u : 0x0000ffffu) : 0u;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        mask_frag(vf[dt % VD], vm);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(o[dt][qt], vf[dt % VD], pf[qt]);
        if (dt + VD < DT) load_v_frag<T, DH>(vf[dt % VD], vb, (dt + VD) * 16 + l16, lg);
      }
    }
  };

#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p) {
    if (p < n_tiles) {
      issue_k(t_first + p * kBKV, sK[p]);
      issue_v(t_first + p * kBKV, sV[p]);
    }
  }
  qload();
  // unrolled over the ring, so every buffer address is a constant
  for (int ti = 0; ti < n_tiles; ti += NBUF) {
    tile(ti, sK[0], sV[0], sK[NBUF - 1], sV[NBUF - 1]);
    if (ti + 1 >= n_tiles) break;
    tile(ti + 1, sK[1], sV[1], sK[0], sV[0]);
    if constexpr (NBUF == 3) {
      if (ti + 2 >= n_tiles) break;
      tile(ti + 2, sK[2], sV[2], sK[1], sV[1]);
    }
  }

  // ---- finish: lanes sharing a query (same l16) hold partial sums of l
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
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
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) op[dt * 16 + lg * 4 + i] = f32_to_bf16(o[dt][qt][i] * inv);
    } else {
      const long long prow = static_cast<long long>(split) * a.Hkv * R + static_cast<long long>(g) * R + rr;
      T *op = reinterpret_cast<T *>(a.o_part) + prow * DH;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float f[4] = {o[dt][qt][0] * inv, o[dt][qt][1] * inv, o[dt][qt][2] * inv, o[dt][qt][3] * inv};
        store4_pk(op + dt * 16 + lg * 4, f);
      }
      if (lg == 0) {
        a.ml_part[prow * 2] = m_run[qt];
        a.ml_part[prow * 2 + 1] = l;
      }
    }
  }
}


// Merge of the split-KV partials, one wave per (kv head, row): lane s reads
// split s's (max, sum) and the wave forms w_s = exp(m_s - M) / sum_s l_s
// exp(m_s - M) by reductions (no barrier); every lane then adds its four
// columns over the splits in order.
// BP: the partial rows are bf16 and already divided by their split's l
// (the solo form), so split s is weighted by l_s exp(m_s - M) / L.
template <typename T, bool BP>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a, int dh) {
  const int R = a.n_rep * a.n_tok;
  const long long rows = static_cast<long long>(a.Hkv) * R;
  const int lane = threadIdx.x & 63;
  const long long idx = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (idx >= rows) return;
  // lane s holds split s (n_split <= 64): max and normaliser by wave reductions
  const int ns = a.n_split;
  float m = -1e30f, l = 0.f;
  if (lane < ns) {
    m = a.ml_part[(lane * rows + idx) * 2];
    l = a.ml_part[(lane * rows + idx) * 2 + 1];
  }
  const float M = wave_allmax(m);
  const float e = lane < ns ? __expf(m - M) : 0.f;
  const float L = wave_allsum(l * e);
  const float wl = L > 0.f ? (BP ? l * e : e) / L : 0.f;
  const int g = static_cast<int>(idx / R), rr = static_cast<int>(idx % R);
  const int h = g * a.n_rep + rr / a.n_tok;
  const int j = rr % a.n_tok;
  T *op = static_cast<T *>(a.out) + static_cast<long long>(j) * a.out_ld + h * dh;
  for (int d = lane * 4; d < dh; d += 256) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      // split s's weight from lane s (a wave-uniform index: a VALU read, no LDS)
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s));
      float4 v;
      if constexpr (BP) {
        const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const bf16_t *>(a.o_part) +
                                                         (s * rows + idx) * dh + d);
        v = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                        __uint_as_float(u.y & 0xffff0000u));
      } else {
        v = *reinterpret_cast<const float4 *>(a.o_part + (s * rows + idx) * dh + d);
      }
      acc[0] += w * v.x;
      acc[1] += w * v.y;
      acc[2] += w * v.z;
      acc[3] += w * v.w;
    }
    store4(op + d, acc);
  }
}

// dst[h][d][col0 + j] = src[h][j][d]: values stored dimension-major (V^T)
// through a 64 x 64 LDS tile.
// bf16 with 8-aligned destination columns: 16-byte loads of token rows and
// 16-byte stores of dimension rows, the tile transposed in LDS.
__global__ __launch_bounds__(256) void v_transpose16_kernel(const bf16_t *src, int n, int dh, bf16_t *dst,
                                                            long long dst_hs, int dst_ld, int col0, int ring) {
  __shared__ bf16_t tile[64][72];   // [token][d], rows padded by 16 bytes
  const int h = blockIdx.z;
  const int j0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const bf16_t *s = src + static_cast<long long>(h) * n * dh;
  bf16_t *o = dst + h * dst_hs;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = tid + 256 * q;          // 512 chunks: 64 tokens x 8 chunks of 8 d
    const int jj = c >> 3, dc = (c & 7) * 8;
    const int j = j0 + jj, d = d0 + dc;
    if (j < n && d < dh)
      *reinterpret_cast<uint4 *>(&tile[jj][dc]) = *reinterpret_cast<const uint4 *>(s + static_cast<long long>(j) * dh + d);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = tid + 256 * q;          // 512 chunks: 64 d rows x 8 chunks of 8 tokens
    const int dd = c >> 3, jc = (c & 7) * 8;
    const int d = d0 + dd, j = j0 + jc;
    if (d >= dh || j >= n) continue;
    if (j + 8 <= n) {
      // col0, j and the ring length are multiples of 8: the 8 columns never wrap
      const int col = ring ? (col0 + j) % ring : col0 + j;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = static_cast<uint32_t>(tile[jc + 2 * e][dd]) | (static_cast<uint32_t>(tile[jc + 2 * e + 1][dd]) << 16);
      *reinterpret_cast<uint4 *>(o + static_cast<long long>(d) * dst_ld + col) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      for (int e = 0; j + e < n; ++e) {
        const int col = ring ? (col0 + j + e) % ring : col0 + j + e;
        o[static_cast<long long>(d) * dst_ld + col] = tile[jc + e][dd];
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void v_transpose_kernel(const T *src, int n, int dh, T *dst, long long dst_hs,
                                                          int dst_ld, int col0, int ring) {
  __shared__ T tile[64][65];
  const int h = blockIdx.z;
  const int j0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
  const T *s = src + static_cast<long long>(h) * n * dh;
  T *o = dst + h * dst_hs;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int j = j0 + i, d = d0 + tx;
    if (j < n && d < dh) tile[i][tx] = s[static_cast<long long>(j) * dh + d];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int d = d0 + i, j = j0 + tx;
    if (j < n && d < dh) o[static_cast<long long>(d) * dst_ld + (ring ? (col0 + j) % ring : col0 + j)] = tile[tx][i];
  }
}

template <int DH>
struct SoloCfg {
  static constexpr bool on = (DG_ATTN_SOLO >> (DH == 512 ? 1 : 0)) & 1;
  static constexpr int QT = DH == 512 ? DG_SOLO512_QT : DG_SOLO256_QT;
  static constexpr int NW = DH == 512 ? DG_SOLO512_NW : DG_SOLO256_NW;
  static constexpr int BQ = NW * 16 * QT;
  // three tile buffers where they fit beside nothing else in 160 KB of LDS
  static constexpr int tile_bytes = 2 * kBKV * DH * 2;
  static constexpr int NBUF = (DG_SOLO_NBUF >= 3 && 3 * tile_bytes <= 160 * 1024) ? 3 : 2;
};

template <typename T, int DH>
hipError_t launch_attn_t(const AttnArgs &a, hipStream_t s) {
  using C = AttnCfg<T, DH>;
  const int R = a.n_rep * a.n_tok;
  const int qblocks = (R + C::BQ - 1) / C::BQ;
  bool bf16_parts = false;   // the solo and pair forms write bf16 split partials
  if constexpr (sizeof(T) == 2 && (DH == 256 || DH == 512)) {
    // the solo and pair forms address a head's cache with 32-bit byte offsets
    const bool fits = static_cast<long long>(a.vcache_ld) * DH * static_cast<long long>(sizeof(T)) < (1ll << 31);
    bool solo = false;
    if constexpr (SoloCfg<DH>::on) {
      using S = SoloCfg<DH>;
      if (fits) {
        const int qb = (R + S::BQ - 1) / S::BQ;
        hipLaunchKernelGGL((attn_solo_kernel<DH, S::QT, S::NW, S::NBUF>), dim3(a.Hkv * qb, a.n_split),
                           dim3(S::NW * 64), 0, s, a);
        solo = true;
      }
    }
    if (solo) {
      bf16_parts = true;
    } else if (DG_ATTN_PAIR && fits) {
      hipLaunchKernelGGL((attn_pair_kernel<DH>), dim3(a.Hkv * qblocks, a.n_split), dim3(512), 0, s, a);
      bf16_parts = true;
    } else {
      hipLaunchKernelGGL((attn_fwd_kernel<T, DH>), dim3(a.Hkv * qblocks, a.n_split), dim3(256), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<T, DH>), dim3(a.Hkv * qblocks, a.n_split), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  if (bf16_parts)
    hipLaunchKernelGGL((attn_combine_kernel<T, true>), dim3((a.Hkv * R + 3) / 4), dim3(256), 0, s, a, DH);
  else
    hipLaunchKernelGGL((attn_combine_kernel<T, false>), dim3((a.Hkv * R + 3) / 4), dim3(256), 0, s, a, DH);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_v_transpose(int dtype, const void *src, int n, int Hkv, int dh, void *dst, long long dst_hs,
                              int dst_ld, int col0, hipStream_t s, int ring) {
  if (n <= 0) return hipSuccess;
  dim3 grid((n + 63) / 64, (dh + 63) / 64, Hkv);
  const bool vec = dtype == DG_BF16 && col0 % 8 == 0 && dst_ld % 8 == 0 && dst_hs % 8 == 0 && dh % 8 == 0 &&
                   ring % 8 == 0;
  if (vec)
    hipLaunchKernelGGL(v_transpose16_kernel, grid, dim3(256), 0, s, static_cast<const bf16_t *>(src), n, dh,
                       static_cast<bf16_t *>(dst), dst_hs, dst_ld, col0, ring);
  else if (dtype == DG_BF16)
    hipLaunchKernelGGL(v_transpose_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t *>(src), n, dh,
                       static_cast<bf16_t *>(dst), dst_hs, dst_ld, col0, ring);
  else
    hipLaunchKernelGGL(v_transpose_kernel<float>, grid, dim3(256), 0, s, static_cast<const float *>(src), n, dh,
                       static_cast<float *>(dst), dst_hs, dst_ld, col0, ring);
  return hipGetLastError();
}

// cos/sin of angle th >= 0: reduced modulo 2 pi in fp64 (at th < 2^20 the
// reduction error is below 1e-9 rad), then fp32 sincos on [-pi, pi].
__device__ __forceinline__ float2 cos_sin_reduced(double th) {
  const double q = rint(th * 0.15915494309189535);   // th / (2 pi)
  const float r = static_cast<float>(fma(-q, 6.283185307179586, th));
  float s, c;
  sincosf(r, &s, &c);
  return make_float2(c, s);
}

// Keys rebuilt from the transposed value cache (layers whose keys and values
// share one projection): K[m] = RoPE_m(gamma * V[m]).  A workgroup takes 64
// positions of one head and walks the frequency pairs 64 at a time: the
// value columns t and t + d/2 of its positions go through LDS (coalesced
// reads of the transposed rows), then each thread writes 8 consecutive key
// elements of one position and both halves.  The block's frequencies are
// computed once (fp64) and each angle p * f_t is reduced in fp64 before an
// fp32 sincos, so the pass stays bound by its memory traffic.
template <typename T>
__global__ __launch_bounds__(256) void k_rebuild_kernel(const T *vt, long long vt_hs, int vt_ld, int n_pos, int dh,
                                                        const T *gamma, double base, int n_rot, T *k, long long k_hs) {
  constexpr int NP = 64, NT = 64;
  __shared__ float tile[2][NT][NP + 1];   // [half][t][position]
  __shared__ double freq[NT];
  const int h = blockIdx.y, m0 = blockIdx.x * NP, half = dh >> 1;
  const T *v = vt + h * vt_hs;
  T *kh = k + h * k_hs;
  const int tid = threadIdx.x;
  for (int t0 = 0; t0 < half; t0 += NT) {
    if (tid < NT) freq[tid] = pow(base, -2.0 * static_cast<double>(t0 + tid) / static_cast<double>(dh));
    // columns t0.. t0+NT-1 and their partners, 64 positions each
    for (int e = tid; e < 2 * NT * NP; e += 256) {
      const int hf = e / (NT * NP), r = e % (NT * NP), t = r / NP, p = r % NP;
      const int m = m0 + p, d = t0 + t + hf * half;
      tile[hf][t][p] = (m < n_pos && t0 + t < half) ? to_f32<T>(v[static_cast<long long>(d) * vt_ld + m]) : 0.f;
    }
    __syncthreads();
    // thread: position p, 8 consecutive t of the block
    for (int e = tid; e < NP * (NT / 8); e += 256) {
      const int p = e / (NT / 8), tb = (e % (NT / 8)) * 8;
      const int m = m0 + p;
      if (m < n_pos && t0 + tb < half) {
        float lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = t0 + tb + j;
          float a = tile[0][tb + j][p] * to_f32<T>(gamma[t]);
          float b = tile[1][tb + j][p] * to_f32<T>(gamma[t + half]);
          if (t < n_rot) {
            const float2 cs = cos_sin_reduced(static_cast<double>(m) * freq[tb + j]);
            const float o0 = a * cs.x - b * cs.y, o1 = b * cs.x + a * cs.y;
            a = o0;
            b = o1;
          }
          lo[j] = a;
          hi[j] = b;
        }
        T *row = kh + static_cast<long long>(m) * dh;
        if constexpr (sizeof(T) == 2) {
          store8(row + t0 + tb, lo);
          store8(row + t0 + tb + half, hi);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            row[t0 + tb + j] = lo[j];
            row[t0 + tb + j + half] = hi[j];
          }
        }
      }
    }
    __syncthreads();
  }
}

// bf16 form for d_h = 512 (the global layers): a workgroup issues every
// 16-byte load of its 64 positions (512 value rows x 128 bytes) before it
// stores any to LDS, so it waits on memory once, then each thread writes
// 16-byte chunks of key rows.  Positions past n_pos in the last block are
// read as a clamped in-range column and not written.
constexpr int kRebuildDh = 512;
__global__ __launch_bounds__(256) void k_rebuild16_kernel(const bf16_t *vt, long long vt_hs, int vt_ld, int n_pos,
                                                          const bf16_t *gamma, double base, int n_rot, bf16_t *k,
                                                          long long k_hs) {
  constexpr int NP = 64, DH = kRebuildDh, HALF = DH / 2, PITCH = NP + 8;   // 16 bytes of padding per row
  __shared__ __attribute__((aligned(16))) bf16_t tile[DH][PITCH];          // [d][position]
  __shared__ double freq[HALF];
  const int h = blockIdx.y, m0 = blockIdx.x * NP, tid = threadIdx.x;
  const bf16_t *v = vt + h * vt_hs;
  // 512 rows x 8 chunks of 8 positions: 16 loads per thread, all in flight at once
  uint4 r[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = tid + 256 * i, d = c >> 3, p0 = (c & 7) * 8;
    const int m = m0 + p0 < n_pos ? m0 + p0 : 0;   // n_pos, m0 and p0 are multiples of 8 or clamped in range
    r[i] = *reinterpret_cast<const uint4 *>(v + static_cast<long long>(d) * vt_ld + m);
  }
  for (int t = tid; t < HALF; t += 256)
    freq[t] = t < n_rot ? pow(base, -2.0 * static_cast<double>(t) / static_cast<double>(DH)) : 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = tid + 256 * i, d = c >> 3, p0 = (c & 7) * 8;
    *reinterpret_cast<uint4 *>(&tile[d][p0]) = r[i];
  }
  __syncthreads();
  // thread: one position, 8 consecutive t of a 64-wide t block, both halves
  bf16_t *kh = k + h * k_hs;
  for (int e = tid; e < NP * (HALF / 8); e += 256) {
    const int p = e & (NP - 1), tb = (e >> 6) * 8;
    const int m = m0 + p;
    if (m >= n_pos) continue;
    float lo[8], hi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = tb + j;
      float a = bf16_to_f32(tile[t][p]) * bf16_to_f32(gamma[t]);
      float b = bf16_to_f32(tile[t + HALF][p]) * bf16_to_f32(gamma[t + HALF]);
      if (t < n_rot) {
        const float2 cs = cos_sin_reduced(static_cast<double>(m) * freq[t]);
        const float o0 = a * cs.x - b * cs.y, o1 = b * cs.x + a * cs.y;
        a = o0;
        b = o1;
      }
      lo[j] = a;
      hi[j] = b;
    }
    bf16_t *row = kh + static_cast<long long>(m) * DH;
    store8(row + tb, lo);
    store8(row + tb + HALF, hi);
  }
}

// Workgroups that fill the chip once: one per CU where the double-buffered
// 512-wide tiles take most of the LDS, two per CU otherwise.
int attn_target_workgroups(int dtype, int dh) {
  const int lds = 2 * (kBKV * dh + dh * kBKV) * (dtype == DG_BF16 ? 2 : 4);   // two K + two V^T tiles
  return lds > 80 * 1024 ? DG_ATTN_TGT_LARGE : DG_ATTN_TGT_SMALL;
}

int attn_block_rows(int dtype, int dh) {
  if (dtype == DG_BF16) {
    switch (dh) {
      case 64: return AttnCfg<bf16_t, 64>::BQ;
      case 128: return AttnCfg<bf16_t, 128>::BQ;
      case 256: return SoloCfg<256>::on ? SoloCfg<256>::BQ : AttnCfg<bf16_t, 256>::BQ;
      case 512: return SoloCfg<512>::on ? SoloCfg<512>::BQ : AttnCfg<bf16_t, 512>::BQ;
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

hipError_t launch_rope_table(int pos0, int n_tok, int dh, double base, int n_rot, float2 *tab, hipStream_t s) {
  if (n_tok <= 0) return hipSuccess;
  const long long n = static_cast<long long>(n_tok) * (dh / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, pos0, n_tok,
                     dh, base, n_rot, tab);
  return hipGetLastError();
}

hipError_t launch_k_rebuild(int dtype, const void *vt, long long vt_hs, int vt_ld, int n_pos, int Hkv, int dh,
                            const void *k_norm, double base, int n_rot, void *k, long long k_hs, hipStream_t s) {
  if (n_pos <= 0) return hipSuccess;
  if (dh % 16) return hipErrorInvalidValue;   // 8-element stores in each half
  const dim3 grid((n_pos + 63) / 64, Hkv);
  if (dtype == DG_BF16 && dh == kRebuildDh && vt_ld % 8 == 0 && vt_hs % 8 == 0) {
    hipLaunchKernelGGL(k_rebuild16_kernel, grid, dim3(256), 0, s, static_cast<const bf16_t *>(vt), vt_hs, vt_ld, n_pos,
                       static_cast<const bf16_t *>(k_norm), base, n_rot, static_cast<bf16_t *>(k), k_hs);
    return hipGetLastError();
  }
  if (dtype == DG_BF16)
    hipLaunchKernelGGL(k_rebuild_kernel<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t *>(vt), vt_hs, vt_ld,
                       n_pos, dh, static_cast<const bf16_t *>(k_norm), base, n_rot, static_cast<bf16_t *>(k), k_hs);
  else
    hipLaunchKernelGGL(k_rebuild_kernel<float>, grid, dim3(256), 0, s, static_cast<const float *>(vt), vt_hs, vt_ld,
                       n_pos, dh, static_cast<const float *>(k_norm), base, n_rot, static_cast<float *>(k), k_hs);
  return hipGetLastError();
}

hipError_t launch_norm_rope(const NormRopeArgs &a, int dtype, hipStream_t s) {
  if (a.n_tok <= 0) return hipSuccess;
  if (!a.rope_tab || !a.vt_dst) return hipErrorInvalidValue;
  const bool fused = DG_NORM_ROPE_VT && dtype == DG_BF16 && (a.dh == 256 || a.dh == 512) && a.ld % 8 == 0 &&
                     a.v_off % 8 == 0 && reinterpret_cast<uintptr_t>(a.qkv) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(a.vt_dst) % 16 == 0 && a.vt_col0 % 8 == 0 && a.vt_ld % 8 == 0 &&
                     a.vt_hs % 8 == 0 && a.vt_ring % 8 == 0;
  if (fused) {
    const int tj = a.dh == 256 ? 64 : 32;   // V tile tokens (32 * RH)
    const int n_vt = a.Hkv * ((a.n_tok + tj - 1) / tj);
    const dim3 grid(n_vt + a.n_tok * ((a.Hq + a.Hkv + 3) / 4));
    if (a.dh == 256) hipLaunchKernelGGL((norm_rope_vt_kernel<4, 2>), grid, dim3(256), 0, s, a, n_vt);
    else hipLaunchKernelGGL((norm_rope_vt_kernel<8, 1>), grid, dim3(256), 0, s, a, n_vt);
    return hipGetLastError();
  }
  if (!a.v_dst) return hipErrorInvalidValue;
  const dim3 grid(a.n_tok, (a.Hq + 2 * a.Hkv + 3) / 4);
  if (dtype == DG_BF16) hipLaunchKernelGGL(norm_rope_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(norm_rope_kernel<float>, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_v_transpose(dtype, a.v_dst, a.n_tok, a.Hkv, a.dh, a.vt_dst, a.vt_hs, a.vt_ld, a.vt_col0, s,
                            a.vt_ring);
}

}  // namespace dg
