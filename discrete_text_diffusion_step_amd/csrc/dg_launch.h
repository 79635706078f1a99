// Host-side launcher interface between the C ABI layer and the kernels.
#pragma once
#include "dg_common.h"

namespace dg {

// Wave64 all-reductions in the VALU, no LDS round trips: DPP quad_perm
// [1,0,3,2] and [2,3,0,1] pair lanes l ^ 1 and l ^ 2; row_half_mirror pairs
// the two quads of each 8 lanes and row_mirror the two 8s of each 16 (all
// lanes of a group hold the same value by then, so any pairing across the
// halves will do); gfx950's row swaps (v_permlane16_swap /
// v_permlane32_swap of a register with itself) pair lanes l ^ 16 and l ^ 32.
// Every lane ends with the same value.  Callers run with the whole wave
// active.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_allreduce(float v, Op op) {
  v = op(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_f32<0x141>(v));   // row_half_mirror
  v = op(v, dpp_f32<0x140>(v));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// the same on 32-bit integers (exact for any value)
template <typename Op>
__device__ __forceinline__ int wave_allreduce_i(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  v = op(static_cast<int>(a[0]), static_cast<int>(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  return op(static_cast<int>(b[0]), static_cast<int>(b[1]));
}
__device__ __forceinline__ float wave_allsum(float v) {
  return wave_allreduce(v, [](float x, float y) { return x + y; });
}
__device__ __forceinline__ float wave_allmax(float v) {
  return wave_allreduce(v, [](float x, float y) { return fmaxf(x, y); });
}

}  // namespace dg

namespace dg {

struct NormRopeArgs {
  void *qkv;                 // [n_tok][ld] raw projections (q | k | v)
  long long ld;
  int n_tok, Hq, Hkv, dh;
  int q_off, k_off, v_off;   // column offsets of q, k, v (v_off = k_off when K/V are shared)
  const void *q_norm, *k_norm;
  void *k_dst;               // [Hkv][..][dh], row k_row0 + j
  long long k_head_stride;   // elements between heads
  int k_row0;
  int k_ring = 0;            // > 0: row r of the cache lives at r mod k_ring
  void *v_dst;               // [Hkv][n_tok][dh], row j
  long long v_head_stride;
  int pos0;
  double rope_base;
  int n_rot;                 // frequencies kept (the rest are zero)
  float eps, sqrt_dh;
  int v_unit_rms;
  // [n_tok][dh/2] (cos, sin) of the rotation angles (launch_rope_table)
  const float2 *rope_tab = nullptr;
  // the transposed value cache vt[h][d][col] (vt_hs elements between heads,
  // row pitch vt_ld): token j goes to column vt_col0 + j (mod vt_ring when
  // vt_ring > 0).  launch_norm_rope writes the V heads there, straight from
  // the projection where the shapes allow it, else through v_dst.
  void *vt_dst = nullptr;
  long long vt_hs = 0;
  int vt_ld = 0, vt_col0 = 0, vt_ring = 0;
};

struct AttnArgs {
  const void *q;             // row (token j, head h) at q + j*q_ld + h*dh
  long long q_ld;
  const void *k_cache;       // [Hkv][cap][dh]: keys, position m at row m
  long long cache_hs;
  const void *v_cache;       // [Hkv][dh][cap]: values transposed, position m at column m
  long long vcache_hs;
  int vcache_ld;
  int n_tok, Hq, Hkv, n_rep;
  int kv_len, key_lo;
  int causal, sliding, window;
  int n_split;
  int ring;                  // > 0: cache position m lives at row / column m mod ring
  float *o_part;             // [n_split][Hkv*R][dh]
  float *ml_part;            // [n_split][Hkv*R][2]
  void *out;                 // row (token j, head h) at out + j*out_ld + h*dh
  long long out_ld;
};

struct SampleArgs {
  const void *logits;
  int logits_bf16;
  int n_pos, vocab, n_chunks;
  float inv_t, tau;
  int final_step;
  uint32_t step, canvas_idx, key0, key1;
  float *part;          // [n_pos][n_chunks][4]: m, Z, S, best value
  int *part_idx;        // [n_pos][n_chunks]: argmax index
  int *part_nf;         // [n_pos][n_chunks]: non-finite logits in the slice
  int32_t *tokens;
  uint8_t *commit;
  float *entropy;
  float *rowstats;      // optional [n_pos][2]
  int32_t *n_renoised;
  int commit_rule;      // 0: H < tau per position, 1: sorted cumulative bound
  int token_rule;       // 0: argmax, 1: Gumbel-max draw
  int32_t *pred;        // optional [n_pos] proposals in/out
  int32_t *n_changed;   // optional [1] (with pred)
  int32_t *n_nonfinite; // optional [1]: rows holding a NaN or +-inf logit
};
// rows the sorted cumulative commit rule handles (one workgroup, LDS)
constexpr int kSortedMaxRows = 4096;

// q heads normed and rotated in place, k heads to the key cache, v heads to
// the transposed value cache (vt_dst; v_dst is the row buffer of the
// two-pass form taken when the fused one does not apply)
hipError_t launch_norm_rope(const NormRopeArgs &a, int dtype, hipStream_t s);
// tab[j][t] = (cos, sin) of angle (pos0 + j) * base^(-2t/dh), fp64 angle; t >= n_rot: (1, 0)
hipError_t launch_rope_table(int pos0, int n_tok, int dh, double base, int n_rot, float2 *tab, hipStream_t s);
hipError_t launch_attention(const AttnArgs &a, int dtype, int dh, hipStream_t s);
// k[h][m][:] = RoPE_m(k_norm * V[h][m][:]) for positions m < n_pos, read from
// the transposed value cache vt[h][d][m] (vt_hs elements between heads, row
// pitch vt_ld); split-half rotation of the first n_rot frequencies, angles in
// fp64 as in launch_rope_table.
hipError_t launch_k_rebuild(int dtype, const void *vt, long long vt_hs, int vt_ld, int n_pos, int Hkv, int dh,
                            const void *k_norm, double base, int n_rot, void *k, long long k_hs, hipStream_t s);
// dst[h][d][col0 + j] = src[h][j][d] for j < n (values to the transposed layout);
// ring > 0: column (col0 + j) mod ring
hipError_t launch_v_transpose(int dtype, const void *src, int n, int Hkv, int dh, void *dst, long long dst_hs,
                              int dst_ld, int col0, hipStream_t s, int ring = 0);
// 1: the V heads go from the projection to the transposed cache inside the
// norm/RoPE launch (0: through the row buffer and a transpose launch)
#ifndef DG_NORM_ROPE_VT
#define DG_NORM_ROPE_VT 1
#endif
// Workgroups the split-KV attention grid aims for: kernels whose LDS tiles
// exceed 80 KB run one workgroup per CU, the others two.
#ifndef DG_ATTN_PAIR
#define DG_ATTN_PAIR 1
#endif
// bf16 attention in the solo form (each wave owns whole 16-query tiles over
// the full head dimension), by head dimension: bit 0 for d_h 256, bit 1 for
// d_h 512 (the pair form otherwise); QT query tiles per wave, NW waves per
// workgroup
#ifndef DG_ATTN_SOLO
#define DG_ATTN_SOLO 1
#endif
#ifndef DG_SOLO256_QT
#define DG_SOLO256_QT 1
#endif
#ifndef DG_SOLO256_NW
#define DG_SOLO256_NW 8
#endif
#ifndef DG_SOLO512_QT
#define DG_SOLO512_QT 1
#endif
#ifndef DG_SOLO512_NW
#define DG_SOLO512_NW 8
#endif
#ifndef DG_SOLO_VDEPTH
#define DG_SOLO_VDEPTH 8
#endif
// 1: the pair form waits for the V^T tile before the score exchange's
// barrier (two barriers per tile); 0: a third barrier before P V
#ifndef DG_PAIR_V_AT_EXCHANGE
#define DG_PAIR_V_AT_EXCHANGE 1
#endif
// 1: the softmax's column maximum by VALU row swaps (0: by ds_bpermute)
#ifndef DG_ATTN_PERMLANE
#define DG_ATTN_PERMLANE 1
#endif
#ifndef DG_SOLO_NBUF
#define DG_SOLO_NBUF 2
#endif
#ifndef DG_ATTN_TGT_SMALL
#define DG_ATTN_TGT_SMALL 256
#endif
#ifndef DG_ATTN_TGT_LARGE
#define DG_ATTN_TGT_LARGE 256
#endif
int attn_target_workgroups(int dtype, int dh);
int attn_block_rows(int dtype, int dh);
// logits: n_parts partial sums [n_parts][n_tok][E], added in order
hipError_t launch_router_topk(const float *logits, int n_parts, int n_tok, int E, int k, float scale, int32_t *idx,
                              float *w, hipStream_t s);
hipError_t launch_moe_permute(const int32_t *idx, const float *w, int n_tok, int k, int E, int chunk, int *g_off,
                              int *row_token, float *row_weight, int *pair_row, hipStream_t s);
hipError_t launch_moe_combine(int dtype, void *x, const float *Y, const int *pair_row, int n_tok, int k, int D,
                              float layer_scalar, hipStream_t s);
hipError_t launch_sampler(const SampleArgs &a, hipStream_t s);
hipError_t launch_canvas_noise(int n_pos, int vocab, uint32_t key0, uint32_t key1, uint32_t canvas_idx,
                               int32_t *tokens, hipStream_t s);
hipError_t launch_probs(int dtype, const float *logits, const float *rowstats, int n_pos, int vocab, float inv_t,
                        void *P, hipStream_t s);
hipError_t launch_rmsnorm(int dtype, int n, int D, float eps, const void *x, const void *w, void *y,
                          hipStream_t s);
hipError_t launch_embed(int dtype, const int32_t *tokens, int n, int D, int vocab, const void *E, void *x,
                        hipStream_t s);
hipError_t launch_transpose(int dtype, int rows, int cols, const void *in, void *out, hipStream_t s);
// q[r][c] = E4M3(w[r][c] / scale[r]), scale[r] = max_c |w[r][c]| / 448
hipError_t launch_quantize_fp8(int dtype, const void *w, long long rows, int cols, uint8_t *q, float *scale,
                               hipStream_t s);

// Residual update + the next block's RMSNorm (rows up to residual_norm_max_width()).
int residual_norm_max_width();
hipError_t launch_reduce_add_rmsnorm(int dtype, const float *part, int splits, int n, int D, void *x, const void *w,
                                     float eps, void *h, hipStream_t s);
hipError_t launch_combine_rmsnorm(int dtype, void *x, const float *Y, const int *pair_row, int n, int k, int D,
                                  float layer_scalar, const void *w, float eps, void *h, hipStream_t s);

}  // namespace dg
