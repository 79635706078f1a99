// C ABI of libdgstep: argument validation, workspace layout and the order of
// kernel launches for one canvas denoising step and for a commit (encode).
// Every entry point validates on the host, then only enqueues work on the
// caller's stream.  No allocation, no host synchronisation.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "dg_launch.h"


using namespace dg;

namespace {

#define DG_TRY(expr)                         \
  do {                                       \
    const int st__ = (expr);                 \
    if (st__ != DG_OK) return st__;          \
  } while (0)
#define DG_HIP(expr)                                  \
  do {                                                \
    if ((expr) != hipSuccess) return DG_ERR_HIP;      \
  } while (0)

size_t esize(int dtype) { return dtype == DG_BF16 ? 2 : 4; }
bool dtype_ok(int dtype) { return dtype == DG_BF16 || dtype == DG_F32; }

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures.  Every block is 256-byte aligned.
struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *b) : base(static_cast<char *>(b)) {}
  template <typename T>
  T *take(size_t count) {
    off = (off + 255) & ~static_cast<size_t>(255);
    T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  void *bytes(size_t n) { return take<char>(n); }
};

thread_local dg_kernel_timer *g_timer = nullptr;

// Records the attached timer's events around one launch of kernel class `kt`.
struct TimedLaunch {
  dg_kernel_timer *t;
  hipStream_t s;
  int slot;
  TimedLaunch(int kt, hipStream_t st) : t(nullptr), s(st), slot(-1) {
    if (g_timer && g_timer->kernel == kt) {
      const int every = g_timer->every > 1 ? g_timer->every : 1;
      if (g_timer->seen++ % every == 0 && g_timer->count < g_timer->capacity) {
        t = g_timer;
        slot = t->count++;
        hipEventRecord(static_cast<hipEvent_t>(t->start[slot]), s);
      }
    }
  }
  ~TimedLaunch() {
    if (t) hipEventRecord(static_cast<hipEvent_t>(t->stop[slot]), s);
  }
};

// Streaming MFMA product (tile 16*mt x 16*nt; the four waves split k).
hipError_t sgemm(int dtype, const GemmArgs &a, int mode, int mt, int nt, hipStream_t s) {
  return dtype == DG_BF16 ? launch_gemm_stream<bf16_t>(a, mode, mt, nt, s)
                          : launch_gemm_stream<float>(a, mode, mt, nt, s);
}

hipError_t reduce(int dtype, const float *part, int splits, int M, int N, long long ldc, void *C, int mode,
                  hipStream_t s) {
  return dtype == DG_BF16 ? launch_splitk_reduce<bf16_t>(part, splits, M, N, ldc, C, mode, s)
                          : launch_splitk_reduce<float>(part, splits, M, N, ldc, C, mode, s);
}

GemmArgs dense_args(const void *A, long long lda, int M, int N, int K, void *C, long long ldc) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A;
  g.lda = lda;
  g.M = M;
  g.N = N;
  g.K = K;
  g.ldb = K;
  g.nseg = 1;
  g.seg_start[0] = 0;
  g.seg_start[1] = N;
  g.k_splits = 1;
  g.C = C;
  g.ldc = ldc;
  return g;
}

// Split count for a dense product so that the grid covers the chip: doubles
// while fewer than `target` workgroups would run and each split keeps at
// least 8 k steps of 32 (two per wave).
int choose_ksplit(int M, int N, int K, int bm, int bn, int target, int max_split) {
  const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  int ks = 1;
  while (tiles * ks < target && ks * 2 <= max_split && K % (32 * ks * 2) == 0 && K / (ks * 2) >= 256) ks *= 2;
  return ks;
}

// x (or C) <- dense product with split-K through fp32 partials when it pays.
hipError_t dense_product(int dt, GemmArgs g, int mode, float *part, int ks, hipStream_t s) {
  if (ks <= 1) return sgemm(dt, g, mode, DG_DENSE_MT, DG_DENSE_NT, s);
  void *C = g.C;
  const long long ldc = g.ldc;
  g.C = part;
  g.ldc = g.N;
  g.k_splits = ks;
  hipError_t e = sgemm(dt, g, EPI_PARTIAL_F32, DG_DENSE_MT, DG_DENSE_NT, s);
  if (e != hipSuccess) return e;
  return reduce(dt, part, ks, g.M, g.N, ldc, C, mode, s);
}

// The wide-tile bf16 kernel takes operands with 16-byte aligned rows, a depth
// that is a whole number of its k stages and byte offsets that fit 32 bits
// (A up to a_rows rows; each weight matrix N x K).
bool wide_ok(int dt, const GemmArgs &g, int cfg, long long a_rows) {
  if (dt != DG_BF16) return false;
  const int kst = wide_kstage(cfg);
  if (g.K % kst || g.lda % 8 || g.ldb % 8) return false;
  if (g.g_off && (g.K_x % kst || g.ldb_x % 8)) return false;
  const long long lim = 1LL << 31;
  if (a_rows * g.lda * 2 >= lim) return false;
  const long long nb = g.g_off ? (g.N > g.N_x ? g.N : g.N_x) : g.N;
  const long long ldb = g.g_off && g.ldb_x > g.ldb ? g.ldb_x : g.ldb;
  return nb * ldb * 2 < lim;
}

// Split count of a wide dense product: about one workgroup per compute unit
// (the 256-row tiles run one workgroup per CU), each split a whole number of
// k stages; returns the number of non-empty splits.
int wide_ksplit(const GemmArgs &g, int cfg, int target) {
  int tiles = ((g.M + wide_bm(cfg) - 1) / wide_bm(cfg)) * ((g.N + wide_bn(cfg) - 1) / wide_bn(cfg));
  if (tiles < 1) tiles = 1;
  int ks = target / tiles;   // whole rounds of workgroups: no straggler round
  const int kst = wide_kstage(cfg);
  const int steps = g.K / kst;
  if (ks > steps / 4) ks = steps / 4;   // at least four k stages per split
  if (ks < 1) ks = 1;
  if (g.K <= 0) return 1;
  const int kper = (g.K + ks - 1) / ks;
  const int kper_r = (kper + kst - 1) / kst * kst;
  return (g.K + kper_r - 1) / kper_r;
}

// Wide dense product, through fp32 partials when split.
hipError_t wide_product(GemmArgs g, int mode, int cfg, float *part, int ks, hipStream_t s) {
  if (ks <= 1) return launch_gemm_wide(g, mode, cfg, s);
  void *C = g.C;
  const long long ldc = g.ldc;
  g.C = part;
  g.ldc = g.N;
  g.k_splits = ks;
  hipError_t e = launch_gemm_wide(g, EPI_PARTIAL_F32, cfg, s);
  if (e != hipSuccess) return e;
  return launch_splitk_reduce<bf16_t>(part, ks, g.M, g.N, ldc, C, mode, s);
}

// ------------------------------------------------------------ attention

struct AttnPlan {
  int n, Ntot, Nq, Nk, Nv, R, n_split_max;
  bool qkv_wide, oproj_wide;   // 256-row wide-tile products (bf16)
  int qkv_ks, oproj_ks;        // their split-K counts (fp32 partials when > 1)
};

AttnPlan attn_plan(const dg_attn_cfg *c, int n) {
  AttnPlan p;
  p.n = n;
  p.Nq = c->n_q_heads * c->head_dim;
  p.Nk = c->n_kv_heads * c->head_dim;
  p.Nv = c->shared_kv ? 0 : p.Nk;
  p.Ntot = p.Nq + p.Nk + p.Nv;
  p.R = (c->n_q_heads / c->n_kv_heads) * n;
  const int bq = attn_block_rows(c->dtype, c->head_dim);
  const int blocks = c->n_kv_heads * ((p.R + bq - 1) / (bq > 0 ? bq : 1));
  const int target = attn_target_workgroups(c->dtype, c->head_dim);
  int ns = (target + blocks - 1) / (blocks > 0 ? blocks : 1);
  p.n_split_max = ns < 1 ? 1 : (ns > 16 ? 16 : ns);
  const GemmArgs gq = dense_args(nullptr, c->hidden, n, p.Ntot, c->hidden, nullptr, p.Ntot);
  p.qkv_wide = DG_PROJ_WIDE && wide_ok(c->dtype, gq, DG_PROJ_CFG, n);
  p.qkv_ks = p.qkv_wide ? wide_ksplit(gq, DG_PROJ_CFG, DG_PROJ_TARGET) : 1;
  const GemmArgs go = dense_args(nullptr, p.Nq, n, c->hidden, p.Nq, nullptr, c->hidden);
  p.oproj_wide = DG_PROJ_WIDE && wide_ok(c->dtype, go, WIDE_ROWS256_N128_OP, n);
  p.oproj_ks = p.oproj_wide ? wide_ksplit(go, WIDE_ROWS256_N128_OP, DG_PROJ_TARGET)
                            : choose_ksplit(n, c->hidden, p.Nq, 16 * DG_DENSE_MT, 16 * DG_DENSE_NT, 512, 8);
  return p;
}

struct AttnWs {
  void *h, *qkv, *v_rows, *o;
  float *o_part, *ml_part, *oproj_part, *qkv_part;
  float2 *rope_tab;
};

// A rotation table made once for every layer of one type at one position.
struct RopeTab {
  const float2 *tab = nullptr;
  int pos0 = -1;
};

// p: the projections over all rows; pa: the attention of one canvas
AttnWs attn_carve(const dg_attn_cfg *c, const AttnPlan &p, const AttnPlan &pa, Carve &cv) {
  const size_t es = esize(c->dtype);
  AttnWs w;
  const size_t n = static_cast<size_t>(p.n);
  w.h = cv.bytes(n * c->hidden * es);
  w.qkv = cv.bytes(n * p.Ntot * es);
  w.v_rows = cv.bytes(n * p.Nk * es);   // per canvas [Hkv][C][dh]: V rows of the two-launch norm/RoPE form
  w.o = cv.bytes(n * p.Nq * es);
  const size_t rows = static_cast<size_t>(c->n_kv_heads) * pa.R;
  if (pa.n_split_max > 1) {
    w.o_part = cv.take<float>(pa.n_split_max * rows * c->head_dim);
    w.ml_part = cv.take<float>(pa.n_split_max * rows * 2);
  } else {
    w.o_part = w.ml_part = nullptr;
  }
  w.oproj_part = p.oproj_ks > 1 ? cv.take<float>(p.oproj_ks * n * c->hidden) : nullptr;
  w.qkv_part = p.qkv_ks > 1 ? cv.take<float>(p.qkv_ks * n * p.Ntot) : nullptr;
  w.rope_tab = cv.take<float2>(n * (c->head_dim / 2));
  return w;
}

int check_attn_cfg(const dg_attn_cfg *c) {
  if (!c) return DG_ERR_NULL;
  if (!dtype_ok(c->dtype)) return DG_ERR_DTYPE;
  if (c->hidden <= 0 || c->hidden % 64 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->n_q_heads % c->n_kv_heads || c->head_dim <= 0)
    return DG_ERR_SHAPE;
  if ((c->n_q_heads * c->head_dim) % 64) return DG_ERR_SHAPE;
  // the fused Q|K|V product tiles columns by 128: every segment must fill whole tiles
  if ((c->n_q_heads * c->head_dim) % 128 || (c->n_kv_heads * c->head_dim) % 128) return DG_ERR_UNSUPPORTED;
  if (attn_block_rows(c->dtype, c->head_dim) == 0) return DG_ERR_UNSUPPORTED;
  if (c->layer_type != 0 && c->layer_type != 1) return DG_ERR_SHAPE;
  if (c->layer_type == 0 && c->window <= 0) return DG_ERR_SHAPE;
  if (!(c->rope_base > 0.f) || !(c->rotary_factor >= 0.f && c->rotary_factor <= 1.f)) return DG_ERR_SHAPE;
  if (!(c->rms_eps >= 0.f)) return DG_ERR_SHAPE;
  return DG_OK;
}

// Inside a step the kernel that finishes a residual update also writes the
// next block's pre-norm activations: h = rms(x, w, eps) into `h` (null: none).
struct NextNorm {
  void *h = nullptr;
  const void *w = nullptr;
  float eps = 0.f;
};

bool fused_norm_ok(int D) { return D <= residual_norm_max_width() && D % 8 == 0; }
int rope_rot(const dg_attn_cfg *c) {
  const double rf = c->layer_type == 1 ? c->rotary_factor : 1.0;
  return static_cast<int>(floor(rf * (c->head_dim / 2) + 0.5));
}

// x <- x + Attention(x) for B canvases of C rows each (x holds them back to
// back), canvas b attending over its own cache kvs[b].  The projections run
// over all B*C rows at once; norm/RoPE, the cache writes and attention run
// per canvas.  h_in, when given, already holds rms(x, w_in_norm); rts[b]
// (optional) is canvas b's rotation table.
int attn_impl(const dg_attn_cfg *c, const dg_attn_w *w, dg_kv_layer *const *kvs, int B, int C, int causal,
              void *x, Carve &cv, hipStream_t s, const void *h_in, NextNorm next, const RopeTab *rts) {
  const int n = B * C;
  const AttnPlan p = attn_plan(c, n);
  const AttnPlan pa = B == 1 ? p : attn_plan(c, C);
  const AttnWs ws = attn_carve(c, p, pa, cv);
  const int dt = c->dtype;
  const int D = c->hidden, dh = c->head_dim, Hq = c->n_q_heads, Hkv = c->n_kv_heads;

  const void *h = h_in;
  if (!h) {
    DG_HIP(launch_rmsnorm(dt, n, D, c->rms_eps, x, w->w_in_norm, ws.h, s));
    h = ws.h;
  }

  GemmArgs g = dense_args(h, D, n, p.Ntot, D, ws.qkv, p.Ntot);
  g.nseg = c->shared_kv ? 2 : 3;
  g.seg_start[0] = 0;
  g.seg_start[1] = p.Nq;
  g.seg_start[2] = p.Nq + p.Nk;
  g.seg_start[3] = p.Ntot;
  g.seg_B0[0] = w->w_q;
  g.seg_B0[1] = w->w_k;
  g.seg_B0[2] = w->w_v;
  g.seg_start[g.nseg] = p.Ntot;
  {
    TimedLaunch tl(DG_KT_QKV, s);
    if (p.qkv_wide) {
      DG_HIP(wide_product(g, EPI_STORE, DG_PROJ_CFG, ws.qkv_part, p.qkv_ks, s));
    } else {
      DG_HIP(sgemm(dt, g, EPI_STORE, DG_DENSE_MT, DG_DENSE_NT, s));
    }
  }

  for (int b = 0; b < B; ++b) {
    dg_kv_layer *kv = kvs[b];
    const int P = kv->kv_len;
    void *qkv_b = static_cast<char *>(ws.qkv) + static_cast<size_t>(b) * C * p.Ntot * esize(dt);
    void *vrows_b = static_cast<char *>(ws.v_rows) + static_cast<size_t>(b) * C * p.Nk * esize(dt);
    NormRopeArgs nr;
    nr.qkv = qkv_b;
    nr.ld = p.Ntot;
    nr.n_tok = C;
    nr.Hq = Hq;
    nr.Hkv = Hkv;
    nr.dh = dh;
    nr.q_off = 0;
    nr.k_off = p.Nq;
    nr.v_off = c->shared_kv ? p.Nq : p.Nq + p.Nk;
    nr.q_norm = w->q_norm;
    nr.k_norm = w->k_norm;
    // This call's K rows go to the cache at rows [P, P + C), its V rows
    // transposed into cache columns [P, P + C).  Decode uses those rows as
    // scratch (kv_len stays P); encode keeps them and advances kv_len.
    nr.k_dst = kv->k;
    nr.k_head_stride = static_cast<long long>(kv->capacity) * dh;
    nr.k_row0 = P;
    nr.k_ring = kv->ring ? kv->capacity : 0;
    nr.v_dst = vrows_b;
    nr.v_head_stride = static_cast<long long>(C) * dh;
    const long long vt_cache_hs = static_cast<long long>(dh) * kv->capacity;
    nr.vt_dst = kv->v;
    nr.vt_hs = vt_cache_hs;
    nr.vt_ld = kv->capacity;
    nr.vt_col0 = P;
    nr.vt_ring = kv->ring ? kv->capacity : 0;
    nr.pos0 = P;
    nr.rope_base = c->rope_base;
    nr.n_rot = rope_rot(c);
    nr.eps = c->rms_eps;
    nr.sqrt_dh = static_cast<float>(sqrt(static_cast<double>(dh)));
    nr.v_unit_rms = c->v_unit_rms;
    if (kv->v_only)   // the committed keys, rebuilt from the committed values into the k scratch
      DG_HIP(launch_k_rebuild(dt, kv->v, static_cast<long long>(dh) * kv->capacity, kv->capacity, P, Hkv, dh,
                              w->k_norm, c->rope_base, rope_rot(c), kv->k, static_cast<long long>(kv->capacity) * dh,
                              s));
    if (rts && rts[b].tab && rts[b].pos0 == P) {
      nr.rope_tab = rts[b].tab;
    } else {
      float2 *tab = ws.rope_tab + static_cast<size_t>(b) * C * (dh / 2);
      DG_HIP(launch_rope_table(P, C, dh, c->rope_base, rope_rot(c), tab, s));
      nr.rope_tab = tab;
    }
    DG_HIP(launch_norm_rope(nr, dt, s));

    AttnArgs at;
    at.q = qkv_b;
    at.q_ld = p.Ntot;
    at.k_cache = kv->k;
    at.cache_hs = static_cast<long long>(kv->capacity) * dh;
    at.v_cache = kv->v;
    at.vcache_hs = vt_cache_hs;
    at.vcache_ld = kv->capacity;
    at.n_tok = C;
    at.Hq = Hq;
    at.Hkv = Hkv;
    at.n_rep = Hq / Hkv;
    at.kv_len = P;
    at.ring = kv->ring ? kv->capacity : 0;
    at.sliding = c->layer_type == 0;
    at.window = c->window;
    at.key_lo = (at.sliding && !causal) ? (P > c->window ? P - c->window : 0) : 0;
    at.causal = causal;
    // split the keys so the grid covers the chip, at least 64 keys per slice
    const int n_keys = P + C - at.key_lo;
    int ns = pa.n_split_max;
    const int max_by_keys = (n_keys + 63) / 64;
    if (ns > max_by_keys) ns = max_by_keys;
    if (ns < 1) ns = 1;
    at.n_split = ns;
    at.o_part = ws.o_part;
    at.ml_part = ws.ml_part;
    at.out = static_cast<char *>(ws.o) + static_cast<size_t>(b) * C * p.Nq * esize(dt);
    at.out_ld = p.Nq;
    {
      TimedLaunch tl(DG_KT_ATTN, s);
      DG_HIP(launch_attention(at, dt, dh, s));
    }
  }

  // x += o W_o^T
  {
    GemmArgs o = dense_args(ws.o, p.Nq, n, D, p.Nq, x, D);
    o.seg_B0[0] = w->w_o;
    TimedLaunch tl(DG_KT_OPROJ, s);
    if (next.h && p.oproj_wide && p.oproj_ks > 1 && fused_norm_ok(D)) {
      // split-K partials, then one pass: residual add + the MoE block's pre-norm
      o.C = ws.oproj_part;
      o.ldc = D;
      o.k_splits = p.oproj_ks;
      DG_HIP(launch_gemm_wide(o, EPI_PARTIAL_F32, WIDE_ROWS256_N128_OP, s));
      DG_HIP(launch_reduce_add_rmsnorm(dt, ws.oproj_part, p.oproj_ks, n, D, x, next.w, next.eps, next.h, s));
      next.h = nullptr;
    } else if (p.oproj_wide) {
      DG_HIP(wide_product(o, EPI_ADD, WIDE_ROWS256_N128_OP, ws.oproj_part, p.oproj_ks, s));
    } else {
      DG_HIP(dense_product(dt, o, EPI_ADD, ws.oproj_part, p.oproj_ks, s));
    }
  }
  if (next.h) DG_HIP(launch_rmsnorm(dt, n, D, next.eps, x, next.w, next.h, s));
  if (causal)
    for (int b = 0; b < B; ++b) kvs[b]->kv_len += C;
  return DG_OK;
}

int attn_impl(const dg_attn_cfg *c, const dg_attn_w *w, dg_kv_layer *kv, int n, int causal, void *x, Carve &cv,
              hipStream_t s, const void *h_in = nullptr, NextNorm next = NextNorm(), RopeTab rt = RopeTab()) {
  dg_kv_layer *k1[1] = {kv};
  return attn_impl(c, w, k1, 1, n, causal, x, cv, s, h_in, next, &rt);
}

// Room for this call's rows at positions [kv_len, kv_len + n): a plain
// cache needs kv_len + n <= capacity; a ring (sliding layers) needs the
// window and the new rows to fit at once.
int check_kv_room(const dg_attn_cfg *c, const dg_kv_layer *kv, int n) {
  if (kv->ring != 0 && kv->ring != 1) return DG_ERR_SHAPE;
  if (kv->v_only != 0 && kv->v_only != 1) return DG_ERR_SHAPE;
  // keys rebuilt from values: only where K = RoPE(k_norm * V) holds
  if (kv->v_only && (kv->ring || c->layer_type != 1 || !c->shared_kv || !c->v_unit_rms)) return DG_ERR_UNSUPPORTED;
  if (kv->ring) {
    if (c->layer_type != 0 || c->window <= 0 || kv->capacity % 32) return DG_ERR_UNSUPPORTED;
    if (kv->capacity < c->window + n) return DG_ERR_CAPACITY;
    return DG_OK;
  }
  if (kv->kv_len > kv->capacity) return DG_ERR_SHAPE;
  if (kv->kv_len + n > kv->capacity) return DG_ERR_CAPACITY;   // this call's rows sit at [kv_len, kv_len + n)
  return DG_OK;
}

int check_attn_call(const dg_attn_cfg *c, const dg_attn_w *w, const dg_kv_layer *kv, int n, int causal,
                    const void *x) {
  DG_TRY(check_attn_cfg(c));
  if (!w || !kv || !x) return DG_ERR_NULL;
  if (!w->w_in_norm || !w->w_q || !w->w_k || !w->w_o || !w->q_norm || !w->k_norm) return DG_ERR_NULL;
  if (!c->shared_kv && !w->w_v) return DG_ERR_NULL;
  if (n < 0 || kv->kv_len < 0 || kv->capacity < 0) return DG_ERR_SHAPE;
  if (kv->capacity % 8) return DG_ERR_SHAPE;
  if (n > 0 && (!kv->k || !kv->v)) return DG_ERR_NULL;
  if (causal != 0 && causal != 1) return DG_ERR_SHAPE;
  DG_TRY(check_kv_room(c, kv, n));
  return DG_OK;
}

size_t attn_ws_bytes(const dg_attn_cfg *c, int n, int C = 0) {
  Carve cv(nullptr);
  const AttnPlan p = attn_plan(c, n);
  attn_carve(c, p, C > 0 && C != n ? attn_plan(c, C) : p, cv);
  return cv.off + 256;
}

// ------------------------------------------------------------------ MoE

struct MoeWs {
  void *h;
  float *rl, *tw;
  int32_t *idx;
  int *g_off, *row_token, *pair_row;
  float *row_weight, *Y, *rpart;
  void *H;
};

// bf16 router logits with whole 64-deep stages: one 16 x 16 tile per
// workgroup over the full depth (no split, no reduce); otherwise split-K.
bool router_small_tiles(const dg_moe_cfg *c) { return c->dtype == DG_BF16 && c->hidden % 64 == 0; }

int router_ksplit(const dg_moe_cfg *c, int n) {
  if (router_small_tiles(c)) {
    int ks = DG_ROUTER_KS;
    while (ks > 1 && c->hidden % (64 * ks)) ks >>= 1;
    return ks;
  }
  return choose_ksplit(n, c->n_experts, c->hidden, 16 * DG_DENSE_MT, 16 * DG_DENSE_NT, 256, 16);
}

MoeWs moe_carve(const dg_moe_cfg *c, int n, Carve &cv) {
  const size_t es = esize(c->dtype);
  const size_t rows = static_cast<size_t>(n) * (c->top_k + 1);
  const int fmax = c->ffn > c->shared_ffn ? c->ffn : c->shared_ffn;
  MoeWs w;
  w.h = cv.bytes(static_cast<size_t>(n) * c->hidden * es);
  w.rl = cv.take<float>(static_cast<size_t>(n) * c->n_experts);
  w.idx = cv.take<int32_t>(static_cast<size_t>(n) * c->top_k);
  w.tw = cv.take<float>(static_cast<size_t>(n) * c->top_k);
  w.g_off = cv.take<int>(c->n_experts + 2 + n / 16);   // shared-expert chunks of >= 16 rows
  w.row_token = cv.take<int>(rows);
  w.row_weight = cv.take<float>(rows);
  w.pair_row = cv.take<int>(static_cast<size_t>(n) * c->top_k);
  w.H = cv.bytes(rows * fmax * es);
  w.Y = cv.take<float>(rows * c->hidden);
  w.rpart = cv.take<float>(static_cast<size_t>(router_ksplit(c, n)) * n * c->n_experts);
  return w;
}

int check_moe_cfg(const dg_moe_cfg *c) {
  if (!c) return DG_ERR_NULL;
  if (!dtype_ok(c->dtype)) return DG_ERR_DTYPE;
  if (c->hidden <= 0 || c->hidden % 64 || c->ffn <= 0 || c->ffn % 64 || c->shared_ffn <= 0 ||
      c->shared_ffn % 64)
    return DG_ERR_SHAPE;
  if (c->n_experts <= 0 || c->n_experts > 256 || c->top_k <= 0 || c->top_k > 8 || c->top_k > c->n_experts)
    return DG_ERR_SHAPE;
  if (c->expert_format != DG_EXPERTS_DTYPE && c->expert_format != DG_EXPERTS_FP8_E4M3) return DG_ERR_UNSUPPORTED;
  if (c->expert_format == DG_EXPERTS_FP8_E4M3 && c->dtype != DG_BF16) return DG_ERR_UNSUPPORTED;
  return DG_OK;
}

// x <- layer_scalar * (x + MoE(x)).  h_in, when given, already holds
// rms(x, w_in_norm); next (optional) receives the next layer's pre-norm.
int moe_impl(const dg_moe_cfg *c, const dg_moe_w *w, int n, void *x, const float *rl_in, int32_t *idx_out,
             float *w_out, Carve &cv, hipStream_t s, const void *h_in = nullptr, NextNorm next = NextNorm()) {
  const MoeWs ws = moe_carve(c, n, cv);
  if (n == 0) return DG_OK;
  const int dt = c->dtype, D = c->hidden, E = c->n_experts, k = c->top_k, F = c->ffn, Fs = c->shared_ffn;
  const int fmax = F > Fs ? F : Fs;
  const void *h = h_in;
  if (!h) {
    DG_HIP(launch_rmsnorm(dt, n, D, c->rms_eps, x, w->w_in_norm, ws.h, s));
    h = ws.h;
  }
  const float *rl = rl_in;
  int n_rparts = 1;
  if (!rl) {
    GemmArgs g = dense_args(h, D, n, E, D, ws.rl, E);
    g.seg_B0[0] = w->w_router;
    if (router_small_tiles(c)) {
      // 16 x 16 tiles, split-K partials [ks][n][E]; the top-k pass adds them
      g.C = ws.rpart;
      g.ldc = E;
      g.k_splits = router_ksplit(c, n);
      DG_HIP(sgemm(dt, g, g.k_splits > 1 ? EPI_PARTIAL_F32 : EPI_STORE_F32, 1, 1, s));
      n_rparts = g.k_splits;
      rl = ws.rpart;
    } else {
      DG_HIP(dense_product(dt, g, EPI_STORE_F32, ws.rpart, router_ksplit(c, n), s));
      rl = ws.rl;
    }
  }
  int32_t *idx = idx_out ? idx_out : ws.idx;
  float *tw = w_out ? w_out : ws.tw;
  DG_HIP(launch_router_topk(rl, n_rparts, n, E, k, c->route_scale, idx, tw, s));
  const int rows_per_expert = (n * k + E - 1) / E;
  const int mtile = rows_per_expert > 48 ? 4 : DG_MOE_MT;   // 64-row tiles for long groups
  const bool fp8 = c->expert_format == DG_EXPERTS_FP8_E4M3;
  // long groups (several canvases, prompt commits): 256-row wide tiles, so
  // each expert's weights are streamed once for all of its rows
  const bool wide_l = !fp8 && dt == DG_BF16 && rows_per_expert > DG_WIDE_EXPERTS_L;
  // the shared expert's rows are cut into chunks of one row tile, so its
  // workgroups run side by side with the routed experts' instead of looping
  const int chunk = wide_l ? 256 : 16 * mtile;
  const int n_x = (n + chunk - 1) / chunk;
  DG_HIP(launch_moe_permute(idx, tw, n, k, E, chunk, ws.g_off, ws.row_token, ws.row_weight, ws.pair_row, s));

  // gate/up of every expert (group 0 = shared) with the SwiGLU epilogue
  GemmArgs gu;
  memset(&gu, 0, sizeof(gu));
  gu.A = h;
  gu.lda = D;
  gu.a_rows = ws.row_token;
  gu.seg_B0[0] = w->w_gate;
  gu.seg_B1[0] = w->w_up;
  gu.ldb = D;
  gu.b_gstride = static_cast<long long>(F) * D;
  gu.g_off = ws.g_off;
  gu.n_groups = E + n_x;
  gu.n_xgroups = n_x;
  gu.Bx0 = w->ws_gate;
  gu.Bx1 = w->ws_up;
  gu.N_x = Fs;
  gu.K_x = D;
  gu.ldb_x = D;
  gu.M = n * (k + 1);
  gu.N = F;
  gu.K = D;
  gu.k_splits = 1;
  gu.C = ws.H;
  gu.ldc = fmax;
  const long long moe_rows = static_cast<long long>(n) * (k + 1);
  gu.bs0 = w->s_gate;
  gu.bs1 = w->s_up;
  gu.bxs0 = w->ss_gate;
  gu.bxs1 = w->ss_up;
  // gate/up of short groups: the wide-tile kernel (activation stages shared
  // through LDS by four waves of 16 columns each); down: the carried-ring
  // kernel below, unless the wide form is asked for
  const bool wide_gu = !fp8 && DG_WIDE_EXPERTS_GU && rows_per_expert <= 48 && wide_ok(dt, gu, WIDE_EXPERT_GU, n);
  const bool wide = !fp8 && DG_WIDE_EXPERTS && rows_per_expert <= 48;
  {
    TimedLaunch tl(DG_KT_MOE_GATEUP, s);
    if (fp8) {
      hipError_t e = (DG_WIDE_F8_GU && mtile == DG_WMOE_MT) ? launch_gemm_wide_f8_gu(gu, s) : hipErrorNotSupported;
      if (e == hipErrorNotSupported) e = launch_gemm_f8_grouped(gu, EPI_SWIGLU, mtile, s);
      DG_HIP(e);
    }
    else if (wide_l && wide_ok(dt, gu, WIDE_EXPERT_GU_L, moe_rows))
      DG_HIP(launch_gemm_wide(gu, EPI_SWIGLU, WIDE_EXPERT_GU_L, s));
    else if (wide_gu) DG_HIP(launch_gemm_wide(gu, EPI_SWIGLU, WIDE_EXPERT_GU, s));
    else DG_HIP(sgemm(dt, gu, EPI_SWIGLU, mtile, DG_MOE_NT_GU, s));
  }

  // down projection, scaled by the routing weight of each row
  GemmArgs dn;
  memset(&dn, 0, sizeof(dn));
  dn.A = ws.H;
  dn.lda = fmax;
  dn.seg_B0[0] = w->w_down;
  dn.ldb = F;
  dn.b_gstride = static_cast<long long>(D) * F;
  dn.g_off = ws.g_off;
  dn.n_groups = E + n_x;
  dn.n_xgroups = n_x;
  dn.Bx0 = w->ws_down;
  dn.N_x = D;
  dn.K_x = Fs;
  dn.ldb_x = Fs;
  dn.M = n * (k + 1);
  dn.N = D;
  dn.K = F;
  dn.k_splits = 1;
  dn.C = ws.Y;
  dn.ldc = D;
  dn.rowscale = ws.row_weight;
  dn.bs0 = w->s_down;
  dn.bxs0 = w->ss_down;
  {
    TimedLaunch tl(DG_KT_MOE_DOWN, s);
    if (fp8) {
      hipError_t e = hipErrorNotSupported;
      if (DG_DN_RING) e = launch_gemm_down_ring(dn, mtile == DG_MOE_MT ? DG_DN_MT : mtile, true, s);
      if (e == hipErrorNotSupported) e = launch_gemm_f8_grouped(dn, EPI_ROWSCALE_F32, mtile, s);
      DG_HIP(e);
    }
    else if (wide_l && wide_ok(dt, dn, WIDE_EXPERT_DN_L, moe_rows))
      DG_HIP(launch_gemm_wide(dn, EPI_ROWSCALE_F32, WIDE_EXPERT_DN_L, s));
    else if (wide && wide_ok(dt, dn, WIDE_EXPERT_DN, moe_rows))
      DG_HIP(launch_gemm_wide(dn, EPI_ROWSCALE_F32, WIDE_EXPERT_DN, s));
    else {
      const int dmt = mtile == DG_MOE_MT ? DG_DN_MT : mtile;
      hipError_t e = hipErrorNotSupported;
      if (DG_DN_RING && dt == DG_BF16) e = launch_gemm_down_ring(dn, dmt, false, s);
      if (e == hipErrorNotSupported) e = sgemm(dt, dn, EPI_ROWSCALE_F32, dmt, DG_MOE_NT_DN, s);
      DG_HIP(e);
    }
  }

  if (next.h && fused_norm_ok(D)) {
    DG_HIP(launch_combine_rmsnorm(dt, x, ws.Y, ws.pair_row, n, k, D, c->layer_scalar, next.w, next.eps, next.h, s));
  } else {
    DG_HIP(launch_moe_combine(dt, x, ws.Y, ws.pair_row, n, k, D, c->layer_scalar, s));
    if (next.h) DG_HIP(launch_rmsnorm(dt, n, D, next.eps, x, next.w, next.h, s));
  }
  return DG_OK;
}

int check_moe_call(const dg_moe_cfg *c, const dg_moe_w *w, int n, const void *x, const float *rl_in) {
  DG_TRY(check_moe_cfg(c));
  if (!w || !x) return DG_ERR_NULL;
  if (!w->w_in_norm || !w->w_gate || !w->w_up || !w->w_down || !w->ws_gate || !w->ws_up || !w->ws_down)
    return DG_ERR_NULL;
  if (!rl_in && !w->w_router) return DG_ERR_NULL;
  if (c->expert_format == DG_EXPERTS_FP8_E4M3 &&
      (!w->s_gate || !w->s_up || !w->s_down || !w->ss_gate || !w->ss_up || !w->ss_down))
    return DG_ERR_NULL;
  if (n < 0) return DG_ERR_SHAPE;
  return DG_OK;
}

size_t moe_ws_bytes(const dg_moe_cfg *c, int n) {
  Carve cv(nullptr);
  moe_carve(c, n, cv);
  return cv.off + 256;
}

// -------------------------------------------------------------- sampler

int sample_chunks(int vocab) {
  int nc = 1;
  while (nc < 16 && vocab % (nc * 2 * 2048) == 0) nc *= 2;
  return nc;
}

struct SampleWs {
  float *part;
  int *part_idx, *part_nf;
};

SampleWs sample_carve(int n, int vocab, Carve &cv) {
  const int nc = sample_chunks(vocab);
  SampleWs w;
  w.part = cv.take<float>(static_cast<size_t>(n) * nc * 4);
  w.part_idx = cv.take<int>(static_cast<size_t>(n) * nc);
  w.part_nf = cv.take<int>(static_cast<size_t>(n) * nc);
  return w;
}

double temperature(const dg_sampler_cfg *c) {
  if (c->n_steps <= 1) return c->t_max;
  return static_cast<double>(c->t_max) +
         (static_cast<double>(c->t_min) - static_cast<double>(c->t_max)) * c->step / (c->n_steps - 1);
}

int check_sampler_cfg(const dg_sampler_cfg *c) {
  if (!c) return DG_ERR_NULL;
  if (c->vocab <= 0 || c->vocab % 8) return DG_ERR_SHAPE;
  if (!(c->t_max > 0.f) || !(c->t_min > 0.f) || c->n_steps < 1 || c->step < 0) return DG_ERR_SHAPE;
  if (!(temperature(c) > 0.0)) return DG_ERR_SHAPE;
  if (c->commit_rule != DG_COMMIT_ENTROPY && c->commit_rule != DG_COMMIT_SORTED_CUMULATIVE) return DG_ERR_UNSUPPORTED;
  if (c->token_rule != DG_TOKEN_ARGMAX && c->token_rule != DG_TOKEN_GUMBEL) return DG_ERR_UNSUPPORTED;
  return DG_OK;
}

SampleArgs sample_args(const dg_sampler_cfg *c, int n, int32_t *tok, uint8_t *commit, float *ent, float *rowstats,
                       int32_t *nre, int32_t *pred, int32_t *n_changed, int32_t *n_nonfinite) {
  SampleArgs a;
  memset(&a, 0, sizeof(a));
  a.n_pos = n;
  a.vocab = c->vocab;
  a.inv_t = static_cast<float>(1.0 / temperature(c));
  a.tau = c->tau;
  a.final_step = c->final_step;
  a.step = static_cast<uint32_t>(c->step);
  a.canvas_idx = c->canvas_idx;
  a.key0 = static_cast<uint32_t>(c->seed & 0xffffffffull);
  a.key1 = static_cast<uint32_t>(c->seed >> 32);
  a.tokens = tok;
  a.commit = commit;
  a.entropy = ent;
  a.rowstats = rowstats;
  a.n_renoised = nre;
  a.commit_rule = c->commit_rule;
  a.token_rule = c->token_rule;
  a.pred = pred;
  a.n_changed = pred ? n_changed : nullptr;
  a.n_nonfinite = n_nonfinite;
  return a;
}

int sample_impl(const dg_sampler_cfg *c, int n, const void *logits, int ldt, int32_t *tok, uint8_t *commit,
                float *ent, float *rowstats, int32_t *nre, int32_t *pred, int32_t *n_changed, int32_t *n_nonfinite,
                Carve &cv, hipStream_t s) {
  const SampleWs ws = sample_carve(n, c->vocab, cv);
  if (c->commit_rule == DG_COMMIT_SORTED_CUMULATIVE && n > kSortedMaxRows) return DG_ERR_SHAPE;
  SampleArgs a = sample_args(c, n, tok, commit, ent, rowstats, nre, pred, n_changed, n_nonfinite);
  a.logits = logits;
  a.logits_bf16 = ldt == DG_BF16;
  a.n_chunks = sample_chunks(c->vocab);
  a.part = ws.part;
  a.part_idx = ws.part_idx;
  a.part_nf = ws.part_nf;
  DG_HIP(launch_sampler(a, s));
  return DG_OK;
}

// ----------------------------------------------------- head, soft embedding

struct SoftPlan {
  bool wide;
  int ks;
};

// P.E contracts over the vocabulary: split-K over it, through fp32 partials.
SoftPlan softembed_plan(int dt, int n, int D, int V) {
  GemmArgs g = dense_args(nullptr, V, n, D, V, nullptr, D);
  SoftPlan p;
  p.wide = wide_ok(dt, g, DG_SOFT_CFG, n);
  p.ks = p.wide ? wide_ksplit(g, DG_SOFT_CFG, 256)
                : choose_ksplit(n, D, V, 16 * DG_DENSE_MT, 16 * DG_DENSE_NT, 512, 32);
  return p;
}

struct SoftWs {
  void *P;
  float *part;
};

SoftWs soft_carve(int n, int D, int V, int dtype, Carve &cv) {
  SoftWs w;
  w.P = cv.bytes(static_cast<size_t>(n) * V * esize(dtype));
  const int ks = softembed_plan(dtype, n, D, V).ks;
  w.part = ks > 1 ? cv.take<float>(static_cast<size_t>(ks) * n * D) : nullptr;
  return w;
}

// u = P E for n rows; the probabilities of canvas b (rows [b*C, (b+1)*C))
// are tempered with sc[b]'s temperature (B = 1, C = n: one canvas).
int soft_embed_impl(const dg_sampler_cfg *sc, int n, int D, int dt, const float *logits, const float *rowstats,
                    const void *embed_t, void *u, Carve &cv, hipStream_t s, int B = 1) {
  const int V = sc->vocab;
  const SoftWs ws = soft_carve(n, D, V, dt, cv);
  if (n == 0) return DG_OK;
  const int C = n / B;
  for (int b = 0; b < B; ++b)
    DG_HIP(launch_probs(dt, logits + static_cast<size_t>(b) * C * V, rowstats + static_cast<size_t>(b) * C * 2, C, V,
                        static_cast<float>(1.0 / temperature(&sc[b])),
                        static_cast<char *>(ws.P) + static_cast<size_t>(b) * C * V * esize(dt), s));
  const SoftPlan pl = softembed_plan(dt, n, D, V);
  {
    GemmArgs g = dense_args(ws.P, V, n, D, V, u, D);
    g.seg_B0[0] = embed_t;
    g.tile_order = 1;
    TimedLaunch tl(DG_KT_SOFT_EMBED, s);
    if (pl.wide) DG_HIP(wide_product(g, EPI_STORE, DG_SOFT_CFG, ws.part, pl.ks, s));
    else DG_HIP(dense_product(dt, g, EPI_STORE, ws.part, pl.ks, s));
  }
  return DG_OK;
}

int lm_head_impl(int n, int D, int V, float eps, int dt, const void *x, const void *wn, const void *E, float *logits,
                 Carve &cv, hipStream_t s) {
  void *h = cv.bytes(static_cast<size_t>(n) * D * esize(dt));
  if (n == 0) return DG_OK;
  DG_HIP(launch_rmsnorm(dt, n, D, eps, x, wn, h, s));
  GemmArgs g = dense_args(h, D, n, V, D, logits, V);
  g.seg_B0[0] = E;
  g.tile_order = 0;
  TimedLaunch tl(DG_KT_LM_HEAD, s);
  if (wide_ok(dt, g, DG_HEAD_CFG, n)) DG_HIP(launch_gemm_wide(g, EPI_STORE_F32, DG_HEAD_CFG, s));
  else DG_HIP(sgemm(dt, g, EPI_STORE_F32, DG_DENSE_MT, DG_DENSE_NT, s));
  return DG_OK;
}

// ---------------------------------------------------------- whole model

int check_model(const dg_model_cfg *c) {
  if (!c) return DG_ERR_NULL;
  if (!dtype_ok(c->dtype)) return DG_ERR_DTYPE;
  DG_TRY(check_attn_cfg(&c->sliding));
  DG_TRY(check_attn_cfg(&c->global));
  DG_TRY(check_moe_cfg(&c->moe));
  if (c->sliding.dtype != c->dtype || c->global.dtype != c->dtype || c->moe.dtype != c->dtype) return DG_ERR_DTYPE;
  const int D = c->sliding.hidden;
  if (c->global.hidden != D || c->moe.hidden != D) return DG_ERR_SHAPE;
  if (c->n_layers <= 0 || c->global_every <= 0 || c->vocab <= 0 || c->vocab % 64 || c->sc_ffn < 0 ||
      c->sc_ffn % 64)
    return DG_ERR_SHAPE;
  return DG_OK;
}

const dg_attn_cfg *layer_cfg(const dg_model_cfg *c, int l) {
  return (l % c->global_every) == c->global_every - 1 ? &c->global : &c->sliding;
}

// n rows in canvases of C rows (C = n: one canvas)
size_t layer_ws_bytes(const dg_model_cfg *c, int n, int C) {
  size_t m = moe_ws_bytes(&c->moe, n);
  const size_t a0 = attn_ws_bytes(&c->sliding, n, C), a1 = attn_ws_bytes(&c->global, n, C);
  if (a0 > m) m = a0;
  if (a1 > m) m = a1;
  return m;
}

struct StepWs {
  void *x, *h, *g_sc;   // h: pre-norm activations handed from block to block
  float *logits, *rowstats;
  float2 *tab[2];       // rotation tables of the sliding and the global layers
  void *rest;
};

StepWs step_carve(const dg_model_cfg *c, int n, bool need_logits, Carve &cv, int C = 0) {
  const size_t es = esize(c->dtype);
  const int D = c->sliding.hidden;
  StepWs w;
  w.x = cv.bytes(static_cast<size_t>(n) * D * es);
  w.h = cv.bytes(static_cast<size_t>(n) * D * es);
  w.g_sc = cv.bytes(static_cast<size_t>(n) * (c->sc_ffn > 0 ? c->sc_ffn : 1) * es);
  w.logits = need_logits ? cv.take<float>(static_cast<size_t>(n) * c->vocab) : nullptr;
  w.rowstats = cv.take<float>(static_cast<size_t>(n) * 2);
  w.tab[0] = cv.take<float2>(static_cast<size_t>(n) * (c->sliding.head_dim / 2));
  w.tab[1] = cv.take<float2>(static_cast<size_t>(n) * (c->global.head_dim / 2));
  size_t tail = layer_ws_bytes(c, n, C > 0 ? C : n);
  {
    Carve t(nullptr);
    t.bytes(static_cast<size_t>(n) * D * es);
    sample_carve(n, c->vocab, t);
    if (t.off > tail) tail = t.off;
  }
  {
    Carve t(nullptr);
    soft_carve(n, D, c->vocab, c->dtype, t);
    if (t.off > tail) tail = t.off;
  }
  w.rest = cv.bytes(tail + 256);
  return w;
}

// Rotation tables of every canvas for the first layer of each type (every
// layer of a type sits at the same position in a step); rt[2*b + t] is
// canvas b's table for type t (0 sliding, 1 global).  A layer at another
// position makes its own.
int make_rope_tabs(const dg_model_cfg *cfg, const dg_kv_cache *kv, int B, int C, const StepWs &sw, RopeTab *rt,
                   hipStream_t s) {
  for (int t = 0; t < 2; ++t) {
    for (int l = 0; l < cfg->n_layers; ++l) {
      const dg_attn_cfg *ac = layer_cfg(cfg, l);
      if ((ac == &cfg->global) != (t == 1)) continue;
      for (int b = 0; b < B; ++b) {
        RopeTab &r = rt[2 * b + t];
        r.pos0 = kv[b].layer[l].kv_len;
        r.tab = sw.tab[t] + static_cast<size_t>(b) * C * (ac->head_dim / 2);
        DG_HIP(launch_rope_table(r.pos0, C, ac->head_dim, ac->rope_base, rope_rot(ac), sw.tab[t] +
                                 static_cast<size_t>(b) * C * (ac->head_dim / 2), s));
      }
      break;
    }
  }
  return DG_OK;
}

}  // namespace

// Built-in scratch of dg_sample_renoise_noalloc: the sampler's per-row,
// per-vocabulary-slice partial statistics for up to kNoAllocSlots
// (row, slice) pairs.  Each GPU holds its own copy for the life of the
// process.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in); it uses the device address taken once per device.
namespace {
constexpr size_t kNoAllocSlots = 8192 * 16;   // e.g. 8192 rows x 16 slices
constexpr size_t kNoAllocScratchBytes = kNoAllocSlots * (4 * sizeof(float) + 2 * sizeof(int)) + 3 * 256;
constexpr int kMaxDevices = 64;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
void *g_scratch_dev[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's address of `scratch`, taken on the first call on
// that device (hipGetSymbolAddress with the device current); nullptr if it
// cannot be taken.
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_dev[dev] = p;
  }
  return g_scratch_dev[dev];
}
}  // namespace

// ====================================================================== ABI

extern "C" {

void dg_set_kernel_timer(dg_kernel_timer *timer) { g_timer = timer; }

const char *dg_status_string(int st) {
  switch (st) {
    case DG_OK: return "ok";
    case DG_ERR_NULL: return "required pointer is NULL";
    case DG_ERR_SHAPE: return "invalid or inconsistent size";
    case DG_ERR_UNSUPPORTED: return "configuration not supported by the built kernels";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_DTYPE: return "invalid or mismatched dtype";
    case DG_ERR_HIP: return "HIP launch failed";
    case DG_ERR_CAPACITY: return "KV cache capacity exceeded";
  }
  return "unknown status";
}

size_t dg_attn_workspace_bytes(const dg_attn_cfg *cfg, int n_tok) {
  if (check_attn_cfg(cfg) != DG_OK || n_tok < 0) return 0;
  return attn_ws_bytes(cfg, n_tok);
}

int dg_attn_layer(const dg_attn_cfg *cfg, const dg_attn_w *w, dg_kv_layer *kv, int n_tok, int causal, void *x,
                  void *ws, size_t ws_bytes, void *stream) {
  DG_TRY(check_attn_call(cfg, w, kv, n_tok, causal, x));
  if (n_tok == 0) return DG_OK;
  if (!ws) return DG_ERR_NULL;
  if (ws_bytes < attn_ws_bytes(cfg, n_tok)) return DG_ERR_WORKSPACE;
  Carve cv(ws);
  return attn_impl(cfg, w, kv, n_tok, causal, x, cv, static_cast<hipStream_t>(stream));
}

size_t dg_moe_workspace_bytes(const dg_moe_cfg *cfg, int n_tok) {
  if (check_moe_cfg(cfg) != DG_OK || n_tok < 0) return 0;
  return moe_ws_bytes(cfg, n_tok);
}

int dg_moe_block(const dg_moe_cfg *cfg, const dg_moe_w *w, int n_tok, void *x, const float *rl_in,
                 int32_t *idx_out, float *w_out, void *ws, size_t ws_bytes, void *stream) {
  DG_TRY(check_moe_call(cfg, w, n_tok, x, rl_in));
  if (n_tok == 0) return DG_OK;
  if (!ws) return DG_ERR_NULL;
  if (ws_bytes < moe_ws_bytes(cfg, n_tok)) return DG_ERR_WORKSPACE;
  Carve cv(ws);
  return moe_impl(cfg, w, n_tok, x, rl_in, idx_out, w_out, cv, static_cast<hipStream_t>(stream));
}

int dg_quantize_fp8(int dtype, const void *w, long long rows, int cols, uint8_t *q, float *scale, void *stream) {
  if (!dtype_ok(dtype)) return DG_ERR_DTYPE;
  if (rows < 0 || cols <= 0 || rows > 0x7fffffffLL) return DG_ERR_SHAPE;
  if (rows == 0) return DG_OK;
  if (!w || !q || !scale) return DG_ERR_NULL;
  if (launch_quantize_fp8(dtype, w, rows, cols, q, scale, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DG_ERR_HIP;
  return DG_OK;
}

size_t dg_sample_workspace_bytes(int n_pos, int vocab) {
  if (n_pos < 0 || vocab <= 0) return 0;
  Carve cv(nullptr);
  sample_carve(n_pos, vocab, cv);
  return cv.off + 256;
}

int dg_sample_renoise(const dg_sampler_cfg *cfg, int n_pos, const void *logits, int logits_dtype, int32_t *tok,
                      uint8_t *commit, float *ent, float *rowstats, int32_t *nre, int32_t *pred,
                      int32_t *n_changed, int32_t *n_nonfinite, void *ws, size_t ws_bytes, void *stream) {
  DG_TRY(check_sampler_cfg(cfg));
  if (!dtype_ok(logits_dtype)) return DG_ERR_DTYPE;
  if (n_pos < 0) return DG_ERR_SHAPE;
  if (!logits || !tok || !commit || !ent || !nre || !ws) return DG_ERR_NULL;
  if (ws_bytes < dg_sample_workspace_bytes(n_pos, cfg->vocab)) return DG_ERR_WORKSPACE;
  Carve cv(ws);
  return sample_impl(cfg, n_pos, logits, logits_dtype, tok, commit, ent, rowstats, nre, pred, n_changed,
                     n_nonfinite, cv, static_cast<hipStream_t>(stream));
}

size_t dg_sample_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int dg_sample_renoise_noalloc(const dg_sampler_cfg *cfg, int n_pos, const void *logits, int logits_dtype,
                              int32_t *tok, uint8_t *commit, float *ent, float *rowstats, int32_t *nre,
                              int32_t *pred, int32_t *n_changed, int32_t *n_nonfinite, void *stream) {
  DG_TRY(check_sampler_cfg(cfg));
  if (!dtype_ok(logits_dtype)) return DG_ERR_DTYPE;
  if (n_pos < 0) return DG_ERR_SHAPE;
  if (!logits || !tok || !commit || !ent || !nre) return DG_ERR_NULL;
  // the partial statistics must fit the built-in scratch
  if (dg_sample_workspace_bytes(n_pos, cfg->vocab) > kNoAllocScratchBytes) return DG_ERR_WORKSPACE;
  void *ws = scratch_address();
  if (!ws) return DG_ERR_HIP;
  Carve cv(ws);
  return sample_impl(cfg, n_pos, logits, logits_dtype, tok, commit, ent, rowstats, nre, pred, n_changed,
                     n_nonfinite, cv, static_cast<hipStream_t>(stream));
}

int dg_canvas_noise(int n_pos, int vocab, uint64_t seed, uint32_t canvas_idx, int32_t *tokens, void *stream) {
  if (!tokens) return DG_ERR_NULL;
  if (n_pos < 0 || vocab <= 0) return DG_ERR_SHAPE;
  if (launch_canvas_noise(n_pos, vocab, static_cast<uint32_t>(seed & 0xffffffffull), static_cast<uint32_t>(seed >> 32),
                          canvas_idx, tokens, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DG_ERR_HIP;
  return DG_OK;
}

size_t dg_lm_head_workspace_bytes(int n_pos, int hidden, int dtype) {
  if (n_pos < 0 || hidden <= 0 || !dtype_ok(dtype)) return 0;
  return static_cast<size_t>(n_pos) * hidden * esize(dtype) + 512;
}

int dg_lm_head(int n_pos, int hidden, int vocab, float eps, int dtype, const void *x, const void *wn, const void *E,
               float *logits, void *ws, size_t ws_bytes, void *stream) {
  if (!dtype_ok(dtype)) return DG_ERR_DTYPE;
  if (n_pos < 0 || hidden <= 0 || hidden % 64 || vocab <= 0 || vocab % 8) return DG_ERR_SHAPE;
  if (!x || !wn || !E || !logits || !ws) return DG_ERR_NULL;
  if (ws_bytes < dg_lm_head_workspace_bytes(n_pos, hidden, dtype)) return DG_ERR_WORKSPACE;
  Carve cv(ws);
  return lm_head_impl(n_pos, hidden, vocab, eps, dtype, x, wn, E, logits, cv, static_cast<hipStream_t>(stream));
}

size_t dg_soft_embed_workspace_bytes(int n_pos, int hidden, int vocab, int dtype) {
  if (n_pos < 0 || hidden <= 0 || vocab <= 0 || !dtype_ok(dtype)) return 0;
  Carve cv(nullptr);
  soft_carve(n_pos, hidden, vocab, dtype, cv);
  return cv.off + 256;
}

int dg_soft_embed(const dg_sampler_cfg *scfg, int n_pos, int hidden, int dtype, const float *logits,
                  const float *rowstats, const void *embed_t, void *u, void *ws, size_t ws_bytes, void *stream) {
  DG_TRY(check_sampler_cfg(scfg));
  if (!dtype_ok(dtype)) return DG_ERR_DTYPE;
  if (n_pos < 0 || hidden <= 0 || hidden % 64 || scfg->vocab % 64) return DG_ERR_SHAPE;
  if (!logits || !rowstats || !embed_t || !u || !ws) return DG_ERR_NULL;
  if (ws_bytes < dg_soft_embed_workspace_bytes(n_pos, hidden, scfg->vocab, dtype)) return DG_ERR_WORKSPACE;
  Carve cv(ws);
  return soft_embed_impl(scfg, n_pos, hidden, dtype, logits, rowstats, embed_t, u, cv,
                         static_cast<hipStream_t>(stream));
}

int dg_embed_transpose(int vocab, int hidden, int dtype, const void *E, void *Et, void *stream) {
  if (!dtype_ok(dtype)) return DG_ERR_DTYPE;
  if (vocab <= 0 || hidden <= 0) return DG_ERR_SHAPE;
  if (!E || !Et) return DG_ERR_NULL;
  if (launch_transpose(dtype, vocab, hidden, E, Et, static_cast<hipStream_t>(stream)) != hipSuccess) return DG_ERR_HIP;
  return DG_OK;
}

int dg_rmsnorm(int n, int hidden, float eps, int dtype, const void *x, const void *w, void *y, void *stream) {
  if (!dtype_ok(dtype)) return DG_ERR_DTYPE;
  if (n < 0 || hidden <= 0 || hidden % 8) return DG_ERR_SHAPE;
  if (!x || !w || !y) return DG_ERR_NULL;
  if (launch_rmsnorm(dtype, n, hidden, eps, x, w, y, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DG_ERR_HIP;
  return DG_OK;
}

size_t dg_workspace_bytes(const dg_model_cfg *cfg, int max_canvas_tokens, int max_commit_tokens) {
  if (check_model(cfg) != DG_OK || max_canvas_tokens < 0 || max_commit_tokens < 0) return 0;
  Carve a(nullptr), b(nullptr);
  step_carve(cfg, max_canvas_tokens, true, a);
  step_carve(cfg, max_commit_tokens, false, b);
  return (a.off > b.off ? a.off : b.off) + 256;
}

static int check_model_w(const dg_model_cfg *c, const dg_model_w *w, bool need_head) {
  if (!w || !w->embed || !w->attn || !w->moe || !w->layer_scalar) return DG_ERR_NULL;
  for (int l = 0; l < c->n_layers; ++l) {
    const dg_attn_cfg *ac = (l % c->global_every) == c->global_every - 1 ? &c->global : &c->sliding;
    const dg_attn_w &a = w->attn[l];
    if (!a.w_in_norm || !a.w_q || !a.w_k || !a.w_o || !a.q_norm || !a.k_norm) return DG_ERR_NULL;
    if (!ac->shared_kv && !a.w_v) return DG_ERR_NULL;
    const dg_moe_w &m = w->moe[l];
    if (!m.w_in_norm || !m.w_gate || !m.w_up || !m.w_down || !m.ws_gate || !m.ws_up || !m.ws_down)
      return DG_ERR_NULL;
    if (c->moe.expert_format == DG_EXPERTS_FP8_E4M3 &&
        (!m.s_gate || !m.s_up || !m.s_down || !m.ss_gate || !m.ss_up || !m.ss_down))
      return DG_ERR_NULL;
    const bool router = m.w_router || (w->router_logits && w->router_logits[l]);
    if (!router) return DG_ERR_NULL;
  }
  if (need_head && (!w->w_final_norm || !w->embed_t)) return DG_ERR_NULL;
  if (c->sc_ffn > 0 && need_head && (!w->sc_gate || !w->sc_up || !w->sc_down)) return DG_ERR_NULL;
  return DG_OK;
}

static int check_kv(const dg_model_cfg *c, const dg_kv_cache *kv) {
  if (!kv || !kv->layer) return DG_ERR_NULL;
  if (kv->n_layers != c->n_layers) return DG_ERR_SHAPE;
  const int P = kv->layer[0].kv_len;
  for (int l = 0; l < c->n_layers; ++l) {
    const dg_kv_layer &L = kv->layer[l];
    if (L.kv_len != P || L.kv_len < 0 || L.capacity % 8) return DG_ERR_SHAPE;
    if (!L.ring && L.kv_len > L.capacity) return DG_ERR_SHAPE;
    if (!L.k || !L.v) return DG_ERR_NULL;
  }
  return DG_OK;
}

}  // extern "C"

namespace {

// One denoising step of B canvases of C rows (st's buffers hold them back to
// back; kv[b] and scfg[b] are canvas b's).
int step_impl(const dg_model_cfg *cfg, const dg_model_w *w, const dg_kv_cache *kv, dg_canvas_state *st,
              const dg_sampler_cfg *scfg, int B, void *ws, size_t ws_bytes, hipStream_t s) {
  DG_TRY(check_model(cfg));
  DG_TRY(check_model_w(cfg, w, true));
  if (!kv || !scfg) return DG_ERR_NULL;
  if (B <= 0) return DG_ERR_SHAPE;
  if (!st || !st->tokens || !st->u || !st->commit || !st->entropy || !st->n_renoised) return DG_ERR_NULL;
  const int C = st->canvas_len;
  if (C <= 0) return DG_ERR_SHAPE;
  for (int b = 0; b < B; ++b) {
    DG_TRY(check_sampler_cfg(&scfg[b]));
    if (scfg[b].vocab != cfg->vocab) return DG_ERR_SHAPE;
    if (scfg[b].commit_rule == DG_COMMIT_SORTED_CUMULATIVE && C > kSortedMaxRows) return DG_ERR_SHAPE;
    DG_TRY(check_kv(cfg, &kv[b]));
    for (int l = 0; l < cfg->n_layers; ++l) DG_TRY(check_kv_room(layer_cfg(cfg, l), &kv[b].layer[l], C));
  }
  const int n = B * C;
  if (!ws) return DG_ERR_NULL;
  Carve cv(ws);
  const StepWs sw = step_carve(cfg, n, st->logits == nullptr, cv, C);
  if (ws_bytes < cv.off) return DG_ERR_WORKSPACE;
  const int dt = cfg->dtype, D = cfg->sliding.hidden, V = cfg->vocab;

  DG_HIP(launch_embed(dt, st->tokens, n, D, V, w->embed, sw.x, s));
  std::vector<RopeTab> rt(2 * B);
  DG_TRY(make_rope_tabs(cfg, kv, B, C, sw, rt.data(), s));
  if (st->use_u && cfg->sc_ffn > 0) {
    GemmArgs g = dense_args(st->u, D, n, cfg->sc_ffn, D, sw.g_sc, cfg->sc_ffn);
    g.seg_B0[0] = w->sc_gate;
    g.seg_B1[0] = w->sc_up;
    DG_HIP(sgemm(dt, g, EPI_SWIGLU, 4, DG_MOE_NT_GU, s));   // 64-row tiles: its own kernel instance
    GemmArgs d = dense_args(sw.g_sc, cfg->sc_ffn, n, D, cfg->sc_ffn, sw.x, D);
    d.seg_B0[0] = w->sc_down;
    DG_HIP(sgemm(dt, d, EPI_ADD, DG_DENSE_MT, DG_DENSE_NT, s));
  }
  std::vector<dg_kv_layer> Ls(B);
  std::vector<dg_kv_layer *> Lp(B);
  std::vector<RopeTab> rl(B);
  for (int l = 0; l < cfg->n_layers; ++l) {
    Carve c1(sw.rest);
    const dg_attn_cfg *ac = layer_cfg(cfg, l);
    const int t = ac == &cfg->global ? 1 : 0;
    for (int b = 0; b < B; ++b) {
      Ls[b] = kv[b].layer[l];   // decode: the caller's kv_len stays as it is
      Lp[b] = &Ls[b];
      rl[b] = rt[2 * b + t];
    }
    dg_moe_cfg mc = cfg->moe;
    mc.layer_scalar = w->layer_scalar[l];
    NextNorm to_moe;
    to_moe.h = sw.h;
    to_moe.w = w->moe[l].w_in_norm;
    to_moe.eps = mc.rms_eps;
    DG_TRY(attn_impl(ac, &w->attn[l], Lp.data(), B, C, 0, sw.x, c1, s, l == 0 ? nullptr : sw.h, to_moe, rl.data()));
    NextNorm to_attn;
    if (l + 1 < cfg->n_layers) {
      to_attn.h = sw.h;
      to_attn.w = w->attn[l + 1].w_in_norm;
      to_attn.eps = layer_cfg(cfg, l + 1)->rms_eps;
    }
    Carve c2(sw.rest);
    DG_TRY(moe_impl(&mc, &w->moe[l], n, sw.x, w->router_logits ? w->router_logits[l] : nullptr, nullptr, nullptr, c2,
                    s, sw.h, to_attn));
  }
  float *logits = st->logits ? st->logits : sw.logits;
  {
    Carve c(sw.rest);
    DG_TRY(lm_head_impl(n, D, V, cfg->rms_eps, dt, sw.x, w->w_final_norm, w->embed, logits, c, s));
  }
  for (int b = 0; b < B; ++b) {
    Carve c(sw.rest);
    const size_t r0 = static_cast<size_t>(b) * C;
    DG_TRY(sample_impl(&scfg[b], C, logits + r0 * V, DG_F32, st->tokens + r0, st->commit + r0, st->entropy + r0,
                       sw.rowstats + 2 * r0, st->n_renoised + b, st->pred ? st->pred + r0 : nullptr,
                       st->n_changed ? st->n_changed + b : nullptr,
                       st->n_nonfinite ? st->n_nonfinite + b : nullptr, c, s));
  }
  if (cfg->sc_ffn > 0) {
    Carve c(sw.rest);
    DG_TRY(soft_embed_impl(scfg, n, D, dt, logits, sw.rowstats, w->embed_t, st->u, c, s, B));
  }
  return DG_OK;
}

}  // namespace

extern "C" {

int dg_canvas_step(const dg_model_cfg *cfg, const dg_model_w *w, const dg_kv_cache *kv, dg_canvas_state *st,
                   const dg_sampler_cfg *scfg, void *ws, size_t ws_bytes, void *stream) {
  return step_impl(cfg, w, kv, st, scfg, 1, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

int dg_canvas_step_batch(const dg_model_cfg *cfg, const dg_model_w *w, const dg_kv_cache *kv, dg_canvas_state *st,
                         const dg_sampler_cfg *scfg, int n_canvas, void *ws, size_t ws_bytes, void *stream) {
  return step_impl(cfg, w, kv, st, scfg, n_canvas, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t dg_workspace_bytes_batch(const dg_model_cfg *cfg, int n_canvas, int canvas_len) {
  if (!cfg || n_canvas <= 0 || canvas_len <= 0) return 0;
  Carve a(nullptr);
  step_carve(cfg, n_canvas * canvas_len, true, a, canvas_len);
  return a.off + 256;
}

int dg_commit_canvas(const dg_model_cfg *cfg, const dg_model_w *w, dg_kv_cache *kv, const int32_t *tokens, int n,
                     void *ws, size_t ws_bytes, void *stream) {
  DG_TRY(check_model(cfg));
  DG_TRY(check_model_w(cfg, w, false));
  DG_TRY(check_kv(cfg, kv));
  if (!tokens) return DG_ERR_NULL;
  if (n < 0) return DG_ERR_SHAPE;
  if (n == 0) return DG_OK;
  for (int l = 0; l < cfg->n_layers; ++l)
    DG_TRY(check_kv_room(layer_cfg(cfg, l), &kv->layer[l], n));
  if (!ws) return DG_ERR_NULL;
  Carve cv(ws);
  const StepWs sw = step_carve(cfg, n, false, cv);
  if (ws_bytes < cv.off) return DG_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = cfg->dtype, D = cfg->sliding.hidden;
  DG_HIP(launch_embed(dt, tokens, n, D, cfg->vocab, w->embed, sw.x, s));
  RopeTab rt[2];
  DG_TRY(make_rope_tabs(cfg, kv, 1, n, sw, rt, s));
  const int L = cfg->n_layers;
  for (int l = 0; l < L; ++l) {
    const dg_attn_cfg *ac = layer_cfg(cfg, l);
    dg_kv_layer &KL = kv->layer[l];
    if (l == L - 1) {
      // last layer: only its K/V are needed (pre-norm, projections, norm/RoPE, append)
      Carve c1(sw.rest);
      const AttnPlan p = attn_plan(ac, n);
      const AttnWs aw = attn_carve(ac, p, p, c1);
      const void *hA = sw.h;   // written by the previous MoE block
      if (l == 0) {
        DG_HIP(launch_rmsnorm(dt, n, D, ac->rms_eps, sw.x, w->attn[l].w_in_norm, aw.h, s));
        hA = aw.h;
      }
      GemmArgs g = dense_args(hA, D, n, p.Nk + p.Nv, D, aw.qkv, p.Ntot);
      // write k|v at column Nq of the qkv rows so the norm/RoPE pass reads the usual layout
      g.C = static_cast<char *>(aw.qkv) + static_cast<size_t>(p.Nq) * esize(dt);
      g.nseg = ac->shared_kv ? 1 : 2;
      g.seg_start[0] = 0;
      g.seg_start[1] = p.Nk;
      g.seg_start[2] = p.Nk + p.Nv;
      g.seg_B0[0] = w->attn[l].w_k;
      g.seg_B0[1] = w->attn[l].w_v;
      DG_HIP(sgemm(dt, g, EPI_STORE, DG_DENSE_MT, DG_DENSE_NT, s));
      NormRopeArgs nr;
      nr.qkv = aw.qkv;
      nr.ld = p.Ntot;
      nr.n_tok = n;
      nr.Hq = 0;
      nr.Hkv = ac->n_kv_heads;
      nr.dh = ac->head_dim;
      nr.q_off = 0;
      nr.k_off = p.Nq;
      nr.v_off = ac->shared_kv ? p.Nq : p.Nq + p.Nk;
      nr.q_norm = w->attn[l].q_norm;
      nr.k_norm = w->attn[l].k_norm;
      nr.k_dst = KL.k;
      nr.k_head_stride = static_cast<long long>(KL.capacity) * ac->head_dim;
      nr.k_row0 = KL.kv_len;
      nr.k_ring = KL.ring ? KL.capacity : 0;
      nr.v_dst = aw.v_rows;
      nr.v_head_stride = static_cast<long long>(n) * ac->head_dim;
      nr.vt_dst = KL.v;
      nr.vt_hs = static_cast<long long>(ac->head_dim) * KL.capacity;
      nr.vt_ld = KL.capacity;
      nr.vt_col0 = KL.kv_len;
      nr.vt_ring = KL.ring ? KL.capacity : 0;
      nr.pos0 = KL.kv_len;
      nr.rope_base = ac->rope_base;
      nr.n_rot = rope_rot(ac);
      nr.eps = ac->rms_eps;
      nr.sqrt_dh = static_cast<float>(sqrt(static_cast<double>(ac->head_dim)));
      nr.v_unit_rms = ac->v_unit_rms;
      const RopeTab &r = rt[ac == &cfg->global ? 1 : 0];
      if (r.tab && r.pos0 == KL.kv_len) {
        nr.rope_tab = r.tab;
      } else {
        DG_HIP(launch_rope_table(KL.kv_len, n, ac->head_dim, ac->rope_base, rope_rot(ac), aw.rope_tab, s));
        nr.rope_tab = aw.rope_tab;
      }
      DG_HIP(launch_norm_rope(nr, dt, s));
      KL.kv_len += n;
      break;
    }
    Carve c1(sw.rest);
    dg_moe_cfg mc = cfg->moe;
    mc.layer_scalar = w->layer_scalar[l];
    NextNorm to_moe;
    to_moe.h = sw.h;
    to_moe.w = w->moe[l].w_in_norm;
    to_moe.eps = mc.rms_eps;
    DG_TRY(attn_impl(ac, &w->attn[l], &KL, n, 1, sw.x, c1, s, l == 0 ? nullptr : sw.h, to_moe,
                     rt[ac == &cfg->global ? 1 : 0]));
    NextNorm to_attn;   // the next layer (possibly the K/V-only last one) reads its pre-norm from sw.h
    to_attn.h = sw.h;
    to_attn.w = w->attn[l + 1].w_in_norm;
    to_attn.eps = layer_cfg(cfg, l + 1)->rms_eps;
    Carve c2(sw.rest);
    DG_TRY(moe_impl(&mc, &w->moe[l], n, sw.x, w->router_logits ? w->router_logits[l] : nullptr, nullptr, nullptr, c2,
                    s, sw.h, to_attn));
  }
  return DG_OK;
}

}  // extern "C"
