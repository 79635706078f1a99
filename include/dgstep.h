/*
 * dgstep.h -- C ABI of libdgstep: one denoising step of a DiffusionGemma-style
 * discrete text diffusion model over a canvas of tokens, on one MI355X (gfx950).
 *
 * Sources (five web pages on DiffusionGemma, cited by page and section):
 *   aitrends.kr notebook summary  -- QK-norm paragraph + rms code, RoPE
 *       paragraph + rotate code, attention paragraph + projection code,
 *       sampler paragraph, glossary (Scalar QK Norm, Partial RoPE, Layer
 *       Scalar, Self-conditioning, MoE, Sliding-window Attention);
 *   thakicloud "DiffusionGemma 26B-A4B" post -- Architecture;
 *   velog "DiffusionGemma Self-conditioning" post -- Self-conditioning,
 *       DiffusionGemma structure;
 *   DiffusionGemma Technical Report review -- section 1 (Canvas, Adaptive
 *       Stopping);
 *   aibars.net news -- block-autoregressive denoising and self-correction.
 *
 * Conventions shared by every entry point
 *   - Pointers inside weight, cache and state records, and every tensor
 *     argument, are DEVICE pointers owned by the caller.  Config records and
 *     the arrays of per-layer records are HOST memory.  The library never
 *     allocates or frees device memory and keeps no mutable global state;
 *     scratch memory is the caller's workspace `ws` of `ws_bytes` bytes,
 *     256-byte aligned, sized by the matching *_workspace_bytes query (the
 *     one exception, dg_sample_renoise_noalloc, uses a built-in per-GPU
 *     scratch array instead).
 *   - `stream` is a hipStream_t (NULL = the null stream).  All device work is
 *     enqueued asynchronously on it; nothing synchronises with the host.
 *   - Arguments are validated on the host before any HIP call; a failed
 *     check returns a negative dg_status and enqueues nothing.  A launch
 *     failure returns DG_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation of the stream.
 *   - Layout is row-major.  Weight matrices are [out, in] (y = x W^T, as in
 *     the projection code on the aitrends page).  A head-major activation
 *     row [n_heads * head_dim] holds head n at columns [n*d, (n+1)*d).
 *   - dtype selects the element type of activations, weights and KV cache:
 *     DG_BF16 (bfloat16, fp32 accumulation) or DG_F32.  Router logits, LM
 *     logits, entropies and partial sums are always fp32.
 *   - Canvas positions are contiguous: token j of a call sits at absolute
 *     position kv_len + j (rotate(x, layer_type, start_idx) on the aitrends
 *     page).
 */
#ifndef DGSTEP_H
#define DGSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_NULL = -1,        /* a required pointer is NULL */
  DG_ERR_SHAPE = -2,       /* a size is non-positive, inconsistent or misaligned */
  DG_ERR_UNSUPPORTED = -3, /* valid but not built (e.g. a head_dim without a kernel) */
  DG_ERR_WORKSPACE = -4,   /* ws_bytes smaller than the workspace query returns */
  DG_ERR_DTYPE = -5,       /* unknown dtype, or dtypes that must agree do not */
  DG_ERR_HIP = -6,         /* a HIP launch failed */
  DG_ERR_CAPACITY = -7     /* the KV cache cannot hold the rows to append */
} dg_status;

typedef enum { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

/* ---------------------------------------------------------------- attention */

/* One attention layer (aitrends page: attention paragraph and projection code;
 * glossary "Sliding-window Attention").  layer_type 0 = sliding window: the
 * canvas sees itself plus the last `window` committed rows; 1 = global: the
 * canvas sees every committed row.  Global layers share the K/V projection
 * (shared_kv = 1, W_v = W_k) and normalise V to unit RMS (v_unit_rms = 1);
 * their RoPE keeps only the first rotary_factor of the frequencies. */
typedef struct {
  int hidden;          /* D, multiple of 64 */
  int n_q_heads;       /* Hq, multiple of n_kv_heads */
  int n_kv_heads;      /* Hkv */
  int head_dim;        /* d_h: 64, 128, 256 or 512 */
  int layer_type;      /* 0 sliding window, 1 global */
  int window;          /* W, committed rows visible in front of the canvas (sliding) */
  int shared_kv;       /* 1: the value projection is the key projection */
  int v_unit_rms;      /* 1: v <- rms(v, 1) per head */
  float rope_base;     /* f_t = rope_base^(-2t/d_h) */
  float rotary_factor; /* fraction of the d_h/2 frequencies kept (global layers) */
  float rms_eps;       /* added to the L2 norm */
  int dtype;           /* dg_dtype */
} dg_attn_cfg;

typedef struct {
  const void *w_in_norm; /* [D]              pre-attention RMSNorm weight */
  const void *w_q;       /* [Hq*d_h, D] */
  const void *w_k;       /* [Hkv*d_h, D] */
  const void *w_v;       /* [Hkv*d_h, D], ignored (may be NULL) when shared_kv */
  const void *w_o;       /* [D, Hq*d_h] */
  const void *q_norm;    /* [d_h] QK-norm weights (constant vectors in the trained model) */
  const void *k_norm;    /* [d_h] */
} dg_attn_w;

/* Keys/values of one layer, stored after QK-norm and RoPE at their own
 * positions, in the layer dtype:
 *   k: [Hkv][capacity][d_h]  (position m at row m)
 *   v: [Hkv][d_h][capacity]  (transposed: position m at column m, so the
 *                             probability-times-value product reads values
 *                             key-contiguously)
 * Positions [0, kv_len) are committed.  Every call places its own n_tok rows
 * at positions [kv_len, kv_len + n_tok), so capacity must be at least
 * kv_len + n_tok, and a multiple of 8. */
typedef struct {
  void *k;
  void *v;
  int capacity;
  int kv_len;
  int ring;            /* 0: position m at row m (kv_len + n_tok <= capacity).
                        * 1 (sliding layers only): position m at row m mod
                        * capacity, so the cache holds only the window and the
                        * rows in flight: capacity a multiple of 32 and at least
                        * window + n_tok; kv_len counts all committed positions
                        * (aitrends glossary Sliding-window: only the last
                        * window rows are ever read). */
  int v_only;          /* 0: k holds the layer's keys.  1 (global layers with
                        * shared_kv and v_unit_rms only; not with ring): only
                        * v is kept.  Since W_v = W_k, the stored value is the
                        * unit-RMS raw key and K = RoPE_p(k_norm * V) (aitrends
                        * attention paragraph: KV cache saving / reconstruction
                        * with W_v = W_k), so every call rebuilds the keys of
                        * positions [0, kv_len) from v into k, which is then
                        * scratch of the same [Hkv][capacity][d_h] shape that
                        * all v_only layers of a stack may share. */
} dg_kv_layer;

/* Workspace bytes for dg_attn_layer with at most n_tok tokens per call. */
size_t dg_attn_workspace_bytes(const dg_attn_cfg *cfg, int n_tok);

/* x <- x + Attention(rms(x)) for n_tok tokens at positions kv_len.. .
 * causal = 0 (decode): the canvas attends bidirectionally to the visible
 *   committed rows and to itself; its K/V rows are written at
 *   [kv_len, kv_len + n_tok) as scratch and kv_len is left unchanged.
 * causal = 1 (encode/commit): key m is visible to the query at position p iff
 *   m <= p (and m > p - window in sliding layers); this call's post-norm/RoPE
 *   K/V rows are written to the cache at [kv_len, kv_len + n_tok) and
 *   kv->kv_len is advanced on the host when the work is enqueued.
 * x_inout: [n_tok, D] device, layer dtype.  Softmax scale is 1 (scalar
 * QK-norm fixes the temperature; aitrends QK-norm paragraph). */
int dg_attn_layer(const dg_attn_cfg *cfg, const dg_attn_w *w, dg_kv_layer *kv, int n_tok,
                  int causal, void *x_inout, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------- MoE */

/* MoE block (aitrends glossary "MoE"; thakicloud Architecture: 128 experts,
 * 8 active + 1 shared).  Experts are bias-free SwiGLU FFNs.  The router takes
 * softmax over the experts, keeps the top_k (ties to the lower id),
 * renormalises over them and multiplies by route_scale; the shared expert is
 * always added.  The layer scalar rescales the layer output (glossary
 * "Layer Scalar"): x <- layer_scalar * (x + y). */
typedef struct {
  int hidden;          /* D, multiple of 64 */
  int n_experts;       /* E <= 256 */
  int top_k;           /* <= 8, <= E */
  int ffn;             /* F, multiple of 64 */
  int shared_ffn;      /* F_s, multiple of 64 */
  float route_scale;
  float rms_eps;
  float layer_scalar;
  int dtype;
  int expert_format;   /* dg_expert_format */
} dg_moe_cfg;

/* Storage of the expert matrices (routed and shared).
 * DG_EXPERTS_DTYPE: in the layer dtype.
 * DG_EXPERTS_FP8_E4M3: OCP 8-bit E4M3 codes (1 byte each, same [.., N, K]
 *   layout) with one fp32 scale per matrix row (s_* / ss_* below), as made by
 *   dg_quantize_fp8; the weight is scale * value(code).  Activations stay in
 *   the layer dtype, which must be DG_BF16.  The pages run the model in FP8
 *   (aitrends notebook summary, generation-speed paragraph) without fixing a
 *   scheme; weight-only FP8 with row scales is the reading taken. */
typedef enum { DG_EXPERTS_DTYPE = 0, DG_EXPERTS_FP8_E4M3 = 1 } dg_expert_format;

typedef struct {
  const void *w_in_norm; /* [D] pre-MoE RMSNorm weight */
  const void *w_router;  /* [E, D]; may be NULL when router logits are injected */
  const void *w_gate;    /* [E, F, D] */
  const void *w_up;      /* [E, F, D] */
  const void *w_down;    /* [E, D, F] */
  const void *ws_gate;   /* [F_s, D] shared expert */
  const void *ws_up;     /* [F_s, D] */
  const void *ws_down;   /* [D, F_s] */
  /* fp32 row scales, DG_EXPERTS_FP8_E4M3 only (NULL otherwise) */
  const float *s_gate;   /* [E, F] */
  const float *s_up;     /* [E, F] */
  const float *s_down;   /* [E, D] */
  const float *ss_gate;  /* [F_s] */
  const float *ss_up;    /* [F_s] */
  const float *ss_down;  /* [D] */
} dg_moe_w;

/* Row-wise OCP E4M3 quantisation of a [rows, cols] matrix w (dtype, device):
 *   scale[r] = max_c |w[r][c]| / 448 in fp32 (1 for an all-zero row),
 *   q[r][c]  = E4M3(w[r][c] / scale[r]), fp32 division, rounded to nearest
 *              with ties to even, saturating at 448.
 * q [rows, cols] uint8 and scale [rows] fp32 are device buffers owned by the
 * caller.  Expert stacks [E, N, K] are quantised as E*N rows of K.
 * Enqueued on stream; returns DG_ERR_SHAPE for rows < 0 or cols <= 0. */
int dg_quantize_fp8(int dtype, const void *w, long long rows, int cols, uint8_t *q, float *scale, void *stream);

size_t dg_moe_workspace_bytes(const dg_moe_cfg *cfg, int n_tok);

/* x <- layer_scalar * (x + MoE(rms(x))) for n_tok tokens.
 * router_logits_in: optional [n_tok, E] fp32 device logits used instead of
 *   rms(x) W_router^T (lets callers feed both sides identical logits).
 * topk_idx_out [n_tok, top_k] int32 and topk_w_out [n_tok, top_k] fp32 are
 *   optional device outputs, in descending-score order. */
int dg_moe_block(const dg_moe_cfg *cfg, const dg_moe_w *w, int n_tok, void *x_inout,
                 const float *router_logits_in, int32_t *topk_idx_out, float *topk_w_out,
                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ sampler */

/* Entropy-bound sampler (aitrends sampler paragraph; aibars self-correction):
 * temperature t_i falls linearly from t_max (step 0) to t_min (step
 * n_steps-1); for every position the entropy H of softmax(l/t_i) (nats) is
 * computed; positions with H < tau commit their argmax token (lowest id on
 * ties), the others are re-noised with a uniform random token.  Tokens come
 * from Philox4x32-10 (Salmon et al., SC'11) with key = (seed lo, seed hi) and
 * counter = (position, step, canvas_idx, 0): token = (X0 * vocab) >> 32.
 * final_step != 0 commits every position. */
typedef struct {
  int vocab;
  float tau;           /* entropy bound, nats */
  float t_max, t_min;  /* temperature schedule */
  int n_steps;         /* schedule length (max denoising steps) */
  int step;            /* this step, 0-based */
  uint32_t canvas_idx;
  uint64_t seed;
  int final_step;
  int commit_rule;     /* dg_commit_rule (0: per position) */
  int token_rule;      /* dg_token_rule (0: argmax) */
} dg_sampler_cfg;

/* Variants of the sampler (the pages fix the low-entropy "prefix within the
 * entropy bound" and an adaptive stop on entropy and output stability, not
 * their exact form; aitrends sampler paragraph, secrett2633 review
 * section 1 Adaptive Stopping):
 * DG_COMMIT_ENTROPY: position j commits iff H_j < tau.
 * DG_COMMIT_SORTED_CUMULATIVE: positions in ascending entropy order (ties:
 *   lower position first); the position at each rank commits iff the summed
 *   entropy of the positions ranked before it is <= tau (the EB-sampler of
 *   Ben-Hamu et al. 2025); the lowest-entropy position always commits.
 *   n_pos <= 4096.
 * DG_TOKEN_ARGMAX: the proposal is the argmax of the logits (lowest id).
 * DG_TOKEN_GUMBEL: the proposal is argmax_v (l_v/t + g_v), a draw from
 *   softmax(l/t) by the Gumbel-max property; g_v = -ln(-ln u_v) with u from
 *   Philox4x32-10, counter (position, step, canvas_idx, 1 + v/4), word v%4:
 *   k = word >> 9, u = (k + 1/2) 2^-23 (-ln u through log1p of -(1-u) when
 *   u >= 1/2). */
typedef enum { DG_COMMIT_ENTROPY = 0, DG_COMMIT_SORTED_CUMULATIVE = 1 } dg_commit_rule;
typedef enum { DG_TOKEN_ARGMAX = 0, DG_TOKEN_GUMBEL = 1 } dg_token_rule;

size_t dg_sample_workspace_bytes(int n_pos, int vocab);

/* logits: [n_pos, vocab] device, fp32 (logits_dtype DG_F32) or bf16.
 * Outputs (device): tokens_out [n_pos] int32, commit_out [n_pos] uint8 (1 =
 * committed), entropy_out [n_pos] fp32, n_renoised_out [1] int32.
 * rowstats_out: optional [n_pos, 2] fp32 = (max of l/t, sum of exp(l/t - max)),
 * the statistics dg_soft_embed needs.
 * pred_inout: optional [n_pos] int32: in, the previous step's proposals (-1
 *   before the first step); out, this step's.  n_changed_out: optional [1]
 *   int32, the number of positions whose proposal changed (read only with
 *   pred_inout): the output-stability signal for adaptive stop.
 * n_nonfinite_out: optional [1] int32, the number of rows holding at least
 *   one NaN or +-inf logit (failure detection).  Such a row's entropy is NaN,
 *   so it is re-noised unless final_step; a NaN logit is never proposed, and a
 *   row with no number at all proposes token 0. */
int dg_sample_renoise(const dg_sampler_cfg *cfg, int n_pos, const void *logits, int logits_dtype,
                      int32_t *tokens_out, uint8_t *commit_out, float *entropy_out,
                      float *rowstats_out, int32_t *n_renoised_out, int32_t *pred_inout,
                      int32_t *n_changed_out, int32_t *n_nonfinite_out, void *ws, size_t ws_bytes,
                      void *stream);

/* dg_sample_renoise without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and results as
 * dg_sample_renoise (the same kernels); the partial statistics live in a
 * scratch array built into the library, one per GPU, held until the process
 * ends: at most dg_sample_noalloc_max_bytes() bytes, which covers
 * n_pos * (vocabulary slices) <= 131072 (8192 positions at any vocabulary).
 * Larger calls return DG_ERR_WORKSPACE before any HIP call.  Nothing is
 * allocated: the scratch address is taken once per device on the first call
 * there (DG_ERR_HIP if that fails).  Every call on one GPU uses the same
 * scratch, so calls that overlap on one GPU (several streams or threads at
 * once) race; serialise them. */
size_t dg_sample_noalloc_max_bytes(void);
int dg_sample_renoise_noalloc(const dg_sampler_cfg *cfg, int n_pos, const void *logits, int logits_dtype,
                              int32_t *tokens_out, uint8_t *commit_out, float *entropy_out,
                              float *rowstats_out, int32_t *n_renoised_out, int32_t *pred_inout,
                              int32_t *n_changed_out, int32_t *n_nonfinite_out, void *stream);

/* Initial canvas: n_pos uniform random tokens (counter step word 0xFFFFFFFF;
 * aibars text-diffusion paragraph: generation starts from a noise block). */
int dg_canvas_noise(int n_pos, int vocab, uint64_t seed, uint32_t canvas_idx, int32_t *tokens_out,
                    void *stream);

/* ------------------------------------------------- tied head, self-condition */

/* Tied LM head: logits = rms(x, w_final_norm) E^T, the output head sharing
 * the embedding table (aitrends notebook summary, details paragraphs: tied
 * embedding; thakicloud Architecture: vocabulary 262,144).  Reading: a final
 * RMSNorm precedes the head and no soft-cap follows it (the pages name the
 * norm helper for the block inputs only).
 * x [n_pos, D] and embed [vocab, D] in `dtype` (device); w_final_norm [D];
 * logits_out [n_pos, vocab] fp32 (device, caller-owned); ws holds the normed
 * rows.  hidden a multiple of 64, vocab of 8; DG_ERR_SHAPE / DG_ERR_NULL /
 * DG_ERR_WORKSPACE before any launch. */
size_t dg_lm_head_workspace_bytes(int n_pos, int hidden, int dtype);
int dg_lm_head(int n_pos, int hidden, int vocab, float rms_eps, int dtype, const void *x,
               const void *w_final_norm, const void *embed, float *logits_out, void *ws,
               size_t ws_bytes, void *stream);

/* Self-conditioning soft embedding (aitrends glossary "Self-conditioning";
 * velog Self-conditioning): u = P E with P = softmax(l / t_i) from fp32 logits
 * and the (max, sum) row statistics dg_sample_renoise wrote; t_i comes from
 * the sampler record.  embed_t is the [D, vocab] transposed copy of the
 * embedding table made once by dg_embed_transpose.  u_out [n_pos, D] dtype. */
size_t dg_soft_embed_workspace_bytes(int n_pos, int hidden, int vocab, int dtype);
int dg_soft_embed(const dg_sampler_cfg *scfg, int n_pos, int hidden, int dtype, const float *logits,
                  const float *rowstats, const void *embed_t, void *u_out, void *ws,
                  size_t ws_bytes, void *stream);

/* embed_t[d][v] = embed[v][d]: the layout copy dg_soft_embed streams. */
int dg_embed_transpose(int vocab, int hidden, int dtype, const void *embed, void *embed_t,
                       void *stream);

/* -------------------------------------------------------------- whole model */

typedef struct {
  dg_attn_cfg sliding;  /* config of the sliding-window layers */
  dg_attn_cfg global;   /* config of the global layers */
  dg_moe_cfg moe;       /* shared by every layer (layer_scalar taken per layer) */
  int n_layers;
  int global_every;     /* layer l is global iff l % global_every == global_every - 1 */
  int vocab;
  int sc_ffn;           /* self-conditioning MLP width, 0 = no self-conditioning */
  float rms_eps;        /* final norm */
  int dtype;
} dg_model_cfg;

typedef struct {
  const void *embed;         /* [vocab, D] embedding table, also the tied LM head */
  const void *embed_t;       /* [D, vocab] transposed copy (dg_embed_transpose) */
  const void *w_final_norm;  /* [D] */
  const void *sc_gate;       /* [sc_ffn, D] self-conditioning MLP (SwiGLU, no bias) */
  const void *sc_up;         /* [sc_ffn, D] */
  const void *sc_down;       /* [D, sc_ffn] */
  const dg_attn_w *attn;     /* host array [n_layers] */
  const dg_moe_w *moe;       /* host array [n_layers] */
  const float *layer_scalar; /* host array [n_layers] */
  /* Optional (NULL: the router product runs).  Host array [n_layers] of
   * device pointers, each [rows, n_experts] fp32 router logits used by that
   * layer's MoE block in place of rms(x) W_router^T, rows = the tokens of
   * the call (all canvases of a batch, back to back).  A NULL entry computes
   * that layer's logits.  Lets a caller feed the device and a reference the
   * same routing (as dg_moe_block's router_logits_in). */
  const float *const *router_logits;
} dg_model_w;

typedef struct {
  dg_kv_layer *layer;  /* host array [n_layers] */
  int n_layers;
} dg_kv_cache;

/* Per-canvas state carried between steps (all device buffers). */
typedef struct {
  int32_t *tokens;     /* [canvas_len] in: current canvas, out: next canvas */
  void *u;             /* [canvas_len, D] dtype: in: P.E of the previous step, out: this step's */
  int use_u;           /* 0 on the first step: u is not read (self-conditioning input 0) */
  uint8_t *commit;     /* [canvas_len] out */
  float *entropy;      /* [canvas_len] out */
  int32_t *n_renoised; /* [1] out: positions re-noised this step (adaptive stop when 0) */
  float *logits;       /* [canvas_len, vocab] fp32 out (optional: NULL keeps them in ws) */
  int canvas_len;
  int32_t *pred;       /* optional [canvas_len]: proposals in/out, as dg_sample_renoise's pred_inout */
  int32_t *n_changed;  /* optional [1] out: proposals changed this step (needs pred) */
  int32_t *n_nonfinite; /* optional [1] out: positions whose logits hold a NaN or +-inf */
} dg_canvas_state;

/* Workspace bytes for dg_canvas_step with canvases of up to max_canvas_tokens
 * positions (logits kept in the workspace) and dg_commit_canvas with up to
 * max_commit_tokens tokens per call (e.g. a prompt). */
size_t dg_workspace_bytes(const dg_model_cfg *cfg, int max_canvas_tokens, int max_commit_tokens);

/* One denoising step over the canvas (DiffusionGemma Technical Report review,
 * section 1 Canvas: every position of the block is predicted in parallel at
 * each step; aitrends notebook summary, attention paragraph: decode attends
 * over [committed cache | canvas] without a causal mask; sampler paragraph:
 * the entropy bound fixes confident positions and re-noises the rest; velog
 * Self-conditioning: the previous step's expected embedding feeds the next).
 * x = E[tokens] + MLP_sc(u); every layer in decode mode (attention then MoE,
 * x <- layer_scalar * (x + y)); final norm + tied head; sampler; u <- P.E for
 * the next step.  Committed rows are only read; cache rows [kv_len, kv_len +
 * canvas_len) are scratch.  No device-to-host transfer: n_renoised (and
 * n_changed, n_nonfinite) stay on the device.  Every layer's kv_len must be
 * equal; the capacity must hold kv_len + canvas_len (DG_ERR_CAPACITY). */
int dg_canvas_step(const dg_model_cfg *cfg, const dg_model_w *w, const dg_kv_cache *kv,
                   dg_canvas_state *state, const dg_sampler_cfg *scfg, void *ws, size_t ws_bytes,
                   void *stream);

/* n_canvas independent canvases (separate sequences, each with its own KV
 * cache) in one forward: the projections, experts, head and P.E run over all
 * n_canvas * canvas_len rows at once, so every weight is streamed once for
 * all of them; norm/RoPE, the cache writes, attention and the sampler run
 * per canvas.  kv[b] and scfg[b] belong to canvas b (arrays of n_canvas);
 * the buffers of st hold the canvases back to back (tokens, commit,
 * entropy, pred: [n_canvas * canvas_len]; u: [n_canvas * canvas_len, D];
 * logits: [n_canvas * canvas_len, vocab]; n_renoised, n_changed:
 * [n_canvas]); st->canvas_len is one canvas's length.  Each canvas's result
 * is the one dg_canvas_step gives for it alone.  Workspace:
 * dg_workspace_bytes_batch. */
int dg_canvas_step_batch(const dg_model_cfg *cfg, const dg_model_w *w, const dg_kv_cache *kv,
                         dg_canvas_state *st, const dg_sampler_cfg *scfg, int n_canvas, void *ws, size_t ws_bytes,
                         void *stream);
size_t dg_workspace_bytes_batch(const dg_model_cfg *cfg, int n_canvas, int canvas_len);

/* Commit (encode): run the n_tok final tokens causally through the stack and
 * append every layer's K/V at [kv_len, kv_len + n_tok); the last layer stops
 * after its K/V (aitrends attention paragraph: work after the last layer is
 * skipped).  Every layer's kv_len is advanced by n_tok on the host. */
int dg_commit_canvas(const dg_model_cfg *cfg, const dg_model_w *w, dg_kv_cache *kv,
                     const int32_t *tokens, int n_tok, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------ profiling */

/* Optional kernel timer.  The caller creates `capacity` pairs of hipEvent_t
 * and attaches the record with dg_set_kernel_timer; while attached, the
 * library records start[i] / stop[i] on the launching stream around every
 * `every`-th launch of the selected kernel class (0 or 1: each launch) and
 * increments `count` (launches past `capacity` are not timed).  `seen`
 * counts the launches of the class since it was set (the caller sets it to
 * 0).  Each recorded event adds a few microseconds between kernels, so a
 * caller timing a whole step samples launches.  The attachment is per host
 * thread; NULL detaches.  This pointer is the library's only state and is
 * off by default. */
enum {
  DG_KT_NONE = 0,
  DG_KT_MOE_GATEUP = 1,  /* grouped expert gate/up product with the SwiGLU epilogue */
  DG_KT_MOE_DOWN = 2,    /* grouped expert down product */
  DG_KT_LM_HEAD = 3,     /* tied-head product */
  DG_KT_ATTN = 4,        /* attention core */
  DG_KT_SOFT_EMBED = 5,  /* P.E product */
  DG_KT_QKV = 6,         /* fused Q|K|V projection */
  DG_KT_OPROJ = 7        /* output projection (with its split-K partials) */
};
typedef struct {
  void **start;   /* hipEvent_t[capacity] */
  void **stop;    /* hipEvent_t[capacity] */
  int capacity;
  int count;
  int kernel;     /* DG_KT_* */
  int every;      /* record every `every`-th launch (0 or 1: each) */
  int seen;       /* launches of the class seen while attached */
} dg_kernel_timer;

void dg_set_kernel_timer(dg_kernel_timer *timer);

/* ----------------------------------------------------------- roof probes */

/* Not operations of the pages: two probes of the device's attainable roofs,
 * against which the kernels' roofline fractions are reported beside the
 * datasheet figures.  Both are enqueued on `stream` and produce results the
 * caller checks exactly.
 *
 * dg_probe_hbm_read: n_groups workgroups of 256 threads read `bytes` (a
 * multiple of 16, buf 16-byte aligned) once with 16-byte non-temporal loads,
 * sixteen in flight per thread, each workgroup its own contiguous span.
 * sink[g] (uint32, n_groups of them, device) receives the wrapping sum of the
 * 32-bit words workgroup g read; the sum over g is the wrapping sum of every
 * word of the buffer.  A buffer well beyond the last-level cache measures
 * HBM.  DG_ERR_NULL / DG_ERR_SHAPE (n_groups outside [1, 65536], bytes or buf
 * misaligned) before any HIP call.
 *
 * dg_probe_mfma_bf16: n_groups workgroups of four waves; each wave runs
 * `iters` rounds (a multiple of 16) of 16 independent 16x16x32 bf16 MFMAs
 * with every A element a and every B element b (both rounded to bf16).
 * sink[4g + w] (float, device) = 16 * iters * 32 * a * b for wave w of
 * workgroup g, exact when every partial sum is representable.
 * dg_probe_mfma_flops gives the launch's floating-point operations
 * (2 * 16 * 16 * 32 per MFMA), 0 for invalid arguments. */
int dg_probe_hbm_read(const void *buf, size_t bytes, uint32_t *sink, int n_groups, void *stream);
int dg_probe_mfma_bf16(int iters, float a, float b, float *sink, int n_groups, void *stream);
long long dg_probe_mfma_flops(int iters, int n_groups);

/* ------------------------------------------------------------------ misc */

/* RMSNorm rows (aitrends rms code): y = w * x * sqrt(D) / (||x|| + eps).
 * x, y [n, D] dtype, w [D] dtype.  y may alias x. */
int dg_rmsnorm(int n, int hidden, float eps, int dtype, const void *x, const void *w, void *y,
               void *stream);

const char *dg_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* DGSTEP_H */
