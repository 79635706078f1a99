/* Host-side argument validation of every libdgstep entry point, for a build
 * of the library whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Every call below must be rejected (or, for
 * the size queries, answered) on the host before any HIP call, so the
 * program needs no GPU.  Host records (configs, per-layer arrays, cache and
 * state records) are real host memory; device pointers are placeholders
 * that the library must never dereference on the host.
 * Exit status 0 when every return code is the expected one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dgstep.h"

static int n_checks = 0, n_fail = 0;

static void expect(const char *what, long got, long want) {
  ++n_checks;
  if (got != want) {
    ++n_fail;
    printf("FAIL %s: got %ld, want %ld\n", what, got, want);
  }
}

#define DEV ((void *)256)

static dg_attn_cfg sliding(void) {
  dg_attn_cfg c;
  memset(&c, 0, sizeof(c));
  c.hidden = 2816;
  c.n_q_heads = 16;
  c.n_kv_heads = 8;
  c.head_dim = 256;
  c.layer_type = 0;
  c.window = 1024;
  c.rope_base = 10000.f;
  c.rotary_factor = 1.f;
  c.rms_eps = 1e-6f;
  c.dtype = DG_BF16;
  return c;
}

static dg_attn_cfg global_cfg(void) {
  dg_attn_cfg c = sliding();
  c.n_kv_heads = 2;
  c.head_dim = 512;
  c.layer_type = 1;
  c.shared_kv = 1;
  c.v_unit_rms = 1;
  c.rope_base = 1e6f;
  c.rotary_factor = 0.25f;
  return c;
}

static dg_moe_cfg moe(void) {
  dg_moe_cfg c;
  memset(&c, 0, sizeof(c));
  c.hidden = 2816;
  c.n_experts = 128;
  c.top_k = 8;
  c.ffn = 704;
  c.shared_ffn = 704;
  c.route_scale = 1.f;
  c.rms_eps = 1e-6f;
  c.layer_scalar = 1.f;
  c.dtype = DG_BF16;
  return c;
}

static dg_sampler_cfg sampler(void) {
  dg_sampler_cfg c;
  memset(&c, 0, sizeof(c));
  c.vocab = 262144;
  c.tau = 6.2f;
  c.t_max = 1.f;
  c.t_min = 1.f;
  c.n_steps = 48;
  c.seed = 1;
  return c;
}

static void check_attention(void) {
  dg_attn_cfg c = sliding();
  dg_attn_w w;
  void **wp = (void **)&w;
  for (size_t i = 0; i < sizeof(w) / sizeof(void *); ++i) wp[i] = DEV;
  dg_kv_layer kv = {DEV, DEV, 4096, 2048, 0};
  expect("attn ws bytes > 0", dg_attn_workspace_bytes(&c, 256) > 0, 1);
  expect("attn ws bytes null cfg", (long)dg_attn_workspace_bytes(NULL, 256), 0);
  expect("attn null cfg", dg_attn_layer(NULL, &w, &kv, 256, 0, DEV, DEV, 1ull << 40, NULL), DG_ERR_NULL);
  expect("attn null x", dg_attn_layer(&c, &w, &kv, 256, 0, NULL, DEV, 1ull << 40, NULL), DG_ERR_NULL);
  expect("attn ws small", dg_attn_layer(&c, &w, &kv, 256, 0, DEV, DEV, 1024, NULL), DG_ERR_WORKSPACE);
  expect("attn causal 2", dg_attn_layer(&c, &w, &kv, 256, 2, DEV, DEV, 1ull << 40, NULL), DG_ERR_SHAPE);
  expect("attn n < 0", dg_attn_layer(&c, &w, &kv, -1, 0, DEV, DEV, 1ull << 40, NULL), DG_ERR_SHAPE);
  expect("attn n = 0", dg_attn_layer(&c, &w, &kv, 0, 0, DEV, DEV, 1ull << 40, NULL), DG_OK);
  dg_kv_layer full = {DEV, DEV, 2104, 2048, 0};
  expect("attn capacity", dg_attn_layer(&c, &w, &full, 256, 1, DEV, DEV, 1ull << 40, NULL), DG_ERR_CAPACITY);
  dg_kv_layer ring = {DEV, DEV, 1112, 2048, 1};   /* a multiple of 8, not of 32 */
  expect("attn ring capacity %32", dg_attn_layer(&c, &w, &ring, 256, 1, DEV, DEV, 1ull << 40, NULL),
         DG_ERR_UNSUPPORTED);
  dg_attn_cfg bad = c;
  bad.head_dim = 96;
  expect("attn head_dim 96", dg_attn_layer(&bad, &w, &kv, 256, 0, DEV, DEV, 1ull << 40, NULL), DG_ERR_UNSUPPORTED);
  bad = c;
  bad.dtype = 9;
  expect("attn dtype", dg_attn_layer(&bad, &w, &kv, 256, 0, DEV, DEV, 1ull << 40, NULL), DG_ERR_DTYPE);
  bad = c;
  bad.rope_base = -1.f;
  expect("attn rope base", dg_attn_layer(&bad, &w, &kv, 256, 0, DEV, DEV, 1ull << 40, NULL), DG_ERR_SHAPE);
  w.w_v = NULL;
  expect("attn w_v null (not shared)", dg_attn_layer(&c, &w, &kv, 256, 0, DEV, DEV, 1ull << 40, NULL), DG_ERR_NULL);
}

static void check_moe(void) {
  dg_moe_cfg c = moe();
  dg_moe_w w;
  memset(&w, 0, sizeof(w));
  w.w_in_norm = w.w_router = w.w_gate = w.w_up = w.w_down = w.ws_gate = w.ws_up = w.ws_down = DEV;
  expect("moe ws bytes > 0", dg_moe_workspace_bytes(&c, 256) > 0, 1);
  expect("moe null w", dg_moe_block(&c, NULL, 256, DEV, NULL, NULL, NULL, DEV, 1ull << 40, NULL), DG_ERR_NULL);
  expect("moe ws small", dg_moe_block(&c, &w, 256, DEV, NULL, NULL, NULL, DEV, 64, NULL), DG_ERR_WORKSPACE);
  dg_moe_cfg bad = c;
  bad.top_k = 9;
  expect("moe top_k 9", dg_moe_block(&bad, &w, 256, DEV, NULL, NULL, NULL, DEV, 1ull << 40, NULL), DG_ERR_SHAPE);
  bad = c;
  bad.expert_format = DG_EXPERTS_FP8_E4M3;
  expect("moe fp8 without scales", dg_moe_block(&bad, &w, 256, DEV, NULL, NULL, NULL, DEV, 1ull << 40, NULL),
         DG_ERR_NULL);
  bad.dtype = DG_F32;
  expect("moe fp8 with f32", dg_moe_block(&bad, &w, 256, DEV, NULL, NULL, NULL, DEV, 1ull << 40, NULL),
         DG_ERR_UNSUPPORTED);
  w.w_router = NULL;
  expect("moe no router, no logits", dg_moe_block(&c, &w, 256, DEV, NULL, NULL, NULL, DEV, 1ull << 40, NULL),
         DG_ERR_NULL);
  expect("fp8 quantise rows < 0", dg_quantize_fp8(DG_BF16, DEV, -1, 64, DEV, DEV, NULL), DG_ERR_SHAPE);
  expect("fp8 quantise dtype", dg_quantize_fp8(7, DEV, 4, 64, DEV, DEV, NULL), DG_ERR_DTYPE);
  expect("fp8 quantise rows 0", dg_quantize_fp8(DG_BF16, DEV, 0, 64, DEV, DEV, NULL), DG_OK);
}

static void check_sampler_head(void) {
  dg_sampler_cfg s = sampler();
  expect("sample ws bytes > 0", dg_sample_workspace_bytes(256, 262144) > 0, 1);
  expect("sample null cfg", dg_sample_renoise(NULL, 8, DEV, 0, DEV, DEV, DEV, NULL, DEV, NULL, NULL, NULL, DEV,
                                              1ull << 30, NULL), DG_ERR_NULL);
  expect("sample ws small", dg_sample_renoise(&s, 8, DEV, 0, DEV, DEV, DEV, NULL, DEV, NULL, NULL, NULL, DEV, 8,
                                              NULL), DG_ERR_WORKSPACE);
  dg_sampler_cfg bad = s;
  bad.vocab = 262143;
  expect("sample vocab %8", dg_sample_renoise(&bad, 8, DEV, 0, DEV, DEV, DEV, NULL, DEV, NULL, NULL, NULL, DEV,
                                              1ull << 30, NULL), DG_ERR_SHAPE);
  bad = s;
  bad.t_max = 0.f;
  expect("sample t_max 0", dg_sample_renoise(&bad, 8, DEV, 0, DEV, DEV, DEV, NULL, DEV, NULL, NULL, NULL, DEV,
                                             1ull << 30, NULL), DG_ERR_SHAPE);
  bad = s;
  bad.commit_rule = 5;
  expect("sample commit rule", dg_sample_renoise(&bad, 8, DEV, 0, DEV, DEV, DEV, NULL, DEV, NULL, NULL, NULL, DEV,
                                                 1ull << 30, NULL), DG_ERR_UNSUPPORTED);
  expect("noalloc max bytes", dg_sample_noalloc_max_bytes() > 0, 1);
  expect("noalloc too many rows", dg_sample_renoise_noalloc(&s, 8193, DEV, 0, DEV, DEV, DEV, NULL, DEV, NULL, NULL,
                                                            NULL, NULL), DG_ERR_WORKSPACE);
  expect("noalloc null logits", dg_sample_renoise_noalloc(&s, 8, NULL, 0, DEV, DEV, DEV, NULL, DEV, NULL, NULL, NULL,
                                                          NULL), DG_ERR_NULL);
  expect("noise null", dg_canvas_noise(8, 64, 1, 0, NULL, NULL), DG_ERR_NULL);
  expect("noise vocab", dg_canvas_noise(8, 0, 1, 0, DEV, NULL), DG_ERR_SHAPE);
  expect("head ws bytes", dg_lm_head_workspace_bytes(256, 2816, DG_BF16) > 0, 1);
  expect("head hidden %64", dg_lm_head(256, 100, 262144, 1e-6f, DG_BF16, DEV, DEV, DEV, DEV, DEV, 1ull << 30, NULL),
         DG_ERR_SHAPE);
  expect("head null", dg_lm_head(256, 2816, 262144, 1e-6f, DG_BF16, NULL, DEV, DEV, DEV, DEV, 1ull << 30, NULL),
         DG_ERR_NULL);
  expect("soft ws bytes", dg_soft_embed_workspace_bytes(256, 2816, 262144, DG_BF16) > 0, 1);
  expect("soft null", dg_soft_embed(&s, 256, 2816, DG_BF16, NULL, DEV, DEV, DEV, DEV, 1ull << 40, NULL),
         DG_ERR_NULL);
  expect("soft ws small", dg_soft_embed(&s, 256, 2816, DG_BF16, DEV, DEV, DEV, DEV, DEV, 16, NULL),
         DG_ERR_WORKSPACE);
  expect("transpose dtype", dg_embed_transpose(64, 64, 5, DEV, DEV, NULL), DG_ERR_DTYPE);
  expect("rmsnorm hidden %8", dg_rmsnorm(4, 12, 1e-6f, DG_BF16, DEV, DEV, DEV, NULL), DG_ERR_SHAPE);
  expect("status ok", dg_status_string(DG_OK) != NULL, 1);
  for (int st = -7; st <= 0; ++st) expect("status string", strcmp(dg_status_string(st), "unknown status") != 0, 1);
  expect("status unknown", strcmp(dg_status_string(-99), "unknown status"), 0);
}

enum { L = 6 };

static void check_model(void) {
  dg_model_cfg c;
  memset(&c, 0, sizeof(c));
  c.sliding = sliding();
  c.global = global_cfg();
  c.moe = moe();
  c.n_layers = L;
  c.global_every = 6;
  c.vocab = 262144;
  c.sc_ffn = 704;
  c.rms_eps = 1e-6f;
  c.dtype = DG_BF16;
  dg_attn_w aw[L];
  dg_moe_w mw[L];
  float ls[L];
  dg_kv_layer kl[L];
  for (int l = 0; l < L; ++l) {
    void **p = (void **)&aw[l];
    for (size_t i = 0; i < sizeof(dg_attn_w) / sizeof(void *); ++i) p[i] = DEV;
    memset(&mw[l], 0, sizeof(dg_moe_w));
    mw[l].w_in_norm = mw[l].w_router = mw[l].w_gate = mw[l].w_up = mw[l].w_down = DEV;
    mw[l].ws_gate = mw[l].ws_up = mw[l].ws_down = DEV;
    ls[l] = 1.f;
    kl[l].k = kl[l].v = DEV;
    kl[l].capacity = 8192;
    kl[l].kv_len = 4096;
    kl[l].ring = 0;
  }
  dg_model_w w;
  memset(&w, 0, sizeof(w));
  w.embed = w.embed_t = w.w_final_norm = w.sc_gate = w.sc_up = w.sc_down = DEV;
  w.attn = aw;
  w.moe = mw;
  w.layer_scalar = ls;
  dg_kv_cache kv = {kl, L};
  dg_canvas_state st;
  memset(&st, 0, sizeof(st));
  st.tokens = st.n_renoised = DEV;
  st.u = DEV;
  st.commit = DEV;
  st.entropy = DEV;
  st.canvas_len = 256;
  dg_sampler_cfg s = sampler();
  size_t ws = dg_workspace_bytes(&c, 256, 4096);
  expect("model ws bytes > 0", ws > 0, 1);
  expect("batch ws bytes > 0", dg_workspace_bytes_batch(&c, 8, 256) > 0, 1);
  expect("step ws small", dg_canvas_step(&c, &w, &kv, &st, &s, DEV, 64, NULL), DG_ERR_WORKSPACE);
  expect("step null state", dg_canvas_step(&c, &w, &kv, NULL, &s, DEV, ws, NULL), DG_ERR_NULL);
  expect("batch 0 canvases", dg_canvas_step_batch(&c, &w, &kv, &st, &s, 0, DEV, ws, NULL), DG_ERR_SHAPE);
  dg_sampler_cfg sv = s;
  sv.vocab = 4096;
  expect("step sampler vocab", dg_canvas_step(&c, &w, &kv, &st, &sv, DEV, ws, NULL), DG_ERR_SHAPE);
  kl[3].kv_len = 4000;
  expect("step uneven kv_len", dg_canvas_step(&c, &w, &kv, &st, &s, DEV, ws, NULL), DG_ERR_SHAPE);
  kl[3].kv_len = 4096;
  kl[2].capacity = 4200;
  expect("step capacity", dg_canvas_step(&c, &w, &kv, &st, &s, DEV, ws, NULL), DG_ERR_CAPACITY);
  expect("commit capacity", dg_commit_canvas(&c, &w, &kv, DEV, 256, DEV, ws, NULL), DG_ERR_CAPACITY);
  kl[2].capacity = 8192;
  mw[4].w_router = NULL;
  expect("step layer 4 router null", dg_canvas_step(&c, &w, &kv, &st, &s, DEV, ws, NULL), DG_ERR_NULL);
  const float *rl[L] = {0};
  rl[4] = (const float *)DEV;
  w.router_logits = rl;
  expect("step ws small (injected router)", dg_canvas_step(&c, &w, &kv, &st, &s, DEV, 64, NULL), DG_ERR_WORKSPACE);
  w.router_logits = NULL;
  mw[4].w_router = DEV;
  aw[5].w_o = NULL;
  expect("step layer 5 w_o null", dg_canvas_step(&c, &w, &kv, &st, &s, DEV, ws, NULL), DG_ERR_NULL);
  aw[5].w_o = DEV;
  expect("commit n < 0", dg_commit_canvas(&c, &w, &kv, DEV, -5, DEV, ws, NULL), DG_ERR_SHAPE);
  expect("commit n = 0", dg_commit_canvas(&c, &w, &kv, DEV, 0, DEV, ws, NULL), DG_OK);
  dg_model_cfg bad = c;
  bad.global.hidden = 2880;
  expect("model hidden mismatch", dg_canvas_step(&bad, &w, &kv, &st, &s, DEV, ws, NULL), DG_ERR_SHAPE);
  bad = c;
  bad.moe.dtype = DG_F32;
  expect("model dtype mismatch", dg_canvas_step(&bad, &w, &kv, &st, &s, DEV, ws, NULL), DG_ERR_DTYPE);
  dg_set_kernel_timer(NULL);
}

int main(void) {
  check_attention();
  check_moe();
  check_sampler_head();
  check_model();
  printf("%d checks, %d failed\n", n_checks, n_fail);
  return n_fail ? 1 : 0;
}
