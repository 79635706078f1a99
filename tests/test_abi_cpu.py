"""C-ABI checks that need no GPU: the library loads, exports every declared
entry point, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dgstep.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_entry_point():
    L = B.lib()
    names = declared_functions()
    assert len(names) >= 17
    for n in ("dg_canvas_step", "dg_attn_layer", "dg_moe_block", "dg_sample_renoise", "dg_commit_canvas"):
        assert n in names
    for n in names:
        assert hasattr(L, n), n


STRUCTS = {
    "dg_attn_cfg": B.AttnCfg, "dg_attn_w": B.AttnW, "dg_kv_layer": B.KVLayer, "dg_moe_cfg": B.MoeCfg,
    "dg_moe_w": B.MoeW, "dg_sampler_cfg": B.SamplerCfg, "dg_model_cfg": B.ModelCfg, "dg_model_w": B.ModelW,
    "dg_kv_cache": B.KVCache, "dg_canvas_state": B.CanvasState, "dg_kernel_timer": B.KernelTimer,
}
C_NAME = {"global_": "global"}   # binding field names that differ from the header's


def test_struct_layouts_match_header(tmp_path):
    """Every ctypes mirror of a header struct has the header's size and field
    offsets, as a C compiler lays them out (the header is compiled as C)."""
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "dgstep.h"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'  printf("{cname} . %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {C_NAME.get(f, f)}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {(a, b): int(c) for a, b, c in (ln.split() for ln in out if ln)}
    for cname, py in STRUCTS.items():
        assert got[(cname, ".")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_status_strings():
    for s in range(-7, 1):
        assert B.dg_status_string(s) != "unknown status"
    assert B.dg_status_string(-99) == "unknown status"


def _attn_c(**over):
    cfg = synth.sliding_cfg()
    cfg.update(over)
    return B.attn_cfg_c(cfg)


def test_attn_validation_codes():
    L = B.lib()
    w = B.AttnW(*(ctypes.c_void_p(256) for _ in range(7)))
    kv = B.KVLayer(ctypes.c_void_p(256), ctypes.c_void_p(256), 4096, 2048, 0)
    x = ctypes.c_void_p(256)
    ws = ctypes.c_void_p(256)
    call = lambda c, n=256, causal=0, kvv=kv, wsb=1 << 40, xx=x, ww=w: L.dg_attn_layer(
        ctypes.byref(c), ctypes.byref(ww), ctypes.byref(kvv), n, causal, xx, ws, wsb, None)
    assert call(_attn_c(), xx=None) == -1
    assert call(_attn_c(), ww=B.AttnW()) == -1
    assert call(_attn_c(head_dim=96)) == -3
    assert call(_attn_c(hidden=100)) == -2
    assert call(_attn_c(n_q_heads=12, n_kv_heads=8)) == -2
    assert call(_attn_c(), n=-1) == -2
    assert call(_attn_c(), causal=2) == -2
    assert call(_attn_c(), wsb=1024) == -4
    full = B.KVLayer(ctypes.c_void_p(256), ctypes.c_void_p(256), 2104, 2048, 0)
    assert call(_attn_c(), causal=1, kvv=full) == -7
    c = _attn_c()
    c.dtype = 7
    assert call(c) == -5
    # keys rebuilt from values only where W_v = W_k and V is unit-RMS (global layers), never in a ring
    vo = B.KVLayer(ctypes.c_void_p(256), ctypes.c_void_p(256), 4096, 2048, 0, 1)
    assert call(_attn_c(), kvv=vo) == -3
    g = B.attn_cfg_c(synth.global_cfg())
    vo_ring = B.KVLayer(ctypes.c_void_p(256), ctypes.c_void_p(256), 4096, 2048, 1, 1)
    assert call(g, kvv=vo_ring) == -3
    bad = B.KVLayer(ctypes.c_void_p(256), ctypes.c_void_p(256), 4096, 2048, 0, 2)
    assert call(g, kvv=bad) == -2
    # zero tokens is a no-op
    assert call(_attn_c(), n=0) == 0


def test_moe_validation_codes():
    L = B.lib()
    m = synth.moe_cfg(2816, 128, 8, 704, 704)
    w = B.MoeW(*(ctypes.c_void_p(256) for _ in range(8)))
    call = lambda c, n=256, ww=w, rl=None, wsb=1 << 40: L.dg_moe_block(
        ctypes.byref(c), ctypes.byref(ww), n, ctypes.c_void_p(256), rl, None, None, ctypes.c_void_p(256), wsb, None)
    assert call(B.moe_cfg_c(dict(m, top_k=9))) == -2
    assert call(B.moe_cfg_c(dict(m, n_experts=300))) == -2
    assert call(B.moe_cfg_c(dict(m, ffn=700))) == -2
    wr = B.MoeW(*(ctypes.c_void_p(256) for _ in range(8)))
    wr.w_router = None
    assert call(B.moe_cfg_c(m), ww=wr) == -1
    assert call(B.moe_cfg_c(m), wsb=16) == -4
    assert call(B.moe_cfg_c(m), n=0) == 0


def test_sampler_validation_codes():
    L = B.lib()
    p = ctypes.c_void_p(256)
    call = lambda s, n=256, ldt=0, wsb=1 << 30: L.dg_sample_renoise(
        ctypes.byref(s), n, p, ldt, p, p, p, None, p, None, None, None, p, wsb, None)
    assert call(B.sampler_cfg_c(synth.sampler_cfg(262144, t_max=0.0))) == -2
    assert call(B.sampler_cfg_c(synth.sampler_cfg(262143))) == -2
    assert call(B.sampler_cfg_c(synth.sampler_cfg(262144)), ldt=3) == -5
    assert call(B.sampler_cfg_c(synth.sampler_cfg(262144)), wsb=8) == -4
    assert L.dg_sample_renoise(None, 1, p, 0, p, p, p, None, p, None, None, None, p, 1 << 30, None) == -1
    bad = B.sampler_cfg_c(synth.sampler_cfg(262144))
    bad.commit_rule = 2
    assert call(bad) == -3
    bad = B.sampler_cfg_c(synth.sampler_cfg(262144))
    bad.token_rule = 5
    assert call(bad) == -3
    # the sorted cumulative rule ranks at most 4096 positions in one workgroup
    big = B.sampler_cfg_c(dict(synth.sampler_cfg(262144), commit_rule="sorted_cumulative"))
    assert call(big, n=4097) == -2


def test_sampler_noalloc_validation_codes():
    """The allocation-free sampler rejects what the built-in scratch cannot
    hold (and bad arguments) on the host, before any HIP call."""
    L = B.lib()
    p = ctypes.c_void_p(256)
    cap = L.dg_sample_noalloc_max_bytes()
    assert 0 < cap <= 8 << 20
    call = lambda s, n, ldt=0: L.dg_sample_renoise_noalloc(ctypes.byref(s), n, p, ldt, p, p, p, None, p, None,
                                                          None, None, None)
    s = B.sampler_cfg_c(synth.sampler_cfg(262144))
    # 16 vocabulary slices per row at V = 262144: 8192 rows fit, 8193 do not
    assert L.dg_sample_workspace_bytes(8192, 262144) <= cap < L.dg_sample_workspace_bytes(8193, 262144)
    assert call(s, 8193) == -4
    assert call(s, 100000) == -4
    assert call(s, 8, ldt=3) == -5
    assert call(s, -1) == -2
    assert L.dg_sample_renoise_noalloc(None, 1, p, 0, p, p, p, None, p, None, None, None, None) == -1
    assert L.dg_sample_renoise_noalloc(ctypes.byref(s), 1, None, 0, p, p, p, None, p, None, None, None, None) == -1


def test_workspace_queries_grow_with_tokens():
    L = B.lib()
    c = _attn_c()
    a = L.dg_attn_workspace_bytes(ctypes.byref(c), 64)
    b = L.dg_attn_workspace_bytes(ctypes.byref(c), 256)
    assert 0 < a < b
    m = B.model_cfg_c(synth.full_model_cfg())
    s1 = L.dg_workspace_bytes(ctypes.byref(m), 256, 0)
    s2 = L.dg_workspace_bytes(ctypes.byref(m), 256, 4096)
    assert 0 < s1 <= s2
    # canvas workspace holds the fp32 logits of the 262,144-wide head
    assert s1 > 256 * 262144 * 4
    bad = B.model_cfg_c(dict(synth.full_model_cfg(), n_layers=0))
    assert L.dg_workspace_bytes(ctypes.byref(bad), 256, 0) == 0


def test_model_entry_points_validate():
    L = B.lib()
    m = B.model_cfg_c(synth.full_model_cfg())
    s = B.sampler_cfg_c(synth.sampler_cfg(262144))
    assert L.dg_canvas_step(ctypes.byref(m), None, None, None, ctypes.byref(s), None, 0, None) == -1
    assert L.dg_commit_canvas(ctypes.byref(m), None, None, None, 256, None, 0, None) == -1
    mm = B.model_cfg_c(dict(synth.full_model_cfg(), dtype="f32"))   # layer dtypes disagree
    assert L.dg_canvas_step(ctypes.byref(mm), None, None, None, ctypes.byref(s), None, 0, None) == -5


def test_fp8_expert_validation_codes():
    L = B.lib()
    m = synth.moe_cfg(2816, 128, 8, 704, 704)
    w8 = B.MoeW(*(ctypes.c_void_p(256) for _ in range(len(B.MOE_W_NAMES))))
    call = lambda c, ww=w8: L.dg_moe_block(ctypes.byref(c), ctypes.byref(ww), 256, ctypes.c_void_p(256), None,
                                           None, None, ctypes.c_void_p(256), 1 << 40, None)
    bad = B.moe_cfg_c(m)
    bad.expert_format = 5
    assert call(bad) == -3
    assert call(B.moe_cfg_c(dict(m, dtype="f32", expert_format="fp8_e4m3"))) == -3
    no_scale = B.MoeW(*(ctypes.c_void_p(256) for _ in range(len(B.MOE_W_NAMES))))
    no_scale.s_down = None
    assert call(B.moe_cfg_c(dict(m, expert_format="fp8_e4m3")), ww=no_scale) == -1


def test_quantize_fp8_validation_codes():
    L = B.lib()
    p = ctypes.c_void_p(256)
    assert L.dg_quantize_fp8(7, p, 4, 64, p, p, None) == -5
    assert L.dg_quantize_fp8(1, p, -1, 64, p, p, None) == -2
    assert L.dg_quantize_fp8(1, p, 4, 0, p, p, None) == -2
    assert L.dg_quantize_fp8(1, None, 4, 64, p, p, None) == -1
    assert L.dg_quantize_fp8(1, p, 0, 64, None, None, None) == 0


def test_ring_cache_validation_codes():
    L = B.lib()
    w = B.AttnW(*(ctypes.c_void_p(256) for _ in range(7)))
    x = ctypes.c_void_p(256)
    call = lambda c, kvv, n=256: L.dg_attn_layer(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kvv), n, 0, x,
                                                 ctypes.c_void_p(256), 1 << 40, None)
    ring = lambda cap, kvl: B.KVLayer(ctypes.c_void_p(256), ctypes.c_void_p(256), cap, kvl, 1)
    # window 1024 + 256 tokens: 1280 rows; kv_len may run far past the ring
    assert call(_attn_c(), ring(1280, 9000), n=0) == 0
    assert call(_attn_c(), ring(1272, 100)) == -3              # not a multiple of 32
    assert call(_attn_c(), ring(1248, 100)) == -7              # window + tokens do not fit
    g = synth.global_cfg()
    assert call(B.attn_cfg_c(g), ring(1280, 100)) == -3        # rings are for sliding layers
    bad = ring(1280, 100)
    bad.ring = 2
    assert call(_attn_c(), bad) == -2


def test_probe_validation_codes():
    L = B.lib()
    p = ctypes.c_void_p(256)
    assert L.dg_probe_hbm_read(None, 1024, p, 8, None) == -1
    assert L.dg_probe_hbm_read(p, 1024, None, 8, None) == -1
    assert L.dg_probe_hbm_read(p, 1000, p, 8, None) == -2          # bytes not a multiple of 16
    assert L.dg_probe_hbm_read(ctypes.c_void_p(264), 1024, p, 8, None) == -2   # buffer not 16-byte aligned
    assert L.dg_probe_hbm_read(p, 1024, p, 0, None) == -2
    assert L.dg_probe_hbm_read(p, 1024, p, 65537, None) == -2
    assert L.dg_probe_hbm_read(p, 0, p, 8, None) == 0               # nothing to read: no launch
    assert L.dg_probe_mfma_bf16(16, 1.0, 1.0, None, 8, None) == -1
    assert L.dg_probe_mfma_bf16(24, 1.0, 1.0, p, 8, None) == -2     # rounds not a multiple of 16
    assert L.dg_probe_mfma_bf16(-16, 1.0, 1.0, p, 8, None) == -2
    assert L.dg_probe_mfma_bf16(16, 1.0, 1.0, p, 0, None) == -2
    assert B.dg_probe_mfma_flops(32, 3) == 3 * 4 * 32 * 16 * (2 * 16 * 16 * 32)
    assert B.dg_probe_mfma_flops(24, 3) == 0 and B.dg_probe_mfma_flops(32, 0) == 0
