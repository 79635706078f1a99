"""Thin Python binding over libdgstep's C ABI (argument marshalling only).

Every computation runs in the HIP kernels of libdgstep.so; PyTorch provides
device memory and the current stream.  Functions carry the C entry points'
names.  Loading fails loudly when the library has not been built.
"""
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdgstep.so")

DG_F32, DG_BF16 = 0, 1
_DT = {"f32": DG_F32, "bf16": DG_BF16}
STATUS = {0: "DG_OK", -1: "DG_ERR_NULL", -2: "DG_ERR_SHAPE", -3: "DG_ERR_UNSUPPORTED",
          -4: "DG_ERR_WORKSPACE", -5: "DG_ERR_DTYPE", -6: "DG_ERR_HIP", -7: "DG_ERR_CAPACITY"}

c_int, c_float, c_size, c_void = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class DGError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


class AttnCfg(ctypes.Structure):
    _fields_ = [("hidden", c_int), ("n_q_heads", c_int), ("n_kv_heads", c_int), ("head_dim", c_int),
                ("layer_type", c_int), ("window", c_int), ("shared_kv", c_int), ("v_unit_rms", c_int),
                ("rope_base", c_float), ("rotary_factor", c_float), ("rms_eps", c_float), ("dtype", c_int)]


class AttnW(ctypes.Structure):
    _fields_ = [(n, c_void) for n in ("w_in_norm", "w_q", "w_k", "w_v", "w_o", "q_norm", "k_norm")]


class KVLayer(ctypes.Structure):
    _fields_ = [("k", c_void), ("v", c_void), ("capacity", c_int), ("kv_len", c_int), ("ring", c_int),
                ("v_only", c_int)]


class MoeCfg(ctypes.Structure):
    _fields_ = [("hidden", c_int), ("n_experts", c_int), ("top_k", c_int), ("ffn", c_int),
                ("shared_ffn", c_int), ("route_scale", c_float), ("rms_eps", c_float),
                ("layer_scalar", c_float), ("dtype", c_int), ("expert_format", c_int)]


MOE_W_NAMES = ("w_in_norm", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
               "s_gate", "s_up", "s_down", "ss_gate", "ss_up", "ss_down")
EXPERT_MATRICES = ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")
_EF = {"dtype": 0, "fp8_e4m3": 1}


class MoeW(ctypes.Structure):
    _fields_ = [(n, c_void) for n in MOE_W_NAMES]


class SamplerCfg(ctypes.Structure):
    _fields_ = [("vocab", c_int), ("tau", c_float), ("t_max", c_float), ("t_min", c_float),
                ("n_steps", c_int), ("step", c_int), ("canvas_idx", ctypes.c_uint32),
                ("seed", ctypes.c_uint64), ("final_step", c_int), ("commit_rule", c_int), ("token_rule", c_int)]


COMMIT_RULES = {"entropy": 0, "sorted_cumulative": 1}
TOKEN_RULES = {"argmax": 0, "gumbel": 1}


class ModelCfg(ctypes.Structure):
    _fields_ = [("sliding", AttnCfg), ("global_", AttnCfg), ("moe", MoeCfg), ("n_layers", c_int),
                ("global_every", c_int), ("vocab", c_int), ("sc_ffn", c_int), ("rms_eps", c_float),
                ("dtype", c_int)]


class ModelW(ctypes.Structure):
    _fields_ = [("embed", c_void), ("embed_t", c_void), ("w_final_norm", c_void), ("sc_gate", c_void),
                ("sc_up", c_void), ("sc_down", c_void), ("attn", ctypes.POINTER(AttnW)),
                ("moe", ctypes.POINTER(MoeW)), ("layer_scalar", ctypes.POINTER(c_float)),
                ("router_logits", ctypes.POINTER(c_void))]


class KVCache(ctypes.Structure):
    _fields_ = [("layer", ctypes.POINTER(KVLayer)), ("n_layers", c_int)]


class CanvasState(ctypes.Structure):
    _fields_ = [("tokens", c_void), ("u", c_void), ("use_u", c_int), ("commit", c_void),
                ("entropy", c_void), ("n_renoised", c_void), ("logits", c_void), ("canvas_len", c_int),
                ("pred", c_void), ("n_changed", c_void), ("n_nonfinite", c_void)]


class KernelTimer(ctypes.Structure):
    _fields_ = [("start", ctypes.POINTER(c_void)), ("stop", ctypes.POINTER(c_void)), ("capacity", c_int),
                ("count", c_int), ("kernel", c_int), ("every", c_int), ("seen", c_int)]


DG_KT = {"moe_gateup": 1, "moe_down": 2, "lm_head": 3, "attn": 4, "soft_embed": 5, "qkv": 6, "oproj": 7}

_LIB = None


def lib(path=None):
    """Load libdgstep.so (built in-tree by build.py); raise if it is missing.
    `path` (or the DGSTEP_LIB environment variable) selects another build of
    the library on the first call."""
    global _LIB
    if _LIB is None:
        path = path or os.environ.get("DGSTEP_LIB") or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run discrete_text_diffusion_step_amd/build.py")
        L = ctypes.CDLL(path)
        P = ctypes.POINTER
        sig = {
            "dg_status_string": (ctypes.c_char_p, [c_int]),
            "dg_attn_workspace_bytes": (c_size, [P(AttnCfg), c_int]),
            "dg_attn_layer": (c_int, [P(AttnCfg), P(AttnW), P(KVLayer), c_int, c_int, c_void, c_void, c_size,
                                      c_void]),
            "dg_moe_workspace_bytes": (c_size, [P(MoeCfg), c_int]),
            "dg_moe_block": (c_int, [P(MoeCfg), P(MoeW), c_int, c_void, c_void, c_void, c_void, c_void, c_size,
                                     c_void]),
            "dg_quantize_fp8": (c_int, [c_int, c_void, ctypes.c_longlong, c_int, c_void, c_void, c_void]),
            "dg_sample_workspace_bytes": (c_size, [c_int, c_int]),
            "dg_sample_renoise": (c_int, [P(SamplerCfg), c_int, c_void, c_int, c_void, c_void, c_void, c_void,
                                          c_void, c_void, c_void, c_void, c_void, c_size, c_void]),
            "dg_sample_noalloc_max_bytes": (c_size, []),
            "dg_sample_renoise_noalloc": (c_int, [P(SamplerCfg), c_int, c_void, c_int, c_void, c_void, c_void,
                                                  c_void, c_void, c_void, c_void, c_void, c_void]),
            "dg_canvas_noise": (c_int, [c_int, c_int, ctypes.c_uint64, ctypes.c_uint32, c_void, c_void]),
            "dg_lm_head_workspace_bytes": (c_size, [c_int, c_int, c_int]),
            "dg_lm_head": (c_int, [c_int, c_int, c_int, c_float, c_int, c_void, c_void, c_void, c_void, c_void,
                                   c_size, c_void]),
            "dg_soft_embed_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int]),
            "dg_soft_embed": (c_int, [P(SamplerCfg), c_int, c_int, c_int, c_void, c_void, c_void, c_void, c_void,
                                      c_size, c_void]),
            "dg_embed_transpose": (c_int, [c_int, c_int, c_int, c_void, c_void, c_void]),
            "dg_workspace_bytes": (c_size, [P(ModelCfg), c_int, c_int]),
            "dg_canvas_step": (c_int, [P(ModelCfg), P(ModelW), P(KVCache), P(CanvasState), P(SamplerCfg),
                                       c_void, c_size, c_void]),
            "dg_canvas_step_batch": (c_int, [P(ModelCfg), P(ModelW), P(KVCache), P(CanvasState), P(SamplerCfg),
                                             c_int, c_void, c_size, c_void]),
            "dg_workspace_bytes_batch": (c_size, [P(ModelCfg), c_int, c_int]),
            "dg_commit_canvas": (c_int, [P(ModelCfg), P(ModelW), P(KVCache), c_void, c_int, c_void, c_size,
                                         c_void]),
            "dg_rmsnorm": (c_int, [c_int, c_int, c_float, c_int, c_void, c_void, c_void, c_void]),
            "dg_set_kernel_timer": (None, [P(KernelTimer)]),
            "dg_probe_hbm_read": (c_int, [c_void, c_size, c_void, c_int, c_void]),
            "dg_probe_mfma_bf16": (c_int, [c_int, c_float, c_float, c_void, c_int, c_void]),
            "dg_probe_mfma_flops": (ctypes.c_longlong, [c_int, c_int]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


# ----------------------------------------------------------------- helpers


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def check(status, where):
    if status != 0:
        raise DGError(status, where)


_WS = {}


def workspace(nbytes, device=None):
    """A cached device workspace of at least nbytes (256-byte aligned by torch)."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    cur = _WS.get(dev)
    if cur is None or cur.numel() < nbytes:
        cur = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)
        _WS[dev] = cur
    return cur


def attn_cfg_c(c):
    return AttnCfg(c["hidden"], c["n_q_heads"], c["n_kv_heads"], c["head_dim"], c["layer_type"],
                   c.get("window", 0), c["shared_kv"], c["v_unit_rms"], c["rope_base"],
                   c["rotary_factor"], c["rms_eps"], _DT[c["dtype"]])


def attn_w_c(w):
    return AttnW(*(ptr(w.get(n)) for n in ("w_in_norm", "w_q", "w_k", "w_v", "w_o", "q_norm", "k_norm")))


def moe_cfg_c(c, layer_scalar=None):
    return MoeCfg(c["hidden"], c["n_experts"], c["top_k"], c["ffn"], c["shared_ffn"], c["route_scale"],
                  c["rms_eps"], c["layer_scalar"] if layer_scalar is None else layer_scalar, _DT[c["dtype"]],
                  _EF[c.get("expert_format", "dtype")])


def moe_w_c(w):
    return MoeW(*(ptr(w.get(n)) for n in MOE_W_NAMES))


def sampler_cfg_c(c):
    return SamplerCfg(c["vocab"], c["tau"], c["t_max"], c["t_min"], c["n_steps"], c["step"],
                      c["canvas_idx"] & 0xFFFFFFFF, c["seed"], 1 if c.get("final_step") else 0,
                      COMMIT_RULES[c.get("commit_rule", "entropy")], TOKEN_RULES[c.get("token_rule", "argmax")])


def model_cfg_c(m):
    return ModelCfg(attn_cfg_c(m["sliding"]), attn_cfg_c(m["global"]), moe_cfg_c(m["moe"]), m["n_layers"],
                    m["global_every"], m["vocab"], m["sc_ffn"], m["rms_eps"], _DT[m["dtype"]])


# ------------------------------------------------------------ entry points


def dg_status_string(status):
    return lib().dg_status_string(status).decode()


def dg_attn_layer(cfg, w, k_cache, v_cache, kv_len, x, causal, stream=None, ring=False, v_only=False):
    """x <- x + Attention(x) in place; returns the new committed length.
    k_cache [Hkv][capacity][d_h]; v_cache transposed, [Hkv][d_h][capacity];
    ring: position m at row m mod capacity (sliding layers); v_only: the
    keys of the committed positions are rebuilt from v_cache into k_cache."""
    L = lib()
    c = attn_cfg_c(cfg)
    n = x.shape[0]
    kv = KVLayer(ptr(k_cache), ptr(v_cache), k_cache.shape[1] if k_cache is not None else 0, kv_len,
                 1 if ring else 0, 1 if v_only else 0)
    nb = L.dg_attn_workspace_bytes(ctypes.byref(c), n)
    ws = workspace(nb, x.device)
    check(L.dg_attn_layer(ctypes.byref(c), ctypes.byref(attn_w_c(w)), ctypes.byref(kv), n, int(causal), ptr(x),
                          ptr(ws), ws.numel(), stream_handle(stream)), "dg_attn_layer")
    return kv.kv_len


def dg_moe_block(cfg, w, x, router_logits=None, want_topk=False, stream=None):
    """x <- layer_scalar * (x + MoE(x)) in place; optionally returns (idx, weights)."""
    L = lib()
    c = moe_cfg_c(cfg)
    n = x.shape[0]
    idx = wts = None
    if want_topk:
        idx = torch.empty(n, cfg["top_k"], dtype=torch.int32, device=x.device)
        wts = torch.empty(n, cfg["top_k"], dtype=torch.float32, device=x.device)
    nb = L.dg_moe_workspace_bytes(ctypes.byref(c), n)
    ws = workspace(nb, x.device)
    rl = None if router_logits is None else router_logits.contiguous()
    check(L.dg_moe_block(ctypes.byref(c), ctypes.byref(moe_w_c(w)), n, ptr(x), ptr(rl), ptr(idx), ptr(wts),
                         ptr(ws), ws.numel(), stream_handle(stream)), "dg_moe_block")
    return idx, wts


def _dtype_name(t):
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {t.dtype}")


def dg_quantize_fp8(w, stream=None):
    """Row-wise OCP E4M3 codes and fp32 row scales of w [..., K] (bf16/fp32)."""
    w = w.contiguous()
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    sc = torch.empty(w.shape[:-1], dtype=torch.float32, device=w.device)
    check(lib().dg_quantize_fp8(_DT[_dtype_name(w)], ptr(w), rows, K, ptr(q), ptr(sc), stream_handle(stream)),
          "dg_quantize_fp8")
    return q, sc


def quantize_moe_weights(w, stream=None):
    """A MoE weight dict with every expert matrix as E4M3 codes + row scales
    (use with cfg["expert_format"] = "fp8_e4m3")."""
    out = dict(w)
    for n in EXPERT_MATRICES:
        q, sc = dg_quantize_fp8(w[n], stream)
        out[n] = q
        out["s" + n[1:] if n.startswith("w_") else "ss" + n[2:]] = sc
    return out


def dg_sample_renoise(scfg, logits, want_rowstats=True, pred=None, stream=None):
    """Sampler outputs; pred (optional int32 [n], -1 before the first step)
    holds the previous proposals and receives this step's, and the result
    then carries n_changed.  n_nonfinite counts rows holding a NaN or +-inf."""
    L = lib()
    n, V = logits.shape
    dev = logits.device
    out = dict(tokens=torch.empty(n, dtype=torch.int32, device=dev),
               commit=torch.empty(n, dtype=torch.uint8, device=dev),
               entropy=torch.empty(n, dtype=torch.float32, device=dev),
               n_renoised=torch.empty(1, dtype=torch.int32, device=dev),
               rowstats=torch.empty(n, 2, dtype=torch.float32, device=dev) if want_rowstats else None,
               n_changed=torch.empty(1, dtype=torch.int32, device=dev) if pred is not None else None,
               n_nonfinite=torch.empty(1, dtype=torch.int32, device=dev))
    c = sampler_cfg_c(scfg)
    ws = workspace(L.dg_sample_workspace_bytes(n, V), dev)
    ldt = DG_BF16 if logits.dtype == torch.bfloat16 else DG_F32
    check(L.dg_sample_renoise(ctypes.byref(c), n, ptr(logits), ldt, ptr(out["tokens"]), ptr(out["commit"]),
                              ptr(out["entropy"]), ptr(out["rowstats"]), ptr(out["n_renoised"]), ptr(pred),
                              ptr(out["n_changed"]), ptr(out["n_nonfinite"]), ptr(ws), ws.numel(),
                              stream_handle(stream)),
          "dg_sample_renoise")
    return out


def dg_sample_renoise_noalloc(scfg, logits, want_rowstats=True, pred=None, stream=None):
    """dg_sample_renoise on the library's built-in scratch (no workspace);
    the outputs are allocated here, by the caller's side."""
    L = lib()
    n, V = logits.shape
    dev = logits.device
    out = dict(tokens=torch.empty(n, dtype=torch.int32, device=dev),
               commit=torch.empty(n, dtype=torch.uint8, device=dev),
               entropy=torch.empty(n, dtype=torch.float32, device=dev),
               n_renoised=torch.empty(1, dtype=torch.int32, device=dev),
               rowstats=torch.empty(n, 2, dtype=torch.float32, device=dev) if want_rowstats else None,
               n_changed=torch.empty(1, dtype=torch.int32, device=dev) if pred is not None else None,
               n_nonfinite=torch.empty(1, dtype=torch.int32, device=dev))
    c = sampler_cfg_c(scfg)
    ldt = DG_BF16 if logits.dtype == torch.bfloat16 else DG_F32
    check(L.dg_sample_renoise_noalloc(ctypes.byref(c), n, ptr(logits), ldt, ptr(out["tokens"]), ptr(out["commit"]),
                                      ptr(out["entropy"]), ptr(out["rowstats"]), ptr(out["n_renoised"]), ptr(pred),
                                      ptr(out["n_changed"]), ptr(out["n_nonfinite"]), stream_handle(stream)),
          "dg_sample_renoise_noalloc")
    return out


def dg_canvas_noise(n, vocab, seed, canvas_idx, device="cuda", stream=None):
    t = torch.empty(n, dtype=torch.int32, device=device)
    check(lib().dg_canvas_noise(n, vocab, seed, canvas_idx & 0xFFFFFFFF, ptr(t), stream_handle(stream)),
          "dg_canvas_noise")
    return t


def dg_lm_head(x, w_final_norm, embed, eps, stream=None):
    L = lib()
    n, D = x.shape
    V = embed.shape[0]
    dt = DG_BF16 if x.dtype == torch.bfloat16 else DG_F32
    logits = torch.empty(n, V, dtype=torch.float32, device=x.device)
    ws = workspace(L.dg_lm_head_workspace_bytes(n, D, dt), x.device)
    check(L.dg_lm_head(n, D, V, eps, dt, ptr(x), ptr(w_final_norm), ptr(embed), ptr(logits), ptr(ws), ws.numel(),
                       stream_handle(stream)), "dg_lm_head")
    return logits


def dg_soft_embed(scfg, logits, rowstats, embed_t, dtype, stream=None):
    L = lib()
    n = logits.shape[0]
    D = embed_t.shape[0]
    dt = _DT[dtype]
    u = torch.empty(n, D, dtype=torch.bfloat16 if dt == DG_BF16 else torch.float32, device=logits.device)
    c = sampler_cfg_c(scfg)
    ws = workspace(L.dg_soft_embed_workspace_bytes(n, D, scfg["vocab"], dt), logits.device)
    check(L.dg_soft_embed(ctypes.byref(c), n, D, dt, ptr(logits), ptr(rowstats), ptr(embed_t), ptr(u), ptr(ws),
                          ws.numel(), stream_handle(stream)), "dg_soft_embed")
    return u


def dg_embed_transpose(embed, stream=None):
    V, D = embed.shape
    et = torch.empty(D, V, dtype=embed.dtype, device=embed.device)
    dt = DG_BF16 if embed.dtype == torch.bfloat16 else DG_F32
    check(lib().dg_embed_transpose(V, D, dt, ptr(embed), ptr(et), stream_handle(stream)), "dg_embed_transpose")
    return et


def dg_rmsnorm(x, w, eps, out=None, stream=None):
    n, D = x.shape
    y = torch.empty_like(x) if out is None else out
    dt = DG_BF16 if x.dtype == torch.bfloat16 else DG_F32
    check(lib().dg_rmsnorm(n, D, eps, dt, ptr(x), ptr(w), ptr(y), stream_handle(stream)), "dg_rmsnorm")
    return y


def dg_probe_hbm_read(buf, n_groups=2048, sink=None, stream=None):
    """Read-only stream over `buf` (a device tensor); returns the sink, one
    wrapping uint32 sum per workgroup (int32 tensor holding the bits)."""
    if sink is None:
        sink = torch.empty(n_groups, dtype=torch.int32, device=buf.device)
    check(lib().dg_probe_hbm_read(ptr(buf), buf.numel() * buf.element_size(), ptr(sink), n_groups,
                                  stream_handle(stream)), "dg_probe_hbm_read")
    return sink


def dg_probe_mfma_bf16(iters, a=1.0, b=2.0 ** -10, n_groups=1024, sink=None, stream=None):
    """MFMA loop; returns the per-wave sink (float32, 4 per workgroup)."""
    if sink is None:
        sink = torch.empty(4 * n_groups, dtype=torch.float32, device="cuda")
    check(lib().dg_probe_mfma_bf16(iters, a, b, ptr(sink), n_groups, stream_handle(stream)), "dg_probe_mfma_bf16")
    return sink


def dg_probe_mfma_flops(iters, n_groups):
    return lib().dg_probe_mfma_flops(iters, n_groups)


class Model:
    """Device weights of a whole stack plus the C records that point at them."""

    def __init__(self, mcfg, weights):
        self.cfg = mcfg
        self.w = weights
        self.c_cfg = model_cfg_c(mcfg)
        L = mcfg["n_layers"]
        self._attn = (AttnW * L)(*[attn_w_c(a) for a in weights["attn"]])
        self._moe = (MoeW * L)(*[moe_w_c(m) for m in weights["moe"]])
        self._ls = (c_float * L)(*weights["layer_scalar"])
        if weights.get("embed_t") is None:
            weights["embed_t"] = dg_embed_transpose(weights["embed"])
        sc = weights.get("sc") or {}
        self.c_w = ModelW(ptr(weights["embed"]), ptr(weights["embed_t"]), ptr(weights["w_final_norm"]),
                          ptr(sc.get("sc_gate")), ptr(sc.get("sc_up")), ptr(sc.get("sc_down")),
                          self._attn, self._moe, self._ls, None)
        self._rl = None

    def set_router_logits(self, logits):
        """Per-layer fp32 router logits [rows, n_experts] (device tensors, one
        per layer, None entries computed) used instead of the router product
        by the next calls; None restores the router product everywhere."""
        if logits is None:
            self._rl = None
            self.c_w.router_logits = None
            return
        assert len(logits) == self.cfg["n_layers"]
        self._rl_t = [None if t is None else t.contiguous() for t in logits]
        self._rl = (c_void * len(logits))(*[None if t is None else t.data_ptr() for t in self._rl_t])
        self.c_w.router_logits = ctypes.cast(self._rl, ctypes.POINTER(c_void))


def ring_capacity(window, max_tokens):
    """Rows of a sliding-layer ring: the window plus one call's tokens, in 32s."""
    return (window + max_tokens + 31) // 32 * 32


class KV:
    """Per-layer caches, K [Hkv][capacity][d_h] and V transposed [Hkv][d_h][capacity],
    and the C record over them.  ring_tokens > 0 gives the sliding layers a
    ring of ring_capacity(window, ring_tokens) rows instead of `capacity`
    (every call then adds at most ring_tokens positions).  v_only_global:
    the global layers keep only V; one K scratch is shared by all of them
    (their keys are rebuilt from V by every call)."""

    def __init__(self, mcfg, capacity, device="cuda", tensors=None, ring_tokens=0, v_only_global=False):
        L = mcfg["n_layers"]
        dt = torch.bfloat16 if mcfg["dtype"] == "bf16" else torch.float32
        self.k, self.v, caps, rings, vonly = [], [], [], [], []
        k_scratch = None
        for l in range(L):
            glob = (l % mcfg["global_every"]) == mcfg["global_every"] - 1
            c = mcfg["global"] if glob else mcfg["sliding"]
            ring = bool(ring_tokens) and not glob
            cap = ring_capacity(c["window"], ring_tokens) if ring else capacity
            caps.append(cap)
            rings.append(1 if ring else 0)
            vo = bool(v_only_global) and glob
            vonly.append(1 if vo else 0)
            if tensors is not None:
                self.k.append(tensors[0][l])
                self.v.append(tensors[1][l])
            else:
                if vo:
                    if k_scratch is None:
                        k_scratch = torch.zeros(c["n_kv_heads"], cap, c["head_dim"], dtype=dt, device=device)
                    self.k.append(k_scratch)
                else:
                    self.k.append(torch.zeros(c["n_kv_heads"], cap, c["head_dim"], dtype=dt, device=device))
                self.v.append(torch.zeros(c["n_kv_heads"], c["head_dim"], cap, dtype=dt, device=device))
        self._layers = (KVLayer * L)(*[KVLayer(ptr(self.k[l]), ptr(self.v[l]), caps[l], 0, rings[l], vonly[l])
                                       for l in range(L)])
        self.c = KVCache(self._layers, L)
        self.ring_tokens = ring_tokens

    @property
    def kv_len(self):
        return self._layers[0].kv_len

    def set_len(self, n):
        for l in range(self.c.n_layers):
            self._layers[l].kv_len = n


def dg_workspace_bytes(mcfg_c, max_canvas, max_commit):
    return lib().dg_workspace_bytes(ctypes.byref(mcfg_c), max_canvas, max_commit)


def dg_workspace_bytes_batch(mcfg_c, n_canvas, canvas_len):
    return lib().dg_workspace_bytes_batch(ctypes.byref(mcfg_c), n_canvas, canvas_len)


class Canvas:
    """Device state carried across denoising steps for n_canvas canvases of n
    positions, stored back to back (one canvas by default)."""

    def __init__(self, n, hidden, dtype, device="cuda", keep_logits_vocab=0, n_canvas=1):
        dt = torch.bfloat16 if dtype == "bf16" else torch.float32
        m = n * n_canvas
        self.tokens = torch.zeros(m, dtype=torch.int32, device=device)
        self.u = torch.zeros(m, hidden, dtype=dt, device=device)
        self.commit = torch.zeros(m, dtype=torch.uint8, device=device)
        self.entropy = torch.zeros(m, dtype=torch.float32, device=device)
        self.n_renoised = torch.zeros(n_canvas, dtype=torch.int32, device=device)
        self.logits = (torch.empty(m, keep_logits_vocab, dtype=torch.float32, device=device)
                       if keep_logits_vocab else None)
        self.use_u = 0
        self.n = n
        self.n_canvas = n_canvas
        # proposals of the previous step (-1: none yet) and how many changed
        self.pred = torch.full((m,), -1, dtype=torch.int32, device=device)
        self.n_changed = torch.zeros(n_canvas, dtype=torch.int32, device=device)
        # positions whose logits held a NaN or +-inf in the last step
        self.n_nonfinite = torch.zeros(n_canvas, dtype=torch.int32, device=device)

    def c_state(self):
        return CanvasState(ptr(self.tokens), ptr(self.u), self.use_u, ptr(self.commit), ptr(self.entropy),
                           ptr(self.n_renoised), ptr(self.logits), self.n, ptr(self.pred), ptr(self.n_changed),
                           ptr(self.n_nonfinite))


def dg_canvas_step(model, kv, canvas, scfg, ws=None, stream=None):
    L = lib()
    st = canvas.c_state()
    c = sampler_cfg_c(scfg)
    if ws is None:
        ws = workspace(L.dg_workspace_bytes(ctypes.byref(model.c_cfg), canvas.n, 0), canvas.tokens.device)
    check(L.dg_canvas_step(ctypes.byref(model.c_cfg), ctypes.byref(model.c_w), ctypes.byref(kv.c),
                           ctypes.byref(st), ctypes.byref(c), ptr(ws), ws.numel(), stream_handle(stream)),
          "dg_canvas_step")
    canvas.use_u = 1 if model.cfg["sc_ffn"] > 0 else 0


def dg_canvas_step_batch(model, kvs, canvas, scfgs, ws=None, stream=None):
    """One step of canvas.n_canvas canvases in one forward; kvs[b] and
    scfgs[b] belong to canvas b."""
    L = lib()
    B = canvas.n_canvas
    assert len(kvs) == B and len(scfgs) == B
    st = canvas.c_state()
    cs = (SamplerCfg * B)(*[sampler_cfg_c(c) for c in scfgs])
    ks = (KVCache * B)(*[kv.c for kv in kvs])
    if ws is None:
        ws = workspace(L.dg_workspace_bytes_batch(ctypes.byref(model.c_cfg), B, canvas.n), canvas.tokens.device)
    check(L.dg_canvas_step_batch(ctypes.byref(model.c_cfg), ctypes.byref(model.c_w), ks, ctypes.byref(st), cs, B,
                                 ptr(ws), ws.numel(), stream_handle(stream)), "dg_canvas_step_batch")
    canvas.use_u = 1 if model.cfg["sc_ffn"] > 0 else 0


def dg_commit_canvas(model, kv, tokens, ws=None, stream=None):
    L = lib()
    n = tokens.shape[0]
    if ws is None:
        ws = workspace(L.dg_workspace_bytes(ctypes.byref(model.c_cfg), 0, n), tokens.device)
    check(L.dg_commit_canvas(ctypes.byref(model.c_cfg), ctypes.byref(model.c_w), ctypes.byref(kv.c), ptr(tokens), n,
                             ptr(ws), ws.numel(), stream_handle(stream)), "dg_commit_canvas")


class kernel_timer:
    """Context manager timing launches of one kernel class with HIP events
    recorded by the library on the launching stream: every `every`-th launch
    (each event adds a few microseconds between kernels)."""

    def __init__(self, kind, capacity=4096, every=1):
        self.kind = DG_KT[kind]
        self.cap = capacity
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(capacity)]
        for a, b in self.ev:   # materialise the underlying hipEvent_t handles
            a.record()
            b.record()
        torch.cuda.synchronize()
        self._start = (c_void * capacity)(*[a.cuda_event for a, _ in self.ev])
        self._stop = (c_void * capacity)(*[b.cuda_event for _, b in self.ev])
        self.t = KernelTimer(self._start, self._stop, capacity, 0, self.kind, every, 0)

    def __enter__(self):
        lib().dg_set_kernel_timer(ctypes.byref(self.t))
        return self

    def __exit__(self, *exc):
        lib().dg_set_kernel_timer(None)
        return False

    def durations_ms(self):
        torch.cuda.synchronize()
        return [self.ev[i][0].elapsed_time(self.ev[i][1]) for i in range(self.t.count)]
