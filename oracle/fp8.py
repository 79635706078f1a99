"""OCP FP8 E4M3 expert weights for the oracle (test infrastructure only).

The pages run the model in FP8 on H100s (aitrends.kr notebook summary, the
generation-speed paragraph) without fixing a scheme.  Reading taken here:
weight-only FP8 for the expert matrices (routed and shared), one fp32 scale
per output row, activations unchanged.

E4M3 is the OCP 8-bit floating point format (OFP8 specification, E4M3):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds
the subnormals m * 2^-9; the all-ones pattern S.1111.111 is NaN and there are
no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.

Row quantisation (the reading for the scale, stated as arithmetic so the
integer codes are reproducible):
    scale_r = fp32(max_c |w_rc|) / fp32(448)     (fp32 division; 1 for a zero row)
    q_rc    = E4M3(fp32(w_rc) / scale_r)          (fp32 division, then round to
                                                   nearest even, saturating at 448)
    dequant = scale_r * E4M3 value of q_rc
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Float64 value of each E4M3 code (NaN for the two NaN patterns)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    v = s * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(v):
    """E4M3 code of each value: round to nearest, ties to the even code,
    magnitudes above 448 saturate to 448.  NaN input is an error."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = (np.signbit(v)).astype(np.int64) << 7
    a = np.minimum(np.abs(v), E4M3_MAX)
    out = np.zeros(a.shape, dtype=np.int64)
    # subnormal range (below the smallest normal 2^-6): steps of 2^-9; the
    # rounded step count 0..8 is the code itself (8 is the smallest normal)
    sub = a < 2.0 ** -6
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    # normal range: a = f * 2^x with f in [0.5, 1) -> 1.mmm * 2^(x-1)
    nrm = ~sub
    f, x = np.frexp(a[nrm])
    e = x.astype(np.int64) - 1                       # unbiased exponent, -6..8
    frac8 = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)   # 0..8, ties even
    carry = frac8 == 8
    e = np.where(carry, e + 1, e)
    frac8 = np.where(carry, 0, frac8)
    out[nrm] = ((e + 7) << 3) | frac8
    # saturation keeps the top code at 448 (S.1111.110)
    out = np.minimum(out, 0x7E)
    return (out | sign).astype(np.uint8)


def quantize_rows(w):
    """Row-wise E4M3 quantisation of w [rows, cols] (values exact in fp32).
    Returns codes uint8 [rows, cols] and scales float32 [rows]."""
    w32 = np.asarray(w, dtype=np.float64).astype(np.float32)
    amax = np.abs(w32).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    ratio = (w32 / scale[:, None]).astype(np.float32)   # IEEE fp32 division
    return e4m3_encode(ratio.astype(np.float64)), scale


def dequantize_rows(q, scale):
    """scale_r * value(q_rc) in float64."""
    return np.asarray(scale, dtype=np.float64)[:, None] * e4m3_decode(q)


def quantize_experts(w):
    """Quantise every expert matrix of a MoE weight dict (routed [E, N, K]
    stacks row by row, shared [N, K]).  Returns (codes, scales, dequantised)
    dicts keyed by the weight names."""
    codes, scales, deq = {}, {}, {}
    for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        a = np.asarray(w[name], dtype=np.float64)
        flat = a.reshape(-1, a.shape[-1])
        q, s = quantize_rows(flat)
        codes[name] = q.reshape(a.shape)
        scales[name] = s.reshape(a.shape[:-1])
        deq[name] = dequantize_rows(q, s).reshape(a.shape)
    return codes, scales, deq
