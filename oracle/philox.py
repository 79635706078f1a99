"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE ONLY: this module belongs to the CPU oracle.  Only the
test-suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the product library never does.

Definition followed: Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
as easy as 1, 2, 3" (SC'11), the Philox-4x32 bijection with 10 rounds.
One round maps the counter (c0, c1, c2, c3) under the round key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with 32x32->64-bit products split into high and low words, M0 = 0xD2511F53
and M1 = 0xCD9E8D57.  Between rounds the key is advanced by the Weyl
constants (0x9E3779B9, 0xBB67AE85), modulo 2**32.

The pages ask for "uniform random tokens" for re-noising (aibars.net news,
section on block-autoregressive denoising and self-correction; aitrends.kr
notebook summary, sampler paragraph) but name no generator; Philox with
seed 1 is the reading adopted for reproducibility.

Pinned by the published known-answer vectors (tests/golden/philox_kat.txt).
"""
import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32_10(ctr, key):
    """Apply the 10-round Philox-4x32 bijection.

    ctr: array-like [..., 4] of uint32 counters; key: array-like [..., 2].
    Returns uint32 array [..., 4].  Vectorised over leading axes.
    """
    c = np.asarray(ctr, dtype=np.uint64) & _MASK
    k = np.asarray(key, dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
    for r in range(10):
        if r > 0:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0          # < 2**64, exact in uint64
        p1 = _M1 * c2
        hi0, lo0 = p0 >> _SH, p0 & _MASK
        hi1, lo1 = p1 >> _SH, p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def uniform_token(x0, vocab):
    """Map a 32-bit uniform word to a token id in [0, vocab): floor(x0*vocab / 2**32).

    Exactly uniform when vocab is a power of two (every id gets 2**32/vocab words).
    """
    x = np.asarray(x0, dtype=np.uint64)
    return ((x * np.uint64(vocab)) >> _SH).astype(np.int64)
