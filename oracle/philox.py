"""Philox4x64-10 counter-based generator and the uniform token draw.

Definition (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC'11): a 4x64-bit counter and a 2x64-bit key; each of 10 rounds
takes the two 128-bit products M0*c0 and M1*c2, and forms the new counter
(hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key
is bumped by the Weyl constants (W0, W1) between rounds.

The token draw: the explainer's uniform-state noise replaces a token by a
token drawn uniformly from the vocabulary ("Diffusione dello stato uniforme";
the comparison table's starting point "token casuali campionati dal
vocabolario").  Reading taken: counter = (position i, draw index t, canvas b,
block k), key = (seed, 0); the token is floor(w0 * V / 2^64) where w0 is word 0
of the output block -- exactly uniform when V is a power of two.
"""
import numpy as np

M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
MASK64 = (1 << 64) - 1


def philox4x64_10(ctr, key):
    """One output block (4 words) for counter ctr=(c0,c1,c2,c3), key=(k0,k1)."""
    c0, c1, c2, c3 = (int(v) & MASK64 for v in ctr)
    k0, k1 = (int(v) & MASK64 for v in key)
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return (c0, c1, c2, c3)


def uniform_token(seed, t, b, k, i, V):
    w0 = philox4x64_10((i, t, b, k), (seed, 0))[0]
    return (w0 * V) >> 64


def draw_tokens(seed, t, block, B, C, V):
    """Tokens [B, C] drawn for every position of every canvas at draw index t."""
    out = np.empty((B, C), np.int64)
    for b in range(B):
        for i in range(C):
            out[b, i] = uniform_token(seed, t, b, block, i, V)
    return out


# ---- vectorised form for bulk statistics (same definition, numpy uint64) ----

def _mul128(a, m):
    """(hi, lo) of a * m for uint64 arrays a and a Python-int constant m."""
    a = a.astype(np.uint64)
    mask = np.uint64(0xFFFFFFFF)
    a_lo, a_hi = a & mask, a >> np.uint64(32)
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll = a_lo * m_lo
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> np.uint64(32)) + (lh & mask) + (hl & mask)
    lo = (ll & mask) | ((mid & mask) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x64-10 over arrays of counters (uint64)."""
    c0, c1, c2, c3 = (np.asarray(v, np.uint64).copy() for v in (c0, c1, c2, c3))
    k0 = np.asarray(k0, np.uint64).copy()
    k1 = np.asarray(k1, np.uint64).copy()
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = k0 + np.uint64(W0)
                k1 = k1 + np.uint64(W1)
            hi0, lo0 = _mul128(c0, M0)
            hi1, lo1 = _mul128(c2, M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform_tokens_np(seed, t, b, k, i, V):
    """Vectorised uniform_token over arrays of (t, b, k, i)."""
    i = np.asarray(i, np.uint64)
    z = np.zeros_like(i)
    w0 = philox4x64_10_np(i, np.asarray(t, np.uint64) + z, np.asarray(b, np.uint64) + z,
                          np.asarray(k, np.uint64) + z, np.uint64(seed) + z, z)[0]
    hi, _ = _mul128(w0, int(V))
    return hi.astype(np.int64)
