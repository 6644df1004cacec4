"""Seeded generators.  numpy's PCG64 via SeedSequence([workload, tensor, i, j])
makes every tensor reproducible on any machine; the tensor ids are

  0 E (embedding table)      1-4 Wq, Wk, Wv, Wo      5-6 cached K, V
  7 planted token ids y      8 amplitude jitter      9 hidden-state noise

Floating tensors are drawn in float32 and stored either as float32 (``f32``
workloads) or as bfloat16 bit patterns in uint16 (``bf16`` workloads),
rounded to nearest-even.  Nothing here knows how the step computes.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

from .configs import Config

_ROWS_PER_CHUNK = 16384


def bf16_bits_from_f32(x):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even
    (inputs here are finite)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).copy()
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def f32_from_bf16_bits(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x, dtype):
    return bf16_bits_from_f32(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def from_storage(a, dtype):
    """Stored tensor -> float32 values (exact)."""
    return f32_from_bf16_bits(a) if dtype == "bf16" else np.asarray(a, np.float32)


def _rng(cfg, *ids):
    return np.random.default_rng(np.random.SeedSequence([cfg.index, *ids]))


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def gen_embedding(cfg: Config, std=0.02):
    """E[V, d] ~ N(0, std^2), drawn in chunks of 16384 rows (chunk id = row block)."""
    V, d = cfg.V, cfg.d
    out = np.empty((V, d), np.uint16 if cfg.dtype == "bf16" else np.float32)

    def one(ci):
        r0 = ci * _ROWS_PER_CHUNK
        r1 = min(V, r0 + _ROWS_PER_CHUNK)
        x = _rng(cfg, 0, ci).standard_normal((r1 - r0, d), dtype=np.float32)
        x *= np.float32(std)
        out[r0:r1] = to_storage(x, cfg.dtype)

    n = (V + _ROWS_PER_CHUNK - 1) // _ROWS_PER_CHUNK
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, range(n)))
    return out


def gen_weights(cfg: Config):
    """Projection weights, each ~ N(0, 1/d), stored output-major like a linear
    layer's weight: Wq[Hq*dh, d], Wk/Wv[Hkv*dh, d], Wo[d, Hq*dh]."""
    s = np.float32(cfg.d ** -0.5)
    shapes = {"Wq": (cfg.Hq * cfg.dh, cfg.d), "Wk": (cfg.Hkv * cfg.dh, cfg.d),
              "Wv": (cfg.Hkv * cfg.dh, cfg.d), "Wo": (cfg.d, cfg.Hq * cfg.dh)}
    out = {}
    for tid, (k, shp) in enumerate(shapes.items(), start=1):
        x = _rng(cfg, tid).standard_normal(shp, dtype=np.float32) * s
        out[k] = to_storage(x, cfg.dtype)
    return out


def gen_cache(cfg: Config):
    """Cached keys/values [B, Hkv, cap, dh]; rows [0, L) ~ N(0, cache_std^2),
    rows [L, cap) zero (room for appended blocks)."""
    shp = (cfg.B, cfg.Hkv, cfg.cap, cfg.dh)
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    K = np.zeros(shp, dt)
    V = np.zeros(shp, dt)
    s = np.float32(cfg.cache_std)
    for tid, T in ((5, K), (6, V)):
        for b in range(cfg.B):
            for g in range(cfg.Hkv):
                x = _rng(cfg, tid, b, g).standard_normal((cfg.L, cfg.dh), dtype=np.float32) * s
                T[b, g, :cfg.L] = to_storage(x, cfg.dtype)
    return K, V


def signal_amplitude(cfg: Config, std=0.02):
    """Amplitude a of the planted direction so that the median position's
    confidence sits near the mean threshold.  With u = std*a the planted logit
    is about u*sqrt(d) and the other V-1 logits are about N(0, u^2), so the
    confidence is tau when u*sqrt(d) - u^2/2 = ln(V-1) + ln(tau/(1-tau));
    the smaller root of that quadratic is taken."""
    taus = cfg.tau
    tau = 0.5 * (taus[0] + taus[1])
    K = math.log(cfg.V - 1) + math.log(tau / (1 - tau))
    u = math.sqrt(cfg.d) - math.sqrt(cfg.d - 2 * K)
    return u / std


def gen_hidden(cfg: Config, E_store, block=0, noise=0.1, jitter=0.1):
    """Canvas hidden states H[B, C, d] and planted ids y[B, C]:
    H_i = a_i * E[y_i]/|E[y_i]| + N(0, noise^2), a_i = a*(1 + jitter*xi_i),
    built from the stored (rounded) rows of E, then stored."""
    a = signal_amplitude(cfg)
    H = np.empty((cfg.B, cfg.C, cfg.d), np.uint16 if cfg.dtype == "bf16" else np.float32)
    Y = np.empty((cfg.B, cfg.C), np.int32)
    for b in range(cfg.B):
        y = _rng(cfg, 7, b, block).integers(0, cfg.V, size=cfg.C, dtype=np.int64)
        xi = _rng(cfg, 8, b, block).standard_normal(cfg.C)
        nz = _rng(cfg, 9, b, block).standard_normal((cfg.C, cfg.d), dtype=np.float32)
        e = from_storage(E_store[y], cfg.dtype).astype(np.float64)
        e /= np.linalg.norm(e, axis=1, keepdims=True)
        h = (a * (1.0 + jitter * xi))[:, None] * e + noise * nz.astype(np.float64)
        H[b] = to_storage(h.astype(np.float32), cfg.dtype)
        Y[b] = y.astype(np.int32)
    return H, Y


@dataclass
class Problem:
    cfg: Config
    E: np.ndarray
    W: dict
    Kc: np.ndarray
    Vc: np.ndarray
    H: list = field(default_factory=list)   # per block [B, C, d]
    Y: list = field(default_factory=list)   # per block [B, C]


def gen_problem(cfg: Config, with_cache=True):
    E = gen_embedding(cfg)
    W = gen_weights(cfg)
    if with_cache:
        Kc, Vc = gen_cache(cfg)
    else:
        Kc = Vc = None
    p = Problem(cfg, E, W, Kc, Vc)
    for k in range(cfg.blocks):
        H, Y = gen_hidden(cfg, E, k)
        p.H.append(H)
        p.Y.append(Y)
    return p
