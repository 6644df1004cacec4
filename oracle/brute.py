"""Brute-force oracle: the denoise step in scalar pure-Python loops.

Written separately from ``step.py`` (no numpy arithmetic; every dot product
and sum is ``math.fsum`` over Python floats), for canvases of at most 16
tokens.  It serves to pin the numpy oracle: a transposed operand, a wrong
index, a dropped term or a wrong sign in either shows up as a disagreement.
Same readings of the DiffusionGemma explainer as ``step.py`` (see there).
"""
import math
import struct

from .philox import uniform_token


def _round(v, dtype):
    if dtype == "bf16":
        if v == 0.0:
            return 0.0
        m, e = math.frexp(v)
        return math.ldexp(round(m * 256.0) / 256.0, e)   # round(): ties to even
    if dtype == "f32":
        return struct.unpack("f", struct.pack("f", v))[0]
    raise ValueError(dtype)


def _dot(u, w):
    return math.fsum(a * b for a, b in zip(u, w))


def _softmax_stats(scores):
    m = max(scores)
    ps = [math.exp(s - m) if s != -math.inf else 0.0 for s in scores]
    return m, ps, math.fsum(ps)


def step(H, E, W, Kc, Vc, L, x, S_prev, tau, seed, t, block, dtype):
    """Same contract as oracle.step.denoise_step, inputs as nested lists (or
    anything indexable) of Python floats / ints."""
    B, C, d = len(H), len(H[0]), len(H[0][0])
    dh = len(Kc[0][0][0])
    Hq = len(W["Wq"]) // dh
    Hkv = len(W["Wk"]) // dh
    G = Hq // Hkv
    V = len(E)
    rs = lambda v: _round(v, dtype)

    # 1 assemble
    X = [[[rs(H[b][i][e] + E[x[b][i]][e] + (S_prev[b][i][e] if S_prev is not None else 0.0))
           for e in range(d)] for i in range(C)] for b in range(B)]
    # 2 projections (weights are [out][in])
    def proj(Wm, nh):
        return [[[[rs(_dot(X[b][i], Wm[hh * dh + f])) for f in range(dh)]
                  for hh in range(nh)] for i in range(C)] for b in range(B)]
    Q = proj(W["Wq"], Hq)
    Kn = proj(W["Wk"], Hkv)
    Vn = proj(W["Wv"], Hkv)
    # 3 bidirectional attention over [cache || canvas]
    O = [[[None] * Hq for _ in range(C)] for _ in range(B)]
    sc = 1.0 / math.sqrt(dh)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            keys = [Kc[b][g][j] for j in range(L)] + [Kn[b][j][g] for j in range(C)]
            vals = [Vc[b][g][j] for j in range(L)] + [Vn[b][j][g] for j in range(C)]
            for i in range(C):
                s = [_dot(Q[b][i][h], k) * sc for k in keys]
                _, ps, l = _softmax_stats(s)
                O[b][i][h] = [rs(math.fsum(p * v[f] for p, v in zip(ps, vals)) / l)
                              for f in range(dh)]
    # 4 residual output projection
    Z = []
    for b in range(B):
        for i in range(C):
            o = [O[b][i][h][f] for h in range(Hq) for f in range(dh)]
            Z.append([rs(X[b][i][e] + _dot(o, W["Wo"][e])) for e in range(d)])
    # 5 vocabulary head, confidence, self-conditioning
    ms, as_, lses, cs, Ss = [], [], [], [], []
    for z in Z:
        lg = [_dot(z, E[v]) for v in range(V)]
        m, ps, l = _softmax_stats(lg)
        a = lg.index(m)
        lse = m + math.log(l)
        ms.append(m)
        as_.append(a)
        lses.append(lse)
        cs.append(math.exp(m - lse))
        Ss.append([rs(math.fsum(p * E[v][e] for v, p in enumerate(ps)) / l) for e in range(d)])
    # 6 renoise
    tau32 = struct.unpack("f", struct.pack("f", tau))[0]
    x_new, mask = [], []
    for r in range(B * C):
        b, i = divmod(r, C)
        if cs[r] < tau32:
            x_new.append(uniform_token(seed, t, b, block, i, V))
            mask.append(1)
        else:
            x_new.append(as_[r])
            mask.append(0)
    return dict(X=X, Q=Q, Kn=Kn, Vn=Vn, O=O, Z=Z, m=ms, a=as_, lse=lses, c=cs, S=Ss,
                x_new=x_new, mask=mask)
