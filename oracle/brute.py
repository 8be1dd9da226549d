"""Scalar-loop brute force of exact autoregressive WhiteMatter execution
(test infrastructure only).

Written separately from ``wm_oracle`` — plain Python floats, explicit index
loops, ``math`` only, no numpy arithmetic — so that a vectorisation slip
there (a transposed operand, a wrong reshape, a misplaced axis) shows up as
a disagreement. It follows the same sources and readings (the paperlayer.ai
summary §3 Method and the onedev.kr summary's "how it works" / "what
differs" sections); see ``wm_oracle`` for the list of readings.

Tiny shapes only: the cost is O(T^2 * L * D * max(D, F)) Python operations.
"""
from __future__ import annotations

import math


def _rms(vec, gain, eps):
    ss = 0.0
    for v in vec:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(vec) + eps)
    return [vec[i] * r * gain[i] for i in range(len(vec))]


def _matvec(Wm, vec):
    """Wm is a list of rows [out][in]."""
    out = []
    for row in Wm:
        acc = 0.0
        for i in range(len(vec)):
            acc += row[i] * vec[i]
        out.append(acc)
    return out


def _rot(vec, pos, base):
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for m in range(h):
        theta = pos * base ** (-(2.0 * m) / d)
        c, s = math.cos(theta), math.sin(theta)
        out[m] = vec[m] * c - vec[m + h] * s
        out[m + h] = vec[m] * s + vec[m + h] * c
    return out


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def brute_ar(w, weights, tokens):
    """Exact autoregressive rollout of every sequence in ``tokens`` [B][T].

    Returns (K, V, logits): K[b][j][h][i] is the d-vector stored for channel
    j, KV head h, position i; logits[b][i] the V logits of token i.
    """
    W = {n: _tolist(a) for n, a in weights.items()}
    L, D, Hq, Hkv, d, k, p = w.L, w.D, w.Hq, w.Hkv, w.d, w.k, w.p
    G = Hq // Hkv
    eps, base = w.eps, w.rope_base
    toks = _tolist(tokens)
    Kout, Vout, Lout = [], [], []
    for b in range(len(toks)):
        T = len(toks[b])
        K = [[[None] * T for _ in range(Hkv)] for _ in range(k)]
        Vv = [[[None] * T for _ in range(Hkv)] for _ in range(k)]
        logits_b = []
        for i in range(T):
            h = list(W["embed"][toks[b][i]])
            states = []
            for l in range(L):
                states.append(list(h))
                a = _rms(h, W["attn_norm"][l], eps)
                qfull = _matvec(W["wq"][l], a)
                o = [0.0] * (Hq * d)
                c = l % k
                for hq in range(Hq):
                    qh = _rot(_rms(qfull[hq * d:(hq + 1) * d], W["q_norm"][l], eps), i, base)
                    hk = hq // G
                    if i == 0:
                        continue
                    scores = []
                    for s in range(i):
                        kv = K[c][hk][s]
                        dot = 0.0
                        for e in range(d):
                            dot += qh[e] * kv[e]
                        scores.append(dot / math.sqrt(d))
                    mx = max(scores)
                    ex = [math.exp(x - mx) for x in scores]
                    z = sum(ex)
                    for s in range(i):
                        vv = Vv[c][hk][s]
                        for e in range(d):
                            o[hq * d + e] += ex[s] / z * vv[e]
                att = _matvec(W["wo"][l], o)
                h = [h[e] + att[e] for e in range(D)]
                bn = _rms(h, W["ffn_norm"][l], eps)
                gt = _matvec(W["w_gate"][l], bn)
                up = _matvec(W["w_up"][l], bn)
                act = [gt[f] / (1.0 + math.exp(-gt[f])) * up[f] for f in range(len(gt))]
                dn = _matvec(W["w_down"][l], act)
                h = [h[e] + dn[e] for e in range(D)]
            logits_b.append(_matvec(W["lm_head"], _rms(h, W["final_norm"], eps)))
            # pool, both branches, then append at position i
            for beta in range(2):
                normed = [_rms(states[l], W["src_norm"][beta][l], eps) for l in range(L)]
                u = []
                for l in range(0, L, p):
                    u.extend(normed[l])
                r = _matvec(W["router"][beta], u)
                for j in range(k):
                    mj = [0.0] * D
                    for l in range(L):
                        wt = r[l * k + j]
                        for e in range(D):
                            mj[e] += wt * normed[l][e]
                    cj = _rms(mj, W["chan_norm"][beta][j], eps)
                    proj = _matvec(W["wk"][j] if beta == 0 else W["wv"][j], cj)
                    for hk in range(Hkv):
                        piece = proj[hk * d:(hk + 1) * d]
                        if beta == 0:
                            K[j][hk][i] = _rot(_rms(piece, W["k_norm"][j], eps), i, base)
                        else:
                            Vv[j][hk][i] = piece
        Kout.append(K)
        Vout.append(Vv)
        Lout.append(logits_b)
    return Kout, Vout, Lout
