"""Error model of bf16 matrix-product operands (test support; NOT a reference).

Evaluates the first layer stack + key branch of the pool for tokens at
position 0 (no attention term) in float64, with an option to round to bf16
every tensor that feeds a bf16 matrix product or is stored as bf16: the
normalised-input operands of the Q / gate-up / LM-head products, the SwiGLU
activation, the state stack, the router operand and the mixed channel. Its
only use is to measure how far exact bf16 rounding alone moves the result
from the exact definition, which sets the tolerance of the full-depth bf16
parity tests. With rounding off it reduces to the definition (checked
against the oracle in test_bf16_error_model.py).
"""
import numpy as np

from wm_inputs import round_bf16

ROUNDING_POINTS = ("S", "hb", "act", "router", "mb")


def _rb(x, on):
    return round_bf16(np.asarray(x, np.float32)).astype(np.float64) if on else x


def _rinv(x, eps):
    return 1.0 / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)


def _rope(x, pos, base):
    d = x.shape[-1]
    ang = np.asarray(pos, np.float64)[:, None, None] * base ** (-2.0 * np.arange(d // 2) / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], -1)


def position0(w, W, tokens, rounding=()):
    """logits [N, V] and keys [k, N, Hkv, d] of tokens at position 0."""
    R = {p: p in rounding for p in ROUNDING_POINTS}
    Wd = {n: np.asarray(a, np.float64) for n, a in W.items()}
    eps = w.eps
    N = len(tokens)
    h = Wd["embed"][np.asarray(tokens)]
    S = []
    for l in range(w.L):
        S.append(_rb(h, R["S"]))
        # the attention term is zero at position 0
        b = _rb(h * Wd["ffn_norm"][l], R["hb"]) * _rinv(h, eps)
        act = _rb((b @ Wd["w_gate"][l].T) / (1 + np.exp(-(b @ Wd["w_gate"][l].T))) * (b @ Wd["w_up"][l].T), R["act"])
        h = h + act @ Wd["w_down"][l].T
    S = np.stack(S)
    logits = (_rb(h * Wd["final_norm"], R["hb"]) * _rinv(h, eps)) @ Wd["lm_head"].T
    rinv = [_rinv(S[l], eps) for l in range(w.L)]
    u = np.concatenate([_rb(S[l] * rinv[l] * Wd["src_norm"][0, l], R["router"]) for l in range(0, w.L, w.p)], -1)
    A = (u @ Wd["router"][0].T).reshape(N, w.L, w.k)
    keys = []
    for j in range(w.k):
        m = sum(A[:, l, j, None] * rinv[l] * Wd["src_norm"][0, l] * S[l] for l in range(w.L))
        c = _rb(m * Wd["chan_norm"][0, j], R["mb"]) * _rinv(m, eps)
        kj = (c @ Wd["wk"][j].T).reshape(N, w.Hkv, w.d)
        kj = kj * _rinv(kj, eps) * Wd["k_norm"][j]
        keys.append(_rope(kj, np.zeros(N), w.rope_base))
    return logits, np.stack(keys)


FF_ROUNDING_POINTS = ("S", "hb", "act", "router", "mix", "mb", "q", "kv", "p", "o")


def _rmsnorm(x, g, eps):
    return x * _rinv(x, eps) * g


def _attend_strict(q, K, V, rb_p):
    """q [T, Hq, d], K/V [T, Hkv, d]: position i attends to s < i; the
    probabilities pass through rb_p before the value product."""
    T, Hq, d = q.shape
    G = Hq // K.shape[1]
    out = np.zeros_like(q)
    vis = np.arange(T)[None, :] < np.arange(T)[:, None]
    for hq in range(Hq):
        sc = np.where(vis, q[:, hq] @ K[:, hq // G].T / np.sqrt(d), -np.inf)
        mx = np.max(sc, 1, keepdims=True)
        ok = np.isfinite(mx[:, 0])
        p = np.where(vis, np.exp(sc - np.where(ok[:, None], mx, 0.0)), 0.0)
        den = p.sum(1, keepdims=True)
        out[ok, hq] = rb_p(p[ok]) @ V[:, hq // G] / den[ok]
    return out


def ff_forward(w, W, tokens, rounding=()):
    """The feedback-free forward (k = L; channel l from states 0..l, router
    over the sampled states r <= l; strict attention) of whole sequences in
    float64, optionally rounding to bf16 every tensor the HIP path stores or
    feeds to a bf16 product: stored states, normalised GEMM operands, router
    input, the mix operands (weights times row scale, gained states), the mixed
    channel, queries, cached keys/values, attention probabilities and outputs,
    and the SwiGLU activation. Returns (K, V [L, B, Hkv, T, d], logits)."""
    R = {p: p in rounding for p in FF_ROUNDING_POINTS}
    rb = lambda x, p: _rb(x, R[p])
    Wd = {n: np.asarray(a, np.float64) for n, a in W.items()}
    eps, L, D = w.eps, w.L, w.D
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    pos = np.arange(T)
    Kc = np.zeros((L, B, w.Hkv, T, w.d))
    Vc = np.zeros_like(Kc)
    logits = np.zeros((B, T, w.V))
    for b in range(B):
        h = Wd["embed"][tokens[b]]
        S = []
        for l in range(L):
            S.append(rb(h, "S"))
            rinv = [_rinv(S[s], eps) for s in range(l + 1)]
            sampled = [r for r in range(0, L, w.p) if r <= l]
            kv = []
            for beta in (0, 1):
                g = Wd["src_norm"][beta]
                u = np.concatenate([rb(S[r] * rinv[r] * g[r], "router") for r in sampled], -1)
                Wr = Wd["router"][beta].reshape(L, w.k, w.R * D)[:l + 1, l, :len(sampled) * D]
                A = u @ Wr.T
                m = sum(rb(A[:, s, None] * rinv[s], "mix") * rb(g[s] * S[s], "mix") for s in range(l + 1))
                c = rb(m * Wd["chan_norm"][beta, l], "mb") * _rinv(m, eps)
                x = (c @ Wd["wk" if beta == 0 else "wv"][l].T).reshape(T, w.Hkv, w.d)
                if beta == 0:
                    x = _rope(_rmsnorm(x, Wd["k_norm"][l], eps), pos, w.rope_base)
                kv.append(rb(x, "kv"))
            Kc[l, b] = kv[0].transpose(1, 0, 2)
            Vc[l, b] = kv[1].transpose(1, 0, 2)
            a = rb(h * Wd["attn_norm"][l], "hb") * _rinv(h, eps)
            q = rb(_rope(_rmsnorm((a @ Wd["wq"][l].T).reshape(T, w.Hq, w.d), Wd["q_norm"][l], eps), pos, w.rope_base),
                   "q")
            o = rb(_attend_strict(q, kv[0], kv[1], lambda p: rb(p, "p")), "o")
            h = h + o.reshape(T, -1) @ Wd["wo"][l].T
            f = rb(h * Wd["ffn_norm"][l], "hb") * _rinv(h, eps)
            gt = f @ Wd["w_gate"][l].T
            act = rb(gt / (1 + np.exp(-gt)) * (f @ Wd["w_up"][l].T), "act")
            h = h + act @ Wd["w_down"][l].T
        logits[b] = (rb(h * Wd["final_norm"], "hb") * _rinv(h, eps)) @ Wd["lm_head"].T
    return Kc, Vc, logits
