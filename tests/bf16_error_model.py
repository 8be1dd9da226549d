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
