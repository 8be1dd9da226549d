"""Error model of the bf16 HIP path (test support; NOT a reference).

The oracle evaluates the WhiteMatter definition exactly (float64). The bf16
HIP path stores some tensors as bf16 and feeds others to bf16 matrix products;
each such tensor is rounded once to the nearest bf16 (relative error <= 2^-9).
This module evaluates the same definition in float64 with an option to round
any subset of those tensors, at the places where the HIP path rounds them,
and nothing else. Its uses:

* measure how far bf16 rounding alone moves a result from the exact
  definition (the floor of any bf16 implementation that rounds there), which
  sets the bf16 tolerances of the GPU parity tests;
* attribute that floor to the individual rounding points;
* a second reference for the GPU tests: with every point rounded, the model
  differs from the HIP path only by accumulation order (float32 sums in a
  different order) and by the rare operand whose float32 value lies on the
  other side of a bf16 rounding boundary.

With no rounding the model is the definition (checked against the oracle in
tests/test_bf16_error_model.py).

Rounding points of a group step (``STEP_ROUNDING_POINTS``):

  S     the state stack (the input of each block) stored as bf16
  hb    the operand of a normalised-input product (Q, gate/up, LM head):
        gain (.) h rounded, the row's 1/rms applied to the product after
  q     the normed, rotated queries stored for the attention
  p     the attention probabilities (exp(s - max)) fed to the value product;
        the denominator sums the unrounded values
  o     the attention output stored for the output projection
  act   the SwiGLU activation stored for the down projection
  u     the router input: a normalised state (many rows: S * 1/rms, the
        source gains folded into the router weights; few rows: with the gain)
  wf    the router weights times the source gains (many rows only)
  mixw  the mixing weights A[l, j] * 1/rms_l fed to the mix product
  mixs  the gained states gamma_l (.) S_l fed to the mix product
  mb    the mixed channel times its channel gain, m_j (.) rho_j, the 1/rms of
        m_j applied to the projection after
  kv    the appended keys and values stored in the cache
"""
import numpy as np

from wm_inputs import round_bf16

STEP_ROUNDING_POINTS = ("S", "hb", "q", "p", "o", "act", "u", "wf", "mixw", "mixs", "mb", "kv")


JITTER = None  # a numpy Generator while draws of the rounding are being sampled (set by jittered())


def _rb(x, on):
    if not on:
        return x
    if JITTER is not None:
        # a relative perturbation of the size float32 evaluation-order
        # differences leave before a value is rounded
        x = x * (1.0 + JITTER.uniform(-2.0 ** -20, 2.0 ** -20, np.shape(x)))
    return round_bf16(np.asarray(x, np.float32)).astype(np.float64)


class jittered:
    """Context: every rounding perturbs its input by a random relative amount
    of about 1e-6 first, so each run draws the bf16 roundings anew (as a
    bf16 implementation summing in another order does)."""

    def __init__(self, seed):
        self.seed = seed

    def __enter__(self):
        global JITTER
        JITTER = np.random.default_rng(self.seed)

    def __exit__(self, *exc):
        global JITTER
        JITTER = None


def _rinv(x, eps):
    return 1.0 / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)


def _rmsnorm(x, g, eps):
    return x * _rinv(x, eps) * g


def _rope(x, pos, base):
    """x [N, H, d] at positions pos [N]; element m pairs with m + d/2."""
    d = x.shape[-1]
    ang = np.asarray(pos, np.float64)[:, None, None] * base ** (-2.0 * np.arange(d // 2) / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], -1)


def _attend(q, pos, bidx, Kc, Vc, c, rb_p):
    """Strict-causal attention of rows q [N, Hq, d] to cache channel c; the
    probabilities pass through rb_p before the value product."""
    N, Hq, d = q.shape
    Hkv = Kc.shape[2]
    G = Hq // Hkv
    out = np.zeros((N, Hq, d))
    for n in range(N):
        i = int(pos[n])
        if i == 0:
            continue
        b = int(bidx[n])
        for hk in range(Hkv):
            s = q[n, hk * G:(hk + 1) * G] @ Kc[c, b, hk, :i].T / np.sqrt(d)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[n, hk * G:(hk + 1) * G] = rb_p(p) @ Vc[c, b, hk, :i] / p.sum(axis=1, keepdims=True)
    return out


def step(w, W, tok, pos, bidx, Kc, Vc, rounding=(), many_rows=True, want_logits=False):
    """One group step of the rows (tok[n] at position pos[n] of sequence
    bidx[n]) against the cache Kc/Vc [k, B, Hkv, T, d] (not modified).

    Returns (K_new, V_new [k, N, Hkv, d] as they would be appended, logits
    [N, V] or None, S [L, N, D])."""
    R = {p: p in rounding for p in STEP_ROUNDING_POINTS}
    rb = lambda x, p: _rb(x, R[p])
    Wd = {n: np.asarray(a, np.float64) for n, a in W.items()}
    Kc = np.asarray(Kc, np.float64)
    Vc = np.asarray(Vc, np.float64)
    eps, L, D = w.eps, w.L, w.D
    N = len(tok)
    h = Wd["embed"][np.asarray(tok)]
    S = np.empty((L, N, D))
    for l in range(L):
        S[l] = rb(h, "S")
        a = rb(h * Wd["attn_norm"][l], "hb") * _rinv(h, eps)
        q = _rope(_rmsnorm((a @ Wd["wq"][l].T).reshape(N, w.Hq, w.d), Wd["q_norm"][l], eps), pos, w.rope_base)
        o = _attend(rb(q, "q"), pos, bidx, Kc, Vc, l % w.k, lambda p: rb(p, "p"))
        h = h + rb(o.reshape(N, -1), "o") @ Wd["wo"][l].T
        f = rb(h * Wd["ffn_norm"][l], "hb") * _rinv(h, eps)
        gt = f @ Wd["w_gate"][l].T
        h = h + rb(gt / (1 + np.exp(-gt)) * (f @ Wd["w_up"][l].T), "act") @ Wd["w_down"][l].T
    logits = None
    if want_logits:
        logits = (rb(h * Wd["final_norm"], "hb") * _rinv(h, eps)) @ Wd["lm_head"].T
    rinv = [_rinv(S[l], eps) for l in range(L)]
    out = []
    for beta in (0, 1):
        g = Wd["src_norm"][beta]
        if many_rows:
            u = np.concatenate([rb(S[r] * rinv[r], "u") for r in range(0, L, w.p)], -1)
            Wr = np.concatenate([Wd["router"][beta][:, i * D:(i + 1) * D] * g[r]
                                 for i, r in enumerate(range(0, L, w.p))], -1)
            A = (u @ rb(Wr, "wf").T).reshape(N, L, w.k)
        else:
            u = np.concatenate([rb(S[r] * rinv[r] * g[r], "u") for r in range(0, L, w.p)], -1)
            A = (u @ Wd["router"][beta].T).reshape(N, L, w.k)
        xs = np.empty((w.k, N, w.Hkv, w.d))
        for j in range(w.k):
            m = sum(rb(A[:, l, j, None] * rinv[l], "mixw") * rb(g[l] * S[l], "mixs") for l in range(L))
            c = rb(m * Wd["chan_norm"][beta, j], "mb") * _rinv(m, eps)
            x = (c @ Wd["wk" if beta == 0 else "wv"][j].T).reshape(N, w.Hkv, w.d)
            if beta == 0:
                x = _rope(_rmsnorm(x, Wd["k_norm"][j], eps), pos, w.rope_base)
            xs[j] = rb(x, "kv")
        out.append(xs)
    return out[0], out[1], logits, S


FF_ROUNDING_POINTS = ("S", "hb", "router", "mix", "mb", "q", "kv", "p", "o", "act")


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


FEW_ROWS = 128  # group steps of at most this many rows take the few-row pool path


def cyclic_pass(w, W, tokens, cache, g, rounding=(), want_logits=False):
    """One cyclic pass of the model (groups G_q = {i : i mod g = q} in order,
    each step reading the cache as it stood when the step began, then
    appending its rows' keys and values) over tokens [B, T]; ``cache`` (a pair
    of float64 arrays [k, B, Hkv, T_max, d]) is updated in place.  Each step
    takes the pool path the HIP library takes for its row count.  Returns
    logits [B, T, V] (zeros where not computed) or None."""
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    logits = np.zeros((B, T, w.V)) if want_logits else None
    for q in range(min(g, T)):
        m = np.arange(q, T, g)
        bidx = np.repeat(np.arange(B), len(m))
        pos = np.tile(m, B)
        K, V, lg, _ = step(w, W, tokens[bidx, pos], pos, bidx, cache[0], cache[1], rounding,
                           many_rows=len(pos) > FEW_ROWS, want_logits=want_logits)
        cache[0][:, bidx, :, pos] = K.transpose(1, 0, 2, 3)
        cache[1][:, bidx, :, pos] = V.transpose(1, 0, 2, 3)
        if want_logits:
            logits[bidx, pos] = lg
    return logits


VANILLA_ROUNDING_POINTS = ("hb", "q", "p", "o", "act", "kv")


def _causal(q, qpos, K, V, kpos, rb_p):
    """Inclusive causal attention (key s visible to query i when kpos[s] <=
    qpos[i]) of q [N, Hq, d] to K/V [S, Hkv, d]; probabilities through rb_p."""
    N, Hq, d = q.shape
    G = Hq // K.shape[1]
    vis = kpos[None, :] <= qpos[:, None]
    out = np.zeros_like(q)
    for hq in range(Hq):
        sc = np.where(vis, q[:, hq] @ K[:, hq // G].T / np.sqrt(d), -np.inf)
        p = np.where(vis, np.exp(sc - sc.max(1, keepdims=True)), 0.0)
        out[:, hq] = rb_p(p) @ V[:, hq // G] / p.sum(1, keepdims=True)
    return out


def _vanilla_block(w, Wd, l, h, pos, Kprev, Vprev, kpos_prev, rb):
    """Block l of the vanilla model for rows h [N, D] at positions pos: their
    own keys/values (appended) plus the cached ones at kpos_prev."""
    eps = w.eps
    N = h.shape[0]
    a = rb(h * Wd["attn_norm"][l], "hb") * _rinv(h, eps)
    q = rb(_rope(_rmsnorm((a @ Wd["wq"][l].T).reshape(N, w.Hq, w.d), Wd["q_norm"][l], eps), pos, w.rope_base), "q")
    K = rb(_rope(_rmsnorm((a @ Wd["wk"][l].T).reshape(N, w.Hkv, w.d), Wd["k_norm"][l], eps), pos, w.rope_base),
           "kv")
    V = rb((a @ Wd["wv"][l].T).reshape(N, w.Hkv, w.d), "kv")
    Ka, Va = np.concatenate([Kprev, K]), np.concatenate([Vprev, V])
    o = _causal(q, pos, Ka, Va, np.concatenate([kpos_prev, pos]), lambda p: rb(p, "p"))
    h = h + rb(o.reshape(N, -1), "o") @ Wd["wo"][l].T
    f = rb(h * Wd["ffn_norm"][l], "hb") * _rinv(h, eps)
    gt = f @ Wd["w_gate"][l].T
    return h + rb(gt / (1 + np.exp(-gt)) * (f @ Wd["w_up"][l].T), "act") @ Wd["w_down"][l].T, K, V


def vanilla_forward(w, W, tokens, rounding=()):
    """The vanilla comparison model (per-layer keys/values, causal s <= i)
    over whole sequences tokens [B, T]. Returns (K, V [L, B, Hkv, T, d],
    logits [B, T, V])."""
    rb = lambda x, p: _rb(x, p in rounding)
    Wd = {n: np.asarray(a, np.float64) for n, a in W.items()}
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    pos = np.arange(T)
    Kc = np.zeros((w.L, B, w.Hkv, T, w.d))
    Vc = np.zeros_like(Kc)
    logits = np.zeros((B, T, w.V))
    none = np.zeros((0, w.Hkv, w.d))
    for b in range(B):
        h = Wd["embed"][tokens[b]]
        for l in range(w.L):
            h, K, V = _vanilla_block(w, Wd, l, h, pos, none, none, np.zeros(0, int), rb)
            Kc[l, b], Vc[l, b] = K.transpose(1, 0, 2), V.transpose(1, 0, 2)
        logits[b] = (rb(h * Wd["final_norm"], "hb") * _rinv(h, w.eps)) @ Wd["lm_head"].T
    return Kc, Vc, logits


def vanilla_decode_step(w, W, tokens_t, t, Kc, Vc, rounding=()):
    """One vanilla decode step at position t against the per-layer cache Kc/Vc
    [L, B, Hkv, T_max, d] (positions < t used, not modified). Returns
    (K, V [L, B, Hkv, d] of slot t, logits [B, V])."""
    rb = lambda x, p: _rb(x, p in rounding)
    Wd = {n: np.asarray(a, np.float64) for n, a in W.items()}
    B = len(tokens_t)
    Kt = np.zeros((w.L, B, w.Hkv, w.d))
    Vt = np.zeros_like(Kt)
    logits = np.zeros((B, w.V))
    kpos = np.arange(t)
    for b in range(B):
        h = Wd["embed"][np.asarray(tokens_t)[b:b + 1]]
        for l in range(w.L):
            Kp = np.asarray(Kc[l, b, :, :t], np.float64).transpose(1, 0, 2)
            Vp = np.asarray(Vc[l, b, :, :t], np.float64).transpose(1, 0, 2)
            h, K, V = _vanilla_block(w, Wd, l, h, np.array([t]), Kp, Vp, kpos, rb)
            Kt[l, b], Vt[l, b] = K[0], V[0]
        logits[b] = ((rb(h * Wd["final_norm"], "hb") * _rinv(h, w.eps)) @ Wd["lm_head"].T)[0]
    return Kt, Vt, logits
