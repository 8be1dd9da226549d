"""WhiteMatter oracle, float64 numpy (test infrastructure only; see package docstring).

Sources (the pages are web summaries of arXiv 2608.18486):

* [PL§3]  paperlayer.ai, "WhiteMatter: All-to-All Cross-Layer Connections via
          KV Mixing", section 3 METHOD (cross-layer KV pool, per-layer
          channel selection, execution schedules).
* [OD-how] onedev.kr, "WhiteMatter가 모든 층의 KV 재사용으로 캐시를 절반으로
          줄인다", section "어떻게 동작하나" (how it works): order of source
          RMSNorm -> router (stride p) -> signed mix -> channel RMSNorm ->
          per-channel K/V projection -> key norm + RoPE.
* [OD-diff] same page, section "무엇과 다른가" (what differs): strict causal
          attention s < i, append after the layer stack, fixed point
          KV = Model(X; KV), Jacobi and cyclic Gauss-Seidel groups
          G_q = {i : i mod g = q} processed for q = 0..g-1.
* [OD-use] same page, section "어떻게 쓰나" (how used): Qwen3-based decoder.

Readings where the pages are silent (each one is listed with its reason in
the design notes of this repository):

* R1  the L pooled states of a token are the inputs of its L blocks:
      h_0 = embedding, ..., h_{L-1}; h_L only feeds the LM head.
* R2  two branches (key, value), same structure, separate parameters.
* R3  the router is linear, no bias, no activation; its input is the
      concatenation of the normalised states of layers 0, p, 2p, ... < L in
      ascending order; output element l*k + j is the weight of source layer
      l in channel j.
* R4  one source-norm gain per (branch, layer); R6 W_K^j, W_V^j are
      [Hkv*d, D], no bias, output split head-major.
* R7  RMSNorm(x; g) = x / sqrt(mean(x^2) + eps) * g, eps = 1e-6.
* R8  queries get a per-head RMSNorm (gain per layer) before RoPE, as in
      Qwen3; keys get the per-channel key norm of [PL§3]/[OD-how].
* R9  RoPE pairs element m with m + d/2; angle = position * base^(-2m/d),
      position 0-based.
* R10 a query with no key (position 0) attends to nothing: output 0.
* R11 the initial cache is all zeros and unwritten slots are attended.
* R12 inside one group step every token reads the cache as it was when the
      step began; the step's own entries are written after all its tokens.
* R14 logits of a token come from its own group step.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64

__all__ = [
    "rmsnorm", "rope", "rope_angles", "silu", "group_positions", "channel_of_layer",
    "n_groups_nonempty", "cache_elems", "tokset_rows", "new_cache", "attend",
    "stack_forward", "router_weights", "mix_channels", "pool", "lm_logits", "step",
    "ar", "cyclic_pass", "jacobi_pass", "decode_step", "mix_kv", "channel_attn", "Model",
    "vanilla_new_cache", "vanilla_forward", "vanilla_decode_step", "ff_forward",
]


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------

def rmsnorm(x, gain, eps):
    """R7: x / sqrt(mean(x^2) + eps) * gain over the last axis ([OD-how]: every
    source state, every mixed channel; [PL§3]: keys)."""
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gain, F64)


def rope_angles(pos, d, base):
    """R9: angle[..., m] = pos * base^(-2m/d), m < d/2, in float64."""
    m = np.arange(d // 2, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * m / d)
    return np.asarray(pos, F64)[..., None] * inv_freq


def rope(x, pos, base):
    """Rotary embedding of x[..., H, d] at positions pos (shape x.shape[:-2]);
    element m is rotated together with element m + d/2 (R9)."""
    x = np.asarray(x, F64)
    d = x.shape[-1]
    h = d // 2
    ang = rope_angles(pos, d, base)[..., None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


# ---------------------------------------------------------------------------
# integer structure
# ---------------------------------------------------------------------------

def group_positions(T, g, q):
    """[OD-diff]: G_q = {i in [0, T) : i mod g = q}, ascending."""
    return list(range(q, T, g))


def n_groups_nonempty(T, g):
    return min(g, T)


def channel_of_layer(layer, k):
    """[PL§3] per-layer channel selection: layer l reads channel l mod k."""
    return layer % k


def cache_elems(k, B, T, Hkv, d):
    """[PL§3]: each of the key and value caches holds k*T*Hkv*d elements per
    sequence (k/L of an L-layer cache)."""
    return k * B * T * Hkv * d


def tokset_rows(B, M, s0, s_step):
    """Rows of a token set: row r = b*M + m sits at position s0 + m*s_step of
    sequence b. Returns (bidx, pos) int arrays of length B*M."""
    b = np.repeat(np.arange(B), M)
    m = np.tile(np.arange(M), B)
    return b, s0 + m * s_step


def new_cache(w, B):
    """R11: zero-initialised key and value caches [k, B, Hkv, T_max, d]."""
    shape = (w.k, B, w.Hkv, w.T_max, w.d)
    return np.zeros(shape, F64), np.zeros(shape, F64)


# ---------------------------------------------------------------------------
# the model
# ---------------------------------------------------------------------------

class Model:
    """Workload shape + float64 copies of the weights (names as in wm_inputs)."""

    def __init__(self, w, weights):
        self.w = w
        self.W = {n: np.asarray(a, F64) for n, a in weights.items()}


def attend(q, pos, bidx, Kc, Vc, c):
    """Strict causal GQA attention of each row to cache channel c ([OD-diff]:
    token i sees only s < i; [PL§3]: one channel per consumer layer).

    q [N, Hq, d]; Kc/Vc [k, B, Hkv, T_max, d]. Query head h uses KV head
    h // (Hq/Hkv). R10: a row at position 0 gets 0.
    """
    N, Hq, d = q.shape
    Hkv = Kc.shape[2]
    G = Hq // Hkv
    out = np.zeros((N, Hq, d), F64)
    for n in range(N):
        i = int(pos[n])
        if i == 0:
            continue
        b = int(bidx[n])
        for hk in range(Hkv):
            K = np.asarray(Kc[c, b, hk, :i], F64)
            V = np.asarray(Vc[c, b, hk, :i], F64)
            s = q[n, hk * G:(hk + 1) * G] @ K.T / math.sqrt(d)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[n, hk * G:(hk + 1) * G] = p @ V
    return out


def stack_forward(M, tok, pos, bidx, Kc, Vc):
    """Layer stack of every row against a fixed cache.

    Pre-norm Qwen3-style blocks ([OD-use]); layer l attends to channel
    l mod k ([PL§3]). Returns the state stack S [L, N, D] (R1: S[l] is the
    input of block l) and the final residual h_L [N, D].
    """
    w, W = M.w, M.W
    N = len(tok)
    h = W["embed"][np.asarray(tok)]
    S = np.empty((w.L, N, w.D), F64)
    for l in range(w.L):
        S[l] = h
        a = rmsnorm(h, W["attn_norm"][l], w.eps)
        q = (a @ W["wq"][l].T).reshape(N, w.Hq, w.d)
        q = rope(rmsnorm(q, W["q_norm"][l], w.eps), pos, w.rope_base)
        o = attend(q, pos, bidx, Kc, Vc, channel_of_layer(l, w.k))
        h = h + o.reshape(N, w.Hq * w.d) @ W["wo"][l].T
        b = rmsnorm(h, W["ffn_norm"][l], w.eps)
        h = h + (silu(b @ W["w_gate"][l].T) * (b @ W["w_up"][l].T)) @ W["w_down"][l].T
    return S, h


def _normed_sources(M, S, beta):
    w, W = M.w, M.W
    return [rmsnorm(S[l], W["src_norm"][beta, l], w.eps) for l in range(w.L)]


def router_weights(M, S, beta):
    """[OD-how]: the router reads only every p-th normalised source state and
    emits signed weights for all L source layers and k channels (R3).
    Returns A [N, L, k]."""
    w, W = M.w, M.W
    n = _normed_sources(M, S, beta)
    u = np.concatenate([n[l] for l in range(0, w.L, w.p)], axis=-1)
    return (u @ W["router"][beta].T).reshape(S.shape[1], w.L, w.k)


def mix_channels(M, S, beta, A=None):
    """m_j = sum_l A[l, j] * RMSNorm(S[l]) for j < k ([OD-how]). ``A`` may be a
    static [L, k] matrix (the static-mixing variant of the analysis section)
    or None for the router. Returns m [k, N, D]."""
    w = M.w
    n = _normed_sources(M, S, beta)
    if A is None:
        A = router_weights(M, S, beta)
    else:
        A = np.broadcast_to(np.asarray(A, F64), (S.shape[1], w.L, w.k))
    m = np.zeros((w.k, S.shape[1], w.D), F64)
    for j in range(w.k):
        for l in range(w.L):
            m[j] += A[:, l, j, None] * n[l]
    return m


def pool(M, S, pos, static_A=None):
    """Cross-layer KV pool of a set of tokens ([PL§3], [OD-how]).

    For each branch: mix the L normalised states into k channels, RMSNorm
    each channel, project with that channel's own matrix; keys then get the
    per-channel key norm (per head) and RoPE at the token's position, values
    stay raw. Returns K_new, V_new [k, N, Hkv, d].
    """
    w, W = M.w, M.W
    N = S.shape[1]
    out = []
    for beta in (0, 1):
        m = mix_channels(M, S, beta, None if static_A is None else static_A[beta])
        xs = np.empty((w.k, N, w.Hkv, w.d), F64)
        for j in range(w.k):
            c = rmsnorm(m[j], W["chan_norm"][beta, j], w.eps)
            if beta == 0:
                kj = (c @ W["wk"][j].T).reshape(N, w.Hkv, w.d)
                xs[j] = rope(rmsnorm(kj, W["k_norm"][j], w.eps), pos, w.rope_base)
            else:
                xs[j] = (c @ W["wv"][j].T).reshape(N, w.Hkv, w.d)
        out.append(xs)
    return out[0], out[1]


def lm_logits(M, hL):
    """Final RMSNorm then LM head (Qwen3-style decoder, [OD-use])."""
    w, W = M.w, M.W
    return rmsnorm(hL, W["final_norm"], w.eps) @ W["lm_head"].T


def _write(Kc, Vc, Kn, Vn, bidx, pos):
    for n in range(len(pos)):
        Kc[:, bidx[n], :, pos[n]] = Kn[:, n]
        Vc[:, bidx[n], :, pos[n]] = Vn[:, n]


def step(M, tokens, cache, bidx, pos, want_logits=False, static_A=None):
    """One group step: every row is evaluated against the same cache (R12),
    then the rows' pooled channels are written (append after the stack,
    [PL§3]). ``cache`` is updated in place. Returns logits [N, V] or None."""
    Kc, Vc = cache
    tok = np.asarray(tokens)[bidx, pos]
    S, hL = stack_forward(M, tok, pos, bidx, Kc, Vc)
    Kn, Vn = pool(M, S, pos, static_A)
    _write(Kc, Vc, Kn, Vn, bidx, pos)
    return lm_logits(M, hL) if want_logits else None


def ar(M, tokens, want_logits=False, static_A=None):
    """Exact autoregressive execution ([PL§3] execution schedules): token by
    token, each appended after its own stack. Returns (cache, logits[B,T,V])."""
    w = M.w
    B, T = np.asarray(tokens).shape
    cache = new_cache(w, B)
    logits = np.zeros((B, T, w.V), F64) if want_logits else None
    for i in range(T):
        bidx, pos = tokset_rows(B, 1, i, 1)
        lg = step(M, tokens, cache, bidx, pos, want_logits, static_A)
        if want_logits:
            logits[:, i] = lg
    return cache, logits


def cyclic_pass(M, tokens, cache, g, want_logits=False, static_A=None):
    """One cyclic Gauss-Seidel pass ([OD-diff]): groups G_q for q = 0..g-1 in
    order, tokens of a group in parallel, each group's entries visible to
    the later groups of the same pass. Updates ``cache`` in place; returns
    logits [B, T, V] (zeros where not computed) or None."""
    w = M.w
    B, T = np.asarray(tokens).shape
    logits = np.zeros((B, T, w.V), F64) if want_logits else None
    for q in range(min(g, T)):
        Mq = len(group_positions(T, g, q))
        bidx, pos = tokset_rows(B, Mq, q, g)
        lg = step(M, tokens, cache, bidx, pos, want_logits, static_A)
        if want_logits:
            logits[bidx, pos] = lg
    return logits


def jacobi_pass(M, tokens, cache, want_logits=False, static_A=None):
    """Jacobi pass ([PL§3]): all tokens in parallel, updates seen next pass
    only; the cyclic pass with g = 1."""
    return cyclic_pass(M, tokens, cache, 1, want_logits, static_A)


def decode_step(M, tokens_t, t, cache):
    """One decode step at position t for every sequence: stack against s < t,
    then append the token's channels at slot t ([PL§3]). tokens_t [B].
    Updates ``cache`` in place; returns logits [B, V]."""
    B = len(tokens_t)
    toks = np.zeros((B, t + 1), np.int64)
    toks[:, t] = tokens_t
    bidx, pos = tokset_rows(B, 1, t, 1)
    return step(M, toks, cache, bidx, pos, want_logits=True)


def mix_kv(M, S, B, Mrows, s0, s_step, cache, static_A=None):
    """Pool + append for a given state stack S [L, B*Mrows, D] whose rows sit at
    positions s0 + m*s_step; writes into ``cache`` in place. ``static_A``:
    constant [L, k] mixing per branch (the static-mixing variant) or None."""
    bidx, pos = tokset_rows(B, Mrows, s0, s_step)
    Kn, Vn = pool(M, np.asarray(S, F64), pos, static_A)
    _write(cache[0], cache[1], Kn, Vn, bidx, pos)


def channel_attn(w, layer, q, B, Mrows, s0, s_step, cache):
    """Consumer layer ``layer`` attention (channel layer mod k, strict causal)
    of already normalised and rotated queries q [B*Mrows, Hq, d].
    Returns [B*Mrows, Hq*d]."""
    bidx, pos = tokset_rows(B, Mrows, s0, s_step)
    o = attend(np.asarray(q, F64), pos, bidx, cache[0], cache[1], channel_of_layer(layer, w.k))
    return o.reshape(len(pos), w.Hq * w.d)


# ---------------------------------------------------------------------------
# vanilla baseline: the model the pages' efficiency figures compare against
# ---------------------------------------------------------------------------
# The same decoder with ordinary per-layer attention ([OD-use] Qwen3-style;
# the comparison model of [OD-diff] / [PL§3]): block l projects its own input
# to keys and values (W_K^l, W_V^l, key norm, RoPE), and position i attends to
# positions s <= i of its own layer (standard causal attention). The weight
# arrays wk / wv / k_norm hold one entry per layer (k = L).

def vanilla_new_cache(w, B):
    """Per-layer key and value caches [L, B, Hkv, T_max, d], zeros."""
    shape = (w.L, B, w.Hkv, w.T_max, w.d)
    return np.zeros(shape, F64), np.zeros(shape, F64)


def _vanilla_kv(M, l, a, pos):
    w, W = M.w, M.W
    N = a.shape[0]
    K = rope(rmsnorm((a @ W["wk"][l].T).reshape(N, w.Hkv, w.d), W["k_norm"][l], w.eps), pos, w.rope_base)
    V = (a @ W["wv"][l].T).reshape(N, w.Hkv, w.d)
    return K, V


def _causal_attention(q, K, V, qpos, kpos, inclusive):
    """Dense masked softmax attention of one sequence: q [N, Hq, d] at
    positions qpos, K/V [S, Hkv, d] at positions kpos; key s is visible to
    query i when kpos[s] <= qpos[i] (inclusive) or < (strict). Queries with no
    visible key get 0."""
    N, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    vis = (kpos[None, :] <= qpos[:, None]) if inclusive else (kpos[None, :] < qpos[:, None])
    out = np.zeros((N, Hq, d), F64)
    for hq in range(Hq):
        hk = hq // G
        sc = q[:, hq] @ K[:, hk].T / math.sqrt(d)
        sc = np.where(vis, sc, -np.inf)
        mx = np.max(sc, axis=1, keepdims=True)
        ok = np.isfinite(mx[:, 0])
        p = np.where(vis, np.exp(sc - np.where(ok[:, None], mx, 0.0)), 0.0)
        den = p.sum(axis=1, keepdims=True)
        out[ok, hq] = (p[ok] / den[ok]) @ V[:, hk]
    return out


def vanilla_forward(M, tokens, inclusive=True, want_logits=True):
    """Causal forward of whole sequences tokens [B, T] in one pass: every
    block computes the keys and values of all positions from its own input and
    attends causally (s <= i; strict s < i when ``inclusive`` is False).
    Returns (cache [L, B, Hkv, T_max, d] x 2 with positions < T filled,
    logits [B, T, V] or None)."""
    w, W = M.w, M.W
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    Kc, Vc = vanilla_new_cache(w, B)
    logits = np.zeros((B, T, w.V), F64) if want_logits else None
    pos = np.arange(T)
    for b in range(B):
        h = W["embed"][tokens[b]]
        for l in range(w.L):
            a = rmsnorm(h, W["attn_norm"][l], w.eps)
            q = rope(rmsnorm((a @ W["wq"][l].T).reshape(T, w.Hq, w.d), W["q_norm"][l], w.eps), pos, w.rope_base)
            K, V = _vanilla_kv(M, l, a, pos)
            Kc[l, b, :, :T] = K.transpose(1, 0, 2)
            Vc[l, b, :, :T] = V.transpose(1, 0, 2)
            o = _causal_attention(q, K, V, pos, pos, inclusive)
            h = h + o.reshape(T, w.Hq * w.d) @ W["wo"][l].T
            f = rmsnorm(h, W["ffn_norm"][l], w.eps)
            h = h + (silu(f @ W["w_gate"][l].T) * (f @ W["w_up"][l].T)) @ W["w_down"][l].T
        if want_logits:
            logits[b] = lm_logits(M, h)
    return (Kc, Vc), logits


def vanilla_decode_step(M, tokens_t, t, cache):
    """One decode step of the vanilla model at position t: block l appends the
    token's key and value at slot t of layer l, then attends to s <= t.
    ``cache`` (vanilla layout) is updated in place. Returns logits [B, V]."""
    w, W = M.w, M.W
    Kc, Vc = cache
    B = len(tokens_t)
    out = np.zeros((B, w.V), F64)
    pos = np.array([t])
    kpos = np.arange(t + 1)
    for b in range(B):
        h = W["embed"][np.asarray(tokens_t)[b:b + 1]]
        for l in range(w.L):
            a = rmsnorm(h, W["attn_norm"][l], w.eps)
            q = rope(rmsnorm((a @ W["wq"][l].T).reshape(1, w.Hq, w.d), W["q_norm"][l], w.eps), pos, w.rope_base)
            K, V = _vanilla_kv(M, l, a, pos)
            Kc[l, b, :, t] = K[0]
            Vc[l, b, :, t] = V[0]
            Ks = np.asarray(Kc[l, b, :, :t + 1], F64).transpose(1, 0, 2)
            Vs = np.asarray(Vc[l, b, :, :t + 1], F64).transpose(1, 0, 2)
            o = _causal_attention(q, Ks, Vs, pos, kpos, True)
            h = h + o.reshape(1, w.Hq * w.d) @ W["wo"][l].T
            f = rmsnorm(h, W["ffn_norm"][l], w.eps)
            h = h + (silu(f @ W["w_gate"][l].T) * (f @ W["w_up"][l].T)) @ W["w_down"][l].T
        out[b] = lm_logits(M, h)[0]
    return out


# ---------------------------------------------------------------------------
# feedback-free variant
# ---------------------------------------------------------------------------
# [PL§5] analysis / [OD] ablations: layer l sees only the states 0..l, so
# there is no deep-to-shallow feedback and no iteration. Reading (the pages
# give no more): k = L, consumer layer l reads channel l; channel l of a token
# mixes only its states 0..l, with router weights computed from the sampled
# normalised states r <= l (r in 0, p, 2p, ...) and the router rows of
# channel l; attention stays strictly causal (s < i). Then the channel-l keys
# and values of every position are known once layer l's input is, so one
# layer-synchronous pass computes the model.

def _ff_channel(M, S_upto, l, pos):
    """Keys/values of channel l for rows whose states 0..l are S_upto
    [l+1, N, D]. Returns K, V [N, Hkv, d]."""
    w, W = M.w, M.W
    N = S_upto.shape[1]
    sampled = [r for r in range(0, w.L, w.p) if r <= l]
    RD = w.R * w.D
    out = []
    for beta in (0, 1):
        n = [rmsnorm(S_upto[r], W["src_norm"][beta, r], w.eps) for r in range(l + 1)]
        u = np.concatenate([n[r] for r in sampled], axis=-1)          # [N, |sampled| * D]
        Wr = W["router"][beta].reshape(w.L, w.k, RD)[:, l, :len(sampled) * w.D]  # rows (src, channel l)
        A = u @ Wr[:l + 1].T                                              # [N, l+1]: sources 0..l
        m = np.zeros((N, w.D), F64)
        for src in range(l + 1):
            m += A[:, src, None] * n[src]
        c = rmsnorm(m, W["chan_norm"][beta, l], w.eps)
        if beta == 0:
            out.append(rope(rmsnorm((c @ W["wk"][l].T).reshape(N, w.Hkv, w.d), W["k_norm"][l], w.eps), pos,
                            w.rope_base))
        else:
            out.append((c @ W["wv"][l].T).reshape(N, w.Hkv, w.d))
    return out[0], out[1]


def ff_forward(M, tokens, want_logits=True, states=None):
    """The feedback-free model over whole sequences tokens [B, T] in one
    layer-synchronous pass. Returns (cache [k = L, B, Hkv, T_max, d] x 2 with
    positions < T filled, logits [B, T, V] or None). If ``states`` is a list,
    the state stack [L, T, D] of every sequence is appended to it."""
    w, W = M.w, M.W
    assert w.k == w.L, "the feedback-free model has one channel per layer"
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    Kc, Vc = new_cache(w, B)
    logits = np.zeros((B, T, w.V), F64) if want_logits else None
    pos = np.arange(T)
    for b in range(B):
        h = W["embed"][tokens[b]]
        S = np.empty((w.L, T, w.D), F64)
        for l in range(w.L):
            S[l] = h
            K, V = _ff_channel(M, S[:l + 1], l, pos)
            Kc[l, b, :, :T] = K.transpose(1, 0, 2)
            Vc[l, b, :, :T] = V.transpose(1, 0, 2)
            a = rmsnorm(h, W["attn_norm"][l], w.eps)
            q = rope(rmsnorm((a @ W["wq"][l].T).reshape(T, w.Hq, w.d), W["q_norm"][l], w.eps), pos, w.rope_base)
            o = _causal_attention(q, K, V, pos, pos, False)
            h = h + o.reshape(T, w.Hq * w.d) @ W["wo"][l].T
            f = rmsnorm(h, W["ffn_norm"][l], w.eps)
            h = h + (silu(f @ W["w_gate"][l].T) * (f @ W["w_up"][l].T)) @ W["w_down"][l].T
        if states is not None:
            states.append(S)
        if want_logits:
            logits[b] = lm_logits(M, h)
    return (Kc, Vc), logits
