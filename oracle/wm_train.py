"""Training step with truncated backpropagation — oracle, TEST INFRASTRUCTURE
ONLY (see the package docstring: only tests, the smoke check and the bench's
CPU baseline may use it).

Sources:

* [OD-diff] onedev.kr, "WhiteMatter가 모든 층의 KV 재사용으로 캐시를 절반으로
  줄인다", section "무엇과 다른가" (what differs): training uses truncated
  backpropagation, sending gradients only through the last n_g passes.
* [OD-use] same page, section "어떻게 쓰나" (how used): WhiteMatter trains with
  one cyclic pass without gradients followed by two passes with gradients.
* [PL§3] paperlayer.ai, §3 METHOD, "Execution schedules": parallel training
  treats the feedback dependency as a fixed-point problem solved by passes.
* [PL§4] same page, §4 EXPERIMENTS, "Compute cost": the training FLOP
  multiplier is below the pass count because of the truncation.

Readings (the pages do not spell these out; each is listed with its reason in
the design notes of this repository):

* R25 the training objective is next-token cross-entropy on the logits of the
      last pass: position i < T-1 of sequence b predicts tokens[b, i+1]; the
      loss is the mean over the B*(T-1) predictions.
* R26 truncation: the passes start from the zero cache (R11); the cache left
      by the n_nograd passes without gradient is a constant, and the gradient
      flows through the n_grad passes after it, including, inside a pass,
      from a group step back to the earlier group steps whose cache entries
      it read.
* R27 the gradient is taken with respect to every parameter of the model
      (the wm_inputs.weight_shapes names), summed over the batch through the
      mean of R25.

Two independent computations of the same objective live here:

``truncated_loss``  float64 numpy, built only from ``wm_oracle`` (cyclic
                    passes as defined there, then the R25 cross-entropy); the
                    tests take central finite differences of it.
``train_step``      the same forward written with torch float64 CPU ops (the
                    steps of ``wm_oracle.stack_forward`` / ``pool`` /
                    ``cyclic_pass`` in the same order) so that torch.autograd
                    gives the gradient; the tests pin its forward to
                    ``wm_oracle`` and its gradient to the finite differences
                    of ``truncated_loss``.
"""
from __future__ import annotations

import math

import numpy as np

from . import wm_oracle as O

PARAM_NAMES = ("embed", "lm_head", "final_norm", "attn_norm", "wq", "q_norm", "wo", "ffn_norm", "w_gate",
               "w_up", "w_down", "src_norm", "router", "chan_norm", "wk", "wv", "k_norm")


# ---------------------------------------------------------------------------
# float64 numpy objective (finite-difference reference)
# ---------------------------------------------------------------------------

def next_token_ce(logits, tokens):
    """R25: mean over b, i < T-1 of logsumexp(logits[b, i]) - logits[b, i, tokens[b, i+1]]."""
    z = np.asarray(logits, np.float64)[:, :-1]
    tgt = np.asarray(tokens)[:, 1:]
    zmax = z.max(axis=-1, keepdims=True)
    lse = np.log(np.exp(z - zmax).sum(axis=-1)) + zmax[..., 0]
    picked = np.take_along_axis(z, tgt[..., None].astype(np.int64), axis=-1)[..., 0]
    return float(np.mean(lse - picked))


def truncated_loss(M_nograd, M_grad, tokens, g, n_nograd=1, n_grad=2):
    """R25/R26 with wm_oracle: n_nograd cyclic passes from the zero cache with
    the weights of ``M_nograd``, then n_grad passes with those of ``M_grad``;
    the loss of the last pass's logits.  With M_nograd fixed at the base
    weights and M_grad perturbed, central differences of this function are
    the truncated gradient."""
    B, T = np.asarray(tokens).shape
    cache = O.new_cache(M_grad.w, B)
    for _ in range(n_nograd):
        O.cyclic_pass(M_nograd, tokens, cache, g)
    logits = None
    for i in range(n_grad):
        logits = O.cyclic_pass(M_grad, tokens, cache, g, want_logits=(i == n_grad - 1))
    return next_token_ce(logits, tokens)


# ---------------------------------------------------------------------------
# torch float64 forward + autograd
# ---------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _rms(x, g, eps):
    torch = _torch()
    return x / torch.sqrt((x * x).mean(-1, keepdim=True) + eps) * g


def _rope(x, pos, base):
    """x [N, H, d] at positions pos [N]; element m turns with m + d/2 (R9)."""
    torch = _torch()
    d = x.shape[-1]
    h = d // 2
    ang = torch.from_numpy(O.rope_angles(np.asarray(pos), d, base))[:, None, :]
    c, s = torch.cos(ang).to(x.dtype), torch.sin(ang).to(x.dtype)
    x1, x2 = x[..., :h], x[..., h:]
    return torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], dim=-1)


def _attend(q, pos, bidx, Kc, Vc, c):
    """Strict-causal attention (s < i) of rows q [N, Hq, d] to channel c; a row
    at position 0 gets 0 (R10).  Keys at s >= i get probability exactly 0."""
    torch = _torch()
    N, Hq, d = q.shape
    Hkv, T = Kc.shape[2], Kc.shape[3]
    G = Hq // Hkv
    K = Kc[c][torch.as_tensor(bidx)]  # [N, Hkv, T, d]
    V = Vc[c][torch.as_tensor(bidx)]
    s = torch.matmul(q.reshape(N, Hkv, G, d), K.transpose(-1, -2)) / math.sqrt(d)  # [N, Hkv, G, T]
    masked = torch.arange(T)[None, :] >= torch.as_tensor(np.asarray(pos))[:, None]
    s = s.masked_fill(masked[:, None, None, :], -math.inf)
    m = s.amax(dim=-1, keepdim=True).detach()  # (softmax does not depend on the shift)
    m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
    p = torch.exp(s - m)
    den = p.sum(dim=-1, keepdim=True)
    den = torch.where(den > 0, den, torch.ones_like(den))
    return torch.matmul(p / den, V).reshape(N, Hq, d)


def _stack(P, w, tok, pos, bidx, Kc, Vc):
    """wm_oracle.stack_forward in torch: returns S [L, N, D] and h_L."""
    torch = _torch()
    N = len(tok)
    h = P["embed"][torch.as_tensor(tok)]
    S = []
    for l in range(w.L):
        S.append(h)
        a = _rms(h, P["attn_norm"][l], w.eps)
        q = (a @ P["wq"][l].T).reshape(N, w.Hq, w.d)
        q = _rope(_rms(q, P["q_norm"][l], w.eps), pos, w.rope_base)
        o = _attend(q, pos, bidx, Kc, Vc, O.channel_of_layer(l, w.k))
        h = h + o.reshape(N, w.Hq * w.d) @ P["wo"][l].T
        b = _rms(h, P["ffn_norm"][l], w.eps)
        gt = b @ P["w_gate"][l].T
        h = h + (gt * torch.sigmoid(gt) * (b @ P["w_up"][l].T)) @ P["w_down"][l].T
    return torch.stack(S), h


def _pool(P, w, S, pos):
    """wm_oracle.pool in torch: K_new, V_new [k, N, Hkv, d]."""
    torch = _torch()
    N = S.shape[1]
    out = []
    for beta in (0, 1):
        n = [_rms(S[l], P["src_norm"][beta, l], w.eps) for l in range(w.L)]
        u = torch.cat([n[l] for l in range(0, w.L, w.p)], dim=-1)
        A = (u @ P["router"][beta].T).reshape(N, w.L, w.k)
        xs = []
        for j in range(w.k):
            m = torch.zeros_like(n[0])
            for l in range(w.L):
                m = m + A[:, l, j, None] * n[l]
            c = _rms(m, P["chan_norm"][beta, j], w.eps)
            if beta == 0:
                kj = (c @ P["wk"][j].T).reshape(N, w.Hkv, w.d)
                xs.append(_rope(_rms(kj, P["k_norm"][j], w.eps), pos, w.rope_base))
            else:
                xs.append((c @ P["wv"][j].T).reshape(N, w.Hkv, w.d))
        out.append(torch.stack(xs))
    return out[0], out[1]


def _pass(P, w, tokens, Kc, Vc, g, want_logits):
    """wm_oracle.cyclic_pass in torch, the cache as values (each group writes
    into a copy, so the entries an earlier step read stay as they were)."""
    torch = _torch()
    B, T = tokens.shape
    logits = torch.zeros((B, T, w.V), dtype=Kc.dtype) if want_logits else None
    for q in range(O.n_groups_nonempty(T, g)):
        Mq = len(O.group_positions(T, g, q))
        bidx, pos = O.tokset_rows(B, Mq, q, g)
        tok = tokens[bidx, pos]
        S, hL = _stack(P, w, tok, pos, bidx, Kc, Vc)
        Kn, Vn = _pool(P, w, S, pos)
        Kc, Vc = Kc.clone(), Vc.clone()
        ib, ip = torch.as_tensor(bidx), torch.as_tensor(pos)
        Kc[:, ib, :, ip] = Kn.permute(1, 0, 2, 3)
        Vc[:, ib, :, ip] = Vn.permute(1, 0, 2, 3)
        if want_logits:
            lg = _rms(hL, P["final_norm"], w.eps) @ P["lm_head"].T
            logits = logits.index_put((ib, ip), lg)
    return Kc, Vc, logits


def _ce(logits, tokens):
    torch = _torch()
    z = logits[:, :-1]
    tgt = torch.as_tensor(np.asarray(tokens)[:, 1:].astype(np.int64))
    return (torch.logsumexp(z, dim=-1) - torch.gather(z, -1, tgt[..., None])[..., 0]).mean()


def forward_passes(M, tokens, g, n_passes):
    """The torch forward alone (no gradient): cache and last-pass logits after
    n_passes cyclic passes from the zero cache, as float64 numpy."""
    torch = _torch()
    w = M.w
    tokens = np.asarray(tokens)
    with torch.no_grad():
        P = {n: torch.from_numpy(np.asarray(M.W[n], np.float64)) for n in PARAM_NAMES}
        shape = (w.k, tokens.shape[0], w.Hkv, w.T_max, w.d)
        Kc, Vc = torch.zeros(shape, dtype=torch.float64), torch.zeros(shape, dtype=torch.float64)
        lg = None
        for i in range(n_passes):
            Kc, Vc, lg = _pass(P, w, tokens, Kc, Vc, g, want_logits=(i == n_passes - 1))
    return Kc.numpy(), Vc.numpy(), lg.numpy()


def train_step(M, tokens, g, n_nograd=1, n_grad=2, dtype=None):
    """R25-R27: loss and gradient of one training step.  Returns (loss,
    {name: float64 array of the parameter's shape}).  ``dtype`` (a torch
    float type, float64 by default) is the arithmetic; float32 gives the
    rounding floor of a float32 implementation of the same steps."""
    torch = _torch()
    dtype = torch.float64 if dtype is None else dtype
    w = M.w
    tokens = np.asarray(tokens)
    P = {n: torch.tensor(np.asarray(M.W[n], np.float64), dtype=dtype, requires_grad=True) for n in PARAM_NAMES}
    shape = (w.k, tokens.shape[0], w.Hkv, w.T_max, w.d)
    Kc, Vc = torch.zeros(shape, dtype=dtype), torch.zeros(shape, dtype=dtype)
    with torch.no_grad():
        for _ in range(n_nograd):
            Kc, Vc, _ = _pass(P, w, tokens, Kc, Vc, g, want_logits=False)
    Kc, Vc = Kc.detach(), Vc.detach()
    logits = None
    for i in range(n_grad):
        Kc, Vc, logits = _pass(P, w, tokens, Kc, Vc, g, want_logits=(i == n_grad - 1))
    loss = _ce(logits, tokens)
    loss.backward()
    return float(loss.detach()), {n: P[n].grad.numpy().astype(np.float64) for n in PARAM_NAMES}
