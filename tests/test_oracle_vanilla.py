"""Pins of the oracle's vanilla baseline (per-layer K/V, causal attention):
the comparison model of the pages' efficiency figures.

  * With the strict mask (s < i) the vanilla forward is the WhiteMatter model
    run token by token with k = L, a one-hot static mixing (channel j = source
    state j), unit source gains, channel gains equal to the attention-norm
    gains and eps = 0 (then RMSNorm(RMSNorm(h; 1); g) = RMSNorm(h; g)): two
    independent formulations of the same function.
  * Causality: changing the last token changes no earlier cache entry or
    logit.
  * A single token attends only to itself: its attention output is its own
    value vector (closed form of a one-element softmax).
  * The decode step continues the forward: forward over T tokens, then one
    step at t = T, equals the forward over T + 1 tokens at position T.
"""
import numpy as np
import pytest

import oracle as O
from tests.helpers import max_abs_rel
from wm_inputs import WORKLOADS, make_tokens, make_weights


def _tiny(T=24, eps=None):
    w = WORKLOADS["tiny_fp32"]
    w = w.replace(k=w.L, T=T, T_max=T + 1)
    if eps is not None:
        w = w.replace(eps=eps)
    W = make_weights(w, seed=0, gains="perturbed")
    tok = make_tokens(w, seed=1, B=2, T=T, dist="uniform")
    return w, W, tok


def test_strict_vanilla_is_one_hot_whitematter():
    w, W, tok = _tiny(eps=0.0)
    W = dict(W)
    W["src_norm"] = np.ones_like(W["src_norm"])
    W["chan_norm"] = np.stack([W["attn_norm"], W["attn_norm"]])  # [2, k = L, D]
    onehot = np.eye(w.L)
    wm_cache, wm_logits = O.ar(O.Model(w, W), tok, want_logits=True, static_A=(onehot, onehot))
    (Kv, Vv), v_logits = O.vanilla_forward(O.Model(w, W), tok, inclusive=False)
    T = tok.shape[1]
    assert max_abs_rel(Kv[..., :T, :], wm_cache[0][..., :T, :]) < 1e-12
    assert max_abs_rel(Vv[..., :T, :], wm_cache[1][..., :T, :]) < 1e-12
    assert max_abs_rel(v_logits, wm_logits) < 1e-12
    # and the mask matters: the inclusive model differs
    (_, _), inc_logits = O.vanilla_forward(O.Model(w, W), tok, inclusive=True)
    assert max_abs_rel(inc_logits, v_logits) > 1e-3


def test_vanilla_is_causal():
    w, W, tok = _tiny()
    M = O.Model(w, W)
    (K1, V1), lg1 = O.vanilla_forward(M, tok)
    tok2 = tok.copy()
    tok2[:, -1] = (tok2[:, -1] + 7) % w.V
    (K2, V2), lg2 = O.vanilla_forward(M, tok2)
    T = tok.shape[1]
    np.testing.assert_array_equal(K1[..., :T - 1, :], K2[..., :T - 1, :])
    np.testing.assert_array_equal(V1[..., :T - 1, :], V2[..., :T - 1, :])
    np.testing.assert_array_equal(lg1[:, :T - 1], lg2[:, :T - 1])
    assert np.abs(lg1[:, T - 1] - lg2[:, T - 1]).max() > 0


def test_single_token_attends_to_itself():
    w, W, tok = _tiny(T=1)
    M = O.Model(w, W)
    (Kc, Vc), lg = O.vanilla_forward(M, tok)
    G = w.Hq // w.Hkv
    for b in range(tok.shape[0]):
        h = W["embed"][tok[b, 0]].astype(np.float64)
        for l in range(w.L):
            a = h / np.sqrt(np.mean(h * h) + w.eps) * W["attn_norm"][l]
            v = (a @ W["wv"][l].T.astype(np.float64)).reshape(w.Hkv, w.d)
            assert max_abs_rel(Vc[l, b, :, 0], v) < 1e-12
            o = np.concatenate([v[hq // G] for hq in range(w.Hq)])  # softmax over one key = 1
            h = h + o @ W["wo"][l].T.astype(np.float64)
            f = h / np.sqrt(np.mean(h * h) + w.eps) * W["ffn_norm"][l]
            g_, u_ = f @ W["w_gate"][l].T.astype(np.float64), f @ W["w_up"][l].T.astype(np.float64)
            h = h + (g_ / (1.0 + np.exp(-g_)) * u_) @ W["w_down"][l].T.astype(np.float64)
        hn = h / np.sqrt(np.mean(h * h) + w.eps) * W["final_norm"]
        assert max_abs_rel(lg[b, 0], hn @ W["lm_head"].T.astype(np.float64)) < 1e-12


def test_decode_continues_the_forward():
    w, W, tok = _tiny(T=12)
    M = O.Model(w, W)
    T = tok.shape[1] - 1
    (Kc, Vc), _ = O.vanilla_forward(M, tok[:, :T], want_logits=False)
    lg = O.vanilla_decode_step(M, tok[:, T], T, (Kc, Vc))
    (Kf, Vf), lgf = O.vanilla_forward(M, tok)
    assert max_abs_rel(lg, lgf[:, T]) < 1e-12
    assert max_abs_rel(Kc[..., :T + 1, :], Kf[..., :T + 1, :]) < 1e-12
    assert max_abs_rel(Vc[..., :T + 1, :], Vf[..., :T + 1, :]) < 1e-12


# ---------------------------------------------------------------- feedback-free variant

def _ff_case(T=20, p=2):
    w = WORKLOADS["tiny_fp32"]
    w = w.replace(k=w.L, p=p, T=T, T_max=T)
    W = make_weights(w, seed=0, gains="perturbed")
    tok = make_tokens(w, seed=1, B=2, T=T, dist="uniform")
    return w, W, tok


@pytest.mark.parametrize("p", [1, 2, 3])
def test_feedback_free_is_whitematter_with_a_masked_router(p):
    """The layer-synchronous feedback-free forward equals the WhiteMatter model
    (k = L) run token by token once the router rows of channel l are zeroed
    for sources l' > l and for the input blocks of sampled states r > l: then
    every channel of the full model depends on states 0..l only."""
    w, W, tok = _ff_case(p=p)
    (Kf, Vf), lgf = O.ff_forward(O.Model(w, W), tok)
    Wm = dict(W)
    router = W["router"].copy().reshape(2, w.L, w.k, w.R, w.D)
    for l in range(w.L):            # channel
        for src in range(w.L):
            if src > l:
                router[:, src, l] = 0.0
        for ri, r in enumerate(range(0, w.L, w.p)):
            if r > l:
                router[:, :, l, ri] = 0.0
    Wm["router"] = router.reshape(W["router"].shape)
    cache, lg = O.ar(O.Model(w, Wm), tok, want_logits=True)
    T = tok.shape[1]
    assert max_abs_rel(Kf[..., :T, :], cache[0][..., :T, :]) < 1e-12
    assert max_abs_rel(Vf[..., :T, :], cache[1][..., :T, :]) < 1e-12
    assert max_abs_rel(lgf, lg) < 1e-12
    # and the unmasked router does give a different model (deep states matter)
    cache2, lg2 = O.ar(O.Model(w, W), tok, want_logits=True)
    assert max_abs_rel(lg2, lg) > 1e-4


def test_feedback_free_is_causal():
    w, W, tok = _ff_case()
    M = O.Model(w, W)
    (K1, V1), lg1 = O.ff_forward(M, tok)
    tok2 = tok.copy()
    tok2[:, -1] = (tok2[:, -1] + 5) % w.V
    (K2, V2), lg2 = O.ff_forward(M, tok2)
    T = tok.shape[1]
    np.testing.assert_array_equal(K1[..., :T - 1, :], K2[..., :T - 1, :])
    np.testing.assert_array_equal(lg1[:, :T - 1], lg2[:, :T - 1])
