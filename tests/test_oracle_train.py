"""The training oracle (oracle/wm_train.py) pinned to things other than itself.

* Its torch forward is the numpy oracle's cyclic pass (caches and logits at
  1e-12 after several passes), and its loss is the numpy R25 cross-entropy of
  those logits.
* Its gradient equals central finite differences of the truncated objective
  computed by the numpy oracle alone (``truncated_loss``, whose no-gradient
  passes run at the base weights): on every parameter tensor, at its
  largest-gradient entry and at random entries, for the cyclic (g = 2),
  Jacobi (g = 1) and autoregressive (g = T) schedules.
* The truncation matters and is the one the pages describe: finite
  differences of the untruncated objective (the first pass perturbed too)
  differ from the truncated gradient, and equal the gradient of a step with
  no pass left out (n_nograd = 0, n_grad = 3).
"""
import numpy as np
import pytest

import oracle as O
from oracle import wm_train as TR
from wm_inputs import WORKLOADS, make_tokens, make_weights

FD_H = 1e-5


def _fd_case(g=2, **kw):
    w = WORKLOADS["tiny_fp32"].replace(L=3, D=16, Hq=2, Hkv=1, d=8, F=24, k=2, p=2, V=11, B=2, T=6, T_max=6, g=g,
                                       **kw)
    W = make_weights(w, seed=0, gains="perturbed")
    W = {n: a.astype(np.float64) for n, a in W.items()}
    tokens = make_tokens(w, seed=1)
    return w, W, tokens


def _entries(grad, rng, n_random=3):
    flat = np.abs(grad).ravel()
    idx = [int(np.argmax(flat))] + [int(i) for i in rng.choice(flat.size, n_random, replace=False)]
    return [np.unravel_index(i, grad.shape) for i in idx]


def _fd(w, W, tokens, g, name, ix, n_nograd, n_grad, perturb_nograd):
    def f(delta):
        Wp = dict(W)
        Wp[name] = W[name].copy()
        Wp[name][ix] += delta
        Mg = O.Model(w, Wp)
        Mn = Mg if perturb_nograd else O.Model(w, W)
        return TR.truncated_loss(Mn, Mg, tokens, g, n_nograd, n_grad)

    # central differences at h and h/2, Richardson-combined (error O(h^4): the
    # RMSNorms of small states make the loss strongly curved)
    d1 = (f(FD_H) - f(-FD_H)) / (2 * FD_H)
    d2 = (f(FD_H / 2) - f(-FD_H / 2)) / FD_H
    return (4 * d2 - d1) / 3


def test_forward_is_the_oracle():
    w = WORKLOADS["tiny_fp32"].replace(B=2, T=24, T_max=32, g=5, L=3, k=2)
    W = make_weights(w, seed=0, gains="perturbed")
    tokens = make_tokens(w, seed=1)
    K, V, lg = TR.forward_passes(O.Model(w, W), tokens, w.g, 3)
    M = O.Model(w, W)
    cache = O.new_cache(w, w.B)
    for i in range(3):
        ref = O.cyclic_pass(M, tokens, cache, w.g, want_logits=(i == 2))
    scale = lambda a: max(np.max(np.abs(a)), 1e-30)
    assert np.max(np.abs(K - cache[0])) / scale(cache[0]) < 1e-12
    assert np.max(np.abs(V - cache[1])) / scale(cache[1]) < 1e-12
    assert np.max(np.abs(lg - ref)) / scale(ref) < 1e-12


def test_loss_is_the_numpy_cross_entropy():
    w, W, tokens = _fd_case()
    M = O.Model(w, W)
    loss, _ = TR.train_step(M, tokens, w.g, 1, 2)
    assert abs(loss - TR.truncated_loss(M, M, tokens, w.g, 1, 2)) < 1e-12
    # the R25 cross-entropy written out for one prediction
    lg = np.array([[[0.5, -1.0, 2.0], [0.0, 0.0, 0.0]]])
    tok = np.array([[0, 2]])
    assert abs(TR.next_token_ce(lg, tok) - (np.log(np.exp(0.5) + np.exp(-1.0) + np.exp(2.0)) - 2.0)) < 1e-15


@pytest.mark.parametrize("g", [2, 1, 6])
def test_gradient_matches_central_differences(g):
    w, W, tokens = _fd_case(g=g)
    loss, grads = TR.train_step(O.Model(w, W), tokens, g, 1, 2)
    rng = np.random.default_rng(7)
    worst = 0.0
    for name in TR.PARAM_NAMES:
        gmax = np.max(np.abs(grads[name]))
        assert gmax > 0, name  # every parameter reaches the loss
        for ix in _entries(grads[name], rng):
            fd = _fd(w, W, tokens, g, name, ix, 1, 2, perturb_nograd=False)
            err = abs(fd - grads[name][ix]) / gmax
            worst = max(worst, err)
            assert err < 1e-6, (name, ix, fd, grads[name][ix])
    print(f"g={g}: loss {loss:.6f}, worst |fd - autograd| / max|grad| = {worst:.1e}")


def test_truncation_is_in_effect():
    """The first pass is left out of the gradient: the untruncated objective's
    finite differences differ from the truncated gradient, and they are the
    gradient of n_nograd = 0, n_grad = 3."""
    w, W, tokens = _fd_case()
    M = O.Model(w, W)
    _, gt = TR.train_step(M, tokens, w.g, 1, 2)
    _, gfull = TR.train_step(M, tokens, w.g, 0, 3)
    rng = np.random.default_rng(11)
    gap = 0.0
    for name in ("wq", "router", "wk", "src_norm", "embed"):
        gmax = np.max(np.abs(gfull[name]))
        for ix in _entries(gfull[name], rng, 2):
            fd = _fd(w, W, tokens, w.g, name, ix, 1, 2, perturb_nograd=True)
            assert abs(fd - gfull[name][ix]) / gmax < 1e-6, (name, ix)
            gap = max(gap, abs(fd - gt[name][ix]) / gmax)
    print(f"largest gap between the untruncated derivative and the truncated gradient: {gap:.2e}")
    assert gap > 1e-3
