"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a closed form, a library
routine the definition reduces to (torch's rms_norm / scaled_dot_product_attention /
complex multiplication), an invariant of the method stated on the pages, or the
separately written scalar brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle as O
from oracle.brute import brute_ar
from tests.helpers import max_abs_rel
from wm_inputs import WORKLOADS, make_tokens, make_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# a tiny model: GQA (G=2), k < L, stride p=2 reads layers 0 and 2
TINY = WORKLOADS["tiny_fp32"].replace(L=3, D=16, Hq=4, Hkv=2, d=8, F=24, k=2, p=2, V=13,
                                       B=2, T=7, T_max=8)


def tiny_model(w=TINY, scale=10.0, gains="perturbed", seed=0):
    """Weights N(0, 0.02) * scale so that the feedback path has O(1) effect."""
    W = make_weights(w, seed=seed, gains=gains)
    for n in W:
        if n not in ("final_norm", "attn_norm", "q_norm", "ffn_norm", "src_norm", "chan_norm", "k_norm"):
            W[n] = W[n].astype(np.float64) * scale
    return O.Model(w, W)


def tiny_tokens(w=TINY, seed=1):
    return make_tokens(w, seed=seed, dist="uniform")


# ---------------------------------------------------------------------------
# elementwise definitions
# ---------------------------------------------------------------------------

def test_rmsnorm_matches_torch_rms_norm():
    r = np.random.default_rng(0)
    x = r.standard_normal((5, 33))
    g = 1 + 0.1 * r.standard_normal(33)
    ref = Fnn.rms_norm(torch.from_numpy(x), (33,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    assert max_abs_rel(O.rmsnorm(x, g, 1e-6), ref) < 1e-14


def test_rmsnorm_constant_vector_closed_form():
    c, eps = -3.0, 1e-6
    y = O.rmsnorm(np.full(8, c), np.arange(1, 9, dtype=float), eps)
    assert np.allclose(y, c / math.sqrt(c * c + eps) * np.arange(1, 9), rtol=0, atol=1e-15)


def test_rope_is_complex_rotation_of_half_split_pairs():
    # element m and m + d/2 form the complex number x_m + i x_{m+d/2}, rotated by pos*base^(-2m/d)
    r = np.random.default_rng(1)
    d, base = 16, 1e6
    x = r.standard_normal((3, 2, d))
    pos = np.array([0, 5, 2047])
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    theta = pos[:, None, None] * base ** (-np.arange(d // 2) * 2.0 / d)
    zr = z * np.exp(1j * theta)
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.max(np.abs(O.rope(x, pos, base) - ref)) < 1e-12
    assert np.array_equal(O.rope(x[:1], pos[:1], base), x[:1])  # position 0 is the identity


def test_rope_scores_depend_on_relative_position_only():
    r = np.random.default_rng(2)
    q, k = r.standard_normal((1, 1, 32)), r.standard_normal((1, 1, 32))
    s1 = np.sum(O.rope(q, np.array([9]), 1e4) * O.rope(k, np.array([4]), 1e4))
    s2 = np.sum(O.rope(q, np.array([109]), 1e4) * O.rope(k, np.array([104]), 1e4))
    assert abs(s1 - s2) < 1e-10


def test_attend_matches_sdpa_with_strict_causal_mask():
    r = np.random.default_rng(3)
    k_, B, Hkv, Tm, d, Hq = 3, 2, 2, 12, 8, 6
    Kc, Vc = r.standard_normal((2, k_, B, Hkv, Tm, d))
    B_, M, s0, st = 2, 4, 1, 3  # positions 1, 4, 7, 10
    bidx, pos = O.tokset_rows(B_, M, s0, st)
    q = r.standard_normal((B_ * M, Hq, d))
    c = 2
    got = O.attend(q, pos, bidx, Kc, Vc, c)
    G = Hq // Hkv
    for n in range(len(pos)):
        K = torch.from_numpy(Kc[c, bidx[n]]).repeat_interleave(G, 0)  # [Hq, Tm, d]
        V = torch.from_numpy(Vc[c, bidx[n]]).repeat_interleave(G, 0)
        mask = torch.arange(Tm) < int(pos[n])  # strict: s < i
        ref = Fnn.scaled_dot_product_attention(torch.from_numpy(q[n])[:, None], K, V,
                                               attn_mask=mask[None, None, :])[:, 0].numpy()
        assert max_abs_rel(got[n], ref) < 1e-13


def test_attend_position_zero_is_zero():
    Kc = np.ones((1, 1, 1, 4, 4))
    out = O.attend(np.ones((1, 1, 4)), np.array([0]), np.array([0]), Kc, Kc, 0)
    assert np.array_equal(out, np.zeros_like(out))


# ---------------------------------------------------------------------------
# integer structure
# ---------------------------------------------------------------------------

def test_group_schedule_golden():
    with open(os.path.join(GOLDEN, "group_schedule.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        T, g = case["T"], case["g"]
        got = [O.group_positions(T, g, q) for q in range(g)]
        assert got == case["groups"]


@pytest.mark.parametrize("T,g", [(128, 16), (7, 3), (5, 9), (2048, 16), (1, 1), (10, 10)])
def test_group_schedule_partitions_positions(T, g):
    seen = []
    for q in range(g):
        G = O.group_positions(T, g, q)
        assert all(i % g == q for i in G)
        assert len(G) == max(0, -(-(T - q) // g))
        seen += G
    assert sorted(seen) == list(range(T))


def test_channel_of_layer_and_cache_size():
    with open(os.path.join(GOLDEN, "cache_size.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        L, k = case["L"], case["k"]
        assert [O.channel_of_layer(l, k) for l in range(L)] == case["channel_of_layer"]
        ratio = O.cache_elems(k, 3, 100, 2, 64) / O.cache_elems(L, 3, 100, 2, 64)
        assert ratio == pytest.approx(case["ratio_to_vanilla"], rel=0, abs=1e-15)


# ---------------------------------------------------------------------------
# router and mix
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L,p,blk,l0,j0", [(3, 2, 1, 2, 1), (4, 3, 1, 0, 0), (5, 1, 4, 3, 1)])
def test_one_hot_router_closed_form(L, p, blk, l0, j0):
    """Router weight matrix with a single entry: A[l0, j0] = -0.7 * n_{p*blk}[col0]
    and every other weight 0, so channel j0 = A[l0, j0] * n_{l0}, others 0."""
    w = TINY.replace(L=L, p=p)
    M = tiny_model(w)
    col0 = 5
    R = w.R
    for beta in (0, 1):
        M.W["router"][beta] = 0.0
        M.W["router"][beta][l0 * w.k + j0, blk * w.D + col0] = -0.7
    S = np.random.default_rng(4).standard_normal((L, 3, w.D))
    assert M.W["router"].shape[-1] == R * w.D
    for beta in (0, 1):
        n_src = O.rmsnorm(S[p * blk], M.W["src_norm"][beta, p * blk], w.eps)
        n_l0 = O.rmsnorm(S[l0], M.W["src_norm"][beta, l0], w.eps)
        A = O.router_weights(M, S, beta)
        expect = np.zeros_like(A)
        expect[:, l0, j0] = -0.7 * n_src[:, col0]
        assert np.max(np.abs(A - expect)) < 1e-15
        m = O.mix_channels(M, S, beta)
        expect_m = np.zeros_like(m)
        expect_m[j0] = expect[:, l0, j0, None] * n_l0
        assert np.max(np.abs(m - expect_m)) < 1e-14


def test_router_reads_only_every_pth_layer():
    M = tiny_model()
    S = np.random.default_rng(5).standard_normal((TINY.L, 4, TINY.D))
    A0 = O.router_weights(M, S, 0)
    S1 = S.copy()
    S1[1] *= 3.0  # layer 1 is not read with p = 2 ...
    assert np.array_equal(O.router_weights(M, S1, 0), A0)
    S1[1] += 1.0  # ... but a change of direction still changes the mixed channels
    assert not np.allclose(O.mix_channels(M, S1, 0), O.mix_channels(M, S, 0))
    S2 = S.copy()
    S2[2] += 1.0  # layer 2 is read
    assert not np.allclose(O.router_weights(M, S2, 0), A0)


def test_router_weights_are_signed_and_branches_differ():
    M = tiny_model()
    S = np.random.default_rng(6).standard_normal((TINY.L, 6, TINY.D))
    AK, AV = O.router_weights(M, S, 0), O.router_weights(M, S, 1)
    assert (AK < 0).any() and (AK > 0).any()
    assert not np.allclose(AK, AV)


# ---------------------------------------------------------------------------
# special case: static identity mixing with k = L is a vanilla decoder
# ---------------------------------------------------------------------------

def _torch_rope(x, pos, base):
    d = x.shape[-1]
    z = torch.complex(x[..., : d // 2], x[..., d // 2:])
    ang = pos.to(torch.float64)[:, None, None] * base ** (-torch.arange(d // 2, dtype=torch.float64) * 2 / d)
    zr = z * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([zr.real, zr.imag], -1)


def _vanilla_decoder(w, W, tokens):
    """Pre-norm GQA decoder in one parallel pass (torch CPU float64): layer l's
    keys/values come from its own block input through the (doubled) RMSNorm and
    its own projection; the mask is strict (s < i)."""
    t = {n: torch.from_numpy(np.asarray(a, np.float64)) for n, a in W.items()}
    B, T = tokens.shape
    pos = torch.arange(T)
    h = t["embed"][torch.from_numpy(tokens.astype(np.int64))]
    G = w.Hq // w.Hkv
    Ks, Vs = [], []
    mask = pos[None, :] < pos[:, None]
    for l in range(w.L):
        a = Fnn.rms_norm(h, (w.D,), t["attn_norm"][l], w.eps)
        q = Fnn.rms_norm(Fnn.linear(a, t["wq"][l]).view(B, T, w.Hq, w.d), (w.d,), t["q_norm"][l], w.eps)
        q = _torch_rope(q, pos, w.rope_base)
        ck = Fnn.rms_norm(Fnn.rms_norm(h, (w.D,), t["src_norm"][0, l], w.eps), (w.D,), t["chan_norm"][0, l], w.eps)
        cv = Fnn.rms_norm(Fnn.rms_norm(h, (w.D,), t["src_norm"][1, l], w.eps), (w.D,), t["chan_norm"][1, l], w.eps)
        kk = Fnn.rms_norm(Fnn.linear(ck, t["wk"][l]).view(B, T, w.Hkv, w.d), (w.d,), t["k_norm"][l], w.eps)
        kk = _torch_rope(kk, pos, w.rope_base)
        vv = Fnn.linear(cv, t["wv"][l]).view(B, T, w.Hkv, w.d)
        Ks.append(kk)
        Vs.append(vv)
        o = Fnn.scaled_dot_product_attention(q.transpose(1, 2), kk.transpose(1, 2).repeat_interleave(G, 1),
                                             vv.transpose(1, 2).repeat_interleave(G, 1), attn_mask=mask)
        o = o.transpose(1, 2).clone()
        o[:, 0] = 0.0  # the first token has no key
        h = h + Fnn.linear(o.reshape(B, T, w.Hq * w.d), t["wo"][l])
        b = Fnn.rms_norm(h, (w.D,), t["ffn_norm"][l], w.eps)
        h = h + Fnn.linear(Fnn.silu(Fnn.linear(b, t["w_gate"][l])) * Fnn.linear(b, t["w_up"][l]), t["w_down"][l])
    logits = Fnn.linear(Fnn.rms_norm(h, (w.D,), t["final_norm"], w.eps), t["lm_head"])
    K = torch.stack(Ks).permute(0, 1, 3, 2, 4).numpy()  # [L, B, Hkv, T, d]
    V = torch.stack(Vs).permute(0, 1, 3, 2, 4).numpy()
    return K, V, logits.numpy()


def test_static_identity_mix_with_k_equal_L_is_vanilla_decoder():
    w = TINY.replace(k=TINY.L)
    M = tiny_model(w, gains="ones")
    tokens = tiny_tokens(w)
    A = np.stack([np.eye(w.L), np.eye(w.L)])
    (Kc, Vc), logits = O.ar(M, tokens, want_logits=True, static_A=A)
    K, V, lg = _vanilla_decoder(w, M.W, tokens)
    T = tokens.shape[1]
    # RMSNorm(RMSNorm(x)) = RMSNorm(x) * (1 + O(eps)): relative 1e-6 at most
    assert max_abs_rel(Kc[:, :, :, :T], K) < 2e-6
    assert max_abs_rel(Vc[:, :, :, :T], V) < 2e-6
    assert max_abs_rel(logits, lg) < 2e-6


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("w", [TINY, TINY.replace(L=4, k=3, p=3, Hq=2, Hkv=1, T=5)])
def test_oracle_ar_matches_scalar_brute_force(w):
    M = tiny_model(w)
    tokens = tiny_tokens(w)
    (Kc, Vc), logits = O.ar(M, tokens, want_logits=True)
    Kb, Vb, Lb = brute_ar(w, M.W, tokens)
    T = tokens.shape[1]
    Kb = np.array(Kb).transpose(0, 1, 2, 3, 4)  # [B, k, Hkv, T, d]
    Vb = np.array(Vb)
    assert max_abs_rel(Kc[:, :, :, :T].transpose(1, 0, 2, 3, 4), Kb) < 1e-12
    assert max_abs_rel(Vc[:, :, :, :T].transpose(1, 0, 2, 3, 4), Vb) < 1e-12
    assert max_abs_rel(logits, np.array(Lb)) < 1e-12


# ---------------------------------------------------------------------------
# schedules (fixed point, Jacobi, cyclic Gauss-Seidel)
# ---------------------------------------------------------------------------

def _copy(c):
    return c[0].copy(), c[1].copy()


def _pos_err(c, ref, T):
    """Per-position max abs difference over both caches, positions < T."""
    e = np.maximum(np.abs(c[0] - ref[0]).max(axis=(0, 1, 2, 4)), np.abs(c[1] - ref[1]).max(axis=(0, 1, 2, 4)))
    return e[:T]


@pytest.fixture(scope="module")
def tiny_ar():
    M = tiny_model()
    tokens = tiny_tokens()
    cache, logits = O.ar(M, tokens, want_logits=True)
    return M, tokens, cache, logits


def test_ar_is_the_fixed_point(tiny_ar):
    M, tokens, cache, _ = tiny_ar
    c = _copy(cache)
    O.jacobi_pass(M, tokens, c)
    assert _pos_err(c, cache, TINY.T).max() < 1e-12
    c = _copy(cache)
    O.cyclic_pass(M, tokens, c, 3)
    assert _pos_err(c, cache, TINY.T).max() < 1e-12


@pytest.mark.parametrize("g", [TINY.T, TINY.T + 3])
def test_cyclic_with_g_at_least_T_is_ar_in_one_pass(tiny_ar, g):
    M, tokens, cache, logits = tiny_ar
    c = O.new_cache(TINY, TINY.B)
    lg = O.cyclic_pass(M, tokens, c, g, want_logits=True)
    assert _pos_err(c, cache, TINY.T).max() < 1e-12
    assert max_abs_rel(lg, logits) < 1e-12


@pytest.mark.parametrize("g", [1, 2, 3])
def test_cyclic_prefix_exactness_bound_is_tight(tiny_ar, g):
    """After pass n, positions < n*g equal AR; position n*g does not (strict
    causality + Gauss-Seidel visibility between groups, none inside one)."""
    M, tokens, cache, _ = tiny_ar
    T = TINY.T
    c = O.new_cache(TINY, TINY.B)
    n_exact = -(-T // g)
    for n in range(1, n_exact + 1):
        O.cyclic_pass(M, tokens, c, g)
        e = _pos_err(c, cache, T)
        assert e[: min(T, n * g)].max() < 1e-12
        if n * g < T:
            assert e[n * g] > 1e-6
    assert e.max() < 1e-12


def test_jacobi_from_random_start_reaches_the_same_fixed_point(tiny_ar):
    M, tokens, cache, _ = tiny_ar
    r = np.random.default_rng(7)
    c = (r.standard_normal(cache[0].shape), r.standard_normal(cache[1].shape))
    for _ in range(TINY.T):
        O.jacobi_pass(M, tokens, c)
    assert _pos_err(c, cache, TINY.T).max() < 1e-12


def test_batch_independence(tiny_ar):
    M, tokens, cache, logits = tiny_ar
    for b in range(TINY.B):
        c1, l1 = O.ar(M, tokens[b:b + 1], want_logits=True)
        assert np.max(np.abs(c1[0][:, 0] - cache[0][:, b])) < 1e-13
        assert np.max(np.abs(l1[0] - logits[b])) < 1e-13


def test_decode_step_extends_ar(tiny_ar):
    M, tokens, cache, logits = tiny_ar
    T = TINY.T
    c, _ = O.ar(M, tokens[:, : T - 1])
    lg = O.decode_step(M, tokens[:, T - 1], T - 1, c)
    assert _pos_err(c, cache, T).max() < 1e-12
    assert max_abs_rel(lg, logits[:, T - 1]) < 1e-12


def test_mix_kv_and_channel_attn_agree_with_a_group_step(tiny_ar):
    M, tokens, cache, _ = tiny_ar
    w = TINY
    g, q = 3, 1
    Mq = len(O.group_positions(w.T, g, q))
    bidx, pos = O.tokset_rows(w.B, Mq, q, g)
    S, _ = O.stack_forward(M, tokens[bidx, pos], pos, bidx, cache[0], cache[1])
    c = O.new_cache(w, w.B)
    O.mix_kv(M, S, w.B, Mq, q, g, c)
    for n in range(len(pos)):
        assert np.max(np.abs(c[0][:, bidx[n], :, pos[n]] - cache[0][:, bidx[n], :, pos[n]])) < 1e-12
    # channel_attn reads exactly channel layer mod k: poison every other channel
    qv = np.random.default_rng(8).standard_normal((len(pos), w.Hq, w.d))
    layer = 2
    poisoned = (cache[0].copy(), cache[1].copy())
    for ch in range(w.k):
        if ch != O.channel_of_layer(layer, w.k):
            poisoned[0][ch] = np.nan
            poisoned[1][ch] = np.nan
    # and every slot at or after a row's own position
    out = O.channel_attn(w, layer, qv, w.B, Mq, q, g, poisoned)
    assert np.isfinite(out).all()
    ref = O.channel_attn(w, layer, qv, w.B, Mq, q, g, cache)
    assert np.array_equal(out, ref)


def test_cyclic_final_pass_logits_converge_to_ar(tiny_ar):
    M, tokens, cache, logits = tiny_ar
    c = O.new_cache(TINY, TINY.B)
    g = 2
    for _ in range(-(-TINY.T // g)):
        lg = O.cyclic_pass(M, tokens, c, g, want_logits=True)
    assert max_abs_rel(lg, logits) < 1e-12
