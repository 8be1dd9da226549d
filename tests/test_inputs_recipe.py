"""The seeded input generators shared by the oracle and the HIP path
(`wm_inputs`), checked against the recipe they implement: bf16 rounding
equals torch's float32 -> bfloat16 conversion (round to nearest, ties to
even), weights are N(0, 0.02) and gains 1 or 1 + U(-0.1, 0.1), token ids
follow the truncated Zipf(1.1) law over the vocabulary (rank frequencies
against the closed form), the mix-only state stack is N(0, 1) scaled per
layer by U[0.5, 4], caches hold N(0, 1) before the filled position and 0 or
NaN after it, and every draw is a function of (seed, name) alone."""
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, __file__.rsplit("/tests/", 1)[0])
from wm_inputs import (WORKLOADS, bf16_bits, bf16_to_f32, make_cache, make_tokens,  # noqa: E402
                       make_state_stack, make_weight, make_weights, round_bf16)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** r.integers(-30, 30, 100000),
        # exact ties: the low 16 bits 0x8000 on even and odd bf16 mantissas
        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40], np.float32),
    ])
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert np.array_equal(bf16_to_f32(ref), round_bf16(x))


def test_weights_and_gains():
    w = WORKLOADS["small_prefill"].replace(dtype="f32")
    wq = make_weight(w, "wq", seed=0)
    assert wq.shape == (w.L, w.Hq * w.d, w.D)
    assert abs(wq.mean()) < 1e-3 and abs(wq.std() / 0.02 - 1) < 0.01
    assert np.all(make_weight(w, "attn_norm") == 1.0)
    g = make_weight(w, "attn_norm", gains="perturbed")
    assert g.min() >= 0.9 and g.max() <= 1.1 and g.std() > 0.05
    # bf16 workloads store bf16-representable values
    wb = make_weight(WORKLOADS["small_prefill"], "wq", seed=0)
    assert np.array_equal(wb, round_bf16(wb))


def test_draws_depend_on_seed_and_name_only():
    w = WORKLOADS["tiny_fp32"]
    a, b = make_weights(w, seed=3), make_weights(w, seed=3)
    assert all(np.array_equal(a[n], b[n]) for n in a)
    assert not np.array_equal(make_weight(w, "wq", seed=3), make_weight(w, "wq", seed=4))
    # different names draw different streams even at equal shapes
    assert not np.array_equal(make_weight(w, "w_gate", seed=3), make_weight(w, "w_up", seed=3))


def test_zipf_token_ranks():
    w = WORKLOADS["small_prefill"]
    t = make_tokens(w, seed=1, B=8, T=2048)
    assert t.dtype == np.int32 and t.shape == (8, 2048)
    assert t.min() >= 0 and t.max() < w.V
    n = t.size
    p = np.arange(1, w.V + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    counts = np.bincount(t.ravel(), minlength=w.V)
    # id i has rank i + 1; the most frequent ranks within 5 binomial sigmas
    for i in range(8):
        sd = np.sqrt(n * p[i] * (1 - p[i]))
        assert abs(counts[i] - n * p[i]) < 5 * sd, (i, counts[i], n * p[i])
    # the tail beyond rank 1000 carries its closed-form share
    tail = p[1000:].sum()
    assert abs(counts[1000:].sum() / n - tail) < 5 * np.sqrt(tail * (1 - tail) / n)
    u = make_tokens(WORKLOADS["tiny_fp32"], seed=1)
    assert u.min() >= 0 and u.max() < WORKLOADS["tiny_fp32"].V


def test_state_stack_per_layer_scale():
    w = WORKLOADS["mix_bf16"].replace(dtype="f32")
    S = make_state_stack(w, 4096, seed=2)
    assert S.shape == (w.L, 4096, w.D)
    sd = S.reshape(w.L, -1).std(axis=1)
    assert sd.min() > 0.5 * 0.98 and sd.max() < 4.0 * 1.02
    assert len(np.unique(np.round(sd, 2))) == w.L  # one scale per layer
    assert np.abs(S.reshape(w.L, -1).mean(axis=1)).max() < 0.05 * sd.max()


@pytest.mark.parametrize("poison", [False, True])
def test_cache_fill(poison):
    w = WORKLOADS["decode_d512"].replace(T_max=64, dtype="f32")
    K, V = make_cache(w, B=2, filled=40, seed=3, poison=poison)
    assert K.shape == (w.k, 2, w.Hkv, 64, w.d)
    for x in (K, V):
        head = x[:, :, :, :40]
        assert np.isfinite(head).all() and abs(head.std() - 1) < 0.02
        rest = x[:, :, :, 40:]
        assert np.isnan(rest).all() if poison else np.all(rest == 0)
    assert not np.array_equal(K[:, :, :, :40], V[:, :, :, :40])
