"""How far exact bf16 operand rounding alone moves the full-depth stack from the
exact (float64) definition — the basis of TOL_BF16_DEEP in the GPU tests.

For the 16- and 28-layer bf16 workloads, rounding every matrix-product operand
and stored state to bf16 (and nothing else) already moves the keys by more
than 2e-2 max-abs-relative, so no bf16 implementation can meet 2e-2 there
against the exact oracle; the full-depth parity tests therefore use
TOL_BF16_DEEP = 1e-1, about twice the error measured here. At 4 layers the
same rounding stays below 2e-2, and the reduced-depth bf16 tests keep 2e-2.
"""
import numpy as np
import pytest

import oracle as O
from tests.bf16_error_model import ROUNDING_POINTS, position0
from tests.helpers import max_abs_rel
from wm_inputs import WORKLOADS, make_tokens, make_weights

TOL_BF16 = 2e-2
TOL_BF16_DEEP = 1e-1


def _case(name, L=None, rows=32):
    w = WORKLOADS[name].replace(B=1)
    if L is not None:
        w = w.replace(L=L, k=min(w.k, L))
    W = make_weights(w, seed=0, gains="perturbed")
    tok = make_tokens(w, seed=1, B=rows, T=1)[:, 0]
    return w, W, tok


@pytest.mark.parametrize("name,L,rows", [("decode_d512", None, 32), ("small_prefill", 4, 32),
                                         ("prefill_1p3b", None, 8)])
def test_exact_bf16_rounding_error_bounds(name, L, rows):
    w, W, tok = _case(name, L, rows)
    lg0, K0 = position0(w, W, tok)
    # with no rounding the model is the definition: agree with the oracle
    M = O.Model(w, W)
    cache = O.new_cache(w.replace(T_max=1), rows)
    bidx, pos = np.arange(rows), np.zeros(rows, int)
    lgo = O.step(M, tok[:, None], cache, bidx, pos, want_logits=True)
    assert max_abs_rel(lg0, lgo) < 1e-12
    assert max_abs_rel(K0, cache[0][:, :, :, 0]) < 1e-12
    lg, K = position0(w, W, tok, ROUNDING_POINTS)
    e_lg, e_k = max_abs_rel(lg, lg0), max_abs_rel(K, K0)
    print(f"{name} L={w.L}: exact bf16 rounding -> logits {e_lg:.2e}, keys {e_k:.2e}")
    if w.L >= 16:
        assert e_k > TOL_BF16            # 2e-2 is out of reach at this depth
        assert max(e_lg, e_k) < TOL_BF16_DEEP / 1.5
    else:
        assert max(e_lg, e_k) < TOL_BF16


def test_feedback_free_bf16_rounding_floor():
    """The feedback-free variant in bf16 (the GPU test shapes: L = k = 4,
    D512, 2 x 64 and 3 x 256 positions): exact bf16 rounding of the stored and
    product-feeding tensors alone moves the cached keys by up to 1.6e-1 from
    the exact definition (a few tokens whose router outputs are small against
    their terms amplify the rounding of the router input), so 2e-2 is out of
    reach for any bf16 implementation; the GPU test holds the variant to
    TOL_FF_BF16 = 2.5e-1 against the oracle, about 1.5 times this floor."""
    import oracle as O
    from tests.bf16_error_model import FF_ROUNDING_POINTS, ff_forward
    for B, T in ((2, 64), (3, 256)):
        w = WORKLOADS["small_prefill"].replace(L=4, k=4, B=B, T=T)
        W = make_weights(w, seed=0, gains="perturbed")
        tok = make_tokens(w, seed=1)
        K0, V0, lg0 = ff_forward(w, W, tok)
        (Ko, Vo), lgo = O.ff_forward(O.Model(w, W), tok)
        assert max_abs_rel(K0, Ko[..., :T, :]) < 1e-12 and max_abs_rel(lg0, lgo) < 1e-12  # no rounding: the oracle
        K1, V1, lg1 = ff_forward(w, W, tok, FF_ROUNDING_POINTS)
        ek, ev, el = max_abs_rel(K1, K0), max_abs_rel(V1, V0), max_abs_rel(lg1, lg0)
        print(f"feedback-free B{B} T{T}: exact bf16 rounding -> K {ek:.2e}, V {ev:.2e}, logits {el:.2e}")
        assert max(ek, ev) > TOL_BF16                # 2e-2 is out of reach for bf16 here
        assert max(ek, ev, el) < 2.5e-1 / 1.5
