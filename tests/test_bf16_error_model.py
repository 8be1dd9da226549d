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
