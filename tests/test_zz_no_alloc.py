"""wm_decode_step_static, the allocation-free decode step (its scratch lives in
the library's static device array), against wm_decode_step with a caller
workspace, through the C ABI (needs an MI355X): on the same inputs both give
the same logits and the same cache, bit for bit, on two calls in a row of the
static entry point, the second with fewer sequences than the first (so its
scratch still holds the first call's values)."""
import pytest
import torch

import decode_token_rmsnorm_amd as wm
from wm_inputs import WORKLOADS, make_cache_device, make_tokens, make_weights

pytestmark = pytest.mark.gpu


def test_static_decode_step_matches_workspace_entry_point():
    w = WORKLOADS["decode_d512"]
    W = make_weights(w, seed=0, gains="perturbed")
    model = wm.Model(w, W, w.dtype, device="cuda")
    for B, t, seed in ((64, 2047, 3), (16, 700, 4)):
        print(f"decode step, B {B}, t {t}: static scratch against a workspace", flush=True)
        K, V = make_cache_device(w, B, filled=t, seed=seed)
        tokens = torch.from_numpy(make_tokens(w, seed=seed, B=B, T=1)[:, 0]).cuda()
        ref = wm.Cache(K.clone(), V.clone())
        got = wm.Cache(K, V)
        lr = wm.decode_step(model, tokens, t, ref)
        lg = wm.decode_step_static(model, tokens, t, got)
        torch.cuda.synchronize()
        assert torch.isfinite(lg).all()
        assert torch.equal(lg, lr)
        assert torch.equal(got.k.view(torch.int16), ref.k.view(torch.int16))
        assert torch.equal(got.v.view(torch.int16), ref.v.view(torch.int16))
        del K, V, ref, got
        torch.cuda.empty_cache()
