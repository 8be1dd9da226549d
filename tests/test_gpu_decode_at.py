"""wm_decode_step_at: the decode step whose position lives in device memory,
and that step captured once in a graph and replayed at successive positions.

* On the tiny fp32 model it matches the oracle's decode step at 1e-4 at
  positions 0, 1, 57 and 127 (the first position, a position with one key,
  an inner one and the last slot), with one call per position from the
  same prefilled cache.
* At the decode workload (B64, bf16) its logits and appended entries equal
  wm_decode_step's bit for bit at positions 2047, 1500 and 1 (at that shape
  the attention takes no key split at any position, so the host's choice
  for the last position is the same choice).
* With 256 sequences (the pool's K/V projection on the streamed kernel,
  reading the position from device memory) it equals wm_decode_step bit for
  bit and writes slot t only.
* Graph replay: one call captured in a torch CUDA graph replays at positions
  2044, 2045, 2046, 1200; before each replay the test writes the next
  position and tokens into the captured buffers, runs the eager
  wm_decode_step on a copy of the cache as it stands, synchronises, and
  then compares the replay's logits and appended entries with it bit for bit.
* A whole cyclic prefill pass captured once replays as three passes that
  equal three eager passes bit for bit.
"""
import numpy as np
import pytest
import torch

import decode_token_rmsnorm_amd as wm
import oracle as O
from wm_inputs import WORKLOADS, make_cache, make_cache_device, make_tokens, make_weights

pytestmark = pytest.mark.gpu


def _mar(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def test_tiny_fp32_against_oracle():
    w = WORKLOADS["tiny_fp32"].replace(B=2)
    W = make_weights(w, seed=0, gains="perturbed")
    model = wm.Model(w, W, "f32")
    M = O.Model(w, W)
    tokens = make_tokens(w, seed=1)
    Kh, Vh = make_cache(w, w.B, filled=w.T_max, seed=3)
    for t in (0, 1, 57, 127):
        print(f"[decode_at] tiny fp32 t={t}", flush=True)
        cache = wm.cache_from_host(model, Kh, Vh)
        tok = torch.from_numpy(tokens[:, t].copy()).cuda()
        tdev = torch.tensor([t], dtype=torch.int32, device="cuda")
        lg = wm.decode_step_at(model, tok, tdev, cache)
        torch.cuda.synchronize()
        ref = (Kh.astype(np.float64), Vh.astype(np.float64))
        ref_lg = O.decode_step(M, tokens[:, t], t, ref)
        e_lg = _mar(lg.cpu().numpy(), ref_lg)
        e_k = _mar(cache.k[:, :, :, t].cpu().numpy(), ref[0][:, :, :, t])
        e_v = _mar(cache.v[:, :, :, t].cpu().numpy(), ref[1][:, :, :, t])
        print(f"  logits {e_lg:.1e}, K {e_k:.1e}, V {e_v:.1e}", flush=True)
        assert max(e_lg, e_k, e_v) <= 1e-4
        # nothing else of the cache changed
        assert np.array_equal(np.delete(cache.k.cpu().numpy(), t, axis=3), np.delete(Kh, t, axis=3))


def _decode_setup():
    w = WORKLOADS["decode_d512"]
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    K, V = make_cache_device(w, w.B, filled=w.T_max, seed=3)
    toks = make_tokens(w, seed=1, B=w.B, T=8)
    return w, model, K, V, toks


def test_decode_bit_exact_against_host_position():
    w, model, K, V, toks = _decode_setup()
    ws = model.workspace(w.B)
    for i, t in enumerate((2047, 1500, 1)):
        print(f"[decode_at] decode_d512 B{w.B} t={t}", flush=True)
        tok = torch.from_numpy(toks[:, i].copy()).cuda()
        c1 = wm.Cache(K.clone(), V.clone())
        c2 = wm.Cache(K.clone(), V.clone())
        l1 = wm.decode_step(model, tok, t, c1, ws=ws)
        l2 = wm.decode_step_at(model, tok, torch.tensor([t], dtype=torch.int32, device="cuda"), c2, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(l1, l2)
        assert torch.equal(c1.k[:, :, :, t], c2.k[:, :, :, t]) and torch.equal(c1.v[:, :, :, t], c2.v[:, :, :, t])
        del c1, c2


def test_decode_256_sequences_device_position():
    """256 sequences: the pool's K/V projection runs on the streamed kernel
    (at least 256 rows), which reads the position from device memory in
    wm_decode_step_at; logits and appended entries equal wm_decode_step's bit
    for bit, and only slot t was written."""
    w = WORKLOADS["decode_d512"].replace(B=256, T_max=256)
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    K, V = make_cache_device(w, w.B, filled=w.T_max, seed=3)
    toks = make_tokens(w, seed=1, B=w.B, T=2)
    ws = model.workspace(w.B)
    for i, t in enumerate((255, 3)):
        print(f"[decode_at] decode_d512 B{w.B} t={t}", flush=True)
        tok = torch.from_numpy(toks[:, i].copy()).cuda()
        c1 = wm.Cache(K.clone(), V.clone())
        c2 = wm.Cache(K.clone(), V.clone())
        l1 = wm.decode_step(model, tok, t, c1, ws=ws)
        l2 = wm.decode_step_at(model, tok, torch.tensor([t], dtype=torch.int32, device="cuda"), c2, ws=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(l1).all()
        assert torch.equal(l1, l2)
        assert torch.equal(c1.k, c2.k) and torch.equal(c1.v, c2.v)
        keep = [s for s in range(w.T_max) if s != t]
        assert torch.equal(c2.k[:, :, :, keep], K[:, :, :, keep]) and torch.equal(c2.v[:, :, :, keep], V[:, :, :, keep])
        assert not torch.equal(c2.k[:, :, :, t], K[:, :, :, t])
        del c1, c2


def test_graph_replay_at_successive_positions():
    w, model, K, V, toks = _decode_setup()
    ws = model.workspace(w.B)
    cache = wm.Cache(K, V)
    tok = torch.empty(w.B, dtype=torch.int32, device="cuda")
    tdev = torch.tensor([2043], dtype=torch.int32, device="cuda")
    logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
    tok.copy_(torch.from_numpy(toks[:, 0].copy()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # (warmup off the capture)
        wm.decode_step_at(model, tok, tdev, cache, logits, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wm.decode_step_at(model, tok, tdev, cache, logits, ws)
    torch.cuda.synchronize()
    ws_ref = model.workspace(w.B)
    for i, t in enumerate((2044, 2045, 2046, 1200)):
        print(f"[decode_at] graph replay {i} at t={t}", flush=True)
        tk = torch.from_numpy(toks[:, i + 1].copy()).cuda()
        ref_cache = wm.Cache(cache.k.clone(), cache.v.clone())
        ref = wm.decode_step(model, tk, t, ref_cache, ws=ws_ref)
        torch.cuda.synchronize()
        tok.copy_(tk)
        tdev.fill_(t)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(logits, ref), i
        assert torch.equal(cache.k[:, :, :, t], ref_cache.k[:, :, :, t]), i
        assert torch.equal(cache.v[:, :, :, t], ref_cache.v[:, :, :, t]), i
        del ref_cache


def test_prefill_pass_graph_replay_equals_eager():
    """A whole cyclic pass (wm_cyclic_prefill_pass: every group step's
    launches) captured once and replayed three times from the zero cache
    gives the caches and logits of three eager passes, bit for bit, on the
    tiny fp32 model (g = 16) and on the small bf16 model's widths at
    B2 T256 (g = 16)."""
    for name, kw, dtype in (("tiny_fp32", dict(B=2), "f32"), ("small_prefill", dict(B=2, T=256, T_max=256), "bf16")):
        w = WORKLOADS[name].replace(**kw)
        print(f"[graph] {name} {kw}", flush=True)
        model = wm.Model(w, make_weights(w, seed=0, gains="perturbed"), dtype)
        tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
        ws = model.workspace(wm.prefill_rows(w.B, w.T, w.g))
        eager = wm.new_cache(model, w.B)
        lg_e = torch.empty(w.B, w.T, w.V, dtype=torch.float32, device="cuda")
        for _ in range(3):
            wm.cyclic_prefill_pass(model, tok, w.g, eager, logits_mode=2, logits=lg_e, ws=ws)
        torch.cuda.synchronize()
        cache = wm.new_cache(model, w.B)
        lg = torch.empty_like(lg_e)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # (warmup off the capture; then reset the cache)
            wm.cyclic_prefill_pass(model, tok, w.g, cache, logits_mode=2, logits=lg, ws=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            wm.cyclic_prefill_pass(model, tok, w.g, cache, logits_mode=2, logits=lg, ws=ws)
        torch.cuda.synchronize()
        cache.k.zero_()
        cache.v.zero_()
        torch.cuda.synchronize()
        for i in range(3):
            graph.replay()
            torch.cuda.synchronize()
        assert torch.equal(cache.k, eager.k) and torch.equal(cache.v, eager.v)
        assert torch.equal(lg, lg_e)
        del graph
