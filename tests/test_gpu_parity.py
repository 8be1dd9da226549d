"""HIP path vs the float64 oracle, through the C ABI (needs an MI355X).

Tolerances (max-abs-relative over a tensor, max|a-b| / max|b|):
  * fp32 runs: 1e-4 (the tiny fp32 model up to 32 dependent group steps, the
    kernels alone, decode); TOL_F32_CHAIN = 4e-4 for tiny-model caches that
    depend on more group steps (g * passes > 32), where plain fp32 evaluation
    of the oracle's own formulas already drifts past 1e-4
    (tests/test_fp32_error_model.py). The same kernels (templated on the
    element type) also run the deep 16- and 28-layer shapes in fp32; where a
    prefill pass feeds the cache back over several positions there the bound
    is TOL_F32_DEEP = 1e-3: fp32 rounding (~6e-8) times the exact oracle's own
    amplification of a perturbation through the cache (~3e3 at 16 layers).
  * bf16 runs: 2e-2 for the kernels alone (pool + append, channel attention,
    at full size). Wherever a layer stack runs, each test also evaluates the
    bf16 error model (tests/bf16_error_model.py: the definition in float64
    with every tensor the HIP path stores or feeds to a bf16 product rounded
    to bf16 there) on the rows it compares; that model's distance from the
    exact oracle is the rounding floor of those rows, and the GPU is held to
    max(2e-2, FLOOR_FACTOR x floor) (bf16_bound).  The floor exceeds 2e-2 at
    full depth and at 4 layers once positions feed back through the cache
    (tests/test_bf16_error_model.py); it is dominated by the bf16 operand of
    the normalised-input products, which any bf16 matrix-core implementation
    has.  The GPU rounds the same tensors in a different summation order, so
    its own error is another draw of the same size: the floor is the larger
    error of two draws of the model's roundings, and FLOOR_FACTOR = 2.5 lies
    above every ratio of one draw to the larger of two others measured on
    the CPU (tests/test_bf16_error_model.py::test_floor_factor).
Integer structure (which slots are written, the group schedule, the pass at
which a schedule reaches the autoregressive fixed point) is checked exactly:
unwritten slots must keep their NaN poison.
"""
import numpy as np
import pytest
import torch

import decode_token_rmsnorm_amd as wm
import oracle as O
from tests import bf16_error_model as EM
from tests.helpers import max_abs_rel
from wm_inputs import (WORKLOADS, make_cache, make_queries, make_state_stack, make_static_mix, make_tokens,
                       make_weights)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_F32_DEEP = 1e-3
TOL_F32_CHAIN = 4e-4
FLOOR_FACTOR = 2.5
DEV = "cuda"


def bf16_bound(floor):
    """Bound of a bf16 comparison against the exact oracle: 2e-2, or
    FLOOR_FACTOR times the bf16 rounding floor measured on the same rows (the
    error model with every rounding point of the HIP path) where that is
    larger."""
    return max(TOL["bf16"], FLOOR_FACTOR * floor)


def two_draws(fn):
    """The rounding model's result twice: as it is, and with the bf16
    roundings drawn anew (every rounded value perturbed by ~1e-6 first, as a
    different float32 summation order does)."""
    plain = fn()
    with EM.jittered(7):
        return plain, fn()


def floor_of(got, exact, models, what=""):
    """Errors of the GPU result ``got`` and of the rounding model's two draws
    ``models`` against the exact oracle's ``exact`` (lists of arrays compared
    pairwise, max over them); the floor is the larger of the two draws'
    errors.  Prints both and the GPU's distance from the first draw.
    Returns (GPU error, floor)."""
    err = max(max_abs_rel(a, b) for a, b in zip(got, exact))
    floor = max(max_abs_rel(m, b) for model in models for m, b in zip(model, exact))
    em = max(max_abs_rel(a, m) for a, m in zip(got, models[0]))
    print(f"  {what}: vs oracle {err:.2e}, rounding floor {floor:.2e} (bound {bf16_bound(floor):.2e}), "
          f"vs error model {em:.2e}", flush=True)
    return err, floor


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from decode_token_rmsnorm_amd import _lib

    _lib.lib()  # fail loudly if the HIP library is missing


def gpu_model(w, W):
    return wm.Model(w, W, w.dtype, device=DEV)


def np_of(t):
    return t.float().cpu().numpy()


def written_mask(w, B, bidx, pos):
    m = np.zeros((B, w.T_max), bool)
    m[bidx, pos] = True
    return m


def assert_cache(w, gk, gv, ref, mask, tol, poison=True):
    """Compare written slots; unwritten slots must still hold the NaN poison."""
    K, V = np_of(gk), np_of(gv)
    for got, exp, name in ((K, ref[0], "K"), (V, ref[1], "V")):
        sel = got.transpose(1, 3, 0, 2, 4)[mask]  # [n, k, Hkv, d]
        ref_sel = np.asarray(exp).transpose(1, 3, 0, 2, 4)[mask]
        err = max_abs_rel(sel, ref_sel)
        print(f"{name}: max-abs-rel {err:.3e} over {sel.shape[0]} slots", flush=True)
        assert err <= tol, (name, err)
        if poison:
            assert np.isnan(got.transpose(1, 3, 0, 2, 4)[~mask]).all(), f"{name}: an unwritten slot was written"


# ---------------------------------------------------------------- wm_mix_kv

@pytest.mark.parametrize("name,B,M,s0,step", [
    ("tiny_fp32", 1, 128, 0, 1),        # every position of cfg tiny
    ("mix_bf16", 3, 37, 5, 7),          # ragged rows (111), strided positions
    ("tiny_fp32", 2, 9, 3, 13),         # ragged fp32
    ("tiny_fp32", 2, 100, 0, 1),        # fp32 past the few-row path (200 rows, split router)
    ("mix_bf16", 3, 300, 2, 5),         # bf16, 900 rows: 128x128 router tiles with k splits
    ("mix_bf16@L4k1", 2, 16, 0, 1),     # one channel over few source layers (MFMA mix)
    ("mix_bf16@L2k1", 2, 16, 0, 1),
    ("mix_bf16@L3k1", 3, 50, 1, 2),
    ("mix_bf16@L16k16", 2, 40, 3, 1),   # few rows, one row per mix block, branches on their own MFMAs
    ("mix_bf16@L28k14", 1, 100, 0, 1),  # the same at 28 source layers (32-layer staging)
])
def test_mix_kv_matches_oracle(name, B, M, s0, step):
    if "@" in name:  # shape variant "<workload>@L<l>k<k>"
        base, var = name.split("@")
        Lv, kv = var[1:].split("k")
        w = WORKLOADS[base].replace(B=B, L=int(Lv), k=int(kv))
    else:
        w = WORKLOADS[name].replace(B=B)
    print(f"mix_kv {name} B={B} M={M} s0={s0} step={step}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    S = make_state_stack(w, B * M, seed=2)
    model = gpu_model(w, {n: W[n] for n in ("src_norm", "router", "chan_norm", "wk", "wv", "k_norm")})
    cache = wm.new_cache(model, B, fill=float("nan"))
    St = torch.from_numpy(S).to(DEV, wm.api.torch_dtype(w.dtype))
    wm.mix_kv(model, St, B, M, s0, step, cache)
    torch.cuda.synchronize()
    ref = O.new_cache(w, B)
    O.mix_kv(O.Model(w, W), S, B, M, s0, step, ref)
    bidx, pos = O.tokset_rows(B, M, s0, step)
    assert_cache(w, cache.k, cache.v, ref, written_mask(w, B, bidx, pos), TOL[w.dtype])


@pytest.mark.parametrize("B,M", [
    (1, 127), (2, 64), (3, 43),         # 127, 128, 129 rows: the few-row router and projection and past them
    (23, 89), (16, 128), (3, 683),      # 2047, 2048, 2049 rows: the 128x128 and the 256x256 tile GEMMs
    (1, 255), (2, 128), (1, 257),       # 255, 256, 257 rows: the tiled projection and the streamed one
    (5, 61),                            # 305 rows: 10 chunks of 32 rows for 16 blocks per channel, the last ragged
])
def test_mix_kv_row_count_boundaries(B, M):
    """Row counts on both sides of the library's kernel switches (bf16)."""
    w = WORKLOADS["mix_bf16"].replace(B=B)
    s0, step = 1, 1
    print(f"mix_kv boundary B={B} M={M} rows={B * M}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    S = make_state_stack(w, B * M, seed=6)
    model = gpu_model(w, {n: W[n] for n in ("src_norm", "router", "chan_norm", "wk", "wv", "k_norm")})
    cache = wm.new_cache(model, B, fill=float("nan"))
    wm.mix_kv(model, torch.from_numpy(S).to(DEV, torch.bfloat16), B, M, s0, step, cache)
    torch.cuda.synchronize()
    ref = O.new_cache(w, B)
    O.mix_kv(O.Model(w, W), S, B, M, s0, step, ref)
    bidx, pos = O.tokset_rows(B, M, s0, step)
    assert_cache(w, cache.k, cache.v, ref, written_mask(w, B, bidx, pos), TOL["bf16"])


@pytest.mark.parametrize("name,B,M,s0,step", [
    ("tiny_fp32", 2, 100, 0, 1),        # fp32 scalar mix
    ("mix_bf16", 3, 37, 5, 7),          # bf16 MFMA mix, few rows
    ("mix_bf16", 3, 300, 2, 5),         # bf16, 900 rows
])
def test_mix_kv_static_mixing_matches_oracle(name, B, M, s0, step):
    """The static-mixing variant: constant [2, L, k] weights replace the router
    (which is not uploaded at all)."""
    w = WORKLOADS[name].replace(B=B)
    print(f"mix_kv static {name} B={B} M={M} s0={s0} step={step}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    A = make_static_mix(w)
    S = make_state_stack(w, B * M, seed=2)
    up = {n: W[n] for n in ("src_norm", "chan_norm", "wk", "wv", "k_norm")}
    up["static_mix"] = A
    model = gpu_model(w, up)
    cache = wm.new_cache(model, B, fill=float("nan"))
    St = torch.from_numpy(S).to(DEV, wm.api.torch_dtype(w.dtype))
    wm.mix_kv(model, St, B, M, s0, step, cache)
    torch.cuda.synchronize()
    ref = O.new_cache(w, B)
    O.mix_kv(O.Model(w, W), S, B, M, s0, step, ref, static_A=(A[0], A[1]))
    bidx, pos = O.tokset_rows(B, M, s0, step)
    assert_cache(w, cache.k, cache.v, ref, written_mask(w, B, bidx, pos), TOL[w.dtype])


def test_prefill_static_mixing_tiny_fp32():
    """Two cyclic passes (g = 16) of the tiny model with static mixing."""
    w = WORKLOADS["tiny_fp32"]
    W = make_weights(w, seed=0, gains="perturbed")
    A = make_static_mix(w)
    tokens = make_tokens(w, seed=1)
    print("prefill static mixing tiny fp32, g=16, 2 passes", flush=True)
    up = {n: a for n, a in W.items() if n != "router"}
    up["static_mix"] = A
    model = gpu_model(w, up)
    cache = wm.new_cache(model, w.B)
    tok = torch.from_numpy(tokens).to(DEV)
    M = O.Model(w, W)
    ref = O.new_cache(w, w.B)
    for n in range(2):
        lg = wm.cyclic_prefill_pass(model, tok, 16, cache, logits_mode=2)
        rl = O.cyclic_pass(M, tokens, ref, 16, want_logits=True, static_A=(A[0], A[1]))
        torch.cuda.synchronize()
        ek = max_abs_rel(np_of(cache.k), ref[0])
        ev = max_abs_rel(np_of(cache.v), ref[1])
        el = max_abs_rel(np_of(lg), rl)
        print(f"  pass {n + 1}: K {ek:.2e} V {ev:.2e} logits {el:.2e}", flush=True)
        assert max(ek, ev, el) <= TOL["f32"]


def test_mix_kv_full_size_sampled_rows_and_deterministic():
    """Mix-only workload at full size [16, 8*2048, 512]; the oracle recomputes a
    seeded sample of 96 rows (rows are independent), and a second launch must
    reproduce the first bit for bit."""
    w = WORKLOADS["mix_bf16"]
    B, M = w.B, w.T
    print("mix_kv full size", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    S = make_state_stack(w, B * M, seed=2)
    model = gpu_model(w, {n: W[n] for n in ("src_norm", "router", "chan_norm", "wk", "wv", "k_norm")})
    cache = wm.new_cache(model, B, fill=float("nan"))
    St = torch.from_numpy(S).to(DEV, torch.bfloat16)
    ws = model.workspace(B * M)
    wm.mix_kv(model, St, B, M, 0, 1, cache, ws=ws)
    torch.cuda.synchronize()
    k1, v1 = cache.k.clone(), cache.v.clone()
    wm.mix_kv(model, St, B, M, 0, 1, cache, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), cache.k.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), cache.v.view(torch.int16))
    rows = np.sort(np.random.default_rng(11).choice(B * M, 96, replace=False))
    bidx, pos = rows // M, rows % M
    Kn, Vn = O.pool(O.Model(w, W), S[:, rows], pos)
    K, V = np_of(cache.k), np_of(cache.v)
    gotK = np.stack([K[:, b, :, p] for b, p in zip(bidx, pos)], 1)
    gotV = np.stack([V[:, b, :, p] for b, p in zip(bidx, pos)], 1)
    eK, eV = max_abs_rel(gotK, Kn), max_abs_rel(gotV, Vn)
    print(f"full-size mix sampled: K {eK:.3e} V {eV:.3e}", flush=True)
    assert eK <= TOL["bf16"] and eV <= TOL["bf16"]
    assert not np.isnan(K[:, :, :, :M]).any()


def test_mix_kv_ragged_large_rows():
    """2331 rows (3 sequences x 777 positions 5, 7, ..., 1557): the router and
    K/V projection run on the 256 x 256 tile GEMM with a partial last tile, and
    the mix has a partial last row block.  Sampled rows, the last partial tile
    among them, against the oracle; slots between and after the written
    positions keep their NaN poison."""
    w = WORKLOADS["mix_bf16"]
    B, M, s0, step = 3, 777, 5, 2
    print(f"mix_kv ragged B{B} M{M}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    S = make_state_stack(w, B * M, seed=4)
    model = gpu_model(w, {n: W[n] for n in ("src_norm", "router", "chan_norm", "wk", "wv", "k_norm")})
    cache = wm.new_cache(model, B, fill=float("nan"))
    wm.mix_kv(model, torch.from_numpy(S).to(DEV, torch.bfloat16), B, M, s0, step, cache)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.choice(B * M - 40, 48, replace=False), np.arange(B * M - 40, B * M)]))
    bidx, pos = rows // M, s0 + (rows % M) * step
    Kn, Vn = O.pool(O.Model(w, W), S[:, rows], pos)
    K, V = np_of(cache.k), np_of(cache.v)
    gotK = np.stack([K[:, b, :, p] for b, p in zip(bidx, pos)], 1)
    gotV = np.stack([V[:, b, :, p] for b, p in zip(bidx, pos)], 1)
    eK, eV = max_abs_rel(gotK, Kn), max_abs_rel(gotV, Vn)
    print(f"ragged mix sampled: K {eK:.3e} V {eV:.3e}", flush=True)
    assert eK <= TOL["bf16"] and eV <= TOL["bf16"]
    written = s0 + np.arange(M) * step
    assert not np.isnan(K[:, :, :, written]).any() and not np.isnan(V[:, :, :, written]).any()
    unwritten = np.setdiff1d(np.arange(w.T_max), written)
    assert np.isnan(K[:, :, :, unwritten]).all() and np.isnan(V[:, :, :, unwritten]).all()


# ---------------------------------------------------------------- wm_channel_attn

@pytest.mark.parametrize("name,B,M,s0,step,layer", [
    ("tiny_fp32", 1, 8, 3, 16, 1),             # fp32, d=32, MHA
    ("small_prefill", 8, 128, 5, 16, 9),       # one cyclic group step of the small model
    ("small_prefill", 2, 300, 0, 1, 3),        # Jacobi-like rows incl. position 0, ragged blocks
    ("prefill_1p3b", 2, 128, 15, 16, 13),      # d=128, G=7 (rows per pair not a tile multiple)
    ("decode_d512", 64, 1, 2047, 1, 5),        # decode shape: one query per sequence, waves split the keys
    ("prefill_1p3b", 4, 1, 2047, 1, 13),       # decode at d=128, G=7: key splits and the combine kernel
    ("small_prefill", 2, 4, 100, 16, 3),       # few rows at 4 positions: per-row masks, idle waves
    ("small_prefill", 1, 16, 0, 1, 2),         # 32 rows exactly, incl. position 0, one partial tile
    ("decode_d512", 2, 1, 0, 1, 0),            # position 0 only: no keys at all
])
def test_channel_attn_matches_oracle(name, B, M, s0, step, layer):
    _check_channel_attn(name, B, M, s0, step, layer)


@pytest.mark.parametrize("name,B,M,s0,step,layer", [
    ("small_prefill", 2, 16, 3, 7, 1),     # 32 query rows per sequence and KV head: one few-row block
    ("small_prefill", 2, 17, 3, 7, 1),     # 34: a second, ragged few-row block
    ("small_prefill", 2, 63, 0, 3, 4),     # 126
    ("small_prefill", 2, 64, 0, 3, 4),     # 128: 4 few-row blocks
    ("small_prefill", 2, 65, 5, 3, 4),     # 130
    ("small_prefill", 1, 256, 1, 7, 4),    # 512: the last row count on the few-row kernel
    ("small_prefill", 1, 257, 1, 7, 4),    # 514: the many-row kernel, a ragged last block
    ("prefill_1p3b", 2, 4, 900, 11, 6),    # G = 7: 28 rows, few-row kernel at d = 128
    ("prefill_1p3b", 2, 5, 900, 11, 6),    # 35
    ("prefill_1p3b", 2, 18, 10, 13, 6),    # 126
    ("prefill_1p3b", 2, 19, 10, 13, 6),    # 133
    ("prefill_1p3b", 1, 73, 3, 11, 6),     # 511: few-row kernel, 16 blocks at d = 128
    ("prefill_1p3b", 1, 74, 3, 11, 6),     # 518: many-row kernel at d = 128
])
def test_channel_attn_kernel_boundaries(name, B, M, s0, step, layer):
    """Query-row counts per (sequence, KV head) on both sides of the
    attention kernel switch (few-row kernel in blocks of 32 rows up to 512
    rows, many-row kernel above) and of the few-row kernel's block edges."""
    _check_channel_attn(name, B, M, s0, step, layer)


def _check_channel_attn(name, B, M, s0, step, layer):
    w = WORKLOADS[name]
    print(f"channel_attn {name} B={B} M={M} s0={s0} step={step} layer={layer}", flush=True)
    maxpos = s0 + (M - 1) * step
    K, V = make_cache(w, B, filled=maxpos, seed=3, poison=True)
    q = make_queries(w, B * M, seed=4)
    model = wm.Model(w, {}, w.dtype, device=DEV)
    cache = wm.cache_from_host(model, K, V)
    qt = torch.from_numpy(q).to(DEV, wm.api.torch_dtype(w.dtype))
    out = wm.channel_attn(model, layer, qt, B, M, s0, step, cache)
    torch.cuda.synchronize()
    Kz, Vz = np.nan_to_num(K, nan=0.0), np.nan_to_num(V, nan=0.0)  # the oracle only reads s < i anyway
    ref = O.channel_attn(w, layer, q, B, M, s0, step, (Kz, Vz))
    got = np_of(out)
    assert np.isfinite(got).all()
    err = max_abs_rel(got, ref)
    print(f"attn err {err:.3e}", flush=True)
    assert err <= TOL[w.dtype]
    bidx, pos = O.tokset_rows(B, M, s0, step)
    assert np.all(got[pos == 0] == 0.0)


# ---------------------------------------------------------------- prefill passes (tiny fp32)

def _run_passes(w, W, tokens, g, npass):
    """GPU and oracle caches/logits after each of npass passes of schedule g."""
    model = gpu_model(w, W)
    cache = wm.new_cache(model, w.B)
    tok = torch.from_numpy(tokens).to(DEV)
    M = O.Model(w, W)
    ref = O.new_cache(w, w.B)
    out = []
    for n in range(npass):
        lg = wm.cyclic_prefill_pass(model, tok, g, cache, logits_mode=2)
        rl = O.cyclic_pass(M, tokens, ref, g, want_logits=True)
        torch.cuda.synchronize()
        out.append(((np_of(cache.k), np_of(cache.v)), np_of(lg), (ref[0].copy(), ref[1].copy()), rl))
    return out


@pytest.fixture(scope="module")
def tiny():
    w = WORKLOADS["tiny_fp32"]
    W = make_weights(w, seed=0, gains="perturbed")
    tokens = make_tokens(w, seed=1)
    return w, W, tokens


@pytest.mark.parametrize("g,npass", [(16, 4), (1, 4), (128, 1), (5, 2)])
def test_prefill_passes_tiny_fp32(tiny, g, npass):
    w, W, tokens = tiny
    print(f"prefill tiny g={g} passes={npass}", flush=True)
    for n, (gc, gl, rc, rl) in enumerate(_run_passes(w, W, tokens, g, npass)):
        ek = max_abs_rel(gc[0][:, :, :, :w.T], rc[0][:, :, :, :w.T])
        ev = max_abs_rel(gc[1][:, :, :, :w.T], rc[1][:, :, :, :w.T])
        el = max_abs_rel(gl, rl)
        tol = TOL["f32"] if g * (n + 1) <= 32 else TOL_F32_CHAIN
        print(f"  pass {n + 1}: K {ek:.2e} V {ev:.2e} logits {el:.2e} (tol {tol:.0e})", flush=True)
        assert max(ek, ev, el) <= tol


def _pass_count(caches, ar, tau):
    """First pass (1-based) whose cache is within tau of the AR cache, or None."""
    for n, c in enumerate(caches):
        if max(max_abs_rel(c[0], ar[0]), max_abs_rel(c[1], ar[1])) <= tau:
            return n + 1
    return None


@pytest.mark.parametrize("T,g,npass", [(128, 16, 9), (32, 1, 33), (128, 5, 27), (128, 4, 33), (128, 8, 17),
                                        (128, 32, 5)])
def test_pass_counts_agree_tiny_fp32(tiny, T, g, npass):
    """The first pass whose cache is within 1e-4 of the same implementation's
    autoregressive cache must be the same pass on the GPU and in the oracle
    (cyclic g=16: 8 = ceil(T/g); Jacobi: T; g=5: ceil(T/5))."""
    w, W, tokens = tiny
    tokens = tokens[:, :T].copy()
    ar = _run_passes(w, W, tokens, T, 1)[0]
    gpu_ar = tuple(x[:, :, :, :T] for x in ar[0])
    ref_ar = tuple(x[:, :, :, :T] for x in ar[2])
    runs = _run_passes(w, W, tokens, g, npass)
    n_gpu = _pass_count([tuple(x[:, :, :, :T] for x in r[0]) for r in runs], gpu_ar, 1e-4)
    n_ref = _pass_count([tuple(x[:, :, :, :T] for x in r[2]) for r in runs], ref_ar, 1e-4)
    print(f"T={T} g={g}: pass count GPU {n_gpu} oracle {n_ref} (closed form {-(-T // g)})", flush=True)
    assert n_gpu == n_ref
    assert n_ref is not None and n_ref <= -(-T // g)


# ---------------------------------------------------------------- deep shapes in fp32

@pytest.mark.parametrize("name,B,T,g,npass", [("small_prefill", 2, 12, 4, 2), ("prefill_1p3b", 1, 6, 3, 1),
                                              ("small_prefill", 3, 9, 9, 1)])
def test_prefill_deep_shapes_fp32(name, B, T, g, npass):
    """16- and 28-layer shapes (D 512 / 1792, GQA 8/4 and 14/2, k 8 / 14) run
    through the fp32 instantiation of the same kernels: cache and all-position
    logits after each pass within TOL_F32_DEEP."""
    w = WORKLOADS[name].replace(B=B, dtype="f32")
    print(f"prefill fp32 {name} B={B} T={T} g={g} passes={npass}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    tokens = make_tokens(w, seed=1, B=B, T=T)
    model = gpu_model(w, W)
    cache = wm.new_cache(model, B, fill=float("nan"))
    cache.k[:, :, :, :T] = 0
    cache.v[:, :, :, :T] = 0
    tok = torch.from_numpy(tokens).to(DEV)
    M = O.Model(w, W)
    ref = O.new_cache(w, B)
    mask = np.zeros((B, w.T_max), bool)
    mask[:, :T] = True
    for n in range(npass):
        lg = wm.cyclic_prefill_pass(model, tok, g, cache, logits_mode=2)
        rl = O.cyclic_pass(M, tokens, ref, g, want_logits=True)
        torch.cuda.synchronize()
        assert_cache(w, cache.k, cache.v, ref, mask, TOL_F32_DEEP)
        el = max_abs_rel(np_of(lg), rl)
        print(f"  pass {n + 1}: logits {el:.3e}", flush=True)
        assert el <= TOL_F32_DEEP


@pytest.mark.parametrize("B", [8, 40, 129])  # 40: the wide vocabulary kernel, one ragged 64-row block;
def test_decode_deep_shape_fp32(B):             # 129: the many-row pool (folded router weights)
    w = WORKLOADS["decode_d512"].replace(B=B, T_max=512, dtype="f32")
    t = 300
    print(f"decode fp32 B={B} t=300", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    K, V = make_cache(w, w.B, filled=t, seed=3, poison=True)
    tokens = make_tokens(w, seed=1, B=w.B, T=1)[:, 0]
    model = gpu_model(w, W)
    cache = wm.cache_from_host(model, K, V)
    lg = wm.decode_step(model, torch.from_numpy(tokens).to(DEV), t, cache)
    torch.cuda.synchronize()
    ref = (np.nan_to_num(K, nan=0.0).astype(np.float64), np.nan_to_num(V, nan=0.0).astype(np.float64))
    rl = O.decode_step(O.Model(w, W), tokens, t, ref)
    el = max_abs_rel(np_of(lg), rl)
    ek = max_abs_rel(np_of(cache.k)[:, :, :, t], ref[0][:, :, :, t])
    ev = max_abs_rel(np_of(cache.v)[:, :, :, t], ref[1][:, :, :, t])
    print(f"decode fp32: logits {el:.2e} K {ek:.2e} V {ev:.2e}", flush=True)
    assert max(el, ek, ev) <= TOL["f32"]
    assert np.isnan(np_of(cache.k)[:, :, :, t + 1:]).all()


def test_decode_1p3b_widths_fp32():
    """A decode step of 64 sequences at the 1.3B widths (two layers): its
    gate/up product has more few-row blocks than compute units (608), so the
    blocks run with fewer waves, each taking a longer k range."""
    w = WORKLOADS["prefill_1p3b"].replace(L=2, k=2, p=1, B=64, T_max=64, dtype="f32")
    t = 40
    print(f"decode fp32 1.3B widths L2 B64 t={t}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    K, V = make_cache(w, w.B, filled=t, seed=3, poison=True)
    tokens = make_tokens(w, seed=1, B=w.B, T=1)[:, 0]
    model = gpu_model(w, W)
    cache = wm.cache_from_host(model, K, V)
    lg = wm.decode_step(model, torch.from_numpy(tokens).to(DEV), t, cache)
    torch.cuda.synchronize()
    ref = (np.nan_to_num(K, nan=0.0).astype(np.float64), np.nan_to_num(V, nan=0.0).astype(np.float64))
    rl = O.decode_step(O.Model(w, W), tokens, t, ref)
    el = max_abs_rel(np_of(lg), rl)
    ek = max_abs_rel(np_of(cache.k)[:, :, :, t], ref[0][:, :, :, t])
    ev = max_abs_rel(np_of(cache.v)[:, :, :, t], ref[1][:, :, :, t])
    print(f"decode fp32 1.3B widths: logits {el:.2e} K {ek:.2e} V {ev:.2e}", flush=True)
    assert max(el, ek, ev) <= TOL["f32"]
    assert np.isnan(np_of(cache.k)[:, :, :, t + 1:]).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_first_position(dtype):
    """A decode step at t = 0: no key to attend to (attention gives 0), slot 0
    appended; every later slot keeps its poison."""
    w = WORKLOADS["decode_d512"].replace(B=4, T_max=64, dtype=dtype)
    print(f"decode {dtype} t=0", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    K, V = make_cache(w, w.B, filled=0, seed=3, poison=True)
    tokens = make_tokens(w, seed=1, B=w.B, T=1)[:, 0]
    model = gpu_model(w, W)
    cache = wm.cache_from_host(model, K, V)
    lg = wm.decode_step(model, torch.from_numpy(tokens).to(DEV), 0, cache)
    torch.cuda.synchronize()
    ref = (np.zeros(K.shape), np.zeros(V.shape))
    rl = O.decode_step(O.Model(w, W), tokens, 0, ref)
    el = max_abs_rel(np_of(lg), rl)
    ek = max_abs_rel(np_of(cache.k)[:, :, :, 0], ref[0][:, :, :, 0])
    ev = max_abs_rel(np_of(cache.v)[:, :, :, 0], ref[1][:, :, :, 0])
    print(f"decode {dtype} t=0: logits {el:.2e} K {ek:.2e} V {ev:.2e}", flush=True)
    if dtype == "f32":
        assert max(el, ek, ev) <= TOL["f32"]
    else:
        zeros = np.zeros(w.B, int)
        mdl = two_draws(lambda: EM.step(w, W, tokens, zeros, np.arange(w.B), ref[0] * 0, ref[1] * 0,
                                        EM.STEP_ROUNDING_POINTS, many_rows=w.B > EM.FEW_ROWS, want_logits=True)[:3])
        err, floor = floor_of([np_of(cache.k)[:, :, :, 0], np_of(cache.v)[:, :, :, 0], np_of(lg)],
                              [ref[0][:, :, :, 0], ref[1][:, :, :, 0], rl], mdl, "decode t=0")
        assert err <= bf16_bound(floor)
    assert np.isnan(np_of(cache.k)[:, :, :, 1:]).all() and np.isnan(np_of(cache.v)[:, :, :, 1:]).all()


def test_out_of_range_token_gives_nan_rows():
    """A token id outside [0, V) is not read from the embedding: its
    sequence's logits and appended entries come out NaN, and every other
    sequence gets, bit for bit, what a run without the bad id gives it."""
    w = WORKLOADS["decode_d512"].replace(B=4, T_max=64)
    t = 20
    print("decode step with ids V and -1", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    K, V = make_cache(w, w.B, filled=t, seed=3)
    tokens = make_tokens(w, seed=1, B=w.B, T=1)[:, 0]
    model = gpu_model(w, W)
    good, bad_cache = wm.cache_from_host(model, K, V), wm.cache_from_host(model, K, V)
    lg = wm.decode_step(model, torch.from_numpy(tokens).to(DEV), t, good)
    bad = tokens.copy()
    bad[1], bad[2] = w.V, -1
    lb = wm.decode_step(model, torch.from_numpy(bad).to(DEV), t, bad_cache)
    torch.cuda.synchronize()
    for b in (1, 2):
        assert torch.isnan(lb[b]).all()
        assert torch.isnan(bad_cache.k[:, b, :, t]).all() and torch.isnan(bad_cache.v[:, b, :, t]).all()
    ok = [0, 3]
    assert torch.isfinite(lg).all() and torch.equal(lg[ok], lb[ok])
    assert torch.equal(good.k[:, ok].view(torch.int16), bad_cache.k[:, ok].view(torch.int16))
    assert torch.equal(good.v[:, ok].view(torch.int16), bad_cache.v[:, ok].view(torch.int16))


# ---------------------------------------------------------------- bf16, short sequences

@pytest.mark.parametrize("name,B,T,g", [("small_prefill", 2, 8, 8), ("prefill_1p3b", 1, 6, 6)])
def test_prefill_short_ar_bf16(name, B, T, g):
    """4-layer versions of the bf16 models (full width), exact AR over a few
    positions, so every token reads the bf16 cache of the ones before it:
    cache and logits within max(2e-2, FLOOR_FACTOR x the rounding floor of the
    same run) (at 4 layers bf16 rounding alone is ~7e-3 at position 0; with
    each position fed back through the cache it exceeds 2e-2)."""
    w = WORKLOADS[name].replace(B=B, L=4, k=min(4, WORKLOADS[name].k))
    print(f"prefill bf16 L=4 {name} B={B} T={T} g={g}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    tokens = make_tokens(w, seed=1, B=B, T=T)
    model = gpu_model(w, W)
    cache = wm.new_cache(model, B, fill=float("nan"))
    cache.k[:, :, :, :T] = 0
    cache.v[:, :, :, :T] = 0
    lg = wm.cyclic_prefill_pass(model, torch.from_numpy(tokens).to(DEV), g, cache, logits_mode=2)
    ref = O.new_cache(w, B)
    rl = O.cyclic_pass(O.Model(w, W), tokens, ref, g, want_logits=True)
    torch.cuda.synchronize()
    def model_run():
        mc = (np.zeros(ref[0].shape), np.zeros(ref[1].shape))
        lm = EM.cyclic_pass(w, W, tokens, mc, g, EM.STEP_ROUNDING_POINTS, want_logits=True)
        return mc[0][..., :T, :], mc[1][..., :T, :], lm

    err, floor = floor_of([np_of(cache.k)[..., :T, :], np_of(cache.v)[..., :T, :], np_of(lg)],
                          [ref[0][..., :T, :], ref[1][..., :T, :], rl], two_draws(model_run),
                          f"AR over {T} positions")
    assert err <= bf16_bound(floor)
    mask = np.zeros((B, w.T_max), bool)
    mask[:, :T] = True
    assert_cache(w, cache.k, cache.v, ref, mask, bf16_bound(floor))  # (and the poison past T)


# ---------------------------------------------------------------- bf16, full size

def _first_group_ref(w, W, tokens, b, many_rows):
    """Oracle keys/values of group 0 (positions 0, g, 2g, ...) of sequence b in
    the first pass (they read only the zero initial cache), [k, Hkv, n, d],
    and two draws of the rounding model's for the pool path ``many_rows``."""
    M = O.Model(w, W)
    Mq = len(O.group_positions(w.T, w.g, 0))
    pos = np.arange(Mq) * w.g
    ref = O.new_cache(w.replace(T_max=w.T), 1)
    O.step(M, tokens[b:b + 1], ref, np.zeros(Mq, int), pos)
    def model_run():
        Km, Vm, _, _ = EM.step(w, W, tokens[b, pos], pos, np.zeros(Mq, int), ref[0] * 0, ref[1] * 0,
                               EM.STEP_ROUNDING_POINTS, many_rows=many_rows)
        return Km.transpose(0, 2, 1, 3), Vm.transpose(0, 2, 1, 3)

    return pos, (ref[0][:, 0][:, :, pos], ref[1][:, 0][:, :, pos]), two_draws(model_run)


def _pre_step_cache(prev, cur, g, q):
    """The cache of one sequence ([k, 1, Hkv, T_max, d] pairs) as group step q
    of a pass reads it: positions of the groups before q as this pass wrote
    them (cur), the others as the previous pass left them (prev)."""
    sel = (np.arange(prev[0].shape[3]) % g) < q
    out = []
    for p, c in zip(prev, cur):
        x = p.copy()
        x[:, :, :, sel] = c[:, :, :, sel]
        out.append(x)
    return out


def _sampled_group_positions(T, g, q, n):
    """n positions of G_q spread evenly over it, its first and last included."""
    m = np.arange(q, T, g)
    return m[np.unique(np.linspace(0, len(m) - 1, n).round().astype(int))]


def check_group_steps(w, W, tok_b, C, steps, n_rows, logits=None, log=print):
    """Compare the cache a pass wrote for one sequence, group step by group
    step, with the oracle run from that implementation's own caches.

    C[n] holds the sequence's keys and values ([k, 1, Hkv, T_max, d] each)
    after pass n (C[0] = the zero initial cache).  For each (n, q) in
    ``steps``, the oracle evaluates group step q of pass n for n_rows sampled
    positions of G_q against the cache that step read (groups < q from C[n],
    the rest from C[n-1]); the entries C[n] holds there must agree.  Rows of
    one step do not interact, so a sample of them is a valid check.  The
    bound is the bf16 rounding floor of the same rows (two draws of the error
    model with every rounding point of the HIP path, against the exact
    oracle) times FLOOR_FACTOR, or 2e-2 where that is larger.  ``logits[n]``: the sequence's
    logits of position T-1 from pass n, checked in the step that holds it.
    Returns a list of (n, q, err vs oracle, floor, err vs error model)."""
    M = O.Model(w, W)
    T, g = w.T, w.g
    out = []
    for n, q in steps:
        pre = _pre_step_cache(C[n - 1], C[n], g, q)
        pos = _sampled_group_positions(T, g, q, n_rows)
        if n > 1 or q > 0:
            # the step's attention reads real keys: every earlier position a
            # step has written by then (all of them after pass 1, the groups
            # before q in pass 1) holds a non-zero entry in every channel
            s = np.arange(pos.max())
            s = s if n > 1 else s[s % g < q]
            assert (np.abs(pre[0][:, 0, :, s]).max(axis=(1, 2)) > 0).all()
        want = logits is not None and pos[-1] == T - 1
        ref = (pre[0].copy(), pre[1].copy())
        zeros = np.zeros(len(pos), int)
        lg_ref = O.step(M, tok_b[None, :], ref, zeros, pos, want_logits=want)
        K_ref, V_ref = ref[0][:, 0][:, :, pos], ref[1][:, 0][:, :, pos]
        def model_run():
            Km, Vm, lg_m, _ = EM.step(w, W, tok_b[pos], pos, zeros, pre[0], pre[1], EM.STEP_ROUNDING_POINTS,
                                      many_rows=True, want_logits=want)
            return [Km.transpose(0, 2, 1, 3), Vm.transpose(0, 2, 1, 3)] + ([lg_m[-1]] if want else [])

        got = [C[n][0][:, 0][:, :, pos], C[n][1][:, 0][:, :, pos]] + ([logits[n]] if want else [])
        exact = [K_ref, V_ref] + ([lg_ref[-1]] if want else [])
        models = two_draws(model_run)
        err = max(max_abs_rel(a, b) for a, b in zip(got, exact))
        floor = max(max_abs_rel(m, b) for md in models for m, b in zip(md, exact))
        em = max(max_abs_rel(a, m) for a, m in zip(got, models[0]))
        log(f"  pass {n} group {q:2d} ({len(pos)} rows{', logits' if want else ''}): vs oracle {err:.2e}, "
            f"rounding floor {floor:.2e}, vs error model {em:.2e}")
        out.append((n, q, err, floor, em))
    return out


@pytest.mark.parametrize("name,B,b,steps,n_rows", [
    ("small_prefill", None, 5, [(1, 1), (1, 15)] + [(2, q) for q in range(16)], 16),
    ("prefill_1p3b", None, 37, [(1, 15), (2, 0), (2, 1), (2, 15)], 16),
    # B = 17: 2176 rows per group step, the large-tile GEMMs end in a partial
    # 256-row tile, which holds the sampled last sequence
    ("small_prefill", 17, 16, [(1, 0), (2, 3)], 16),
])
def test_prefill_full_size_bf16_passes_1_and_2(name, B, b, steps, n_rows):
    """Two full-size bf16 passes (B, T = 2048, g = 16; the launch configuration
    the benchmark times), then every listed group step of one sampled
    sequence re-evaluated by the oracle from the GPU's own caches: after pass
    1 (C1) and pass 2 (C2), group step q of pass 2 read C2 for the groups
    before q and C1 for the others, and must have written what the oracle
    computes from that cache.  Later groups and passes read keys and values
    that earlier steps appended, so the attention, the pool and every
    projection act on real data here (group 0 of pass 1 reads only zeros)."""
    w = WORKLOADS[name] if B is None else WORKLOADS[name].replace(B=B)
    print(f"full-size passes 1-2 {name}, B {w.B}, sampled sequence {b}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    tokens = make_tokens(w, seed=1, B=w.B)
    model = gpu_model(w, W)
    cache = wm.new_cache(model, w.B)
    tok = torch.from_numpy(tokens).to(DEV)
    C = [(np.zeros((w.k, 1, w.Hkv, w.T_max, w.d)), np.zeros((w.k, 1, w.Hkv, w.T_max, w.d)))]
    lgs = [None]
    for n in range(2):
        lg = wm.cyclic_prefill_pass(model, tok, w.g, cache, logits_mode=1)
        torch.cuda.synchronize()
        assert torch.isfinite(lg).all() and torch.isfinite(cache.k).all() and torch.isfinite(cache.v).all()
        C.append((cache.k[:, b:b + 1].double().cpu().numpy(), cache.v[:, b:b + 1].double().cpu().numpy()))
        lgs.append(lg[b].double().cpu().numpy())
    del cache, model
    torch.cuda.empty_cache()
    res = check_group_steps(w, W, tokens[b], C, steps, n_rows, logits=lgs,
                            log=lambda s: print(s, flush=True))
    for n, q, err, floor, em in res:
        assert err <= bf16_bound(floor), (n, q, err, floor)


def test_prefill_ragged_rows_and_features_1p3b_widths():
    """A pass on 8064 rows per group step (B = 63: a ragged last 256-row
    tile) with F = 4800 (2F = 9600: a ragged last gate/up column tile), on a
    2-layer stack of the 1.3B widths; the oracle recomputes the first group
    of the last sequence, whose rows sit in the ragged tile; the oracle's K/V move by 1.4
    when the features past 4096 are dropped and by 0.24 (K) and 1.3 (V) when
    only the last 32 are.  Bound: max(2e-2, FLOOR_FACTOR x the rounding floor
    of the same rows)."""
    w = WORKLOADS["prefill_1p3b"].replace(L=2, k=2, p=1, F=4800)
    B, b = 63, 62
    print(f"ragged pass: L{w.L} D{w.D} F{w.F}, B {B}, sampled sequence {b}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    tokens = make_tokens(w, seed=1, B=B)
    model = gpu_model(w, W)
    cache = wm.new_cache(model, B)
    tok = torch.from_numpy(tokens).to(DEV)
    logits = wm.cyclic_prefill_pass(model, tok, w.g, cache, logits_mode=1)
    torch.cuda.synchronize()
    assert torch.isfinite(logits).all()
    gk = cache.k[:, b].float().cpu().numpy()
    gv = cache.v[:, b].float().cpu().numpy()
    del cache, model
    torch.cuda.empty_cache()
    pos, ref, mdl = _first_group_ref(w, W, tokens, b, many_rows=True)
    err, floor = floor_of([gk[:, :, pos], gv[:, :, pos]], ref, mdl, f"group 0 of sequence {b}")
    assert err <= bf16_bound(floor)


@pytest.mark.parametrize("B,T,g", [
    (1, 256, 2),     # 128 rows per group step: the few-row GEMMs
    (3, 86, 2),      # 129: past them
    (23, 178, 2),    # 2047: the 128x128 tile GEMMs
    (16, 256, 2),    # 2048: the 256x256 tile GEMMs
    (3, 1366, 2),    # 2049: and their ragged last tile
])
def test_prefill_first_group_row_boundaries(B, T, g):
    """One bf16 pass of the small model with a group step of 128, 129, 2047,
    2048 or 2049 rows, on both sides of the library's GEMM switches; the
    oracle recomputes the first group of the last sequence."""
    w = WORKLOADS["small_prefill"].replace(B=B, T=T, g=g)
    b = B - 1
    print(f"prefill B{B} T{T} g{g}: {B * ((T + g - 1) // g)} rows per first group step", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    tokens = make_tokens(w, seed=1)
    model = gpu_model(w, W)
    cache = wm.new_cache(model, B)
    wm.cyclic_prefill_pass(model, torch.from_numpy(tokens).to(DEV), g, cache)
    torch.cuda.synchronize()
    gk = cache.k[:, b].float().cpu().numpy()
    gv = cache.v[:, b].float().cpu().numpy()
    assert np.isfinite(gk[:, :, :T]).all() and np.isfinite(gv[:, :, :T]).all()
    pos, ref, mdl = _first_group_ref(w, W, tokens, b, many_rows=B * ((T + g - 1) // g) > EM.FEW_ROWS)
    err, floor = floor_of([gk[:, :, pos], gv[:, :, pos]], ref, mdl, f"group 0 of sequence {b}")
    assert err <= bf16_bound(floor)


@pytest.mark.parametrize("B", [128, 129])
def test_decode_step_batch_boundary(B):
    """Decode steps of 128 and 129 sequences (the few-row GEMMs and past them)
    at t = 300 on the decode model; logits and the appended slot against the
    oracle, the rest of the cache untouched."""
    w = WORKLOADS["decode_d512"].replace(B=B, T_max=512)  # (a shorter cache keeps the host copies small)
    t = 300
    print(f"decode B{B} t{t}", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    K, V = make_cache(w, B, filled=t, seed=3, poison=True)
    tokens = make_tokens(w, seed=1, B=B, T=1)[:, 0]
    model = gpu_model(w, W)
    cache = wm.cache_from_host(model, K, V)
    lg = wm.decode_step(model, torch.from_numpy(tokens).to(DEV), t, cache)
    torch.cuda.synchronize()
    ref = (np.nan_to_num(K, nan=0.0).astype(np.float64), np.nan_to_num(V, nan=0.0).astype(np.float64))
    mdl = two_draws(lambda: EM.step(w, W, tokens, np.full(B, t), np.arange(B), ref[0], ref[1],
                                    EM.STEP_ROUNDING_POINTS, many_rows=B > EM.FEW_ROWS, want_logits=True)[:3])
    rl = O.decode_step(O.Model(w, W), tokens, t, ref)
    gk, gv = np_of(cache.k), np_of(cache.v)
    err, floor = floor_of([gk[:, :, :, t], gv[:, :, :, t], np_of(lg)], [ref[0][:, :, :, t], ref[1][:, :, :, t], rl],
                          mdl, f"decode B{B} t{t}")
    assert err <= bf16_bound(floor)
    for got, exp in ((gk, ref[0]), (gv, ref[1])):
        assert np.array_equal(got[:, :, :, :t], np.asarray(exp[:, :, :, :t], np.float32))
        assert np.isnan(got[:, :, :, t + 1:]).all()


def test_decode_step_full_size():
    """Decode workload at full size: B=64, 2047 cached positions (seeded N(0,1)
    keys/values in all 16 channels), one new token per sequence at t=2047;
    slots beyond t are NaN-poisoned and must stay so, earlier slots must be
    untouched."""
    w = WORKLOADS["decode_d512"]
    t = 2047
    print("decode full size", flush=True)
    W = make_weights(w, seed=0, gains="perturbed")
    K, V = make_cache(w, w.B, filled=t, seed=3, poison=True)
    tokens = make_tokens(w, seed=1, B=w.B, T=1)[:, 0]
    model = gpu_model(w, W)
    cache = wm.cache_from_host(model, K, V)
    lg = wm.decode_step(model, torch.from_numpy(tokens).to(DEV), t, cache)
    torch.cuda.synchronize()
    ref = (np.nan_to_num(K, nan=0.0).astype(np.float64), np.nan_to_num(V, nan=0.0).astype(np.float64))
    mdl = two_draws(lambda: EM.step(w, W, tokens, np.full(w.B, t), np.arange(w.B), ref[0], ref[1],
                                    EM.STEP_ROUNDING_POINTS, many_rows=w.B > EM.FEW_ROWS, want_logits=True)[:3])
    rl = O.decode_step(O.Model(w, W), tokens, t, ref)
    gk, gv = np_of(cache.k), np_of(cache.v)
    err, floor = floor_of([gk[:, :, :, t], gv[:, :, :, t], np_of(lg)], [ref[0][:, :, :, t], ref[1][:, :, :, t], rl],
                          mdl, "decode B64 t2047")
    assert err <= bf16_bound(floor)
    for got, exp in ((gk, ref[0]), (gv, ref[1])):
        assert np.array_equal(got[:, :, :, :t], np.asarray(exp[:, :, :, :t], np.float32))  # history untouched
