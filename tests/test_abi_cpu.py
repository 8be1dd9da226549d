"""The C-ABI library on the CPU: it loads, exports every function include/wm.h
declares, its host-only helpers match the oracle bit for bit, and every
validated error path returns its code before anything is launched."""
import ctypes
import os
import subprocess

import pytest

import oracle as O
from decode_token_rmsnorm_amd import _lib as C
from wm_inputs import WORKLOADS

pytestmark = pytest.mark.skipif(not os.path.exists(C.LIB_PATH), reason="libwm.so not built")

FAKE = 0x100000  # never dereferenced: every call below fails validation first


def cfg_of(w, dtype=C.WM_BF16, **kw):
    c = C.WmConfig(w.L, w.D, w.Hq, w.Hkv, w.d, w.F, w.k, w.p, w.V, w.T_max, w.eps, w.rope_base, dtype)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_library_exports_every_declared_function():
    names = C.header_functions()
    assert len(names) == 25
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported, set(names) - exported
    L = C.lib()
    for n in names:
        assert getattr(L, n) is not None


@pytest.mark.parametrize("T,g", [(128, 16), (2048, 16), (7, 3), (5, 9), (1, 1), (100, 1), (10, 10)])
def test_group_positions_bit_exact(T, g):
    L = C.lib()
    for q in range(g):
        buf = (ctypes.c_int32 * (T + 1))()
        n = L.wm_group_positions(T, g, q, buf)
        assert n == len(O.group_positions(T, g, q))
        assert list(buf[:n]) == O.group_positions(T, g, q)
    assert L.wm_group_positions(T, g, g, None) == -1
    assert L.wm_group_positions(T, 0, 0, None) == -1


def test_channel_of_layer_and_cache_elems_bit_exact():
    L = C.lib()
    for k in range(1, 17):
        for layer in range(40):
            assert L.wm_channel_of_layer(layer, k) == O.channel_of_layer(layer, k)
    assert L.wm_channel_of_layer(3, 0) == -1
    for name, w in WORKLOADS.items():
        c = cfg_of(w)
        assert L.wm_cache_elems(ctypes.byref(c), w.B) == O.cache_elems(w.k, w.B, w.T_max, w.Hkv, w.d)


def test_workspace_bytes_positive_and_monotone():
    L = C.lib()
    c = cfg_of(WORKLOADS["prefill_1p3b"])
    sizes = [L.wm_workspace_bytes(ctypes.byref(c), r) for r in (1, 64, 1024, 8192)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    assert L.wm_workspace_bytes(ctypes.byref(c), 0) == 0


@pytest.mark.parametrize("field,value,code", [
    ("k", 0, -2), ("k", 17, -2), ("p", 0, -2), ("d", 48, -2), ("Hq", 6, -2), ("D", 96, -2), ("F", 100, -2),
    ("L", 33, -2), ("dtype", 7, -3), ("eps", 0.0, -1), ("T_max", 0, -2),
])
def test_check_config_rejects(field, value, code):
    c = cfg_of(WORKLOADS["decode_d512"], **{field: value})
    assert C.lib().wm_check_config(ctypes.byref(c)) == code
    assert C.last_error() != ""


def _weights(fake=FAKE):
    """Every weight pointer set to `fake` except the optional static_mix (NULL:
    the routed model)."""
    return C.WmWeights(*[None if n == "static_mix" else fake for n in C.WEIGHT_FIELDS])


def test_entry_points_validate_before_launch():
    L = C.lib()
    w = WORKLOADS["small_prefill"]
    c = cfg_of(w)
    W = _weights()
    cache = C.WmCache(FAKE, FAKE, w.B)
    rows = w.B * w.T
    need = L.wm_workspace_bytes(ctypes.byref(c), rows)
    ts = C.WmTokset(w.B, w.T, 0, 1)
    st = lambda: C.lib().wm_last_error()
    # null config / cache / weights
    assert L.wm_mix_kv(None, ctypes.byref(W), FAKE, ts, ctypes.byref(cache), FAKE, need, None) == -1
    assert L.wm_mix_kv(ctypes.byref(c), ctypes.byref(W), FAKE, ts, None, FAKE, need, None) == -1
    assert L.wm_mix_kv(ctypes.byref(c), None, FAKE, ts, ctypes.byref(cache), FAKE, need, None) == -1
    # workspace too small
    assert L.wm_mix_kv(ctypes.byref(c), ctypes.byref(W), FAKE, ts, ctypes.byref(cache), FAKE, need - 1, None) == -4
    # positions beyond the cache
    bad = C.WmTokset(w.B, w.T, 1, 1)
    assert L.wm_mix_kv(ctypes.byref(c), ctypes.byref(W), FAKE, bad, ctypes.byref(cache), FAKE, need, None) == -5
    assert b"beyond" in st()
    # more sequences than the cache holds
    assert L.wm_mix_kv(ctypes.byref(c), ctypes.byref(W), FAKE, C.WmTokset(w.B + 1, 4, 0, 1), ctypes.byref(cache),
                       FAKE, need, None) == -2
    # channel_attn: layer out of range
    assert L.wm_channel_attn(ctypes.byref(c), w.L, FAKE, ts, ctypes.byref(cache), FAKE, FAKE, need, None) == -5
    # prefill: g < 1, T > T_max, bad logits mode, missing logits
    ws_p = L.wm_workspace_bytes(ctypes.byref(c), w.B * 128)
    assert L.wm_cyclic_prefill_pass(ctypes.byref(c), ctypes.byref(W), FAKE, w.T, 0, ctypes.byref(cache), None, 0,
                                    FAKE, ws_p, None) == -2
    assert L.wm_cyclic_prefill_pass(ctypes.byref(c), ctypes.byref(W), FAKE, w.T_max + 1, 16, ctypes.byref(cache),
                                    None, 0, FAKE, ws_p, None) == -5
    assert L.wm_cyclic_prefill_pass(ctypes.byref(c), ctypes.byref(W), FAKE, w.T, 16, ctypes.byref(cache), FAKE, 3,
                                    FAKE, ws_p, None) == -1
    assert L.wm_cyclic_prefill_pass(ctypes.byref(c), ctypes.byref(W), FAKE, w.T, 16, ctypes.byref(cache), None, 1,
                                    FAKE, ws_p, None) == -1
    assert L.wm_cyclic_prefill_pass(ctypes.byref(c), ctypes.byref(W), FAKE, w.T, 16, ctypes.byref(cache), None, 0,
                                    FAKE, ws_p - 256, None) == -4
    W0 = _weights()
    W0.router = None
    assert L.wm_cyclic_prefill_pass(ctypes.byref(c), ctypes.byref(W0), FAKE, w.T, 16, ctypes.byref(cache), None, 0,
                                    FAKE, ws_p, None) == -1
    # with static mixing the router is not needed: the null router passes the
    # weight check and the later (launch-free) workspace check fires instead
    W0.static_mix = FAKE
    assert L.wm_cyclic_prefill_pass(ctypes.byref(c), ctypes.byref(W0), FAKE, w.T, 16, ctypes.byref(cache), None, 0,
                                    FAKE, ws_p - 256, None) == -4
    # decode: t outside [0, T_max)
    ws_d = L.wm_workspace_bytes(ctypes.byref(c), w.B)
    for t in (-1, w.T_max):
        assert L.wm_decode_step(ctypes.byref(c), ctypes.byref(W), FAKE, t, ctypes.byref(cache), FAKE, FAKE, ws_d,
                                None) == -5
    # rope table: null output
    assert L.wm_rope_table(ctypes.byref(c), None, FAKE, None) == -1


def test_static_decode_step_validates_before_launch():
    """wm_decode_step_static checks its arguments, then refuses a step whose
    scratch would exceed the static array (WM_STATIC_SCRATCH_BYTES = 64 MiB),
    before it touches the device."""
    L = C.lib()
    W = _weights()
    w = WORKLOADS["prefill_1p3b"]
    c = cfg_of(w)
    static_bytes = 64 << 20
    assert L.wm_workspace_bytes(ctypes.byref(c), 128) <= static_bytes < L.wm_workspace_bytes(ctypes.byref(c), 129)
    cache = C.WmCache(FAKE, FAKE, 129)
    assert L.wm_decode_step_static(ctypes.byref(c), ctypes.byref(W), FAKE, 5, ctypes.byref(cache), FAKE, None) == -4
    assert b"static scratch" in L.wm_last_error()
    cache = C.WmCache(FAKE, FAKE, 64)
    for t in (-1, w.T_max):
        assert L.wm_decode_step_static(ctypes.byref(c), ctypes.byref(W), FAKE, t, ctypes.byref(cache), FAKE,
                                       None) == -5
    assert L.wm_decode_step_static(ctypes.byref(c), ctypes.byref(W), None, 5, ctypes.byref(cache), FAKE, None) == -1
    assert L.wm_decode_step_static(ctypes.byref(c), ctypes.byref(W), FAKE, 5, ctypes.byref(cache), None, None) == -1
    assert L.wm_decode_step_static(ctypes.byref(c), ctypes.byref(W), FAKE, 5, None, FAKE, None) == -1


def test_vanilla_entry_points_validate_before_launch():
    L = C.lib()
    w = WORKLOADS["small_prefill"]
    cv = cfg_of(w, k=w.L)   # the vanilla model: one cache slot per layer
    cw = cfg_of(w)          # k < L: rejected
    W = _weights()
    cache = C.WmCache(FAKE, FAKE, w.B)
    ws = L.wm_workspace_bytes(ctypes.byref(cv), w.B * 128)
    pre = lambda c, T=w.T, chunk=128, logits=None, mode=0, Wt=W, n=ws: L.wm_vanilla_prefill(
        ctypes.byref(c), ctypes.byref(Wt), FAKE, T, chunk, ctypes.byref(cache), logits, mode, FAKE, n, None)
    assert pre(cw) == -2 and b"one cache slot per layer" in L.wm_last_error()
    assert pre(cv, chunk=0) == -2
    assert pre(cv, T=w.T_max + 1) == -5
    assert pre(cv, mode=3, logits=FAKE) == -1
    assert pre(cv, mode=1) == -1
    assert pre(cv, n=ws - 256) == -4
    W0 = _weights()
    W0.wk = None
    assert pre(cv, Wt=W0) == -1
    W1 = _weights()
    W1.router = None  # not read by the vanilla model: only the launch-free checks run, so use a bad T
    assert pre(cv, Wt=W1, T=0) == -5
    wd = L.wm_workspace_bytes(ctypes.byref(cv), w.B)
    for t in (-1, w.T_max):
        assert L.wm_vanilla_decode_step(ctypes.byref(cv), ctypes.byref(W), FAKE, t, ctypes.byref(cache), FAKE, FAKE,
                                        wd, None) == -5
    assert L.wm_vanilla_decode_step(ctypes.byref(cw), ctypes.byref(W), FAKE, 0, ctypes.byref(cache), FAKE, FAKE, wd,
                                    None) == -2


def test_feedback_free_entry_points_validate_before_launch():
    L = C.lib()
    w = WORKLOADS["small_prefill"]
    cf = cfg_of(w, k=w.L)
    cw = cfg_of(w)
    W = _weights()
    cache = C.WmCache(FAKE, FAKE, w.B)
    ws = L.wm_workspace_bytes(ctypes.byref(cf), w.B * 128)
    pre = lambda c, T=w.T, chunk=128, Wt=W, n=ws: L.wm_feedback_free_prefill(
        ctypes.byref(c), ctypes.byref(Wt), FAKE, T, chunk, ctypes.byref(cache), None, 0, FAKE, n, None)
    assert pre(cw) == -2 and b"one channel per layer" in L.wm_last_error()
    assert pre(cf, chunk=0) == -2
    assert pre(cf, T=w.T_max + 1) == -5
    assert pre(cf, n=ws - 256) == -4
    Ws = _weights()
    Ws.static_mix = FAKE
    assert pre(cf, Wt=Ws) == -1
    Wr = _weights()
    Wr.router = None
    assert pre(cf, Wt=Wr) == -1
    wd = L.wm_workspace_bytes(ctypes.byref(cf), w.B)
    for t in (-1, w.T_max):
        assert L.wm_feedback_free_decode_step(ctypes.byref(cf), ctypes.byref(W), FAKE, t, ctypes.byref(cache), FAKE,
                                              FAKE, wd, None) == -5


def test_peak_probes_validate_before_launch():
    L = C.lib()
    out = ctypes.c_double()
    st = lambda src, dst, n, it=1, o=ctypes.byref(out): L.wm_peak_stream(src, dst, n, it, None, o)
    assert st(None, None, 1024) == -1
    assert st(FAKE, None, 1024, o=None) == -1
    assert st(FAKE, None, 0) == -2
    assert st(FAKE, None, 1000) == -2  # not a multiple of 16
    assert st(FAKE + 8, None, 1024) == -2  # misaligned
    assert st(FAKE, FAKE + 4, 1024) == -2  # misaligned dst
    assert st(FAKE, None, 1024, it=0) == -2
    assert st(FAKE, FAKE + 512, 1024) == -1 and b"overlap" in L.wm_last_error()
    assert L.wm_peak_mfma_bf16(1, None, None) == -1
    assert L.wm_peak_mfma_bf16(0, None, ctypes.byref(out)) == -2


def test_binding_checks_tensors_before_calling():
    """The Python binding rejects what a raw pointer cannot show: token ids of
    another integer type (an int64 tensor read as int32 pairs), a
    non-contiguous view, a CPU tensor, a sequence count other than the
    cache's, and a cache of the wrong element type or shape."""
    import torch

    from decode_token_rmsnorm_amd import api

    class _Cache:
        def __init__(self, k, v):
            self.k, self.v = k, v

        @property
        def B(self):
            return self.k.shape[1]

    class _Model:
        shape = WORKLOADS["decode_d512"].replace(T_max=8)
        dtype = "bf16"
        device = torch.device("cpu")

    m = _Model()
    s = m.shape
    good = torch.zeros((s.k, 3, s.Hkv, s.T_max, s.d), dtype=torch.bfloat16)
    cache = _Cache(good, good.clone())
    api.check_tokens(torch.zeros(3, dtype=torch.int32), cache, m.device, 1)
    api.check_tokens(torch.zeros(3, 5, dtype=torch.int32), cache, m.device, 2)
    api.check_cache(m, cache)
    with pytest.raises(TypeError):
        api.check_tokens(torch.zeros(3, dtype=torch.int64), cache, m.device, 1)
    with pytest.raises(ValueError):
        api.check_tokens(torch.zeros(5, 3, dtype=torch.int32).t(), cache, m.device, 2)
    with pytest.raises(ValueError):
        api.check_tokens(torch.zeros(4, dtype=torch.int32), cache, m.device, 1)
    with pytest.raises(ValueError):
        api.check_tokens(torch.zeros(3, 1, dtype=torch.int32), cache, m.device, 1)
    with pytest.raises(TypeError):
        api.check_cache(m, _Cache(good.float(), good.float()))
    with pytest.raises(ValueError):
        api.check_cache(m, _Cache(good[:, :, :, :4], good[:, :, :, :4]))
    if torch.cuda.is_available():  # (a CPU tensor for a model on the GPU)
        with pytest.raises(ValueError):
            api.check_tensor("tokens", torch.zeros(3, dtype=torch.int32), torch.int32, torch.device("cuda"))


def test_train_step_validates_before_launch():
    """wm_train_step: float32 only, the routed model only (no static mixing),
    2 <= T <= T_max, g >= 1, n_nograd >= 0, n_grad >= 1, every pointer set,
    workspace of at least wm_train_workspace_min_bytes; each refused before any
    launch."""
    L = C.lib()
    w = WORKLOADS["tiny_fp32"]
    c = cfg_of(w, dtype=C.WM_F32)
    W = _weights()
    G = C.WmGrads(*[FAKE for _ in C.GRAD_FIELDS])
    need = L.wm_train_workspace_min_bytes(ctypes.byref(c), w.B, w.T, w.g, 2)
    assert need > 0
    # (one undo slot per gradient step; the full size adds one tape per gradient step)
    assert L.wm_train_workspace_min_bytes(ctypes.byref(c), w.B, w.T, w.g, 3) > need
    assert L.wm_train_workspace_bytes(ctypes.byref(c), w.B, w.T, w.g, 2) > need
    assert L.wm_train_workspace_bytes(ctypes.byref(c), w.B, w.T, w.g, 3) > L.wm_train_workspace_bytes(
        ctypes.byref(c), w.B, w.T, w.g, 2)
    for fn in (L.wm_train_workspace_bytes, L.wm_train_workspace_min_bytes):
        assert fn(ctypes.byref(c), w.B, 1, w.g, 2) == 0
        assert fn(ctypes.byref(c), w.B, w.T, w.g, 0) == 0

    def call(cfg=c, Wt=W, Gt=G, B=w.B, T=w.T, g=w.g, n0=1, n1=2, n=need, loss=FAKE):
        return L.wm_train_step(ctypes.byref(cfg), ctypes.byref(Wt), FAKE, B, T, g, n0, n1,
                               None if Gt is None else ctypes.byref(Gt), loss, FAKE, n, None)

    assert call(cfg=cfg_of(w, dtype=C.WM_BF16)) == -3
    assert call(T=1) == -5 and call(T=w.T_max + 1) == -5
    assert call(g=0) == -2
    assert call(n0=-1) == -1 and call(n1=0) == -1
    assert call(B=0) == -2
    assert call(Gt=None) == -1 and call(loss=None) == -1
    assert call(n=need - 1) == -4
    Ws = _weights()
    Ws.static_mix = FAKE
    assert call(Wt=Ws) == -1 and b"static_mix" in L.wm_last_error()
    W0 = _weights()
    W0.rope_cos = None
    assert call(Wt=W0) == -1
    G0 = C.WmGrads(*[FAKE for _ in C.GRAD_FIELDS])
    G0.router = None
    assert call(Gt=G0) == -1


def test_decode_step_at_validates_before_launch():
    """wm_decode_step_at checks every pointer (the position's included) and the
    workspace on the host; the position's value lives on the device."""
    L = C.lib()
    W = _weights()
    w = WORKLOADS["decode_d512"]
    c = cfg_of(w)
    cache = C.WmCache(FAKE, FAKE, w.B)
    need = L.wm_workspace_bytes(ctypes.byref(c), w.B)
    call = lambda t=FAKE, tok=FAKE, lg=FAKE, n=need, Wt=W, cc=cache: L.wm_decode_step_at(
        ctypes.byref(c), ctypes.byref(Wt), tok, t, None if cc is None else ctypes.byref(cc), lg, FAKE, n, None)
    assert call(t=None) == -1 and call(tok=None) == -1 and call(lg=None) == -1 and call(cc=None) == -1
    assert call(n=need - 1) == -4
    W0 = _weights()
    W0.lm_head = None
    assert call(Wt=W0) == -1


def test_train_binding_checks_before_calling():
    """train_step's binding: float32 models only, [B, T] int32 tokens, and
    gradient tensors of the parameters' shapes, all refused before a call."""
    import torch

    from decode_token_rmsnorm_amd import api
    from wm_inputs import weight_shapes

    w = WORKLOADS["tiny_fp32"]

    class _Model:
        shape = w
        device = torch.device("cpu")

        def __init__(self, dtype):
            self.dtype = dtype
            self.t = {n: torch.zeros(sh) for n, sh in weight_shapes(w).items()}

    tok = torch.zeros(1, 16, dtype=torch.int32)
    with pytest.raises(ValueError):
        api.train_step(_Model("bf16"), tok, 4)
    with pytest.raises(ValueError):
        api.train_step(_Model("f32"), torch.zeros(16, dtype=torch.int32), 4)
    with pytest.raises(TypeError):
        api.train_step(_Model("f32"), tok.long(), 4)
    m = _Model("f32")
    grads = {n: torch.zeros_like(t) for n, t in m.t.items()}
    grads["wq"] = torch.zeros(1, 2, 3)
    with pytest.raises(ValueError):
        api.train_step(m, tok, 4, grads=grads)
