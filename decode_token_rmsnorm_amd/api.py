"""Thin torch-facing wrappers over the C ABI (include/wm.h).

torch supplies device memory and the current HIP stream; every step of the
computation runs in the library's kernels. Names follow the C entry points:
``mix_kv``, ``channel_attn``, ``cyclic_prefill_pass``, ``decode_step``.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as C

GAINS = {"final_norm", "attn_norm", "q_norm", "ffn_norm", "src_norm", "chan_norm", "k_norm", "static_mix"}


def torch_dtype(dtype: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def make_config(shape, dtype: str) -> C.WmConfig:
    """shape: any object with L, D, Hq, Hkv, d, F, k, p, V, T_max, eps, rope_base."""
    return C.WmConfig(shape.L, shape.D, shape.Hq, shape.Hkv, shape.d, shape.F, shape.k, shape.p, shape.V,
                      shape.T_max, shape.eps, shape.rope_base, C.WM_BF16 if dtype == "bf16" else C.WM_F32)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


class Model:
    """Device copies of the weights plus the config and RoPE tables.

    ``weights`` maps the names of include/wm.h to host arrays (float32 holding
    values representable in the workload's dtype); matrices are uploaded in
    that dtype, gains as float32. Missing names stay NULL (a mix-only model).
    """

    def __init__(self, shape, weights: dict, dtype: str, device="cuda"):
        self.shape, self.dtype, self.device = shape, dtype, torch.device(device)
        self.cfg = make_config(shape, dtype)
        C.check("wm_check_config", C.lib().wm_check_config(ctypes.byref(self.cfg)))
        td = torch_dtype(dtype)
        self.t = {}
        for n, a in weights.items():
            x = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
            self.t[n] = x.to(self.device, torch.float32 if n in GAINS else td).contiguous()
        half = shape.d // 2
        self.t["rope_cos"] = torch.empty(shape.T_max, half, dtype=torch.float32, device=self.device)
        self.t["rope_sin"] = torch.empty(shape.T_max, half, dtype=torch.float32, device=self.device)
        C.check("wm_rope_table", C.lib().wm_rope_table(ctypes.byref(self.cfg), self.t["rope_cos"].data_ptr(),
                                                       self.t["rope_sin"].data_ptr(), _stream()))
        self.w = C.WmWeights(*[_ptr(self.t.get(n)) for n in C.WEIGHT_FIELDS])

    def workspace(self, rows: int) -> torch.Tensor:
        n = C.lib().wm_workspace_bytes(ctypes.byref(self.cfg), rows)
        if n == 0:
            raise C.WmError("wm_workspace_bytes", -2)
        return torch.empty(n, dtype=torch.uint8, device=self.device)


@dataclass
class Cache:
    k: torch.Tensor
    v: torch.Tensor

    @property
    def B(self) -> int:
        return self.k.shape[1]

    def c(self) -> C.WmCache:
        return C.WmCache(self.k.data_ptr(), self.v.data_ptr(), self.B)


def new_cache(model: Model, B: int, fill: float = 0.0) -> Cache:
    s = model.shape
    shape = (s.k, B, s.Hkv, s.T_max, s.d)
    td = torch_dtype(model.dtype)
    return Cache(torch.full(shape, fill, dtype=td, device=model.device),
                 torch.full(shape, fill, dtype=td, device=model.device))


def cache_from_host(model: Model, K: np.ndarray, V: np.ndarray) -> Cache:
    td = torch_dtype(model.dtype)
    return Cache(torch.from_numpy(np.ascontiguousarray(K, np.float32)).to(model.device, td),
                 torch.from_numpy(np.ascontiguousarray(V, np.float32)).to(model.device, td))


def _ws(model, ws, rows):
    return model.workspace(rows) if ws is None else ws


def _same_device(a: torch.device, b: torch.device) -> bool:
    if a.type != b.type:
        return False
    if a.type != "cuda":
        return True
    cur = torch.cuda.current_device() if (a.index is None or b.index is None) else None
    return (cur if a.index is None else a.index) == (cur if b.index is None else b.index)


def check_tensor(name: str, t: torch.Tensor, dtype, device, shape=None) -> None:
    """What the C ABI cannot see in a raw pointer: element type, layout,
    device and (where given) shape. Raises before anything is launched."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not _same_device(t.device, torch.device(device)):
        raise ValueError(f"{name} is on {t.device}, the model on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def check_tokens(tokens: torch.Tensor, cache: "Cache", device, ndim: int) -> None:
    """tokens: int32, contiguous, on the model's device, [B] (ndim 1) or [B, T]
    (ndim 2) with B = the cache's sequence count."""
    check_tensor("tokens", tokens, torch.int32, device)
    if tokens.dim() != ndim or tokens.shape[0] != cache.B:
        raise ValueError(f"tokens has shape {tuple(tokens.shape)}; expected {ndim} dims with "
                         f"{cache.B} sequences (the cache's B)")


def check_cache(model: "Model", cache: "Cache") -> None:
    s = model.shape
    shape = (s.k, cache.B, s.Hkv, s.T_max, s.d)
    check_tensor("cache.k", cache.k, torch_dtype(model.dtype), model.device, shape)
    check_tensor("cache.v", cache.v, torch_dtype(model.dtype), model.device, shape)


def mix_kv(model: Model, states: torch.Tensor, B: int, M: int, s0: int, s_step: int, cache: Cache, ws=None,
           stream=None) -> None:
    """Pool + append of the state stack ``states`` [L, B*M, D] (rows b*M + m at
    position s0 + m*s_step) into ``cache``."""
    check_tensor("states", states, torch_dtype(model.dtype), model.device, (model.shape.L, B * M, model.shape.D))
    check_cache(model, cache)
    ws = _ws(model, ws, B * M)
    cc = cache.c()
    C.check("wm_mix_kv", C.lib().wm_mix_kv(ctypes.byref(model.cfg), ctypes.byref(model.w), states.data_ptr(),
                                           C.WmTokset(B, M, s0, s_step), ctypes.byref(cc), ws.data_ptr(),
                                           ws.numel(), _stream(stream)))


def channel_attn(model: Model, layer: int, q: torch.Tensor, B: int, M: int, s0: int, s_step: int, cache: Cache,
                 out=None, ws=None, stream=None) -> torch.Tensor:
    """Strict-causal attention of consumer layer ``layer`` for q [B*M, Hq, d]."""
    s = model.shape
    check_tensor("q", q, torch_dtype(model.dtype), model.device, (B * M, s.Hq, s.d))
    check_cache(model, cache)
    if out is None:
        out = torch.empty(B * M, s.Hq * s.d, dtype=q.dtype, device=q.device)
    ws = _ws(model, ws, B * M)
    cc = cache.c()
    C.check("wm_channel_attn", C.lib().wm_channel_attn(ctypes.byref(model.cfg), layer, q.data_ptr(),
                                                       C.WmTokset(B, M, s0, s_step), ctypes.byref(cc),
                                                       out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


def prefill_rows(B: int, T: int, g: int) -> int:
    return B * (-(-T // g))


def cyclic_prefill_pass(model: Model, tokens: torch.Tensor, g: int, cache: Cache, logits_mode: int = 0,
                        logits=None, ws=None, stream=None):
    """One cyclic Gauss-Seidel pass over tokens [B, T] (int32, device)."""
    check_tokens(tokens, cache, model.device, 2)
    check_cache(model, cache)
    B, T = tokens.shape
    if logits_mode and logits is None:
        shape = (B, model.shape.V) if logits_mode == 1 else (B, T, model.shape.V)
        logits = torch.empty(shape, dtype=torch.float32, device=tokens.device)
    ws = _ws(model, ws, prefill_rows(B, T, g))
    cc = cache.c()
    C.check("wm_cyclic_prefill_pass",
            C.lib().wm_cyclic_prefill_pass(ctypes.byref(model.cfg), ctypes.byref(model.w), tokens.data_ptr(), T, g,
                                           ctypes.byref(cc), _ptr(logits), logits_mode, ws.data_ptr(), ws.numel(),
                                           _stream(stream)))
    return logits


def decode_step(model: Model, tokens: torch.Tensor, t: int, cache: Cache, logits=None, ws=None, stream=None):
    """One decode step: tokens [B] (int32, device) at position t."""
    check_tokens(tokens, cache, model.device, 1)
    check_cache(model, cache)
    B = tokens.shape[0]
    if logits is None:
        logits = torch.empty(B, model.shape.V, dtype=torch.float32, device=tokens.device)
    ws = _ws(model, ws, B)
    cc = cache.c()
    C.check("wm_decode_step", C.lib().wm_decode_step(ctypes.byref(model.cfg), ctypes.byref(model.w),
                                                     tokens.data_ptr(), t, ctypes.byref(cc), logits.data_ptr(),
                                                     ws.data_ptr(), ws.numel(), _stream(stream)))
    return logits


def decode_step_at(model: Model, tokens: torch.Tensor, t: torch.Tensor, cache: Cache, logits=None, ws=None,
                   stream=None):
    """wm_decode_step_at: a decode step whose position t (int32 tensor of one
    element, on the device) is read by the kernels when they run, so that a
    captured graph of the call replays at whatever position t then holds."""
    check_tokens(tokens, cache, model.device, 1)
    check_cache(model, cache)
    check_tensor("t", t, torch.int32, model.device, (1,))
    B = tokens.shape[0]
    if logits is None:
        logits = torch.empty(B, model.shape.V, dtype=torch.float32, device=tokens.device)
    ws = _ws(model, ws, B)
    cc = cache.c()
    C.check("wm_decode_step_at", C.lib().wm_decode_step_at(ctypes.byref(model.cfg), ctypes.byref(model.w),
                                                           tokens.data_ptr(), t.data_ptr(), ctypes.byref(cc),
                                                           logits.data_ptr(), ws.data_ptr(), ws.numel(),
                                                           _stream(stream)))
    return logits


def decode_step_static(model: Model, tokens: torch.Tensor, t: int, cache: Cache, logits=None, stream=None):
    """wm_decode_step with the library's static scratch (no workspace, no
    allocation inside the call): tokens [B] (int32, device) at position t."""
    check_tokens(tokens, cache, model.device, 1)
    check_cache(model, cache)
    B = tokens.shape[0]
    if logits is None:
        logits = torch.empty(B, model.shape.V, dtype=torch.float32, device=tokens.device)
    cc = cache.c()
    C.check("wm_decode_step_static", C.lib().wm_decode_step_static(ctypes.byref(model.cfg), ctypes.byref(model.w),
                                                                   tokens.data_ptr(), t, ctypes.byref(cc),
                                                                   logits.data_ptr(), _stream(stream)))
    return logits


def _chunked_prefill(fn: str, model: Model, tokens: torch.Tensor, chunk: int, cache: Cache, logits_mode: int,
                     logits, ws, stream):
    check_tokens(tokens, cache, model.device, 2)
    check_cache(model, cache)
    B, T = tokens.shape
    if logits_mode and logits is None:
        shape = (B, model.shape.V) if logits_mode == 1 else (B, T, model.shape.V)
        logits = torch.empty(shape, dtype=torch.float32, device=tokens.device)
    ws = _ws(model, ws, B * min(chunk, T))
    cc = cache.c()
    C.check(fn, getattr(C.lib(), fn)(ctypes.byref(model.cfg), ctypes.byref(model.w), tokens.data_ptr(), T, chunk,
                                     ctypes.byref(cc), _ptr(logits), logits_mode, ws.data_ptr(), ws.numel(),
                                     _stream(stream)))
    return logits


def _one_step(fn: str, model: Model, tokens: torch.Tensor, t: int, cache: Cache, logits, ws, stream):
    check_tokens(tokens, cache, model.device, 1)
    check_cache(model, cache)
    B = tokens.shape[0]
    if logits is None:
        logits = torch.empty(B, model.shape.V, dtype=torch.float32, device=tokens.device)
    ws = _ws(model, ws, B)
    cc = cache.c()
    C.check(fn, getattr(C.lib(), fn)(ctypes.byref(model.cfg), ctypes.byref(model.w), tokens.data_ptr(), t,
                                     ctypes.byref(cc), logits.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))
    return logits


def feedback_free_prefill(model: Model, tokens: torch.Tensor, chunk: int, cache: Cache, logits_mode: int = 0,
                          logits=None, ws=None, stream=None):
    """The feedback-free variant (k = L, channel l from states 0..l) over
    tokens [B, T] in steps of `chunk` consecutive positions."""
    return _chunked_prefill("wm_feedback_free_prefill", model, tokens, chunk, cache, logits_mode, logits, ws, stream)


def feedback_free_decode_step(model: Model, tokens: torch.Tensor, t: int, cache: Cache, logits=None, ws=None,
                              stream=None):
    """One decode step of the feedback-free variant at position t."""
    return _one_step("wm_feedback_free_decode_step", model, tokens, t, cache, logits, ws, stream)


def vanilla_prefill(model: Model, tokens: torch.Tensor, chunk: int, cache: Cache, logits_mode: int = 0,
                    logits=None, ws=None, stream=None):
    """The vanilla comparison model (per-layer K/V, causal s <= i) over tokens
    [B, T] (int32, device) in steps of `chunk` consecutive positions; the model
    needs k = L (one cache slot per layer)."""
    check_tokens(tokens, cache, model.device, 2)
    check_cache(model, cache)
    B, T = tokens.shape
    if logits_mode and logits is None:
        shape = (B, model.shape.V) if logits_mode == 1 else (B, T, model.shape.V)
        logits = torch.empty(shape, dtype=torch.float32, device=tokens.device)
    ws = _ws(model, ws, B * min(chunk, T))
    cc = cache.c()
    C.check("wm_vanilla_prefill",
            C.lib().wm_vanilla_prefill(ctypes.byref(model.cfg), ctypes.byref(model.w), tokens.data_ptr(), T, chunk,
                                       ctypes.byref(cc), _ptr(logits), logits_mode, ws.data_ptr(), ws.numel(),
                                       _stream(stream)))
    return logits


def vanilla_decode_step(model: Model, tokens: torch.Tensor, t: int, cache: Cache, logits=None, ws=None,
                        stream=None):
    """One decode step of the vanilla comparison model at position t."""
    check_tokens(tokens, cache, model.device, 1)
    check_cache(model, cache)
    B = tokens.shape[0]
    if logits is None:
        logits = torch.empty(B, model.shape.V, dtype=torch.float32, device=tokens.device)
    ws = _ws(model, ws, B)
    cc = cache.c()
    C.check("wm_vanilla_decode_step",
            C.lib().wm_vanilla_decode_step(ctypes.byref(model.cfg), ctypes.byref(model.w), tokens.data_ptr(), t,
                                           ctypes.byref(cc), logits.data_ptr(), ws.data_ptr(), ws.numel(),
                                           _stream(stream)))
    return logits


def peak_stream(src: torch.Tensor, dst: torch.Tensor = None, iters: int = 10, stream=None) -> float:
    """GB/s the device reaches streaming src's bytes: a read (dst None) or a
    copy into dst (counted as read + write). Measurement support only."""
    nbytes = src.numel() * src.element_size()
    if dst is not None and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    out = ctypes.c_double()
    C.check("wm_peak_stream", C.lib().wm_peak_stream(src.data_ptr(), _ptr(dst), nbytes, iters, _stream(stream),
                                                     ctypes.byref(out)))
    return out.value


def peak_mfma_bf16(iters: int = 10, stream=None) -> float:
    """TFLOP/s of a register-resident 32x32x16 bf16 MFMA loop on every compute
    unit. Measurement support only."""
    out = ctypes.c_double()
    C.check("wm_peak_mfma_bf16", C.lib().wm_peak_mfma_bf16(iters, _stream(stream), ctypes.byref(out)))
    return out.value


def train_workspace(model: Model, B: int, T: int, g: int, n_grad: int = 2, keep_tapes: bool = True) -> torch.Tensor:
    """Workspace of a training step: with keep_tapes the size that also keeps
    every gradient step's forward intermediates (when that stays within 64
    GiB), else the minimum, with which the step recomputes them."""
    fn = "wm_train_workspace_bytes" if keep_tapes else "wm_train_workspace_min_bytes"
    n = getattr(C.lib(), fn)(ctypes.byref(model.cfg), B, T, g, n_grad)
    if n == 0:
        raise C.WmError(fn, -2)
    return torch.empty(n, dtype=torch.uint8, device=model.device)


def train_step(model: Model, tokens: torch.Tensor, g: int, n_nograd: int = 1, n_grad: int = 2, grads=None,
               ws=None, stream=None):
    """One training step with truncated backpropagation on tokens [B, T]
    (int32, device), float32 models only: n_nograd cyclic passes without
    gradient, n_grad with it, next-token cross-entropy of the last pass.
    Returns (loss: float32 device tensor [1], grads: {name: float32 tensor of
    the parameter's shape}); ``grads`` may be given to be overwritten."""
    if model.dtype != "f32":
        raise ValueError("the training step runs on float32 models only")
    check_tensor("tokens", tokens, torch.int32, model.device)
    if tokens.dim() != 2:
        raise ValueError(f"tokens must be [B, T], got shape {tuple(tokens.shape)}")
    B, T = tokens.shape
    if grads is None:
        grads = {n: torch.empty_like(model.t[n]) for n in C.GRAD_FIELDS}
    for n in C.GRAD_FIELDS:
        check_tensor(f"grads[{n}]", grads[n], torch.float32, model.device, tuple(model.t[n].shape))
    if ws is None:
        ws = train_workspace(model, B, T, g, n_grad)
    loss = torch.empty(1, dtype=torch.float32, device=model.device)
    gw = C.WmGrads(*[grads[n].data_ptr() for n in C.GRAD_FIELDS])
    C.check("wm_train_step", C.lib().wm_train_step(ctypes.byref(model.cfg), ctypes.byref(model.w), tokens.data_ptr(),
                                                   B, T, g, n_nograd, n_grad, ctypes.byref(gw), loss.data_ptr(),
                                                   ws.data_ptr(), ws.numel(), _stream(stream)))
    return loss, grads
