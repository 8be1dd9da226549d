"""ctypes view of the C ABI declared in include/wm.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "wm.h")

c_i32, c_f32, c_vp, c_size = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

WM_F32, WM_BF16 = 0, 1
STATUS = {0: "WM_OK", -1: "WM_ERR_ARG", -2: "WM_ERR_SHAPE", -3: "WM_ERR_DTYPE", -4: "WM_ERR_WORKSPACE",
          -5: "WM_ERR_RANGE", -6: "WM_ERR_HIP"}


class WmConfig(ctypes.Structure):
    _fields_ = [("L", c_i32), ("D", c_i32), ("Hq", c_i32), ("Hkv", c_i32), ("d", c_i32), ("F", c_i32),
                ("k", c_i32), ("p", c_i32), ("V", c_i32), ("T_max", c_i32), ("eps", c_f32),
                ("rope_base", c_f32), ("dtype", c_i32)]


WEIGHT_FIELDS = ["embed", "lm_head", "final_norm", "attn_norm", "wq", "q_norm", "wo", "ffn_norm", "w_gate", "w_up",
                 "w_down", "src_norm", "router", "chan_norm", "wk", "wv", "k_norm", "rope_cos", "rope_sin",
                 "static_mix"]


class WmWeights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in WEIGHT_FIELDS]


GRAD_FIELDS = ["embed", "lm_head", "final_norm", "attn_norm", "wq", "q_norm", "wo", "ffn_norm", "w_gate", "w_up",
               "w_down", "src_norm", "router", "chan_norm", "wk", "wv", "k_norm"]


class WmGrads(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in GRAD_FIELDS]


class WmCache(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp), ("B", c_i32)]


class WmTokset(ctypes.Structure):
    _fields_ = [("B", c_i32), ("M", c_i32), ("s0", c_i32), ("s_step", c_i32)]


P = ctypes.POINTER
_SIGS = {
    "wm_last_error": (ctypes.c_char_p, []),
    "wm_check_config": (c_i32, [P(WmConfig)]),
    "wm_group_positions": (c_i32, [c_i32, c_i32, c_i32, P(c_i32)]),
    "wm_channel_of_layer": (c_i32, [c_i32, c_i32]),
    "wm_cache_elems": (ctypes.c_int64, [P(WmConfig), c_i32]),
    "wm_workspace_bytes": (c_size, [P(WmConfig), c_i32]),
    "wm_rope_table": (c_i32, [P(WmConfig), c_vp, c_vp, c_vp]),
    "wm_mix_kv": (c_i32, [P(WmConfig), P(WmWeights), c_vp, WmTokset, P(WmCache), c_vp, c_size, c_vp]),
    "wm_channel_attn": (c_i32, [P(WmConfig), c_i32, c_vp, WmTokset, P(WmCache), c_vp, c_vp, c_size, c_vp]),
    "wm_cyclic_prefill_pass": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, c_i32, P(WmCache), c_vp, c_i32,
                                       c_vp, c_size, c_vp]),
    "wm_decode_step": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, P(WmCache), c_vp, c_vp, c_size, c_vp]),
    "wm_decode_step_static": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, P(WmCache), c_vp, c_vp]),
    "wm_decode_step_at": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_vp, P(WmCache), c_vp, c_vp, c_size, c_vp]),
    "wm_vanilla_prefill": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, c_i32, P(WmCache), c_vp, c_i32, c_vp,
                                   c_size, c_vp]),
    "wm_vanilla_decode_step": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, P(WmCache), c_vp, c_vp, c_size,
                                       c_vp]),
    "wm_feedback_free_prefill": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, c_i32, P(WmCache), c_vp, c_i32,
                                         c_vp, c_size, c_vp]),
    "wm_feedback_free_decode_step": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, P(WmCache), c_vp, c_vp,
                                             c_size, c_vp]),
    "wm_train_workspace_bytes": (c_size, [P(WmConfig), c_i32, c_i32, c_i32, c_i32]),
    "wm_train_workspace_min_bytes": (c_size, [P(WmConfig), c_i32, c_i32, c_i32, c_i32]),
    "wm_train_step": (c_i32, [P(WmConfig), P(WmWeights), c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, P(WmGrads), c_vp,
                              c_vp, c_size, c_vp]),
    "wm_profile_begin": (c_i32, [ctypes.c_uint32]),
    "wm_profile_read": (c_i32, [P(ctypes.c_int64), P(ctypes.c_double)]),
    "wm_profile_end": (c_i32, []),
    "wm_peak_stream": (c_i32, [c_vp, c_vp, ctypes.c_int64, c_i32, c_vp, P(ctypes.c_double)]),
    "wm_peak_mfma_bf16": (c_i32, [c_i32, c_vp, P(ctypes.c_double)]),
}

KINDS = ["qproj", "attn", "oproj", "gateup", "down", "router", "mix", "kvproj", "lmhead", "embed"]

_lib = None


def header_functions(path: str = HEADER) -> list:
    """Names of the functions include/wm.h declares."""
    with open(path) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(wm_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """The loaded HIP library. Raises if it has not been built: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                               f"g.build()'` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().wm_last_error().decode()


class WmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {last_error()}")


def check(fn: str, status: int) -> None:
    if status != 0:
        raise WmError(fn, status)
