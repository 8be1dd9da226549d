"""Seeded synthetic inputs for the WhiteMatter KV-pool path.

This module is the only code shared by the oracle and the HIP path's tests
and bench. It holds no arithmetic of the method itself: it only draws
random weights, tokens, state stacks and caches, rounds them to bf16 where
a workload is bf16, and names the five workloads.

Recipe (see the paperlayer.ai and onedev.kr summaries of WhiteMatter,
arXiv 2608.18486, for the model family these shapes come from):

* every matrix (embedding, LM head, W_Q, W_O, FFN, routers, W_K, W_V) is
  N(0, 0.02) in float32, drawn from its own stream
  ``Generator(PCG64(SeedSequence([seed, crc32(name)])))``;
* norm gains are 1.0, or ``1 + U(-0.1, 0.1)`` when ``gains="perturbed"``
  (used by tests so that a gain applied to the wrong layer or channel shows);
* token ids: truncated Zipf(1.1) over the vocabulary (rank r has weight
  r**-1.1, id = r - 1), uniform ids for the tiny fp32 workload;
* a state stack for the mix-only workload: N(0, 1) times a per-layer scale
  drawn from U[0.5, 4];
* a pre-filled decode cache: N(0, 1) keys and values at positions < t.

For bf16 workloads every value is rounded to the nearest bf16 (ties to
even) and returned as float32 holding a bf16-representable value, so that
both sides start from bit-identical inputs.
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np

# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    L: int
    D: int
    Hq: int
    Hkv: int
    d: int
    F: int
    k: int
    p: int
    V: int
    B: int
    T: int
    T_max: int
    g: int
    passes: int
    dtype: str  # "f32" or "bf16"
    token_dist: str  # "uniform" or "zipf"
    eps: float = 1e-6
    rope_base: float = 1e6

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def R(self) -> int:
        """Number of layers the router reads (layers 0, p, 2p, ... < L)."""
        return (self.L + self.p - 1) // self.p


WORKLOADS = {
    # Tiny fp32 decoder: L4 D128 4x32 MHA, FFN 384, k=2, p=2, V=512, B=1,
    # T=128, cyclic g=16 for 4 passes.
    "tiny_fp32": Workload("tiny_fp32", L=4, D=128, Hq=4, Hkv=4, d=32, F=384, k=2, p=2,
                          V=512, B=1, T=128, T_max=128, g=16, passes=4, dtype="f32",
                          token_dist="uniform"),
    # Mix kernel alone: state stack [16, 8, 2048, 512], k=8, 4 KV heads x 64.
    # (Hq, F and V are not used by the mix; they are the small model's.)
    "mix_bf16": Workload("mix_bf16", L=16, D=512, Hq=8, Hkv=4, d=64, F=1536, k=8, p=2,
                         V=32768, B=8, T=2048, T_max=2048, g=1, passes=1, dtype="bf16",
                         token_dist="zipf"),
    # Small half-cache model, cyclic prefill g=16, 3 passes.
    "small_prefill": Workload("small_prefill", L=16, D=512, Hq=8, Hkv=4, d=64, F=1536, k=8,
                              p=2, V=32768, B=8, T=2048, T_max=2048, g=16, passes=3,
                              dtype="bf16", token_dist="zipf"),
    # Decode step, full cache (k=16), batch 64, 2047 cached positions.
    "decode_d512": Workload("decode_d512", L=16, D=512, Hq=8, Hkv=4, d=64, F=1536, k=16,
                            p=2, V=32768, B=64, T=2047, T_max=2048, g=1, passes=1,
                            dtype="bf16", token_dist="zipf"),
    # 1.3B-scale half-cache model, cyclic prefill g=16, 1 + 2 passes.
    "prefill_1p3b": Workload("prefill_1p3b", L=28, D=1792, Hq=14, Hkv=2, d=128, F=4864,
                             k=14, p=2, V=32768, B=64, T=2048, T_max=2048, g=16, passes=3,
                             dtype="bf16", token_dist="zipf"),
}

# ---------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# ---------------------------------------------------------------------------


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bf16_bits(x))


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


# ---------------------------------------------------------------------------
# weights
# ---------------------------------------------------------------------------


def weight_shapes(w: Workload) -> dict:
    """Name -> shape of every parameter. Matrices are row-major [out, in].

    Index 0 of the leading "2" axis is the key branch, 1 the value branch.
    """
    L, D, Hq, Hkv, d, F, k, V, R = w.L, w.D, w.Hq, w.Hkv, w.d, w.F, w.k, w.V, w.R
    return {
        "embed": (V, D), "lm_head": (V, D), "final_norm": (D,),
        "attn_norm": (L, D), "wq": (L, Hq * d, D), "q_norm": (L, d), "wo": (L, D, Hq * d),
        "ffn_norm": (L, D), "w_gate": (L, F, D), "w_up": (L, F, D), "w_down": (L, D, F),
        "src_norm": (2, L, D), "router": (2, L * k, R * D), "chan_norm": (2, k, D),
        "wk": (k, Hkv * d, D), "wv": (k, Hkv * d, D), "k_norm": (k, d),
    }


GAIN_NAMES = ("final_norm", "attn_norm", "q_norm", "ffn_norm", "src_norm", "chan_norm", "k_norm")
POOL_NAMES = ("src_norm", "router", "chan_norm", "wk", "wv", "k_norm")


def make_weight(w: Workload, name: str, seed: int = 0, gains: str = "ones") -> np.ndarray:
    shape = weight_shapes(w)[name]
    if name in GAIN_NAMES:
        if gains == "ones":
            return np.ones(shape, np.float32)
        r = _rng(seed, name)
        return _finish(1.0 + r.uniform(-0.1, 0.1, size=shape), w.dtype)
    r = _rng(seed, name)
    return _finish(r.standard_normal(size=shape, dtype=np.float32) * np.float32(0.02), w.dtype)


def make_static_mix(w: Workload, seed: int = 5) -> np.ndarray:
    """[2, L, k] float32 constant signed mixing weights (the static-mixing
    variant): N(0, 1) draws."""
    r = _rng(seed, "static_mix")
    return r.standard_normal(size=(2, w.L, w.k), dtype=np.float32)


def make_weights(w: Workload, seed: int = 0, gains: str = "ones", names=None) -> dict:
    names = list(weight_shapes(w)) if names is None else list(names)
    return {n: make_weight(w, n, seed, gains) for n in names}


# ---------------------------------------------------------------------------
# tokens, state stacks, caches
# ---------------------------------------------------------------------------


def make_tokens(w: Workload, seed: int = 1, B: int | None = None, T: int | None = None,
                dist: str | None = None) -> np.ndarray:
    B = w.B if B is None else B
    T = w.T if T is None else T
    dist = w.token_dist if dist is None else dist
    r = _rng(seed, "tokens")
    if dist == "uniform":
        return r.integers(0, w.V, size=(B, T), dtype=np.int64).astype(np.int32)
    ranks = np.arange(1, w.V + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** -1.1)
    cdf /= cdf[-1]
    u = r.random(size=(B, T))
    return np.minimum(np.searchsorted(cdf, u, side="right"), w.V - 1).astype(np.int32)


def make_state_stack(w: Workload, rows: int, seed: int = 2) -> np.ndarray:
    """[L, rows, D]: N(0,1) scaled per layer by U[0.5, 4]."""
    r = _rng(seed, "states")
    scale = r.uniform(0.5, 4.0, size=(w.L, 1, 1)).astype(np.float32)
    x = r.standard_normal(size=(w.L, rows, w.D), dtype=np.float32) * scale
    return _finish(x, w.dtype)


def make_cache(w: Workload, B: int, filled: int, seed: int = 3, poison: bool = False):
    """Two arrays [k, B, Hkv, T_max, d]: N(0,1) at positions < filled.

    Positions >= filled hold 0, or NaN when ``poison`` is set (a slot that
    must never be read).
    """
    r = _rng(seed, "cache")
    shape = (w.k, B, w.Hkv, w.T_max, w.d)
    out = []
    for _ in range(2):
        x = np.zeros(shape, np.float32)
        x[:, :, :, :filled] = r.standard_normal(size=(w.k, B, w.Hkv, filled, w.d), dtype=np.float32)
        if poison:
            x[:, :, :, filled:] = np.nan
        out.append(_finish(x, w.dtype))
    return out[0], out[1]


def make_queries(w: Workload, rows: int, seed: int = 4) -> np.ndarray:
    """[rows, Hq, d] N(0,1) queries (already normed and rotated, for the attention alone)."""
    r = _rng(seed, "queries")
    return _finish(r.standard_normal(size=(rows, w.Hq, w.d), dtype=np.float32), w.dtype)


def make_cache_device(w: Workload, B: int, filled: int, seed: int = 3, device="cuda"):
    """Like ``make_cache`` but drawn on the device with torch's seeded generator
    (for full-size timing inputs that are never compared with the oracle)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shape = (w.k, B, w.Hkv, w.T_max, w.d)
    out = []
    for _ in range(2):
        x = torch.zeros(shape, dtype=td, device=device)
        x[:, :, :, :filled] = torch.randn((w.k, B, w.Hkv, filled, w.d), generator=g, device=device).to(td)
        out.append(x)
    return out[0], out[1]


def make_state_stack_device(w: Workload, rows: int, seed: int = 2, device="cuda"):
    """Like ``make_state_stack`` but drawn on the device with torch's seeded
    generator (full-size timing inputs, never compared with the oracle)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    scale = torch.rand((w.L, 1, 1), generator=g, device=device) * 3.5 + 0.5
    out = torch.empty((w.L, rows, w.D), dtype=td, device=device)
    for l in range(w.L):  # one layer at a time keeps the fp32 temporary small
        out[l] = (torch.randn((rows, w.D), generator=g, device=device) * scale[l]).to(td)
    return out
