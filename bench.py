"""Benchmark: cyclic-prefill tokens/s per pass (1.3B-scale WhiteMatter model,
L=28 D=1792 14/2 heads x 128, FFN 4864, k=14, p=2, V=32768, B=64, T=2048,
g=16), decode tokens/s (L=16 D=512 8/4 x 64, k=16, B=64, 2047 cached
positions) and the KV-pool mix/append call on a [16, 16384, 512] state stack,
on one GPU, with roofline fractions and the oracle timed on the host cores.

A step is one cyclic Gauss-Seidel prefill pass over the whole batch; the
first (warmup) pass starts from the zero cache and later passes refine it,
as in a 1 + 2 pass prefill. Prints one JSON line.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3   # MI355X float32, dense MFMA (the vector ALU has the same peak)


CSRC = "decode_token_rmsnorm_amd/csrc/"
# committed rocprofv3 HBM-byte summaries and the kernel sources they were taken from
TRAFFIC = {
    "gateup": ("prefill_1p3b_gateup_traffic.md", ["wm_common.hpp", "wm_gemm.hpp", "wm_gemm2.hpp"]),
    "decode_attn": ("decode_d512_attn_traffic.md", ["wm_common.hpp", "wm_attn.hpp", "wm_attn2.hpp"]),
    "mix_kv": ("mix_bf16_mix_kv_traffic.md", ["wm_common.hpp", "wm_gemm.hpp", "wm_gemm2.hpp", "wm_few.hpp",
                                              "wm_pool.hpp", "wm_pool2.hpp", "wm_kvs.hpp", "wm_api.hip"]),
}


def source_hash(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, CSRC + f), "rb").read())
    return h.hexdigest()[:16]


def profiled_traffic(key):
    """HBM bytes per launch (per call for mix_kv) from a committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (calibrated against a plain copy), or None
    when the kernel sources changed since those counters were taken."""
    name, files = TRAFFIC[key]
    try:
        text = open(os.path.join(ROOT, "profiles", name)).read()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith(("-", "|", "#")))
    if fields.get("source_sha256_16", "").strip() != source_hash(files):
        return None
    return int(fields["traffic_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def peak_reset():
    """Start a peak-memory window (weights already on the device count)."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()


def peak_gib():
    """Peak device memory allocated through torch since peak_reset(): weights,
    cache, workspace, tokens and logits (the library allocates nothing)."""
    import torch
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() / 2 ** 30


def profile(kinds_mask):
    from decode_token_rmsnorm_amd import _lib as C
    C.check("wm_profile_begin", C.lib().wm_profile_begin(kinds_mask))


def profile_read():
    from decode_token_rmsnorm_amd import _lib as C
    n = len(C.KINDS)
    counts = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    C.check("wm_profile_read", C.lib().wm_profile_read(counts, ms))
    C.lib().wm_profile_end()
    return {k: (counts[i], ms[i]) for i, k in enumerate(C.KINDS) if counts[i]}


def bench_prefill(steps, warmup):
    import torch
    import decode_token_rmsnorm_amd as wm
    from wm_inputs import WORKLOADS, make_tokens, make_weights

    w = WORKLOADS["prefill_1p3b"]
    t0 = time.time()
    W = make_weights(w, seed=0)
    log(f"[prefill] weights generated in {time.time() - t0:.1f}s")
    model = wm.Model(w, W, "bf16")
    del W
    peak_reset()
    tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
    cache = wm.new_cache(model, w.B)
    rows = wm.prefill_rows(w.B, w.T, w.g)
    ws = model.workspace(rows)
    logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
    for i in range(warmup):
        wm.cyclic_prefill_pass(model, tok, w.g, cache, 1, logits, ws)
        torch.cuda.synchronize()
        log(f"[prefill] warmup pass {i + 1} done")
    from decode_token_rmsnorm_amd import _lib as C
    # Only the gate/up launches are bracketed with events in the timed passes
    # (events around every launch kind add about 4% to a pass).
    profile(1 << C.KINDS.index("gateup"))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        wm.cyclic_prefill_pass(model, tok, w.g, cache, 1, logits, ws)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_pass = [a.elapsed_time(b) for a, b in evs]
    prof = profile_read()
    log(f"[prefill] {steps} passes in {wall:.3f}s: {per_pass}")
    assert torch.isfinite(logits).all(), "non-finite logits"
    n_ga, ms_ga = prof["gateup"]
    flops_ga = 2.0 * rows * (2 * w.F) * w.D
    # the other kinds' times from one further (untimed) pass
    profile(1 << C.KINDS.index("attn") | 1 << C.KINDS.index("qproj") | 1 << C.KINDS.index("oproj")
            | 1 << C.KINDS.index("down"))
    wm.cyclic_prefill_pass(model, tok, w.g, cache, 1, logits, ws)
    torch.cuda.synchronize()
    prof.update(profile_read())
    kern = {k: {"launches": c, "avg_us": 1e3 * m / c} for k, (c, m) in prof.items()}
    res = {
        "wall_s": wall, "per_pass_ms": per_pass, "rows_per_group": rows, "kernels": kern,
        "roofline": {"kernel": "gateup (fused gate/up projection + SwiGLU GEMM)", "bound": "mfma",
                     "achieved": flops_ga / (ms_ga / n_ga * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "traffic": profiled_traffic("gateup"),
                     "algorithmic_per_launch": f"{flops_ga:.4e} FLOP = 2*{rows}*{2 * w.F}*{w.D}"},
    }
    res["roofline"]["frac"] = res["roofline"]["achieved"] / res["roofline"]["peak"]
    # whole-pass MFMA fraction: algorithmic FLOP per pass / pass time
    res["cache_gib"] = 2 * cache.k.numel() * cache.k.element_size() / 2 ** 30
    res["peak_memory_gib"] = peak_gib()
    flop_pass = pass_flops(w)
    res["pass_tflops"] = flop_pass / (wall / steps) / 1e12
    res["pass_flop"] = flop_pass
    del cache, ws, model
    torch.cuda.empty_cache()
    return w, res


def flops_per_token(w, kind="wm", keys=None, lm_head=True):
    """Algorithmic forward FLOP of one token through the whole model (one
    multiply-add = 2 FLOP): the L blocks (Q, O, gate/up, down products), the
    K/V path (WhiteMatter: router, mix and per-channel K/V projections of
    both branches; vanilla: every layer's own K/V projection), attention
    (QK^T and PV) over `keys` keys in every layer, and the LM head.
    keys=None: the average over a whole sequence of w.T positions, (T-1)/2
    keys under WhiteMatter's strict mask and (T+1)/2 under vanilla's causal
    one (the triangle counted once)."""
    T, L, D, F, k, R = w.T, w.L, w.D, w.F, w.k, w.R
    qd, kvd = w.Hq * w.d, w.Hkv * w.d
    f = L * (2 * D * qd * 2 + 2 * D * 2 * F + 2 * F * D)             # Q, O, gate/up, down
    if kind == "wm":
        f += 2 * (2 * R * D * L * k) + 2 * (2 * k * L * D) + 2 * (2 * k * D * kvd)  # router, mix, K/V proj
        keys = (T - 1) / 2 if keys is None else keys
    else:
        f += L * 2 * (2 * D * kvd)                                    # per-layer K/V projections
        keys = (T + 1) / 2 if keys is None else keys
    f += L * w.Hq * w.d * 4 * keys
    return f + (2 * D * w.V if lm_head else 0)


def pass_flops(w):
    """Algorithmic FLOP of one cyclic pass over the batch (strict-causal
    triangle counted once; logits of the last position only, which the LM
    head adds about 0.02% to, left out)."""
    return w.B * w.T * flops_per_token(w, "wm", lm_head=False)


GRAPHS = True  # the graph-replay legs (off for counter-collection runs: --no-graph)


def bench_decode(steps, warmup):
    import torch
    import decode_token_rmsnorm_amd as wm
    from wm_inputs import WORKLOADS, make_cache_device, make_tokens, make_weights

    w = WORKLOADS["decode_d512"]
    t = 2047
    W = make_weights(w, seed=0)
    model = wm.Model(w, W, "bf16")
    peak_reset()
    K, V = make_cache_device(w, w.B, filled=t, seed=3)
    cache = wm.Cache(K, V)
    tok = torch.from_numpy(make_tokens(w, seed=1, B=w.B, T=1)[:, 0].copy()).cuda()
    ws = model.workspace(w.B)
    logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        wm.decode_step(model, tok, t, cache, logits, ws)
    from decode_token_rmsnorm_amd import _lib as C
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wm.decode_step(model, tok, t, cache, logits, ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # attention launches timed with events over as many further steps (events
    # around each of a step's 16 attention launches add about 10% to a step)
    profile(1 << C.KINDS.index("attn"))
    for _ in range(steps):
        wm.decode_step(model, tok, t, cache, logits, ws)
    torch.cuda.synchronize()
    prof = profile_read()
    n_at, ms_at = prof["attn"]
    # per-kind breakdown from a few further (untimed) steps
    profile((1 << len(C.KINDS)) - 1)
    for _ in range(5):
        wm.decode_step(model, tok, t, cache, logits, ws)
    torch.cuda.synchronize()
    kern = {k: {"launches": c, "avg_us": 1e3 * m / c} for k, (c, m) in profile_read().items()}
    profile(0)
    # the same step with its position in device memory (wm_decode_step_at),
    # captured once in a graph and replayed
    g_wall = None
    tdev = torch.tensor([t], dtype=torch.int32, device="cuda")
    if GRAPHS:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            wm.decode_step_at(model, tok, tdev, cache, logits, ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            wm.decode_step_at(model, tok, tdev, cache, logits, ws)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        g_wall = time.perf_counter() - t0
        del graph
    kv_bytes = 2.0 * w.B * w.Hkv * t * w.d * 2  # K and V of one channel, bf16, per layer launch
    ach = kv_bytes / (ms_at / n_at * 1e-3) / 1e9
    return {"workload": "decode_d512: L16 D512 Hq8 Hkv4 d64 F1536 k16 p2 V32768 B64, t=2047 cached, bf16",
            "value": w.B * steps / wall, "unit": "tokens/s", "ms_per_step": 1e3 * wall / steps, "steps": steps,
            "peak_memory_gib": peak_gib(), "cache_gib": 2 * K.numel() * K.element_size() / 2 ** 30,
            "graph_replay": None if g_wall is None else {
                "ms_per_step": 1e3 * g_wall / steps, "value": w.B * steps / g_wall,
                "how": "wm_decode_step_at (position in device memory) captured once, replayed"},
            "kernels_avg_us": kern,
            "roofline": {"kernel": "attn (strict-causal channel attention, attn_few)", "bound": "hbm",
                         "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                         "traffic": profiled_traffic("decode_attn"),
                         "algorithmic_per_launch": f"{kv_bytes:.4e} B = 2*{w.B}*{w.Hkv}*{t}*{w.d}*2"}}


CPU_BASELINE = True  # off with --no-cpu-baseline


def train_cpu_baseline(w, T=24, g=4):
    """The training oracle (float64 torch autograd) on a bounded sample of the
    training workload: one sequence of T positions at the same widths, g
    groups, 1 + 2 passes; tokens/s of training steps."""
    import torch
    from oracle import wm_train as TR
    import oracle as O
    from wm_inputs import make_tokens, make_weights

    ws_ = w.replace(B=1, T=T, T_max=T)
    M = O.Model(ws_, make_weights(ws_, seed=0))
    tokens = make_tokens(ws_, seed=1)
    t0 = time.perf_counter()
    TR.train_step(M, tokens, g, 1, 2)
    dt = time.perf_counter() - t0
    return {"value": T / dt, "unit": "tokens/s (training steps)", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"one sequence of {T} positions at the same widths, g = {g}, 1 + 2 passes, float64 autograd, "
                      f"{dt:.1f} s (attention over at most {T - 1} keys: cheaper per token than the GPU's T = "
                      f"{w.T})"}


def bench_train(steps=1, warmup=1):
    """One training step with truncated backpropagation (wm_train_step: one
    cyclic pass without gradient, two with, next-token cross-entropy of the
    last pass) at the small model's widths in float32: L16 D512 8/4 x 64,
    F1536, k8, p2, V32768, B8 T2048, g16.  tokens/s per step; the
    algorithmic FLOP (a forward pass per pass plus twice a forward per
    gradient pass: 7 forward passes) against the float32 vector peak, since
    every training kernel runs on the vector ALUs in float32."""
    import torch
    import decode_token_rmsnorm_amd as wm
    from wm_inputs import WORKLOADS, make_tokens, make_weights

    w = WORKLOADS["small_prefill"].replace(dtype="f32")
    model = wm.Model(w, make_weights(w, seed=0), "f32")
    tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
    peak_reset()
    ws = wm.train_workspace(model, w.B, w.T, w.g, 2)
    grads = None
    for _ in range(warmup):
        loss, grads = wm.train_step(model, tok, w.g, 1, 2, grads=grads, ws=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        loss, grads = wm.train_step(model, tok, w.g, 1, 2, grads=grads, ws=ws)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    flop = 7 * w.B * w.T * flops_per_token(w, "wm")
    ach = flop / dt / 1e12
    cpu = None if not CPU_BASELINE else train_cpu_baseline(w)
    return {"workload": "small model widths, fp32: L16 D512 Hq8 Hkv4 d64 F1536 k8 p2 V32768, B8 T2048, g16, "
                        "1 pass without + 2 with gradient",
            "cpu_baseline": cpu,
            "value": w.B * w.T / dt, "unit": "tokens/s (training steps)", "s_per_step": dt, "steps": steps,
            "loss": float(loss.item()), "peak_memory_gib": peak_gib(),
            "roofline": {"kernel": "whole training step", "bound": "mfma", "achieved": ach, "peak": FP32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": ach / FP32_PEAK_TFLOPS, "traffic": None,
                         "algorithmic_per_step": f"{flop:.4e} FLOP = 7 forward passes of {w.B}x{w.T} tokens"}}


def graph_passes(model, tok, w, logits, ws):
    """Per-pass ms of w.passes passes from the zero cache, replayed from one
    captured graph of wm_cyclic_prefill_pass."""
    import torch
    import decode_token_rmsnorm_amd as wm

    gcache = wm.new_cache(model, w.B)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        wm.cyclic_prefill_pass(model, tok, w.g, gcache, 1, logits, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wm.cyclic_prefill_pass(model, tok, w.g, gcache, 1, logits, ws)
    gcache.k.zero_()
    gcache.v.zero_()
    gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(w.passes)]
    torch.cuda.synchronize()
    for a, b in gevs:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    out = [a.elapsed_time(b) for a, b in gevs]
    del graph, gcache
    return out


def bench_small_prefill():
    """The small half-cache model (L16 D512 8/4 x 64, F1536, k8, p2, V32768,
    B8, T2048, cyclic g16): three passes from the zero cache, each timed with
    events; the pass against the MFMA roofline of its algorithmic FLOP, and
    per-kind kernel times from one further pass."""
    import torch
    import decode_token_rmsnorm_amd as wm
    from decode_token_rmsnorm_amd import _lib as C
    from wm_inputs import WORKLOADS, make_tokens, make_weights

    w = WORKLOADS["small_prefill"]
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
    rows = wm.prefill_rows(w.B, w.T, w.g)
    ws = model.workspace(rows)
    logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
    # untimed: one pass on a scratch cache (first launches, code loading)
    scratch = wm.new_cache(model, w.B)
    wm.cyclic_prefill_pass(model, tok, w.g, scratch, 1, logits, ws)
    del scratch
    cache = wm.new_cache(model, w.B)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(w.passes)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        wm.cyclic_prefill_pass(model, tok, w.g, cache, 1, logits, ws)
        b.record()
    torch.cuda.synchronize()
    assert torch.isfinite(logits).all(), "non-finite logits"
    per_pass = [a.elapsed_time(b) for a, b in evs]
    profile((1 << len(C.KINDS)) - 1)
    wm.cyclic_prefill_pass(model, tok, w.g, cache, 1, logits, ws)
    torch.cuda.synchronize()
    kern = {k: {"launches": c, "avg_us": 1e3 * m / c, "per_pass_us": 1e3 * m} for k, (c, m) in profile_read().items()}
    profile(0)
    # the same three passes replayed from one captured graph of a pass
    g_per_pass = None if not GRAPHS else graph_passes(model, tok, w, logits, ws)
    flop = pass_flops(w)

    best = min(per_pass)
    ach = flop / (best * 1e-3) / 1e12
    del cache, ws, model
    torch.cuda.empty_cache()
    return {"workload": "small_prefill: L16 D512 Hq8 Hkv4 d64 F1536 k8 p2 V32768, B8 T2048, cyclic g16, 3 passes, "
                        "bf16",
            "per_pass_ms": per_pass, "value": w.B * w.T / (best * 1e-3), "unit": "tokens/s/pass",
            "graph_replay_per_pass_ms": g_per_pass,
            "rows_per_group_step": rows,
            "roofline": {"kernel": "whole pass (all launches of a cyclic pass)", "bound": "mfma", "achieved": ach,
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                         "traffic": None,
                         "algorithmic_per_launch": f"{flop:.4e} FLOP per pass (B*T*{flops_per_token(w, 'wm', lm_head=False):.4e})"},
            "kernels_per_pass_us": kern}


def bench_decode_1p3b(steps=20):
    """Decode at the 1.3B-scale shape (L28 D1792 14/2 x 128, F4864, B64,
    t = 2047 cached positions of seeded keys/values), WhiteMatter half cache
    (k = 14) against the vanilla model (k = L = 28) on the same kernels:
    tokens/s and peak device memory, beside the pages' 1.3B-scale batch-64
    decode figures."""
    import torch
    import decode_token_rmsnorm_amd as wm
    from wm_inputs import WORKLOADS, make_cache_device, make_tokens, make_weights

    out = {}
    t = 2047
    base = WORKLOADS["prefill_1p3b"]
    for name, w, step in (("whitematter", base, wm.decode_step), ("vanilla", base.replace(k=base.L),
                                                                   wm.vanilla_decode_step)):
        model = wm.Model(w, make_weights(w, seed=0), "bf16")
        peak_reset()
        K, V = make_cache_device(w, w.B, filled=t, seed=3)
        cache = wm.Cache(K, V)
        tok = torch.from_numpy(make_tokens(w, seed=1, B=w.B, T=1)[:, 0].copy()).cuda()
        ws = model.workspace(w.B)
        logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
        for _ in range(3):
            step(model, tok, t, cache, logits, ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step(model, tok, t, cache, logits, ws)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        out[name] = {"k": w.k, "value": w.B / wall, "unit": "tokens/s", "ms_per_step": 1e3 * wall,
                     "peak_memory_gib": peak_gib(), "cache_gib": 2 * K.numel() * K.element_size() / 2 ** 30}
        del model, K, V, cache, ws, logits, tok
        torch.cuda.empty_cache()
    out["workload"] = "prefill_1p3b shape decoding: L28 D1792 Hq14 Hkv2 d128 F4864 V32768, B64, t=2047 cached, bf16"
    out["peak_memory_wm_over_vanilla"] = out["whitematter"]["peak_memory_gib"] / out["vanilla"]["peak_memory_gib"]
    return out


def bench_mix(calls, warmup):
    """One wm_mix_kv over the whole state stack [16, 8*2048, 512] (bf16, k=8,
    4 KV heads x 64): pool + append of 16,384 tokens."""
    import torch
    import decode_token_rmsnorm_amd as wm
    from decode_token_rmsnorm_amd import _lib as C
    from wm_inputs import WORKLOADS, make_state_stack_device, make_weights

    w = WORKLOADS["mix_bf16"]
    rows = w.B * w.T
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    states = make_state_stack_device(w, rows, seed=2)
    cache = wm.new_cache(model, w.B)
    ws = model.workspace(rows)
    for _ in range(warmup):
        wm.mix_kv(model, states, w.B, w.T, 0, 1, cache, ws)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(calls):
        wm.mix_kv(model, states, w.B, w.T, 0, 1, cache, ws)
    b.record()
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / calls
    # per-kind kernel times over a few further calls
    profile(1 << C.KINDS.index("router") | 1 << C.KINDS.index("mix") | 1 << C.KINDS.index("kvproj"))
    for _ in range(5):
        wm.mix_kv(model, states, w.B, w.T, 0, 1, cache, ws)
    torch.cuda.synchronize()
    kern = {k: {"launches": c, "avg_us": 1e3 * m / c} for k, (c, m) in profile_read().items()}
    R = w.R
    per_tok = w.L * w.D * 2 + 2 * w.k * w.Hkv * w.d * 2
    wbytes = 2 * (w.L * w.k) * (R * w.D) * 2 + 2 * w.k * (w.Hkv * w.d) * w.D * 2
    nbytes = rows * per_tok + wbytes
    ach = nbytes / (us * 1e-6) / 1e9
    del states, cache, ws, model
    torch.cuda.empty_cache()
    return {"workload": "mix_bf16: state stack [L16, B8*T2048, D512] bf16, router over layers 0,2..14, k8, "
                        "K/V 512 -> 4 x 64, RoPE base 1e6, whole cache written",
            "us_per_call": us, "calls": calls, "kernels_avg_us": kern,
            "roofline": {"kernel": "wm_mix_kv (router + mix + K/V projection and append)", "bound": "hbm",
                         "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                         "traffic": profiled_traffic("mix_kv"),
                         "algorithmic_per_launch": f"{nbytes:.4e} B = {rows}*{per_tok} + {wbytes} weights"}}


def bench_vanilla(steps, decode_steps):
    """The vanilla comparison model (per-layer K/V, causal s <= i, k = L) on the
    same kernels: one prefill pass over the 1.3B-scale workload in steps of
    T/g = 128 positions (the rows per step of the cyclic pass), and decode
    steps on the decode shape (which already has k = L)."""
    import torch
    import decode_token_rmsnorm_amd as wm
    from wm_inputs import WORKLOADS, make_cache_device, make_tokens, make_weights

    out = {}
    w = WORKLOADS["prefill_1p3b"]
    w = w.replace(k=w.L)
    chunk = -(-w.T // w.g)
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    peak_reset()
    tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
    cache = wm.new_cache(model, w.B)
    ws = model.workspace(w.B * chunk)
    logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
    wm.vanilla_prefill(model, tok, chunk, cache, 1, logits, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wm.vanilla_prefill(model, tok, chunk, cache, 1, logits, ws)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    assert torch.isfinite(logits).all(), "non-finite logits"
    cache_bytes = 2 * cache.k.numel() * cache.k.element_size()
    out["prefill"] = {"workload": f"prefill_1p3b with per-layer K/V (k = L = {w.L}), B{w.B} T{w.T}, one causal pass "
                                  f"in steps of {chunk} positions, bf16",
                      "value": w.B * w.T / wall, "unit": "tokens/s", "ms_per_pass": 1e3 * wall, "passes": steps,
                      "cache_gib": cache_bytes / 2 ** 30, "peak_memory_gib": peak_gib()}
    del cache, ws, model, tok
    torch.cuda.empty_cache()

    w = WORKLOADS["decode_d512"]
    assert w.k == w.L
    t = 2047
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    peak_reset()
    K, V = make_cache_device(w, w.B, filled=t, seed=3)
    cache = wm.Cache(K, V)
    tok = torch.from_numpy(make_tokens(w, seed=1, B=w.B, T=1)[:, 0].copy()).cuda()
    ws = model.workspace(w.B)
    logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
    for _ in range(5):
        wm.vanilla_decode_step(model, tok, t, cache, logits, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(decode_steps):
        wm.vanilla_decode_step(model, tok, t, cache, logits, ws)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / decode_steps
    out["decode"] = {"workload": "decode_d512 with per-layer K/V (k = L = 16), B64, t=2047 cached, bf16",
                     "value": w.B / wall, "unit": "tokens/s", "ms_per_step": 1e3 * wall, "steps": decode_steps,
                     "peak_memory_gib": peak_gib(), "cache_gib": 2 * K.numel() * K.element_size() / 2 ** 30}
    del cache, ws, model, K, V
    torch.cuda.empty_cache()
    return out


def bench_variants(steps):
    """The analysis variants on the same kernels: the feedback-free model
    (k = L, channel l from states 0..l, one layer-synchronous pass) on the
    1.3B-scale prefill workload, and static mixing (constant weights, no
    router) in wm_mix_kv on the mix workload, beside the routed call."""
    import torch
    import decode_token_rmsnorm_amd as wm
    from wm_inputs import (WORKLOADS, make_state_stack_device, make_static_mix, make_tokens, make_weights)

    out = {}
    w = WORKLOADS["prefill_1p3b"]
    w = w.replace(k=w.L)
    chunk = -(-w.T // w.g)
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
    cache = wm.new_cache(model, w.B)
    ws = model.workspace(w.B * chunk)
    logits = torch.empty(w.B, w.V, dtype=torch.float32, device="cuda")
    wm.feedback_free_prefill(model, tok, chunk, cache, 1, logits, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wm.feedback_free_prefill(model, tok, chunk, cache, 1, logits, ws)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    assert torch.isfinite(logits).all(), "non-finite logits"
    out["feedback_free_prefill"] = {
        "workload": f"prefill_1p3b, feedback-free (k = L = {w.L}), B{w.B} T{w.T}, one layer-synchronous pass in "
                    f"steps of {chunk} positions, bf16",
        "value": w.B * w.T / wall, "unit": "tokens/s", "ms_per_pass": 1e3 * wall, "passes": steps}
    del cache, ws, model, tok
    torch.cuda.empty_cache()

    w = WORKLOADS["mix_bf16"]
    rows = w.B * w.T
    W = make_weights(w, seed=0)
    states = make_state_stack_device(w, rows, seed=2)
    res = {}
    for name, up in (("routed", {n: W[n] for n in ("src_norm", "router", "chan_norm", "wk", "wv", "k_norm")}),
                     ("static", {**{n: W[n] for n in ("src_norm", "chan_norm", "wk", "wv", "k_norm")},
                                 "static_mix": make_static_mix(w)})):
        model = wm.Model(w, up, "bf16")
        cache = wm.new_cache(model, w.B)
        ws = model.workspace(rows)
        for _ in range(3):
            wm.mix_kv(model, states, w.B, w.T, 0, 1, cache, ws)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(20):
            wm.mix_kv(model, states, w.B, w.T, 0, 1, cache, ws)
        b.record()
        torch.cuda.synchronize()
        res[name] = 1e3 * a.elapsed_time(b) / 20
        del model, cache, ws
    out["static_mixing_mix_kv"] = {"workload": "wm_mix_kv on the state stack [16, 8*2048, 512], k8, bf16",
                                   "us_per_call_routed": res["routed"], "us_per_call_static": res["static"]}
    del states
    torch.cuda.empty_cache()
    return out


def bench_sweep(tau=1e-4):
    """The schedule sweep: (a) per-pass time of the cyclic prefill against g on
    the small bf16 model (L16 D512 k8, B8 T2048), g in {1, 4, 8, 16, 32, T};
    (b) on the tiny fp32 model (L4 D128 k2, T128), the fixed-point residual
    after each pass (max-abs-relative distance of the cache from the same
    implementation's autoregressive cache, i.e. g = T) and n_tau, the first pass
    within tau, beside the closed form ceil(T/g) of strict causality."""
    import torch
    import decode_token_rmsnorm_amd as wm
    from wm_inputs import WORKLOADS, make_tokens, make_weights

    out = {"pass_time": [], "fixed_point": [], "tau": tau}
    w = WORKLOADS["small_prefill"]
    model = wm.Model(w, make_weights(w, seed=0), "bf16")
    tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
    for g in (1, 4, 8, 16, 32, w.T):
        cache = wm.new_cache(model, w.B)
        ws = model.workspace(wm.prefill_rows(w.B, w.T, g))
        wm.cyclic_prefill_pass(model, tok, g, cache, 0, None, ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        wm.cyclic_prefill_pass(model, tok, g, cache, 0, None, ws)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        out["pass_time"].append({"g": g, "ms_per_pass": 1e3 * dt, "tokens_per_s_per_pass": w.B * w.T / dt,
                                 "rows_per_step": wm.prefill_rows(w.B, w.T, g)})
        del cache, ws
    out["pass_time_workload"] = "small_prefill: L16 D512 Hq8 Hkv4 d64 F1536 k8 p2, B8 T2048, bf16"
    del model, tok
    torch.cuda.empty_cache()

    w = WORKLOADS["tiny_fp32"]
    model = wm.Model(w, make_weights(w, seed=0, gains="perturbed"), "f32")
    tok = torch.from_numpy(make_tokens(w, seed=1)).cuda()
    ar = wm.new_cache(model, w.B)
    wm.cyclic_prefill_pass(model, tok, w.T, ar)
    for g in (1, 4, 8, 16, 32, w.T):
        cache = wm.new_cache(model, w.B)
        closed = -(-w.T // g)
        res = []
        for n in range(closed + 1):
            wm.cyclic_prefill_pass(model, tok, g, cache)
            num = max(float((cache.k - ar.k).abs().max()), float((cache.v - ar.v).abs().max()))
            den = max(float(ar.k.abs().max()), float(ar.v.abs().max()))
            res.append(num / den)
        n_tau = next((i + 1 for i, r in enumerate(res) if r <= tau), None)
        out["fixed_point"].append({"g": g, "closed_form_passes": closed, "n_tau": n_tau,
                                   "residual_first_passes": res[:8], "residual_at_closed_form": res[closed - 1]})
    out["fixed_point_workload"] = "tiny_fp32: L4 D128 Hq4 Hkv4 d32 F384 k2 p2 V512, B1 T128, fp32"
    return out


def cpu_baseline(budget_s=10.0):
    """The float64 oracle on a bounded sample of the prefill workload: the last
    group step (q = 15: positions 15, 31, ..., 2047, whose attention spans on
    average as many keys as a whole pass's) of sequences 0, 1, ..., against a
    filled cache (seeded values at every position), one sequence at a time
    until about `budget_s` seconds of CPU work."""
    import numpy as np
    import oracle as O
    from wm_inputs import WORKLOADS, make_tokens, make_weights
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    from wm_inputs import make_cache
    w = WORKLOADS["prefill_1p3b"]
    M = O.Model(w, make_weights(w, seed=0))
    tokens = make_tokens(w, seed=1)
    q = w.g - 1
    bidx, pos = O.tokset_rows(1, len(O.group_positions(w.T, w.g, q)), q, w.g)
    K0, V0 = make_cache(w, 1, filled=w.T, seed=3)
    dt, nseq = 0.0, 0
    while dt < budget_s and nseq < w.B:
        cache = (K0.astype(np.float64), V0.astype(np.float64))
        t0 = time.perf_counter()
        O.step(M, tokens[nseq:nseq + 1], cache, bidx, pos, want_logits=False)
        dt += time.perf_counter() - t0
        nseq += 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:
        blas = "unknown"
    return {"value": nseq * len(pos) / dt, "unit": "tokens/s/pass", "cores": threads, "kind": "oracle",
            "sample": f"sequences 0..{nseq - 1}, group step q={q} ({len(pos)} positions each, up to {w.T - 1} "
                      f"keys) against a filled cache, float64 numpy, {dt:.1f}s",
            "cpu_model": cpu_model, "blas": blas}


def device_peaks():
    """Peaks measured on this GPU in this run: a streaming read and a copy of
    1 GiB (HIP kernels of the library, hipEvent-timed) and a register-resident
    bf16 MFMA loop on every compute unit."""
    import torch
    import decode_token_rmsnorm_amd as wm
    src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    out = {"hbm_read_gbs": wm.peak_stream(src, None, iters=10),
           "hbm_copy_gbs": wm.peak_stream(src, dst, iters=10),
           "bf16_mfma_tflops": wm.peak_mfma_bf16(iters=10),
           "what": "1 GiB streaming read and 1 GiB copy (GB/s, copy counts read + write); 32x32x16 bf16 MFMA loop "
                   "on register operands, 2 blocks of 4 waves per CU (TFLOP/s)"}
    del src, dst
    torch.cuda.empty_cache()
    return out


def with_measured(roof, peak):
    """The roofline object plus its fraction of the peak measured on this GPU."""
    if roof is not None and peak:
        roof["peak_measured"] = peak
        roof["frac_measured"] = roof["achieved"] / peak
    return roof


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-mix", action="store_true")
    ap.add_argument("--skip-vanilla", action="store_true")
    ap.add_argument("--skip-sweep", action="store_true")
    ap.add_argument("--skip-variants", action="store_true")
    ap.add_argument("--skip-small", action="store_true")
    ap.add_argument("--skip-decode-1p3b", action="store_true")
    ap.add_argument("--skip-train", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay legs (counter-collection runs)")
    ap.add_argument("--only", choices=["decode", "mix", "vanilla", "sweep", "variants", "peaks", "small",
                                       "decode_1p3b", "cpu", "train"], default=None,
                    help="profiling aid: run only this part and print its object")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer 3 times (reference for HBM byte counters)")
    a = ap.parse_args()
    if a.copy_calibration:
        import torch
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": 1 << 30, "copies": 3}))
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); the method's batch elements are independent "
              "and would shard as pure data parallelism over sequences; this benchmark runs one GPU.", file=sys.stderr)
        sys.exit(2)
    global GRAPHS, CPU_BASELINE
    GRAPHS = not a.no_graph
    CPU_BASELINE = not a.no_cpu_baseline
    import torch
    torch.cuda.set_device(0)
    if a.only:
        part = (bench_decode(a.decode_steps, 5) if a.only == "decode" else bench_mix(20, 3) if a.only == "mix"
                else device_peaks() if a.only == "peaks" else bench_small_prefill() if a.only == "small"
                else bench_decode_1p3b() if a.only == "decode_1p3b" else cpu_baseline() if a.only == "cpu"
                else bench_train() if a.only == "train"
                else bench_vanilla(a.steps, a.decode_steps) if a.only == "vanilla"
                else bench_variants(a.steps) if a.only == "variants" else bench_sweep())
        print(json.dumps({a.only: part}), flush=True)
        return
    w, pre = bench_prefill(a.steps, a.warmup)
    dec = None if a.skip_decode else bench_decode(a.decode_steps, 5)
    mix = None if a.skip_mix else bench_mix(20, 3)
    van = None if a.skip_vanilla else bench_vanilla(a.steps, a.decode_steps)
    sweep = None if a.skip_sweep else bench_sweep()
    variants = None if a.skip_variants else bench_variants(a.steps)
    small = None if a.skip_small else bench_small_prefill()
    dec13 = None if a.skip_decode_1p3b else bench_decode_1p3b()
    train = None if a.skip_train else bench_train()
    if van is not None:
        # the pages' comparison: WhiteMatter prefill as a share of vanilla's (one
        # vanilla pass against one, and against the workload's 3 passes:
        # 1 no-grad pass + 2), decode tokens/s against vanilla's
        wm_pass = w.B * w.T / (pre["wall_s"] / a.steps)
        van["wm_prefill_per_pass_over_vanilla"] = wm_pass / van["prefill"]["value"]
        van["wm_prefill_3_passes_over_vanilla"] = wm_pass / 3 / van["prefill"]["value"]
        van["prefill_peak_memory_gib"] = {"whitematter": pre["peak_memory_gib"],
                                          "vanilla": van["prefill"]["peak_memory_gib"]}
        if dec is not None:
            van["wm_decode_over_vanilla"] = dec["value"] / van["decode"]["value"]
    peaks = device_peaks()
    with_measured(pre["roofline"], peaks["bf16_mfma_tflops"])
    if dec is not None:
        with_measured(dec["roofline"], peaks["hbm_read_gbs"])
    if mix is not None:
        with_measured(mix["roofline"], peaks["hbm_copy_gbs"])
    cpu = None if a.no_cpu_baseline else cpu_baseline()
    value = w.B * w.T / (pre["wall_s"] / a.steps)
    line = {
        "metric": "cyclic-prefill tokens/s per pass + decode tok/s (1 GPU); % HBM/MFMA peak",
        "value": value, "unit": "tokens/s/pass", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": 1e3 * pre["wall_s"] / a.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) weights, Zipf(1.1) tokens)",
        "config": {"workload": "prefill_1p3b: L28 D1792 Hq14 Hkv2 d128 F4864 k14 p2 V32768, B64 T2048, cyclic g16",
                   "global_batch": w.B, "seq_len": w.T, "groups": w.g, "parallelism": "single GPU"},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu,
        "per_pass_ms": pre["per_pass_ms"],
        "pass_tflops": pre["pass_tflops"],
        "pass_mfma_frac": pre["pass_tflops"] / BF16_PEAK_TFLOPS,
        "pass_mfma_frac_measured": pre["pass_tflops"] / peaks["bf16_mfma_tflops"],
        "device_peaks": peaks,
        "kernels_avg_us": pre["kernels"],
        "peak_memory_gib": pre["peak_memory_gib"],
        "decode": dec,
        "mix_kv": mix,
        "small_prefill": small,
        "decode_1p3b": dec13,
        "train_step": train,
        "vanilla": van,
        "schedule_sweep": sweep,
        "variants": variants,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
