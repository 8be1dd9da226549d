"""WhiteMatter cross-layer KV pool on MI355X (gfx950): HIP kernels behind the
C ABI of include/wm.h, with a thin torch/ctypes binding."""
from . import _lib  # noqa: F401
from .api import (Cache, Model, cache_from_host, channel_attn, cyclic_prefill_pass, decode_step,  # noqa: F401
                  decode_step_at, decode_step_static,
                  feedback_free_decode_step, feedback_free_prefill, mix_kv, new_cache, peak_mfma_bf16, peak_stream,
                  prefill_rows, train_step, train_workspace, vanilla_decode_step, vanilla_prefill)
