"""Oracle for the WhiteMatter KV-pool path — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 CPU implementation of what the hot path computes,
written from the published summaries of WhiteMatter (arXiv 2608.18486):
the paperlayer.ai summary (§3 Method) and the onedev.kr summary (sections
"How it works" / "What differs").  It shares no code with the HIP library
and never imports it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here; the
product path must never route through it.

Modules
-------
``wm_oracle``  vectorised float64 definition (per group step, numpy matmul).
``brute``      a separately written scalar-loop implementation of exact
               autoregressive execution, for tiny shapes only; it pins
               ``wm_oracle`` by brute force.
``wm_train``   the training step with truncated backpropagation: the
               objective from ``wm_oracle`` passes (for finite differences)
               and the same forward in torch float64 for autograd (import it
               as ``oracle.wm_train``; it needs torch).
"""
from .wm_oracle import *  # noqa: F401,F403
