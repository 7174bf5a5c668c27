"""MI355X-native Medusa verify step: HIP kernels behind a C ABI (libmedusa.so).

Submodules
  _lib   ctypes declarations and error handling (no computation)
  api    the verify-step calls by name: medusa_heads_topk, tree_build_candidates,
         tree_attention, evaluate_posterior, kv_compact, plus decoder helpers
  model  model/state wrappers around medusa_forward, medusa_prefill, medusa_step
  build  compiles csrc/*.hip for gfx950 into libmedusa.so
"""
from ._lib import GREEDY, TYPICAL, MedusaError, lib  # noqa: F401
