"""MI355X-native Prefill-On-Decode paged-KV attention.

The compute path is the HIP library ``libpod_attn.so`` (built in-tree from
``csrc/``); this package only marshals arguments to its C ABI.
"""
from .pod import BatchPOD, single_decode_with_kv_cache, kv_views, merge_states, run_static  # noqa: F401
from . import _lib  # noqa: F401

__all__ = ["BatchPOD", "single_decode_with_kv_cache", "kv_views", "merge_states", "run_static"]
