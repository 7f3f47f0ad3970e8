"""Gated DeltaNet verify / commit / rewind / conv-step / chunked-prefill path
for AMD Instinct MI355X (gfx950), behind the C ABI of libgdn.so.

The API names (gdn_verify, gdn_commit, gdn_rewind, gdn_conv_step,
gdn_prefill_chunked, gdn_workspace_size, make_dims, ...) resolve lazily to
the ctypes binding in ``binding``, which raises ImportError when libgdn.so
is not built.  ``workloads`` (seeded synthetic inputs) and ``build`` import
without the library.
"""
from __future__ import annotations

__all__ = ["gdn_conv_step", "gdn_verify", "gdn_commit", "gdn_rewind", "gdn_prefill_chunked",
           "gdn_workspace_size", "gdn_status_string", "gdn_version", "make_dims", "gdn_dims",
           "GdnError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
