"""libgdn: the gated delta rule on MI355X (gfx950), hand-written HIP behind a C ABI.

The Python functions ``gdn_chunk_fwd`` (with ``gdn_chunk_fwd_noalloc``, its variant on
the library's static scratch, and ``gdn_chunk_fwd_gated``, which adds the mixer's output
norm), ``gdn_recurrent_step``, ``gdn_states_fwd`` and the mixer steps around them (``gdn_mixer_prologue``, ``gdn_gated_norm``,
``gdn_recurrent_step_gated``) are a thin ctypes binding over the C entry points of the same
names (include/gdn.h): they check tensors, marshal pointers and the caller's stream, and
launch nothing themselves.  The
library is loaded on first use and its absence raises; there is no CPU fallback.
"""
from .synth import WORKLOADS, Workload, make_decode_pool, make_inputs  # noqa: F401

__all__ = ["WORKLOADS", "Workload", "make_inputs", "make_decode_pool",
           "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_gated", "gdn_recurrent_step", "gdn_states_fwd", "gdn_gated_norm",
           "gdn_recurrent_step_gated", "gdn_mixer_prologue", "library_path"]


def __getattr__(name):
    if name in ("gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_gated", "gdn_recurrent_step", "gdn_states_fwd", "gdn_chunk_fwd_workspace",
                "gdn_states_fwd_workspace", "gdn_gated_norm", "gdn_recurrent_step_gated",
                "gdn_mixer_prologue", "library_path", "load_library", "GdnError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
