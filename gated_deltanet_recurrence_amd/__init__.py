"""MI355X (gfx950) Gated Delta Rule token mixer.

The compute lives in libgdn.so (HIP kernels behind the C ABI declared in
include/gdn.h); this package holds its ctypes binding, the build script and
the seeded synthetic input recipes. Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from ._binding import (GDNError, gdn_decode_mixer_step, gdn_decode_step,  # noqa: F401
                       gdn_decode_step_channel_gated, gdn_prefill_channel_gated,
                       gdn_prefill_channel_workspace_size,
                       gdn_prefill_seqpar, gdn_prefill_seqpar_workspace_size,
                       gdn_mixer_epilogue,
                       gdn_mixer_prologue, gdn_prefill, gdn_prefill_noalloc, gdn_prefill_recurrent,
                       gdn_prefill_apply, gdn_prefill_prepare, gdn_prefill_workspace_size,
                       load)

__all__ = ["GDNError", "gdn_prefill", "gdn_prefill_noalloc", "gdn_prefill_workspace_size", "gdn_prefill_prepare",
           "gdn_prefill_apply", "gdn_prefill_recurrent", "gdn_decode_step",
           "gdn_decode_mixer_step", "gdn_prefill_channel_gated",
           "gdn_prefill_channel_workspace_size",
           "gdn_decode_step_channel_gated", "gdn_prefill_seqpar",
           "gdn_prefill_seqpar_workspace_size",
           "gdn_mixer_prologue", "gdn_mixer_epilogue", "load"]
