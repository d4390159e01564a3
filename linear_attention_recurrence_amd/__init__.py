"""Gated DeltaNet token mixer for AMD Instinct MI355X (gfx950).

The computation lives in libgdn.so (HIP kernels behind the C ABI of include/gdn.h); this
package is its thin Python binding. The library is loaded on first use and an exception is
raised if it has not been built (see ``linear_attention_recurrence_amd.build``).
"""

from ._lib import (GDN_BF16, GDN_F32, GdnError, gdn_channel_decay_decode_step,
                   gdn_channel_decay_prefill, gdn_chunk_prefill, gdn_chunk_prefill_noalloc,
                   gdn_chunk_prefill_conv, gdn_chunk_prefill_conv_workspace_bytes,
                   gdn_chunk_prefill_workspace_bytes, gdn_conv_decode_step, gdn_conv_prep,
                   gdn_conv_window_from_prefill, gdn_decode_step, gdn_decode_step_with_conv,
                   gdn_gated_rmsnorm,
                   gdn_status_string, gdn_verify_step, load)

__all__ = ["GDN_BF16", "GDN_F32", "GdnError", "gdn_channel_decay_decode_step",
           "gdn_channel_decay_prefill", "gdn_chunk_prefill", "gdn_chunk_prefill_noalloc",
           "gdn_chunk_prefill_conv", "gdn_chunk_prefill_conv_workspace_bytes",
           "gdn_chunk_prefill_workspace_bytes", "gdn_conv_decode_step", "gdn_conv_prep",
           "gdn_conv_window_from_prefill", "gdn_decode_step", "gdn_decode_step_with_conv",
           "gdn_gated_rmsnorm",
           "gdn_status_string", "gdn_verify_step", "load"]
