"""io_aware_attention_amd: the fused, tiled attention forward pass for MI355X (gfx950).

The product is the C-ABI library ``libflashfwd.so`` (include/flashfwd.h) built from the
HIP sources in ``csrc/``; ``flashfwd`` is its thin ctypes binding.
"""
from . import flashfwd  # noqa: F401
from .flashfwd import (FlashFwdError, attn_fwd, attn_fwd_splitkv, attn_splitkv_combine,  # noqa: F401
                       attn_splitkv_num_splits, attn_splits_efficiency_rule, attn_status_string,
                       forward, forward_splitkv)
