"""MI355X (gfx950) block-diffusion drafting hot path.

``libdflash.so`` (HIP kernels behind the C ABI of ``include/dflash.h``) does all
the work; ``_abi`` is its ctypes binding (same entry-point names) and
``Drafter`` owns the caller-side buffers of one context.  Build the library
with ``python -m block_diffusion_drafting_ctx_amd.build``; using the binding
without it raises ImportError.
"""

from . import _abi  # noqa: F401
from ._abi import (Config, DFlashError, dflash_check, dflash_clear_errors, dflash_create,  # noqa: F401
                   dflash_draft_block, dflash_fuse_ctx, dflash_kv_layer_bytes, dflash_stage_time,
                   dflash_stage_timing, dflash_stats, dflash_verify, dflash_verify_sample, dflash_verify_static,
                   dflash_version, dflash_workspace_bytes, make_config)
from .drafter import Drafter, kv8_buffer, kv8_scales_view  # noqa: F401
