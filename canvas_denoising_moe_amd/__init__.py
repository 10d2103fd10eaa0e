"""MI355X (gfx950) canvas-denoising library: Python binding of ``include/dg.h``.

The hot path -- a DiffusionGemma-style denoise pass over a canvas of
placeholder tokens (bidirectional canvas attention plus attention into a
cached prompt KV, a top-k routed MoE with a shared expert, a tied LM head,
per-position argmax / confidence and the lock-and-remask step) -- runs
entirely in the HIP kernels of ``_lib/libdg.so``.  This package only
marshals torch tensors (device memory, streams) into the C ABI.
"""
from .binding import (  # noqa: F401
    DG_BF16, DG_EHIP, DG_EINVAL, DG_ENOMEM, DG_ESTATE, DG_EUNSUPPORTED, DG_F32, DG_OK, LIB_PATH,
    Context, DGError, exported_symbols, k_argmax_conf, k_eb_noise, k_eb_rows, k_eb_select, k_lock_select,
    k_moe_route, lib, make_config,
)
