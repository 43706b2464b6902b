"""MI355X (gfx950) exact attention: FlashAttention-style forward, backward and
split-KV decode in hand-written HIP kernels behind a C ABI (include/fa.h).

Python names mirror the C entry points (``fa_fwd``, ``fa_bwd``,
``fa_bwd_stage``, ``fa_fwd_workspace_size``, ``fa_bwd_workspace_size``,
``fa_fwd_paged``, ``fa_fwd_paged_workspace_size``, ``fa_fwd_dropout``,
``fa_bwd_dropout``, ``fa_dropout_mask``, ``fa_fwd_fp8``, ``fa_bwd_noalloc``,
``fa_strerror``, ``fa_version``);
``forward``, ``backward``, ``forward_paged``, ``forward_dropout``,
``backward_dropout``, ``dropout_mask`` and ``forward_fp8`` allocate the
outputs and the workspace and raise on error.
"""

from ._lib import (  # noqa: F401
    FA_BF16,
    FA_F16,
    FA_F32,
    FA_OK,
    FAError,
    LIB_PATH,
    backward,
    backward_dropout,
    fa_bwd,
    fa_bwd_dropout,
    fa_bwd_noalloc,
    fa_bwd_stage,
    fa_bwd_workspace_size,
    fa_dropout_mask,
    fa_fwd,
    fa_fwd_dropout,
    fa_fwd_fp8,
    fa_fwd_paged,
    fa_fwd_paged_workspace_size,
    fa_fwd_workspace_size,
    fa_strerror,
    fa_version,
    dropout_mask,
    forward,
    forward_dropout,
    forward_fp8,
    forward_paged,
    load,
)
