"""draft_block_verification_sv_amd: batched verification of a one-pass diffusion
draft block with the fused entry-wise clipped reverse-KL, as hand-written HIP
kernels for AMD Instinct MI355X (gfx950) behind the C ABI of libspecverify.

The Python layer only marshals tensors into the C ABI; see ``binding``.
"""

from .binding import (  # noqa: F401
    SV_BF16,
    SV_F32,
    SpecVerifyError,
    alloc_workspace,
    branch_lookup,
    clipped_rkl,
    lib,
    length_head,
    length_loss,
    library_path,
    opd_loss,
    opd_loss_grad,
    profile_enable,
    profile_read,
    profile_reset,
    read_probe,
    verify_block,
    verify_block_greedy,
    verify_block_noalloc,
    verify_tree_greedy,
    version,
    workspace_size,
)
