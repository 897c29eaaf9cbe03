"""vocab_sharded_softmax_amd: per-token divergences over a sharded vocabulary on MI355X.

The compute path is libvjsd.so (hand-written HIP kernels for gfx950, C ABI in
``include/vjsd.h``).  ``_abi`` binds every entry point under its C name;
``functional`` wraps them as autograd ops.  Importing the package fails if the
library has not been built.
"""
from ._abi import (ShardSet, VjsdArgumentError, VjsdError, loss_opts, new_part, vjsd_bwd,
                   vjsd_bwd_noalloc, vjsd_forward_backward, vjsd_loss_forward_backward,
                   vjsd_forward, vjsd_fwd, vjsd_loss_backward, vjsd_loss_forward,
                   vjsd_membw_probe, vjsd_merge, vjsd_stats, vjsd_strerror, vjsd_workspace_bytes,
                   ventropy_bwd, ventropy_fwd, vkl_bwd, vkl_fwd, vlogprobs_bwd, vlogprobs_fwd,
                   vtopk_kl_bwd, vtopk_kl_fwd, vce_bwd, vce_fwd, lin_head, lin_operand,
                   vlin_gemm, vlin_scale, vljsd, vljsd_workspace_bytes)
from ._abi import LIB_PATH
from .functional import (cross_entropy, entropy, jsd, jsd_loss, kl_div, linear_jsd, logprobs,
                         topk_kl)

__all__ = [
    "jsd", "jsd_loss", "kl_div", "entropy", "logprobs", "topk_kl", "cross_entropy", "linear_jsd",
    "vlin_gemm", "vljsd", "vljsd_workspace_bytes", "vlin_scale", "lin_operand", "lin_head",
    "vtopk_kl_fwd", "vtopk_kl_bwd", "vce_fwd", "vce_bwd", "ShardSet", "VjsdError", "VjsdArgumentError",
    "vjsd_stats", "vjsd_merge", "vjsd_fwd", "vjsd_forward", "vjsd_bwd", "vjsd_bwd_noalloc",
    "vkl_fwd", "vkl_bwd", "ventropy_fwd",
    "ventropy_bwd", "vlogprobs_fwd", "vlogprobs_bwd", "vjsd_strerror", "vjsd_workspace_bytes",
    "vjsd_membw_probe", "vjsd_loss_forward", "vjsd_loss_backward", "loss_opts", "new_part",
    "vjsd_forward_backward", "vjsd_loss_forward_backward",
    "LIB_PATH",
]
