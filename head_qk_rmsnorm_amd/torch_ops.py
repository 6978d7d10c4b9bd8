"""torch custom-op registration of the fused op and its LayerNorm sibling.

The page "SGLang Diffusion fused operator fused_inplace_qknorm_rope: in-depth
technical analysis" (section 5.3) registers the op as a torch custom op that
declares q and k as mutated, so that torch.compile keeps the in-place update
in the graph instead of reusing stale tensors; section 5.2 gives the
capability query under the name ``can_use_fused_inplace_qknorm_rope``, marked
as a compile-time constant. This module does the same for the HIP library:

* ``torch.ops.qknr.fused_inplace_qknorm_rope(q, k, q_weight, k_weight,
  cos_sin_cache, positions, *, is_neox, eps=1e-6, head_dim=0, rope_dim=0)``
* ``torch.ops.qknr.fused_inplace_qk_layernorm_rope(q, k, q_weight, k_weight,
  q_bias, k_bias, cos_sin_cache, positions, *, is_neox=False, eps=1e-6,
  rope_dim=0)``
* ``can_use_fused_inplace_qknorm_rope(head_dim, rope_dim, is_neox, dtype)``

Every op body calls the ctypes binding (argument marshalling only); the fake
implementations return nothing, as the ops only mutate their inputs.
"""
from typing import Optional

import torch

from . import binding as B

_DTYPES = (torch.bfloat16, torch.float16)


@torch.library.custom_op("qknr::fused_inplace_qknorm_rope", mutates_args=("q", "k"))
def fused_inplace_qknorm_rope(q: torch.Tensor, k: torch.Tensor, q_weight: torch.Tensor,
                              k_weight: torch.Tensor, cos_sin_cache: torch.Tensor,
                              positions: torch.Tensor, *, is_neox: bool, eps: float = 1e-6,
                              head_dim: int = 0, rope_dim: int = 0) -> None:
    B.qknr_inplace(q, k, q_weight, k_weight, cos_sin_cache, positions, is_neox=is_neox,
                   eps=eps, head_dim=head_dim, rope_dim=rope_dim)


@fused_inplace_qknorm_rope.register_fake
def _fused_inplace_qknorm_rope_fake(q, k, q_weight, k_weight, cos_sin_cache, positions, *,
                                    is_neox, eps=1e-6, head_dim=0, rope_dim=0):
    return None


@torch.library.custom_op("qknr::fused_inplace_qk_layernorm_rope", mutates_args=("q", "k"))
def fused_inplace_qk_layernorm_rope(q: torch.Tensor, k: torch.Tensor, q_weight: torch.Tensor,
                                    k_weight: torch.Tensor, q_bias: Optional[torch.Tensor],
                                    k_bias: Optional[torch.Tensor],
                                    cos_sin_cache: Optional[torch.Tensor],
                                    positions: Optional[torch.Tensor], *, is_neox: bool = False,
                                    eps: float = 1e-6, rope_dim: int = 0) -> None:
    B.qknr_layernorm_rope_inplace(q, k, q_weight, k_weight, q_bias, k_bias, cos_sin_cache,
                                  positions, is_neox=is_neox, eps=eps, rope_dim=rope_dim)


@fused_inplace_qk_layernorm_rope.register_fake
def _fused_inplace_qk_layernorm_rope_fake(q, k, q_weight, k_weight, q_bias, k_bias,
                                          cos_sin_cache, positions, *, is_neox=False, eps=1e-6,
                                          rope_dim=0):
    return None


@torch.compiler.assume_constant_result
def can_use_fused_inplace_qknorm_rope(head_dim: int, rope_dim: int, is_neox: bool,
                                      dtype: torch.dtype) -> bool:
    """True if the library takes (head_dim, rope_dim, is_neox) in this I/O dtype
    (a superset of the page's rule; see include/qknr.h)."""
    if dtype not in _DTYPES:
        return False
    return B.qknr_can_use(head_dim, rope_dim, is_neox, dtype)
