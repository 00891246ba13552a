"""The step before the context write, PyTorch-facing: the Gemma hidden norm of
the context states, and precompute_and_store_context_kv as the vLLM API page
"vllm.models.minimax_m3.common.dspark" (MiniMaxM3DSparkModel) composes it:
hidden norm, then the token-major K/V projection with the fused context write
(run in one kernel here, so all_kv is never stored).  Every step runs in the
HIP library; this module checks tensors, allocates the hidden-norm output
with torch when none is given, and passes pointers."""
from __future__ import annotations

import torch

from . import _lib
from .writer import DSparkContextKVWriter, PackedKVWeight


def hidden_norm(x: torch.Tensor, weight: torch.Tensor, eps: float,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """Gemma RMSNorm of each row of x (bf16 [rows, dim], dim % 8 == 0):
    x * rsqrt(mean(x^2) + eps) * (1 + weight), in fp32, rounded to bf16."""
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [rows, dim] tensor")
    rows, dim = x.shape
    if weight.dtype != torch.bfloat16 or tuple(weight.shape) != (dim,) or \
            weight.device != x.device or not weight.is_contiguous():
        raise ValueError(f"weight must be a contiguous bf16 ({dim},) tensor on {x.device}")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or \
            not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like x")
    st = _lib.dspark_hidden_norm(x.data_ptr(), rows, dim, weight.data_ptr(), float(eps),
                                 out.data_ptr(), torch.cuda.current_stream(x.device).cuda_stream)
    if st != _lib.OK:
        raise RuntimeError("hidden norm failed: " + _lib.dspark_ctx_kv_last_error())
    return out


def pack_kv_weight(kv_weight: torch.Tensor) -> PackedKVWeight:
    """The projection weight (bf16 [cols, hidden], cols % 32 == 0,
    hidden % 16 == 0) in the fragment-major layout the packed projection
    kernel loads straight into registers; a permutation, done once per
    weight."""
    if kv_weight.dim() != 2 or kv_weight.dtype != torch.bfloat16 or \
            not kv_weight.is_contiguous() or not kv_weight.is_cuda:
        raise ValueError("kv_weight must be a contiguous bf16 [cols, hidden] device tensor")
    cols, hidden = kv_weight.shape
    out = torch.empty(cols * hidden, dtype=torch.bfloat16, device=kv_weight.device)
    st = _lib.dspark_kv_weight_pack(kv_weight.data_ptr(), cols, hidden, out.data_ptr(),
                                    torch.cuda.current_stream(kv_weight.device).cuda_stream)
    if st != _lib.OK:
        raise RuntimeError("packing the K/V weight failed: " + _lib.dspark_ctx_kv_last_error())
    return PackedKVWeight(out, cols, hidden)


def precompute_and_store_context_kv(writer: DSparkContextKVWriter, context_states: torch.Tensor,
                                    hidden_norm_weight: torch.Tensor, eps: float,
                                    kv_weight: "torch.Tensor | PackedKVWeight",
                                    k_norm_weight: torch.Tensor,
                                    positions: torch.Tensor, cos_sin_cache: torch.Tensor,
                                    rotary_dim: int, slot_mapping: torch.Tensor,
                                    workspace: torch.Tensor | None = None,
                                    all_kv_out: torch.Tensor | None = None) -> None:
    """hidden_norm(context_states) into `workspace` (allocated when None),
    then the projection with every draft layer's context write fused in
    (kv_weight row-major, or packed by pack_kv_weight); all_kv_out, if given,
    also receives the projection's bf16 output [num_ctx, L, 2, nkv, 128]."""
    z = hidden_norm(context_states, hidden_norm_weight, eps, out=workspace)
    writer.project_write(z, kv_weight, k_norm_weight, eps, positions, cos_sin_cache, rotary_dim,
                         slot_mapping, all_kv_out=all_kv_out)
