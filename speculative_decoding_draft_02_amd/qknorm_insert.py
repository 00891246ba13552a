"""PyTorch-facing entry of the draft block's fused QK-norm / RoPE / KV insert.

``fused_qknorm_rope_kv_insert`` takes the arguments with which the vLLM API
page "vllm.models.minimax_m3.common.dspark" calls
ops.fused_minimax_m3_qknorm_rope_kv_insert; ``dspark_qknorm_rope_kv_insert``
mirrors the custom op on that page, with the attention layer and its slot
mapping passed in (there is no attention context here).  Every step runs in
the HIP library; this module checks tensors and passes pointers.
"""
from __future__ import annotations

import torch

from . import _lib

HEAD_DIM = _lib.HEAD_DIM


def _check(name, t, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def fused_qknorm_rope_kv_insert(qkv: torch.Tensor, q_norm_weight: torch.Tensor,
                                k_norm_weight: torch.Tensor, cos_sin_cache: torch.Tensor,
                                positions: torch.Tensor, num_heads: int, num_kv_heads: int,
                                rotary_dim: int, eps: float, *, slot_mapping=None, kv_cache=None,
                                block_size: int = 0, kv_cache_dtype: str = "auto",
                                q_fp8_out=None, q_fp8_scale: float = 1.0, k_scale=None,
                                v_scale=None) -> None:
    """Normalise and rotate qkv's query and key heads in place; with a slot
    mapping, also store the key and value heads into kv_cache; with
    q_fp8_out, also write the rotated queries as e4m3 of q / q_fp8_scale.

    qkv: bf16 [T, (num_heads + 2 num_kv_heads) * 128]; the norm weights bf16
    [128]; cos_sin_cache bf16 [rows, rotary_dim]; positions int64 [T];
    slot_mapping int64 [T] or None; kv_cache [num_blocks, num_kv_heads,
    block_size, 256] bf16 ("auto") or uint8 ("fp8"); q_fp8_out uint8 or
    float8_e4m3fn [T, num_heads * 128]; k_scale / v_scale optional fp32
    one-element device tensors for an fp8 cache (1.0 when not given)."""
    dev = qkv.device
    H, nkv, R = int(num_heads), int(num_kv_heads), int(rotary_dim)
    if qkv.dim() != 2:
        raise ValueError("qkv must be [num_tokens, (num_heads + 2 num_kv_heads) * 128]")
    T = qkv.shape[0]
    _check("qkv", qkv, torch.bfloat16, dev, (T, (H + 2 * nkv) * HEAD_DIM))
    _check("q_norm_weight", q_norm_weight, torch.bfloat16, dev, (HEAD_DIM,))
    _check("k_norm_weight", k_norm_weight, torch.bfloat16, dev, (HEAD_DIM,))
    _check("positions", positions, torch.int64, dev, (T,))
    if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != R:
        raise ValueError(f"cos_sin_cache has shape {tuple(cos_sin_cache.shape)}, "
                         f"expected (rows, {R})")
    _check("cos_sin_cache", cos_sin_cache, torch.bfloat16, dev)
    slots_ptr = cache_ptr = ks_ptr = vs_ptr = None
    nb = bs = 0
    dtype_code = _lib.KV_AUTO
    if slot_mapping is not None:
        _check("slot_mapping", slot_mapping, torch.int64, dev, (T,))
        if kv_cache is None or kv_cache.dim() != 4 or kv_cache.shape[1] != nkv \
                or kv_cache.shape[3] != 2 * HEAD_DIM:
            raise ValueError("kv_cache must be [num_blocks, num_kv_heads, block_size, 256]")
        if kv_cache_dtype in ("fp8", "fp8_e4m3"):
            _check("kv_cache", kv_cache, torch.uint8, dev)
            dtype_code = _lib.KV_FP8_E4M3
        elif kv_cache_dtype == "auto":
            _check("kv_cache", kv_cache, torch.bfloat16, dev)
        else:
            raise ValueError(f"kv_cache_dtype {kv_cache_dtype!r}")
        nb, bs = kv_cache.shape[0], kv_cache.shape[2]
        if block_size and int(block_size) != bs:
            raise ValueError(f"block_size {block_size} != kv_cache.size(2) = {bs}")
        for name, s in (("k_scale", k_scale), ("v_scale", v_scale)):
            if s is not None:
                _check(name, s, torch.float32, dev)
                if s.numel() != 1:
                    raise ValueError(f"{name} must hold one value")
        slots_ptr, cache_ptr = slot_mapping.data_ptr(), kv_cache.data_ptr()
        ks_ptr = k_scale.data_ptr() if k_scale is not None else None
        vs_ptr = v_scale.data_ptr() if v_scale is not None else None
    qf_ptr = None
    if q_fp8_out is not None:
        qf = q_fp8_out.view(torch.uint8) if q_fp8_out.dtype == torch.float8_e4m3fn else q_fp8_out
        _check("q_fp8_out", qf, torch.uint8, dev, (T, H * HEAD_DIM))
        qf_ptr = qf.data_ptr()
    if T == 0:
        return
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = _lib.dspark_qknorm_rope_kv_insert(
        qkv.data_ptr(), T, q_norm_weight.data_ptr(), k_norm_weight.data_ptr(),
        cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], positions.data_ptr(), H, nkv, R,
        float(eps), slots_ptr, cache_ptr, nb, bs, dtype_code, ks_ptr, vs_ptr, qf_ptr,
        float(q_fp8_scale), stream)
    if st != _lib.OK:
        raise RuntimeError("DSpark QK-norm/RoPE insert failed: " + _lib.dspark_ctx_kv_last_error())


def dspark_qknorm_rope_kv_insert(qkv, q_norm_weight, k_norm_weight, cos_sin_cache, positions,
                                 num_heads, num_kv_heads, rotary_dim, eps, q_fp8_out, layer,
                                 slot_mapping) -> None:
    """The custom op's logic with the attention context made explicit:
    ``layer`` carries ``kv_cache`` and ``_q_scale_float``; the insert happens
    when ``slot_mapping`` is not None, with block_size = kv_cache.size(2) and
    an fp8 cache when its storage is uint8.  As in the page's call, no k/v
    scale is passed, so an fp8 insert stores e4m3 of the values themselves."""
    insert = slot_mapping is not None
    kv_cache = layer.kv_cache if insert else None
    fp8 = insert and kv_cache.dtype == torch.uint8
    fused_qknorm_rope_kv_insert(
        qkv, q_norm_weight, k_norm_weight, cos_sin_cache, positions, num_heads, num_kv_heads,
        rotary_dim, eps, slot_mapping=slot_mapping, kv_cache=kv_cache,
        block_size=kv_cache.size(2) if insert else 0, kv_cache_dtype="fp8" if fp8 else "auto",
        q_fp8_out=q_fp8_out, q_fp8_scale=float(getattr(layer, "_q_scale_float", 1.0)))
