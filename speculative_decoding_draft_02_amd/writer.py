"""PyTorch-facing writer for the DSpark fused context-KV write.

Mirrors class DSparkContextKVWriter and rotary_dims_supported on the vLLM API
page "vllm.models.minimax_m3.common.ops.dspark_context_kv": built from the
draft's attention layers (objects carrying ``kv_cache``, ``_k_scale``,
``_v_scale`` and ``kv_cache_dtype``), validated with the same reasons, with
the per-layer offset tables keyed by the layers' data pointers and rebuilt
(outside graph capture only) when a cache is re-bound.  Every step of the
write runs in the HIP library; this module only checks tensors and passes
pointers.  PyTorch supplies device memory and the current stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib

HEAD_DIM = _lib.HEAD_DIM
SUPPORTED_KV_DTYPES = ("auto", "fp8", "fp8_e4m3")


def rotary_dims_supported(rotary_dim: int, head_dim: int) -> bool:
    """The write rotates the leading 16, 32 or 64 dims of a 128-dim head."""
    return bool(_lib.dspark_rotary_dims_supported(int(rotary_dim), int(head_dim)))


def _split_slot_mapping(slot_mapping, num_layers):
    """(shared tensor, None) or (None, list of per-layer tensors)."""
    if isinstance(slot_mapping, torch.Tensor):
        if slot_mapping.dim() == 1:
            return slot_mapping, None
        if slot_mapping.dim() == 2 and slot_mapping.shape[0] == num_layers:
            return None, [slot_mapping[l] for l in range(num_layers)]
        raise ValueError("slot_mapping must be [num_ctx] or [num_layers, num_ctx]")
    maps = list(slot_mapping)
    if len(maps) != num_layers or any(m is None for m in maps):
        raise ValueError(f"expected {num_layers} per-layer slot mappings, none of them None")
    first = maps[0]
    if all(m.data_ptr() == first.data_ptr() for m in maps):
        return first, None
    return None, maps


def check_write_preconditions(positions: torch.Tensor, slot_mapping, cos_sin_rows: int,
                              num_blocks: int, block_size: int) -> None:
    """The write's preconditions that the kernel does not check (as on the
    vLLM API page "vllm.models.minimax_m3.common.ops.dspark_context_kv"):
    every non-padding token's position indexes the cos/sin table, every
    slot is inside the cache, and no two non-padding tokens of a layer share
    a slot.  Raises ValueError naming the first violation.  Costs a host
    sync: meant for debugging (DSparkContextKVWriter(debug_checks=True))."""
    maps = [slot_mapping] if isinstance(slot_mapping, torch.Tensor) and slot_mapping.dim() == 1 \
        else list(slot_mapping)
    capacity = int(num_blocks) * int(block_size)
    for l, slots in enumerate(maps):
        valid = slots >= 0
        pos = positions[valid]
        if pos.numel() and (bool((pos < 0).any()) or bool((pos >= cos_sin_rows).any())):
            raise ValueError(f"a position is outside the cos/sin table of {cos_sin_rows} rows "
                             f"(slot mapping {l})")
        s = slots[valid]
        if s.numel() and bool((s >= capacity).any()):
            raise ValueError(f"a slot is >= num_blocks * block_size = {capacity} "
                             f"(slot mapping {l})")
        if s.numel() != torch.unique(s).numel():
            raise ValueError(f"two tokens share a slot (slot mapping {l})")


@dataclass
class AttnLayer:
    """The attributes of a draft attention layer that the writer reads."""
    kv_cache: torch.Tensor
    _k_scale: torch.Tensor
    _v_scale: torch.Tensor
    kv_cache_dtype: str = "auto"


class PackedKVWeight:
    """A K/V projection weight in the fragment-major layout of
    dspark_kv_weight_pack (include/dspark_project.h): `data` is a bf16
    tensor of cols * hidden elements on the weight's device.  Made by
    project.pack_kv_weight."""

    def __init__(self, data: torch.Tensor, cols: int, hidden: int):
        if data.dtype != torch.bfloat16 or data.numel() != cols * hidden or \
                not data.is_contiguous():
            raise ValueError("data must be a contiguous bf16 tensor of cols * hidden elements")
        self.data, self.cols, self.hidden = data, int(cols), int(hidden)


class DSparkContextKVWriter:
    """Writes precomputed context K/V into every draft layer's KV cache."""

    def __init__(self, attn_layers, debug_checks: bool = False) -> None:
        """debug_checks: check the preconditions the kernel trusts (positions
        in the table, slots in the cache, no shared slots) on every call,
        at the cost of a host sync per call."""
        self._debug_checks = bool(debug_checks)
        layers = list(attn_layers)
        error = self._validate(layers)
        if error is not None:
            raise ValueError(f"unsupported DSpark context-KV layout: {error}")
        self._layers = layers
        cache = layers[0].kv_cache
        self._num_layers = len(layers)
        self._num_kv_heads = cache.shape[1]
        self._kv_cache_dtype = "fp8" if cache.dtype == torch.uint8 else "auto"
        self._table_key = None
        self._handle = None

    @staticmethod
    def _validate(layers) -> str | None:
        if not layers:
            return "no layers"
        ref = None
        for a in layers:
            kv_dtype = getattr(a, "kv_cache_dtype", None)
            if kv_dtype not in SUPPORTED_KV_DTYPES:
                return f"kv_cache_dtype {kv_dtype!r}"
            cache = getattr(a, "kv_cache", None)
            if not isinstance(cache, torch.Tensor) or cache.numel() == 0:
                return "KV cache not bound"
            if cache.dim() != 4 or cache.shape[3] != 2 * HEAD_DIM:
                return f"unexpected cache shape {tuple(cache.shape)}"
            block_size = cache.shape[2]
            if block_size & (block_size - 1):
                return f"block size {block_size} is not a power of two"
            if not cache.is_contiguous():
                return "cache is not contiguous"
            if kv_dtype in ("fp8", "fp8_e4m3"):
                if cache.dtype != torch.uint8:
                    return f"fp8 cache has dtype {cache.dtype}"
            elif cache.dtype != torch.bfloat16:
                return f"cache has dtype {cache.dtype}"
            for name in ("_k_scale", "_v_scale"):
                scale = getattr(a, name, None)
                if (not isinstance(scale, torch.Tensor) or scale.dtype != torch.float32
                        or not scale.is_cuda):
                    return f"{name} is not a CUDA fp32 tensor"
            key = (cache.shape, cache.stride(), cache.dtype, kv_dtype)
            if ref is None:
                ref = key
            elif key != ref:
                return "layers do not share cache shape/stride/dtype"
            if cache.device != layers[0].kv_cache.device:
                return "layers are on different devices"
            delta = cache.data_ptr() - layers[0].kv_cache.data_ptr()
            if delta % (16 * cache.element_size()):
                return "layer caches are not 16-element aligned to each other"
        # what the raw pointers carry (alignment, limits) is checked by the library
        c0 = layers[0].kv_cache
        st = _lib.dspark_ctx_kv_validate(
            len(layers), [a.kv_cache.data_ptr() for a in layers],
            [a._k_scale.data_ptr() for a in layers], [a._v_scale.data_ptr() for a in layers],
            c0.shape[0], c0.shape[1], c0.shape[2], c0.shape[3] // 2,
            _lib.KV_FP8_E4M3 if c0.dtype == torch.uint8 else _lib.KV_AUTO)
        if st != _lib.OK:
            return _lib.dspark_ctx_kv_last_error()
        return None

    @staticmethod
    def supported(attn_layers) -> bool:
        """True when the HIP library is built, the layers' device is a gfx950
        GPU (its fp8 store is OCP E4M3) and the layout validates."""
        try:
            _lib.load()
        except _lib.LibraryMissing:
            return False
        layers = list(attn_layers)
        if not layers or not torch.cuda.is_available():
            return False
        cache = getattr(layers[0], "kv_cache", None)
        if not isinstance(cache, torch.Tensor) or not cache.is_cuda:
            return False
        arch = torch.cuda.get_device_properties(cache.device).gcnArchName
        if not arch.startswith("gfx950"):
            return False
        return DSparkContextKVWriter._validate(layers) is None

    def _ensure_tables(self) -> None:
        layers = self._layers
        key = tuple((a.kv_cache.data_ptr(), a._k_scale.data_ptr(), a._v_scale.data_ptr())
                    for a in layers)
        if key == self._table_key:
            return
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("DSpark context-KV caches were re-bound during graph capture; "
                               "call the writer once outside capture first")
        error = self._validate(layers)
        if error is not None:
            raise ValueError(f"unsupported DSpark context-KV layout: {error}")
        self.close()
        c0 = layers[0].kv_cache
        st, handle = _lib.dspark_ctx_kv_writer_create(
            len(layers), [a.kv_cache.data_ptr() for a in layers],
            [a._k_scale.data_ptr() for a in layers], [a._v_scale.data_ptr() for a in layers],
            c0.shape[0], c0.shape[1], c0.shape[2], c0.shape[3] // 2,
            _lib.KV_FP8_E4M3 if self._kv_cache_dtype == "fp8" else _lib.KV_AUTO)
        if st != _lib.OK:
            raise ValueError("unsupported DSpark context-KV layout: "
                             + _lib.dspark_ctx_kv_last_error())
        self._handle = handle
        self._table_key = key

    def __call__(self, all_kv: torch.Tensor, k_norm_weight: torch.Tensor, eps: float,
                 positions: torch.Tensor, cos_sin_cache: torch.Tensor, rotary_dim: int,
                 slot_mapping) -> None:
        """slot_mapping: one int64 [num_ctx] tensor shared by every layer, or
        a list of L such tensors (one per layer, as the model passes when its
        layers span several KV-cache groups), or an int64 [L, num_ctx]
        tensor.  A list whose entries are all the same tensor is the shared
        case (the rule of _shared_slot_mapping)."""
        num_ctx, L, two, nkv, hd = all_kv.shape
        assert self._num_layers == L and self._num_kv_heads == nkv
        assert two == 2 and hd == HEAD_DIM
        if num_ctx == 0:
            return
        dev = self._layers[0].kv_cache.device
        shared, per_layer = _split_slot_mapping(slot_mapping, L)
        for name, t, dt in (("all_kv", all_kv, torch.bfloat16),
                            ("k_norm_weight", k_norm_weight, torch.bfloat16),
                            ("positions", positions, torch.int64),
                            ("cos_sin_cache", cos_sin_cache, torch.bfloat16)):
            if t.dtype != dt or t.device != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
        for t in ([shared] if shared is not None else per_layer):
            if t.dtype != torch.int64 or t.device != dev or not t.is_contiguous() \
                    or t.shape != (num_ctx,):
                raise ValueError(f"slot mappings must be contiguous int64 ({num_ctx},) "
                                 f"tensors on {dev}")
        if tuple(k_norm_weight.shape) != (L, HEAD_DIM):
            raise ValueError(f"k_norm_weight has shape {tuple(k_norm_weight.shape)}, "
                             f"expected {(L, HEAD_DIM)}")
        if positions.shape != (num_ctx,):
            raise ValueError("positions must have shape (num_ctx,)")
        if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != rotary_dim:
            raise ValueError(f"cos_sin_cache has shape {tuple(cos_sin_cache.shape)}, "
                             f"expected (rows, {rotary_dim})")
        self._ensure_tables()
        if self._debug_checks:
            c0 = self._layers[0].kv_cache
            check_write_preconditions(positions, shared if shared is not None else per_layer,
                                      cos_sin_cache.shape[0], c0.shape[0], c0.shape[2])
        stream = torch.cuda.current_stream(dev).cuda_stream
        if shared is not None:
            st = _lib.dspark_ctx_kv_writer_write(
                self._handle, all_kv.data_ptr(), num_ctx, L, nkv, k_norm_weight.data_ptr(),
                float(eps), positions.data_ptr(), cos_sin_cache.data_ptr(),
                cos_sin_cache.shape[0], int(rotary_dim), shared.data_ptr(), stream)
        else:
            st = _lib.dspark_ctx_kv_writer_write_layer_slots(
                self._handle, all_kv.data_ptr(), num_ctx, L, nkv, k_norm_weight.data_ptr(),
                float(eps), positions.data_ptr(), cos_sin_cache.data_ptr(),
                cos_sin_cache.shape[0], int(rotary_dim), [t.data_ptr() for t in per_layer],
                stream)
        if st != _lib.OK:
            raise RuntimeError("DSpark context-KV write failed: " + _lib.dspark_ctx_kv_last_error())

    def project_write(self, states: torch.Tensor, kv_weight: "torch.Tensor | PackedKVWeight",
                      k_norm_weight: torch.Tensor, eps: float, positions: torch.Tensor,
                      cos_sin_cache: torch.Tensor, rotary_dim: int,
                      slot_mapping: torch.Tensor) -> None:
        """The projection all_kv = states @ kv_weight.T with this write fused
        into its epilogue (all_kv is never stored).  states: bf16
        [num_ctx, hidden], the hidden-norm output; kv_weight: bf16
        [L * 2 * nkv * 128, hidden] ([out, in], rows in all_kv's order), or
        that weight packed by project.pack_kv_weight (same results, bit for
        bit); slot_mapping: one int64 [num_ctx] tensor shared by every layer."""
        L, nkv = self._num_layers, self._num_kv_heads
        dev = self._layers[0].kv_cache.device
        if states.dim() != 2:
            raise ValueError("states must be [num_ctx, hidden]")
        num_ctx, hidden = states.shape
        packed = isinstance(kv_weight, PackedKVWeight)
        if packed:
            if (kv_weight.cols, kv_weight.hidden) != (L * 2 * nkv * HEAD_DIM, hidden):
                raise ValueError(f"the packed weight is for {(kv_weight.cols, kv_weight.hidden)}, "
                                 f"expected {(L * 2 * nkv * HEAD_DIM, hidden)}")
            kv_weight = kv_weight.data
        for name, t, dt in (("states", states, torch.bfloat16),
                            ("kv_weight", kv_weight, torch.bfloat16),
                            ("k_norm_weight", k_norm_weight, torch.bfloat16),
                            ("positions", positions, torch.int64),
                            ("cos_sin_cache", cos_sin_cache, torch.bfloat16),
                            ("slot_mapping", slot_mapping, torch.int64)):
            if t.dtype != dt or t.device != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
        if not packed and tuple(kv_weight.shape) != (L * 2 * nkv * HEAD_DIM, hidden):
            raise ValueError(f"kv_weight has shape {tuple(kv_weight.shape)}, "
                             f"expected {(L * 2 * nkv * HEAD_DIM, hidden)}")
        if tuple(k_norm_weight.shape) != (L, HEAD_DIM):
            raise ValueError(f"k_norm_weight has shape {tuple(k_norm_weight.shape)}")
        if positions.shape != (num_ctx,) or slot_mapping.shape != (num_ctx,):
            raise ValueError("positions and slot_mapping must have shape (num_ctx,)")
        if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != rotary_dim:
            raise ValueError(f"cos_sin_cache has shape {tuple(cos_sin_cache.shape)}")
        if num_ctx == 0:
            return
        self._ensure_tables()
        if self._debug_checks:
            c0 = self._layers[0].kv_cache
            check_write_preconditions(positions, slot_mapping, cos_sin_cache.shape[0],
                                      c0.shape[0], c0.shape[2])
        stream = torch.cuda.current_stream(dev).cuda_stream
        fn = (_lib.dspark_ctx_kv_writer_project_write_packed if packed
              else _lib.dspark_ctx_kv_writer_project_write)
        st = fn(
            self._handle, states.data_ptr(), num_ctx, hidden, kv_weight.data_ptr(), L, nkv,
            k_norm_weight.data_ptr(), float(eps), positions.data_ptr(), cos_sin_cache.data_ptr(),
            cos_sin_cache.shape[0], int(rotary_dim), slot_mapping.data_ptr(), stream)
        if st != _lib.OK:
            raise RuntimeError("DSpark projection + context-KV write failed: "
                               + _lib.dspark_ctx_kv_last_error())

    def close(self) -> None:
        if self._handle is not None:
            _lib.dspark_ctx_kv_writer_destroy(self._handle)
            self._handle = None
            self._table_key = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
