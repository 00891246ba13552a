"""PyTorch-facing writer for the DSpark fused context-KV write.

Offers what class DSparkContextKVWriter and rotary_dims_supported offer on
the vLLM API page "vllm.models.minimax_m3.common.ops.dspark_context_kv": a
writer built from the draft's attention layers (objects carrying
``kv_cache``, ``_k_scale``, ``_v_scale`` and ``kv_cache_dtype``), refused with
the page's reasons when their caches do not fit, and rebuilt (outside graph
capture only) when a cache or scale is re-bound.  The layout rules and every
step of the write live in the HIP library: this module describes the
tensors to it (address, element type, device, shape, strides) and passes
pointers.  PyTorch supplies device memory and the current stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib

HEAD_DIM = _lib.HEAD_DIM


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
    """The write's preconditions that the kernels do not check (as on the
    vLLM API page "vllm.models.minimax_m3.common.ops.dspark_context_kv"),
    exactly as far as the kernels rely on them: the position of every token
    that is stored in at least one layer indexes the cos/sin table (the
    positions of tokens stored in no layer are never read), every slot is
    inside the cache, and no two tokens share a slot within one layer.
    Raises ValueError naming the first violation.  Costs a host sync: meant
    for debugging (DSparkContextKVWriter(debug_checks=True))."""
    maps = [slot_mapping] if isinstance(slot_mapping, torch.Tensor) and slot_mapping.dim() == 1 \
        else list(slot_mapping)
    stored = torch.zeros_like(positions, dtype=torch.bool)
    for slots in maps:
        stored |= slots >= 0
    pos = positions[stored]
    if pos.numel() and (bool((pos < 0).any()) or bool((pos >= cos_sin_rows).any())):
        raise ValueError(f"a stored token's position is outside the cos/sin table of "
                         f"{cos_sin_rows} rows")
    capacity = int(num_blocks) * int(block_size)
    for l, slots in enumerate(maps):
        s = slots[slots >= 0]
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


_ELEMENT_TYPES = {torch.bfloat16: _lib.DTYPE_BF16, torch.uint8: _lib.DTYPE_UINT8,
                  torch.float32: _lib.DTYPE_FP32}


def tensor_info(t) -> _lib.TensorInfo:
    """The facts of one layer attribute that the library's layout rules use
    (a zeroed record when the attribute is not a tensor)."""
    info = _lib.TensorInfo()
    if not isinstance(t, torch.Tensor):
        return info
    info.data = t.data_ptr() or None
    info.dtype = _ELEMENT_TYPES.get(t.dtype, _lib.DTYPE_OTHER)
    info.dtype_name = str(t.dtype).encode()
    info.on_gpu = int(t.is_cuda)
    info.device_index = t.device.index if t.is_cuda else -1
    dims = min(t.dim(), _lib.MAX_DIMS)
    info.ndim = dims
    info.shape[:dims] = list(t.shape[:dims])
    info.strides[:dims] = list(t.stride()[:dims])
    return info


def layer_info(layer) -> _lib.LayerInfo:
    """One attention layer described for dspark_ctx_kv_validate / create."""
    info = _lib.LayerInfo()
    name = getattr(layer, "kv_cache_dtype", None)
    info.kv_cache_dtype = None if name is None else str(name).encode()
    info.kv_cache = tensor_info(getattr(layer, "kv_cache", None))
    info.k_scale = tensor_info(getattr(layer, "_k_scale", None))
    info.v_scale = tensor_info(getattr(layer, "_v_scale", None))
    return info


def layout_error(attn_layers) -> "str | None":
    """Why the library would refuse these layers' caches (the first broken
    rule, in the page's words), or None if it accepts them."""
    infos = [layer_info(a) for a in attn_layers]
    if _lib.dspark_ctx_kv_validate(len(infos), infos) == _lib.OK:
        return None
    return _lib.dspark_ctx_kv_last_error()


def _refuse(reason: str) -> ValueError:
    return ValueError(f"unsupported DSpark context-KV layout: {reason}")


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
        self._layers = list(attn_layers)
        reason = layout_error(self._layers)
        if reason is not None:
            raise _refuse(reason)
        first = self._layers[0].kv_cache
        self._num_layers = len(self._layers)
        self._num_kv_heads = first.shape[1]
        self._debug_checks = bool(debug_checks)
        self._handle = None       # the library's writer
        self._bound_to = None     # the cache and scale addresses it was built for

    @staticmethod
    def supported(attn_layers) -> bool:
        """True when the HIP library is built, the layers live on a gfx950
        GPU (its fp8 conversion is OCP E4M3) and the library accepts their
        layout."""
        try:
            _lib.load()
        except _lib.LibraryMissing:
            return False
        layers = list(attn_layers)
        cache = getattr(layers[0], "kv_cache", None) if layers else None
        if not isinstance(cache, torch.Tensor) or not cache.is_cuda:
            return False
        if not torch.cuda.get_device_properties(cache.device).gcnArchName.startswith("gfx950"):
            return False
        return layout_error(layers) is None

    def _addresses(self) -> tuple:
        return tuple(t.data_ptr() for a in self._layers
                     for t in (a.kv_cache, a._k_scale, a._v_scale))

    def _bind(self) -> None:
        """Build the library's writer on first use, and again whenever a
        layer's cache or scale tensor has been replaced since (never while
        the stream is being captured: a graph must keep its addresses)."""
        addresses = self._addresses()
        if addresses == self._bound_to:
            return
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("DSpark context-KV caches were re-bound during graph capture; "
                               "call the writer once outside capture first")
        infos = [layer_info(a) for a in self._layers]
        st, handle = _lib.dspark_ctx_kv_writer_create(len(infos), infos)
        if st != _lib.OK:
            raise _refuse(_lib.dspark_ctx_kv_last_error())
        self.close()
        self._handle, self._bound_to = handle, addresses

    def _check_inputs(self, num_ctx: int, tensors, slot_tensors) -> None:
        """Element type, device and contiguity of every input (the library
        takes raw pointers and cannot see them)."""
        dev = self._layers[0].kv_cache.device
        for name, t, dt in tensors:
            if t.dtype != dt or t.device != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
        for t in slot_tensors:
            if t.dtype != torch.int64 or t.device != dev or not t.is_contiguous() \
                    or t.shape != (num_ctx,):
                raise ValueError(f"slot mappings must be contiguous int64 ({num_ctx},) "
                                 f"tensors on {dev}")

    def __call__(self, all_kv: torch.Tensor, k_norm_weight: torch.Tensor, eps: float,
                 positions: torch.Tensor, cos_sin_cache: torch.Tensor, rotary_dim: int,
                 slot_mapping) -> None:
        """all_kv: bf16 [num_ctx, L, 2, nkv, 128] (axis 2: K, V).
        slot_mapping: one int64 [num_ctx] tensor shared by every layer, or
        a list of L such tensors (one per layer, as the model passes when its
        layers span several KV-cache groups), or an int64 [L, num_ctx]
        tensor.  A list whose entries are all the same tensor is the shared
        case (the rule of _shared_slot_mapping).  A layer count or kv head
        count other than the writer's is refused by the library."""
        if all_kv.dim() != 5 or all_kv.shape[2] != 2 or all_kv.shape[4] != HEAD_DIM:
            raise ValueError(f"all_kv must be [num_ctx, L, 2, nkv, {HEAD_DIM}], "
                             f"got {tuple(all_kv.shape)}")
        num_ctx, num_layers, _, num_kv_heads, _ = all_kv.shape
        shared, per_layer = _split_slot_mapping(slot_mapping, num_layers)
        self._check_inputs(num_ctx, (("all_kv", all_kv, torch.bfloat16),
                                     ("k_norm_weight", k_norm_weight, torch.bfloat16),
                                     ("positions", positions, torch.int64),
                                     ("cos_sin_cache", cos_sin_cache, torch.bfloat16)),
                           [shared] if shared is not None else per_layer)
        if tuple(k_norm_weight.shape) != (num_layers, HEAD_DIM):
            raise ValueError(f"k_norm_weight has shape {tuple(k_norm_weight.shape)}, "
                             f"expected {(num_layers, HEAD_DIM)}")
        if positions.shape != (num_ctx,):
            raise ValueError("positions must have shape (num_ctx,)")
        if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != rotary_dim:
            raise ValueError(f"cos_sin_cache has shape {tuple(cos_sin_cache.shape)}, "
                             f"expected (rows, {rotary_dim})")
        self._bind()
        if self._debug_checks and num_ctx:
            c0 = self._layers[0].kv_cache
            check_write_preconditions(positions, shared if shared is not None else per_layer,
                                      cos_sin_cache.shape[0], c0.shape[0], c0.shape[2])
        stream = torch.cuda.current_stream(all_kv.device).cuda_stream
        common = (self._handle, all_kv.data_ptr(), num_ctx, num_layers, num_kv_heads,
                  k_norm_weight.data_ptr(), float(eps), positions.data_ptr(),
                  cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], int(rotary_dim))
        if shared is not None:
            st = _lib.dspark_ctx_kv_writer_write(*common, shared.data_ptr(), stream)
        else:
            st = _lib.dspark_ctx_kv_writer_write_layer_slots(
                *common, [t.data_ptr() for t in per_layer], stream)
        if st != _lib.OK:
            raise RuntimeError("DSpark context-KV write failed: " + _lib.dspark_ctx_kv_last_error())

    def project_write(self, states: torch.Tensor, kv_weight: "torch.Tensor | PackedKVWeight",
                      k_norm_weight: torch.Tensor, eps: float, positions: torch.Tensor,
                      cos_sin_cache: torch.Tensor, rotary_dim: int,
                      slot_mapping: torch.Tensor, all_kv_out: "torch.Tensor | None" = None) -> None:
        """The projection all_kv = states @ kv_weight.T with this write fused
        into its epilogue (all_kv is not stored unless all_kv_out is given).
        states: bf16 [num_ctx, hidden], the hidden-norm output; kv_weight:
        bf16 [L * 2 * nkv * 128, hidden] ([out, in], rows in all_kv's order),
        or that weight packed by project.pack_kv_weight (same results, bit
        for bit); slot_mapping: one int64 [num_ctx] tensor shared by every
        layer; all_kv_out: an optional bf16 [num_ctx, L, 2, nkv, 128] tensor
        that also receives the projection's output (the values the write
        normalised and stored)."""
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
        self._check_inputs(num_ctx, (("states", states, torch.bfloat16),
                                     ("kv_weight", kv_weight, torch.bfloat16),
                                     ("k_norm_weight", k_norm_weight, torch.bfloat16),
                                     ("positions", positions, torch.int64),
                                     ("cos_sin_cache", cos_sin_cache, torch.bfloat16),
                                     ("slot_mapping", slot_mapping, torch.int64)), ())
        if not packed and tuple(kv_weight.shape) != (L * 2 * nkv * HEAD_DIM, hidden):
            raise ValueError(f"kv_weight has shape {tuple(kv_weight.shape)}, "
                             f"expected {(L * 2 * nkv * HEAD_DIM, hidden)}")
        if tuple(k_norm_weight.shape) != (L, HEAD_DIM):
            raise ValueError(f"k_norm_weight has shape {tuple(k_norm_weight.shape)}")
        if positions.shape != (num_ctx,) or slot_mapping.shape != (num_ctx,):
            raise ValueError("positions and slot_mapping must have shape (num_ctx,)")
        if cos_sin_cache.dim() != 2 or cos_sin_cache.shape[1] != rotary_dim:
            raise ValueError(f"cos_sin_cache has shape {tuple(cos_sin_cache.shape)}")
        if all_kv_out is not None:
            self._check_inputs(num_ctx, (("all_kv_out", all_kv_out, torch.bfloat16),), ())
            if tuple(all_kv_out.shape) != (num_ctx, L, 2, nkv, HEAD_DIM):
                raise ValueError(f"all_kv_out has shape {tuple(all_kv_out.shape)}, "
                                 f"expected {(num_ctx, L, 2, nkv, HEAD_DIM)}")
        if num_ctx == 0:
            return
        self._bind()
        if self._debug_checks:
            c0 = self._layers[0].kv_cache
            check_write_preconditions(positions, slot_mapping, cos_sin_cache.shape[0],
                                      c0.shape[0], c0.shape[2])
        stream = torch.cuda.current_stream(dev).cuda_stream
        if all_kv_out is not None:
            st = _lib.dspark_ctx_kv_writer_project_write_all_kv(
                self._handle, states.data_ptr(), num_ctx, hidden, kv_weight.data_ptr(),
                int(packed), L, nkv, k_norm_weight.data_ptr(), float(eps), positions.data_ptr(),
                cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], int(rotary_dim),
                slot_mapping.data_ptr(), all_kv_out.data_ptr(), stream)
        else:
            fn = (_lib.dspark_ctx_kv_writer_project_write_packed if packed
                  else _lib.dspark_ctx_kv_writer_project_write)
            st = fn(self._handle, states.data_ptr(), num_ctx, hidden, kv_weight.data_ptr(), L,
                    nkv, k_norm_weight.data_ptr(), float(eps), positions.data_ptr(),
                    cos_sin_cache.data_ptr(), cos_sin_cache.shape[0], int(rotary_dim),
                    slot_mapping.data_ptr(), stream)
        if st != _lib.OK:
            raise RuntimeError("DSpark projection + context-KV write failed: "
                               + _lib.dspark_ctx_kv_last_error())

    def close(self) -> None:
        if self._handle is not None:
            _lib.dspark_ctx_kv_writer_destroy(self._handle)
            self._handle = None
            self._bound_to = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
