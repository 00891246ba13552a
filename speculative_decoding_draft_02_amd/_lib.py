"""ctypes binding of libdspark_ctx_kv.so (include/dspark_ctx_kv.h,
include/dspark_qknorm_insert.h and include/dspark_project.h).

Argument marshalling only: every function here has the name and argument
order of the C entry point it calls, takes device pointers as Python ints,
and returns the C status.  The library must have been built in-tree
(``python -m speculative_decoding_draft_02_amd.build``); loading fails
loudly otherwise, and nothing here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdspark_ctx_kv.so")

HEAD_DIM = 128
MAX_LAYERS = 32
KV_AUTO = 0
KV_FP8_E4M3 = 1
OK = 0
E_LAYOUT = -1
E_ARG = -2
E_HIP = -4
DTYPE_OTHER = 0
DTYPE_BF16 = 1
DTYPE_UINT8 = 2
DTYPE_FP32 = 3
MAX_DIMS = 8


class TensorInfo(ctypes.Structure):
    """struct dspark_tensor_info."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("dtype_name", ctypes.c_char_p), ("on_gpu", ctypes.c_int32),
                ("device_index", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS), ("strides", ctypes.c_int64 * MAX_DIMS)]


class LayerInfo(ctypes.Structure):
    """struct dspark_layer_info."""
    _fields_ = [("kv_cache_dtype", ctypes.c_char_p), ("kv_cache", TensorInfo),
                ("k_scale", TensorInfo), ("v_scale", TensorInfo)]

# every entry point the header declares, with its ctypes signature
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
SIGNATURES = {
    "dspark_ctx_kv_validate": ([_I32, _P], ctypes.c_int),
    "dspark_ctx_kv_writer_create": ([_I32, _P, _P], ctypes.c_int),
    "dspark_ctx_kv_writer_write": ([_P, _P, _I64, _I32, _I32, _P, ctypes.c_float, _P, _P, _I64,
                                    _I32, _P, _P], ctypes.c_int),
    "dspark_ctx_kv_writer_write_layer_slots": ([_P, _P, _I64, _I32, _I32, _P, ctypes.c_float, _P, _P,
                                                _I64, _I32, _P, _P], ctypes.c_int),
    "dspark_ctx_kv_writer_destroy": ([_P], None),
    "dspark_rotary_dims_supported": ([_I32, _I32], ctypes.c_int),
    "dspark_ctx_kv_last_error": ([], ctypes.c_char_p),
    "dspark_hidden_norm": ([_P, _I64, _I32, _P, ctypes.c_float, _P, _P], ctypes.c_int),
    "dspark_ctx_kv_writer_project_write": ([_P, _P, _I64, _I32, _P, _I32, _I32, _P, ctypes.c_float,
                                            _P, _P, _I64, _I32, _P, _P], ctypes.c_int),
    "dspark_ctx_kv_writer_project_write_packed": ([_P, _P, _I64, _I32, _P, _I32, _I32, _P,
                                                   ctypes.c_float, _P, _P, _I64, _I32, _P, _P],
                                                  ctypes.c_int),
    "dspark_ctx_kv_writer_project_write_all_kv": ([_P, _P, _I64, _I32, _P, _I32, _I32, _I32, _P,
                                                   ctypes.c_float, _P, _P, _I64, _I32, _P, _P,
                                                   _P], ctypes.c_int),
    "dspark_kv_weight_pack": ([_P, _I64, _I32, _P, _P], ctypes.c_int),
    "dspark_qknorm_rope_kv_insert": ([_P, _I64, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                      ctypes.c_float, _P, _P, _I64, _I32, _I32, _P, _P, _P,
                                      ctypes.c_float, _P], ctypes.c_int),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                "libdspark_ctx_kv.so is not built (%s); run "
                "`python -m speculative_decoding_draft_02_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _ptr_array(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*[int(p) for p in ptrs])


def dspark_ctx_kv_validate(num_layers, layers) -> int:
    """layers: a sequence of LayerInfo (or a ctypes array of them)."""
    arr = (LayerInfo * max(1, len(layers)))(*layers)
    return load().dspark_ctx_kv_validate(num_layers, ctypes.cast(arr, _P) if len(layers) else None)


def dspark_ctx_kv_writer_create(num_layers, layers):
    """Returns (status, writer handle as int or None)."""
    arr = (LayerInfo * max(1, len(layers)))(*layers)
    out = ctypes.c_void_p(0)
    st = load().dspark_ctx_kv_writer_create(num_layers, ctypes.cast(arr, _P) if len(layers) else None,
                                            ctypes.byref(out))
    return st, out.value


def dspark_ctx_kv_writer_write(writer, all_kv, num_ctx, num_layers, num_kv_heads, k_norm_weight,
                               eps, positions, cos_sin_cache, cos_sin_rows, rotary_dim,
                               slot_mapping, stream) -> int:
    return load().dspark_ctx_kv_writer_write(
        writer, all_kv, num_ctx, num_layers, num_kv_heads, k_norm_weight, eps, positions,
        cos_sin_cache, cos_sin_rows, rotary_dim, slot_mapping, stream)


def dspark_ctx_kv_writer_write_layer_slots(writer, all_kv, num_ctx, num_layers, num_kv_heads,
                                           k_norm_weight, eps, positions, cos_sin_cache,
                                           cos_sin_rows, rotary_dim, slot_mappings, stream) -> int:
    """slot_mappings: a sequence of num_layers device pointers."""
    return load().dspark_ctx_kv_writer_write_layer_slots(
        writer, all_kv, num_ctx, num_layers, num_kv_heads, k_norm_weight, eps, positions,
        cos_sin_cache, cos_sin_rows, rotary_dim,
        ctypes.cast(_ptr_array(slot_mappings), _P), stream)


def dspark_ctx_kv_writer_destroy(writer) -> None:
    load().dspark_ctx_kv_writer_destroy(writer)


def dspark_rotary_dims_supported(rotary_dim, head_dim) -> int:
    return load().dspark_rotary_dims_supported(rotary_dim, head_dim)


def dspark_ctx_kv_last_error() -> str:
    return load().dspark_ctx_kv_last_error().decode()


def dspark_qknorm_rope_kv_insert(qkv, num_tokens, q_norm_weight, k_norm_weight, cos_sin_cache,
                                 cos_sin_rows, positions, num_heads, num_kv_heads, rotary_dim, eps,
                                 slot_mapping, kv_cache, num_blocks, block_size, kv_cache_dtype,
                                 k_scale, v_scale, q_fp8_out, q_fp8_scale, stream) -> int:
    return load().dspark_qknorm_rope_kv_insert(
        qkv, num_tokens, q_norm_weight, k_norm_weight, cos_sin_cache, cos_sin_rows, positions,
        num_heads, num_kv_heads, rotary_dim, eps, slot_mapping, kv_cache, num_blocks, block_size,
        kv_cache_dtype, k_scale, v_scale, q_fp8_out, q_fp8_scale, stream)


def dspark_hidden_norm(x, rows, dim, weight, eps, out, stream) -> int:
    return load().dspark_hidden_norm(x, rows, dim, weight, eps, out, stream)


def dspark_ctx_kv_writer_project_write(writer, states, num_ctx, hidden, kv_weight, num_layers,
                                       num_kv_heads, k_norm_weight, eps, positions, cos_sin_cache,
                                       cos_sin_rows, rotary_dim, slot_mapping, stream) -> int:
    return load().dspark_ctx_kv_writer_project_write(
        writer, states, num_ctx, hidden, kv_weight, num_layers, num_kv_heads, k_norm_weight, eps,
        positions, cos_sin_cache, cos_sin_rows, rotary_dim, slot_mapping, stream)


def dspark_ctx_kv_writer_project_write_packed(writer, states, num_ctx, hidden, packed_kv_weight,
                                              num_layers, num_kv_heads, k_norm_weight, eps,
                                              positions, cos_sin_cache, cos_sin_rows, rotary_dim,
                                              slot_mapping, stream) -> int:
    return load().dspark_ctx_kv_writer_project_write_packed(
        writer, states, num_ctx, hidden, packed_kv_weight, num_layers, num_kv_heads, k_norm_weight,
        eps, positions, cos_sin_cache, cos_sin_rows, rotary_dim, slot_mapping, stream)


def dspark_ctx_kv_writer_project_write_all_kv(writer, states, num_ctx, hidden, kv_weight,
                                              weight_packed, num_layers, num_kv_heads,
                                              k_norm_weight, eps, positions, cos_sin_cache,
                                              cos_sin_rows, rotary_dim, slot_mapping, all_kv_out,
                                              stream) -> int:
    return load().dspark_ctx_kv_writer_project_write_all_kv(
        writer, states, num_ctx, hidden, kv_weight, weight_packed, num_layers, num_kv_heads,
        k_norm_weight, eps, positions, cos_sin_cache, cos_sin_rows, rotary_dim, slot_mapping,
        all_kv_out, stream)


def dspark_kv_weight_pack(kv_weight, cols, hidden, packed, stream) -> int:
    return load().dspark_kv_weight_pack(kv_weight, cols, hidden, packed, stream)
