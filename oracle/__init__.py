"""Exact-value CPU oracle for the DSpark fused context-KV write, the draft
block's fused QK-norm / RoPE / KV insert, and the step before the write (the
hidden norm and the token-major K/V projection).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
package never imports it, and it imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain C, fp64, scalar loops); this
module builds it with gcc, loads it with ctypes and wraps it for numpy
arrays.  What it computes is stated, with its source on the vLLM API page
"vllm.models.minimax_m3.common.ops.dspark_context_kv", in that file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

HEAD_DIM = 128
MAX_CAND = 4
# Relative distance to a bf16 rounding midpoint within which both bf16
# neighbours of the fp32 norm output are correct answers.  A 128-term fp32
# sum, an rsqrt with <= 1 ulp error and three fp32 roundings stay below about
# 2^-21 relative; 2^-18 leaves a factor-8 margin.
NEAR_DELTA = 2.0 ** -18

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc and return its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.dspark_oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.dspark_oracle_bf16_decode.restype = ctypes.c_double
        L.dspark_oracle_bf16_round.argtypes = [ctypes.c_double, ctypes.c_double,
                                               ctypes.POINTER(ctypes.c_int),
                                               ctypes.POINTER(ctypes.c_uint16)]
        L.dspark_oracle_bf16_round.restype = ctypes.c_uint16
        L.dspark_oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.dspark_oracle_e4m3_decode.restype = ctypes.c_double
        L.dspark_oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.dspark_oracle_e4m3_encode.restype = ctypes.c_uint8
        L.dspark_oracle_fp8_store.argtypes = [ctypes.c_uint16, ctypes.c_float]
        L.dspark_oracle_fp8_store.restype = ctypes.c_uint8
        L.dspark_oracle_ctx_kv_write.argtypes = [
            P, i64, i32, i32,            # all_kv, num_ctx, L, nkv
            P, ctypes.c_float,           # k_norm_weight, eps
            P, P, i64, i32,              # positions, cos_sin, cs_rows, R
            P, i64, i64, i32,            # slots, slot_layer_stride, num_blocks, block_size
            i32, P, P,                   # fp8, k_scales, v_scales
            P,                           # caches (void**)
            ctypes.c_double,             # near_delta
            P, P, P, P, i64,             # alt_layer, alt_index, alt_count, alt_codes, cap
            i64, i64]                    # t_begin, t_end
        L.dspark_oracle_ctx_kv_write.restype = i64
        L.dspark_oracle_qknorm_rope_kv_insert.argtypes = [
            P, i64, i32, i32,            # qkv, num_tokens, num_heads, nkv
            P, P, ctypes.c_float,        # q_norm_weight, k_norm_weight, eps
            P, P, i64, i32,              # positions, cos_sin, cs_rows, R
            P, P, i64, i32,              # slot_mapping, cache, num_blocks, block_size
            i32, ctypes.c_float, ctypes.c_float,   # fp8, k_scale, v_scale
            P, ctypes.c_float,           # q_fp8, q_scale
            ctypes.c_double,             # near_delta
            P, P, P, P, i64]             # alt_tag, alt_index, alt_count, alt_codes, cap
        L.dspark_oracle_qknorm_rope_kv_insert.restype = i64
        L.dspark_oracle_gemma_rms_norm.argtypes = [P, i64, i32, P, ctypes.c_float, P,
                                                   ctypes.c_double, P, P, i64]
        L.dspark_oracle_gemma_rms_norm.restype = i64
        L.dspark_oracle_kv_project.argtypes = [P, i32, P, i64, i64, i64, i64, P, P, P]
        L.dspark_oracle_kv_project.restype = None
        _lib = L
    return _lib


# ------------------------------------------------------------- codecs ----

def bf16_round(z: float, near_delta: float = 0.0):
    """(code, near_tie, other_code) of the one-step bf16 RNE rounding of z."""
    near = ctypes.c_int(0)
    other = ctypes.c_uint16(0)
    code = lib().dspark_oracle_bf16_round(float(z), float(near_delta),
                                          ctypes.byref(near), ctypes.byref(other))
    return int(code), bool(near.value), int(other.value)


def bf16_decode(code: int) -> float:
    return float(lib().dspark_oracle_bf16_decode(int(code) & 0xFFFF))


def e4m3_decode(code: int) -> float:
    return float(lib().dspark_oracle_e4m3_decode(int(code) & 0xFF))


def e4m3_encode(x: float) -> int:
    return int(lib().dspark_oracle_e4m3_encode(float(x)))


def fp8_store(bf16_code: int, scale: float) -> int:
    return int(lib().dspark_oracle_fp8_store(int(bf16_code) & 0xFFFF, float(scale)))


# --------------------------------------------------------- the write ----

@dataclass
class OracleResult:
    caches: list          # per-layer numpy arrays (uint16 or uint8), same shape as the device caches
    alt_layer: np.ndarray  # int64 [n]
    alt_index: np.ndarray  # int64 [n], element index into that layer's flat cache
    alt_count: np.ndarray  # int32 [n]
    alt_codes: np.ndarray  # uint16 [n, 4]


def ctx_kv_write(all_kv, k_norm_weight, eps, positions, cos_sin, rotary_dim,
                 slot_mapping, caches, fp8, k_scales=None, v_scales=None,
                 near_delta: float = NEAR_DELTA, t_begin: int = 0,
                 t_end: int | None = None, alt_capacity: int | None = None) -> OracleResult:
    """Run the oracle on host arrays.  ``caches`` (a list of per-layer numpy
    arrays [num_blocks, nkv, bs, 256], uint16 for bf16 or uint8 for fp8) are
    written in place and returned; every other input is read only.

    all_kv: uint16 [num_ctx, L, 2, nkv, 128]; k_norm_weight: uint16 [L, 128];
    positions: int64 [num_ctx]; slot_mapping: int64 [num_ctx] (shared by every
    layer) or [L, num_ctx] (one mapping per layer); cos_sin: uint16 [rows, R];
    k_scales, v_scales: float32 [L].
    """
    all_kv = np.ascontiguousarray(all_kv, dtype=np.uint16)
    num_ctx, L, two, nkv, hd = all_kv.shape
    assert two == 2 and hd == HEAD_DIM
    w = np.ascontiguousarray(k_norm_weight, dtype=np.uint16)
    assert w.shape == (L, HEAD_DIM)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    cs = np.ascontiguousarray(cos_sin, dtype=np.uint16)
    assert cs.ndim == 2 and cs.shape[1] == rotary_dim
    assert len(caches) == L
    want = np.uint8 if fp8 else np.uint16
    for c in caches:
        assert c.dtype == want and c.flags.c_contiguous and c.ndim == 4
        assert c.shape == caches[0].shape and c.shape[1] == nkv and c.shape[3] == 2 * HEAD_DIM
    num_blocks, _, bs, _ = caches[0].shape
    if slots.ndim == 2:
        assert slots.shape == (L, num_ctx)
        slot_stride = num_ctx
    else:
        assert slots.shape == (num_ctx,)
        slot_stride = 0
    ks = np.ascontiguousarray(k_scales if k_scales is not None else np.ones(L), dtype=np.float32)
    vs = np.ascontiguousarray(v_scales if v_scales is not None else np.ones(L), dtype=np.float32)
    if t_end is None:
        t_end = num_ctx
    ptrs = (ctypes.c_void_p * L)(*[c.ctypes.data for c in caches])

    cap = alt_capacity if alt_capacity is not None else max(1024, (t_end - t_begin) * L * nkv // 16)
    while True:
        a_layer = np.zeros(cap, np.int64)
        a_index = np.zeros(cap, np.int64)
        a_count = np.zeros(cap, np.int32)
        a_codes = np.zeros((cap, MAX_CAND), np.uint16)
        n = lib().dspark_oracle_ctx_kv_write(
            all_kv.ctypes.data, num_ctx, L, nkv, w.ctypes.data, float(eps),
            pos.ctypes.data, cs.ctypes.data, cs.shape[0], rotary_dim,
            slots.ctypes.data, slot_stride, num_blocks, bs, 1 if fp8 else 0,
            ks.ctypes.data, vs.ctypes.data, ctypes.cast(ptrs, ctypes.c_void_p),
            float(near_delta), a_layer.ctypes.data, a_index.ctypes.data,
            a_count.ctypes.data, a_codes.ctypes.data, cap, t_begin, t_end)
        if n < 0:
            raise ValueError("oracle precondition failed (code %d)" % n)
        if n <= cap:
            return OracleResult(caches, a_layer[:n], a_index[:n], a_count[:n], a_codes[:n])
        cap = int(n)


# ------------------------------------------- the draft-block insert ----

@dataclass
class InsertResult:
    qkv: np.ndarray            # uint16 [T, (H + 2 nkv) * 128], q and k heads normed and rotated
    cache: np.ndarray | None   # the cache after the insert (the array passed in), or None
    q_fp8: np.ndarray | None   # uint8 [T, H * 128] or None
    alt_tag: np.ndarray        # int64 [n]: 0 qkv, 1 cache, 2 q_fp8
    alt_index: np.ndarray      # int64 [n], element index into that flat output
    alt_count: np.ndarray      # int32 [n]
    alt_codes: np.ndarray      # uint16 [n, 4]


def qknorm_rope_kv_insert(qkv, num_heads, num_kv_heads, q_norm_weight, k_norm_weight, eps,
                          positions, cos_sin, rotary_dim, slot_mapping=None, cache=None,
                          fp8=False, k_scale=1.0, v_scale=1.0, want_q_fp8=False, q_scale=1.0,
                          near_delta: float = NEAR_DELTA) -> InsertResult:
    """Run the draft-block oracle on host arrays.  ``qkv`` (uint16
    [T, (H + 2 nkv) * 128]) is read only: the updated copy is returned.
    ``cache`` ([num_blocks, nkv, bs, 256], uint16 for bf16 or uint8 for fp8)
    is written in place when slot_mapping is given."""
    src = np.ascontiguousarray(qkv, dtype=np.uint16)
    T = src.shape[0]
    H, nkv = int(num_heads), int(num_kv_heads)
    assert src.shape == (T, (H + 2 * nkv) * HEAD_DIM)
    qw = np.ascontiguousarray(q_norm_weight, dtype=np.uint16).reshape(HEAD_DIM)
    kw = np.ascontiguousarray(k_norm_weight, dtype=np.uint16).reshape(HEAD_DIM)
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    assert pos.shape == (T,)
    cs = np.ascontiguousarray(cos_sin, dtype=np.uint16)
    assert cs.ndim == 2 and cs.shape[1] == rotary_dim
    slots_ptr, cache_ptr, nb, bs = None, None, 0, 0
    if slot_mapping is not None:
        slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        assert slots.shape == (T,)
        assert cache is not None and cache.flags.c_contiguous and cache.ndim == 4
        assert cache.dtype == (np.uint8 if fp8 else np.uint16)
        nb, c_nkv, bs, width = cache.shape
        assert c_nkv == nkv and width == 2 * HEAD_DIM
        slots_ptr, cache_ptr = slots.ctypes.data, cache.ctypes.data
    cap = max(1024, T * (H + nkv) * 2)
    while True:
        out = src.copy()
        qf = np.zeros((T, H * HEAD_DIM), np.uint8) if want_q_fp8 else None
        a_tag = np.zeros(cap, np.int64)
        a_index = np.zeros(cap, np.int64)
        a_count = np.zeros(cap, np.int32)
        a_codes = np.zeros((cap, MAX_CAND), np.uint16)
        n = lib().dspark_oracle_qknorm_rope_kv_insert(
            out.ctypes.data, T, H, nkv, qw.ctypes.data, kw.ctypes.data, float(eps),
            pos.ctypes.data, cs.ctypes.data, cs.shape[0], rotary_dim,
            slots_ptr, cache_ptr, nb, bs, 1 if fp8 else 0, float(k_scale), float(v_scale),
            qf.ctypes.data if qf is not None else None, float(q_scale), float(near_delta),
            a_tag.ctypes.data, a_index.ctypes.data, a_count.ctypes.data, a_codes.ctypes.data,
            cap)
        if n < 0:
            raise ValueError("oracle precondition failed (code %d)" % n)
        if n <= cap:
            return InsertResult(out, cache if slot_mapping is not None else None, qf,
                                a_tag[:n], a_index[:n], a_count[:n], a_codes[:n])
        cap = int(n)


# ------------------------------------------------ the step before the write ----

def gemma_rms_norm(x, w, eps, near_delta: float = NEAR_DELTA):
    """Gemma RMSNorm of each row of x (uint16 bf16 bits [rows, dim]) with
    weight w [dim]: returns (codes [rows, dim], near-tie flat indices, the
    other bf16 neighbour of each)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    rows, dim = x.shape
    w = np.ascontiguousarray(w, dtype=np.uint16).reshape(dim)
    out = np.empty_like(x)
    cap = max(1024, x.size // 64)
    while True:
        idx = np.zeros(cap, np.int64)
        other = np.zeros(cap, np.uint16)
        n = lib().dspark_oracle_gemma_rms_norm(x.ctypes.data, rows, dim, w.ctypes.data, float(eps),
                                               out.ctypes.data, float(near_delta), idx.ctypes.data,
                                               other.ctypes.data, cap)
        if n <= cap:
            return out, idx[:n], other[:n]
        cap = int(n)


def kv_project(z, W, rows=None, cols=None, want_sums: bool = False):
    """bf16 of the exact products z @ W.T for the row range `rows` and column
    range `cols` (each a (begin, end) pair, default all).  z: uint16 [N,
    hidden], W: uint16 [C, hidden].  Returns the codes [r, c] and, with
    want_sums, also the fp64 sums and sums of |products|."""
    z = np.ascontiguousarray(z, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    N, hidden = z.shape
    C, h2 = W.shape
    assert h2 == hidden
    r0, r1 = rows if rows is not None else (0, N)
    c0, c1 = cols if cols is not None else (0, C)
    assert 0 <= r0 <= r1 <= N and 0 <= c0 <= c1 <= C
    out = np.empty((r1 - r0, c1 - c0), np.uint16)
    ex = np.empty(out.shape, np.float64) if want_sums else None
    ab = np.empty(out.shape, np.float64) if want_sums else None
    lib().dspark_oracle_kv_project(z.ctypes.data, hidden, W.ctypes.data, r0, r1, c0, c1,
                                   out.ctypes.data, ex.ctypes.data if want_sums else None,
                                   ab.ctypes.data if want_sums else None)
    return (out, ex, ab) if want_sums else out


def kv_project_sums(z, W):
    """The projection's exact dot products for every row and column, for
    full-size checks: z (uint16 bf16 bits [N, hidden]) and W ([C, hidden])
    decoded to float64, where every bf16 x bf16 product is exact; the sums
    z @ W.T and |z| @ |W|.T are taken by numpy's float64 matrix product (a
    library primitive, any summation order).  Returns (sums, abs_sums, err)
    with |sums - exact| <= err and |abs_sums - sum |products|| <= err
    elementwise, err = gamma_hidden(2^-53) * abs_sums * (1 + gamma) (the
    worst case for any order of n float64 additions of exact products)."""
    z = np.ascontiguousarray(z, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    hidden = z.shape[1]
    assert W.shape[1] == hidden

    def decode(bits):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    zd, wd = decode(z), decode(W)
    sums = zd @ wd.T
    abs_sums = np.abs(zd) @ np.abs(wd).T
    g = hidden * 2.0 ** -53 / (1.0 - hidden * 2.0 ** -53)
    return sums, abs_sums, g * abs_sums * (1.0 + g)
