"""Seeded synthetic inputs for the DSpark context-KV write.

This module only draws inputs.  It holds none of the write's arithmetic, and
both the device path (tests, bench) and the CPU oracle take their inputs from
it.  Random normals come from numpy's PCG64 bits through an inverse-CDF table of
normal quantiles rounded to bf16 by torch's CPU conversion (a library
routine); the RoPE table is
[cos(p * theta_i) | sin(p * theta_i)] with theta_i = 10000^(-2i/R), computed
in fp64 and rounded to bf16 the same way.

The five workloads follow the shapes of a MiniMax-M3.1 DSpark draft (L = 5
draft layers, 128-dim heads, partial RoPE on 16/32/64 dims; the vLLM API page
"vllm.models.minimax_m3.common.ops.dspark_context_kv") and the serving
situations it is used in: a tiny case, a 4 x 1024-token prefill chunk with
bf16 or fp8 caches, a 32768-token long context, and decode-step batches of
1..8 accepted tokens per request.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch
from scipy.special import ndtri

HEAD_DIM = 128
SENTINEL_BF16 = 0xFFFF   # a NaN pattern: never produced by the write
SENTINEL_FP8 = 0xFF      # the e4m3 NaN pattern S.1111.111


@dataclass
class Workload:
    name: str
    num_ctx: int
    num_layers: int
    num_kv_heads: int
    rotary_dim: int
    block_size: int
    num_blocks: int
    fp8: bool
    eps: float
    all_kv: np.ndarray         # uint16 bf16 bits [num_ctx, L, 2, nkv, 128]
    k_norm_weight: np.ndarray  # uint16 bf16 bits [L, 128]
    positions: np.ndarray      # int64 [num_ctx]
    slot_mapping: np.ndarray   # int64 [num_ctx] (shared) or [L, num_ctx] (per layer), < 0 = padding
    cos_sin: np.ndarray        # uint16 bf16 bits [rows, R] = [cos | sin]
    k_scales: np.ndarray       # float32 [L]
    v_scales: np.ndarray       # float32 [L]

    @property
    def sentinel(self) -> int:
        return SENTINEL_FP8 if self.fp8 else SENTINEL_BF16

    @property
    def cache_shape(self):
        return (self.num_blocks, self.num_kv_heads, self.block_size, 2 * HEAD_DIM)

    @property
    def cache_np_dtype(self):
        return np.uint8 if self.fp8 else np.uint16

    @property
    def valid_tokens(self) -> int:
        """Tokens written (shared mapping), or token-layers written / L."""
        return int(np.count_nonzero(self.slot_mapping >= 0)) // (
            self.num_layers if self.slot_mapping.ndim == 2 else 1)

    def new_host_caches(self):
        return [np.full(self.cache_shape, self.sentinel, dtype=self.cache_np_dtype)
                for _ in range(self.num_layers)]

    def algorithmic_bytes(self) -> int:
        """Bytes the write must move: all_kv rows of valid tokens read, cache
        rows written, the cos/sin row and position of each valid token, every
        slot, and the norm weights.  With per-layer mappings a (token, layer)
        is valid on its own and each token reads its cos/sin row once."""
        L, nkv, R = self.num_layers, self.num_kv_heads, self.rotary_dim
        e = 1 if self.fp8 else 2
        if self.slot_mapping.ndim == 2:
            tl = int(np.count_nonzero(self.slot_mapping >= 0))
            tok = int(np.count_nonzero((self.slot_mapping >= 0).any(axis=0)))
            per_tl = 2 * nkv * HEAD_DIM * 2 + nkv * 2 * HEAD_DIM * e
            return tl * per_tl + tok * (2 * R + 8) + 8 * L * self.num_ctx + L * HEAD_DIM * 2
        v = self.valid_tokens
        per_tok = L * 2 * nkv * HEAD_DIM * 2 + L * nkv * 2 * HEAD_DIM * e + 2 * R + 8
        return v * per_tok + 8 * self.num_ctx + L * HEAD_DIM * 2

    def token_layers(self) -> int:
        if self.slot_mapping.ndim == 2:
            return int(np.count_nonzero(self.slot_mapping >= 0))
        return self.valid_tokens * self.num_layers


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32/fp64 array -> uint16 bf16 bits (round to nearest even), by torch."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rope_table(rows: int, rotary_dim: int, theta: float = 10000.0) -> np.ndarray:
    half = rotary_dim // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / rotary_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv_freq[None, :]
    return to_bf16_bits(np.concatenate([np.cos(ang), np.sin(ang)], axis=1))


_QBITS = 22
_QTABLES = {}


def _normal_table(std):
    """bf16 bits of the N(0, std) quantiles at (i + 1/2) / 2^22, i < 2^22."""
    tab = _QTABLES.get(std)
    if tab is None:
        u = (np.arange(1 << _QBITS, dtype=np.float64) + 0.5) / (1 << _QBITS)
        tab = to_bf16_bits(ndtri(u) * std)
        _QTABLES[std] = tab
    return tab


def _normal_bf16(rng, shape, std):
    """N(0, std) samples as bf16 bits, by inverse CDF: 22 random bits pick one
    of 2^22 equally likely quantiles (the tails beyond 5.17 std are cut).
    Filled in chunks so that no large temporary is created."""
    tab = _normal_table(float(std))
    out = np.empty(shape, np.uint16)
    flat = out.reshape(-1)
    chunk = 1 << 20
    for s in range(0, flat.size, chunk):
        n = min(chunk, flat.size - s)
        raw = rng.bit_generator.random_raw((n + 1) // 2)
        idx = (raw.view(np.uint32)[:n] >> (32 - _QBITS))
        np.take(tab, idx, out=flat[s:s + n])
    return out


def _pad(rng, slots, count):
    if count:
        idx = rng.choice(slots.size, size=count, replace=False)
        slots[idx] = -1
    return slots


NAMES = ["tiny", "prefill_bf16", "prefill_fp8", "long_fp8", "decode_bf16"]

DESCRIPTIONS = [
    "num_ctx=64 L=1 nkv=2 R=64 bs=16 8 blocks bf16 cache, ~10% padding",
    "num_ctx=4096 (4 x 1024) L=5 nkv=8 R=64 bs=64 512 blocks/layer bf16 caches, 2% padding",
    "num_ctx=4096 (4 x 1024) L=5 nkv=8 R=64 bs=64 512 blocks/layer fp8 e4m3 caches, 2% padding",
    "num_ctx=32768 (positions 8192..40959) L=5 nkv=8 R=32 bs=16 4096 blocks/layer fp8 e4m3 caches",
    "decode: 64 requests x 1..8 tokens L=5 nkv=4 R=16 bs=128 512 blocks/layer bf16 caches, 25% padding",
]


def make(index: int, variant: int = 0) -> Workload:
    """Workload ``index`` (0..4, in the order of NAMES).  ``variant`` > 0
    draws an independent input set of the same shape (fresh values, slots
    and positions) for benchmarks that rotate inputs."""
    seed = 1000 + index + 7919 * variant
    rng = np.random.default_rng(seed)
    eps = 1e-6
    if index == 0:
        N, L, nkv, R, bs, nb, fp8 = 64, 1, 2, 64, 16, 8, False
        all_kv = _normal_bf16(rng, (N, L, 2, nkv, HEAD_DIM), 1.0)
        w = _normal_bf16(rng, (L, HEAD_DIM), 0.1)
        ks = np.ones(L, np.float32)
        vs = np.ones(L, np.float32)
        slots = rng.permutation(nb * bs)[:N].astype(np.int64)
        slots = _pad(rng, slots, int(round(0.10 * N)))
        positions = np.arange(N, dtype=np.int64)
        cs = rope_table(4096, R)
    elif index in (1, 2):
        fp8 = index == 2
        reqs, per = 4, 1024
        N, L, nkv, R, bs, nb = reqs * per, 5, 8, 64, 64, 512
        all_kv = _normal_bf16(rng, (N, L, 2, nkv, HEAD_DIM), 4.0 if fp8 else 1.0)
        w = _normal_bf16(rng, (L, HEAD_DIM), 0.1)
        if fp8:
            ks = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
            vs = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
        else:
            ks = np.ones(L, np.float32)
            vs = np.ones(L, np.float32)
        bpr = per // bs
        blocks = rng.permutation(nb)[:reqs * bpr].reshape(reqs, bpr)
        j = np.arange(per, dtype=np.int64)
        slots = np.concatenate([blocks[r][j // bs] * bs + j % bs for r in range(reqs)]).astype(np.int64)
        slots = _pad(rng, slots, int(round(0.02 * N)))
        positions = np.tile(np.arange(per, dtype=np.int64), reqs)
        cs = rope_table(4096, R)
        if fp8:
            # Deterministic saturation probes in V: +-(448 * v_scale) times
            # {0.999, 1, 464/448, 1.2, 3}, at the first valid token, head 0.
            t0 = int(np.flatnonzero(slots >= 0)[0])
            mult = np.array([0.999, 1.0, 464.0 / 448.0, 1.2, 3.0])
            for l in range(L):
                vals = np.concatenate([mult, -mult]) * 448.0 * float(vs[l])
                all_kv[t0, l, 1, 0, :vals.size] = to_bf16_bits(vals.astype(np.float32))
    elif index == 3:
        N, L, nkv, R, bs, nb, fp8 = 32768, 5, 8, 32, 16, 4096, True
        all_kv = _normal_bf16(rng, (N, L, 2, nkv, HEAD_DIM), 1.0)
        w = _normal_bf16(rng, (L, HEAD_DIM), 0.1)
        ks = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
        vs = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
        perm = rng.permutation(nb).astype(np.int64)
        positions = np.arange(8192, 8192 + N, dtype=np.int64)
        slots = perm[positions // bs] * bs + positions % bs
        cs = rope_table(65536, R)
    elif index == 4:
        L, nkv, R, bs, nb, fp8 = 5, 4, 16, 128, 512, False
        reqs = 64
        n_i = rng.integers(1, 9, size=reqs)
        N = int(n_i.sum())
        all_kv = _normal_bf16(rng, (N, L, 2, nkv, HEAD_DIM), 1.0)
        w = _normal_bf16(rng, (L, HEAD_DIM), 0.1)
        ks = np.ones(L, np.float32)
        vs = np.ones(L, np.float32)
        p0 = rng.integers(0, 131072 - 8 + 1, size=reqs)
        free_blocks = list(rng.permutation(nb))
        pos_list, slot_list = [], []
        for r in range(reqs):
            p = np.arange(p0[r], p0[r] + n_i[r], dtype=np.int64)
            logical = p // bs
            first = int(logical[0])
            table = [int(free_blocks.pop()) for _ in range(int(logical[-1]) - first + 1)]
            slot_list.append(np.array([table[int(lb) - first] for lb in logical], np.int64) * bs + p % bs)
            pos_list.append(p)
        positions = np.concatenate(pos_list)
        slots = _pad(rng, np.concatenate(slot_list), int(round(0.25 * N)))
        cs = rope_table(131072, R)
    else:
        raise ValueError("workload index must be 0..4")
    return Workload(NAMES[index], N, L, nkv, R, bs, nb, fp8, eps,
                    np.ascontiguousarray(all_kv), np.ascontiguousarray(w),
                    positions, slots, cs, ks, vs)


def per_layer_slots(wl: Workload, seed: int, pad_fraction: float = 0.05) -> Workload:
    """The same inputs with one slot mapping per layer ([L, num_ctx]): every
    layer places the tokens in its own random blocks (as when the draft's
    layers belong to different KV-cache groups) and pads its own tokens."""
    import dataclasses
    rng = np.random.default_rng(seed)
    L, N, bs, nb = wl.num_layers, wl.num_ctx, wl.block_size, wl.num_blocks
    base = wl.slot_mapping if wl.slot_mapping.ndim == 1 else wl.slot_mapping[0]
    maps = np.empty((L, N), np.int64)
    for l in range(L):
        perm = rng.permutation(nb)
        s = np.where(base >= 0, perm[np.maximum(base, 0) // bs] * bs + np.maximum(base, 0) % bs, -1)
        maps[l] = _pad(rng, s.astype(np.int64), int(round(pad_fraction * N)))
    return dataclasses.replace(wl, slot_mapping=maps)


def padding_positions_off_table(wl):
    """The same inputs with the position of every token that is stored in no
    layer moved off the cos/sin table: -1, rows, -1, rows, ... (rows =
    cos_sin.shape[0]).  Such a position is never used as an index, so the
    result of the write must not change.  Takes a Workload or a
    ProjectWorkload (anything with positions, slot_mapping and cos_sin)."""
    import dataclasses
    stored = wl.slot_mapping >= 0
    if stored.ndim == 2:
        stored = stored.any(axis=0)
    pos = wl.positions.copy()
    idle = np.flatnonzero(~stored)
    pos[idle] = np.where(np.arange(idle.size) % 2 == 0, -1, wl.cos_sin.shape[0])
    return dataclasses.replace(wl, positions=pos)


def head_shard(wl: Workload, tp: int, rank: int) -> Workload:
    """One rank's share under head (tensor) parallelism: kv heads
    [rank * nkv / tp, (rank + 1) * nkv / tp) of every token and layer, written
    into caches that hold only those heads.  Slots, positions, norm weights
    and the cos/sin table are the same on every rank."""
    import dataclasses
    nkv = wl.num_kv_heads
    if tp < 1 or nkv % tp or not 0 <= rank < tp:
        raise ValueError("tp must divide num_kv_heads and 0 <= rank < tp")
    h = nkv // tp
    part = np.ascontiguousarray(wl.all_kv[:, :, :, rank * h:(rank + 1) * h, :])
    return dataclasses.replace(wl, name="%s_tp%d_rank%d" % (wl.name, tp, rank),
                               num_kv_heads=h, all_kv=part)


def relocate_blocks(wl: Workload, seed: int) -> Workload:
    """The same tokens placed in other cache blocks: every block of a shared
    slot mapping is moved by one random permutation of the blocks (offsets in
    a block and padding kept), so requests stay block-contiguous."""
    import dataclasses
    if wl.slot_mapping.ndim != 1:
        raise ValueError("relocate_blocks takes a shared slot mapping")
    perm = np.random.default_rng(seed).permutation(wl.num_blocks)
    s = wl.slot_mapping
    bs = wl.block_size
    moved = np.where(s >= 0, perm[np.maximum(s, 0) // bs] * bs + np.maximum(s, 0) % bs, s)
    return dataclasses.replace(wl, slot_mapping=moved.astype(np.int64))


def custom(num_ctx, num_layers, num_kv_heads, rotary_dim, block_size, num_blocks,
           fp8, seed, pad_fraction=0.1, kv_std=1.0, w_std=0.1, cs_rows=None,
           eps=1e-6) -> Workload:
    """A small workload of arbitrary shape with unique random slots."""
    rng = np.random.default_rng(seed)
    N, L, nkv = num_ctx, num_layers, num_kv_heads
    assert N <= num_blocks * block_size
    all_kv = _normal_bf16(rng, (N, L, 2, nkv, HEAD_DIM), kv_std)
    w = _normal_bf16(rng, (L, HEAD_DIM), w_std)
    if fp8:
        ks = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
        vs = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
    else:
        ks = np.ones(L, np.float32)
        vs = np.ones(L, np.float32)
    slots = rng.permutation(num_blocks * block_size)[:N].astype(np.int64)
    slots = _pad(rng, slots, int(round(pad_fraction * N)))
    rows = cs_rows if cs_rows is not None else max(N, 1) + 64
    positions = rng.integers(0, rows, size=N).astype(np.int64)
    cs = rope_table(rows, rotary_dim)
    return Workload("custom", N, L, nkv, rotary_dim, block_size, num_blocks, fp8, eps,
                    all_kv, w, positions, slots, cs, ks, vs)


# ----------------------------------------------------------------------------
# The draft block's fused QK-norm / RoPE / KV insert: qkv [T, (H + 2 nkv) * 128]
# for T = requests x 7 query rows (the draft block of the vLLM API page
# "vllm.models.minimax_m3.common.dspark"), each request's rows at consecutive
# positions after its context, stored at the slots its block table gives.

DRAFT_ROWS = 7

@dataclass
class InsertWorkload:
    name: str
    num_tokens: int
    num_heads: int
    num_kv_heads: int
    rotary_dim: int
    block_size: int
    num_blocks: int
    fp8: bool                  # fp8 e4m3 cache (else bf16)
    q_fp8: bool                # the e4m3 query output is requested
    eps: float
    qkv: np.ndarray            # uint16 bf16 bits [T, (H + 2 nkv) * 128]
    q_norm_weight: np.ndarray  # uint16 bf16 bits [128]
    k_norm_weight: np.ndarray  # uint16 bf16 bits [128]
    positions: np.ndarray      # int64 [T]
    slot_mapping: np.ndarray | None   # int64 [T] (< 0 = not stored) or None (no insert)
    cos_sin: np.ndarray        # uint16 bf16 bits [rows, R]
    k_scale: float
    v_scale: float
    q_scale: float

    @property
    def heads_per_token(self) -> int:
        return self.num_heads + 2 * self.num_kv_heads

    @property
    def sentinel(self) -> int:
        return SENTINEL_FP8 if self.fp8 else SENTINEL_BF16

    @property
    def cache_shape(self):
        return (self.num_blocks, self.num_kv_heads, self.block_size, 2 * HEAD_DIM)

    def new_host_cache(self) -> np.ndarray:
        return np.full(self.cache_shape, self.sentinel, dtype=np.uint8 if self.fp8 else np.uint16)

    def stored_tokens(self) -> int:
        return 0 if self.slot_mapping is None else int(np.count_nonzero(self.slot_mapping >= 0))

    def algorithmic_bytes(self) -> int:
        """Bytes the op must move: qkv read, its query and key heads written
        back, the stored tokens' K/V cache rows, the q fp8 output, each
        token's cos/sin row, position and slot, and the two norm weights."""
        T, H, nkv, R = self.num_tokens, self.num_heads, self.num_kv_heads, self.rotary_dim
        e = 1 if self.fp8 else 2
        b = T * (self.heads_per_token * HEAD_DIM * 2 + (H + nkv) * HEAD_DIM * 2 + 2 * R + 8)
        if self.slot_mapping is not None:
            b += 8 * T + self.stored_tokens() * 2 * nkv * HEAD_DIM * e
        if self.q_fp8:
            b += T * H * HEAD_DIM
        return b + 2 * HEAD_DIM * 2


INSERT_NAMES = ["insert_tiny", "insert_draft_bf16", "insert_draft_fp8"]

INSERT_DESCRIPTIONS = [
    "3 requests x 7 rows, H=4 nkv=2 R=64 bs=16 8 blocks bf16 cache, q fp8 out, 1 padded row",
    "64 requests x 7 rows (448 tokens), H=32 nkv=8 R=64 bs=64 512 blocks bf16 cache, 2% padding",
    "64 requests x 7 rows (448 tokens), H=32 nkv=8 R=64 bs=64 512 blocks fp8 e4m3 cache "
    "with k/v scales, q fp8 out, 2% padding",
]


def _draft_block(rng, reqs, bs, nb, max_pos):
    """Positions and slots of `reqs` requests' draft rows: request r's rows
    sit at p0_r .. p0_r + 6 and at the slots of its own random blocks."""
    p0 = rng.integers(0, max_pos - DRAFT_ROWS + 1, size=reqs)
    free_blocks = list(rng.permutation(nb))
    pos_list, slot_list = [], []
    for r in range(reqs):
        p = np.arange(p0[r], p0[r] + DRAFT_ROWS, dtype=np.int64)
        logical = p // bs
        first = int(logical[0])
        table = [int(free_blocks.pop()) for _ in range(int(logical[-1]) - first + 1)]
        slot_list.append(np.array([table[int(lb) - first] for lb in logical], np.int64) * bs + p % bs)
        pos_list.append(p)
    return np.concatenate(pos_list), np.concatenate(slot_list)


def insert_make(index: int, variant: int = 0) -> InsertWorkload:
    """Draft-block workload ``index`` (0..2, in the order of INSERT_NAMES)."""
    rng = np.random.default_rng(2000 + index + 7919 * variant)
    if index == 0:
        reqs, H, nkv, R, bs, nb, fp8, qf, std, rows = 3, 4, 2, 64, 16, 8, False, True, 1.0, 4096
    elif index in (1, 2):
        fp8 = index == 2
        reqs, H, nkv, R, bs, nb, qf, std, rows = 64, 32, 8, 64, 64, 512, fp8, 4.0 if fp8 else 1.0, 131072
    else:
        raise ValueError("insert workload index must be 0..2")
    T = reqs * DRAFT_ROWS
    qkv = _normal_bf16(rng, (T, (H + 2 * nkv) * HEAD_DIM), std)
    qw = _normal_bf16(rng, (HEAD_DIM,), 0.1)
    kw = _normal_bf16(rng, (HEAD_DIM,), 0.1)
    positions, slots = _draft_block(rng, reqs, bs, nb, rows)
    slots = _pad(rng, slots, 1 if index == 0 else int(round(0.02 * T)))
    ks, vs, qs = 1.0, 1.0, 1.0
    if fp8:
        ks, vs = (float(np.float32(x)) for x in rng.uniform(0.05, 0.5, size=2))
    if qf:
        qs = float(np.float32(rng.uniform(0.05, 0.5)))
    return InsertWorkload(INSERT_NAMES[index], T, H, nkv, R, bs, nb, fp8, qf, 1e-6, qkv, qw, kw,
                          positions, slots, rope_table(rows, R), ks, vs, qs)


def insert_custom(num_tokens, num_heads, num_kv_heads, rotary_dim, block_size, num_blocks, fp8,
                  q_fp8, seed, pad_fraction=0.1, std=1.0, insert=True, cs_rows=None,
                  eps=1e-6) -> InsertWorkload:
    """A small draft-block workload of arbitrary shape with unique random slots."""
    rng = np.random.default_rng(seed)
    T, H, nkv = num_tokens, num_heads, num_kv_heads
    assert not insert or T <= num_blocks * block_size
    qkv = _normal_bf16(rng, (T, (H + 2 * nkv) * HEAD_DIM), std)
    qw = _normal_bf16(rng, (HEAD_DIM,), 0.1)
    kw = _normal_bf16(rng, (HEAD_DIM,), 0.1)
    rows = cs_rows if cs_rows is not None else max(T, 1) + 64
    positions = rng.integers(0, rows, size=T).astype(np.int64)
    slots = None
    if insert:
        slots = rng.permutation(num_blocks * block_size)[:T].astype(np.int64)
        slots = _pad(rng, slots, int(round(pad_fraction * T)))
    ks, vs = (float(np.float32(x)) for x in rng.uniform(0.05, 0.5, size=2)) if fp8 else (1.0, 1.0)
    qs = float(np.float32(rng.uniform(0.05, 0.5))) if q_fp8 else 1.0
    return InsertWorkload("insert_custom", T, H, nkv, rotary_dim, block_size, num_blocks, fp8,
                          q_fp8, eps, qkv, qw, kw, positions, slots, rope_table(rows, rotary_dim),
                          ks, vs, qs)


# ----------------------------------------------------------------------------
# The step before the write: hidden_norm on the context states and the
# token-major K/V projection (vLLM API page "vllm.models.minimax_m3.common.dspark":
# _normalize_context_states, _project_context_kv_token_major), whose output
# all_kv [N, L, 2, nkv, 128] the write consumes.  W is a linear layer's
# [out, in] weight with out = L * 2 * nkv * 128 in all_kv's column order.

@dataclass
class ProjectWorkload:
    name: str
    num_ctx: int
    hidden: int
    num_layers: int
    num_kv_heads: int
    rotary_dim: int
    block_size: int
    num_blocks: int
    fp8: bool
    eps: float
    states: np.ndarray              # uint16 bf16 bits [N, hidden]
    hidden_norm_weight: np.ndarray  # uint16 bf16 bits [hidden]
    kv_weight: np.ndarray           # uint16 bf16 bits [L * 2 * nkv * 128, hidden]
    k_norm_weight: np.ndarray       # uint16 bf16 bits [L, 128]
    positions: np.ndarray           # int64 [N]
    slot_mapping: np.ndarray        # int64 [N]
    cos_sin: np.ndarray             # uint16 bf16 bits [rows, R]
    k_scales: np.ndarray            # float32 [L]
    v_scales: np.ndarray            # float32 [L]
    normalized: bool = False        # states are already the hidden_norm output

    @property
    def out_features(self) -> int:
        return self.num_layers * 2 * self.num_kv_heads * HEAD_DIM

    def write_workload(self, all_kv_bits: np.ndarray) -> Workload:
        """The context write this projection feeds, with the given all_kv."""
        return Workload(self.name + "_write", self.num_ctx, self.num_layers, self.num_kv_heads,
                        self.rotary_dim, self.block_size, self.num_blocks, self.fp8, self.eps,
                        np.ascontiguousarray(all_kv_bits.reshape(
                            self.num_ctx, self.num_layers, 2, self.num_kv_heads, HEAD_DIM)),
                        self.k_norm_weight, self.positions, self.slot_mapping, self.cos_sin,
                        self.k_scales, self.v_scales)

    def gemm_flops(self) -> int:
        return 2 * self.num_ctx * self.hidden * self.out_features


PROJECT_NAMES = ["project_tiny", "project_prefill_bf16", "project_prefill_fp8"]

PROJECT_DESCRIPTIONS = [
    "N=64 hidden=256 L=2 nkv=2 R=64 bs=16 8 blocks bf16 cache, ~10% padding",
    "N=4096 (4 x 1024) hidden=6144 L=5 nkv=8 R=64 bs=64 512 blocks bf16 caches, 2% padding",
    "N=4096 (4 x 1024) hidden=6144 L=5 nkv=8 R=64 bs=64 512 blocks fp8 e4m3 caches, 2% padding",
]


def _quantized(rng, shape, max_int, exp):
    """Integers uniform in [-max_int, max_int] times 2^exp, as bf16 bits
    (exact: max_int < 256)."""
    k = rng.integers(-max_int, max_int + 1, size=shape).astype(np.float32)
    return to_bf16_bits(k * np.float32(2.0 ** exp))


def project_make(index: int, variant: int = 0) -> ProjectWorkload:
    """Workload ``index`` (0..2, in the order of PROJECT_NAMES)."""
    rng = np.random.default_rng(3000 + index + 7919 * variant)
    if index == 0:
        N, hidden, L, nkv, R, bs, nb, fp8, pad, rows = 64, 256, 2, 2, 64, 16, 8, False, 0.10, 4096
    elif index in (1, 2):
        N, hidden, L, nkv, R, bs, nb, fp8, pad, rows = 4096, 6144, 5, 8, 64, 64, 512, index == 2, 0.02, 4096
    else:
        raise ValueError("project workload index must be 0..2")
    C = L * 2 * nkv * HEAD_DIM
    states = _normal_bf16(rng, (N, hidden), 1.0)
    hw = _normal_bf16(rng, (hidden,), 0.1)
    W = _normal_bf16(rng, (C, hidden), 1.0 / np.sqrt(hidden))
    kw = _normal_bf16(rng, (L, HEAD_DIM), 0.1)
    if fp8:
        ks = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
        vs = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
    else:
        ks = np.ones(L, np.float32)
        vs = np.ones(L, np.float32)
    if index == 0:
        slots = rng.permutation(nb * bs)[:N].astype(np.int64)
        positions = np.arange(N, dtype=np.int64)
    else:
        reqs, per = 4, 1024
        bpr = per // bs
        blocks = rng.permutation(nb)[:reqs * bpr].reshape(reqs, bpr)
        j = np.arange(per, dtype=np.int64)
        slots = np.concatenate([blocks[r][j // bs] * bs + j % bs for r in range(reqs)]).astype(np.int64)
        positions = np.tile(np.arange(per, dtype=np.int64), reqs)
    slots = _pad(rng, slots, int(round(pad * N)))
    return ProjectWorkload(PROJECT_NAMES[index], N, hidden, L, nkv, R, bs, nb, fp8, 1e-6,
                           states, hw, W, kw, positions, slots, rope_table(rows, R), ks, vs)


def project_exact(num_ctx, hidden, num_layers, num_kv_heads, rotary_dim, block_size,
                  num_blocks, fp8, seed, pad_fraction=0.1) -> ProjectWorkload:
    """Normalized states and weights on coarse grids, z = k 2^-5 (|k| <= 63)
    and W = m 2^-9 (|m| <= 31): every product is a multiple of 2^-14 below
    0.12 and every partial sum of up to 8192 terms stays below 1024 = 2^24 *
    2^-14, so fp32 accumulation in any order gives the exact sum."""
    assert hidden <= 8192
    rng = np.random.default_rng(seed)
    N, L, nkv = num_ctx, num_layers, num_kv_heads
    C = L * 2 * nkv * HEAD_DIM
    z = _quantized(rng, (N, hidden), 63, -5)
    W = _quantized(rng, (C, hidden), 31, -9)
    kw = _normal_bf16(rng, (L, HEAD_DIM), 0.1)
    if fp8:
        ks = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
        vs = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
    else:
        ks = np.ones(L, np.float32)
        vs = np.ones(L, np.float32)
    slots = rng.permutation(num_blocks * block_size)[:N].astype(np.int64)
    slots = _pad(rng, slots, int(round(pad_fraction * N)))
    rows = N + 64
    positions = rng.integers(0, rows, size=N).astype(np.int64)
    return ProjectWorkload("project_exact", N, hidden, L, nkv, rotary_dim, block_size, num_blocks,
                           fp8, 1e-6, z, np.zeros(hidden, np.uint16), W, kw, positions, slots,
                           rope_table(rows, rotary_dim), ks, vs, normalized=True)


def project_custom(num_ctx, hidden, num_layers, num_kv_heads, rotary_dim, block_size,
                   num_blocks, fp8, seed, pad_fraction=0.1) -> ProjectWorkload:
    """Gaussian states (taken as the hidden-norm output) and weight of any
    shape: z ~ N(0, 1), W ~ N(0, 1 / hidden), slots unique in the cache,
    positions uniform over a table of num_ctx + 64 rows."""
    rng = np.random.default_rng(seed)
    N, L, nkv = num_ctx, num_layers, num_kv_heads
    C = L * 2 * nkv * HEAD_DIM
    z = _normal_bf16(rng, (N, hidden), 1.0)
    W = _normal_bf16(rng, (C, hidden), 1.0 / np.sqrt(hidden))
    kw = _normal_bf16(rng, (L, HEAD_DIM), 0.1)
    if fp8:
        ks = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
        vs = rng.uniform(0.05, 0.5, size=L).astype(np.float32)
    else:
        ks = np.ones(L, np.float32)
        vs = np.ones(L, np.float32)
    slots = rng.permutation(num_blocks * block_size)[:N].astype(np.int64)
    slots = _pad(rng, slots, int(round(pad_fraction * N)))
    rows = N + 64
    positions = rng.integers(0, rows, size=N).astype(np.int64)
    return ProjectWorkload("project_custom", N, hidden, L, nkv, rotary_dim, block_size, num_blocks,
                           fp8, 1e-6, z, np.zeros(hidden, np.uint16), W, kw, positions, slots,
                           rope_table(rows, rotary_dim), ks, vs, normalized=True)
