"""Shared helpers for the tests: row specs, single-row runs of the oracle and
an independent PyTorch CPU version of the unfused chain."""
from __future__ import annotations

import numpy as np
import torch

from speculative_decoding_draft_02_amd import workloads as W

HEAD_DIM = 128


def bf16_bits(values) -> np.ndarray:
    return W.to_bf16_bits(np.asarray(values, dtype=np.float64))


def bits_to_f32(codes: np.ndarray) -> np.ndarray:
    return (np.asarray(codes, dtype=np.uint32) << 16).view(np.float32)


def row_from_spec(spec, n=HEAD_DIM, dtype=float):
    row = np.full(n, spec.get("all", 0), dtype=dtype)
    for k, v in (spec.get("at") or {}).items():
        row[int(k)] = v
    return row


def run_oracle_rows(oracle, k_rows, v_rows, w_rows, positions, rotary_dim, cos_sin=None,
                    eps=1e-6, fp8=False, k_scale=1.0, v_scale=1.0, block_size=1,
                    slots=None, num_blocks=None):
    """Write N tokens of one layer and one head, token t at slot t (or
    ``slots``), and return (K codes [N,128], V codes [N,128], result)."""
    k_rows = np.atleast_2d(np.asarray(k_rows, dtype=np.uint16))
    v_rows = np.atleast_2d(np.asarray(v_rows, dtype=np.uint16))
    N = k_rows.shape[0]
    all_kv = np.stack([k_rows, v_rows], axis=1)[:, None, :, None, :]  # [N,1,2,1,128]
    w = np.asarray(w_rows, dtype=np.uint16).reshape(1, HEAD_DIM)
    pos = np.asarray(positions, dtype=np.int64).reshape(N)
    if cos_sin is None:
        cos_sin = W.rope_table(int(pos.max()) + 1, rotary_dim)
    slots = np.arange(N, dtype=np.int64) if slots is None else np.asarray(slots, np.int64)
    nb = num_blocks if num_blocks is not None else (N + block_size - 1) // block_size
    dt = np.uint8 if fp8 else np.uint16
    cache = np.full((nb, 1, block_size, 256), 0xFF if fp8 else 0xFFFF, dtype=dt)
    res = oracle.ctx_kv_write(all_kv, w, eps, pos, cos_sin, rotary_dim, slots, [cache],
                              fp8, np.array([k_scale], np.float32),
                              np.array([v_scale], np.float32))
    rows = cache.reshape(-1, 256)
    sel = slots[slots >= 0]
    return rows[sel, :128], rows[sel, 128:], res


def compact_blocks(wl: W.Workload) -> W.Workload:
    """The same workload with its used cache blocks renumbered 0..n-1, so the
    host caches hold only blocks that some slot touches (same values, same
    in-block offsets; keeps CPU-side tests small)."""
    import dataclasses
    s = wl.slot_mapping
    blocks = np.unique(s[s >= 0] // wl.block_size)
    remap = {int(b): i for i, b in enumerate(blocks)}
    flat = np.array([remap[int(x) // wl.block_size] * wl.block_size + int(x) % wl.block_size
                     if x >= 0 else -1 for x in s.reshape(-1)], np.int64)
    return dataclasses.replace(wl, slot_mapping=flat.reshape(s.shape), num_blocks=max(len(blocks), 1))


# ------------------------------------------------------------------------
# The unfused chain on the CPU with PyTorch library ops in fp32, written from
# the list of steps the fused write replaces (vLLM API page
# "vllm.models.minimax_m3.common.ops.dspark_context_kv", module docstring):
# permute copy, per-layer K norm + stack, positions.repeat, rotary_embedding
# (NeoX), per-layer reshape_and_cache_flash.  It is an independent second
# implementation used to cross-check the oracle, not the oracle itself.

def torch_unfused(wl: W.Workload):
    kv = torch.from_numpy(wl.all_kv.view(np.int16)).view(torch.bfloat16)  # [N,L,2,H,D]
    N, L, _, H, D = kv.shape
    R = wl.rotary_dim
    all_k = kv[:, :, 0].permute(1, 0, 2, 3).contiguous()          # [L,N,H,D]
    all_v = kv[:, :, 1].permute(1, 0, 2, 3).contiguous()
    w = torch.from_numpy(wl.k_norm_weight.view(np.int16)).view(torch.bfloat16).float()
    normed = []
    for l in range(L):
        x = all_k[l].float()
        var = x.pow(2).mean(dim=-1, keepdim=True)
        normed.append((x * torch.rsqrt(var + wl.eps) * (1.0 + w[l])).to(torch.bfloat16))
    k = torch.stack(normed)                                        # [L,N,H,D]
    pos = torch.from_numpy(wl.positions).repeat(L)                 # [L*N]
    cs = torch.from_numpy(wl.cos_sin.view(np.int16)).view(torch.bfloat16)
    cos = cs[pos, : R // 2].float().view(L, N, 1, R // 2)
    sin = cs[pos, R // 2:].float().view(L, N, 1, R // 2)
    x1 = k[..., : R // 2].float()
    x2 = k[..., R // 2: R].float()
    o1 = (x1 * cos - x2 * sin).to(torch.bfloat16)
    o2 = (x2 * cos + x1 * sin).to(torch.bfloat16)
    k = torch.cat([o1, o2, k[..., R:]], dim=-1)
    caches = wl.new_host_caches()
    all_slots = torch.from_numpy(wl.slot_mapping)
    for l in range(L):
        # per-layer reshape_and_cache_flash: layer l's own mapping if given
        slots = all_slots[l] if all_slots.dim() == 2 else all_slots
        valid = torch.nonzero(slots >= 0).flatten()
        s = slots[valid]
        blk, off = s // wl.block_size, s % wl.block_size
        kk, vv = k[l, valid], all_v[l, valid]                      # [V,H,D]
        if wl.fp8:
            kq = (kk.float() / float(wl.k_scales[l])).clamp(-448.0, 448.0)
            vq = (vv.float() / float(wl.v_scales[l])).clamp(-448.0, 448.0)
            kb = kq.to(torch.float8_e4m3fn).view(torch.uint8)
            vb = vq.to(torch.float8_e4m3fn).view(torch.uint8)
            flat = torch.from_numpy(caches[l].reshape(-1, 256))
        else:
            kb = kk.view(torch.int16)
            vb = vv.view(torch.int16)
            flat = torch.from_numpy(caches[l].view(np.int16).reshape(-1, 256))
        for h in range(H):
            rows = (blk * H + h) * wl.block_size + off
            flat[rows, :128] = kb[:, h]
            flat[rows, 128:] = vb[:, h]
    return caches


# ------------------------------------------------------------------------
# The draft block's QK-norm / RoPE / KV insert, written independently with
# PyTorch CPU ops in fp32 from its description on the vLLM API page
# "vllm.models.minimax_m3.common.dspark" (dspark_qknorm_rope_kv_insert): the
# per-head Gemma RMSNorm of the query heads (q weight) and key heads (k
# weight), rounded to bf16; NeoX RoPE on the leading R dims, rounded to bf16;
# the key and value heads of every token with slot >= 0 stored as
# reshape_and_cache_flash would; the rotated queries as e4m3 of q / q_scale.

def torch_insert(wl):
    """Returns (qkv uint16 [T, W], cache or None, q_fp8 uint8 or None)."""
    T, H, nkv, R = wl.num_tokens, wl.num_heads, wl.num_kv_heads, wl.rotary_dim
    x = torch.from_numpy(wl.qkv.view(np.int16)).view(torch.bfloat16).view(T, H + 2 * nkv, HEAD_DIM)
    qw = torch.from_numpy(wl.q_norm_weight.view(np.int16)).view(torch.bfloat16).float()
    kw = torch.from_numpy(wl.k_norm_weight.view(np.int16)).view(torch.bfloat16).float()

    def norm(h, w):
        hf = h.float()
        var = hf.pow(2).mean(dim=-1, keepdim=True)
        return (hf * torch.rsqrt(var + wl.eps) * (1.0 + w)).to(torch.bfloat16)

    cs = torch.from_numpy(wl.cos_sin.view(np.int16)).view(torch.bfloat16)
    pos = torch.from_numpy(wl.positions)
    cos = cs[pos, : R // 2].float().view(T, 1, R // 2)
    sin = cs[pos, R // 2:].float().view(T, 1, R // 2)

    def rope(y):
        x1, x2 = y[..., : R // 2].float(), y[..., R // 2: R].float()
        return torch.cat([(x1 * cos - x2 * sin).to(torch.bfloat16),
                          (x2 * cos + x1 * sin).to(torch.bfloat16), y[..., R:]], dim=-1)

    q = rope(norm(x[:, :H], qw))
    k = rope(norm(x[:, H:H + nkv], kw))
    v = x[:, H + nkv:]
    out = torch.cat([q, k, v], dim=1).reshape(T, -1).view(torch.int16).numpy().view(np.uint16).copy()

    def e4m3(t, s):
        return (t.float() / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)

    qf = e4m3(q, wl.q_scale).reshape(T, -1).numpy().copy() if wl.q_fp8 else None
    cache = None
    if wl.slot_mapping is not None:
        cache = wl.new_host_cache()
        slots = torch.from_numpy(wl.slot_mapping)
        valid = torch.nonzero(slots >= 0).flatten()
        s = slots[valid]
        blk, off = s // wl.block_size, s % wl.block_size
        if wl.fp8:
            kb, vb = e4m3(k[valid], wl.k_scale), e4m3(v[valid], wl.v_scale)
            flat = torch.from_numpy(cache.reshape(-1, 256))
        else:
            kb, vb = k[valid].view(torch.int16), v[valid].view(torch.int16)
            flat = torch.from_numpy(cache.view(np.int16).reshape(-1, 256))
        for h in range(nkv):
            rows = (blk * nkv + h) * wl.block_size + off
            flat[rows, :128] = kb[:, h]
            flat[rows, 128:] = vb[:, h]
    return out, cache, qf


def run_insert_oracle(oracle, wl, **kw):
    cache = wl.new_host_cache() if wl.slot_mapping is not None else None
    return oracle.qknorm_rope_kv_insert(
        wl.qkv, wl.num_heads, wl.num_kv_heads, wl.q_norm_weight, wl.k_norm_weight, wl.eps,
        wl.positions, wl.cos_sin, wl.rotary_dim, slot_mapping=wl.slot_mapping, cache=cache,
        fp8=wl.fp8, k_scale=wl.k_scale, v_scale=wl.v_scale, want_q_fp8=wl.q_fp8,
        q_scale=wl.q_scale, **kw)


# ------------------------------------------------------------------------
# A third implementation of the write, in numpy float32 arithmetic written
# out literally: the 128-term sum of squares added sequentially in fp32,
# rsqrt as 1 / sqrt in fp32, the products and RoPE terms each rounded to
# fp32, then bf16 (and e4m3 of the fp32 quotient for fp8 caches).

def numpy_f32_write(wl):
    f32 = np.float32
    N, L, _, H, D = wl.all_kv.shape
    R = wl.rotary_dim
    k = bits_to_f32(wl.all_kv[:, :, 0]).astype(f32)               # [N, L, H, D]
    v = wl.all_kv[:, :, 1]
    w = bits_to_f32(wl.k_norm_weight).astype(f32)                 # [L, D]
    ss = np.zeros((N, L, H), f32)
    for i in range(D):                                            # sequential fp32 sum
        ss = (ss + k[..., i] * k[..., i]).astype(f32)
    r = (f32(1.0) / np.sqrt((ss / f32(D) + f32(wl.eps)).astype(f32))).astype(f32)
    xr = (k * r[..., None]).astype(f32)
    y = bits_to_f32(bf16_bits((xr * (f32(1.0) + w[None, :, None, :])).astype(f32))).astype(f32)
    cs = bits_to_f32(wl.cos_sin[wl.positions]).astype(f32)        # [N, R]
    c = cs[:, None, None, : R // 2]
    s = cs[:, None, None, R // 2:]
    a, b = y[..., : R // 2], y[..., R // 2: R]
    out = y.copy()
    out[..., : R // 2] = bits_to_f32(bf16_bits((a * c - b * s).astype(f32)))
    out[..., R // 2: R] = bits_to_f32(bf16_bits((b * c + a * s).astype(f32)))
    kb = bf16_bits(out)                                           # [N, L, H, D] codes
    caches = wl.new_host_caches()
    slots = wl.slot_mapping
    for l in range(L):
        sl = slots[l] if slots.ndim == 2 else slots
        for t in np.flatnonzero(sl >= 0):
            blk, off = sl[t] // wl.block_size, sl[t] % wl.block_size
            for h in range(H):
                row = caches[l][blk, h, off]
                if wl.fp8:
                    kq = torch.from_numpy(np.clip(bits_to_f32(kb[t, l, h]) / f32(wl.k_scales[l]),
                                                  -448, 448).astype(f32))
                    vq = torch.from_numpy(np.clip(bits_to_f32(v[t, l, h]) / f32(wl.v_scales[l]),
                                                  -448, 448).astype(f32))
                    row[:128] = kq.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                    row[128:] = vq.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                else:
                    row[:128] = kb[t, l, h]
                    row[128:] = v[t, l, h]
    return caches
