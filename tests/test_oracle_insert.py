"""Pins of the oracle's draft-block QK-norm / RoPE / KV insert against what
the vLLM API page "vllm.models.minimax_m3.common.dspark"
(dspark_qknorm_rope_kv_insert) and the mathematics fix: an independent
PyTorch composite of the op, the context write's (separately pinned) per-row
result for the same heads, closed forms, invariants and planted mistakes."""
import numpy as np
import pytest

from oracle import compare as C
from speculative_decoding_draft_02_amd import workloads as W
from tests._util import bf16_bits, run_insert_oracle, torch_insert

HEAD_DIM = 128

SWEEP = [
    # (T, H, nkv, R, bs, blocks, fp8 cache, q fp8, insert, pad)
    (1, 1, 1, 16, 1, 2, False, False, True, 0.0),      # 3 heads per token: not a multiple of 4
    (7, 4, 2, 64, 16, 2, False, True, True, 0.15),
    (7, 4, 2, 32, 4, 4, True, True, True, 0.0),
    (14, 8, 2, 64, 8, 4, True, False, True, 0.3),
    (5, 3, 1, 16, 2, 8, True, True, True, 0.2),        # 5 heads per token
    (9, 2, 1, 64, 16, 1, False, True, False, 0.0),     # no insert
    (6, 2, 2, 32, 2, 4, False, False, True, 1.0),      # every slot is padding
    (21, 6, 3, 64, 4, 8, True, True, True, 0.1),
]


def _ids(s):
    return "T%d-H%d-kv%d-R%d-bs%d-%s%s%s" % (s[0], s[1], s[2], s[3], s[4], "fp8" if s[6] else "bf16",
                                            "-qfp8" if s[7] else "", "" if s[8] else "-noins")


def _custom(shape, seed):
    T, H, nkv, R, bs, nb, fp8, qf, ins, pad = shape
    return W.insert_custom(T, H, nkv, R, bs, nb, fp8, qf, seed=seed, pad_fraction=pad,
                           std=4.0 if fp8 else 1.0, insert=ins)


@pytest.mark.parametrize("shape", SWEEP, ids=_ids)
def test_oracle_insert_vs_torch_composite(oracle_lib, shape):
    wl = _custom(shape, seed=hash(shape) % 1000)
    qkv, cache, qf = torch_insert(wl)
    res = run_insert_oracle(oracle_lib, wl)
    rep = C.compare_insert(qkv, cache, qf, res, wl.num_heads, wl.num_kv_heads,
                           wl.slot_mapping, wl.fp8, wl.sentinel)
    assert rep.failures == 0, rep.totals()
    assert (res.cache is None) == (wl.slot_mapping is None)
    assert (res.q_fp8 is None) == (not wl.q_fp8)


@pytest.mark.parametrize("index", [0, 1, 2])
def test_oracle_insert_vs_torch_composite_workloads(oracle_lib, index):
    wl = W.insert_make(index)
    qkv, cache, qf = torch_insert(wl)
    res = run_insert_oracle(oracle_lib, wl)
    rep = C.compare_insert(qkv, cache, qf, res, wl.num_heads, wl.num_kv_heads,
                           wl.slot_mapping, wl.fp8, wl.sentinel)
    tot = rep.totals()
    assert rep.failures == 0, tot
    assert tot["q"]["exact"] >= 0.99 * tot["q"]["n"]
    assert tot["k"]["exact"] >= 0.99 * tot["k"]["n"]


def test_oracle_insert_equals_context_write_rows(oracle_lib):
    """Each query head is what the context write makes of it as a K row with
    the q weight, each key head likewise with the k weight, and the stored
    rows are that write's rows: the insert only adds head bookkeeping."""
    wl = W.insert_custom(6, 3, 2, 32, 4, 4, True, True, seed=5, pad_fraction=0.2)
    res = run_insert_oracle(oracle_lib, wl)
    T, H, nkv = wl.num_tokens, wl.num_heads, wl.num_kv_heads
    x = wl.qkv.reshape(T, H + 2 * nkv, HEAD_DIM)
    out = res.qkv.reshape(T, H + 2 * nkv, HEAD_DIM)
    qf = res.q_fp8.reshape(T, H, HEAD_DIM)
    for heads, w, scale, kind in ((range(H), wl.q_norm_weight, wl.q_scale, "q"),
                                  (range(H, H + nkv), wl.k_norm_weight, wl.k_scale, "k")):
        for hh in heads:
            # one layer, one kv head: K row = this head, V row = the token's value head
            vh = H + nkv + (hh - H if kind == "k" else 0)
            all_kv = np.stack([x[:, hh], x[:, vh]], axis=1)[:, None, :, None, :]
            for fp8 in (False, True):
                ref = [np.full((T, 1, 1, 256), 0xFF if fp8 else 0xFFFF,
                               np.uint8 if fp8 else np.uint16)]
                oracle_lib.ctx_kv_write(all_kv, w.reshape(1, HEAD_DIM), wl.eps, wl.positions,
                                        wl.cos_sin, wl.rotary_dim, np.arange(T), ref, fp8,
                                        np.array([scale], np.float32),
                                        np.array([wl.v_scale], np.float32))
                rows = ref[0].reshape(T, 256)
                if not fp8:
                    assert np.array_equal(out[:, hh], rows[:, :128]), (kind, hh)
                elif kind == "q":
                    assert np.array_equal(qf[:, hh], rows[:, :128]), hh
                else:
                    # the cache rows of stored tokens
                    c = res.cache.reshape(-1, 256)
                    for t in np.flatnonzero(wl.slot_mapping >= 0):
                        s = int(wl.slot_mapping[t])
                        r = ((s // wl.block_size) * nkv + (hh - H)) * wl.block_size + s % wl.block_size
                        assert np.array_equal(c[r], rows[t]), (t, hh)
    # value heads are untouched in qkv
    assert np.array_equal(out[:, H + nkv:], x[:, H + nkv:])


def test_oracle_insert_closed_forms(oracle_lib):
    """Constant heads: the norm gives bf16(a / sqrt(a^2 + eps) * (1 + w));
    at a position whose row is cos = 0, sin = 1 (a quarter turn) the rotated
    dims become (-y[i + R/2], y[i]); other dims keep y."""
    R, T, H, nkv = 32, 2, 2, 1
    wl = W.insert_custom(T, H, nkv, R, 4, 2, False, False, seed=1, pad_fraction=0.0)
    qkv = np.zeros((T, (H + 2 * nkv), HEAD_DIM))
    qkv[0, 0, :] = 3.0                              # q head 0: constant 3, w = 0
    ramp = np.linspace(-1.0, 1.0, HEAD_DIM)
    qkv[1, 2, :] = ramp                             # token 1's key head
    qkv[:, 3, :] = 0.75                             # value heads
    wl.qkv = bf16_bits(qkv).reshape(T, -1)
    wl.q_norm_weight = bf16_bits(np.zeros(HEAD_DIM))
    wl.k_norm_weight = bf16_bits(np.full(HEAD_DIM, 0.5))
    cs = np.zeros((2, R))
    cs[0, :R // 2] = 1.0                            # row 0: identity
    cs[1, R // 2:] = 1.0                            # row 1: quarter turn
    wl.cos_sin = bf16_bits(cs)
    wl.positions = np.array([0, 1], np.int64)
    res = run_insert_oracle(oracle_lib, wl)
    out = res.qkv.reshape(T, H + 2 * nkv, HEAD_DIM)
    one = int(bf16_bits([3.0 / np.sqrt(9.0 + 1e-6)])[0])
    assert one == 0x3F80                            # rounds to 1.0
    assert np.all(out[0, 0] == one)
    # token 1 key head: y = bf16(ramp / rms * 1.5), rotated a quarter turn
    bits = bf16_bits(ramp)
    xr = (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)
    y = bf16_bits(xr / np.sqrt(np.mean(xr ** 2) + 1e-6) * 1.5)
    want = y.copy()
    want[:R // 2] = y[R // 2:R] ^ 0x8000
    want[R // 2:R] = y[:R // 2]
    assert np.array_equal(out[1, 2], want)
    # value heads unchanged
    assert np.all(out[:, 3] == bf16_bits([0.75])[0])


def test_oracle_insert_q_fp8_is_the_scaled_rounding(oracle_lib):
    """Every q fp8 code is the e4m3 value nearest q / q_scale (saturating at
    448), checked by decoding against all 127 non-negative e4m3 values."""
    wl = W.insert_custom(7, 4, 2, 64, 16, 2, False, True, seed=9, pad_fraction=0.0)
    res = run_insert_oracle(oracle_lib, wl)
    T, H = wl.num_tokens, wl.num_heads
    q = res.qkv.reshape(T, -1)[:, :H * HEAD_DIM]
    qv = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    target = np.clip(qv / np.float64(np.float32(wl.q_scale)), -448.0, 448.0)
    grid = np.array([oracle_lib.e4m3_decode(c) for c in range(0x7F)])     # +0 .. 448
    got = np.array([oracle_lib.e4m3_decode(int(c)) for c in res.q_fp8.reshape(-1)])
    best = np.abs(np.abs(target.reshape(-1))[:, None] - grid[None, :]).min(axis=1)
    assert np.all(np.abs(np.abs(got) - np.abs(target.reshape(-1))) <= best + 1e-12)
    assert np.all((got == 0) | (np.sign(got) == np.sign(target.reshape(-1))))


def test_oracle_insert_without_slots_leaves_no_cache(oracle_lib):
    wl = W.insert_custom(5, 2, 1, 16, 4, 4, False, False, seed=3, insert=False)
    res = run_insert_oracle(oracle_lib, wl)
    assert res.cache is None and res.q_fp8 is None
    wl2 = W.insert_custom(5, 2, 1, 16, 4, 4, False, False, seed=3, insert=True)
    res2 = run_insert_oracle(oracle_lib, wl2)
    assert np.array_equal(res.qkv, res2.qkv)


def test_insert_acceptance_rule_catches_planted_mistakes(oracle_lib):
    """Mistakes planted in an oracle-side copy of the outputs are reported:
    a q sign flip, a 2-ulp k error, a v bit change in qkv, a stray cache
    write, a cache row with the wrong head, a q fp8 code two steps off."""
    wl = W.insert_custom(8, 4, 2, 32, 4, 8, True, True, seed=11, pad_fraction=0.25, std=4.0)
    res = run_insert_oracle(oracle_lib, wl)
    args = (res, wl.num_heads, wl.num_kv_heads, wl.slot_mapping, wl.fp8, wl.sentinel)
    assert C.compare_insert(res.qkv.copy(), res.cache.copy(), res.q_fp8.copy(), *args).failures == 0
    t = int(np.flatnonzero(wl.slot_mapping >= 0)[0])
    s = int(wl.slot_mapping[t])
    row = ((s // 4) * 2 + 1) * 4 + s % 4
    W_ = (wl.num_heads + 2 * wl.num_kv_heads) * HEAD_DIM
    for mutate in ("q_sign", "k_two_ulp", "v_bit", "stray", "wrong_head", "qfp8"):
        qkv, cache, qf = res.qkv.copy(), res.cache.copy(), res.q_fp8.copy()
        c2 = cache.reshape(-1, 256)
        if mutate == "q_sign":
            qkv[t, 5] ^= 0x8000
            if qkv[t, 5] in (0, 0x8000):
                qkv[t, 5] = 0x4000
        elif mutate == "k_two_ulp":
            qkv[t, 4 * HEAD_DIM + 40] += 2
        elif mutate == "v_bit":
            qkv[t, W_ - 1] ^= 1
        elif mutate == "stray":
            untouched = np.flatnonzero(np.all(c2 == wl.sentinel, axis=1))
            c2[untouched[0], 0] = 0
        elif mutate == "wrong_head":
            c2[row, :128] = c2[row - 4, :128] if c2[row - 4, 0] != wl.sentinel else 0x11
        else:
            qf[t, 3] = qf[t, 3] + 2 if (qf[t, 3] & 0x7F) < 0x7C else qf[t, 3] - 2
        rep = C.compare_insert(qkv, cache, qf, *args)
        assert rep.failures > 0, mutate
