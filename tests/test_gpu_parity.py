"""Parity of the HIP context-KV write (through the C ABI) with the oracle, on
MI355X.  Acceptance rule: oracle/compare.py (V bit-exact in bf16 caches, K
within 1 bf16 ulp of the oracle's code or a near-tie alternate, fp8 within
one e4m3 step, every other byte untouched)."""
import json

import numpy as np
import pytest
import torch

from oracle import compare as C
from speculative_decoding_draft_02_amd import workloads as W
from speculative_decoding_draft_02_amd.writer import AttnLayer, DSparkContextKVWriter

from _device import DeviceInputs, cache_codes, make_layers, run_device, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch


def _check(oracle_lib, wl, reverse=False, label=""):
    print("case", label or wl.name, flush=True)
    dev = run_device(wl, reverse=reverse)
    ref = run_oracle(oracle_lib, wl)
    rep = C.compare(dev, ref, wl.slot_mapping, wl.fp8, wl.sentinel)
    tot = rep.totals()
    print(label or wl.name, json.dumps(tot), "alternates", int(ref.alt_index.size), flush=True)
    assert rep.failures == 0, rep.summary()
    return tot


@pytest.mark.parametrize("index", range(5), ids=W.NAMES)
def test_workload_parity(oracle_lib, index):
    wl = W.make(index)
    tot = _check(oracle_lib, wl)
    # V is a bit copy (bf16) or an exact fp32 division + RNE (fp8)
    assert tot["v"]["exact"] == tot["v"]["n"]


@pytest.mark.parametrize("rank", [0, 3])
def test_head_shard_parity(oracle_lib, rank):
    """One rank's share of the 4096-token bf16 prefill under 4-way head
    parallelism (2 of 8 kv heads, the general row mapping), at full size."""
    wl = W.head_shard(W.make(1), 4, rank)
    tot = _check(oracle_lib, wl)
    assert tot["v"]["exact"] == tot["v"]["n"]


SWEEP = [
    # N, L, nkv, R, bs, blocks, fp8, pad
    (1, 1, 1, 16, 1, 1, False, 0.0),
    (1, 1, 1, 64, 1, 1, True, 0.0),
    (7, 2, 3, 32, 2, 8, False, 0.3),
    (65, 3, 1, 64, 16, 8, True, 0.1),
    (65, 3, 8, 16, 128, 2, False, 0.1),
    (300, 5, 8, 64, 64, 16, True, 0.05),
    (300, 5, 2, 32, 16, 32, False, 0.5),
    (129, 8, 4, 16, 4, 64, True, 0.2),
    (50, 9, 2, 64, 8, 16, False, 0.1),      # L > 8: two passes over the layer groups
    (50, 12, 3, 32, 1, 64, True, 0.1),
    (33, 4, 5, 64, 32, 4, False, 0.0),
    (257, 6, 7, 16, 2, 200, True, 0.25),
    (16, 2, 2, 32, 16, 1, False, 1.0),      # every token is padding
    # larger writes: the general mapping (every layer of a row group in one
    # wave, chunked for L > 8) and uniform fp8 rows
    (2100, 3, 3, 16, 16, 200, False, 0.2),
    (3200, 9, 2, 64, 8, 512, False, 0.1),   # L > 8 in chunks
    (4200, 12, 3, 32, 4, 1200, True, 0.1),  # L > 8 in chunks, fp8
    (3300, 4, 4, 64, 16, 256, True, 0.05),  # uniform rows, fp8: groups of 2 layers
    (3300, 3, 4, 32, 16, 256, True, 0.05),  # uniform rows, fp8, L = 3: one wave per row group
    # one token per wave beyond 16384 waves: bf16 in one wave per row group
    # (L = 2) and in groups of 3 layers (L = 9)
    (4200, 2, 16, 32, 16, 300, False, 0.1),
    (8200, 9, 8, 64, 16, 520, False, 0.02),
]


@pytest.mark.parametrize("shape", SWEEP, ids=lambda s: "N%d-L%d-H%d-R%d-bs%d-%s-pad%.2f" % (
    s[0], s[1], s[2], s[3], s[4], "fp8" if s[6] else "bf16", s[7]))
def test_sweep_parity(oracle_lib, shape):
    N, L, nkv, R, bs, nb, fp8, pad = shape
    wl = W.custom(N, L, nkv, R, bs, nb, fp8, seed=17 * N + L, pad_fraction=pad,
                  kv_std=4.0 if fp8 else 1.0)
    _check(oracle_lib, wl, reverse=(L % 2 == 1))


# the largest supported shapes: DSPARK_MAX_LAYERS layers (one wave per
# layer, groups of two (fp8) or three (bf16) layers per wave, and whole row groups per wave in
# chunks of 8 layers), many kv heads, a large block
MAX_CASES = [
    # N, L, nkv, R, bs, blocks, fp8, pad
    (40, 32, 2, 64, 16, 4, False, 0.1),     # per-layer split
    (40, 32, 2, 32, 16, 4, True, 0.1),
    (1600, 32, 4, 16, 64, 32, False, 0.05),  # 1600 waves, bf16: one layer per wave
    (1600, 32, 4, 16, 64, 32, True, 0.05),   # ... fp8: sixteen groups of 2 layers
    (3200, 32, 2, 32, 64, 64, False, 0.05),  # general mapping, 1600 waves: chunks of 8
    (50, 2, 64, 64, 16, 8, True, 0.1),      # 64 kv heads
    (300, 2, 2, 32, 2048, 2, False, 0.1),   # 2048-token blocks
]


@pytest.mark.parametrize("shape", MAX_CASES, ids=lambda s: "N%d-L%d-H%d-R%d-bs%d-%s" % (
    s[0], s[1], s[2], s[3], s[4], "fp8" if s[6] else "bf16"))
def test_maximum_shapes(oracle_lib, shape):
    N, L, nkv, R, bs, nb, fp8, pad = shape
    wl = W.custom(N, L, nkv, R, bs, nb, fp8, seed=N + L + nkv, pad_fraction=pad,
                  kv_std=4.0 if fp8 else 1.0)
    _check(oracle_lib, wl, reverse=(L == 32), label="max")


def test_maximum_layers_with_per_layer_slots(oracle_lib):
    wl = W.custom(200, 32, 2, 32, 16, 32, True, seed=12, pad_fraction=0.05, kv_std=4.0)
    wl = W.per_layer_slots(wl, seed=13, pad_fraction=0.1)
    _check(oracle_lib, wl, label="max-layer-slots")


def test_layers_allocated_in_reverse_order(oracle_lib):
    """Negative per-layer cache offsets (layer 0 allocated last)."""
    wl = W.custom(200, 5, 4, 64, 16, 64, False, seed=5, pad_fraction=0.1)
    _check(oracle_lib, wl, reverse=True, label="reverse")


@pytest.mark.parametrize("scale", [0.05, 0.3, 1.0, 1.0 / 448.0])
def test_fp8_store_every_bf16_value(oracle_lib, scale):
    """Every finite bf16 bit pattern as V, through the e4m3 store at one scale:
    the device's division + clamp + conversion must give the oracle's code."""
    codes = np.arange(65536, dtype=np.uint32)
    finite = codes[((codes >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    n = (finite.size + 127) // 128
    v = np.zeros(n * 128, np.uint16)
    v[:finite.size] = finite
    wl = W.custom(n, 1, 1, 16, 1, n, True, seed=1, pad_fraction=0.0)
    wl.all_kv[:, 0, 1, 0, :] = v.reshape(n, 128)
    wl.v_scales[:] = np.float32(scale)
    wl.slot_mapping[:] = np.arange(n)
    dev = run_device(wl)
    ref = run_oracle(oracle_lib, wl)
    got = dev[0].reshape(n, 256)[:, 128:]
    want = ref.caches[0].reshape(n, 256)[:, 128:]
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    print("scale", scale, "mismatches", bad.size, flush=True)
    assert bad.size == 0, [(hex(int(v[i])), hex(int(got.reshape(-1)[i])), hex(int(want.reshape(-1)[i])))
                           for i in bad[:10]]


def test_fp8_k_saturates(oracle_lib):
    wl = W.custom(64, 2, 2, 64, 16, 8, True, seed=2, pad_fraction=0.0)
    wl.k_scales[:] = np.float32(1.0 / 448.0)
    _check(oracle_lib, wl, label="k_saturates")
    dev = run_device(wl)
    k = np.concatenate([c.reshape(-1, 256)[:, :128].reshape(-1) for c in dev])
    k = k[k != 0xFF]
    # the norm output has RMS ~1, so about a third of K exceeds 1 = 448 * k_scale
    assert np.count_nonzero((k & 0x7F) == 0x7E) > 0.2 * k.size


def test_num_ctx_zero():
    wl = W.custom(0, 2, 2, 32, 16, 4, False, seed=1, pad_fraction=0.0)
    layers = make_layers(wl)
    writer = DSparkContextKVWriter(layers)
    DeviceInputs(wl).call(writer)
    torch.cuda.synchronize()
    for a in layers:
        assert np.all(cache_codes(a.kv_cache) == 0xFFFF)


def test_graph_capture_replays_match_eager(oracle_lib):
    """A write captured in a HIP graph: replays (with eager work and cache
    resets between them) each give the eager result; a changed scale value
    is read at replay time."""
    wl = W.make(4)
    wl2 = W.custom(100, 5, 4, 16, 128, 512, True, seed=9, pad_fraction=0.25)
    # 1700 fp8 waves: the launch with groups of two layers per wave
    wl3 = W.custom(1700, 5, 4, 32, 128, 512, True, seed=10, pad_fraction=0.05)
    for w in (wl, wl2, wl3):
        print("case graph", w.name, w.fp8, flush=True)
        layers = make_layers(w)
        writer = DSparkContextKVWriter(layers)
        inp = DeviceInputs(w)
        inp.call(writer)                      # eager (also builds the tables)
        torch.cuda.synchronize()
        eager = [cache_codes(a.kv_cache) for a in layers]
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                inp.call(writer)
        torch.cuda.synchronize()
        for rep in range(4):
            for a in layers:
                a.kv_cache.view(torch.uint8).fill_(0xFF)
            junk = torch.randn(1 << 20, device="cuda:0").sum()  # unrelated eager work
            g.replay()
            torch.cuda.synchronize()
            for l, a in enumerate(layers):
                assert np.array_equal(cache_codes(a.kv_cache), eager[l]), (rep, l)
        if w.fp8:
            # scale values are dereferenced on the device at every replay
            for a in layers:
                a._v_scale.mul_(2.0)
            w.v_scales[:] = w.v_scales * 2
            for a in layers:
                a.kv_cache.fill_(0xFF)
            g.replay()
            torch.cuda.synchronize()
            ref = run_oracle(oracle_lib, w)
            rep = C.compare([cache_codes(a.kv_cache) for a in layers], ref, w.slot_mapping,
                            True, w.sentinel)
            assert rep.failures == 0, rep.totals()
        del g
        writer.close()


def test_rebind_rebuilds_tables(oracle_lib):
    wl = W.custom(40, 3, 2, 64, 16, 8, False, seed=12, pad_fraction=0.1)
    layers = make_layers(wl)
    writer = DSparkContextKVWriter(layers)
    inp = DeviceInputs(wl)
    inp.call(writer)
    torch.cuda.synchronize()
    first = [cache_codes(a.kv_cache) for a in layers]
    # re-bind: new cache allocations for every layer
    old = [a.kv_cache for a in layers]
    for a in layers:
        a.kv_cache = torch.full_like(a.kv_cache.view(torch.int16), -1).view(torch.bfloat16)
    inp.call(writer)
    torch.cuda.synchronize()
    for l, a in enumerate(layers):
        assert np.array_equal(cache_codes(a.kv_cache), first[l])
    del old


def test_error_paths():
    wl = W.custom(8, 2, 2, 32, 16, 4, False, seed=3, pad_fraction=0.0)
    layers = make_layers(wl)
    writer = DSparkContextKVWriter(layers)
    inp = DeviceInputs(wl)
    with pytest.raises(RuntimeError, match="rotary_dim 48"):
        writer(inp.all_kv, inp.w, 1e-6, inp.positions,
               torch.zeros(64, 48, dtype=torch.bfloat16, device="cuda:0"), 48, inp.slots)
    with pytest.raises(RuntimeError, match="built for 2 and 2"):
        writer(inp.all_kv[:, :1].contiguous(), inp.w[:1].contiguous(), 1e-6, inp.positions,
               inp.cos_sin, 32, inp.slots)
    with pytest.raises(ValueError, match="all_kv must be"):
        writer(inp.all_kv[..., :64].contiguous(), inp.w, 1e-6, inp.positions, inp.cos_sin, 32,
               inp.slots)
    with pytest.raises(ValueError, match="positions"):
        writer(inp.all_kv, inp.w, 1e-6, inp.positions.to(torch.int32), inp.cos_sin, 32, inp.slots)
    # odd block size and misaligned caches are refused at construction
    bad = [AttnLayer(torch.zeros(4, 2, 12, 256, dtype=torch.bfloat16, device="cuda:0"),
                     layers[0]._k_scale, layers[0]._v_scale)]
    with pytest.raises(ValueError, match="not a power of two"):
        DSparkContextKVWriter(bad)
    big = torch.zeros(2 * 4 * 2 * 16 * 256 + 8, dtype=torch.bfloat16, device="cuda:0")
    c0 = big[:4 * 2 * 16 * 256].view(4, 2, 16, 256)
    c1 = big[4 * 2 * 16 * 256 + 8:].view(4, 2, 16, 256)
    mis = [AttnLayer(c0, layers[0]._k_scale, layers[0]._v_scale),
           AttnLayer(c1, layers[1]._k_scale, layers[1]._v_scale)]
    with pytest.raises(ValueError, match="16-element aligned"):
        DSparkContextKVWriter(mis)
    assert DSparkContextKVWriter.supported(layers)


# ---------------------------------------- positions of padding tokens --
#
# A token stored in no layer never has its position used as a table index,
# so its position may lie off the table: here every such token carries -1 or
# cos_sin_rows, and the caches must equal the oracle's (which reads no
# position of an unstored token) on every launch path.
PADDING_POSITION_CASES = [
    # N, L, nkv, R, bs, blocks, fp8, pad, per-layer mappings
    (300, 5, 8, 64, 64, 16, False, 0.3, False),    # one token per wave, one layer per wave
    (3300, 4, 4, 64, 16, 256, True, 0.2, False),   # one token per wave, fp8 groups of 2
    (8200, 2, 8, 64, 16, 520, False, 0.2, False),  # one token per wave, whole row groups
    (300, 5, 2, 32, 16, 32, False, 0.5, False),    # general mapping, one layer per wave
    (2100, 3, 3, 16, 16, 200, False, 0.3, False),  # general mapping, whole row groups
    (3200, 9, 2, 64, 8, 512, False, 0.1, False),   # general mapping, chunks of 8 layers
    (16, 2, 2, 32, 16, 1, False, 1.0, False),      # every token is padding
    (300, 5, 8, 64, 64, 32, False, 0.3, True),     # per-layer, one layer per wave
    (2100, 9, 8, 32, 16, 140, True, 0.3, True),    # per-layer, fp8 groups of 2
    (8200, 2, 8, 64, 16, 520, False, 0.2, True),   # per-layer, whole row groups
    (129, 3, 2, 16, 4, 80, False, 0.3, True),      # per-layer, general rows
    (2100, 3, 3, 32, 16, 200, True, 0.3, True),    # per-layer, general rows, whole groups
]


@pytest.mark.parametrize("shape", PADDING_POSITION_CASES, ids=lambda s: "N%d-L%d-H%d-%s%s" % (
    s[0], s[1], s[2], "fp8" if s[6] else "bf16", "-layer-slots" if s[8] else ""))
def test_padding_positions_off_the_table(oracle_lib, shape):
    N, L, nkv, R, bs, nb, fp8, pad, per_layer = shape
    wl = W.custom(N, L, nkv, R, bs, nb, fp8, seed=31 * N + L, pad_fraction=pad,
                  kv_std=4.0 if fp8 else 1.0)
    if per_layer:
        wl = W.per_layer_slots(wl, seed=N + 5, pad_fraction=0.1)
    wl = W.padding_positions_off_table(wl)
    off = (wl.positions < 0) | (wl.positions >= wl.cos_sin.shape[0])
    assert off.any() or pad == 0
    _check(oracle_lib, wl, label="padding-positions")


# ------------------------------------------------- per-layer slot mappings --

LAYER_SLOT_CASES = [
    # N, L, nkv, R, bs, blocks, fp8
    (300, 5, 8, 64, 64, 32, False),
    (300, 5, 8, 32, 16, 64, True),
    (129, 3, 2, 16, 4, 80, False),
    (65, 9, 3, 64, 8, 32, True),       # L > 8: chunked pass
    (257, 4, 5, 32, 128, 8, False),
    # beyond the one-layer split: groups of 2 layers (fp8, L = 9) and whole
    # row groups (bf16, L = 2)
    (2100, 9, 8, 32, 16, 140, True),   # more than 4096 waves
    (8200, 2, 8, 64, 16, 520, False),  # more than 16384 waves
]


@pytest.mark.parametrize("shape", LAYER_SLOT_CASES, ids=lambda s: "N%d-L%d-H%d-R%d-bs%d-%s" % (
    s[0], s[1], s[2], s[3], s[4], "fp8" if s[6] else "bf16"))
def test_per_layer_slot_parity(oracle_lib, shape):
    N, L, nkv, R, bs, nb, fp8 = shape
    wl = W.custom(N, L, nkv, R, bs, nb, fp8, seed=7 * N + L, pad_fraction=0.05,
                  kv_std=4.0 if fp8 else 1.0)
    wl = W.per_layer_slots(wl, seed=N + 3, pad_fraction=0.15)
    _check(oracle_lib, wl, label="layer-slots")


def test_per_layer_slot_list_forms():
    """A list of the same tensor takes the shared path; a list of distinct
    tensors and an [L, N] tensor give the same caches."""
    wl = W.per_layer_slots(W.custom(100, 3, 4, 32, 16, 32, False, seed=3, pad_fraction=0.1),
                           seed=4, pad_fraction=0.1)
    outs = []
    for form in ("tensor", "list"):
        layers = make_layers(wl)
        writer = DSparkContextKVWriter(layers)
        inp = DeviceInputs(wl)
        slots = inp.slots if form == "tensor" else [inp.slots[l].clone() for l in range(3)]
        writer(inp.all_kv, inp.w, wl.eps, inp.positions, inp.cos_sin, wl.rotary_dim, slots)
        torch.cuda.synchronize()
        outs.append([cache_codes(a.kv_cache) for a in layers])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    # identical per-layer mappings equal the shared write
    wl2 = W.custom(100, 3, 4, 32, 16, 32, False, seed=5, pad_fraction=0.1)
    res = []
    for form in ("shared", "same-list", "stacked"):
        layers = make_layers(wl2)
        writer = DSparkContextKVWriter(layers)
        inp = DeviceInputs(wl2)
        slots = {"shared": inp.slots, "same-list": [inp.slots] * 3,
                 "stacked": inp.slots.unsqueeze(0).repeat(3, 1).contiguous()}[form]
        writer(inp.all_kv, inp.w, wl2.eps, inp.positions, inp.cos_sin, wl2.rotary_dim, slots)
        torch.cuda.synchronize()
        res.append([cache_codes(a.kv_cache) for a in layers])
    for other in res[1:]:
        for a, b in zip(res[0], other):
            assert np.array_equal(a, b)


def test_debug_checks_refuse_bad_inputs_before_launch(oracle_lib):
    """With debug_checks the writer refuses a shared slot or an out-of-table
    position before any launch (the caches stay untouched), and writes as
    usual otherwise."""
    wl = W.make(0)
    layers = make_layers(wl)
    writer = DSparkContextKVWriter(layers, debug_checks=True)
    x = DeviceInputs(wl)
    bad = x.slots.clone()
    valid = torch.nonzero(bad >= 0).flatten()
    bad[valid[1]] = bad[valid[0]]
    with pytest.raises(ValueError, match="share a slot"):
        writer(x.all_kv, x.w, x.eps, x.positions, x.cos_sin, x.rotary_dim, bad)
    far = x.positions.clone()
    far[valid[0]] = x.cos_sin.shape[0]
    with pytest.raises(ValueError, match="cos/sin table"):
        writer(x.all_kv, x.w, x.eps, far, x.cos_sin, x.rotary_dim, x.slots)
    torch.cuda.synchronize()
    assert all(bool((cache_codes(a.kv_cache) == wl.sentinel).all()) for a in layers)
    x.call(writer)
    torch.cuda.synchronize()
    ref = run_oracle(oracle_lib, wl)
    got = [cache_codes(a.kv_cache) for a in layers]
    assert C.compare(got, ref, wl.slot_mapping, wl.fp8, wl.sentinel).failures == 0
    writer.close()
