"""Parity of the HIP draft-block QK-norm / RoPE / KV insert (through the C ABI)
with the oracle, on MI355X.  Acceptance rule: oracle/compare.py
(compare_insert: query and key heads within 1 bf16 ulp of the oracle's code or
a near-tie alternate, value heads and bf16 V cache rows bit-exact, fp8 within
one e4m3 step, every cache row no slot names untouched)."""
import json
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import compare as C
from speculative_decoding_draft_02_amd import workloads as W
from speculative_decoding_draft_02_amd.qknorm_insert import (dspark_qknorm_rope_kv_insert,
                                                             fused_qknorm_rope_kv_insert)
from tests._util import run_insert_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    arch = torch.cuda.get_device_properties(0).gcnArchName
    assert arch.startswith("gfx950"), arch


def _bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _codes(t):
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Inputs:
    """A workload's inputs on the device, with a sentinel-filled cache and
    q fp8 output."""

    def __init__(self, wl):
        self.wl = wl
        self.qkv = _bf16(wl.qkv)
        self.qw = _bf16(wl.q_norm_weight)
        self.kw = _bf16(wl.k_norm_weight)
        self.cs = _bf16(wl.cos_sin)
        self.pos = torch.from_numpy(wl.positions).to(DEV)
        self.slots = None if wl.slot_mapping is None else torch.from_numpy(wl.slot_mapping).to(DEV)
        self.cache = None
        if wl.slot_mapping is not None:
            if wl.fp8:
                self.cache = torch.full(wl.cache_shape, W.SENTINEL_FP8, dtype=torch.uint8, device=DEV)
            else:
                self.cache = torch.full(wl.cache_shape, -1, dtype=torch.int16,
                                        device=DEV).view(torch.bfloat16)
        self.ks = torch.tensor([wl.k_scale], dtype=torch.float32, device=DEV)
        self.vs = torch.tensor([wl.v_scale], dtype=torch.float32, device=DEV)
        self.qf = None
        if wl.q_fp8:
            self.qf = torch.full((wl.num_tokens, wl.num_heads * 128), 0xFF, dtype=torch.uint8,
                                 device=DEV)

    def call(self, scales=True):
        wl = self.wl
        fused_qknorm_rope_kv_insert(
            self.qkv, self.qw, self.kw, self.cs, self.pos, wl.num_heads, wl.num_kv_heads,
            wl.rotary_dim, wl.eps, slot_mapping=self.slots, kv_cache=self.cache,
            block_size=wl.block_size, kv_cache_dtype="fp8" if wl.fp8 else "auto",
            q_fp8_out=self.qf, q_fp8_scale=wl.q_scale,
            k_scale=self.ks if scales else None, v_scale=self.vs if scales else None)

    def outputs(self):
        torch.cuda.synchronize()
        return (_codes(self.qkv), None if self.cache is None else _codes(self.cache),
                None if self.qf is None else _codes(self.qf))


def _check(oracle_lib, wl, label, inputs=None):
    print("case", label, flush=True)
    x = inputs or Inputs(wl)
    if inputs is None:
        x.call()
    qkv, cache, qf = x.outputs()
    ref = run_insert_oracle(oracle_lib, wl)
    rep = C.compare_insert(qkv, cache, qf, ref, wl.num_heads, wl.num_kv_heads, wl.slot_mapping,
                           wl.fp8, wl.sentinel)
    tot = rep.totals()
    print(label, json.dumps(tot), "alternates", int(ref.alt_index.size), flush=True)
    assert rep.failures == 0, tot
    return tot


@pytest.mark.parametrize("index", range(3), ids=W.INSERT_NAMES)
def test_insert_workload_parity(oracle_lib, index):
    wl = W.insert_make(index)
    tot = _check(oracle_lib, wl, wl.name)
    assert tot["v"]["exact"] == tot["v"]["n"]
    if "cache_v" in tot:
        assert tot["cache_v"]["exact"] == tot["cache_v"]["n"]


SWEEP = [
    # (T, H, nkv, R, bs, blocks, fp8 cache, q fp8, insert, pad)
    (1, 1, 1, 16, 1, 2, False, False, True, 0.0),      # 3 heads per token
    (1, 1, 1, 64, 1, 2, True, True, True, 0.0),
    (7, 4, 2, 64, 16, 2, False, True, True, 0.15),
    (7, 4, 2, 32, 4, 4, True, True, True, 0.0),
    (14, 8, 2, 64, 8, 4, True, False, True, 0.3),
    (5, 3, 1, 16, 2, 8, True, True, True, 0.2),        # 5 heads per token
    (9, 2, 1, 64, 16, 1, False, True, False, 0.0),     # no insert
    (6, 2, 2, 32, 2, 4, False, False, True, 1.0),      # every slot is padding
    (63, 6, 3, 64, 4, 64, True, True, True, 0.1),      # 12 heads per token
    (77, 5, 3, 32, 16, 8, False, True, True, 0.1),     # 11 heads per token, ragged tail
    (448, 8, 2, 64, 64, 16, True, True, True, 0.02),   # a tensor-parallel shard's heads
    (2048, 32, 8, 64, 64, 64, True, True, True, 0.05),  # 256 requests' draft rows
    (1001, 7, 1, 16, 128, 16, False, False, True, 0.3),  # 9 heads per token
    (20, 128, 16, 64, 16, 8, True, True, True, 0.1),   # 160 heads per token
    (50, 4, 2, 32, 2048, 1, False, True, True, 0.1),   # 2048-token blocks
]


def _ids(s):
    return "T%d-H%d-kv%d-R%d-bs%d-%s%s%s" % (s[0], s[1], s[2], s[3], s[4], "fp8" if s[6] else "bf16",
                                            "-qfp8" if s[7] else "", "" if s[8] else "-noins")


@pytest.mark.parametrize("shape", SWEEP, ids=_ids)
def test_insert_shape_sweep(oracle_lib, shape):
    T, H, nkv, R, bs, nb, fp8, qf, ins, pad = shape
    wl = W.insert_custom(T, H, nkv, R, bs, nb, fp8, qf, seed=77 + T, pad_fraction=pad,
                         std=4.0 if fp8 else 1.0, insert=ins)
    _check(oracle_lib, wl, _ids(shape))


def test_insert_without_scales_stores_unit_scale(oracle_lib):
    """No k/v scale tensors (the page's call passes none): an fp8 insert
    stores e4m3 of the values themselves."""
    wl = W.insert_custom(64, 4, 2, 32, 16, 8, True, True, seed=5, std=4.0)
    wl.k_scale = wl.v_scale = 1.0
    x = Inputs(wl)
    x.call(scales=False)
    _check(oracle_lib, wl, "fp8 without scales", x)


def test_insert_custom_op_mirror(oracle_lib):
    """dspark_qknorm_rope_kv_insert with a layer object: block size from the
    cache, fp8 from its uint8 storage, q scale from _q_scale_float."""
    wl = W.insert_custom(21, 4, 2, 64, 16, 8, True, True, seed=6, std=4.0)
    wl.k_scale = wl.v_scale = 1.0
    x = Inputs(wl)
    layer = SimpleNamespace(kv_cache=x.cache, _q_scale_float=wl.q_scale)
    dspark_qknorm_rope_kv_insert(x.qkv, x.qw, x.kw, x.cs, x.pos, wl.num_heads, wl.num_kv_heads,
                                 wl.rotary_dim, wl.eps, x.qf.view(torch.float8_e4m3fn), layer,
                                 x.slots)
    _check(oracle_lib, wl, "custom-op mirror", x)
    # without a slot mapping nothing is stored
    wl2 = W.insert_custom(21, 4, 2, 64, 16, 8, True, False, seed=6, std=4.0, insert=False)
    y = Inputs(wl2)
    cache = torch.full(wl.cache_shape, W.SENTINEL_FP8, dtype=torch.uint8, device=DEV)
    dspark_qknorm_rope_kv_insert(y.qkv, y.qw, y.kw, y.cs, y.pos, wl2.num_heads, wl2.num_kv_heads,
                                 wl2.rotary_dim, wl2.eps, None,
                                 SimpleNamespace(kv_cache=cache, _q_scale_float=1.0), None)
    _check(oracle_lib, wl2, "custom-op mirror, no insert", y)
    assert bool((cache == W.SENTINEL_FP8).all())


def test_insert_zero_tokens_is_a_noop():
    wl = W.insert_custom(0, 4, 2, 64, 16, 2, False, True, seed=1)
    x = Inputs(wl)
    x.call()
    torch.cuda.synchronize()
    assert bool((x.cache.view(torch.int16) == -1).all())


def test_insert_graph_capture_replays(oracle_lib):
    """One captured insert, replayed with fresh qkv values copied in between
    (a fill kernel, not a memset, resets the outputs): every replay matches
    the oracle on its inputs."""
    wls = [W.insert_custom(140, 8, 2, 32, 16, 16, True, True, seed=40 + i, std=4.0)
           for i in range(3)]
    for w in wls[1:]:                      # same slots and positions, new values
        w.slot_mapping, w.positions, w.cos_sin = wls[0].slot_mapping, wls[0].positions, wls[0].cos_sin
        w.q_norm_weight, w.k_norm_weight = wls[0].q_norm_weight, wls[0].k_norm_weight
        w.k_scale, w.v_scale, w.q_scale = wls[0].k_scale, wls[0].v_scale, wls[0].q_scale
    x = Inputs(wls[0])
    src = [_bf16(w.qkv) for w in wls]
    x.qkv.copy_(src[0])
    x.call()                                           # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            x.call()
    torch.cuda.synchronize()
    for i, w in enumerate(wls):
        x.qkv.copy_(src[i])
        x.cache.fill_(W.SENTINEL_FP8)
        x.qf.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        x.wl = w
        _check(oracle_lib, w, "graph replay %d" % i, x)


def test_insert_argument_errors():
    wl = W.insert_custom(7, 4, 2, 64, 16, 2, False, True, seed=2)
    x = Inputs(wl)
    with pytest.raises(ValueError, match="qkv has shape"):
        fused_qknorm_rope_kv_insert(x.qkv, x.qw, x.kw, x.cs, x.pos, 5, 2, 64, 1e-6)
    with pytest.raises(ValueError, match="cos_sin_cache"):
        fused_qknorm_rope_kv_insert(x.qkv, x.qw, x.kw, x.cs, x.pos, 4, 2, 32, 1e-6)
    with pytest.raises(ValueError, match="block_size"):
        fused_qknorm_rope_kv_insert(x.qkv, x.qw, x.kw, x.cs, x.pos, 4, 2, 64, 1e-6,
                                    slot_mapping=x.slots, kv_cache=x.cache, block_size=32)
    with pytest.raises(RuntimeError, match="q_fp8_scale"):
        fused_qknorm_rope_kv_insert(x.qkv, x.qw, x.kw, x.cs, x.pos, 4, 2, 64, 1e-6,
                                    q_fp8_out=x.qf, q_fp8_scale=0.0)
    torch.cuda.synchronize()
    # nothing ran: the inputs are as they were
    assert np.array_equal(_codes(x.qkv), wl.qkv)
