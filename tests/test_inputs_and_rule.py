"""CPU checks of the test infrastructure around the oracle: the seeded input
generators are deterministic (their bytes are pinned), the bench's byte
count equals the bytes the write actually moves, and the acceptance rule's
ordinal distance behaves as stated (adjacent codes 1 apart, +0 and -0
equal, order of the values preserved)."""
import hashlib

import numpy as np
import pytest
import torch

from oracle import compare as C
from speculative_decoding_draft_02_amd import workloads as W

WRITE_FIELDS = ("all_kv", "k_norm_weight", "positions", "slot_mapping", "cos_sin", "k_scales",
                "v_scales")
INSERT_FIELDS = ("qkv", "q_norm_weight", "k_norm_weight", "positions", "slot_mapping", "cos_sin",
                 "k_scale", "v_scale", "q_scale")
PROJECT_FIELDS = ("states", "hidden_norm_weight", "kv_weight", "k_norm_weight", "positions",
                  "slot_mapping", "cos_sin", "k_scales", "v_scales")


def _digest(obj, names):
    h = hashlib.sha256()
    for name in names:
        v = getattr(obj, name)
        h.update(np.ascontiguousarray(v).tobytes() if isinstance(v, np.ndarray) else repr(v).encode())
    return h.hexdigest()[:16]


# first 16 hex digits of the sha256 of every generated array, in field order;
# a change here means the inputs changed, and every stored figure with them
WRITE_DIGESTS = {0: "67e7781b8528a264", 1: "c84197122cd643d3", 2: "1a9738c36070da07",
                 3: "e93a57d374808c1b", 4: "161403d57030e0e0"}
INSERT_DIGESTS = {0: "c280474bda20244e", 1: "0d87dad70b4083c8", 2: "fbfa4959eddf4d7a"}
PROJECT_DIGESTS = {0: "b3921ef88d1528d9", 1: "7a36a40117fa74cc", 2: "d96352117429eaf4"}


@pytest.mark.parametrize("index", range(5), ids=W.NAMES)
def test_write_inputs_are_pinned(index):
    assert _digest(W.make(index), WRITE_FIELDS) == WRITE_DIGESTS[index]


@pytest.mark.parametrize("index", range(3))
def test_insert_and_projection_inputs_are_pinned(index):
    assert _digest(W.insert_make(index), INSERT_FIELDS) == INSERT_DIGESTS[index]
    assert _digest(W.project_make(index), PROJECT_FIELDS) == PROJECT_DIGESTS[index]


def test_gaussian_projection_inputs_are_pinned():
    wl = W.project_custom(777, 448, 2, 2, 64, 16, 64, False, seed=31, pad_fraction=0.1)
    assert _digest(wl, PROJECT_FIELDS) == "05e66dac3b647c56"
    s = wl.slot_mapping[wl.slot_mapping >= 0]
    assert np.unique(s).size == s.size and s.max() < wl.num_blocks * wl.block_size
    assert wl.positions.max() < wl.cos_sin.shape[0]


def test_generated_slots_are_unique_and_in_range():
    for index in (0, 1, 2, 4):
        wl = W.make(index)
        s = wl.slot_mapping[wl.slot_mapping >= 0]
        assert np.unique(s).size == s.size
        assert s.max() < wl.num_blocks * wl.block_size
        assert wl.positions.min() >= 0 and wl.positions.max() < wl.cos_sin.shape[0]


@pytest.mark.parametrize("case", ["tiny", "decode", "fp8", "layer-slots"])
def test_byte_count_equals_the_bytes_moved(oracle_lib, case):
    """The bench's algorithmic bytes, against what the oracle's write actually
    touches: cache bytes counted as the elements that differ from the
    sentinel (a NaN pattern the write never produces), reads from the valid
    tokens' rows, positions, cos/sin rows, every slot and the weights."""
    if case == "tiny":
        wl = W.make(0)
    elif case == "decode":
        wl = W.make(4)
    elif case == "fp8":
        wl = W.custom(300, 3, 4, 32, 16, 64, True, seed=8, pad_fraction=0.2, kv_std=4.0)
    else:
        wl = W.per_layer_slots(W.custom(200, 3, 4, 64, 16, 64, False, seed=9, pad_fraction=0.1),
                               seed=10, pad_fraction=0.2)
    res = oracle_lib.ctx_kv_write(wl.all_kv, wl.k_norm_weight, wl.eps, wl.positions, wl.cos_sin,
                                  wl.rotary_dim, wl.slot_mapping, wl.new_host_caches(), wl.fp8,
                                  wl.k_scales, wl.v_scales)
    e = 1 if wl.fp8 else 2
    written = sum(int(np.count_nonzero(c != wl.sentinel)) for c in res.caches) * e
    L, nkv, R, N = wl.num_layers, wl.num_kv_heads, wl.rotary_dim, wl.num_ctx
    if wl.slot_mapping.ndim == 1:
        valid = int(np.count_nonzero(wl.slot_mapping >= 0))
        read_rows = valid * L * 2 * nkv * 256
        per_token = valid * (2 * R + 8)
        slots = 8 * N
    else:
        token_layers = int(np.count_nonzero(wl.slot_mapping >= 0))
        tokens = int(np.count_nonzero((wl.slot_mapping >= 0).any(axis=0)))
        read_rows = token_layers * 2 * nkv * 256
        per_token = tokens * (2 * R + 8)
        slots = 8 * N * L
    assert written == (token_layers if wl.slot_mapping.ndim == 2 else valid * L) * nkv * 256 * e
    assert wl.algorithmic_bytes() == read_rows + written + per_token + slots + 256 * L


def test_ordinal_distance_bf16():
    codes = np.array([0x3F80, 0x3F81, 0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F], np.uint16)
    o = C.ordinal_bf16(codes)
    assert o[1] - o[0] == 1                      # adjacent codes
    assert o[2] == o[3] == 0                     # +0 and -0 are equal
    assert o[4] - o[5] == 2                      # smallest subnormals of either sign: 2 steps
    assert o[6] == -o[7]                         # symmetric about zero
    # ordering of the values is preserved over every finite bf16 code
    allc = np.arange(65536, dtype=np.uint32)
    finite = allc[((allc >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    vals = (finite.astype(np.uint32) << 16).view(np.float32)
    order = np.argsort(vals, kind="stable")
    ords = C.ordinal_bf16(finite)[order]
    assert np.all(np.diff(ords) >= 0)
    assert np.count_nonzero(np.diff(ords) == 0) == 1     # only +0 / -0 coincide


def test_ordinal_distance_e4m3():
    allc = np.arange(256, dtype=np.uint8)
    finite = allc[(allc & 0x7F) != 0x7F]
    vals = torch.from_numpy(finite).view(torch.float8_e4m3fn).float().numpy()
    order = np.argsort(vals, kind="stable")
    ords = C.ordinal_e4m3(finite)[order]
    assert np.all(np.diff(ords) >= 0)
    assert np.count_nonzero(np.diff(ords) == 0) == 1     # only +0 / -0 coincide
    assert C.ordinal_e4m3(np.array([0x7E], np.uint8))[0] - C.ordinal_e4m3(np.array([0x7D], np.uint8))[0] == 1


def test_rule_counts_one_ulp_and_signed_zero(oracle_lib):
    """A K code one step off is counted as within 1, a K of -0 against +0
    likewise (equal under the rule), and neither is a failure; two steps
    off is a failure."""
    wl = W.custom(8, 1, 2, 32, 4, 4, False, seed=12, pad_fraction=0.0)
    res = oracle_lib.ctx_kv_write(wl.all_kv, wl.k_norm_weight, wl.eps, wl.positions, wl.cos_sin,
                                  32, wl.slot_mapping, wl.new_host_caches(), False)
    dev = [c.copy() for c in res.caches]
    rows = dev[0].reshape(-1, 256)
    written = np.flatnonzero(rows[:, 0] != wl.sentinel)
    r0 = written[0]
    rows[r0, 100] = rows[r0, 100] + 1 if rows[r0, 100] & 0x7FFF < 0x7F7F else rows[r0, 100] - 1
    base = C.compare(dev, res, wl.slot_mapping, False, wl.sentinel).totals()
    assert base["k"]["fail"] == 0 and base["k"]["within1"] >= 1
    ref_rows = res.caches[0].reshape(-1, 256)
    # +0 in a copy of the oracle's result against -0 on the device side
    import dataclasses
    ref0 = [c.copy() for c in res.caches]
    ref0[0].reshape(-1, 256)[written[2], 7] = 0x0000
    rows[written[2], 7] = 0x8000
    tot = C.compare(dev, dataclasses.replace(res, caches=ref0), wl.slot_mapping, False,
                    wl.sentinel).totals()
    assert tot["k"]["fail"] == 0
    rows[written[1], 5] = ref_rows[written[1], 5] + 2
    assert C.compare(dev, res, wl.slot_mapping, False, wl.sentinel).totals()["k"]["fail"] >= 1
