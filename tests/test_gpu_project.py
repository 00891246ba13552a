"""Parity of the step before the write on MI355X (through the C ABI): the
Gemma hidden norm, and the token-major K/V projection on the matrix cores
with the context write fused into its epilogue.

* Hidden norm: bit-exact with the oracle except at recorded near ties, where
  the other bf16 neighbour is also correct.
* Projection + write on exactly-summable grids (every fp32 partial sum is
  exact, so the projection has one correct result): the caches meet the
  context write's acceptance rule against the oracle's write of the oracle's
  projection (V bit-exact in bf16 caches).
* The full-size pipeline on Gaussian data, element by element: every all_kv
  value the fused kernel computed (returned through its all_kv output) lies
  in the interval that the fp32 accumulation bound gives around the exact
  projection of the device's own hidden-norm output (oracle/compare.py:
  worst case for any order, and Higham and Mary's probabilistic bound), and
  every cache element meets the write's rule against the oracle's write of
  that all_kv; every unwritten cache row is untouched.
* The packed weight: its layout is the documented permutation (bit-exact),
  and the projection from it writes the same bytes as the projection from
  the row-major weight, at small shapes and at the full prefill size."""
import json

import numpy as np
import pytest
import torch

from oracle import compare as C
from speculative_decoding_draft_02_amd import workloads as W
from speculative_decoding_draft_02_amd import _lib
from speculative_decoding_draft_02_amd.project import (hidden_norm, pack_kv_weight,
                                                      precompute_and_store_context_kv)
from speculative_decoding_draft_02_amd.writer import AttnLayer, DSparkContextKVWriter
from tests._util import bits_to_f32

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
    return t.cpu().numpy() if t.dtype == torch.uint8 else t.view(torch.int16).cpu().numpy().view(np.uint16)


def _layers(wl):
    out = []
    for l in range(wl.num_layers):
        shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, 256)
        if wl.fp8:
            cache = torch.full(shape, W.SENTINEL_FP8, dtype=torch.uint8, device=DEV)
        else:
            cache = torch.full(shape, -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        ks = torch.tensor([float(wl.k_scales[l])], dtype=torch.float32, device=DEV)
        vs = torch.tensor([float(wl.v_scales[l])], dtype=torch.float32, device=DEV)
        out.append(AttnLayer(cache, ks, vs, "fp8" if wl.fp8 else "auto"))
    return out


@pytest.mark.parametrize("rows,dim", [(1, 8), (5, 256), (300, 1000), (64, 6144), (7, 12288)])
def test_hidden_norm_parity(oracle_lib, rows, dim):
    print("case hidden_norm", rows, dim, flush=True)
    rng = np.random.default_rng(rows * 7 + dim)
    x = W._normal_bf16(rng, (rows, dim), 1.0)
    w = W._normal_bf16(rng, (dim,), 0.1)
    got = _codes(hidden_norm(_bf16(x), _bf16(w), 1e-6))
    ref, idx, other = oracle_lib.gemma_rms_norm(x, w, 1e-6)
    diff = np.flatnonzero(got.reshape(-1) != ref.reshape(-1))
    alt = dict(zip(idx.tolist(), other.tolist()))
    bad = [int(i) for i in diff if alt.get(int(i)) != int(got.reshape(-1)[i])]
    print("hidden_norm", rows, dim, "differences", diff.size, "near ties", idx.size, flush=True)
    assert not bad, bad[:10]


def test_hidden_norm_in_place(oracle_lib):
    rng = np.random.default_rng(3)
    x = W._normal_bf16(rng, (33, 512), 2.0)
    w = W._normal_bf16(rng, (512,), 0.1)
    t = _bf16(x)
    hidden_norm(t, _bf16(w), 1e-6, out=t)
    ref, idx, other = oracle_lib.gemma_rms_norm(x, w, 1e-6)
    got = _codes(t)
    diff = np.flatnonzero(got.reshape(-1) != ref.reshape(-1))
    alt = dict(zip(idx.tolist(), other.tolist()))
    assert all(alt.get(int(i)) == int(got.reshape(-1)[i]) for i in diff)


EXACT_SWEEP = [
    # (N, hidden, L, nkv, R, bs, blocks, fp8, pad); with a packed weight the
    # column counts 2 L nkv 128 that are multiples of 512 run 128 x 512 tiles,
    # the others (L nkv odd: the first three cases) 256 x 256 tiles
    (1, 64, 1, 1, 16, 1, 2, False, 0.0),
    (300, 256, 2, 2, 64, 16, 32, False, 0.1),
    (300, 512, 1, 3, 32, 4, 128, True, 0.2),
    (513, 192, 2, 1, 16, 2, 300, True, 0.0),
    (256, 1024, 3, 2, 64, 64, 8, False, 0.5),
    (1000, 128, 1, 8, 32, 128, 8, True, 0.05),
    (700, 2048, 2, 4, 64, 16, 64, False, 0.02),
    # k in whole rings of five 32-wide stages, no tail
    (200, 320, 2, 2, 32, 16, 32, False, 0.1),
    (333, 960, 1, 4, 16, 8, 64, True, 0.1),
    # the largest layer count: 32 layers x 2 kinds x 1 head = 64 heads
    (300, 128, 32, 1, 64, 16, 32, False, 0.1),
    # 129 x 2 tiles of 128 x 512 with a packed weight: on a 256-CU device 256
    # whole tiles and the last two tiles in 64-token halves in one launch,
    # the very last half wholly past the last token
    (16448, 128, 2, 2, 64, 16, 1100, False, 0.05),
    (16448, 64, 1, 4, 32, 16, 1100, True, 0.05),
    # one 128 x 512 tile in two halves: the second wholly past the only
    # token, or holding one token
    (1, 64, 2, 1, 16, 1, 2, True, 0.0),
    (65, 128, 1, 2, 32, 4, 32, False, 0.0),
]


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("shape", EXACT_SWEEP,
                         ids=lambda s: "N%d-h%d-L%d-kv%d-R%d-bs%d-%s" % (s[0], s[1], s[2], s[3], s[4], s[5],
                                                                      "fp8" if s[7] else "bf16"))
def test_project_write_exact_grids(oracle_lib, shape, packed):
    N, hidden, L, nkv, R, bs, nb, fp8, pad = shape
    print("case project exact", shape, "packed" if packed else "row-major", flush=True)
    wl = W.project_exact(N, hidden, L, nkv, R, bs, nb, fp8, seed=N + hidden, pad_fraction=pad)
    layers = _layers(wl)
    writer = DSparkContextKVWriter(layers)
    weight = pack_kv_weight(_bf16(wl.kv_weight)) if packed else _bf16(wl.kv_weight)
    writer.project_write(_bf16(wl.states), weight, _bf16(wl.k_norm_weight), wl.eps,
                         torch.from_numpy(wl.positions).to(DEV), _bf16(wl.cos_sin), R,
                         torch.from_numpy(wl.slot_mapping).to(DEV))
    torch.cuda.synchronize()
    got = [_codes(a.kv_cache) for a in layers]
    all_kv = oracle_lib.kv_project(wl.states, wl.kv_weight)
    ww = wl.write_workload(all_kv)
    ref = oracle_lib.ctx_kv_write(ww.all_kv, ww.k_norm_weight, ww.eps, ww.positions, ww.cos_sin, R,
                                  ww.slot_mapping, ww.new_host_caches(), fp8, ww.k_scales,
                                  ww.v_scales)
    rep = C.compare(got, ref, ww.slot_mapping, fp8, ww.sentinel)
    tot = rep.totals()
    print("project exact", shape, json.dumps(tot), flush=True)
    assert rep.failures == 0, tot
    if not fp8:
        assert tot["v"]["exact"] == tot["v"]["n"]
    writer.close()


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_project_write_padding_positions_off_the_table(oracle_lib, packed):
    """Padding tokens (and the rows past num_ctx in the last tile) stage
    cos/sin row 0, never their own position: with every padding token's
    position at -1 or cos_sin_rows the caches still equal the oracle's."""
    wl = W.project_exact(700, 256, 2, 4, 64, 16, 64, False, seed=77, pad_fraction=0.3)
    wl = W.padding_positions_off_table(wl)
    assert ((wl.positions < 0) | (wl.positions >= wl.cos_sin.shape[0])).any()
    print("case project padding positions", "packed" if packed else "row-major", flush=True)
    layers = _layers(wl)
    writer = DSparkContextKVWriter(layers)
    weight = pack_kv_weight(_bf16(wl.kv_weight)) if packed else _bf16(wl.kv_weight)
    writer.project_write(_bf16(wl.states), weight, _bf16(wl.k_norm_weight), wl.eps,
                         torch.from_numpy(wl.positions).to(DEV), _bf16(wl.cos_sin),
                         wl.rotary_dim, torch.from_numpy(wl.slot_mapping).to(DEV))
    torch.cuda.synchronize()
    got = [_codes(a.kv_cache) for a in layers]
    ww = wl.write_workload(oracle_lib.kv_project(wl.states, wl.kv_weight))
    ref = oracle_lib.ctx_kv_write(ww.all_kv, ww.k_norm_weight, ww.eps, ww.positions, ww.cos_sin,
                                  ww.rotary_dim, ww.slot_mapping, ww.new_host_caches(), False)
    rep = C.compare(got, ref, ww.slot_mapping, False, ww.sentinel)
    assert rep.failures == 0, rep.totals()
    writer.close()


LAM = 9.0   # the probabilistic bound's lambda (oracle/compare.py, projection_bound)


@pytest.mark.parametrize("index", [1, 2], ids=W.PROJECT_NAMES[1:])
def test_project_pipeline_full_size(oracle_lib, index):
    """hidden norm + fused projection/write at the full prefill shape (4096
    tokens, hidden 6144, 5 layers x 8 kv heads), Gaussian data, with both
    weight layouts, checked element by element:
      1. the hidden norm of every row (bit-exact but for recorded near ties);
      2. every all_kv value the fused kernel computed (its all_kv output) lies
         in [RNE(exact - b), RNE(exact + b)] around the exact projection of
         the device's own z, for the worst-case b (any order) and for the
         tight probabilistic b, and at least 99.9% are the exact rounding;
      3. every stored cache element meets the write's acceptance rule
         against the oracle's write of that all_kv (every token, layer, kv
         head and element; every row no slot names untouched);
      4. the same call without the all_kv output writes the same bytes."""
    wl = W.project_make(index)
    print("case project pipeline", wl.name, flush=True)
    N, L, nkv, hidden = wl.num_ctx, wl.num_layers, wl.num_kv_heads, wl.hidden
    states = _bf16(wl.states)
    z_dev = hidden_norm(states, _bf16(wl.hidden_norm_weight), wl.eps)
    args = (_bf16(wl.k_norm_weight), wl.eps, torch.from_numpy(wl.positions).to(DEV),
            _bf16(wl.cos_sin), wl.rotary_dim, torch.from_numpy(wl.slot_mapping).to(DEV))
    torch.cuda.synchronize()

    # 1. the hidden norm on every row
    z_ref, idx, other = oracle_lib.gemma_rms_norm(wl.states, wl.hidden_norm_weight, wl.eps)
    z_got = _codes(z_dev)
    diff = np.flatnonzero(z_got.reshape(-1) != z_ref.reshape(-1))
    alt = dict(zip(idx.tolist(), other.tolist()))
    assert all(alt.get(int(i)) == int(z_got.reshape(-1)[i]) for i in diff)

    # the exact projection of the device's z, every row and column
    sums, abs_sums, err = oracle_lib.kv_project_sums(z_got, wl.kv_weight)
    bounds = {name: C.projection_bound(abs_sums, hidden, lam=lam, sum_err=err)
              for name, lam in (("worst", None), ("probabilistic", LAM))}
    exact_codes = W.to_bf16_bits(C.rne_bf16(sums))
    del abs_sums

    results = {}
    for packed in (False, True):
        layers = _layers(wl)
        writer = DSparkContextKVWriter(layers)
        weight = pack_kv_weight(_bf16(wl.kv_weight)) if packed else _bf16(wl.kv_weight)
        all_kv = torch.empty((N, L, 2, nkv, 128), dtype=torch.bfloat16, device=DEV)
        z_again = torch.empty_like(states)
        kw_, eps_, pos_, cs_, R_, slots_ = args
        precompute_and_store_context_kv(writer, states, _bf16(wl.hidden_norm_weight), eps_,
                                        weight, kw_, pos_, cs_, R_, slots_, workspace=z_again,
                                        all_kv_out=all_kv)
        torch.cuda.synchronize()
        assert torch.equal(z_again.view(torch.int16), z_dev.view(torch.int16))
        akv = _codes(all_kv).reshape(N, -1)
        caches = [_codes(a.kv_cache) for a in layers]
        tag = "packed" if packed else "row-major"

        # 2. every all_kv value inside its interval
        got = bits_to_f32(akv).astype(np.float64)
        for name, b in bounds.items():
            lo, hi = C.all_kv_interval(sums, b)
            out = (got < lo) | (got > hi)
            assert not out.any(), (tag, name, int(out.sum()))
        frac = float(np.mean(akv == exact_codes))
        print("project pipeline", wl.name, tag, "all_kv bit-exact %.6f of %d" % (frac, akv.size),
              flush=True)
        assert frac > 0.999

        # 3. the caches: the oracle's write of the kernel's own all_kv
        ww = wl.write_workload(akv)
        ref = oracle_lib.ctx_kv_write(ww.all_kv, ww.k_norm_weight, ww.eps, ww.positions,
                                      ww.cos_sin, ww.rotary_dim, ww.slot_mapping,
                                      ww.new_host_caches(), wl.fp8, ww.k_scales, ww.v_scales)
        rep = C.compare(caches, ref, ww.slot_mapping, wl.fp8, ww.sentinel)
        tot = rep.totals()
        print("project pipeline", wl.name, tag, json.dumps(tot), flush=True)
        assert rep.failures == 0, tot
        if not wl.fp8:
            assert tot["v"]["exact"] == tot["v"]["n"]

        # 4. without the all_kv output: the same bytes
        for a in layers:
            a.kv_cache.view(torch.uint8).fill_(0xFF)
        writer.project_write(z_dev, weight, *args)
        torch.cuda.synchronize()
        assert all(np.array_equal(_codes(a.kv_cache), c) for a, c in zip(layers, caches))
        writer.close()
        results[packed] = (akv, caches)
    # both weight layouts accumulate the same products in the same order
    assert np.array_equal(results[False][0], results[True][0])
    assert all(np.array_equal(x, y) for x, y in zip(results[False][1], results[True][1]))


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_project_write_graph_capture(oracle_lib, packed):
    """The fused projection/write captured once and replayed: every replay
    writes the oracle's result (the caches are refilled between replays)."""
    wl = W.project_exact(300, 256, 2, 2, 32, 16, 32, True, seed=5)
    layers = _layers(wl)
    writer = DSparkContextKVWriter(layers)
    weight = pack_kv_weight(_bf16(wl.kv_weight)) if packed else _bf16(wl.kv_weight)
    args = (_bf16(wl.states), weight, _bf16(wl.k_norm_weight), wl.eps,
            torch.from_numpy(wl.positions).to(DEV), _bf16(wl.cos_sin), wl.rotary_dim,
            torch.from_numpy(wl.slot_mapping).to(DEV))
    writer.project_write(*args)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            writer.project_write(*args)
    all_kv = oracle_lib.kv_project(wl.states, wl.kv_weight)
    ww = wl.write_workload(all_kv)
    ref = oracle_lib.ctx_kv_write(ww.all_kv, ww.k_norm_weight, ww.eps, ww.positions, ww.cos_sin,
                                  ww.rotary_dim, ww.slot_mapping, ww.new_host_caches(), True,
                                  ww.k_scales, ww.v_scales)
    for rep in range(3):
        for a in layers:
            a.kv_cache.fill_(W.SENTINEL_FP8)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [_codes(a.kv_cache) for a in layers]
        assert C.compare(got, ref, ww.slot_mapping, True, ww.sentinel).failures == 0, rep
    writer.close()


def test_project_write_debug_checks(oracle_lib):
    """With debug_checks the projection refuses a slot outside the cache
    before any launch; valid inputs write as usual."""
    wl = W.project_exact(100, 128, 1, 2, 32, 16, 8, False, seed=3, pad_fraction=0.1)
    layers = _layers(wl)
    writer = DSparkContextKVWriter(layers, debug_checks=True)
    args = [_bf16(wl.states), _bf16(wl.kv_weight), _bf16(wl.k_norm_weight), wl.eps,
            torch.from_numpy(wl.positions).to(DEV), _bf16(wl.cos_sin), 32]
    slots = torch.from_numpy(wl.slot_mapping).to(DEV)
    bad = slots.clone()
    bad[int(torch.nonzero(bad >= 0)[0])] = wl.num_blocks * wl.block_size
    with pytest.raises(ValueError, match="num_blocks"):
        writer.project_write(*args, bad)
    torch.cuda.synchronize()
    assert all(bool((_codes(a.kv_cache) == 0xFFFF).all()) for a in layers)
    writer.project_write(*args, slots)
    torch.cuda.synchronize()
    got = [_codes(a.kv_cache) for a in layers]
    ww = wl.write_workload(oracle_lib.kv_project(wl.states, wl.kv_weight))
    ref = oracle_lib.ctx_kv_write(ww.all_kv, ww.k_norm_weight, ww.eps, ww.positions, ww.cos_sin,
                                  32, ww.slot_mapping, ww.new_host_caches(), False,
                                  ww.k_scales, ww.v_scales)
    assert C.compare(got, ref, ww.slot_mapping, False, ww.sentinel).failures == 0
    writer.close()


def _packed_reference(w_bits):
    """The documented fragment-major index of every weight element, applied
    with numpy: element (c, k) at ((c // 32) * (hidden // 16) + k // 16) * 512
    + 8 * (c % 32 + 32 * ((k % 16) // 8)) + k % 8."""
    cols, hidden = w_bits.shape
    c = np.arange(cols)[:, None]
    k = np.arange(hidden)[None, :]
    idx = ((c // 32) * (hidden // 16) + k // 16) * 512 + 8 * (c % 32 + 32 * ((k % 16) // 8)) + k % 8
    out = np.zeros(cols * hidden, np.uint16)
    out[idx.reshape(-1)] = w_bits.reshape(-1)
    return out


@pytest.mark.parametrize("cols,hidden", [(32, 16), (96, 80), (2560, 6144)])
def test_pack_kv_weight_layout(cols, hidden):
    """The packing is a permutation onto the documented index (every input
    bit pattern moved, none changed), checked against numpy."""
    rng = np.random.default_rng(cols + hidden)
    w_bits = rng.integers(0, 1 << 16, size=(cols, hidden), dtype=np.uint16)
    packed = pack_kv_weight(_bf16(w_bits))
    torch.cuda.synchronize()
    assert (packed.cols, packed.hidden) == (cols, hidden)
    got = packed.data.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, _packed_reference(w_bits))


def test_pack_kv_weight_errors():
    """Sizes the layout cannot take and overlapping buffers are refused
    before any launch, with a reason."""
    w = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(64 * 64, dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    assert _lib.dspark_kv_weight_pack(w.data_ptr(), 48, 64, out.data_ptr(), s) == _lib.E_ARG
    assert "multiple of 32" in _lib.dspark_ctx_kv_last_error()
    assert _lib.dspark_kv_weight_pack(w.data_ptr(), 64, 24, out.data_ptr(), s) == _lib.E_ARG
    assert "multiple of 16" in _lib.dspark_ctx_kv_last_error()
    assert _lib.dspark_kv_weight_pack(w.data_ptr(), 64, 64, w.data_ptr() + 1024, s) == _lib.E_ARG
    assert "overlaps" in _lib.dspark_ctx_kv_last_error()
    with pytest.raises(ValueError):
        pack_kv_weight(w.t())


def _run_projection(wl, weight, R=None):
    layers = _layers(wl)
    writer = DSparkContextKVWriter(layers)
    writer.project_write(_bf16(wl.states), weight, _bf16(wl.k_norm_weight), wl.eps,
                         torch.from_numpy(wl.positions).to(DEV), _bf16(wl.cos_sin),
                         R or wl.rotary_dim, torch.from_numpy(wl.slot_mapping).to(DEV))
    torch.cuda.synchronize()
    got = [_codes(a.kv_cache) for a in layers]
    writer.close()
    return got


@pytest.mark.parametrize("case", ["small-bf16", "small-fp8", "tail-bf16", "halves-fp8", "full-bf16",
                                  "full-fp8"])
def test_packed_projection_equals_row_major(case):
    """The packed kernels accumulate the same products in the same order as
    the row-major one, so the caches they write are identical byte for byte:
    on Gaussian data (no exact grid), with a ragged token tail and a k range
    that ends inside a ring round, with whole tiles and 64-token halves in
    one launch, and at the full prefill size."""
    if case == "halves-fp8":
        wl = W.project_custom(16400, 192, 1, 4, 64, 16, 1100, True, seed=34, pad_fraction=0.1)
    elif case == "small-bf16":
        wl = W.project_custom(777, 448, 2, 2, 64, 16, 64, False, seed=31, pad_fraction=0.1)
    elif case == "small-fp8":
        wl = W.project_custom(513, 960, 3, 1, 32, 8, 256, True, seed=32, pad_fraction=0.2)
    elif case == "tail-bf16":
        wl = W.project_custom(33, 64, 1, 2, 16, 4, 16, False, seed=33, pad_fraction=0.0)
    else:
        wl = W.project_make(1 if case == "full-bf16" else 2)
    print("case packed == row-major", case, flush=True)
    ref = _run_projection(wl, _bf16(wl.kv_weight))
    got = _run_projection(wl, pack_kv_weight(_bf16(wl.kv_weight)))
    for l, (g, r) in enumerate(zip(got, ref)):
        assert np.array_equal(g, r), (case, l, int(np.count_nonzero(g != r)))


def test_packed_weight_for_another_shape_is_refused():
    """A weight packed for another (cols, hidden) is refused before any
    launch, and the caches stay untouched."""
    wl = W.project_exact(64, 128, 1, 2, 32, 16, 8, False, seed=9, pad_fraction=0.0)
    layers = _layers(wl)
    writer = DSparkContextKVWriter(layers)
    other = pack_kv_weight(torch.zeros(2 * 2 * 128, 192, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="packed weight"):
        writer.project_write(_bf16(wl.states), other, _bf16(wl.k_norm_weight), wl.eps,
                             torch.from_numpy(wl.positions).to(DEV), _bf16(wl.cos_sin), 32,
                             torch.from_numpy(wl.slot_mapping).to(DEV))
    torch.cuda.synchronize()
    assert all(bool((_codes(a.kv_cache) == 0xFFFF).all()) for a in layers)
    writer.close()
