"""Pins of the oracle's step before the write (vLLM API page
"vllm.models.minimax_m3.common.dspark": the Gemma hidden_norm and the
token-major K/V projection): the K norm of the pinned context-write oracle,
a PyTorch fp32 composite, closed forms, exact integer sums on coarse grids,
and numpy's float64 matrix product."""
import numpy as np
import pytest
import torch

from speculative_decoding_draft_02_amd import workloads as W
from tests._util import bf16_bits, bits_to_f32


def _torch_bf16(x64):
    return torch.from_numpy(np.asarray(x64, np.float64)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_hidden_norm_at_128_is_the_pinned_k_norm(oracle_lib):
    """At dim 128 the hidden norm is the K norm of the context write, whose
    output the write stores unrotated at position 0 (cos 1, sin 0)."""
    rng = np.random.default_rng(4)
    N = 40
    x = W._normal_bf16(rng, (N, 128), 1.0)
    w = W._normal_bf16(rng, (128,), 0.1)
    out, idx, other = oracle_lib.gemma_rms_norm(x, w, 1e-6)
    all_kv = np.stack([x, x], axis=1)[:, None, :, None, :]
    cache = [np.full((N, 1, 1, 256), 0xFFFF, np.uint16)]
    oracle_lib.ctx_kv_write(all_kv, w.reshape(1, 128), 1e-6, np.zeros(N, np.int64),
                            W.rope_table(1, 64), 64, np.arange(N), cache, False)
    assert np.array_equal(out, cache[0].reshape(N, 256)[:, :128])


@pytest.mark.parametrize("dim", [256, 6144])
def test_hidden_norm_vs_torch(oracle_lib, dim):
    rng = np.random.default_rng(dim)
    x = W._normal_bf16(rng, (24, dim), 1.0)
    w = W._normal_bf16(rng, (dim,), 0.1)
    out, idx, other = oracle_lib.gemma_rms_norm(x, w, 1e-6)
    xt = torch.from_numpy(bits_to_f32(x))
    wt = torch.from_numpy(bits_to_f32(w))
    ref = (xt * torch.rsqrt(xt.pow(2).mean(-1, keepdim=True) + 1e-6) * (1.0 + wt)).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    diff = np.flatnonzero(out.reshape(-1) != ref.reshape(-1))
    # every difference is a recorded near tie, and the torch value is the other neighbour
    alt = dict(zip(idx.tolist(), other.tolist()))
    for i in diff:
        assert alt.get(int(i)) == int(ref.reshape(-1)[i]), i
    assert diff.size <= 0.01 * out.size


def test_hidden_norm_closed_forms(oracle_lib):
    dim = 512
    x = np.zeros((3, dim))
    x[0, :] = 0.5                  # constant row: 0.5 / sqrt(0.25 + eps) -> 1.0
    x[1, 7] = 3.0                  # one-hot: 3 / sqrt(9 / dim + eps)
    x[2, :] = -2.0                 # with w = 1 on every element: -2.0
    w = np.zeros(dim)
    out, _, _ = oracle_lib.gemma_rms_norm(bf16_bits(x), bf16_bits(w), 1e-6)
    assert np.all(out[0] == 0x3F80)
    want = int(bf16_bits([3.0 / np.sqrt(9.0 / dim + 1e-6)])[0])
    assert out[1, 7] == want and np.all(np.delete(out[1], 7) == 0)
    out2, _, _ = oracle_lib.gemma_rms_norm(bf16_bits(x[2:]), bf16_bits(np.ones(dim)), 1e-6)
    assert np.all(out2 == bf16_bits([-2.0])[0])


def test_projection_exact_on_coarse_grids(oracle_lib):
    """z = k 2^-5, W = m 2^-9: the sum is an integer times 2^-14 that int64
    arithmetic gives exactly; the oracle's fp64 sum must equal it and its
    code must be that value rounded to bf16 once."""
    wl = W.project_exact(48, 512, 2, 2, 32, 16, 8, False, seed=7)
    zi = np.rint(bits_to_f32(wl.states).astype(np.float64) * 32).astype(np.int64)
    wi = np.rint(bits_to_f32(wl.kv_weight).astype(np.float64) * 512).astype(np.int64)
    exact_int = zi @ wi.T
    codes, ex, ab = oracle_lib.kv_project(wl.states, wl.kv_weight, want_sums=True)
    assert np.array_equal(ex, exact_int.astype(np.float64) * 2.0 ** -14)
    assert np.array_equal(ab, (np.abs(zi) @ np.abs(wi).T).astype(np.float64) * 2.0 ** -14)
    assert np.array_equal(codes, _torch_bf16(exact_int.astype(np.float64) * 2.0 ** -14))
    # the grids keep every partial sum below 2^24 units: any fp32 order is exact
    assert np.abs(ab).max() < 1024


def test_projection_vs_numpy_float64(oracle_lib):
    rng = np.random.default_rng(11)
    z = W._normal_bf16(rng, (20, 1024), 1.0)
    Wt = W._normal_bf16(rng, (300, 1024), 1.0 / 32)
    codes, ex, ab = oracle_lib.kv_project(z, Wt, want_sums=True)
    ref = bits_to_f32(z).astype(np.float64) @ bits_to_f32(Wt).astype(np.float64).T
    assert np.allclose(ex, ref, rtol=0, atol=1e-12 * np.abs(ab).max())
    assert np.array_equal(codes, _torch_bf16(ex))
    # a block is the same slice of the whole product
    blk = oracle_lib.kv_project(z, Wt, rows=(3, 9), cols=(100, 228))
    assert np.array_equal(blk, codes[3:9, 100:228])


def test_projection_catches_a_transposed_operand(oracle_lib):
    """Planted on the CPU: W used as [in, out] instead of [out, in] gives a
    different product on a square case."""
    rng = np.random.default_rng(12)
    z = W._normal_bf16(rng, (8, 256), 1.0)
    Wt = W._normal_bf16(rng, (256, 256), 1.0 / 16)
    good = oracle_lib.kv_project(z, Wt)
    bad = oracle_lib.kv_project(z, np.ascontiguousarray(Wt.T))
    ref = _torch_bf16(bits_to_f32(z).astype(np.float64) @ bits_to_f32(Wt).astype(np.float64).T)
    assert np.array_equal(good, ref) and not np.array_equal(bad, ref)
