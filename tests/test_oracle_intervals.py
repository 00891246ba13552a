"""Pins of the acceptance intervals of the fused projection + write on
general (non-grid) data (oracle/compare.py: rne_bf16, projection_bound,
all_kv_interval, write_intervals) and of the oracle's full-size exact sums
(oracle.kv_project_sums), on the CPU.

What pins them: the one-step bf16 rounding equals the oracle's pinned C
codec; the float64 matrix-product sums stay within their stated bound of the
exact-product sums of the C oracle; on Gaussian rows at the projection's
hidden size (6144) the exact value and every fp32 summation order tried
(sequential, reversed, numpy's pairwise, blocked by 32, and blocks of 16
summed exactly then accumulated, as a matrix-core accumulation might) land
inside the intervals, before and after the write's norm, RoPE and fp8
conversion; and planted mistakes in the checked values (a sign flip, +2
ulp, swapped RoPE halves) fall outside."""
import numpy as np
import pytest

from oracle import compare as C
from speculative_decoding_draft_02_amd import workloads as W
from tests._util import bits_to_f32

HIDDEN = 6144
LAM = 9.0


def test_rne_bf16_is_the_oracle_codec(oracle_lib):
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(1500) * np.exp2(rng.integers(-30, 30, 1500)))
    vals += list(rng.standard_normal(300) * 2.0 ** -130)          # bf16 subnormal range
    # exact midpoints between bf16 neighbours, and points 2^-30 away from them
    for k, e in zip(rng.integers(128, 256, 400), rng.integers(-40, 40, 400)):
        mid = (k + 0.5) * 2.0 ** (e - 8)
        vals += [mid, -mid, mid * (1 + 2.0 ** -30), mid * (1 - 2.0 ** -30)]
    vals += [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 2.0 ** -133, 1.5 * 2.0 ** -133]
    x = np.array(vals)
    got = C.rne_bf16(x)
    ref = np.array([oracle_lib.bf16_decode(oracle_lib.bf16_round(v)[0]) for v in vals])
    assert np.array_equal(got, ref)
    # the double-rounding trap (fp64 -> fp32 -> bf16 would round up to 1 + 2^-7)
    assert C.rne_bf16(1.0 + 2.0 ** -8 - 2.0 ** -40) == 1.0


def test_bound_factors():
    assert C.gamma(6144) == pytest.approx(6144 * 2.0 ** -24, rel=1e-3)
    g = C.gamma_prob(6144, LAM)
    assert g == pytest.approx(LAM * np.sqrt(6144) * 2.0 ** -24, rel=1e-3)
    assert g < C.gamma(6144) / 8
    # the model's failure probability per value at the projection's sizes
    assert C.prob_bound_failure(6144, LAM) < 1e-13


def test_full_sums_within_their_bound_of_the_exact_products(oracle_lib):
    rng = np.random.default_rng(5)
    z = W._normal_bf16(rng, (37, HIDDEN), 1.0)
    Wt = W._normal_bf16(rng, (130, HIDDEN), 0.02)
    codes, exact, absum = oracle_lib.kv_project(z, Wt, want_sums=True)
    sums, abs_sums, err = oracle_lib.kv_project_sums(z, Wt)
    assert np.all(np.abs(sums - exact) <= err)
    assert np.all(np.abs(abs_sums - absum) <= err)
    assert np.all(err <= 1e-11 * abs_sums)
    # rounded once, the sums give the C oracle's codes
    assert np.array_equal(W.to_bf16_bits(C.rne_bf16(sums)), codes)


def _case(seed, T=32, R=64, fp8=False):
    """One (layer, kv head) of the projection: T tokens, K and V columns."""
    rng = np.random.default_rng(seed)
    z = W._normal_bf16(rng, (T, HIDDEN), 1.0)
    Wt = W._normal_bf16(rng, (256, HIDDEN), 0.02)
    w = W._normal_bf16(rng, (1, 128), 0.1)
    cs = W.rope_table(4096, R)
    pos = rng.integers(0, 4096, T).astype(np.int64)
    scale = np.float32(rng.uniform(0.02, 0.1))
    return z, Wt, w, cs, pos, scale


def _fp32_orders(z, Wt):
    """The projection in float32 by several summation orders (exact
    products): {name: float32 [T, C]}."""
    zf, wf = bits_to_f32(z), bits_to_f32(Wt)
    out = {}
    prods = zf[:, None, :] * wf[None, :, :]            # exact in float32 (8 x 8 bits)
    out["sequential"] = np.cumsum(prods, axis=-1, dtype=np.float32)[..., -1]
    out["reversed"] = np.cumsum(prods[..., ::-1], axis=-1, dtype=np.float32)[..., -1]
    out["pairwise"] = np.add.reduce(prods, axis=-1, dtype=np.float32)
    blocks = np.cumsum(prods.reshape(*prods.shape[:2], -1, 32), axis=-1, dtype=np.float32)[..., -1]
    out["blocked32"] = np.cumsum(blocks, axis=-1, dtype=np.float32)[..., -1]
    b16 = prods.reshape(*prods.shape[:2], -1, 16).astype(np.float64).sum(axis=-1)
    acc = np.zeros(prods.shape[:2], np.float32)
    for k in range(b16.shape[-1]):
        acc = (acc.astype(np.float64) + b16[..., k]).astype(np.float32)
    out["exact16_then_fp32"] = acc
    return out


def _write(oracle_lib, all_kv_bits, w, cs, pos, R, fp8, scale):
    """The oracle's write of one layer / one head at slots 0..T-1; returns
    the stored K and V codes [T, 128] each."""
    T = all_kv_bits.shape[0]
    bs = 16
    nb = (T + bs - 1) // bs
    cache = [np.full((nb, 1, bs, 256), 0xFF if fp8 else 0xFFFF, np.uint8 if fp8 else np.uint16)]
    akv = np.ascontiguousarray(all_kv_bits.reshape(T, 1, 2, 1, 128))
    oracle_lib.ctx_kv_write(akv, w, 1e-6, pos, cs, R, np.arange(T, dtype=np.int64), cache, fp8,
                            np.array([scale], np.float32), np.array([scale], np.float32))
    rows = cache[0].reshape(-1, 256)[:T]
    return rows[:, :128], rows[:, 128:]


def _stored_interval(lo, hi, fp8, scale):
    """Ordinal code bounds of the stored values."""
    if fp8:
        enc = np.vectorize(lambda v: C.ordinal_e4m3(np.array([_e4m3(v)]))[0])
        return enc(lo / float(scale)), enc(hi / float(scale))
    return C.ordinal_bf16(W.to_bf16_bits(lo)), C.ordinal_bf16(W.to_bf16_bits(hi))


_E4M3 = None


def _e4m3(v):
    import oracle
    return oracle.e4m3_encode(float(np.float32(v)))


def _ord(codes, fp8):
    return C.ordinal_e4m3(codes) if fp8 else C.ordinal_bf16(codes)


def _judge(oracle_lib, fp8, intervals=C.write_intervals, seed=21):
    """Apply an interval rule to the exact value and the fp32 orders (which
    must all pass) and to planted mistakes (which must be flagged).  Returns
    (orders_inside, flagged fractions by mistake)."""
    R = 64
    z, Wt, w, cs, pos, scale = _case(seed + fp8, R=R, fp8=fp8)
    codes, exact, absum = oracle_lib.kv_project(z, Wt, want_sums=True)
    wf = bits_to_f32(w[0]).astype(np.float64)
    csf = bits_to_f32(cs[pos]).astype(np.float64)
    cos, sin = csf[:, :R // 2], csf[:, R // 2:]
    bounds = {"worst": C.projection_bound(absum, HIDDEN),
              "probabilistic": C.projection_bound(absum, HIDDEN, lam=LAM)}
    iv = {}
    for name, b in bounds.items():
        k_lo, k_hi = intervals(exact[:, :128], b[:, :128], wf, cos, sin, R, 0)
        v_lo, v_hi = intervals(exact[:, 128:], b[:, 128:], wf, cos, sin, R, 1)
        iv[name] = (_stored_interval(k_lo, k_hi, fp8, scale), _stored_interval(v_lo, v_hi, fp8, scale))

    def outside(name, kcodes, vcodes):
        (klo, khi), (vlo, vhi) = iv[name]
        kd, vd = _ord(kcodes, fp8), _ord(vcodes, fp8)
        return ((kd < klo) | (kd > khi)), ((vd < vlo) | (vd > vhi))

    # the exact value and every fp32 order, through the write
    results = {"exact": codes}
    for name, acc in _fp32_orders(z, Wt).items():
        results[name] = W.to_bf16_bits(acc)
    inside = True
    for name, akv in results.items():
        k, v = _write(oracle_lib, akv, w, cs, pos, R, fp8, scale)
        for bname in bounds:
            ko, vo = outside(bname, k, v)
            inside &= not ko.any() and not vo.any()
    differs = sum(int(np.count_nonzero(a != codes)) for a in results.values())

    # planted mistakes in the checked values
    k, v = _write(oracle_lib, codes, w, cs, pos, R, fp8, scale)
    sign = 0x80 if fp8 else 0x8000
    nz_k, nz_v = (_ord(k, fp8) != 0), (_ord(v, fp8) != 0)

    def plus2(c):
        o = _ord(c, fp8) + 2
        return np.where(o < 0, sign | np.abs(o), np.abs(o)).astype(c.dtype)

    swapped = k.copy()
    swapped[:, :R // 2], swapped[:, R // 2:R] = k[:, R // 2:R], k[:, :R // 2]
    flagged = {}
    for bname in bounds:
        ko, vo = outside(bname, k ^ sign, v ^ sign)
        flagged[bname, "sign K"], flagged[bname, "sign V"] = ko[nz_k].mean(), vo[nz_v].mean()
        ko, vo = outside(bname, plus2(k), plus2(v))
        flagged[bname, "+2 K"], flagged[bname, "+2 V"] = ko.mean(), vo.mean()
        ko, _ = outside(bname, swapped, v)
        flagged[bname, "swap K"] = ko[:, :R].mean()
    return inside, differs, flagged


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_intervals_hold_every_order_and_catch_planted_mistakes(oracle_lib, fp8):
    inside, differs, f = _judge(oracle_lib, fp8)
    print({"%s %s" % k: round(float(v), 3) for k, v in f.items()})
    assert inside
    assert differs > 0          # the orders really differ from the exact rounding somewhere
    # tight (probabilistic) intervals: every planted mistake is flagged widely
    assert f["probabilistic", "sign K"] > 0.99 and f["probabilistic", "sign V"] > 0.99
    assert f["probabilistic", "+2 V"] > 0.7 and f["probabilistic", "+2 K"] > 0.4
    assert f["probabilistic", "swap K"] > 0.9
    # worst-case intervals still catch the sign flip and the swap
    assert f["worst", "sign K"] > 0.9 and f["worst", "sign V"] > 0.9
    assert f["worst", "swap K"] > 0.5


def _mutant(old, new):
    """write_intervals with one planted mistake (source text replaced)."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(C.write_intervals))
    assert src.count(old) == 1, old
    ns = dict(vars(C))
    exec(src.replace(old, new), ns)
    return ns["write_intervals"]


MUTANTS = {
    "RoPE first-half sign": ("_widen(ac_lo - ps_hi, ac_hi - ps_lo)",
                             "_widen(ac_lo + ps_lo, ac_hi + ps_hi)"),
    "RoPE halves paired wrongly": ("p_lo, p_hi = ylo[:, h:R], yhi[:, h:R]",
                                   "p_lo, p_hi = ylo[:, :h], yhi[:, :h]"),
    "norm weight dropped": ("g = 1.0 + k_norm_weight[None, :]", "g = 1.0"),
    "far too wide": ("return klo, khi", "return klo - 4 * np.abs(klo), khi + 4 * np.abs(khi)"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mistakes_in_the_rule_are_caught(oracle_lib, name):
    """A plausible slip in write_intervals either puts a correct result
    outside or lets a planted mistake through."""
    inside, _, f = _judge(oracle_lib, False, intervals=_mutant(*MUTANTS[name]))
    caught = (f["probabilistic", "+2 K"] > 0.4 and f["probabilistic", "swap K"] > 0.9
              and f["probabilistic", "sign K"] > 0.99)
    assert not (inside and caught), name
