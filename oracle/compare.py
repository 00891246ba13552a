"""Acceptance rule for the context-KV write: device caches vs the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Rule, per written element (a written row is cache_l[slot / bs, h, slot % bs, :]
for a token with slot >= 0):
  * V in a bf16 cache: bit-exact (the unfused path stores V unchanged);
  * K in a bf16 cache: ordinal bf16 distance <= 1 from the oracle's code or
    from one of its near-tie alternates;
  * fp8 cache, K and V: ordinal e4m3 distance <= 1 from the oracle's code or
    an alternate; +0 and -0 count as equal.
Every byte that is not in a written row must equal its value before the call.

Ordinal distance treats a sign-magnitude code as the integer +mag or -mag,
so neighbouring representable values are one apart and both zeros are 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def ordinal_bf16(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int64)
    mag = c & 0x7FFF
    return np.where(c & 0x8000, -mag, mag)


def ordinal_e4m3(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


@dataclass
class PartStats:
    n: int = 0
    exact: int = 0         # bit-equal to the oracle's code
    within1: int = 0       # not bit-equal, ordinal distance <= 1 (+0 vs -0 is 0)
    by_alternate: int = 0  # farther than 1 from the code, within 1 of an alternate
    fail: int = 0
    max_dist: int = 0

    def as_dict(self):
        return dict(n=self.n, exact=self.exact, within1=self.within1,
                    by_alternate=self.by_alternate, fail=self.fail, max_dist=self.max_dist)


@dataclass
class LayerReport:
    k: PartStats = field(default_factory=PartStats)
    v: PartStats = field(default_factory=PartStats)
    untouched_bad: int = 0


@dataclass
class Report:
    layers: list
    fp8: bool

    @property
    def failures(self) -> int:
        return sum(l.k.fail + l.v.fail + l.untouched_bad for l in self.layers)

    def summary(self) -> dict:
        out = {"fp8": self.fp8, "failures": self.failures, "layers": []}
        for l in self.layers:
            out["layers"].append({"k": l.k.as_dict(), "v": l.v.as_dict(),
                                  "untouched_bad": l.untouched_bad})
        return out

    def totals(self) -> dict:
        tot = {}
        for part in ("k", "v"):
            agg = PartStats()
            for l in self.layers:
                s = getattr(l, part)
                agg.n += s.n
                agg.exact += s.exact
                agg.within1 += s.within1
                agg.by_alternate += s.by_alternate
                agg.fail += s.fail
                agg.max_dist = max(agg.max_dist, s.max_dist)
            tot[part] = agg.as_dict()
        tot["untouched_bad"] = sum(l.untouched_bad for l in self.layers)
        tot["failures"] = self.failures
        return tot


def written_rows(slot_mapping: np.ndarray, nkv: int, block_size: int) -> np.ndarray:
    """Flat row indices (into a cache viewed as [-1, 256]) of every written
    row, ordered by (token, head)."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    valid = slots[slots >= 0]
    blk = valid // block_size
    off = valid % block_size
    h = np.arange(nkv, dtype=np.int64)
    rows = (blk[:, None] * nkv + h[None, :]) * block_size + off[:, None]
    return rows.reshape(-1)


def compare(device_caches, oracle_result, slot_mapping, fp8: bool, sentinel: int,
            block_size: int | None = None) -> Report:
    """Compare device caches (numpy, same dtype/shape as the oracle's) with
    the oracle's caches and alternates.  ``slot_mapping`` is [num_ctx]
    (shared) or [L, num_ctx] (per layer).  ``sentinel`` is the byte/element
    value every cache held before the call."""
    oc = oracle_result.caches
    L = len(oc)
    nkv = oc[0].shape[1]
    bs = oc[0].shape[2] if block_size is None else block_size
    slots = np.asarray(slot_mapping, dtype=np.int64)
    per_layer = slots.ndim == 2          # [L, num_ctx]: one mapping per layer
    ordf = ordinal_e4m3 if fp8 else ordinal_bf16
    layers = []
    for l in range(L):
        rows = written_rows(slots[l] if per_layer else slots, nkv, bs)
        rep = LayerReport()
        dev = np.asarray(device_caches[l]).reshape(-1, 256)
        ora = oc[l].reshape(-1, 256)
        assert dev.dtype == ora.dtype and dev.shape == ora.shape

        # untouched bytes: everything outside the written rows keeps the sentinel
        mask = np.ones(dev.shape[0], dtype=bool)
        mask[rows] = False
        rep.untouched_bad = int(np.count_nonzero(dev[mask] != sentinel))

        g = dev[rows]
        o = ora[rows]
        # alternates of this layer, keyed by flat element index
        sel = oracle_result.alt_layer == l
        alt_idx = oracle_result.alt_index[sel]
        alt_cnt = oracle_result.alt_count[sel]
        alt_codes = oracle_result.alt_codes[sel]
        alt_map = {int(i): alt_codes[k, :alt_cnt[k]] for k, i in enumerate(alt_idx)}

        for part, sl, stats in (("k", slice(0, 128), rep.k), ("v", slice(128, 256), rep.v)):
            gp = g[:, sl]
            op = o[:, sl]
            stats.n = gp.size
            if part == "v" and not fp8:
                neq = gp != op
                stats.exact = int(gp.size - np.count_nonzero(neq))
                stats.fail = int(np.count_nonzero(neq))
                if stats.fail:
                    stats.max_dist = int(np.abs(ordf(gp[neq]) - ordf(op[neq])).max())
                continue
            d = np.abs(ordf(gp) - ordf(op))
            same = gp == op
            stats.exact = int(np.count_nonzero(same))
            stats.within1 = int(np.count_nonzero((d <= 1) & ~same))
            far = np.argwhere(d > 1)
            maxd = int(d.max()) if d.size else 0
            for r_i, c_i in far:
                flat = int(rows[r_i]) * 256 + sl.start + int(c_i)
                cands = alt_map.get(flat)
                ok = False
                if cands is not None:
                    dd = np.abs(ordf(np.asarray(cands)) - ordf(np.asarray([gp[r_i, c_i]])))
                    ok = bool(dd.min() <= 1)
                if ok:
                    stats.by_alternate += 1
                else:
                    stats.fail += 1
            stats.max_dist = maxd
        layers.append(rep)
    return Report(layers=layers, fp8=fp8)


# ------------------------------------------------ the draft-block insert ----
#
# The same rule for dspark_qknorm_rope_kv_insert's three outputs:
#   * qkv, q and k heads: ordinal bf16 distance <= 1 from the oracle's code or
#     an alternate; v heads: bit-exact (they are not touched);
#   * the cache: as above (K bf16 within 1 / alternates, V bf16 bit-exact,
#     fp8 within 1 e4m3 step), and every row no slot names keeps the sentinel;
#   * q_fp8: ordinal e4m3 distance <= 1 from the oracle's code or an alternate.

def _grade(dev: np.ndarray, ora: np.ndarray, flat_index: np.ndarray, alt_map: dict,
           ordf, bit_exact: bool) -> PartStats:
    s = PartStats(n=int(dev.size))
    if dev.size == 0:
        return s
    same = dev == ora
    s.exact = int(np.count_nonzero(same))
    if bit_exact:
        s.fail = int(dev.size - s.exact)
        if s.fail:
            s.max_dist = int(np.abs(ordf(dev[~same]) - ordf(ora[~same])).max())
        return s
    d = np.abs(ordf(dev) - ordf(ora))
    s.within1 = int(np.count_nonzero((d <= 1) & ~same))
    s.max_dist = int(d.max())
    for pos in np.flatnonzero(d.reshape(-1) > 1):
        cands = alt_map.get(int(flat_index.reshape(-1)[pos]))
        got = dev.reshape(-1)[pos]
        if cands is not None and np.abs(ordf(np.asarray(cands)) - ordf(np.asarray([got]))).min() <= 1:
            s.by_alternate += 1
        else:
            s.fail += 1
    return s


@dataclass
class InsertReport:
    parts: dict
    untouched_bad: int

    @property
    def failures(self) -> int:
        return sum(p.fail for p in self.parts.values()) + self.untouched_bad

    def totals(self) -> dict:
        out = {k: v.as_dict() for k, v in self.parts.items()}
        out["untouched_bad"] = self.untouched_bad
        out["failures"] = self.failures
        return out


def compare_insert(dev_qkv, dev_cache, dev_q_fp8, oracle_result, num_heads: int,
                   num_kv_heads: int, slot_mapping, fp8: bool, sentinel: int) -> InsertReport:
    """Grade the device outputs of the draft-block insert against the oracle's
    (an oracle.InsertResult); dev_cache / dev_q_fp8 may be None when the call
    had no insert / no q fp8 output."""
    H, nkv = num_heads, num_kv_heads
    r = oracle_result

    def alt_map(tag):
        sel = r.alt_tag == tag
        idx, cnt, codes = r.alt_index[sel], r.alt_count[sel], r.alt_codes[sel]
        return {int(i): codes[k, :cnt[k]] for k, i in enumerate(idx)}

    parts = {}
    dq = np.asarray(dev_qkv)
    oq = r.qkv
    assert dq.shape == oq.shape and dq.dtype == oq.dtype
    T, width = oq.shape
    flat = np.arange(T * width, dtype=np.int64).reshape(T, width)
    m = alt_map(0)
    qe, ke = H * 128, (H + nkv) * 128
    parts["q"] = _grade(dq[:, :qe], oq[:, :qe], flat[:, :qe], m, ordinal_bf16, False)
    parts["k"] = _grade(dq[:, qe:ke], oq[:, qe:ke], flat[:, qe:ke], m, ordinal_bf16, False)
    parts["v"] = _grade(dq[:, ke:], oq[:, ke:], flat[:, ke:], m, ordinal_bf16, True)

    untouched = 0
    if r.cache is not None:
        dc = np.asarray(dev_cache)
        oc = r.cache
        assert dc.shape == oc.shape and dc.dtype == oc.dtype
        bs = oc.shape[2]
        rows = written_rows(slot_mapping, nkv, bs)
        d2 = dc.reshape(-1, 256)
        o2 = oc.reshape(-1, 256)
        mask = np.ones(d2.shape[0], dtype=bool)
        mask[rows] = False
        untouched = int(np.count_nonzero(d2[mask] != sentinel))
        cflat = rows[:, None] * 256 + np.arange(256, dtype=np.int64)[None, :]
        m = alt_map(1)
        ordf = ordinal_e4m3 if fp8 else ordinal_bf16
        parts["cache_k"] = _grade(d2[rows, :128], o2[rows, :128], cflat[:, :128], m, ordf, False)
        parts["cache_v"] = _grade(d2[rows, 128:], o2[rows, 128:], cflat[:, 128:], m, ordf,
                                  not fp8)
    if r.q_fp8 is not None:
        df = np.asarray(dev_q_fp8)
        assert df.shape == r.q_fp8.shape
        qflat = np.arange(df.size, dtype=np.int64).reshape(df.shape)
        parts["q_fp8"] = _grade(df, r.q_fp8, qflat, alt_map(2), ordinal_e4m3, False)
    return InsertReport(parts=parts, untouched_bad=untouched)


# ------------------------------------- projection + write on general data ----
#
# With Gaussian data the device's fp32 accumulation of the projection is not
# exact, so its bf16 all_kv may differ from the exactly rounded value.  The
# acceptance is then an interval per value, derived from the arithmetic:
#   * all_kv: |acc - exact| <= b, where b bounds the fp32 summation error of
#     the hidden-size dot product (exact bf16 x bf16 products), either in the
#     worst case for any order (Higham, Accuracy and Stability of Numerical
#     Algorithms, 2nd ed., eq. 3.5 and section 4.2: gamma_n sum|z W|,
#     gamma_n = n u / (1 - n u)) or, tighter, by the probabilistic bound of
#     Higham and Mary (SIAM J. Sci. Comput. 41(5), 2019, Theorem 3.1): with
#     rounding errors modelled as independent and of mean zero, for any order
#     |acc - exact| <= gamma~_n(lam) sum|z W|, gamma~_n(lam) = exp(lam sqrt(n)
#     u + n u^2 / (1 - u)) - 1, except with probability at most
#     2 n exp(-lam^2 (1 - u)^2 / 2) per value.  bf16 rounding is monotone, so
#     the device's all_kv lies in [RNE(exact - b), RNE(exact + b)];
#   * K (write_intervals): the norm's r over the interval box, x r (1 + w)
#     over the corners, RoPE over the corners, each fp32 stage widened by
#     2^-19 relative (fp32 evaluation and v_rsq_f32), then rounded to bf16
#     outward;
#   * fp8: e4m3 of value / scale is monotone, so the interval maps through.

U32 = 2.0 ** -24            # unit roundoff of fp32
U64 = 2.0 ** -53            # unit roundoff of fp64
_WIDEN = 2.0 ** -19
BF16_MIN_SUBNORMAL = 2.0 ** -133


def rne_bf16(x64):
    """Each float64 value rounded once, to nearest with ties to even, onto
    the bf16 grid (8 significant bits, exponents down to -126, subnormal step
    2^-133), returned as float64.  Values beyond the bf16 range are not
    expected here."""
    x = np.asarray(x64, dtype=np.float64)
    m, e = np.frexp(x)                        # x = m 2^e, 0.5 <= |m| < 1
    # the grid step at x: 2^(e - 8) for normal bf16 values, 2^-133 below 2^-126
    step_exp = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(x, -step_exp)), step_exp)


def gamma(n: int, u: float = U32) -> float:
    """Worst-case relative error factor of n roundings: n u / (1 - n u)."""
    return n * u / (1.0 - n * u)


def gamma_prob(n: int, lam: float, u: float = U32) -> float:
    """Higham and Mary's probabilistic factor gamma~_n(lam)."""
    return float(np.expm1(lam * np.sqrt(n) * u + n * u * u / (1.0 - u)))


def prob_bound_failure(n: int, lam: float, u: float = U32) -> float:
    """Per-value probability that the probabilistic bound does not hold
    (the model's union bound): 2 n exp(-lam^2 (1 - u)^2 / 2)."""
    return float(2.0 * n * np.exp(-lam * lam * (1.0 - u) ** 2 / 2.0))


def projection_bound(abs_sum, hidden: int, lam=None, sum_err=0.0):
    """Bound b on |device fp32 dot product - exact| for dot products of
    `hidden` exact products with sum of |products| abs_sum: the worst case
    for any order when lam is None, else the probabilistic bound at lam.
    sum_err: how far the caller's exact sums and abs_sum may themselves be
    off (fp64 evaluation), added on top."""
    g = gamma(hidden) if lam is None else gamma_prob(hidden, lam)
    return g * (np.asarray(abs_sum, np.float64) + sum_err) + sum_err


def all_kv_interval(exact, b):
    """[lo, hi] (bf16 values as float64) that the device's bf16 all_kv must
    lie in, given the exact dot products and the bound b."""
    return rne_bf16(exact - b), rne_bf16(exact + b)


def _widen(lo, hi):
    return (lo - np.abs(lo) * _WIDEN - 1e-38, hi + np.abs(hi) * _WIDEN + 1e-38)


def write_intervals(exact, b, k_norm_weight, cos, sin, rotary_dim, kv, eps=1e-6):
    """Bounds [lo, hi] (float64, bf16 values) of the stored values of one
    all_kv row group.  exact, b: [T, 128] exact dot products and their error
    bounds for one (layer, kv, head); k_norm_weight: [128] float; cos, sin:
    [T, R/2] float; kv 0 = K."""
    xlo, xhi = all_kv_interval(exact, b)
    if kv == 1:
        return xlo, xhi
    # the norm's r over the box: mean x^2 between the smallest and largest squares
    sq_lo = np.where((xlo <= 0) & (xhi >= 0), 0.0, np.minimum(xlo * xlo, xhi * xhi))
    sq_hi = np.maximum(xlo * xlo, xhi * xhi)
    eps = float(np.float32(eps))
    r_lo = 1.0 / np.sqrt(sq_hi.mean(axis=1, keepdims=True) + eps)
    r_hi = 1.0 / np.sqrt(sq_lo.mean(axis=1, keepdims=True) + eps)
    r_lo, r_hi = _widen(r_lo, r_hi)
    g = 1.0 + k_norm_weight[None, :]
    c = np.stack([xlo * r_lo * g, xlo * r_hi * g, xhi * r_lo * g, xhi * r_hi * g])
    ylo, yhi = _widen(c.min(axis=0), c.max(axis=0))
    ylo, yhi = rne_bf16(ylo), rne_bf16(yhi)
    R = rotary_dim
    h = R // 2
    klo, khi = ylo.copy(), yhi.copy()
    a_lo, a_hi = ylo[:, :h], yhi[:, :h]
    p_lo, p_hi = ylo[:, h:R], yhi[:, h:R]

    def prod(lo, hi, s):
        v = np.stack([lo * s, hi * s])
        return v.min(axis=0), v.max(axis=0)

    ac_lo, ac_hi = prod(a_lo, a_hi, cos)
    ps_lo, ps_hi = prod(p_lo, p_hi, sin)
    pc_lo, pc_hi = prod(p_lo, p_hi, cos)
    as_lo, as_hi = prod(a_lo, a_hi, sin)
    f_lo, f_hi = _widen(ac_lo - ps_hi, ac_hi - ps_lo)     # first half: a c - p s
    s_lo, s_hi = _widen(pc_lo + as_lo, pc_hi + as_hi)     # second half: p c + a s
    klo[:, :h], khi[:, :h] = rne_bf16(f_lo), rne_bf16(f_hi)
    klo[:, h:R], khi[:, h:R] = rne_bf16(s_lo), rne_bf16(s_hi)
    return klo, khi
