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
