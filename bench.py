#!/usr/bin/env python3
"""Benchmark of the fused DSpark context-KV write on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one write (norm + RoPE + store of every layer's context K/V) over
one batch of synthetic input already resident in HBM.  The headline line is
the 4 x 1024-token prefill chunk with bf16 caches (L = 5 draft layers, 8 kv
heads, 128-dim heads, rotary dim 64); the fp8, long-context and decode
workloads are measured in the same run and reported under "workloads".

Throughput is algorithmic bytes / time: all_kv rows read for valid tokens,
cache rows written, the cos/sin row and position of each valid token, every
slot, and the norm weights.  Inputs rotate over several independently drawn
sets so that one cycle's footprint exceeds the 256 MB last-level cache and
the figure is HBM bandwidth, not cache bandwidth.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from speculative_decoding_draft_02_amd import _lib  # noqa: E402
from speculative_decoding_draft_02_amd import workloads as W  # noqa: E402
from speculative_decoding_draft_02_amd.writer import AttnLayer, DSparkContextKVWriter  # noqa: E402

METRIC = "context-KV write HBM GB/s (% of MI355X peak) and token-layers/s"
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["speculative_decoding_draft_02_amd/csrc/ctx_kv_kernel.hip",
                  "speculative_decoding_draft_02_amd/csrc/ctx_kv_writer.cpp",
                  "speculative_decoding_draft_02_amd/csrc/ctx_kv_args.h",
                  "speculative_decoding_draft_02_amd/csrc/writer_state.h",
                  "speculative_decoding_draft_02_amd/csrc/device_common.h",
                  "speculative_decoding_draft_02_amd/csrc/qknorm_insert_kernel.hip",
                  "speculative_decoding_draft_02_amd/csrc/qknorm_insert.cpp",
                  "speculative_decoding_draft_02_amd/csrc/qknorm_insert_args.h"]
HEADLINE = 1   # index of the prefill bf16 workload


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bf16_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


class Setup:
    """Caches + writer for a workload shape, and `n_sets` input sets."""

    def __init__(self, index: int, n_sets: int, dev, layer_slots: bool = False, tp: int = 1):
        self.index = index
        self.sets = [W.make(index, variant=v) for v in range(n_sets)]
        if tp > 1:
            # every rank's share of every set, each in relocated blocks: a
            # cycle still reads and writes more than the last-level cache
            self.sets = [W.relocate_blocks(W.head_shard(s, tp, r), seed=31 * v + r)
                         for v, s in enumerate(self.sets) for r in range(tp)]
        if layer_slots:
            self.sets = [W.per_layer_slots(s, seed=77 + v, pad_fraction=0.02)
                         for v, s in enumerate(self.sets)]
        wl = self.sets[0]
        self.wl = wl
        layers = []
        for l in range(wl.num_layers):
            if wl.fp8:
                cache = torch.full(wl.cache_shape, 0xFF, dtype=torch.uint8, device=dev)
            else:
                cache = torch.full(wl.cache_shape, -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
            ks = torch.tensor([float(wl.k_scales[l])], dtype=torch.float32, device=dev)
            vs = torch.tensor([float(wl.v_scales[l])], dtype=torch.float32, device=dev)
            layers.append(AttnLayer(cache, ks, vs, "fp8" if wl.fp8 else "auto"))
        self.layers = layers
        self.writer = DSparkContextKVWriter(layers)
        self.inputs = []
        for s in self.sets:
            self.inputs.append(dict(
                all_kv=bf16_dev(s.all_kv, dev), w=bf16_dev(s.k_norm_weight, dev),
                positions=torch.from_numpy(s.positions).to(dev),
                cos_sin=bf16_dev(s.cos_sin, dev),
                slots=torch.from_numpy(s.slot_mapping).to(dev)))
        # one checked call through the Python writer builds the tables
        i0 = self.inputs[0]
        self.writer(i0["all_kv"], i0["w"], wl.eps, i0["positions"], i0["cos_sin"],
                    wl.rotary_dim, i0["slots"])
        self.layer_slots = layer_slots
        torch.cuda.synchronize()
        self.handle = self.writer._handle
        self.bytes = [s.algorithmic_bytes() for s in self.sets]
        self.token_layers = [s.token_layers() for s in self.sets]
        # C-ABI argument tuples, built once: the timed loop only calls
        lib = _lib.load()
        if layer_slots:
            self._write = lib.dspark_ctx_kv_writer_write_layer_slots
            self._tables = [(ctypes.c_void_p * wl.num_layers)(
                *[i["slots"][l].data_ptr() for l in range(wl.num_layers)]) for i in self.inputs]
            slot_args = [ctypes.cast(t, ctypes.c_void_p) for t in self._tables]
        else:
            self._write = lib.dspark_ctx_kv_writer_write
            slot_args = [i["slots"].data_ptr() for i in self.inputs]
        # every set passes its own token count (sets of one workload may
        # differ in it: the decode batches draw the tokens per request)
        for st in self.sets:
            assert (st.num_layers, st.num_kv_heads, st.cache_shape, st.fp8) == \
                (wl.num_layers, wl.num_kv_heads, wl.cache_shape, wl.fp8)
        self._args = [(self.handle, i["all_kv"].data_ptr(), st.num_ctx, st.num_layers,
                       st.num_kv_heads, i["w"].data_ptr(), st.eps, i["positions"].data_ptr(),
                       i["cos_sin"].data_ptr(), i["cos_sin"].shape[0], st.rotary_dim, sa)
                      for st, i, sa in zip(self.sets, self.inputs, slot_args)]

    def launch(self, k: int, stream_ptr) -> None:
        """One write of input set k % n through the C ABI (the same tensors
        the Python writer checked when it built the tables)."""
        st = self._write(*self._args[k % len(self._args)], stream_ptr)
        if st != _lib.OK:
            raise RuntimeError(_lib.dspark_ctx_kv_last_error())


class InsertSetup:
    """The draft block's QK-norm / RoPE / KV insert: `n_sets` independently
    drawn draft blocks (qkv, positions, slots, q fp8 output) over one cache,
    so that a cycle of launches streams more than the last-level cache
    holds.  Every launch is one call of the C ABI."""

    def __init__(self, index: int, n_sets: int, dev):
        self.sets = [W.insert_make(index, variant=v) for v in range(n_sets)]
        wl = self.sets[0]
        self.wl = wl
        if wl.fp8:
            self.cache = torch.full(wl.cache_shape, 0xFF, dtype=torch.uint8, device=dev)
        else:
            self.cache = torch.full(wl.cache_shape, -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
        self.ks = torch.tensor([wl.k_scale], dtype=torch.float32, device=dev)
        self.vs = torch.tensor([wl.v_scale], dtype=torch.float32, device=dev)
        self.qw = bf16_dev(wl.q_norm_weight, dev)
        self.kw = bf16_dev(wl.k_norm_weight, dev)
        self.cs = bf16_dev(wl.cos_sin, dev)
        self.inputs = []
        for s in self.sets:
            self.inputs.append(dict(
                qkv=bf16_dev(s.qkv, dev), positions=torch.from_numpy(s.positions).to(dev),
                slots=torch.from_numpy(s.slot_mapping).to(dev),
                qf=torch.empty((s.num_tokens, s.num_heads * 128), dtype=torch.uint8, device=dev)
                if s.q_fp8 else None))
        self.bytes = [s.algorithmic_bytes() for s in self.sets]
        self.token_layers = [s.num_tokens for s in self.sets]
        lib = _lib.load()
        self._call = lib.dspark_qknorm_rope_kv_insert
        for st in self.sets:       # one cache and one set of weights serve every set
            assert (st.num_heads, st.num_kv_heads, st.cache_shape, st.fp8, st.rotary_dim) == \
                (wl.num_heads, wl.num_kv_heads, wl.cache_shape, wl.fp8, wl.rotary_dim)
        self._args = [(i["qkv"].data_ptr(), st.num_tokens, self.qw.data_ptr(), self.kw.data_ptr(),
                       self.cs.data_ptr(), self.cs.shape[0], i["positions"].data_ptr(),
                       wl.num_heads, wl.num_kv_heads, wl.rotary_dim, wl.eps,
                       i["slots"].data_ptr(), self.cache.data_ptr(), wl.num_blocks,
                       wl.block_size, _lib.KV_FP8_E4M3 if wl.fp8 else _lib.KV_AUTO,
                       self.ks.data_ptr() if wl.fp8 else None,
                       self.vs.data_ptr() if wl.fp8 else None,
                       i["qf"].data_ptr() if i["qf"] is not None else None, wl.q_scale)
                      for st, i in zip(self.sets, self.inputs)]

    def launch(self, k: int, stream_ptr) -> None:
        st = self._call(*self._args[k % len(self._args)], stream_ptr)
        if st != _lib.OK:
            raise RuntimeError(_lib.dspark_ctx_kv_last_error())


# The GPU's clock settles over the first ~20 ms of sustained work, so every
# timed region is preceded by at least this much back-to-back work of the
# same launch, whatever --warmup says (--warmup sets the minimum number of
# warm-up calls); the timed region itself is exactly --steps launches.
WARMUP_FLOOR_S = 0.2
# untimed launches queued between the synchronisation and the start event
PREROLL = 4


def warm_up(launch, calls: int, floor_s: float = None) -> int:
    """At least `calls` calls of launch(k) and at least floor_s seconds
    (default WARMUP_FLOOR_S) of them (checked every 64 calls at a
    synchronisation point); returns the number of calls made."""
    floor_s = WARMUP_FLOOR_S if floor_s is None else floor_s
    k = 0
    t0 = time.perf_counter()
    while k < calls or time.perf_counter() - t0 < floor_s:
        launch(k)
        k += 1
        if k % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return k


def time_eager(setup: Setup, steps: int, warmup: int, stream):
    """Warm up (warm_up), then time exactly `steps` back-to-back launches
    with one HIP event pair around the region on the launch stream.  A
    second, untimed pass with an event pair around every launch gives the
    spread of single kernel durations."""
    sp = stream.cuda_stream
    with torch.cuda.stream(stream):
        warmup = warm_up(lambda k: setup.launch(k, sp), warmup)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        # untimed launches queued ahead of the start event: the region starts
        # on a busy GPU, so the host's latency to its first launch is not in it
        for k in range(PREROLL):
            setup.launch(warmup + k, sp)
        warmup += PREROLL
        start.record(stream)
        for k in range(steps):
            setup.launch(warmup + k, sp)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        region = start.elapsed_time(end) * 1e-3
        # diagnostic pass (not the timed region): one event pair per launch
        n_diag = min(steps, 50)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_diag)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_diag)]
        for k in range(n_diag):
            starts[k].record(stream)
            setup.launch(k, sp)
            ends[k].record(stream)
        torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) * 1e-3
    nbytes = np.array([setup.bytes[(warmup + k) % len(setup.bytes)] for k in range(steps)])
    ntl = np.array([setup.token_layers[(warmup + k) % len(setup.bytes)] for k in range(steps)])
    return dict(region_s=region, wall_s=wall, single_s=per, bytes=nbytes, token_layers=ntl)


def time_graph(setup, steps: int, warmup: int, stream, per_graph: int = 50):
    """Capture `per_graph` writes in one HIP graph (rotating over the setup's
    input sets) and replay it until `steps` writes have run; per-call time =
    region / steps."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            sp = torch.cuda.current_stream().cuda_stream
            for k in range(per_graph):
                setup.launch(k, sp)
        warm_up(lambda k: g.replay(), max(1, warmup // per_graph))
        replays = max(1, steps // per_graph)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g.replay()          # untimed, queued ahead of the start event
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
    region = start.elapsed_time(end) * 1e-3
    del g
    n = replays * per_graph
    nb = [setup.bytes[k % len(setup.bytes)] for k in range(per_graph)]
    ntl = [setup.token_layers[k % len(setup.bytes)] for k in range(per_graph)]
    return dict(region_s=region, per_call_s=region / n, calls=n, bytes=float(np.mean(nb)),
                token_layers=float(np.mean(ntl)))


def copy_reference(dev, stream, nbytes: int = 82_214_912, reps: int = 50):
    """Device-to-device copy of one prefill call's all_kv volume (reads and
    writes the same byte count as the bf16 write's main streams): the
    practical bandwidth ceiling of a pure stream on this GPU, for context."""
    src = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(4)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(4)]
    for b in src + dst:
        b.fill_(1)
    with torch.cuda.stream(stream):
        for k in range(8):
            dst[k % 4].copy_(src[k % 4])
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(reps):
            dst[k % 4].copy_(src[k % 4])
        end.record(stream)
        torch.cuda.synchronize()
    t = start.elapsed_time(end) * 1e-3 / reps
    del src, dst
    return {"bytes_read_plus_written": 2 * nbytes, "us": t * 1e6, "GB_s": 2 * nbytes / t / 1e9,
            "how": "torch copy_ of %d bytes, 4 buffer pairs rotated, %d copies" % (nbytes, reps)}


def unfused_write(all_kv, k_norm_weight, eps, positions, cos_sin, rotary_dim, slot_mapping,
                  caches, fp8, k_scales, v_scales):
    """The base path the fused write replaces (vLLM API page
    "vllm.models.minimax_m3.common.ops.dspark_context_kv", module docstring),
    in PyTorch ops on the GPU: the permute copy, one Gemma K norm per layer and
    a stack, positions.repeat, NeoX rotary on the stacked K, and one cache
    write per layer.  A measurement comparator (and a cross-check of the
    oracle), never a fallback: the product path has none.  Unlike vLLM's
    reshape_and_cache_flash kernel, the PyTorch cache write needs the valid
    token list, so this chain syncs once per call (torch.nonzero)."""
    N, L, _, H, D = all_kv.shape
    R = rotary_dim
    all_k = all_kv[:, :, 0].permute(1, 0, 2, 3).contiguous()       # [L, N, H, D]
    all_v = all_kv[:, :, 1].permute(1, 0, 2, 3).contiguous()
    normed = []
    for l in range(L):
        x = all_k[l].float()
        var = x.pow(2).mean(dim=-1, keepdim=True)
        normed.append((x * torch.rsqrt(var + eps) * (1.0 + k_norm_weight[l].float()))
                      .to(torch.bfloat16))
    k = torch.stack(normed).view(L * N, H, D)
    pos = positions.repeat(L)
    cs = cos_sin[pos]
    cos = cs[:, : R // 2].float().unsqueeze(1)
    sin = cs[:, R // 2:].float().unsqueeze(1)
    x1 = k[..., : R // 2].float()
    x2 = k[..., R // 2: R].float()
    k[..., : R // 2] = (x1 * cos - x2 * sin).to(torch.bfloat16)
    k[..., R // 2: R] = (x2 * cos + x1 * sin).to(torch.bfloat16)
    k = k.view(L, N, H, D)
    valid = torch.nonzero(slot_mapping >= 0).squeeze(1)
    s = slot_mapping[valid]
    bs = caches[0].shape[2]
    heads = torch.arange(H, device=s.device)
    rows = ((s // bs)[:, None] * H + heads[None, :]) * bs + (s % bs)[:, None]   # [V, H]
    rows = rows.reshape(-1)
    for l in range(L):
        kk = k[l, valid].reshape(-1, D)
        vv = all_v[l, valid].reshape(-1, D)
        if fp8:
            kk = (kk.float() / k_scales[l]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
            vv = (vv.float() / v_scales[l]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        flat = caches[l].view(-1, 2 * D)
        flat[rows] = torch.cat([kk, vv], dim=1)


class UnfusedSetup:
    """The same workload and input sets, written by the unfused PyTorch chain."""

    def __init__(self, setup: "Setup", dev):
        self.s = setup
        self.caches = [a.kv_cache for a in setup.layers]
        self.ks = [a._k_scale for a in setup.layers]
        self.vs = [a._v_scale for a in setup.layers]
        self.bytes = setup.bytes
        self.token_layers = setup.token_layers

    def launch(self, k: int, stream_ptr) -> None:
        wl = self.s.wl
        i = self.s.inputs[k % len(self.s.inputs)]
        unfused_write(i["all_kv"], i["w"], wl.eps, i["positions"], i["cos_sin"], wl.rotary_dim,
                      i["slots"], self.caches, wl.fp8, self.ks, self.vs)


def time_unfused(setup: UnfusedSetup, steps: int, warmup: int, stream):
    """Wall-clock-free timing of the unfused chain: HIP events around `steps`
    calls on the stream (each call syncs once for its valid-token list)."""
    with torch.cuda.stream(stream):
        for k in range(warmup):
            setup.launch(k, None)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for k in range(steps):
            setup.launch(warmup + k, None)
        end.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / steps


def count_device_ops(fn, stream):
    """Device operations (kernels, copies, fills) one call of fn puts on the
    GPU, counted with torch's profiler outside any timed region; None if the
    profiler is unavailable."""
    try:
        from torch.profiler import ProfilerActivity, profile
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            with profile(activities=[ProfilerActivity.CUDA]) as prof:
                fn()
                torch.cuda.synchronize()
        return sum(1 for e in prof.events()
                   if e.device_type == torch.autograd.DeviceType.CUDA)
    except Exception:   # profiler support differs between builds: report nothing
        return None


BF16_MFMA_PEAK_TFLOPS = 2500.0


class ProjectSetup:
    """The step before the write at one workload: context states, hidden-norm
    weight, the stacked K/V projection and the layers' caches."""

    def __init__(self, index: int, dev):
        wl = W.project_make(index)
        self.wl = wl
        layers = []
        for l in range(wl.num_layers):
            shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, 256)
            if wl.fp8:
                cache = torch.full(shape, 0xFF, dtype=torch.uint8, device=dev)
            else:
                cache = torch.full(shape, -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
            layers.append(AttnLayer(cache, torch.tensor([float(wl.k_scales[l])], device=dev),
                                    torch.tensor([float(wl.v_scales[l])], device=dev),
                                    "fp8" if wl.fp8 else "auto"))
        self.layers = layers
        self.writer = DSparkContextKVWriter(layers)
        self.states = bf16_dev(wl.states, dev)
        self.hw = bf16_dev(wl.hidden_norm_weight, dev)
        self.W = bf16_dev(wl.kv_weight, dev)
        self.kw = bf16_dev(wl.k_norm_weight, dev)
        self.pos = torch.from_numpy(wl.positions).to(dev)
        self.cs = bf16_dev(wl.cos_sin, dev)
        self.slots = torch.from_numpy(wl.slot_mapping).to(dev)
        self.z = torch.empty_like(self.states)
        from speculative_decoding_draft_02_amd.project import hidden_norm, pack_kv_weight
        self._hidden_norm = hidden_norm
        self._pack = pack_kv_weight
        self.Wp = pack_kv_weight(self.W)

    def pack(self):
        """The one-time packing of the weight (not part of a step)."""
        self.Wp = self._pack(self.W)

    def norm(self):
        self._hidden_norm(self.states, self.hw, self.wl.eps, out=self.z)

    def project_write(self):
        wl = self.wl
        self.writer.project_write(self.z, self.W, self.kw, wl.eps, self.pos, self.cs,
                                  wl.rotary_dim, self.slots)

    def project_write_packed(self):
        wl = self.wl
        self.writer.project_write(self.z, self.Wp, self.kw, wl.eps, self.pos, self.cs,
                                  wl.rotary_dim, self.slots)

    def unfused(self):
        """hidden norm, the projection as a library GEMM (torch's linear, on
        hipBLASLt), all_kv stored, then the context write kernel."""
        wl = self.wl
        self.norm()
        all_kv = torch.nn.functional.linear(self.z, self.W)
        self.writer(all_kv.view(wl.num_ctx, wl.num_layers, 2, wl.num_kv_heads, 128), self.kw,
                    wl.eps, self.pos, self.cs, wl.rotary_dim, self.slots)


def time_calls(fn, steps: int, warmup: int, stream) -> float:
    """Seconds per call of fn (a sequence of launches) over `steps` calls
    bracketed by HIP events on the stream."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / steps


def small_copy_reference(nbytes_moved: float, n_bufs: int, stream, per_graph: int = 64,
                         replays: int = 16):
    """Graph-replayed device copies that read and write nbytes_moved / 2
    bytes each, over n_bufs rotated buffer pairs: what a plain stream of the
    same size achieves, the practical ceiling of a small launch."""
    n = int(nbytes_moved // 2) // 16 * 16
    dev = torch.device("cuda:0")
    src = [torch.ones(n, dtype=torch.uint8, device=dev) for _ in range(n_bufs)]
    dst = [torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(n_bufs)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for k in range(per_graph):
                dst[k % n_bufs].copy_(src[k % n_bufs])
        g.replay()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(replays):
            g.replay()
        end.record(stream)
        torch.cuda.synchronize()
    t = start.elapsed_time(end) * 1e-3 / (replays * per_graph)
    del g, src, dst
    return {"us_per_copy": t * 1e6, "GB_s": 2 * n / t / 1e9,
            "how": "torch copy_ of %d bytes under HIP-graph replay, %d buffer pairs" % (n, n_bufs)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# the box this bench runs on allots 16 CPUs to each GPU: the oracle's
# all-core leg uses at most that many threads
CPU_THREAD_CAP = 16


def token_prefix(wl, n: int):
    """The workload's first n tokens (same caches, tables and weights)."""
    import dataclasses
    return dataclasses.replace(wl, num_ctx=n, all_kv=wl.all_kv[:n], positions=wl.positions[:n],
                               slot_mapping=wl.slot_mapping[..., :n])


def cpu_baseline(target_s: float = 1.0):
    """The oracle (plain C in fp64 with near-tie tracking; test
    infrastructure: only this leg of the bench uses it) on this host's
    cores, per workload, on a bounded sample: the workload's first tokens,
    as many as one single-threaded pass covers in about target_s (the whole
    call when it is smaller), timed single-threaded and with one contiguous
    token range per thread (its C code runs with the GIL released), best of
    3 runs each; rates are the sample's algorithmic bytes and token-layers
    over its time.  Reported as a baseline for context, not as a target."""
    sys.path.insert(0, ROOT)
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    oracle.build()
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(CPU_THREAD_CAP, avail))
    per = {}
    for index, name in enumerate(W.NAMES):
        full = W.make(index)

        def timed(wl, n_threads, runs):
            caches = wl.new_host_caches()
            bounds = np.linspace(0, wl.num_ctx, n_threads + 1).astype(int)

            def run(i):
                oracle.ctx_kv_write(wl.all_kv, wl.k_norm_weight, wl.eps, wl.positions,
                                    wl.cos_sin, wl.rotary_dim, wl.slot_mapping, caches, wl.fp8,
                                    wl.k_scales, wl.v_scales, t_begin=bounds[i],
                                    t_end=bounds[i + 1])
            ts = []
            with ThreadPoolExecutor(n_threads) as ex:
                for _ in range(runs):
                    t0 = time.perf_counter()
                    list(ex.map(run, range(n_threads)))
                    ts.append(time.perf_counter() - t0)
            return min(ts)

        probe = min(full.num_ctx, 64)
        per_token = timed(token_prefix(full, probe), 1, 1) / probe
        n = int(min(full.num_ctx, max(probe, target_s / max(per_token, 1e-9))))
        wl = token_prefix(full, n)
        t1, tn = timed(wl, 1, 3), timed(wl, threads, 3)
        b, tl = wl.algorithmic_bytes(), wl.token_layers()
        per[name] = {"sample_tokens": n, "of_tokens": full.num_ctx,
                     "single_thread_GB_s": b / t1 / 1e9, "all_threads_GB_s": b / tn / 1e9,
                     "single_thread_token_layers_per_s": tl / t1,
                     "all_threads_token_layers_per_s": tl / tn,
                     "single_thread_s": t1, "all_threads_s": tn, "threads": threads}
        log("cpu baseline", name, json.dumps(per[name]))
    h = per[W.NAMES[HEADLINE]]
    return {"value": h["all_threads_GB_s"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "prefill_bf16's first %d of %d tokens (the headline; every workload's "
                      "sample under per_workload), best of 3 runs on %d threads, one contiguous "
                      "token range each; single-threaded figures alongside"
                      % (h["sample_tokens"], h["of_tokens"], threads),
            "host_cores": os.cpu_count(), "cores_available": avail,
            "thread_cap": "%d threads: the CPU share of one GPU on the measuring box"
                          % CPU_THREAD_CAP,
            "cpu": cpu_model(),
            "single_thread": {"value": h["single_thread_GB_s"], "unit": "GB/s", "cores": 1},
            "per_workload": per}


def traffic_for(name: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


# The launch each measured workload takes (ctx_kv_kernel.hip, launch_one:
# one wave per 4 (token, kv head) rows and per layer or group of layers).
KERNELS = {
    "prefill_bf16": "ctx_kv_write_kernel<R=64, bf16 cache, one layer per wave, 4 heads of one "
                    "token per wave>",
    "prefill_fp8": "ctx_kv_write_kernel<R=64, e4m3 cache, groups of 3 layers per wave, 4 heads "
                   "of one token per wave>",
    "long_fp8": "ctx_kv_write_kernel<R=32, e4m3 cache, groups of 3 layers per wave, 4 heads of "
                "one token per wave>",
    "decode_bf16": "ctx_kv_write_kernel<R=16, bf16 cache, one layer per wave, 4 heads of one "
                   "token per wave> under HIP-graph replay",
    "prefill_bf16_layer_slots": "ctx_kv_write_kernel<R=64, bf16 cache, per-layer slots, one "
                                "layer per wave>",
    "prefill_bf16_tp4_shard": "ctx_kv_write_kernel<R=64, bf16 cache, general row mapping "
                              "(nkv = 2), every layer of a row group in one wave>",
    "project_prefill_bf16": "project_write_packed_wide_kernel<R=64, bf16 cache> (packed weight, "
                            "128 x 512 tiles, the last round in 64-token halves)",
    "project_prefill_fp8": "project_write_packed_wide_kernel<R=64, e4m3 cache> (packed weight, "
                           "128 x 512 tiles, the last round in 64-token halves)",
    "insert_draft_bf16": "qknorm_insert_kernel<R=64, bf16 cache>",
    "insert_draft_fp8": "qknorm_insert_kernel<R=64, e4m3 cache, q fp8>",
}


def roofline_entry(name: str, r: dict):
    """The roofline block of one measured workload: the dominant kernel's
    algorithmic bytes (or flops) per launch over its average launch
    duration in the timed region, against the MI355X's published peak."""
    if "project_write_TFLOP_s" in r:
        return {"bound": "mfma", "achieved": r["project_write_TFLOP_s"],
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": r["project_write_TFLOP_s"] / BF16_MFMA_PEAK_TFLOPS, "traffic": None,
                "kernel": KERNELS.get(name, name), "kernel_us_avg": r["project_write_us"],
                "algorithmic_flops_per_launch": r["gemm_flops"]}
    gbs = r.get("kernel_GB_s", r.get("GB_s"))
    if gbs is None:
        return None
    us = r.get("kernel_us_avg", r.get("us_per_call"))
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": traffic_for(name),
            "kernel": KERNELS.get(name, name), "kernel_us_avg": us,
            "algorithmic_bytes_per_launch": r.get("bytes_per_call")}


def main():
    global WARMUP_FLOOR_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # untimed calls before each timed region: the GPU's clock settles over
    # the first ~20 ms of sustained work (an fp8 prefill timed after 20 calls
    # read 27.8 us, after another ~9 ms of calls 24.9 us, then 23.7 us)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="minimum warm-up calls before each timed region (at least %.0f ms "
                         "of launches are made in any case)" % (WARMUP_FLOOR_S * 1e3))
    ap.add_argument("--warmup-floor-ms", type=float, default=WARMUP_FLOOR_S * 1e3,
                    help="minimum milliseconds of launches before each timed region (counter "
                         "runs, which serialise every launch, set 0)")
    ap.add_argument("--workload", default="all", choices=["all", "insert", "project"] + W.NAMES)
    ap.add_argument("--insert-sets", type=int, default=32,
                    help="draft blocks rotated in the insert's graph")
    ap.add_argument("--sets", type=int, default=4, help="input sets rotated in the timed loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip timing the unfused PyTorch chain")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    args = ap.parse_args()
    WARMUP_FLOOR_S = max(0.0, args.warmup_floor_ms) / 1e3

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the write is "
              "independent per token and per kv head, so ranks would shard without any "
              "exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    _lib.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)

    if args.calib_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 x %d bytes read + written" % n)
        del src, dst

    reference_copy = copy_reference(dev, stream)
    log("reference copy", json.dumps(reference_copy))

    names = W.NAMES if args.workload == "all" else [n for n in W.NAMES if n == args.workload]
    results = {}
    for name in names:
        index = W.NAMES.index(name)
        if index == 0:
            continue   # the tiny case is a parity case, not a bench line
        log("workload", name, "setup")
        if index == 4:
            setup = Setup(index, 1, dev)
            r = time_graph(setup, max(args.steps, 1000), args.warmup, stream)
            per = r["per_call_s"]
            results[name] = {"us_per_call": per * 1e6, "GB_s": r["bytes"] / per / 1e9,
                             "token_layers_per_s": r["token_layers"] / per,
                             "timing": "%d writes as HIP-graph replays (50 writes per graph)"
                                       % r["calls"],
                             "bytes_per_call": r["bytes"]}
            # a plain copy of the same byte volume under the same replay (one
            # buffer pair, as the write reuses one input set): the practical
            # ceiling of a launch this small
            ref = small_copy_reference(r["bytes"], 1, stream, per_graph=50)
            results[name]["same_size_copy"] = ref
            results[name]["pct_of_same_size_copy"] = 100.0 * results[name]["GB_s"] / ref["GB_s"]
        else:
            n_sets = 1 if index == 3 else args.sets
            setup = Setup(index, n_sets, dev)
            r = time_eager(setup, args.steps, args.warmup, stream)
            k = r["single_s"]
            avg = r["region_s"] / args.steps
            results[name] = {
                "ms_per_step": avg * 1e3,
                "GB_s": float(r["bytes"].sum() / r["region_s"] / 1e9),
                "kernel_us_avg": avg * 1e6,
                "kernel_GB_s": float(r["bytes"].mean() / avg / 1e9),
                "single_launch_us_median": float(np.median(k) * 1e6),
                "single_launch_us_p10": float(np.percentile(k, 10) * 1e6),
                "single_launch_us_p90": float(np.percentile(k, 90) * 1e6),
                "token_layers_per_s": float(r["token_layers"].sum() / r["region_s"]),
                "bytes_per_call": int(r["bytes"].mean()),
                "input_sets": n_sets,
                "wall_s": r["wall_s"],
            }
            if setup.wl.fp8:
                # e4m3 codes at +-448 (0x7E / 0xFE) left in the caches: the
                # saturating store at work (the V probes of the fp8 prefill)
                results[name]["saturated_codes_in_caches"] = int(sum(
                    int(((a.kv_cache == 0x7E) | (a.kv_cache == 0xFE)).sum()) for a in setup.layers))
        results[name]["pct_of_hbm_peak"] = 100.0 * results[name].get("kernel_GB_s", results[name]["GB_s"]) / HBM_PEAK_GBS
        if not args.no_unfused:
            # the base path the fused write replaces, on the same inputs and caches
            us = UnfusedSetup(setup, dev)
            ut = time_unfused(us, min(args.steps, 50), 3, stream)
            unfused_ops = count_device_ops(lambda: us.launch(0, None), stream)
            fused_ops = count_device_ops(lambda: setup.launch(0, stream.cuda_stream), stream)
            fused_us = results[name].get("kernel_us_avg", results[name].get("us_per_call"))
            results[name]["unfused_torch"] = {
                "us_per_call": ut * 1e6, "speedup_of_fused": ut * 1e6 / fused_us,
                "how": "permute copy, per-layer Gemma K norm + stack, positions.repeat, NeoX "
                       "rotary, per-layer cache write, in PyTorch ops (one host sync per call "
                       "for the valid-token list); eager, %d calls" % min(args.steps, 50),
                "device_ops_per_call": unfused_ops,
                "fused_device_ops_per_call": fused_ops}
        log(name, json.dumps(results[name]))
        del setup
        torch.cuda.empty_cache()

    if args.workload in ("all", "prefill_bf16"):
        # the prefill shape with one slot mapping per layer (layers in
        # different KV-cache groups), through the per-layer entry point
        log("workload prefill_bf16_layer_slots setup")
        setup = Setup(HEADLINE, args.sets, dev, layer_slots=True)
        r = time_eager(setup, args.steps, args.warmup, stream)
        avg = r["region_s"] / args.steps
        results["prefill_bf16_layer_slots"] = {
            "ms_per_step": avg * 1e3, "GB_s": float(r["bytes"].sum() / r["region_s"] / 1e9),
            "kernel_us_avg": avg * 1e6, "kernel_GB_s": float(r["bytes"].mean() / avg / 1e9),
            "token_layers_per_s": float(r["token_layers"].sum() / r["region_s"]),
            "bytes_per_call": int(r["bytes"].mean()), "input_sets": args.sets,
            "note": "per-layer block tables, 2% padding per layer"}
        results["prefill_bf16_layer_slots"]["pct_of_hbm_peak"] = \
            100.0 * results["prefill_bf16_layer_slots"]["kernel_GB_s"] / HBM_PEAK_GBS
        log("prefill_bf16_layer_slots", json.dumps(results["prefill_bf16_layer_slots"]))
        del setup
        torch.cuda.empty_cache()

    if args.workload in ("all", "prefill_bf16"):
        # one rank's share of the prefill write under 4-way head parallelism
        # (2 of the 8 kv heads): the shape a single GPU of a TP-4 group writes
        log("workload prefill_bf16_tp4_shard setup")
        setup = Setup(HEADLINE, args.sets, dev, tp=4)
        r = time_eager(setup, args.steps, args.warmup, stream)
        avg = r["region_s"] / args.steps
        res = {
            "ms_per_step": avg * 1e3, "GB_s": float(r["bytes"].sum() / r["region_s"] / 1e9),
            "kernel_us_avg": avg * 1e6, "kernel_GB_s": float(r["bytes"].mean() / avg / 1e9),
            "token_layers_per_s": float(r["token_layers"].sum() / r["region_s"]),
            "bytes_per_call": int(r["bytes"].mean()), "input_sets": len(setup.sets),
            "note": "one rank's 2 of 8 kv heads (nkv = 2), the prefill's tokens and positions; "
                    "input sets = every rank's heads of each prefill set, blocks relocated"}
        res["pct_of_hbm_peak"] = 100.0 * res["kernel_GB_s"] / HBM_PEAK_GBS
        results["prefill_bf16_tp4_shard"] = res
        log("prefill_bf16_tp4_shard", json.dumps(res))
        del setup
        torch.cuda.empty_cache()

    if args.workload in ("all", "project"):
        # the step before the write: hidden norm, then the projection on the
        # matrix cores with the write fused into its epilogue
        for index in (1, 2):
            name = W.PROJECT_NAMES[index]
            log("workload", name, "setup")
            ps = ProjectSetup(index, dev)
            # the clock settles over the first calls: warm both paths, then
            # alternate rounds of each and take the medians
            steps = max(10, min(args.steps, 20))
            for fn in (ps.norm, ps.project_write, ps.project_write_packed, ps.unfused, ps.pack):
                time_calls(fn, 10, 0, stream)
            rounds = {"norm": [], "pw": [], "pwp": [], "fused": [], "fusedp": [], "unfused": [],
                      "pack": []}
            for _ in range(5):
                rounds["norm"].append(time_calls(ps.norm, steps, 0, stream))
                rounds["pw"].append(time_calls(ps.project_write, steps, 0, stream))
                rounds["pwp"].append(time_calls(ps.project_write_packed, steps, 0, stream))
                rounds["fused"].append(time_calls(lambda: (ps.norm(), ps.project_write()),
                                                  steps, 0, stream))
                rounds["fusedp"].append(time_calls(lambda: (ps.norm(), ps.project_write_packed()),
                                                   steps, 0, stream))
                rounds["unfused"].append(time_calls(ps.unfused, steps, 0, stream))
                rounds["pack"].append(time_calls(ps.pack, 3, 0, stream))
            t_norm, t_pw, t_pwp, t_fused, t_fusedp, t_unfused, t_pack = (
                float(np.median(rounds[k]))
                for k in ("norm", "pw", "pwp", "fused", "fusedp", "unfused", "pack"))
            wl = ps.wl
            flops = wl.gemm_flops()
            norm_bytes = 2 * wl.num_ctx * wl.hidden * 2 + wl.hidden * 2
            # the product path packs the weight once, when it is loaded; the
            # row-major kernel (no packing) is reported beside it
            results[name] = {
                "config": W.PROJECT_DESCRIPTIONS[index],
                "weight": "packed once in the fragment-major layout (dspark_kv_weight_pack)",
                "hidden_norm_us": t_norm * 1e6,
                "hidden_norm_GB_s": norm_bytes / t_norm / 1e9,
                "project_write_us": t_pwp * 1e6,
                "project_write_TFLOP_s": flops / t_pwp / 1e12,
                "pct_of_bf16_mfma_peak": 100.0 * flops / t_pwp / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                "pipeline_us": t_fusedp * 1e6,
                "unfused_pipeline_us": t_unfused * 1e6,
                "unfused_pipeline": "hidden norm, torch linear (hipBLASLt) writing all_kv, "
                                    "context write kernel",
                "speedup_of_fused": t_unfused / t_fusedp,
                "weight_pack_us_once": t_pack * 1e6,
                "row_major_weight": {
                    "project_write_us": t_pw * 1e6,
                    "project_write_TFLOP_s": flops / t_pw / 1e12,
                    "pct_of_bf16_mfma_peak": 100.0 * flops / t_pw / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                    "pipeline_us": t_fused * 1e6,
                    "speedup_of_fused": t_unfused / t_fused,
                    "how": "the same projection from the row-major [out, in] weight "
                           "(project_write_kernel, 256 x 256 tiles); same bytes written"},
                "gemm_flops": flops,
                "timing": "medians of 5 alternating rounds of %d calls each, after 10 "
                          "warm-up calls per path" % steps}
            log(name, json.dumps(results[name]))
            del ps
            torch.cuda.empty_cache()

    if args.workload in ("all", "insert"):
        # the draft block's fused QK-norm / RoPE / KV insert (448 draft rows)
        for index in (1, 2):
            name = W.INSERT_NAMES[index]
            log("workload", name, "setup")
            setup = InsertSetup(index, args.insert_sets, dev)
            r = time_graph(setup, max(args.steps, 1000), args.warmup, stream,
                           per_graph=2 * args.insert_sets)
            per = r["per_call_s"]
            results[name] = {"us_per_call": per * 1e6, "GB_s": r["bytes"] / per / 1e9,
                             "tokens_per_s": r["token_layers"] / per,
                             "timing": "%d calls as HIP-graph replays over %d draft blocks"
                                       % (r["calls"], args.insert_sets),
                             "bytes_per_call": r["bytes"],
                             "config": W.INSERT_DESCRIPTIONS[index]}
            results[name]["pct_of_hbm_peak"] = 100.0 * results[name]["GB_s"] / HBM_PEAK_GBS
            ref = small_copy_reference(r["bytes"], args.insert_sets, stream)
            results[name]["same_size_copy"] = ref
            results[name]["pct_of_same_size_copy"] = 100.0 * results[name]["GB_s"] / ref["GB_s"]
            log(name, json.dumps(results[name]))
            del setup
            torch.cuda.empty_cache()

    head = W.NAMES[HEADLINE]
    out = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "warmup_policy": "at least --warmup calls and at least %.0f ms of back-to-back "
                            "launches of the same workload before each timed region "
                            "(--warmup-floor-ms); after the synchronisation that opens the "
                            "region, %d untimed launches are queued ahead of the start event so "
                            "that the region starts on a busy GPU; the timed region is exactly "
                            "--steps launches" % (WARMUP_FLOOR_S * 1e3, PREROLL)}
    rooflines = {n: roofline_entry(n, r) for n, r in results.items()}
    if head in results:
        h = results[head]
        out.update({"value": h["GB_s"], "ms_per_step": h["ms_per_step"],
                    "token_layers_per_s": h["token_layers_per_s"],
                    "pct_of_hbm_peak": 100.0 * h["GB_s"] / HBM_PEAK_GBS})
        out["config"] = {"workload": head + ": " + W.DESCRIPTIONS[HEADLINE],
                         "num_ctx": 4096, "layers": 5, "kv_heads": 8, "head_dim": 128,
                         "rotary_dim": 64, "cache": "bf16", "io": "bf16 in, bf16 cache",
                         "arithmetic": "fp32 norm and RoPE, bf16 rounding of each result",
                         "input_sets_rotated": h["input_sets"]}
        out["roofline"] = dict(rooflines[head])
    else:
        name = next(iter(results))
        r0 = results[name]
        out.update({"value": r0.get("GB_s", r0.get("project_write_TFLOP_s")),
                    "ms_per_step": r0.get("ms_per_step", r0.get("us_per_call",
                                                                r0.get("pipeline_us", 0)) / 1e3)})
        desc = (W.DESCRIPTIONS[W.NAMES.index(name)] if name in W.NAMES
                else results[name].get("config", ""))
        out["config"] = {"workload": name + ": " + desc}
        out["roofline"] = dict(rooflines[name]) if rooflines.get(name) else {}
    # every measured workload's roofline, next to the headline's
    out["roofline"]["per_workload"] = {n: r for n, r in rooflines.items() if r is not None}
    out["workloads"] = results
    out["reference_copy"] = reference_copy
    if not args.no_cpu_baseline and any(n in W.NAMES for n in results):
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
