"""Device-side helpers for the GPU tests: move a workload to the GPU, run the
HIP write through the Python writer (which calls the C ABI), and bring the
caches back as numpy arrays of raw codes."""
from __future__ import annotations

import numpy as np
import torch

from speculative_decoding_draft_02_amd import workloads as W
from speculative_decoding_draft_02_amd.writer import AttnLayer, DSparkContextKVWriter

DEV = "cuda:0"


def new_cache(wl: W.Workload, device=DEV) -> torch.Tensor:
    if wl.fp8:
        return torch.full(wl.cache_shape, W.SENTINEL_FP8, dtype=torch.uint8, device=device)
    return torch.full(wl.cache_shape, -1, dtype=torch.int16, device=device).view(torch.bfloat16)


def make_layers(wl: W.Workload, device=DEV, reverse=False):
    """One separately allocated cache and two scale tensors per layer."""
    order = range(wl.num_layers - 1, -1, -1) if reverse else range(wl.num_layers)
    caches, ks, vs = {}, {}, {}
    for l in order:
        caches[l] = new_cache(wl, device)
        ks[l] = torch.tensor([float(wl.k_scales[l])], dtype=torch.float32, device=device)
        vs[l] = torch.tensor([float(wl.v_scales[l])], dtype=torch.float32, device=device)
    kind = "fp8" if wl.fp8 else "auto"
    return [AttnLayer(caches[l], ks[l], vs[l], kind) for l in range(wl.num_layers)]


def bf16_tensor(bits: np.ndarray, device=DEV) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class DeviceInputs:
    def __init__(self, wl: W.Workload, device=DEV):
        self.all_kv = bf16_tensor(wl.all_kv, device)
        self.w = bf16_tensor(wl.k_norm_weight, device)
        self.positions = torch.from_numpy(wl.positions).to(device)
        self.cos_sin = bf16_tensor(wl.cos_sin, device)
        self.slots = torch.from_numpy(wl.slot_mapping).to(device)
        self.eps = wl.eps
        self.rotary_dim = wl.rotary_dim

    def call(self, writer):
        writer(self.all_kv, self.w, self.eps, self.positions, self.cos_sin, self.rotary_dim,
               self.slots)


def cache_codes(cache: torch.Tensor) -> np.ndarray:
    if cache.dtype == torch.uint8:
        return cache.cpu().numpy()
    return cache.view(torch.int16).cpu().numpy().view(np.uint16)


def run_device(wl: W.Workload, reverse=False):
    layers = make_layers(wl, reverse=reverse)
    writer = DSparkContextKVWriter(layers)
    DeviceInputs(wl).call(writer)
    torch.cuda.synchronize()
    out = [cache_codes(a.kv_cache) for a in layers]
    writer.close()
    return out


def run_oracle(oracle, wl: W.Workload):
    caches = wl.new_host_caches()
    return oracle.ctx_kv_write(wl.all_kv, wl.k_norm_weight, wl.eps, wl.positions, wl.cos_sin,
                               wl.rotary_dim, wl.slot_mapping, caches, wl.fp8,
                               wl.k_scales, wl.v_scales)
