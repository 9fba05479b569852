"""Helpers for the GPU parity tests: seeded paged caches built on the host,
uploaded with torch, plus the host-side bookkeeping needed to feed the same
values to the CPU oracle. Nothing here computes any part of the method."""
from __future__ import annotations

import sys

import numpy as np
import torch

from compressed_paged_kv_gqa_amd import synth, zp


def announce(msg):
    """Names the case on stdout before a GPU step (survives a lost box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def tol_for(dtype):
    return 1e-5 if dtype == "f32" else 2e-2


class HostCache:
    """Seeded host copy of a paged cache and its device twin."""

    def __init__(self, geom: zp.CacheGeometry, seed, config, with_global=True, f_scale=0.01):
        self.geom = geom
        G = geom
        shape = (G.num_layers, G.num_blocks, G.num_kv_heads, G.block_size, G.head_dim)
        self.K = np.empty(shape, np.float32)
        self.V = np.empty(shape, np.float32)
        for l in range(G.num_layers):
            self.K[l] = synth.cast(synth.rng(seed, config, l, "prompt_k").standard_normal(shape[1:]), G.dtype)
            self.V[l] = synth.cast(synth.rng(seed, config, l, "prompt_v").standard_normal(shape[1:]), G.dtype)
        self.Q = synth.cast(synth.rng(seed, config, 0, "prompt_q").standard_normal(
            (G.num_layers, G.max_slots, G.num_kv_heads, G.group, G.window, G.head_dim)), G.dtype)
        self.F = (synth.rng(seed, config, 0, "gscore").random(shape[:4]) * f_scale).astype(np.float32)
        self.dev = zp.PagedKVCache(geom, with_global=with_global)
        self.upload()

    def upload(self):
        dt = self.geom.torch_dtype()
        self.dev.k.copy_(torch.from_numpy(self.K).to(dt))
        self.dev.v.copy_(torch.from_numpy(self.V).to(dt))
        self.dev.qwin.copy_(torch.from_numpy(self.Q).to(dt))
        if self.dev.gscore is not None:
            self.dev.gscore.copy_(torch.from_numpy(self.F))

    def plant_heavy(self, seed, config, frac=0.02, scale=4.0):
        g = synth.rng(seed, config, 0, "heavy")
        m = g.random(self.K.shape[:4]) < frac
        self.K = synth.cast(self.K * np.where(m, scale, 1.0)[..., None], self.geom.dtype)


def device_k(cache):
    return cache.dev.k.float().cpu().numpy()


def device_v(cache):
    return cache.dev.v.float().cpu().numpy()


def random_tables(seed, config, lens_blocks, pool, stride):
    """Disjoint random block tables: request r gets lens_blocks[r] blocks."""
    g = synth.rng(seed, config, 0, "misc")
    perm = g.permutation(pool)
    assert sum(lens_blocks) <= pool
    tab = np.full((len(lens_blocks), stride), -1, np.int32)
    at = 0
    for r, nb in enumerate(lens_blocks):
        tab[r, :nb] = perm[at:at + nb]
        at += nb
    return tab


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()
