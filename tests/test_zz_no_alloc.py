"""zp_paged_decode_noalloc: the decode entry point for callers that cannot
allocate device memory. Its split partials live in the library's static
device scratch instead of a caller workspace; the kernels are the same, so
outputs, log-sum-exp, the appended K/V and the captured window queries must
match zp_paged_decode (with a workspace) bit for bit. Two calls in a row on
one GPU, the second with a smaller batch (the scratch still holds the first
call's partials), plus device error bits through the caller's error word and
the host-side rejection of a call whose partials exceed the scratch.
"""
import ctypes as C

import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import synth, zp

from gpu_cases import HostCache, announce, dev_i32, random_tables


def _geom(dtype, d, h_q, h_kv, b, w, pool, slots):
    return zp.CacheGeometry(num_layers=2, num_blocks=pool, block_size=b, num_kv_heads=h_kv,
                            num_q_heads=h_q, head_dim=d, window=w, max_slots=slots, n_max=2,
                            dtype=dtype)


def _compare(dtype, d, h_q, h_kv, b, w, lens, seed, layer=1):
    announce(f"noalloc decode dtype={dtype} d={d} hq={h_q} hkv={h_kv} b={b} lens={lens}")
    B = len(lens)
    nb = [-(-n // b) for n in lens]
    pool = sum(nb) + 3
    geom = _geom(dtype, d, h_q, h_kv, b, w, pool, B)
    max_len = max(lens)
    need = zp.zp_decode_workspace_size(geom, B, max_len)
    hc = HostCache(geom, seed, 1)
    tab = dev_i32(random_tables(seed, 1, nb, pool, max(nb) + 1))
    g = synth.rng(seed, 1, layer, "step_q")
    dt = geom.torch_dtype()
    q = torch.from_numpy(synth.cast(g.standard_normal((B, h_q, d)), dtype)).to(dt).cuda()
    kn = torch.from_numpy(synth.cast(g.standard_normal((B, h_kv, d)), dtype)).to(dt).cuda()
    vn = torch.from_numpy(synth.cast(g.standard_normal((B, h_kv, d)), dtype)).to(dt).cuda()
    seq = dev_i32(lens)
    qslot = dev_i32(np.arange(B))
    gq = h_q // h_kv

    def fresh_lse():
        hc.dev.qwin_lse = torch.full((2, B, h_kv, gq, w), 9.0, dtype=torch.float32,
                                     device="cuda")

    # with a workspace
    fresh_lse()
    out_a = torch.full((B, h_q, d), 7.0, dtype=dt, device="cuda")
    lse_a = torch.zeros((B, h_q), dtype=torch.float32, device="cuda")
    ws = zp.new_workspace(need)
    zp.zp_paged_decode(hc.dev, layer, q, kn, vn, tab, seq, max_len, qslot, out_a, lse_a, ws)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    after_a = [t.clone() for t in (hc.dev.k, hc.dev.v, hc.dev.qwin, hc.dev.qwin_lse)]
    # the same call without one, from the same cache contents
    hc.upload()
    fresh_lse()
    out_b = torch.full((B, h_q, d), 7.0, dtype=dt, device="cuda")
    lse_b = torch.zeros((B, h_q), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    zp.zp_paged_decode_noalloc(hc.dev, layer, q, kn, vn, tab, seq, max_len, qslot, out_b, lse_b,
                               err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    bits = (lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32))
    assert torch.equal(bits(out_a), bits(out_b))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
    for x, y in zip(after_a, (hc.dev.k, hc.dev.v, hc.dev.qwin, hc.dev.qwin_lse)):
        assert torch.equal(bits(x), bits(y))
    return need


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode_two_calls_shrinking():
    # 4 long sequences: split over several workgroups, partials in the scratch
    need1 = _compare("bf16", 128, 32, 8, 256, 16, [8192, 5000, 7777, 300], seed=21)
    # then a smaller batch on the same GPU: the scratch holds the first
    # call's partials, which must not leak into this one
    need2 = _compare("bf16", 128, 32, 8, 256, 16, [3000, 1500], seed=22)
    assert need1 > need2 > 256
    # fp32 tiny geometry, single and split rows
    _compare("f32", 64, 4, 1, 16, 8, [200, 17, 1], seed=23)


@pytest.mark.gpu
def test_noalloc_decode_reports_device_errors_in_callers_word():
    announce("noalloc decode bad block id")
    geom = zp.CacheGeometry(num_layers=1, num_blocks=4, block_size=16, num_kv_heads=1,
                            num_q_heads=4, head_dim=64, window=8, max_slots=1, n_max=2, dtype="f32")
    hc = HostCache(geom, 5, 2)
    tab = np.array([[0, 99, 2]], np.int32)      # 99 is outside the pool: masked and flagged
    q = torch.randn(1, 4, 64, device="cuda")
    k = torch.randn(1, 1, 64, device="cuda")
    out = torch.zeros(1, 4, 64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    zp.zp_paged_decode_noalloc(hc.dev, 0, q, k, k.clone(), dev_i32(tab), dev_i32([40]), 40, None,
                               out, None, err)
    torch.cuda.synchronize()
    assert int(err.item()) & zp.ZP_DEVERR_BLOCK_ID
    assert torch.isfinite(out).all()


def test_noalloc_decode_rejects_calls_beyond_the_scratch_on_the_host():
    """64 query / 8 kv heads, 199 sequences: the split partials would take
    more than ZP_DECODE_SCRATCH_BYTES. Rejected before any HIP call."""
    g = zp.CacheGeometry(num_layers=1, num_blocks=100000, block_size=256, num_kv_heads=8,
                         num_q_heads=64, head_dim=128, window=16, max_slots=8, n_max=8,
                         dtype="bf16").c()
    need = zp.lib().zp_decode_workspace_size(C.byref(g), 199, 1 << 20)
    assert need - 256 > zp.ZP_DECODE_SCRATCH_BYTES
    cache = zp.Cache(1, 1, 1, None)
    st = zp.lib().zp_paged_decode_noalloc(C.byref(g), C.byref(cache), 0, 199, 1, 1, 1, 1, 8, 1,
                                          1 << 20, None, 1, None, None, None)
    assert st == zp.ZP_EINVAL and "scratch" in zp.lib().zp_last_error().decode()
    # an empty batch is a no-op, NULL buffers are rejected
    assert zp.lib().zp_paged_decode_noalloc(C.byref(g), C.byref(cache), 0, 0, None, None, None,
                                            None, 8, None, 16, None, None, None, None,
                                            None) == zp.ZP_OK
    st = zp.lib().zp_paged_decode_noalloc(C.byref(g), C.byref(cache), 0, 1, None, 1, 1, 1, 8, 1,
                                          16, None, 1, None, None, None)
    assert st == zp.ZP_EINVAL
