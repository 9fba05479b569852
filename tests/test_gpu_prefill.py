"""GPU parity of zp_paged_prefill against the float64 oracle.

Zipage (arXiv 2603.08743) Sec. 3 / Sec. 6: attention over a block table is
ordinary causal softmax attention over the resident tokens; Sec. 4.1: the
prompt is written in full; Sec. 4.2: the queries of the last w slots of the
final block go to the query cache; Sec. 4.4: a chunk may follow ctx tokens
(shared prefix blocks) already in the cache.
Bar: max |out - ref| <= tol * max |ref| per (token, query head) on sampled
rows, tol 1e-5 for fp32 and 2e-2 for bf16; lse within 2e-5 (fp32) / 2e-3
(bf16) absolute; appended K/V, captured window queries bit-exact.
"""
import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import synth, zp
from oracle import zipage as Z

from gpu_cases import HostCache, announce, dev_i32, device_k, device_v, random_tables, tol_for

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, d, h_q, h_kv, b, w, q_lens, ctx_lens
    ("f32", 64, 4, 1, 16, 8, [200, 1, 37], [0, 0, 16]),
    ("bf16", 128, 32, 8, 256, 16, [4096, 300, 17, 512], [0, 0, 700, 1024]),
    ("bf16", 64, 8, 8, 32, 16, [130, 64, 1], [0, 33, 5]),
    ("bf16", 128, 16, 2, 64, 8, [257, 1000], [0, 100]),
    ("bf16", 128, 8, 8, 16, 16, [95, 16], [0, 32]),
    ("bf16", 64, 16, 2, 128, 16, [640, 3], [130, 0]),
    ("f32", 128, 16, 2, 64, 2, [70, 129], [0, 64]),
    ("bf16", 128, 8, 4, 64, 8, [200, 65], [0, 70]),     # g = 2 on the LDS-copy kernel
    ("bf16", 64, 4, 4, 128, 16, [300, 1], [10, 0]),     # g = 1 on the LDS-copy kernel
]


def _sample_rows(rng, qlen, b, w, ctx, k=24):
    """First and last rows, rows of the final block's window, tile and block
    edges, and random rows."""
    rows = {0, qlen - 1}
    last = ctx + qlen - 1
    for off in range(b - w, b):
        p = (last // b) * b + off
        if ctx <= p <= last:
            rows.add(p - ctx)
    for e in (15, 16, 31, 32, 63, 64, 127, 128, 255, 256, 1023, 1024):
        if e < qlen:
            rows.add(e)
    rows.update(rng.integers(0, qlen, min(k, qlen)).tolist())
    return sorted(rows)


def _run(dtype, d, h_q, h_kv, b, w, q_lens, ctx_lens, seed=5, layer=1, sample=24, noslot=None,
         min_stride=0, k_ramp=0.0):
    announce(f"prefill dtype={dtype} d={d} hq={h_q} hkv={h_kv} b={b} w={w} q={q_lens} ctx={ctx_lens}")
    nreq = len(q_lens)
    g = h_q // h_kv
    ntok = [c + n for c, n in zip(ctx_lens, q_lens)]
    nb = [-(-n // b) for n in ntok]
    stride = max(max(nb) + 1, min_stride)
    pool = sum(nb) + 2
    geom = zp.CacheGeometry(num_layers=2, num_blocks=pool, block_size=b, num_kv_heads=h_kv,
                            num_q_heads=h_q, head_dim=d, window=w, max_slots=nreq + 1, n_max=2,
                            dtype=dtype)
    hc = HostCache(geom, seed, 2)
    hc.dev.qwin_lse = torch.full((2, nreq + 1, h_kv, g, w), 5.0, dtype=torch.float32,
                                 device="cuda")
    tab = random_tables(seed, 2, nb, pool, stride)
    T = sum(q_lens)
    gen = synth.rng(seed, 2, layer, "prompt_q")
    q = synth.cast(gen.standard_normal((T, h_q, d)), dtype)
    kn = gen.standard_normal((T, h_kv, d)) * np.where(gen.random((T, h_kv)) < 0.02, 4.0, 1.0)[..., None]
    if k_ramp:
        # every key dimension grows with the position: the logits of queries
        # with a positive coordinate sum climb from tile to tile
        kn = kn + k_ramp * (np.arange(T) / 64.0)[:, None, None]
    kn = synth.cast(kn, dtype)
    vn = synth.cast(gen.standard_normal((T, h_kv, d)), dtype)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    qslot = np.arange(nreq, dtype=np.int32) + 1
    if noslot is not None:
        qslot[noslot] = -1          # scheduled without a query slot
    dt = geom.torch_dtype()
    tq = torch.from_numpy(q).to(dt).cuda()
    tk = torch.from_numpy(kn).to(dt).cuda()
    tv = torch.from_numpy(vn).to(dt).cuda()
    out = torch.full((T, h_q, d), 7.0, dtype=dt, device="cuda")
    lse = torch.zeros((T, h_q), dtype=torch.float32, device="cuda")
    qwin0 = hc.dev.qwin.float().cpu().numpy()
    ws = zp.new_workspace(zp.zp_prefill_workspace_size(geom, nreq))
    zp.zp_paged_prefill(hc.dev, layer, tq, tk, tv, dev_i32(cu), dev_i32(np.array(ctx_lens, np.int32)),
                        max(q_lens), dev_i32(tab), dev_i32(qslot), out, lse, ws)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    out_h = out.float().cpu().numpy()
    lse_h = lse.cpu().numpy()
    Kd, Vd = device_k(hc), device_v(hc)
    qwin = hc.dev.qwin.float().cpu().numpy()
    qlse = hc.dev.qwin_lse.cpu().numpy()
    tol = tol_for(dtype)
    ltol = 2e-5 if dtype == "f32" else 2e-3
    srng = np.random.default_rng(seed)
    worst = 0.0
    for r in range(nreq):
        c0, n, ctx = cu[r], q_lens[r], ctx_lens[r]
        if n == 0:       # an empty chunk: nothing appended, attended or captured
            continue
        # appended rows bit-exact, context rows untouched
        for h in range(h_kv):
            Kr = Z.gather_sequence(Kd[layer, :, h], tab[r], ntok[r], b)
            Vr = Z.gather_sequence(Vd[layer, :, h], tab[r], ntok[r], b)
            np.testing.assert_array_equal(Kr[ctx:], kn[c0:c0 + n, h])
            np.testing.assert_array_equal(Vr[ctx:], vn[c0:c0 + n, h])
            np.testing.assert_array_equal(Kr[:ctx], Z.gather_sequence(hc.K[layer, :, h], tab[r], ctx, b))
        K = np.stack([Z.gather_sequence(Kd[layer, :, h], tab[r], ntok[r], b) for h in range(h_kv)])
        V = np.stack([Z.gather_sequence(Vd[layer, :, h], tab[r], ntok[r], b) for h in range(h_kv)])
        rows = _sample_rows(srng, n, b, w, ctx, sample)
        O, L = Z.prefill_attention(q[c0:c0 + n], K, V, ctx, rows=rows)
        for x, i in enumerate(rows):
            for j in range(h_q):
                ref = O[x, j]
                err = np.abs(out_h[c0 + i, j] - ref).max() / np.abs(ref).max()
                worst = max(worst, err)
                assert err <= tol, f"req {r} row {i} head {j}: {err}"
            np.testing.assert_allclose(lse_h[c0 + i], L[x], rtol=0, atol=ltol)
        # window rows of the final block: query and lse captured, nothing else
        last = ctx + n - 1
        slot = qslot[r]
        if slot < 0:
            np.testing.assert_array_equal(qwin[layer, r + 1], qwin0[layer, r + 1])
            assert np.all(qlse[layer, r + 1] == 5.0)
            continue
        for off in range(b - w, b):
            p = (last // b) * b + off
            u = off - (b - w)
            if ctx <= p <= last:
                i = p - ctx
                for gi in range(g):
                    np.testing.assert_array_equal(qwin[layer, slot, :, gi, u],
                                                  q[c0 + i].reshape(h_kv, g, d)[:, gi])
                    np.testing.assert_array_equal(qlse[layer, slot, :, gi, u],
                                                  lse_h[c0 + i].reshape(h_kv, g)[:, gi])
            else:
                np.testing.assert_array_equal(qwin[layer, slot, :, :, u], qwin0[layer, slot, :, :, u])
                assert np.all(qlse[layer, slot, :, :, u] == 5.0)
    print(f"[prefill] worst relative error {worst:.3g}")


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-g{c[2] // c[3]}-b{c[4]}" for c in CASES])
def test_prefill_parity(case):
    _run(*case)


@pytest.mark.parametrize("b", [16, 256])   # register-staged and LDS-copy kernels
def test_prefill_empty_chunks_in_a_batch(b):
    _run("bf16", 128, 16, 2, b, 8, [70, 0, 300, 0], [0, 0, 40, 0])


def test_prefill_rising_logits_move_the_maximum_every_tile():
    # keys ramped so some rows' logits rise ~11 (log2 units) per 32-key
    # tile: the running maximum moves on almost every tile, through the
    # path that takes the row maxima, rescales and forms the weights again
    _run("bf16", 128, 16, 2, 256, 16, [1500, 700], [0, 300], k_ramp=16.0)
    _run("bf16", 128, 32, 8, 256, 16, [600], [0], k_ramp=16.0)


def test_prefill_wide_table_big_blocks():
    """Blocks of >= 64 tokens normally take the kernel that stages the block
    table in LDS; a table wider than that stage takes the general kernel."""
    _run("bf16", 128, 16, 2, 64, 8, [300, 70], [0, 130], min_stride=3000)


def test_prefill_without_query_slot_captures_nothing():
    _run("bf16", 128, 16, 2, 64, 8, [130, 100, 70], [0, 0, 64], noslot=1)
    _run("f32", 64, 4, 1, 16, 8, [40, 37], [0, 16], noslot=0)


@pytest.mark.parametrize("b", [16, 64])   # per-key lookups; one lookup per 64-key tile
def test_prefill_reports_bad_block_ids_without_faulting(b):
    announce(f"prefill bad block id b={b}")
    geom = zp.CacheGeometry(num_layers=1, num_blocks=8, block_size=b, num_kv_heads=2,
                            num_q_heads=8, head_dim=64, window=8, max_slots=1, n_max=2,
                            dtype="bf16")
    cache = zp.PagedKVCache(geom)
    tab = np.array([[0, 1, 99, 3]], np.int32)        # block 99 does not exist
    T = 3 * b + b // 2
    q = torch.randn((T, 8, 64), device="cuda").bfloat16()
    k = torch.randn((T, 2, 64), device="cuda").bfloat16()
    out = torch.zeros_like(q)
    ws = zp.new_workspace(zp.zp_prefill_workspace_size(geom, 1))
    zp.zp_paged_prefill(cache, 0, q, k, k, dev_i32([0, T]), dev_i32([0]), T, dev_i32(tab), None,
                        out, None, ws)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) & zp.ZP_DEVERR_BLOCK_ID
    # a chunk longer than max_q_len is skipped with a length error
    zp.zp_workspace_clear_errors(ws)
    zp.zp_paged_prefill(cache, 0, q, k, k, dev_i32([0, T]), dev_i32([0]), T - 1,
                        dev_i32([[0, 1, 2, 3]]), None, out, None, ws)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) & zp.ZP_DEVERR_SEQ_LEN


def test_prefill_bench_launch_sampled():
    """The launch bench.py times: 64 prompts of 4096 tokens in one call, the
    Qwen3-8B attention shape (32 query / 8 kv heads, d 128, bf16, blocks of
    256), so the LDS-copy kernel runs with its workgroups renumbered over
    the 8 XCDs. The inputs are too large for the host generator; they come
    from torch's seeded generator on the device, and the oracle gets the
    same values. Checked on three requests (first, middle, last, so on
    different XCD slots): sampled rows in every head against the float64
    oracle, every appended K/V block bit-exact, the final block's window
    queries and log-sum-exp."""
    R, T, b, NB = 64, 4096, 256, 16
    h_q, h_kv, d, w = 32, 8, 128, 16
    g = h_q // h_kv
    announce(f"prefill bench launch {R} x {T}")
    geom = zp.CacheGeometry(num_layers=1, num_blocks=R * NB + 8, block_size=b, num_kv_heads=h_kv,
                            num_q_heads=h_q, head_dim=d, window=w, max_slots=R, n_max=8,
                            dtype="bf16")
    cache = zp.PagedKVCache(geom, with_global=False, with_window_lse=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41)
    q = torch.randn((R * T, h_q, d), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((R * T, h_kv, d), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((R * T, h_kv, d), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.full_like(q, 7.0)
    lse = torch.zeros((R * T, h_q), dtype=torch.float32, device="cuda")
    tables = torch.randperm(R * NB, generator=gen, device="cuda").to(torch.int32).view(R, NB)
    cu = torch.arange(0, (R + 1) * T, T, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(R, dtype=torch.int32, device="cuda")
    qslot = torch.arange(R, dtype=torch.int32, device="cuda")
    ws = zp.new_workspace(zp.zp_prefill_workspace_size(geom, R))
    zp.zp_paged_prefill(cache, 0, q, k, v, cu, ctx, T, tables.contiguous(), qslot, out, lse, ws)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    tab = tables.cpu().numpy()
    srng = np.random.default_rng(41)
    worst = 0.0
    for r in (0, 37, R - 1):
        c0 = r * T
        # appended K/V: every block of the request, bit-exact
        for blk in range(NB):
            rows = slice(c0 + blk * b, c0 + (blk + 1) * b)
            assert torch.equal(cache.k[0, tab[r, blk]], k[rows].transpose(0, 1))
            assert torch.equal(cache.v[0, tab[r, blk]], v[rows].transpose(0, 1))
        qf = q[c0:c0 + T].float().cpu().numpy()
        K = k[c0:c0 + T].float().cpu().numpy().transpose(1, 0, 2)
        V = v[c0:c0 + T].float().cpu().numpy().transpose(1, 0, 2)
        rows = _sample_rows(srng, T, b, w, 0, k=8)
        O, L = Z.prefill_attention(qf, K, V, 0, rows=rows)
        out_h = out[c0:c0 + T].float().cpu().numpy()
        lse_h = lse[c0:c0 + T].cpu().numpy()
        for x, i in enumerate(rows):
            for j in range(h_q):
                err = np.abs(out_h[i, j] - O[x, j]).max() / np.abs(O[x, j]).max()
                worst = max(worst, err)
                assert err <= 2e-2, f"req {r} row {i} head {j}: {err}"
            np.testing.assert_allclose(lse_h[i], L[x], rtol=0, atol=2e-3)
        # the final block's 16 window rows: queries and log-sum-exp captured
        for u in range(w):
            i = T - w + u
            assert torch.equal(cache.qwin[0, r, :, :, u], q[c0 + i].view(h_kv, g, d))
            np.testing.assert_array_equal(cache.qwin_lse[0, r, :, :, u].cpu().numpy(),
                                          lse_h[i].reshape(h_kv, g))
    print(f"[prefill bench launch] worst relative error {worst:.3g}")
