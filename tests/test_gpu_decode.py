"""GPU parity of zp_paged_decode against the float64 oracle.

Zipage (arXiv 2603.08743) Sec. 3 / Sec. 6: decode attention over a block
table is softmax attention over the resident tokens; Sec. 4.2: the query of
each of the last w slots of a block goes to the query cache.
Bar: max |out - ref| <= tol * max |ref| per (sequence, query head), tol 1e-5
for fp32 and 2e-2 for bf16; appended K/V and captured queries bit-exact.
"""
import math

import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import synth, zp
from oracle import zipage as Z

from gpu_cases import HostCache, announce, dev_i32, random_tables, tol_for

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, d, h_q, h_kv, b, w, lens (resident after the append)
    ("f32", 64, 4, 1, 16, 8, [1, 17, 208, 16, 300]),
    ("bf16", 128, 32, 8, 256, 16, [1, 255, 256, 257, 1793, 2048, 3000, 4097]),
    ("bf16", 64, 8, 8, 32, 16, [5, 64, 640]),
    ("f32", 128, 16, 2, 64, 2, [70, 129, 1200]),
    ("bf16", 128, 8, 4, 128, 8, [1, 1024, 2500]),
]


def _run_case(dtype, d, h_q, h_kv, b, w, lens, seed=3, layer=1, skip_rows=(), poison_tail=False):
    announce(f"decode dtype={dtype} d={d} hq={h_q} hkv={h_kv} b={b} lens={lens} poison={poison_tail}")
    B = len(lens)
    nb = [-(-n // b) for n in lens]
    stride = max(nb) + 1
    pool = sum(nb) + 3
    geom = zp.CacheGeometry(num_layers=2, num_blocks=pool, block_size=b, num_kv_heads=h_kv,
                            num_q_heads=h_q, head_dim=d, window=w, max_slots=B, n_max=2,
                            dtype=dtype)
    hc = HostCache(geom, seed, 1)
    tab = random_tables(seed, 1, nb, pool, stride)
    if poison_tail:
        # slots at and after the new token's, in its block, were never
        # written: NaN there must not reach the output
        for r, n in enumerate(lens):
            pg = tab[r][(n - 1) // b]
            hc.K[:, pg, :, (n - 1) % b:] = np.nan
            hc.V[:, pg, :, (n - 1) % b:] = np.nan
        hc.upload()
    g = synth.rng(seed, 1, layer, "step_q")
    q = synth.cast(g.standard_normal((B, h_q, d)), dtype)
    kn = synth.cast(g.standard_normal((B, h_kv, d)), dtype)
    vn = synth.cast(g.standard_normal((B, h_kv, d)), dtype)
    seq = np.array(lens, np.int32)
    for r in skip_rows:
        seq[r] = 0
    qslot = np.arange(B, dtype=np.int32)
    dt = geom.torch_dtype()
    tq = torch.from_numpy(q).to(dt).cuda()
    tk = torch.from_numpy(kn).to(dt).cuda()
    tv = torch.from_numpy(vn).to(dt).cuda()
    out = torch.full((B, h_q, d), 7.0, dtype=dt, device="cuda")
    lse = torch.zeros((B, h_q), dtype=torch.float32, device="cuda")
    max_len = max(lens)
    g = h_q // h_kv
    hc.dev.qwin_lse = torch.full((2, B, h_kv, g, w), 9.0, dtype=torch.float32, device="cuda")
    ws = zp.new_workspace(zp.zp_decode_workspace_size(geom, B, max_len))
    zp.zp_paged_decode(hc.dev, layer, tq, tk, tv, dev_i32(tab), dev_i32(seq), max_len,
                       dev_i32(qslot), out, lse, ws)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    out_h = out.float().cpu().numpy().astype(np.float64)
    lse_h = lse.cpu().numpy()
    tol = tol_for(dtype)
    K_after = hc.dev.k.float().cpu().numpy()
    V_after = hc.dev.v.float().cpu().numpy()
    Q_after = hc.dev.qwin.float().cpu().numpy()
    QL_after = hc.dev.qwin_lse.cpu().numpy()
    expK, expV, expQ = hc.K.copy(), hc.V.copy(), hc.Q.copy()
    expQL = np.full_like(QL_after, 9.0)
    for r in range(B):
        if seq[r] <= 0:
            assert np.all(out_h[r] == 7.0)
            continue
        n = lens[r]
        Kr = np.stack([Z.gather_sequence(hc.K[layer, :, h], tab[r], n - 1, b) for h in range(h_kv)])
        Vr = np.stack([Z.gather_sequence(hc.V[layer, :, h], tab[r], n - 1, b) for h in range(h_kv)])
        Kr = np.concatenate([Kr, kn[r][:, None, :].astype(np.float64)], axis=1)
        Vr = np.concatenate([Vr, vn[r][:, None, :].astype(np.float64)], axis=1)
        o_ref, lse_ref = Z.decode_attention(q[r], Kr, Vr)
        for j in range(h_q):
            err = np.abs(out_h[r, j] - o_ref[j]).max()
            assert err <= tol * np.abs(o_ref[j]).max(), (r, j, err)
        np.testing.assert_allclose(lse_h[r], lse_ref, atol=1e-4 if dtype == "bf16" else 2e-5)
        pg, sl = tab[r][(n - 1) // b], (n - 1) % b
        expK[layer, pg, :, sl] = kn[r]
        expV[layer, pg, :, sl] = vn[r]
        if sl >= b - w:
            gq = h_q // h_kv
            expQ[layer, r] = expQ[layer, r]
            for j in range(h_q):
                expQ[layer, r, j // gq, j % gq, sl - (b - w)] = q[r, j]
                expQL[layer, r, j // gq, j % gq, sl - (b - w)] = lse_h[r, j]
    np.testing.assert_array_equal(K_after, expK)
    np.testing.assert_array_equal(V_after, expV)
    np.testing.assert_array_equal(Q_after, expQ)
    np.testing.assert_array_equal(QL_after, expQL)   # window rows' lse next to their query


def test_decode_ignores_unwritten_slots():
    """Slots of the last block past the sequence hold whatever was there
    before (here NaN): masked tokens contribute nothing, not even NaN."""
    _run_case("bf16", 64, 4, 2, 16, 8, [13, 16, 17, 200, 1], poison_tail=True)
    _run_case("f32", 64, 4, 1, 16, 8, [1, 17, 30, 16, 300], poison_tail=True)
    _run_case("bf16", 128, 32, 8, 256, 16, [1, 300, 2047, 4000], poison_tail=True)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-d{c[1]}-g{c[2]//c[3]}-b{c[4]}" for c in CASES])
def test_decode_parity(case):
    _run_case(*case)


def test_decode_split_over_many_small_blocks():
    """A split that spans more than 64 block ids. With 256 (sequence,
    kv-head) items at this shape the launch covers each sequence with one
    split (one workgroup of a CU's wavefronts per item), so a 1300-token
    sequence of 16-token blocks walks 82 block ids: the first 64 come from
    a lane of a register, the rest from LDS."""
    rng = np.random.default_rng(11)
    lens = [int(x) for x in rng.integers(1, 300, 128)]
    for r, n in zip((3, 40, 77, 127), (1025, 1040, 1299, 1300)):
        lens[r] = n
    _run_case("bf16", 128, 8, 2, 16, 16, lens)


# Lengths whose chunk counts (16 tokens each) leave every remainder mod 4,
# including sequences shorter than one round of the four wavefronts.
_TAIL_LENS = [1, 2, 15, 16, 17, 33, 48, 49, 64, 65, 100, 130, 200, 257, 300, 513, 1809, 1825, 2048]


def _tail_lens(count, long_ok, seed):
    rng = np.random.default_rng(seed)
    base = [n for n in _TAIL_LENS if long_ok or n <= 600]
    extra = [int(x) for x in rng.integers(1, 600, count - len(base))]
    return base + extra


@pytest.mark.parametrize("dtype,d,h_q,h_kv,b,count,poison", [
    ("bf16", 128, 32, 8, 256, 40, True),
    ("bf16", 64, 32, 8, 64, 40, False),
    ("f32", 128, 16, 2, 128, 130, False),
])
def test_decode_four_wave_workgroups_all_rows(dtype, d, h_q, h_kv, b, count, poison):
    """Batches with more (sequence, kv-head) items than a quarter of the GPU's
    resident wavefronts take 4-wavefront workgroups, one per item. Every row
    is checked against the oracle, with every count of 16-token chunks modulo
    the 4 wavefronts (sequences shorter than one round included), 8-row loads
    (bf16, d = 64), fp32, and (poison) unwritten NaN slots after the token,
    which the last chunk's load range leaves unread."""
    lens = _tail_lens(count, long_ok=(b == 256), seed=5)
    _run_case(dtype, d, h_q, h_kv, b, 16, lens, poison_tail=poison)


def test_decode_skips_rows_with_zero_length():
    _run_case("bf16", 128, 32, 8, 256, 16, [300, 1000, 2000], skip_rows=(1,))


def test_decode_reports_bad_block_ids_without_faulting():
    """A table entry outside the pool is masked out and flagged; the kernel
    never dereferences it."""
    announce("decode bad block id")
    geom = zp.CacheGeometry(num_layers=1, num_blocks=4, block_size=16, num_kv_heads=1,
                            num_q_heads=4, head_dim=64, window=8, max_slots=1, n_max=2, dtype="f32")
    hc = HostCache(geom, 5, 2)
    tab = np.array([[0, 99, 2]], np.int32)
    q = torch.randn(1, 4, 64, device="cuda")
    k = torch.randn(1, 1, 64, device="cuda")
    out = torch.zeros(1, 4, 64, device="cuda")
    ws = zp.new_workspace(zp.zp_decode_workspace_size(geom, 1, 40))
    zp.zp_paged_decode(hc.dev, 0, q, k, k.clone(), dev_i32(tab), dev_i32([40]), 40, None, out,
                       None, ws)
    assert zp.zp_workspace_errors(ws) & zp.ZP_DEVERR_BLOCK_ID
    assert torch.isfinite(out).all()
    zp.zp_workspace_clear_errors(ws)
    assert zp.zp_workspace_errors(ws) == 0
    # a length beyond the launch bound poisons the row and is flagged
    zp.zp_paged_decode(hc.dev, 0, q, k, k.clone(), dev_i32(tab), dev_i32([41]), 40, None, out,
                       None, ws)
    assert zp.zp_workspace_errors(ws) & zp.ZP_DEVERR_SEQ_LEN
    assert torch.isnan(out).all()


def test_decode_bench_launch_configuration_sampled():
    """256 sequences x 8 kv-heads with 1793..2048 resident tokens (one layer of
    the timed workload, one workgroup per (sequence, kv-head)); eight rows
    are checked against the oracle one by one."""
    announce("decode 256x8 bench configuration")
    B, h_q, h_kv, d, b = 256, 32, 8, 128, 256
    g = synth.rng(5, 3, 0, "lengths")
    lens = (7 * b + g.integers(1, b + 1, B)).astype(np.int32)
    geom = zp.CacheGeometry(num_layers=1, num_blocks=B * 8 + 4, block_size=b,
                            num_kv_heads=h_kv, num_q_heads=h_q, head_dim=d, window=16,
                            max_slots=B, n_max=8, dtype="bf16")
    cache = zp.PagedKVCache(geom, with_global=False)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    cache.k.normal_(generator=gen)
    cache.v.normal_(generator=gen)
    perm = torch.from_numpy(g.permutation(B * 8).astype(np.int32)).cuda()
    tab = perm.view(B, 8).contiguous()
    q = torch.randn(B, h_q, d, generator=gen, device="cuda").to(torch.bfloat16)
    kn = torch.randn(B, h_kv, d, generator=gen, device="cuda").to(torch.bfloat16)
    vn = torch.randn(B, h_kv, d, generator=gen, device="cuda").to(torch.bfloat16)
    # host snapshot of the inputs before the kernel touches the cache
    rows = [0, 1, 77, 128, 200, 254, 255, int(np.argmax(lens))]
    tab_h = tab.cpu().numpy()
    snap = {r: (cache.k[0, tab[r].long()].float().cpu().numpy(),
                cache.v[0, tab[r].long()].float().cpu().numpy()) for r in rows}
    out = torch.empty(B, h_q, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, h_q, device="cuda")
    ws = zp.new_workspace(zp.zp_decode_workspace_size(geom, B, 8 * b))
    assert ws.numel() == 256                     # no split partials at this width
    zp.zp_paged_decode(cache, 0, q, kn, vn, tab, dev_i32(lens), 8 * b, None, out, lse, ws)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    qh, kh, vh = q.float().cpu().numpy(), kn.float().cpu().numpy(), vn.float().cpu().numpy()
    oh, lh = out.float().cpu().numpy(), lse.cpu().numpy()
    for r in rows:
        n = int(lens[r])
        Kp, Vp = snap[r]                          # [8 pages][h_kv][b][d]
        K = Kp.transpose(1, 0, 2, 3).reshape(h_kv, 8 * b, d)[:, :n].astype(np.float64)
        V = Vp.transpose(1, 0, 2, 3).reshape(h_kv, 8 * b, d)[:, :n].astype(np.float64)
        K[:, n - 1] = kh[r]
        V[:, n - 1] = vh[r]
        o_ref, lse_ref = Z.decode_attention(qh[r], K, V)
        for j in range(h_q):
            assert np.abs(oh[r, j] - o_ref[j]).max() <= 2e-2 * np.abs(o_ref[j]).max(), (r, j)
        np.testing.assert_allclose(lh[r], lse_ref, atol=1e-4)
        pg, sl = tab_h[r][(n - 1) // b], (n - 1) % b
        np.testing.assert_array_equal(cache.k[0, pg, :, sl].float().cpu().numpy(), kh[r])
