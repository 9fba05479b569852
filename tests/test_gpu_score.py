"""GPU parity of zp_score_tokens against the float64 oracle.

Zipage (arXiv 2603.08743): App. C.2 Alg. 1 (window logits, causal last block,
softmax, GQA max, window mean), App. C.3 Alg. 2 (global score with F updated
in place), App. C.4 (pooling), App. C.5 eq. (4) / C.7 / C.8 (lightning
redundancy, tempered softmax), App. C.6 Alg. 3 (flash redundancy over the
whole sequence), Sec. 4.2 (+inf window).

Bar: the GPU accumulates in fp32 from inputs that both sides hold exactly,
so |S_gpu - S_ref| <= 2e-5 * max|S_ref| over the finite entries, +inf
exactly on the window, and the updated global score f_new within the same
bound; the cache's F must be left untouched. Cases with
p below the planted-cluster cosines check the redundancy threshold logic
where no cosine lies near p (the test asserts that margin on the oracle side).
"""
import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import synth, zp
from oracle import zipage as Z

from gpu_cases import HostCache, announce, dev_i32, random_tables

pytestmark = pytest.mark.gpu

SCORE_TOL = 2e-5


def _oracle_params(sp: zp.ScoreParams):
    return Z.ScoreParams(alpha=sp.alpha, lam=sp.lam, tau=sp.tau, p=sp.p,
                         pool_kernel=sp.pool_kernel, use_global=sp.use_global,
                         global_reduce=sp.global_reduce,
                         use_pool=sp.use_pool, pool_first_only=sp.pool_first_only,
                         use_redundancy=sp.use_redundancy, redundancy=sp.redundancy)


def _planted_keys(hc, seed):
    """Replace every key by a positive multiple of one of eight basis
    directions: in-block cosines are then exactly 0 (different directions,
    disjoint support, exact on both sides) or 1 up to rounding, far from any
    threshold p in [0, 0.99)."""
    g = synth.rng(seed, 9, 0, "misc")
    G = hc.geom
    lab = g.integers(0, 8, hc.K.shape[:4])
    sc = g.uniform(0.5, 3.0, hc.K.shape[:4])
    K = np.zeros_like(hc.K)
    np.put_along_axis(K, lab[..., None], sc[..., None], axis=-1)
    hc.K = synth.cast(K, G.dtype)


def _window_lse(Qw, K, b):
    """log-sum-exp of each window row's causal attention row (oracle logits)."""
    A = Z.window_logits(Qw, K, b)              # [g][w][n], -inf past each query
    m = A.max(axis=-1, keepdims=True)
    return (m[..., 0] + np.log(np.exp(A - m).sum(axis=-1)))


def _run(dtype, d, h_q, h_kv, b, w, nblocks, first, sp, L=3, layer_begin=1, layer_count=2,
         seed=11, planted=False, heavy=True, lse=None, repeat=1, lse_all=False):
    announce(f"score dtype={dtype} d={d} g={h_q // h_kv} b={b} w={w} N={nblocks} first={first} "
             f"sp={sp}")
    nreq = len(nblocks)
    max_blocks = max(nblocks)
    pool = sum(nblocks) + 2
    geom = zp.CacheGeometry(num_layers=L, num_blocks=pool, block_size=b, num_kv_heads=h_kv,
                            num_q_heads=h_q, head_dim=d, window=w, max_slots=nreq + 1, n_max=2,
                            dtype=dtype)
    hc = HostCache(geom, seed, 2)
    if heavy:
        hc.plant_heavy(seed, 2)
    tab = random_tables(seed, 2, nblocks, pool, max_blocks + 1)
    if planted:
        _planted_keys(hc, seed)
    hc.upload()
    qslot = np.array([(r + 1) % (nreq + 1) for r in range(nreq)], np.int32)
    firsts = np.array([first(r) for r in range(nreq)], np.uint8)
    stride = max_blocks * b + 5
    scores = torch.full((layer_count, nreq, h_kv, stride), -7.0, device="cuda")
    f_new = torch.full_like(scores, -5.0) if sp.use_global else None
    F_before = hc.dev.gscore.clone()
    lse_valid = None
    if lse is not None:
        # window log-sum-exp from the oracle for the requests that have it;
        # a far-off value elsewhere, which must not be used
        g = h_q // h_kv
        tbl = np.full((L, nreq + 1, h_kv, g, w), 1.0e3, np.float32)
        flags = np.array([1 if lse(r) else 0 for r in range(nreq)], np.uint8)
        for li in range(layer_count):
            l = layer_begin + li
            for r in range(nreq):
                if flags[r] and nblocks[r] > 0:
                    for h in range(h_kv):
                        K = Z.gather_sequence(hc.K[l, :, h], tab[r], nblocks[r] * b, b)
                        tbl[l, qslot[r], h] = _window_lse(hc.Q[l, qslot[r], h], K, b)
        hc.dev.qwin_lse = torch.from_numpy(tbl).cuda()
        lse_valid = torch.from_numpy(flags).cuda()
    ws = zp.new_workspace(zp.zp_score_workspace_size(geom, layer_count, nreq, max_blocks))
    zp.zp_score_tokens(hc.dev, sp, layer_begin, layer_count, dev_i32(tab), dev_i32(nblocks),
                       max_blocks, dev_i32(qslot), torch.from_numpy(firsts).cuda(), scores, f_new,
                       ws, window_lse_valid=lse_valid)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    assert torch.equal(hc.dev.gscore, F_before)        # the cache's F is only read
    for _ in range(repeat - 1):
        # the same call again, into fresh outputs and a fresh workspace: every
        # score and history value must come out with the same bits
        sc2 = torch.full_like(scores, -7.0)
        fn2 = torch.full_like(f_new, -5.0) if f_new is not None else None
        ws2 = zp.new_workspace(ws.numel())
        # with lse_all the repeats say "every request has it" by the call
        # flag instead of the per-request array (which is then not passed)
        zp.zp_score_tokens(hc.dev, sp, layer_begin, layer_count, dev_i32(tab), dev_i32(nblocks),
                           max_blocks, dev_i32(qslot), torch.from_numpy(firsts).cuda(), sc2, fn2,
                           ws2, window_lse_valid=None if lse_all else lse_valid,
                           window_lse_all=lse_all)
        torch.cuda.synchronize()
        assert torch.equal(sc2.view(torch.int32), scores.view(torch.int32))
        if f_new is not None:
            assert torch.equal(fn2.view(torch.int32), f_new.view(torch.int32))
    S_gpu = scores.cpu().numpy()
    Fn_gpu = f_new.cpu().numpy() if f_new is not None else None
    op = _oracle_params(sp)
    worst = 0.0
    for li in range(layer_count):
        l = layer_begin + li
        for r in range(nreq):
            n = nblocks[r] * b
            if n == 0:  # a request without blocks is skipped: nothing written
                assert np.all(S_gpu[li, r] == -7.0)
                assert Fn_gpu is None or np.all(Fn_gpu[li, r] == -5.0)
                continue
            for h in range(h_kv):
                K = Z.gather_sequence(hc.K[l, :, h], tab[r], n, b)
                Fo = Z.gather_sequence(hc.F[l, :, h], tab[r], n, b)
                S_ref, F_ref, parts = Z.score_tokens(hc.Q[l, qslot[r], h], K, Fo, bool(firsts[r]),
                                                     b, op, return_parts=True)
                if sp.use_redundancy and planted:
                    # no cosine within 1e-3 of p: the threshold decision is robust
                    # (within blocks for lightning, over the sequence for flash)
                    span = n if sp.redundancy == "flash" else b
                    for i in range(n // span):
                        C = Z.cosine_matrix(K[i * span:(i + 1) * span], K[i * span:(i + 1) * span])
                        np.fill_diagonal(C, 0)
                        off = C[C != 0]
                        assert off.size == 0 or np.min(np.abs(off - sp.p)) > 1e-3
                got = S_gpu[li, r, h]
                assert np.all(got[n:] == -7.0)          # nothing written past n
                got = got[:n]
                fin = np.isfinite(S_ref)
                assert np.array_equal(np.isinf(got), ~fin) and np.all(got[~fin] > 0)
                scale = np.abs(S_ref[fin]).max()
                err = np.abs(got[fin] - S_ref[fin]).max() / scale
                worst = max(worst, err)
                assert err <= SCORE_TOL, (li, r, h, err)
                if sp.use_global:
                    Fg = Fn_gpu[li, r, h]
                    assert np.all(Fg[n:] == -5.0)
                    np.testing.assert_allclose(Fg[:n], F_ref, atol=SCORE_TOL * np.abs(F_ref).max())
    print(f"max relative score error {worst:.3e}", flush=True)


DEFAULT = zp.ScoreParams()


def test_score_tiny_fp32_first_compression():
    _run("f32", 64, 4, 1, 16, 8, [13], lambda r: 1, DEFAULT, L=1, layer_begin=0, layer_count=1)


def test_score_tiny_fp32_later_compression_every_part():
    sp = zp.ScoreParams(pool_first_only=False)
    _run("f32", 64, 4, 1, 16, 8, [4, 6, 5], lambda r: r == 1, sp)


def test_score_qwen_shape_bf16_mixed_first():
    _run("bf16", 128, 32, 8, 256, 16, [8, 16, 9], lambda r: r % 2, DEFAULT)


@pytest.mark.parametrize("flags", [
    dict(use_global=False, use_pool=False, use_redundancy=False),
    dict(use_pool=False),
    dict(use_redundancy=False),
    dict(use_global=False, pool_kernel=3),
    dict(global_reduce="sum"),
    dict(global_reduce="sum", use_pool=False, use_redundancy=False),
])
def test_score_flag_combinations(flags):
    sp = zp.ScoreParams(**flags)
    _run("bf16", 128, 32, 8, 256, 16, [8, 8], lambda r: r == 0, sp, L=2, layer_begin=0,
         layer_count=2)


@pytest.mark.parametrize("p", [0.0, 0.5])
def test_score_redundancy_threshold_planted_serving_shape(p):
    """Planted clusters in blocks of 256 (d 128, g 4, w 16: the persistent
    kernel), first and later compressions, several requests per workgroup."""
    sp = zp.ScoreParams(p=p, pool_first_only=False)
    _run("bf16", 128, 32, 8, 256, 16, [5, 3, 7], lambda r: r != 1, sp, planted=True, heavy=False)


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5])
def test_score_redundancy_threshold_sweep_planted(p):
    sp = zp.ScoreParams(p=p, use_global=False, use_pool=False)
    _run("bf16", 128, 16, 4, 64, 16, [4, 3], lambda r: 1, sp, planted=True, heavy=False)


def test_score_other_shapes():
    _run("bf16", 64, 8, 8, 32, 16, [5, 2], lambda r: 0, DEFAULT, L=1, layer_begin=0,
         layer_count=1)
    _run("f32", 128, 16, 2, 64, 2, [3, 4], lambda r: 1, DEFAULT, L=1, layer_begin=0,
         layer_count=1)


FLASH = zp.ScoreParams(redundancy="flash")


@pytest.mark.parametrize("sp", [DEFAULT, zp.ScoreParams(redundancy="flash", pool_first_only=False)],
                         ids=["lightning", "flash"])
def test_score_more_requests_than_a_wavefront(sp):
    """70 requests of 1-3 blocks on the persistent kernels' shape: each
    workgroup places its first item with 64 requests per step, so items of
    requests 64..69 are found on the second step."""
    nb = [1 + (r * 7) % 3 for r in range(70)]
    _run("bf16", 128, 8, 2, 256, 16, nb, lambda r: r % 3 != 0, sp, L=1, layer_begin=0,
         layer_count=1)


@pytest.mark.parametrize("sp", [DEFAULT, zp.ScoreParams(redundancy="flash")],
                         ids=["lightning", "flash"])
@pytest.mark.parametrize("with_lse", [False, True], ids=["stats", "lse"])
def test_score_requests_without_blocks_among_many(sp, with_lse):
    """130 requests over three 64-request steps of the persistent kernels'
    cursor, a fifth of them with no blocks (first, last and runs of them):
    those are skipped and left unwritten, the rest score as the oracle."""
    nb = [0 if (r % 5 == 0 or r in (1, 2, 129)) else 1 + (r % 2) for r in range(130)]
    _run("bf16", 128, 8, 2, 256, 16, nb, lambda r: r % 2, sp, L=1, layer_begin=0, layer_count=1,
         lse=(lambda r: r % 3 != 1) if with_lse else None)


@pytest.mark.parametrize("sp", [DEFAULT, zp.ScoreParams(redundancy="flash")],
                         ids=["lightning", "flash"])
def test_score_cursor_wraps_layers_past_empty_requests(sp):
    """Three layers of a four-layer cache, 3 kv-heads, the first and last
    two requests without blocks. 9 x 59 = 531 items over 256 workgroups
    give each workgroup two or three consecutive items; the (layer, kv-head)
    boundaries at items 59, 177 (a layer change), 295 and 413 fall inside a
    workgroup's range, so that workgroup steps across the empty requests at
    both ends (the lightning kernel one item at a time, the flash kernel in
    strides). With 2 kv-heads and 2 layers every boundary would fall on the
    start of a range."""
    nb = [0, 10, 9, 11, 10, 9, 10, 0, 0]
    _run("bf16", 128, 12, 3, 256, 16, nb, lambda r: r % 2, sp, L=4, layer_begin=1,
         layer_count=3, lse=lambda r: r != 3)


def test_score_flash_redundancy_qwen_shape_bf16():
    _run("bf16", 128, 32, 8, 256, 16, [8, 16, 9], lambda r: r % 2, FLASH)


def test_score_flash_redundancy_tiny_fp32_and_single_block():
    _run("f32", 64, 4, 1, 16, 8, [13, 1, 4], lambda r: r != 2, FLASH, L=1, layer_begin=0,
         layer_count=1)
    _run("f32", 128, 16, 2, 128, 16, [3, 5], lambda r: 1, FLASH, L=1, layer_begin=0,
         layer_count=1)


@pytest.mark.parametrize("p", [0.0, 0.5])
def test_score_flash_redundancy_planted_clusters_across_blocks(p):
    # eight directions spread over all blocks: every column has partners above
    # p in other blocks, so the zero-out tags carry across row blocks
    sp = zp.ScoreParams(p=p, use_global=False, use_pool=False, redundancy="flash")
    _run("bf16", 128, 16, 4, 64, 16, [4, 7], lambda r: 1, sp, planted=True, heavy=False)
    _run("bf16", 64, 8, 8, 32, 16, [5, 2], lambda r: 0, sp, L=1, layer_begin=0, layer_count=1,
         planted=True, heavy=False)


@pytest.mark.parametrize("p", [0.0, 0.5])
def test_score_flash_redundancy_planted_serving_shape(p):
    """Planted clusters over blocks of 256 (d 128, g 4: the persistent flash
    kernel), so each column's highest row above p can lie in any row block;
    several column blocks per workgroup, ragged requests."""
    sp = zp.ScoreParams(p=p, pool_first_only=False, redundancy="flash")
    _run("bf16", 128, 32, 8, 256, 16, [5, 3, 7], lambda r: r != 1, sp, planted=True, heavy=False)


@pytest.mark.parametrize("red", ["lightning", "flash"])
def test_score_with_window_lse_qwen_shape(red):
    # requests 0 and 2 bring their window rows' log-sum-exp: one pass over K
    sp = zp.ScoreParams(redundancy=red)
    _run("bf16", 128, 32, 8, 256, 16, [8, 16, 9], lambda r: r % 2, sp, lse=lambda r: r != 1)


@pytest.mark.parametrize("red", ["lightning", "flash"])
def test_score_window_lse_all_flag_same_bits(red):
    # every request carries its window log-sum-exp: the call flag (no
    # statistics launch, no flag array) gives the bits of the per-request flags
    sp = zp.ScoreParams(redundancy=red)
    _run("bf16", 128, 32, 8, 256, 16, [8, 16, 9], lambda r: r % 2, sp, lse=lambda r: True,
         repeat=2, lse_all=True)
    _run("bf16", 128, 16, 2, 64, 8, [3, 5], lambda r: 1, sp, L=1, layer_begin=0, layer_count=1,
         lse=lambda r: True, repeat=2, lse_all=True)


def test_score_global_sum_reduce_every_path():
    """App. C.3's decayed sum-reduce on the one-pass (window LSE given) and
    the statistics paths, fp32 and bf16, mixed first / later compressions."""
    sp = zp.ScoreParams(global_reduce="sum", pool_first_only=False)
    _run("f32", 64, 4, 1, 16, 8, [4, 6, 5], lambda r: r == 1, sp)
    _run("bf16", 128, 32, 8, 256, 16, [8, 16, 9], lambda r: r % 2, sp, lse=lambda r: r != 1)


def test_score_with_window_lse_other_windows():
    # w != 16 takes the general S0 path inside the first pass
    _run("f32", 64, 4, 1, 16, 8, [13, 4], lambda r: r == 0, DEFAULT, L=1, layer_begin=0,
         layer_count=1, lse=lambda r: True)
    _run("bf16", 128, 16, 2, 64, 8, [3, 5], lambda r: 1, DEFAULT, L=1, layer_begin=0,
         layer_count=1, lse=lambda r: r == 1)


@pytest.mark.parametrize("redundancy", ["lightning", "flash"])
def test_score_bit_reproducible(redundancy):
    """Scores are the same bits on every run. Threshold 0 makes nearly every
    column of every cosine matrix zero one entry (the most order-dependent
    sums), and planted clusters stack many zeroed entries on one row."""
    sp = zp.ScoreParams(p=0.0, redundancy=redundancy, pool_first_only=False)
    _run("bf16", 128, 32, 8, 256, 16, [8, 16, 9], lambda r: r % 2, sp, repeat=4)
    sp = zp.ScoreParams(p=0.5, redundancy=redundancy, use_global=False)
    _run("bf16", 128, 16, 4, 64, 16, [6, 3], lambda r: 1, sp, planted=True, heavy=False, repeat=4)


@pytest.mark.parametrize("red", ["lightning", "flash"])
def test_score_request_past_max_blocks_is_flagged_and_skipped(red):
    """A request whose block count exceeds max_blocks raises the sequence-length
    error and is left unwritten; the other requests score as they do when it
    has no blocks at all."""
    announce(f"score past-max-blocks red={red}")
    b, nb, maxb = 256, [2, 5, 3], 3
    geom = zp.CacheGeometry(num_layers=1, num_blocks=sum(nb) + 2, block_size=b, num_kv_heads=2,
                            num_q_heads=8, head_dim=128, window=16, max_slots=4, n_max=2,
                            dtype="bf16")
    hc = HostCache(geom, 5, 2)
    hc.plant_heavy(5, 2)
    hc.upload()
    tab = dev_i32(random_tables(5, 2, nb, geom.num_blocks, max(nb)))
    qslot = dev_i32(np.array([1, 2, 3], np.int32))
    first = torch.ones(3, dtype=torch.uint8, device="cuda")
    sp = zp.ScoreParams(redundancy=red)
    out = []
    for counts in ([2, 5, 3], [2, 0, 3]):
        sc = torch.full((1, 3, 2, maxb * b), -7.0, device="cuda")
        fn = torch.full_like(sc, -5.0)
        ws = zp.new_workspace(zp.zp_score_workspace_size(geom, 1, 3, maxb))
        zp.zp_score_tokens(hc.dev, sp, 0, 1, tab, dev_i32(np.array(counts, np.int32)), maxb,
                           qslot, first, sc, fn, ws)
        torch.cuda.synchronize()
        out.append((sc.cpu().numpy(), fn.cpu().numpy(), zp.zp_workspace_errors(ws)))
    (s_bad, f_bad, e_bad), (s_ok, f_ok, e_ok) = out
    assert e_bad & zp.ZP_DEVERR_SEQ_LEN and e_ok == 0
    assert np.all(s_bad[:, 1] == -7.0) and np.all(f_bad[:, 1] == -5.0)
    for r in (0, 2):
        np.testing.assert_allclose(s_bad[:, r], s_ok[:, r], rtol=1e-6, atol=0)
        np.testing.assert_allclose(f_bad[:, r], f_ok[:, r], rtol=1e-6, atol=0)
