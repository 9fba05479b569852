"""The compression chain at full width, in the shape bench.py's compression
kernels are timed on: 64 requests x 4096 tokens (16 full blocks of 256), one
layer of the Qwen3-8B attention shape (32 query / 8 kv heads, d 128, bf16,
window 16), first compression with lightning or flash redundancy, keep 7
blocks (1792 tokens) into each request's own first blocks (Zipage, arXiv 2603.08743,
Sec. 4.2, App. C.2-C.8, Alg. 4).

Every (request, kv-head) unit, 512 of them:
  - the kept list is the top-k of the GPU's own scores (oracle topk_keep,
    bit-exact, ties newer first) and holds the window;
  - the compacted K, V and global-score rows are the old rows at the kept
    positions, in order, in the target blocks (bit-exact).
Sampled units (requests spread over every workgroup range of the persistent
scoring kernel, two of them through the window log-sum-exp path, two
through the statistics pass, three kv-heads each): the scores against the
float64 oracle, and the kept set against the oracle's scores under the 1e-6
tie rule. A third case gives every request its window log-sum-exp and says
so by the call flag, as the timed compression leg does.
"""
import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import zp
from oracle import zipage as Z

from gpu_cases import HostCache, announce, dev_i32, random_tables
from keptsets import check_kept
from test_gpu_score import SCORE_TOL, _oracle_params, _window_lse

pytestmark = pytest.mark.gpu

R, NB, BS, D, HQ, HKV, W, NMAX = 64, 16, 256, 128, 32, 8, 16, 8
SAMPLE_REQ = {0: True, 21: False, 42: True, 63: False}   # request -> window LSE given
SAMPLE_HEADS = [0, 3, 7]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("redundancy,all_lse", [("lightning", False), ("flash", False),
                                               ("lightning", True)],
                         ids=["lightning", "flash", "lightning-all-lse"])
def test_burst_full_width_compression_chain(redundancy, all_lse):
    announce(f"burst full width: {R} requests x {NB * BS} tokens, {redundancy}, "
             f"keep {(NMAX - 1) * BS}, all window lse {all_lse}")
    sample = {r: True for r in SAMPLE_REQ} if all_lse else SAMPLE_REQ
    n, keep, g = NB * BS, (NMAX - 1) * BS, HQ // HKV
    pool = R * NB + 4
    geom = zp.CacheGeometry(num_layers=1, num_blocks=pool, block_size=BS, num_kv_heads=HKV,
                            num_q_heads=HQ, head_dim=D, window=W, max_slots=R, n_max=NMAX,
                            dtype="bf16")
    seed = 23
    hc = HostCache(geom, seed, 2)
    hc.plant_heavy(seed, 2)
    hc.upload()
    tab = random_tables(seed, 2, [NB] * R, pool, NB)
    dst = tab[:, :NMAX - 1].copy()
    qslot = np.arange(R, dtype=np.int32)
    first = np.ones(R, np.uint8)
    lse_ok = np.zeros(R, np.uint8)
    sp = zp.ScoreParams(redundancy=redundancy)
    op = _oracle_params(sp)
    # window log-sum-exp from the oracle for the requests that take that path
    tbl = np.zeros((1, R, HKV, g, W), np.float32)
    Kseq = {}
    for r in range(R):
        given = sample.get(r, False) or all_lse
        if r not in sample and not all_lse:
            continue
        for h in range(HKV):
            if given or h in SAMPLE_HEADS:
                Kseq[r, h] = Z.gather_sequence(hc.K[0, :, h], tab[r], n, BS)
            if given:
                tbl[0, r, h] = _window_lse(hc.Q[0, r, h], Kseq[r, h], BS)
        lse_ok[r] = 1 if given else 0
    hc.dev.qwin_lse = torch.from_numpy(tbl).cuda()
    K0, V0, F0 = hc.K.copy(), hc.V.copy(), hc.F.copy()

    scores = torch.full((1, R, HKV, n), -7.0, device="cuda")
    f_new = torch.full_like(scores, -5.0)
    sws = zp.new_workspace(zp.zp_score_workspace_size(geom, 1, R, NB))
    tab_d, nblk_d = dev_i32(tab), dev_i32(np.full(R, NB, np.int32))
    zp.zp_score_tokens(hc.dev, sp, 0, 1, tab_d, nblk_d, NB, dev_i32(qslot),
                       torch.from_numpy(first).cuda(), scores, f_new, sws,
                       window_lse_valid=None if all_lse else torch.from_numpy(lse_ok).cuda(),
                       window_lse_all=all_lse)
    kept = torch.full((1, R, HKV, keep), -1, dtype=torch.int32, device="cuda")
    cws = zp.new_workspace(zp.zp_select_workspace_size(geom, 1, R, keep))
    zp.zp_select_compact(hc.dev, 0, 1, scores, tab_d, nblk_d, NB, dev_i32(dst), keep, kept, cws,
                         f_new=f_new)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(sws) == 0 and zp.zp_workspace_errors(cws) == 0
    S = scores.cpu().numpy()[0]
    FN = f_new.cpu().numpy()[0]
    kept_h = kept.cpu().numpy()[0]
    Kd = hc.dev.k.float().cpu().numpy()[0]
    Vd = hc.dev.v.float().cpu().numpy()[0]
    Fd = hc.dev.gscore.cpu().numpy()[0]

    # every unit: top-k of the GPU's own scores, the window kept, the move
    for r in range(R):
        for h in range(HKV):
            s = S[r, h].astype(np.float64)
            assert np.all(np.isinf(s[n - W:])) and np.all(np.isfinite(s[:n - W])), (r, h)
            ref = Z.topk_keep(s, keep)
            np.testing.assert_array_equal(kept_h[r, h], ref, err_msg=f"request {r} head {h}")
            src_rows = np.stack([K0[0, tab[r, t // BS], h, t % BS] for t in ref])
            got = Kd[dst[r], h].reshape(keep, D)
            np.testing.assert_array_equal(got, src_rows, err_msg=f"K request {r} head {h}")
            src_rows = np.stack([V0[0, tab[r, t // BS], h, t % BS] for t in ref])
            np.testing.assert_array_equal(Vd[dst[r], h].reshape(keep, D), src_rows,
                                          err_msg=f"V request {r} head {h}")
            np.testing.assert_array_equal(Fd[dst[r], h].reshape(keep), FN[r, h, ref],
                                          err_msg=f"F request {r} head {h}")
    # sampled units against the oracle
    worst = 0.0
    for r in sample:
        for h in SAMPLE_HEADS:
            Fo = Z.gather_sequence(F0[0, :, h], tab[r], n, BS)
            S_ref, _ = Z.score_tokens(hc.Q[0, r, h], Kseq[r, h], Fo, True, BS, op)
            fin = np.isfinite(S_ref)
            assert np.array_equal(np.isinf(S[r, h]), ~fin)
            err = np.abs(S[r, h][fin] - S_ref[fin]).max() / np.abs(S_ref[fin]).max()
            worst = max(worst, err)
            assert err <= SCORE_TOL, (r, h, err)
            chk = check_kept(kept_h[r, h], S_ref, keep)
            print(f"request {r} head {h} (lse {sample[r]}): score err {err:.2e}; kept "
                  f"{'same' if chk.same else chk.describe()}")
            assert chk.ok, (r, h, chk.describe())
    print(f"burst full width: 512 units top-k + move bit-exact; sampled worst score error {worst:.2e}")
