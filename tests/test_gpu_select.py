"""GPU parity of zp_select_compact against the oracle (bit-exact).

Zipage (arXiv 2603.08743): Sec. 4.2 (top-k with k = (N_max - 1) b, window at
+inf), App. C.6 / Alg. 4 (ordered two-pointer move of K and V, and of F with
element size 1), Sec. 4.4 (targets are the request's own blocks or fresh ones).
The same seeded fp32 score vectors feed both sides, so the kept index sets and
every moved byte must match exactly.
"""
import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import synth, zp
from oracle import zipage as Z

from gpu_cases import HostCache, announce, dev_i32, random_tables

pytestmark = pytest.mark.gpu


def _run(dtype, d, h_kv, b, w, nblocks, keep, fresh_mask, levels, L=2, layer_begin=1,
         layer_count=1, seed=21, with_global=True, no_compact=False, use_f_new=False):
    announce(f"select dtype={dtype} d={d} b={b} N={nblocks} keep={keep} fresh={fresh_mask} "
             f"levels={levels}")
    nreq = len(nblocks)
    n_dst = -(-keep // b)
    n_fresh = sum(sum(1 for i in range(n_dst) if fresh_mask(r, i)) for r in range(nreq))
    pool = sum(nblocks) + n_fresh + 2
    max_blocks = max(nblocks)
    geom = zp.CacheGeometry(num_layers=L, num_blocks=pool, block_size=b, num_kv_heads=h_kv,
                            num_q_heads=h_kv, head_dim=d, window=16, max_slots=1, n_max=2,
                            dtype=dtype)
    hc = HostCache(geom, seed, 3, with_global=with_global)
    tab = random_tables(seed, 3, nblocks, pool, max_blocks)
    used = set(int(x) for x in tab.ravel() if x >= 0)
    free = [p for p in range(pool) if p not in used]
    dst = np.zeros((nreq, n_dst), np.int32)
    for r in range(nreq):
        for i in range(n_dst):
            dst[r, i] = free.pop(0) if fresh_mask(r, i) else tab[r, i]
    stride = max_blocks * b + 3
    S = np.full((layer_count, nreq, h_kv, stride), np.nan, np.float32)
    for li in range(layer_count):
        for r in range(nreq):
            for h in range(h_kv):
                n = nblocks[r] * b
                S[li, r, h, :n] = synth.scores_with_ties(seed + 97 * li + 13 * h, r, n, w, levels)
    FN = (synth.rng(seed, 3, 1, "gscore").random(S.shape) * 0.01).astype(np.float32)
    kept = torch.full((layer_count, nreq, h_kv, keep), -1, dtype=torch.int32, device="cuda")
    ws = zp.new_workspace(zp.zp_select_workspace_size(geom, layer_count, nreq, keep))
    zp.zp_select_compact(hc.dev, layer_begin, layer_count, torch.from_numpy(S).cuda(),
                         dev_i32(tab), dev_i32(nblocks), max_blocks, dev_i32(dst), keep, kept, ws,
                         flags=zp.ZP_SELECT_NO_COMPACT if no_compact else 0,
                         f_new=torch.from_numpy(FN).cuda() if use_f_new else None)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    kept_h = kept.cpu().numpy()
    expK, expV, expF = hc.K.copy(), hc.V.copy(), hc.F.copy()
    for li in range(layer_count):
        l = layer_begin + li
        for r in range(nreq):
            n = nblocks[r] * b
            for h in range(h_kv):
                ref = Z.topk_keep(S[li, r, h, :n].astype(np.float64), keep)
                np.testing.assert_array_equal(kept_h[li, r, h], ref)
                if no_compact:
                    continue
                tag = np.zeros(n, bool)
                tag[ref] = True
                expK[l, :, h] = Z.compact_pages(expK[l, :, h], tab[r], n, dst[r], tag, b)
                expV[l, :, h] = Z.compact_pages(expV[l, :, h], tab[r], n, dst[r], tag, b)
                if use_f_new:
                    # the updated history is moved instead of the cache's old F
                    for j, t in enumerate(ref):
                        expF[l, dst[r][j // b], h, j % b] = FN[li, r, h, t]
                else:
                    expF[l, :, h] = Z.compact_pages(expF[l, :, h], tab[r], n, dst[r], tag, b)
    np.testing.assert_array_equal(hc.dev.k.float().cpu().numpy(), expK)
    np.testing.assert_array_equal(hc.dev.v.float().cpu().numpy(), expV)
    if with_global:
        np.testing.assert_array_equal(hc.dev.gscore.cpu().numpy(), expF)


def test_select_in_place_qwen_shape_with_ties():
    _run("bf16", 128, 8, 256, 16, [8, 8, 9], 7 * 256, lambda r, i: False, levels=5)


def test_select_fresh_targets_prefix_like():
    # the first four target blocks are fresh (shared-prefix positions); the
    # updated global scores come from f_new
    _run("bf16", 128, 8, 256, 16, [8, 10], 7 * 256, lambda r, i: i < 4, levels=None,
         use_f_new=True)


def test_select_mid_length_ragged_with_ties():
    # 4352..8192 tokens per unit (up to 32 keys per thread in the selection)
    _run("bf16", 128, 2, 256, 16, [17, 32, 20], 7 * 256, lambda r, i: r == 1 and i % 3 == 0,
         levels=3, layer_count=1)


def test_select_long_context_to_budget():
    _run("bf16", 128, 2, 256, 16, [64, 128, 20], 7 * 256, lambda r, i: r == 2 and i % 2 == 0,
         levels=3, layer_count=1)


def test_select_tiny_fp32_and_all_kept():
    _run("f32", 64, 1, 16, 8, [13], 48, lambda r, i: False, levels=4, L=1, layer_begin=0)
    _run("f32", 64, 1, 16, 8, [3, 4], 48, lambda r, i: r == 1, levels=None, L=1, layer_begin=0)


def test_select_only_and_no_global():
    _run("bf16", 64, 4, 32, 16, [6, 7], 5 * 32, lambda r, i: False, levels=2, no_compact=True)
    _run("f32", 128, 2, 64, 16, [5], 4 * 64, lambda r, i: i == 3, levels=None,
         with_global=False, L=3, layer_begin=0, layer_count=3)
