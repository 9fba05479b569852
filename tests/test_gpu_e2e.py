"""End-to-end GPU parity: decode steps, the compression trigger, scoring,
selection and compaction driven by the engine, against the oracle's logical
simulation of the same requests (Zipage, arXiv 2603.08743, Sec. 4.1-4.5,
App. C).

Bars: decode outputs within 1e-5 (fp32) / 2e-2 (bf16) of max |ref| per
(step, head); kept sets equal outside the tie zone |S_ref - s_k| <= delta with
delta = max(1e-6 |s_k|, 2 * 2e-5 * max|S_ref|) (the score parity bound: a
membership difference outside it would need a score error above that bound);
inside the zone only the count must match; resident K/V bit-exact when the
kept sets agree.
"""
import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import synth, zp
from compressed_paged_kv_gqa_amd.engine import DecodeEngine
from oracle import zipage as Z

from gpu_cases import announce, tol_for

pytestmark = pytest.mark.gpu

SCORE_TOL = 2e-5


def _oracle_params(sp):
    return Z.ScoreParams(alpha=sp.alpha, lam=sp.lam, tau=sp.tau, p=sp.p,
                         pool_kernel=sp.pool_kernel, use_global=sp.use_global,
                         use_pool=sp.use_pool, pool_first_only=sp.pool_first_only,
                         use_redundancy=sp.use_redundancy)


def _compare_kept(kept_gpu, S_ref, keep):
    """Returns (#outside-zone mismatches, #inside-1e-6-zone, agree?)."""
    ref = Z.topk_keep(S_ref, keep)
    if np.array_equal(np.sort(kept_gpu), ref):
        return 0, True
    fin = np.isfinite(S_ref)
    sk = np.sort(S_ref)[::-1][keep - 1]
    delta = max(1e-6 * abs(sk), 2 * SCORE_TOL * np.abs(S_ref[fin]).max())
    zone = np.abs(S_ref - sk) <= delta
    g = np.zeros(len(S_ref), bool)
    g[kept_gpu] = True
    r = np.zeros(len(S_ref), bool)
    r[ref] = True
    outside = int(np.sum((g != r) & ~zone))
    assert g.sum() == r.sum() == keep
    return outside, False


def _run_requests(cfg, geom, sp, inputs, n_steps, sample, layer_stride=1, async_compress=True):
    """Drives all requests on the GPU; compares `sample` of them with the
    oracle simulation. `inputs[r]` is a synth.RequestInputs."""
    B = len(inputs)
    L, h_q, h_kv, d = geom.num_layers, geom.num_q_heads, geom.num_kv_heads, geom.head_dim
    dt = geom.torch_dtype()
    cap = max(-(-(x.prompt_k.shape[2] + n_steps) // geom.block_size) for x in inputs) + 1
    eng = DecodeEngine(geom, sp, B, cap, layer_stride=layer_stride,
                       async_compress=async_compress, record=True)
    for r, x in enumerate(inputs):
        n0 = x.prompt_k.shape[2]
        eng.add_request(r, n0)
        for l in range(L):
            eng.write_tokens(r, l, 0, torch.from_numpy(x.prompt_k[l]).to(dt).cuda(),
                             torch.from_numpy(x.prompt_v[l]).to(dt).cuda())
            if x.prompt_q is not None:
                b, w = geom.block_size, geom.window
                # window rows of the prompt's last block (when that block is full)
                qw = np.zeros((h_kv, h_q // h_kv, w, d), np.float32)
                for pos in range(n0 - w, n0):
                    row = Z.window_row(pos, b, w)
                    if row >= 0:
                        qw[:, :, row] = x.prompt_q[l, :, pos].reshape(h_kv, h_q // h_kv, d)
                eng.write_window_queries(r, l, torch.from_numpy(qw).to(dt).cuda())
    eng.compress_due_now()
    eng.wait_compressions()
    outs = torch.zeros((n_steps, L, B, h_q, d), dtype=dt, device="cuda")
    q_all = torch.stack([torch.from_numpy(np.stack([x.steps_q[:, l] for x in inputs], 1))
                         for l in range(L)], 1).to(dt).cuda()            # [T][L][B][h_q][d]
    k_all = torch.stack([torch.from_numpy(np.stack([x.steps_k[:, l] for x in inputs], 1))
                         for l in range(L)], 1).to(dt).cuda()
    v_all = torch.stack([torch.from_numpy(np.stack([x.steps_v[:, l] for x in inputs], 1))
                         for l in range(L)], 1).to(dt).cuda()
    for s in range(n_steps):
        act = eng.step(q_all[s], k_all[s], v_all[s], outs[s])
        assert len(act) == B
        eng.wait_compressions()      # keep every request in every step
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(eng.dec_ws) == 0
    outs_h = outs.float().cpu().numpy()
    op = _oracle_params(sp)
    tol = tol_for(geom.dtype)
    worst_out = 0.0
    for r in sample:
        x = inputs[r]
        announce(f"{cfg}: oracle for request {r}")
        res = Z.simulate_request(x.prompt_k, x.prompt_v, x.prompt_q, x.steps_q, x.steps_k,
                                 x.steps_v, geom.block_size, geom.window, geom.n_max, op)
        # compression events of this request, in order
        gpu_events = [(sids.index(r), first, sc, kept) for (sids, first, sc, kept) in eng.log
                      if r in sids]
        assert len(gpu_events) == len(res["events"])
        agree = True
        for (i, first, sc, kept), ev in zip(gpu_events, res["events"]):
            kept_h = kept.cpu().numpy()
            for l in range(L):
                for h in range(h_kv):
                    outside, same = _compare_kept(kept_h[l, i, h], ev["scores"][l, h], geom.keep)
                    assert outside == 0, (cfg, r, l, h)
                    agree &= same
        if not agree:
            print(f"{cfg}: request {r} kept sets differ inside the tie zone; "
                  "decode after it is not comparable", flush=True)
            continue
        for s in range(n_steps):
            for l in range(L):
                for j in range(h_q):
                    ref = res["outputs"][s, l, j]
                    err = np.abs(outs_h[s, l, r, j] - ref).max() / np.abs(ref).max()
                    worst_out = max(worst_out, err)
                    assert err <= tol, (cfg, r, s, l, j, err)
        for l in range(L):
            for h in range(h_kv):
                K, V = eng.resident_kv(r, l, h)
                np.testing.assert_array_equal(K.float().cpu().numpy(), res["K"][l][h])
                np.testing.assert_array_equal(V.float().cpu().numpy(), res["V"][l][h])
    print(f"{cfg}: worst decode error {worst_out:.3e}", flush=True)
    return eng


def test_tiny_fp32_end_to_end():
    """1 layer, 1 request, 4 query / 1 kv head, d 64, fp32, b 16, N_max 4,
    200-token prompt, 8 decode steps filling the window (w 8) -> compression
    to 48 tokens -> 8 more steps into the reserved block."""
    announce("e2e tiny fp32")
    geom = zp.CacheGeometry(num_layers=1, num_blocks=20, block_size=16, num_kv_heads=1,
                            num_q_heads=4, head_dim=64, window=8, max_slots=1, n_max=4,
                            dtype="f32")
    x = synth.request_inputs(1, 1, 1, 4, 1, 64, 200, 16, dtype="f32")
    eng = _run_requests("tiny", geom, zp.ScoreParams(), [x], 16, [0])
    r = eng.reqs[0]
    assert r.n == 48 + 8 and len(r.table) == 4 and eng.compressions == 1
    assert eng.alloc.num_free == 20 - 4


@pytest.mark.timeout(600)
def test_qwen_shape_prefill_compress_then_decode_sampled():
    """Single layer, 32 query / 8 kv heads, d 128, bf16, b 256, N_max 8: 64
    requests with 4096-token prompts compress right after the prompt
    (4096 -> 1792 per kv-head) and then decode 128 steps; four requests are
    checked against the oracle in full."""
    announce("e2e qwen-shape 64x4096")
    B, n0, T = 64, 4096, 128
    geom = zp.CacheGeometry(num_layers=1, num_blocks=B * 16 + 8, block_size=256,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, window=16,
                            max_slots=B, n_max=8, dtype="bf16")
    inputs = []
    for r in range(B):
        inputs.append(synth.request_inputs(2, 2 + 1000 * r, 1, 32, 8, 128, n0, T, dtype="bf16",
                                           prompt_q_last=16))
        if r % 16 == 15:
            announce(f"generated {r + 1}/{B} requests")
    eng = _run_requests("qwen64", geom, zp.ScoreParams(), inputs, T, [0, 17, 42, 63])
    for r in eng.reqs.values():
        assert r.n == 1792 + T and len(r.table) == 8 and not r.first
    assert eng.alloc.num_free == geom.num_blocks - 8 * B
