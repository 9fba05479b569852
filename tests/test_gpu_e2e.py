"""End-to-end GPU parity: decode steps, the compression trigger, scoring,
selection and compaction driven by the engine, against the oracle's logical
simulation of the same requests (Zipage, arXiv 2603.08743, Sec. 4.1-4.5,
App. C).

Bars: decode outputs within 1e-5 (fp32) / 2e-2 (bf16) of max |ref| per
(step, head); kept sets equal to the oracle's outside the tie zone
|S_ref - s_k| <= 1e-6 |s_k| (inside it only the count must match, see
keptsets.py); resident K/V bit-exact. Where a GPU kept set differs from the
oracle's inside the zone, it is one of the equally valid top-k sets, and the
oracle's simulation continues from it, so decode outputs and resident K/V of
that request stay compared after the compression.
"""
import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import synth, zp
from compressed_paged_kv_gqa_amd.engine import DecodeEngine
from oracle import zipage as Z

from gpu_cases import announce, tol_for
from keptsets import check_kept

pytestmark = pytest.mark.gpu


def _oracle_params(sp):
    return Z.ScoreParams(alpha=sp.alpha, lam=sp.lam, tau=sp.tau, p=sp.p,
                         pool_kernel=sp.pool_kernel, use_global=sp.use_global,
                         use_pool=sp.use_pool, pool_first_only=sp.pool_first_only,
                         use_redundancy=sp.use_redundancy)


def _prefill_and_check(cfg, eng, geom, inputs, prompt_q_full, sample, rows_per_req=12):
    """Registers every request and runs its whole prompt through the engine's
    prefill (one ragged batch per layer); checks sampled output rows against
    the oracle's causal prefill."""
    L, h_q, h_kv, d = geom.num_layers, geom.num_q_heads, geom.num_kv_heads, geom.head_dim
    dt = geom.torch_dtype()
    lens = [x.prompt_k.shape[2] for x in inputs]
    for r, n0 in enumerate(lens):
        eng.add_request(r, n0)
    # [L][T][heads][d], requests concatenated along T
    q = torch.from_numpy(np.concatenate([qf.transpose(0, 2, 1, 3) for qf in prompt_q_full], 1))
    k = torch.from_numpy(np.concatenate([x.prompt_k.transpose(0, 2, 1, 3) for x in inputs], 1))
    v = torch.from_numpy(np.concatenate([x.prompt_v.transpose(0, 2, 1, 3) for x in inputs], 1))
    q, k, v = (t.to(dt).cuda().contiguous() for t in (q, k, v))
    out = torch.empty_like(q)
    eng.prefill(list(range(len(inputs))), lens, q, k, v, out)
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(eng.prefill_ws) == 0
    out_h = out.float().cpu().numpy()
    cu = np.concatenate([[0], np.cumsum(lens)])
    tol = tol_for(geom.dtype)
    rng = np.random.default_rng(7)
    worst = 0.0
    for r in sample:
        x = inputs[r]
        rows = sorted(set([0, lens[r] - 1] + rng.integers(0, lens[r], rows_per_req).tolist()))
        for l in range(L):
            O, _ = Z.prefill_attention(prompt_q_full[r][l].transpose(1, 0, 2), x.prompt_k[l],
                                       x.prompt_v[l], 0, rows=rows)
            for a, i in enumerate(rows):
                for j in range(h_q):
                    err = np.abs(out_h[l, cu[r] + i, j] - O[a, j]).max() / np.abs(O[a, j]).max()
                    worst = max(worst, err)
                    assert err <= tol, (cfg, "prefill", r, l, i, j, err)
    print(f"{cfg}: worst prefill error {worst:.3e}", flush=True)


def _run_requests(cfg, geom, sp, inputs, n_steps, sample, layer_stride=1, async_compress=True,
                  wait_each_step=True, prefix_len=0, check_prefix=None, prompt_q_full=None):
    """Drives all requests on the GPU and compares `sample` of them with the
    oracle simulation. `inputs[r]` is a synth.RequestInputs. Every request
    consumes its own next decode input: with wait_each_step=False a
    compressing request sits out decode steps until its side-stream event has
    fired (Sec. 4.5), so requests drift apart in step count. With
    prefix_len > 0 the first prefix_len prompt tokens of every request are
    identical and their blocks are shared (Sec. 4.4). With prompt_q_full
    (per request [L][h_q][n0][d]) the prompts go through zp_paged_prefill
    instead of being written directly; their outputs are checked on sampled
    rows and the window queries are the prompts' last w queries."""
    B = len(inputs)
    L, h_q, h_kv, d = geom.num_layers, geom.num_q_heads, geom.num_kv_heads, geom.head_dim
    b, w = geom.block_size, geom.window
    dt = geom.torch_dtype()
    cap = max(-(-(x.prompt_k.shape[2] + n_steps) // b) for x in inputs) + 1
    eng = DecodeEngine(geom, sp, B, cap, layer_stride=layer_stride,
                       async_compress=async_compress, record=True)
    prefix_table = None
    if prompt_q_full is not None:
        _prefill_and_check(cfg, eng, geom, inputs, prompt_q_full, sample)
    for r, x in enumerate(inputs if prompt_q_full is None else []):
        n0 = x.prompt_k.shape[2]
        share = prefix_table if (prefix_len and r > 0) else None
        table = eng.add_request(r, n0, prefix_table=share)
        if prefix_len and r == 0:
            prefix_table = table[:prefix_len // b]
        start = prefix_len if share else 0
        for l in range(L):
            eng.write_tokens(r, l, start, torch.from_numpy(x.prompt_k[l][:, start:]).to(dt).cuda(),
                             torch.from_numpy(x.prompt_v[l][:, start:]).to(dt).cuda())
            if x.prompt_q is not None:
                qw = np.zeros((h_kv, h_q // h_kv, w, d), np.float32)
                m = x.prompt_q.shape[2]
                for pos in range(n0 - m, n0):
                    row = Z.window_row(pos, b, w)
                    if row >= 0:
                        qw[:, :, row] = x.prompt_q[l, :, pos - (n0 - m)].reshape(h_kv, h_q // h_kv, d)
                eng.write_window_queries(r, l, torch.from_numpy(qw).to(dt).cuda())
    if prefix_table is not None:
        assert all(eng.alloc.refcount(p) == B for p in prefix_table)
        prefix_k = eng.cache.k[:, prefix_table].clone()
    eng.compress_due_now()
    if wait_each_step:
        eng.wait_compressions()
    # per-request decode inputs [B][T][L][...] on the device
    q_req = torch.from_numpy(np.stack([x.steps_q for x in inputs])).to(dt).cuda()
    k_req = torch.from_numpy(np.stack([x.steps_k for x in inputs])).to(dt).cuda()
    v_req = torch.from_numpy(np.stack([x.steps_v for x in inputs])).to(dt).cuda()
    outs = torch.zeros((B, n_steps, L, h_q, d), dtype=dt, device="cuda")
    out_step = torch.empty((L, B, h_q, d), dtype=dt, device="cuda")
    cnt = np.zeros(B, np.int64)
    rows = torch.arange(B, device="cuda")
    guard = 0
    while cnt.min() < n_steps:
        guard += 1
        assert guard < 50 * n_steps, "requests stopped making progress"
        for r in range(B):
            eng.reqs[r].done = cnt[r] >= n_steps
        act = eng.prepare_step()
        if not act:
            eng.poll(wait=True)
            continue
        idx = torch.from_numpy(np.minimum(cnt, n_steps - 1)).cuda()
        q_s = q_req[rows, idx].transpose(0, 1).contiguous()      # [L][B][h_q][d]
        k_s = k_req[rows, idx].transpose(0, 1).contiguous()
        v_s = v_req[rows, idx].transpose(0, 1).contiguous()
        for l in range(L):
            eng.decode_layer(l, q_s[l], k_s[l], v_s[l], out_step[l])
        a = torch.tensor(act, device="cuda")
        outs[a, torch.from_numpy(cnt[act]).cuda()] = out_step[:, a].transpose(0, 1)
        eng.finish_step(act)
        cnt[act] += 1
        if wait_each_step:
            eng.wait_compressions()
    eng.wait_compressions()
    torch.cuda.synchronize()
    assert zp.zp_workspace_errors(eng.dec_ws) == 0
    if check_prefix is not None:
        check_prefix(eng, prefix_table, prefix_k)
    outs_h = outs.float().cpu().numpy()
    op = _oracle_params(sp)
    tol = tol_for(geom.dtype)
    worst_out = 0.0
    for r in sample:
        x = inputs[r]
        announce(f"{cfg}: oracle for request {r} (prompt {x.prompt_k.shape[2]})")
        gpu_events = [(sids.index(r), first, kept.cpu().numpy())
                      for (sids, first, sc, kept) in eng.log if r in sids]

        def choose(e, l, h, S, keep, r=r, gpu_events=gpu_events):
            # the GPU's kept set, accepted only if it is a valid top-k of the
            # oracle's scores under the 1e-6 tie zone
            assert e < len(gpu_events), (cfg, r, "oracle compresses more often than the GPU")
            i, _first, kept_h = gpu_events[e]
            got = np.sort(kept_h[l, i, h])
            c = check_kept(got, S, keep)
            if not c.same:
                print(f"{cfg}: request {r} event {e} layer {l} head {h}: {c.describe()}",
                      flush=True)
            assert c.ok, (cfg, r, e, l, h, c.describe())
            return got

        res = Z.simulate_request(x.prompt_k, x.prompt_v, x.prompt_q, x.steps_q, x.steps_k,
                                 x.steps_v, b, w, geom.n_max, op, choose=choose)
        assert len(gpu_events) == len(res["events"]), (len(gpu_events), len(res["events"]))
        for (i, first, _k), ev in zip(gpu_events, res["events"]):
            assert bool(first[i]) == ev["first"]
        for s in range(n_steps):
            for l in range(L):
                for j in range(h_q):
                    ref = res["outputs"][s, l, j]
                    err = np.abs(outs_h[r, s, l, j] - ref).max() / np.abs(ref).max()
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


@pytest.mark.timeout(900)
def test_shared_prefix_copy_on_compress_sampled():
    """128 requests share one 1024-token prefix (4 blocks, refcount 128) and
    have unique 512-token suffixes; 2048 decode steps, compressions every 256
    steps from step 512. The first compression of each request writes its
    kept tokens to 4 fresh blocks (copy-on-compress) and drops one reference
    of each shared block; the shared blocks' contents never change. Requests
    rejoin decode as their compressions finish (no waiting)."""
    announce("e2e shared prefix 128 x (1024 + 512), 2048 steps")
    B, pre, suf, T = 128, 1024, 512, 2048
    geom = zp.CacheGeometry(num_layers=1, num_blocks=4 + B * 8 + B * 4 + 8, block_size=256,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, window=16,
                            max_slots=B, n_max=8, dtype="bf16")
    base = synth.request_inputs(4, 4, 1, 32, 8, 128, pre, 0, dtype="bf16")
    inputs = []
    for r in range(B):
        x = synth.request_inputs(4, 4000 + r, 1, 32, 8, 128, suf, T, dtype="bf16")
        x.prompt_k = np.concatenate([base.prompt_k, x.prompt_k], axis=2)
        x.prompt_v = np.concatenate([base.prompt_v, x.prompt_v], axis=2)
        inputs.append(x)
        if r % 32 == 31:
            announce(f"generated {r + 1}/{B} requests")

    def check_prefix(eng, prefix_table, prefix_k):
        for p in prefix_table:
            assert eng.alloc.refcount(p) == 0          # every request let go
        # untouched by any compaction (no block was allocated after the first
        # compression, so the freed prefix blocks still hold the prefix)
        assert torch.equal(eng.cache.k[:, prefix_table], prefix_k)
        for r in eng.reqs.values():
            assert not set(r.table) & set(prefix_table) and len(r.table) == 8

    eng = _run_requests("prefix", geom, zp.ScoreParams(), inputs, T, [0, 77, 127],
                        wait_each_step=False, prefix_len=pre, check_prefix=check_prefix)
    assert eng.compressions == B * 7


@pytest.mark.timeout(900)
def test_ragged_long_context_sampled():
    """64 requests with prompts log-uniform in [2048, 32768] tokens, 256 decode
    steps: prompts ending on a block boundary compress at once (up to
    32768 -> 1792 tokens), the others when decode fills their last block,
    while the rest keep decoding (no waiting)."""
    announce("e2e ragged 64 x [2048, 32768], 256 steps")
    B, T = 64, 256
    lens = synth.log_uniform_lengths(5, 5, B, 2048, 32768)
    lens[:4] = [2048, 8192, 32768, 4096]          # some prompts end on a block boundary
    nblocks = sum(-(-(int(n) + T) // 256) for n in lens)
    geom = zp.CacheGeometry(num_layers=1, num_blocks=nblocks + 16, block_size=256,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, window=16,
                            max_slots=B, n_max=8, dtype="bf16")
    inputs = []
    for r in range(B):
        inputs.append(synth.request_inputs(5, 5000 + r, 1, 32, 8, 128, int(lens[r]), T,
                                           dtype="bf16", prompt_q_last=16))
        if r % 16 == 15:
            announce(f"generated {r + 1}/{B} requests")
    order = np.argsort(lens)
    sample = [0, 2, int(order[0]), int(order[B // 2])]
    eng = _run_requests("ragged", geom, zp.ScoreParams(), inputs, T, sample,
                        wait_each_step=False)
    for r in eng.reqs.values():
        assert len(r.table) <= 8


@pytest.mark.timeout(600)
def test_qwen_shape_real_prefill_then_compress_and_decode_sampled():
    """The 4096-token prompts of 16 requests go through zp_paged_prefill
    (bf16 MFMA), which also captures the window queries and their
    log-sum-exp; the compression that the prompt triggers then scores with
    that log-sum-exp in one pass over the keys; 64 decode steps follow. Two
    requests are checked against the oracle in full (prefill rows sampled)."""
    announce("e2e qwen-shape prefill 16x4096")
    B, n0, T = 16, 4096, 64
    geom = zp.CacheGeometry(num_layers=1, num_blocks=B * 16 + 8, block_size=256,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, window=16,
                            max_slots=B, n_max=8, dtype="bf16")
    inputs, qfull = [], []
    for r in range(B):
        x = synth.request_inputs(6, 6000 + r, 1, 32, 8, 128, n0, T, dtype="bf16")
        qf = synth.cast(synth.rng(6, 6000 + r, 0, "prompt_q").standard_normal((1, 32, n0, 128)),
                        "bf16")
        x.prompt_q = qf[:, :, n0 - 16:]          # the window: the prompt's last 16 queries
        inputs.append(x)
        qfull.append(qf)
    eng = _run_requests("qwen16-prefill", geom, zp.ScoreParams(), inputs, T, [0, 11],
                        prompt_q_full=qfull)
    assert eng.compressions == B
    for r in eng.reqs.values():
        assert r.n == 1792 + T and len(r.table) == 8 and not r.first
