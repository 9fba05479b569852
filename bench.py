#!/usr/bin/env python3
"""Decode throughput of the compressed paged KV hot path on one MI355X.

Workload (N=1): a 36-layer Qwen3-8B-shaped attention stack (32 query / 8 kv
heads, head_dim 128, bf16), 256 concurrent sequences, block size 256,
N_max = 8 blocks (k = 1792 tokens kept per compression), window 16. The timed
region is the steady state of long decoding: every sequence has been
compressed before and holds 1793..2048 resident tokens (random phases), and a
compression fires each time a sequence fills its 8th block (~1 sequence per
step), running asynchronously on a side stream (score + select + compact,
layer stride 8). Inputs (K/V pages, per-step q/k/v) are resident in HBM before
timing starts; values are seeded synthetic N(0, 1).

One step = one decode token for every active sequence through all 36 layers
(zp_paged_decode per layer) plus the compressions that become due.

Prints one JSON line (metric, value = decode tokens/s, roofline of the decode
kernel measured with HIP events around every launch of every 10th timed step,
cpu_baseline = the float64 oracle on the host cores on a bounded sample of the
same workload). The line also carries the compression and prefill kernels
timed in isolation, `whole_run`: the same workload from seeded prompts through
prefill, decode and the compressions as they fall due (output tokens per
second of the whole run),
and `serve`: a synthetic request stream served to completion by the library's
scheduler (hybrid and constrained), output tokens per second.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                  [--no-compress-kernels] [--no-whole-run] [--no-serve]
  python bench.py --serve | --whole-run | --compress-kernels | --prefill-kernels   # one part
  python bench.py --copy-calibration     # plain device copy of known size
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "qwen3-8b-attn-36L-256seq-b256-nmax8-steady"
L, B, HQ, HKV, D, BS, NMAX, W = 36, 256, 32, 8, 128, 256, 8, 16
ELEM = 2  # bf16
HBM_PEAK_GBS = 8000.0
SEED = 3
EVENT_EVERY = 10  # timed steps whose decode launches are bracketed by HIP events


def decode_unit_bytes(n):
    """Algorithmic HBM bytes of one (sequence, layer) decode with n resident
    tokens after the append: K and V of the n tokens read once (n-1 from the
    pages, the new one from k_new/v_new), the new K/V written to its page,
    q read and o written."""
    return (2 * n * HKV * D + 2 * HKV * D + 2 * HQ * D) * ELEM


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-steps", type=int, default=16)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--sync-compress", action="store_true",
                    help="run compressions on the decode stream (ablation)")
    ap.add_argument("--compress-kernels", action="store_true",
                    help="only the isolated compression-kernel measurement (one JSON line)")
    ap.add_argument("--no-compress-kernels", action="store_true",
                    help="skip the isolated compression-kernel measurement")
    ap.add_argument("--prefill-kernels", action="store_true",
                    help="only the isolated prefill measurement (one JSON line)")
    ap.add_argument("--serve", action="store_true",
                    help="only the scheduled serving run of a synthetic request stream "
                         "(one JSON line)")
    ap.add_argument("--serve-requests", type=int, default=256)
    ap.add_argument("--serve-mem-gib", type=float, default=24.0,
                    help="HBM given to K/V, F and the query cache (sets M and N_total)")
    ap.add_argument("--serve-policies", default="hybrid,constrained")
    ap.add_argument("--no-serve", action="store_true",
                    help="skip the scheduled serving run in the default line")
    ap.add_argument("--whole-run", action="store_true",
                    help="only the whole run from the prompts (one JSON line)")
    ap.add_argument("--whole-run-steps", type=int, default=2048)
    ap.add_argument("--no-whole-run", action="store_true",
                    help="skip the whole run in the default line")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of 4 GiB, for scaling rocprofv3's
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        t.append(e0.elapsed_time(e1))
    ms = float(np.median(t))
    print(json.dumps({"copy_bytes": n, "ms": ms, "GBps_rw": 2 * n / ms / 1e6}))


def fill_cache(cache, seed):
    """Seeded N(0,1) bf16 K/V for every layer (device generator), small
    positive history in F and random window queries."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for l in range(cache.geom.num_layers):
        cache.k[l].normal_(generator=g)
        cache.v[l].normal_(generator=g)
        if l % 12 == 11:
            torch.cuda.synchronize()
            log(f"filled {l + 1}/{cache.geom.num_layers} layers")
    cache.qwin.normal_(generator=g)
    cache.gscore.uniform_(0.0, 1e-3, generator=g)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_workload(phases, sync_compress=False, record=False):
    """The timed workload: engine, filled caches and per-step inputs
    (q/k/v: 4 variants [4][L][B][...] cycled over the steps; out [L][B][...])."""
    import torch
    from compressed_paged_kv_gqa_amd import zp
    from compressed_paged_kv_gqa_amd.engine import DecodeEngine
    geom = zp.CacheGeometry(num_layers=L, num_blocks=B * NMAX + 16, block_size=BS,
                            num_kv_heads=HKV, num_q_heads=HQ, head_dim=D, window=W,
                            max_slots=B, n_max=NMAX, dtype="bf16")
    eng = DecodeEngine(geom, zp.ScoreParams(), B, NMAX, layer_stride=8,
                       async_compress=not sync_compress, record=record)
    log("filling the K/V cache")
    fill_cache(eng.cache, SEED)
    for s in range(B):
        eng.add_request(s, (NMAX - 1) * BS + int(phases[s]))
        eng.reqs[s].first = False
    g = torch.Generator(device="cuda")
    g.manual_seed(SEED + 1)
    nvar = 4
    q = torch.randn((nvar, L, B, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((nvar, L, B, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((nvar, L, B, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((L, B, HQ, D), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log("setup done")
    return eng, (q, k, v, out)


def run_gpu(args, phases):
    import torch
    eng, (q, k, v, out) = build_workload(phases, args.sync_compress)
    nvar = q.shape[0]
    for i in range(args.warmup):
        eng.step(q[i % nvar], k[i % nvar], v[i % nvar], out)
    torch.cuda.synchronize()
    eng.side.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    K = args.steps
    # Every launch of every EVENT_EVERY-th timed step is bracketed by a pair of
    # HIP events on the decode stream. An event between two launches makes the
    # first drain completely before the second starts; bracketing all 36
    # launches of every step measured 2.5% slower steps (11.74 vs 11.43 ms).
    sampled = [i for i in range(K) if i % EVENT_EVERY == 0]
    ev = {i: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(L)] for i in sampled}
    step_bytes = {}
    tokens0 = eng.decoded_tokens
    comp0, lse0 = eng.compressions, eng.compressions_lse
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        eng.layer_events = ev.get(i)
        act = eng.step(q[i % nvar], k[i % nvar], v[i % nvar], out)
        if i in ev:
            lens = eng.lens_np[act]
            step_bytes[i] = sum(decode_unit_bytes(int(n)) for n in lens)
    torch.cuda.synchronize()
    eng.side.synchronize()
    t1 = time.perf_counter()
    eng.layer_events = None
    elapsed = t1 - t0
    tokens = eng.decoded_tokens - tokens0
    durs = np.array([[a.elapsed_time(b) for (a, b) in ev[i]] for i in sampled])  # ms [steps][L]
    launch_ms = float(durs.mean())
    bytes_per_launch = float(np.mean([step_bytes[i] for i in sampled]))  # same for every layer of a step
    achieved = bytes_per_launch / (launch_ms * 1e-3) / 1e9
    from compressed_paged_kv_gqa_amd import zp
    errs = zp.zp_workspace_errors(eng.dec_ws)
    assert errs == 0, f"device errors {errs}"
    return dict(elapsed=elapsed, tokens=tokens, steps=K, launch_ms=launch_ms,
                bytes_per_launch=bytes_per_launch, achieved_gbs=achieved,
                compressions=eng.compressions - comp0,
                compressions_lse=eng.compressions_lse - lse0, decode_ms_per_step=float(durs.sum(1).mean()))


# --------------------------------------------------------------------------
# Whole run of the 256-sequence workload from its prompts
# --------------------------------------------------------------------------

def whole_run_bench(steps, seed=SEED):
    """The 36-layer, 256-sequence workload from the start: seeded prompt
    lengths U[64, 512), every prompt through zp_paged_prefill (one output
    token each), then `steps` decode steps in which each sequence compresses
    when a block fill leaves it at N_max blocks (asynchronously, layer stride
    8). tokens/s = output tokens / wall time from the first prefill to the
    last decode step (Zipage's TPS, one GPU). Prompt and step q/k/v are
    seeded device tensors; one set of prompt rows serves every layer."""
    import torch
    from compressed_paged_kv_gqa_amd import synth, zp
    from compressed_paged_kv_gqa_amd.engine import DecodeEngine
    plen = synth.rng(seed, 3, 0, "prompt_lengths").integers(64, 512, B)
    geom = zp.CacheGeometry(num_layers=L, num_blocks=B * (NMAX + 1) + 16, block_size=BS,
                            num_kv_heads=HKV, num_q_heads=HQ, head_dim=D, window=W,
                            max_slots=B, n_max=NMAX, dtype="bf16")
    eng = DecodeEngine(geom, zp.ScoreParams(), B, NMAX, layer_stride=8)
    for s in range(B):
        eng.add_request(s, int(plen[s]))
    T = int(plen.sum())
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 11)
    pq = torch.randn((T, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    pk = torch.randn((T, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    pv = torch.randn((T, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    pout = torch.empty((T, HQ, D), dtype=torch.bfloat16, device="cuda")
    lay = lambda x: x.unsqueeze(0).expand(L, *x.shape)   # same rows for every layer
    nvar = 4
    q = torch.randn((nvar, L, B, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((nvar, L, B, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((nvar, L, B, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((L, B, HQ, D), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    log(f"whole run: {B} prompts ({T} tokens), then {steps} decode steps")
    t0 = time.perf_counter()
    eng.prefill(list(range(B)), plen, lay(pq), lay(pk), lay(pv), lay(pout))
    for i in range(steps):
        eng.step(q[i % nvar], k[i % nvar], v[i % nvar], out)
        if (i + 1) % 512 == 0:
            log(f"whole run: {i + 1} steps, {eng.compressions} compressions")
    torch.cuda.synchronize()
    eng.side.synchronize()
    elapsed = time.perf_counter() - t0
    errs = zp.zp_workspace_errors(eng.dec_ws) | zp.zp_workspace_errors(eng.prefill_ws)
    assert errs == 0, f"device errors {errs}"
    tokens = B + eng.decoded_tokens
    return {"workload": f"{B} sequences x {L} layers from prompts U[64,512) through prefill, "
                        f"then {steps} decode steps with compression at N_max={NMAX}",
            "tokens_per_s": round(tokens / elapsed, 1), "seconds": round(elapsed, 2),
            "output_tokens": tokens, "prompt_tokens": T, "compressions": eng.compressions,
            "final_resident_tokens": [int(min(r.n for r in eng.reqs.values())),
                                      int(max(r.n for r in eng.reqs.values()))],
            "decode_steps_of_16384": steps,
            "cut": (f"each sequence decodes up to 16384 tokens in the full workload; this run "
                    f"stops after {steps} steps" if steps < 16384 else "full length")}


# --------------------------------------------------------------------------
# Compression kernels in isolation (score, select + compact)
# --------------------------------------------------------------------------

MFMA_PEAK_TFS = 2500.0   # dense bf16 MFMA, MI355X

# Burst of the 4096-token-prompt workload: 64 requests whose prompts fill 16
# blocks compress at once (first compression: pooling on, no F history).
BURST_REQ, BURST_BLOCKS = 64, 16


def score_unit_cost(n, redundancy, first):
    """Algorithmic (flops, bytes) of scoring one (layer, kv-head, request)
    with n = N*b resident tokens: window logits g*w x n x d and the key
    cosines (within each block for lightning: N*b*b*d; over the sequence for
    flash: n*n*d) as multiply-adds; K read once, the window queries, F read
    unless it is the first compression, scores and the updated history
    written."""
    g = HQ // HKV
    gram = (n // BS) * BS * BS if redundancy == "lightning" else n * n
    flops = 2 * g * W * n * D + 2 * gram * D
    byts = n * D * ELEM + g * W * D * ELEM + (0 if first else 4 * n) + 8 * n
    return flops, byts


def select_unit_bytes(n, keep):
    """Algorithmic bytes of selecting and compacting one (layer, kv-head,
    request): the n scores read once, K and V of the keep kept tokens read
    and written, their global scores read (updated history) and written."""
    return 4 * n + 4 * keep * D * ELEM + 8 * keep


def _time_calls(fn, iters, stream, warm_ms=200.0):
    """HIP-event time per call of fn (ms) over `iters` calls, after untimed
    calls that fill at least warm_ms of GPU time: from idle the clocks take
    ~100 ms of steady work to settle, and calls timed before that ran up to
    25% slower (lightning scoring: 0.311 -> 0.244 ms over its first 120
    calls, then 0.240-0.245)."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    spent, k = 0.0, 1
    while spent < warm_ms:  # back-to-back batches, doubled while short
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1)
        spent += t
        if t < 25.0:
            k *= 2
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def compress_kernel_bench(iters=20):
    """HIP-event time per call of zp_score_tokens (lightning and flash) and
    zp_select_compact at the burst shape, on their own stream with nothing
    else running, against the MFMA and HBM rooflines. The window rows carry
    their log-sum-exp (as after zp_paged_prefill), so scoring reads each key
    once; score_lightning_stats times the path that first gathers the softmax
    statistics itself."""
    import torch
    from compressed_paged_kv_gqa_amd import zp
    R, NB = BURST_REQ, BURST_BLOCKS
    n = NB * BS
    keep = (NMAX - 1) * BS
    geom = zp.CacheGeometry(num_layers=1, num_blocks=R * NB + 8, block_size=BS,
                            num_kv_heads=HKV, num_q_heads=HQ, head_dim=D, window=W,
                            max_slots=R, n_max=NMAX, dtype="bf16")
    cache = zp.PagedKVCache(geom, with_window_lse=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(SEED + 7)
    cache.k.normal_(generator=g)
    cache.v.normal_(generator=g)
    cache.qwin.normal_(generator=g)
    cache.gscore.uniform_(0.0, 1e-3, generator=g)
    cache.qwin_lse.fill_(float(np.log(n)) + 1.0)
    perm = torch.randperm(R * NB, generator=g, device="cuda").to(torch.int32)
    tables = perm.view(R, NB).contiguous()
    dst = tables[:, :NMAX - 1].contiguous()
    nblk = torch.full((R,), NB, dtype=torch.int32, device="cuda")
    qslot = torch.arange(R, dtype=torch.int32, device="cuda")
    first = torch.ones(R, dtype=torch.uint8, device="cuda")
    lse_ok = torch.ones(R, dtype=torch.uint8, device="cuda")
    scores = torch.empty((1, R, HKV, n), dtype=torch.float32, device="cuda")
    f_new = torch.empty_like(scores)
    sws = zp.new_workspace(zp.zp_score_workspace_size(geom, 1, R, NB))
    cws = zp.new_workspace(zp.zp_select_workspace_size(geom, 1, R, keep))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())  # the inputs above are filled on that stream
    units = R * HKV
    out = {"workload": f"{R} requests x {n} tokens ({NB} full blocks) compressing at once, "
                       f"1 layer, bf16, first compression, keep {keep}",
           "units_per_call": units}
    with torch.cuda.stream(stream):
        for name, red, lse in (("score_lightning", "lightning", lse_ok),
                               ("score_lightning_stats", "lightning", None),
                               ("score_flash", "flash", lse_ok)):
            sp = zp.ScoreParams(redundancy=red)
            # all window rows carry their log-sum-exp: the engine then passes
            # window_lse_all as well, and so does this leg
            ms = _time_calls(lambda: zp.zp_score_tokens(cache, sp, 0, 1, tables, nblk, NB, qslot,
                                                        first, scores, f_new, sws, stream=stream,
                                                        window_lse_valid=lse,
                                                        window_lse_all=lse is not None),
                             iters if red == "lightning" else max(3, iters // 4), stream)
            fl, by = score_unit_cost(n, red, True)
            tf = units * fl / (ms * 1e-3) / 1e12
            gb = units * by / (ms * 1e-3) / 1e9
            ideal = max(units * fl / (MFMA_PEAK_TFS * 1e12), units * by / (HBM_PEAK_GBS * 1e9))
            out[name] = {
                "ms_per_call": round(ms, 4), "achieved_tflops": round(tf, 1),
                "mfma_peak_tflops": MFMA_PEAK_TFS, "achieved_gbs": round(gb, 1),
                "bound": "mfma" if units * fl / MFMA_PEAK_TFS / 1e12 > units * by / HBM_PEAK_GBS / 1e9
                else "hbm",
                "frac_of_roofline": round(ideal / (ms * 1e-3), 4),
                "flops_per_unit": fl, "bytes_per_unit": by}
        # scores of the lightning variant feed the selection
        sp = zp.ScoreParams()
        zp.zp_score_tokens(cache, sp, 0, 1, tables, nblk, NB, qslot, first, scores, f_new, sws,
                           stream=stream, window_lse_valid=lse_ok)
        ms = _time_calls(lambda: zp.zp_select_compact(cache, 0, 1, scores, tables, nblk, NB, dst,
                                                      keep, None, cws, stream=stream,
                                                      f_new=f_new), iters, stream)
        by = select_unit_bytes(n, keep)
        gb = units * by / (ms * 1e-3) / 1e9
        out["select_compact"] = {"ms_per_call": round(ms, 4), "achieved_gbs": round(gb, 1),
                                 "bound": "hbm", "frac_of_roofline": round(gb / HBM_PEAK_GBS, 4),
                                 "bytes_per_unit": by}
    stream.synchronize()
    errs = zp.zp_workspace_errors(sws) | zp.zp_workspace_errors(cws)
    assert errs == 0, f"device errors {errs}"
    return out


def prefill_flops(lens):
    """Algorithmic flops of causal prefill: a query at position p multiplies
    q.k and p.v over p + 1 keys in every query head (2 flops per
    multiply-add, two products)."""
    return sum(4 * HQ * D * t * (t + 1) // 2 for t in lens)


def prefill_kernel_bench(iters=5):
    """HIP-event time per call of zp_paged_prefill for 64 prompts of 4096
    tokens (one layer, bf16), the prompt pass of the 4096-token workload,
    against the bf16 MFMA roofline."""
    import torch
    from compressed_paged_kv_gqa_amd import zp
    R, T = BURST_REQ, BURST_BLOCKS * BS
    geom = zp.CacheGeometry(num_layers=1, num_blocks=R * BURST_BLOCKS + 8, block_size=BS,
                            num_kv_heads=HKV, num_q_heads=HQ, head_dim=D, window=W, max_slots=R,
                            n_max=NMAX, dtype="bf16")
    cache = zp.PagedKVCache(geom, with_global=False, with_window_lse=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(SEED + 9)
    q = torch.randn((R * T, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((R * T, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((R * T, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty_like(q)
    lse = torch.empty((R * T, HQ), dtype=torch.float32, device="cuda")
    tables = torch.randperm(R * BURST_BLOCKS, generator=g, device="cuda").to(torch.int32)
    tables = tables.view(R, BURST_BLOCKS).contiguous()
    cu = torch.arange(0, (R + 1) * T, T, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(R, dtype=torch.int32, device="cuda")
    qslot = torch.arange(R, dtype=torch.int32, device="cuda")
    ws = zp.new_workspace(zp.zp_prefill_workspace_size(geom, R))
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())  # the inputs above are filled on that stream
    with torch.cuda.stream(stream):
        ms = _time_calls(lambda: zp.zp_paged_prefill(cache, 0, q, k, v, cu, ctx, T, tables, qslot,
                                                     out, lse, ws, stream=stream), iters, stream)
    stream.synchronize()
    assert zp.zp_workspace_errors(ws) == 0
    fl = prefill_flops([T] * R)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": f"{R} prompts x {T} tokens, 1 layer, bf16, causal, K/V appended to "
                        f"block {BS} pages, window queries and LSE captured",
            "ms_per_call": round(ms, 3), "achieved_tflops": round(tf, 1),
            "mfma_peak_tflops": MFMA_PEAK_TFS, "bound": "mfma",
            "frac_of_roofline": round(tf / MFMA_PEAK_TFS, 4), "flops_per_call": fl}


# --------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# --------------------------------------------------------------------------

def serve_stream(n_req, seed):
    """Synthetic offline request stream standing in for a reasoning benchmark:
    short prompts (uniform 64..1024 tokens) and long, skewed outputs
    (log-uniform 256..4096 tokens), all submitted at once."""
    from compressed_paged_kv_gqa_amd import synth
    g = synth.rng(seed, 9, 0, "serve_stream")
    prompts = g.integers(64, 1025, n_req)
    outs = np.exp(g.uniform(np.log(256), np.log(4096), n_req)).astype(np.int64)
    return [(i, int(p), int(m)) for i, (p, m) in enumerate(zip(prompts, outs))]


def serve_bench(n_req, mem_gib, policies):
    """Every request of the stream through ServingEngine (zp_sched driving
    prefill, decode and asynchronous compression) to completion, once per
    policy. TPS = output tokens / wall time of the whole run."""
    import torch
    from compressed_paged_kv_gqa_amd import engine as E
    from compressed_paged_kv_gqa_amd import zp
    blk = L * 2 * HKV * BS * D * ELEM                 # K and V of one block, all layers
    m_f = L * HKV * BS * 4                            # global score F of one block
    m_q = L * HQ * W * (D * ELEM + 4)                 # query cache + its LSE per slot
    M, NT = zp.zp_capacity(int(mem_gib * (1 << 30)), blk, m_f, m_q, NMAX)
    stream = serve_stream(n_req, SEED)
    cap = 16
    maxpf = 16384
    res = {"workload": f"{n_req} requests (prompts U[64,1024], outputs log-U[256,4096]) "
                       f"through {L} Qwen3-8B-shaped attention layers, bf16, b={BS}, "
                       f"N_max={NMAX}, w={W}",
           "mem_gib": mem_gib, "M": M, "num_blocks": NT,
           "output_tokens": sum(m for _i, _p, m in stream), "policies": {}}
    for pol in policies:
        geom = zp.CacheGeometry(num_layers=L, num_blocks=NT, block_size=BS, num_kv_heads=HKV,
                                num_q_heads=HQ, head_dim=D, window=W, max_slots=M, n_max=NMAX,
                                dtype="bf16")
        eng = E.ServingEngine(geom, zp.ScoreParams(), max_running=min(n_req, 1024),
                              table_cap=cap, max_prefill_tokens=maxpf, policy=pol,
                              layer_stride=8, async_compress=True)
        rows = max(maxpf, cap * BS)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(SEED)
        pool = [torch.randn((2 * rows, h, D), generator=gen, device="cuda").to(torch.bfloat16)
                for h in (HQ, HKV, HKV)]
        state = {"t": 0, "T": 0}

        def inputs(kind, st, layer):
            if layer == 0:
                state["T"] = int(st.len.sum()) if kind == zp.ZP_STEP_PREFILL else st.n
                state["t"] += 1
            o = (state["t"] * 7919 + layer * 131) % rows
            T = state["T"]
            return pool[0][o:o + T], pool[1][o:o + T], pool[2][o:o + T]

        for i, p, m in stream:
            eng.add(i, p, m)
        log(f"serve {pol}: M={M} blocks={NT} requests={n_req}")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        kinds = {zp.ZP_STEP_IDLE: 0, zp.ZP_STEP_PREFILL: 0, zp.ZP_STEP_DECODE: 0}
        max_run = 0
        steps = 0
        while eng.unfinished() > 0:
            st = eng.step(inputs)
            kinds[st.kind] += 1
            steps += 1
            if st.kind == zp.ZP_STEP_DECODE:
                max_run = max(max_run, st.n)
            if steps % 500 == 0:
                log(f"  step {steps}: {eng.unfinished()} unfinished")
        eng.poll(wait=True)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        assert eng.device_errors() == 0
        stt = eng.sched.stats()
        res["policies"][pol] = {
            "tps": round(eng.generated / el, 1), "seconds": round(el, 2), "steps": steps,
            "prefill_steps": kinds[zp.ZP_STEP_PREFILL], "decode_steps": kinds[zp.ZP_STEP_DECODE],
            "idle_steps": kinds[zp.ZP_STEP_IDLE],
            "avg_decode_batch": round(stt["decode_tokens"] / max(1, stt["decode_steps"]), 1),
            "max_decode_batch": max_run, "compressions": stt["compressions"],
            "preemptions": stt["preemptions"], "blocked": stt["blocked"],
            "prefill_tokens": stt["prefill_tokens"]}
        log(f"serve {pol}: {res['policies'][pol]}")
        del eng, pool
        torch.cuda.empty_cache()
    return res


def _oracle_worker(job):
    import threadpoolctl
    with threadpoolctl.threadpool_limits(1):
        return _oracle_sequence(*job)


def _oracle_sequence(sid, phase, steps):
    """One sequence of one layer: `steps` decode steps from 1792 + phase
    resident tokens, compressing when the 8th block fills. Returns
    (compute seconds, compressions)."""
    from compressed_paged_kv_gqa_amd import synth
    from oracle import zipage as Z
    n = (NMAX - 1) * BS + int(phase)
    cap = NMAX * BS
    g = synth.rng(SEED, 30, sid, "prompt_k")
    K = np.zeros((HKV, cap, D))
    V = np.zeros((HKV, cap, D))
    K[:, :n] = synth.round_bf16(g.standard_normal((HKV, n, D)).astype(np.float32))
    V[:, :n] = synth.round_bf16(g.standard_normal((HKV, n, D)).astype(np.float32))
    F = np.zeros((HKV, cap))
    F[:, :n] = g.random((HKV, n)) * 1e-3
    qw = synth.round_bf16(g.standard_normal((HKV, HQ // HKV, W, D)).astype(np.float32))
    sq = synth.round_bf16(g.standard_normal((steps, HQ, D)).astype(np.float32))
    sk = synth.round_bf16(g.standard_normal((steps, HKV, D)).astype(np.float32))
    sv = synth.round_bf16(g.standard_normal((steps, HKV, D)).astype(np.float32))
    params = Z.ScoreParams()
    comp = 0
    t0 = time.perf_counter()
    for s in range(steps):
        K[:, n] = sk[s]
        V[:, n] = sv[s]
        n += 1
        Z.decode_attention(sq[s], K[:, :n], V[:, :n])
        if Z.should_compress(n, BS, NMAX):
            keep = (NMAX - 1) * BS
            for h in range(HKV):
                S, F_new = Z.score_tokens(qw[h], K[h, :n], F[h, :n], False, BS, params)
                kept = Z.topk_keep(S, keep)
                K[h, :keep] = K[h, kept]
                V[h, :keep] = V[h, kept]
                F[h, :keep] = F_new[kept]
            n = keep
            comp += 1
    return time.perf_counter() - t0, comp


CPU_SHARE = 16   # host CPUs one GPU's job may keep busy on a shared GPU host


def oracle_procs():
    """Worker processes for the oracle: one per CPU this process may run on
    (its affinity set), at most the host CPU share of one GPU."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return max(1, min(CPU_SHARE, avail)), avail


def cpu_baseline(phases, steps):
    import multiprocessing as mp
    procs, avail = oracle_procs()
    jobs = [(s, int(phases[s]), steps) for s in range(B)]
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(procs) as pool:
        res = pool.map(_oracle_worker, jobs, chunksize=1)
        wall = time.perf_counter() - t0
        log(f"cpu baseline: 36-layer slice done in {wall:.1f} s; 64 x 4096 workload in full")
        c2 = config2_oracle(pool, procs)
    cpu_s = sum(r[0] for r in res)
    comps = sum(r[1] for r in res)
    tokens_one_layer = B * steps
    # oracle compute rate on `procs` cores (input generation excluded); every
    # token of the workload needs all 36 layers
    value = tokens_one_layer / (cpu_s / procs) / L
    return {"value": round(value, 3), "unit": "tokens/s", "cores": procs, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpus_available": avail,
            "sample": (f"1 of 36 layers x {B} sequences x {steps} decode steps from the same "
                       f"phases ({comps} compressions), float64 NumPy oracle, one "
                       f"single-threaded process per core on {procs} cores (the host CPU share "
                       f"of one GPU; {avail} available to this process, {os.cpu_count()} on the "
                       f"host), {cpu_s:.1f} s of oracle compute ({wall:.1f} s wall with input "
                       f"generation); rate = tokens / (compute s / cores) / 36 layers"),
            "config_64x4096": c2}


# 64 prompts of 4096 tokens compressed at once to 1792, then 128 decode steps
# (one attention layer of the Qwen3-8B shape, bf16 values, 2% heavy keys x4)
C2_REQ, C2_PROMPT, C2_STEPS = 64, 4096, 128


def _oracle_config2_request(r):
    """One request of the 64 x 4096 workload through the oracle: the
    compression its prompt triggers (scores, top-k, compaction of every
    kv-head; first compression, window rows without a log-sum-exp) and 128
    decode steps. Returns the compute seconds (input generation excluded)."""
    import threadpoolctl
    from compressed_paged_kv_gqa_amd import synth
    from oracle import zipage as Z
    g = synth.rng(SEED, 2, r, "prompt_k")
    n = C2_PROMPT
    cap = n + C2_STEPS
    K = np.zeros((HKV, cap, D))
    V = np.zeros((HKV, cap, D))
    heavy = np.where(g.random((HKV, n)) < 0.02, 4.0, 1.0)[..., None]
    K[:, :n] = synth.round_bf16((g.standard_normal((HKV, n, D)) * heavy).astype(np.float32))
    V[:, :n] = synth.round_bf16(g.standard_normal((HKV, n, D)).astype(np.float32))
    qw = synth.round_bf16(g.standard_normal((HKV, HQ // HKV, W, D)).astype(np.float32))
    sq = synth.round_bf16(g.standard_normal((C2_STEPS, HQ, D)).astype(np.float32))
    sk = synth.round_bf16(g.standard_normal((C2_STEPS, HKV, D)).astype(np.float32))
    sv = synth.round_bf16(g.standard_normal((C2_STEPS, HKV, D)).astype(np.float32))
    params = Z.ScoreParams()
    keep = (NMAX - 1) * BS
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        for h in range(HKV):
            S, _F = Z.score_tokens(qw[h], K[h, :n], None, True, BS, params)
            kept = Z.topk_keep(S, keep)
            K[h, :keep] = K[h, kept]
            V[h, :keep] = V[h, kept]
        n = keep
        for s in range(C2_STEPS):
            K[:, n] = sk[s]
            V[:, n] = sv[s]
            n += 1
            Z.decode_attention(sq[s], K[:, :n], V[:, :n])
        return time.perf_counter() - t0


def config2_oracle(pool, procs):
    t0 = time.perf_counter()
    secs = pool.map(_oracle_config2_request, range(C2_REQ), chunksize=1)
    wall = time.perf_counter() - t0
    cpu_s = float(sum(secs))
    tokens = C2_REQ * C2_STEPS
    return {"value": round(tokens / (cpu_s / procs), 2), "unit": "tokens/s", "cores": procs,
            "seconds_compute": round(cpu_s, 1), "seconds_wall": round(wall, 1),
            "sample": (f"the whole workload: {C2_REQ} prompts x {C2_PROMPT} tokens resident, "
                       f"one compression burst to {(NMAX - 1) * BS} tokens per kv-head, then "
                       f"{C2_STEPS} decode steps, 1 layer; rate = decode tokens / (compute s / "
                       f"cores)")}


def config2_gpu():
    """The same 64 x 4096 workload on the GPU: prompts resident in the pages
    (window rows written without log-sum-exp, so scoring gathers its own
    softmax statistics), the compression burst they trigger, then 128 decode
    steps; decode tokens / wall time of both."""
    import torch
    from compressed_paged_kv_gqa_amd import zp
    from compressed_paged_kv_gqa_amd.engine import DecodeEngine
    nb = C2_PROMPT // BS
    geom = zp.CacheGeometry(num_layers=1, num_blocks=C2_REQ * nb + 8, block_size=BS,
                            num_kv_heads=HKV, num_q_heads=HQ, head_dim=D, window=W,
                            max_slots=C2_REQ, n_max=NMAX, dtype="bf16")
    eng = DecodeEngine(geom, zp.ScoreParams(), C2_REQ, nb, layer_stride=1)
    g = torch.Generator(device="cuda")
    g.manual_seed(SEED + 2)
    c = eng.cache
    c.k.normal_(generator=g)
    c.k.mul_(torch.where(torch.rand(c.k.shape[:-1], generator=g, device="cuda") < 0.02, 4.0,
                         1.0).unsqueeze(-1).to(c.k.dtype))
    c.v.normal_(generator=g)
    c.qwin.normal_(generator=g)
    for r in range(C2_REQ):
        eng.add_request(r, C2_PROMPT)
    q = torch.randn((C2_STEPS, 1, C2_REQ, HQ, D), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((C2_STEPS, 1, C2_REQ, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((C2_STEPS, 1, C2_REQ, HKV, D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.empty((1, C2_REQ, HQ, D), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    eng.compress_due_now()
    eng.wait_compressions()
    for i in range(C2_STEPS):
        eng.step(q[i], k[i], v[i], out)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    assert eng.compressions == C2_REQ and zp.zp_workspace_errors(eng.dec_ws) == 0
    tokens = eng.decoded_tokens
    return {"workload": f"{C2_REQ} prompts x {C2_PROMPT} tokens resident, compression burst to "
                        f"{(NMAX - 1) * BS}, then {C2_STEPS} decode steps, 1 layer, bf16, 2% "
                        f"heavy keys x4", "tokens_per_s": round(tokens / el, 1),
            "seconds": round(el, 4), "decode_tokens": tokens}


def practical_peak():
    """Measured bandwidth of plain torch kernels on this GPU, beside the
    nominal 8 TB/s: a 4 GiB device-to-device copy (read + write) and a sum
    over 4 GiB of bf16 (read once)."""
    import torch
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    x = src.view(torch.bfloat16)

    def med(fn):
        t = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return float(np.median(t))
    cp = med(lambda: dst.copy_(src))
    rd = med(lambda: x.sum(dtype=torch.float32))
    del src, dst, x
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * n / cp / 1e6, 1), "read_sum_gbs": round(n / rd / 1e6, 1),
            "note": "torch copy_ of 4 GiB (bytes read + written) and torch sum over 4 GiB "
                    "(bytes read), median of 5"}


# --------------------------------------------------------------------------

def decode_source_sha():
    """First 16 hex digits of the SHA-256 of the decode kernel's sources (the
    kernel file and the device headers it includes, in that order)."""
    h = hashlib.sha256()
    for name in ("zp_decode.hip", "zp_device.h", "zp_internal.h"):
        with open(os.path.join(ROOT, "compressed_paged_kv_gqa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per decode launch from the committed rocprofv3 PMC summary,
    if it was taken with the current decode kernel source."""
    path = os.path.join(ROOT, "profiles", f"paged_decode_pmc_{WORKLOAD}.md")
    if not os.path.exists(path):
        return None
    sha = decode_source_sha()
    text = open(path).read()
    m_sha = re.search(r"decode_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the hot path has no "
              "inter-GPU exchange and the library runs on one GPU.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.compress_kernels:
        print(json.dumps(compress_kernel_bench()), flush=True)
        return
    if args.prefill_kernels:
        print(json.dumps(prefill_kernel_bench()), flush=True)
        return
    if args.serve:
        print(json.dumps(serve_bench(args.serve_requests, args.serve_mem_gib,
                                     args.serve_policies.split(","))), flush=True)
        return
    if args.whole_run:
        print(json.dumps(whole_run_bench(args.whole_run_steps)), flush=True)
        return
    from compressed_paged_kv_gqa_amd import synth
    phases = synth.rng(SEED, 3, 0, "lengths").integers(0, BS, B)
    cpu = None
    if not args.no_cpu_baseline:
        # before this process touches the GPU: the pool's workers are plain
        # CPU processes
        log("cpu baseline: float64 oracle on the host cores")
        cpu = cpu_baseline(phases, args.cpu_sample_steps)
        log(f"cpu baseline: {cpu['value']} tokens/s on {cpu['cores']} cores")
    r = run_gpu(args, phases)
    value = r["tokens"] / r["elapsed"]
    ck = None
    if not args.no_compress_kernels:
        log("compression kernels in isolation")
        ck = compress_kernel_bench()
        log("prefill in isolation")
        ck = {"compress": ck, "prefill": prefill_kernel_bench()}
    log("the 64 x 4096 workload in full")
    c2 = config2_gpu()
    log("practical peak: device copy and read")
    peak = practical_peak()
    whole = None
    if not args.no_whole_run:
        import torch
        torch.cuda.empty_cache()
        log("whole run from the prompts")
        whole = whole_run_bench(args.whole_run_steps)
    serve = None
    if not args.no_serve:
        log("scheduled serving of the synthetic request stream")
        serve = serve_bench(args.serve_requests, args.serve_mem_gib,
                            args.serve_policies.split(","))
    traffic = traffic_from_profiles()
    line = {
        "metric": "decode tok/s at 256 seqs with compression; achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * r["elapsed"] / r["steps"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "layers": L, "sequences": B, "q_heads": HQ,
                   "kv_heads": HKV, "head_dim": D, "block_size": BS, "n_max": NMAX,
                   "window": W, "resident_tokens": "1793-2048 (steady state)",
                   "compression": "async side stream, layer stride 8, lightning redundancy",
                   "compressions_in_timed_steps": r["compressions"],
                   "compressions_with_window_lse": r["compressions_lse"],
                   "window_lse": "the window rows' log-sum-exp comes from decode; a sequence "
                                 "whose first compression falls within 16 steps of the start "
                                 "(phase > 240) scores through the statistics pass"},
        "roofline": {"bound": "hbm", "achieved": round(r["achieved_gbs"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["achieved_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "paged_decode_kernel<bf16,128,4,4>",
                     "avg_launch_ms": round(r["launch_ms"], 4),
                     "algorithmic_bytes_per_launch": round(r["bytes_per_launch"]),
                     "timed_launches": len(range(0, r["steps"], EVENT_EVERY)) * L,
                     "practical_peak": peak,
                     "frac_of_copy": round(r["achieved_gbs"] / peak["copy_gbs"], 4),
                     "frac_of_read": round(r["achieved_gbs"] / peak["read_sum_gbs"], 4)},
        "decode_ms_per_step": round(r["decode_ms_per_step"], 3),
        "config_64x4096": c2,
    }
    if ck is not None:
        line["compress_kernels"] = ck["compress"]
        line["prefill_kernels"] = ck["prefill"]
    if whole is not None:
        line["whole_run"] = whole
    if serve is not None:
        line["serve"] = serve
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
