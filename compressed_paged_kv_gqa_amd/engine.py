"""Host runtime around libzp: per-step decode of a batch of requests, the
compression trigger, target planning, asynchronous compression on a side HIP
stream, and a serving loop driven by the library's scheduler.

Zipage (arXiv 2603.08743): Sec. 4.1 (cap of N_max blocks, trigger after a
step that leaves N >= N_max full blocks, reserved N_max-th block), Sec. 4.2
(query-cache slot per request), Sec. 4.3 and Fig. 2 (constrained / hybrid
scheduling), Sec. 4.4 (shared prefix blocks and their target blocks),
Sec. 4.5 (decoding requests do not wait for compression; a compressing
request rejoins decode once its compression has finished), App. C.1
(compression runs layer_stride layers per launch).

Every numeric step runs in the library's kernels; this module only keeps
block tables and per-request state and enqueues work (torch supplies device
memory and streams). DecodeEngine takes requests added explicitly with their
tokens; ServingEngine takes a request stream and lets zp_sched decide
admission, query slots, preemption and compression.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import zp


@dataclass
class Request:
    sid: int
    table: list
    n: int                      # resident tokens
    first: bool = True          # never compressed so far
    compressing: bool = False
    done: bool = False
    lse_from: int = 0           # window rows at positions >= lse_from carry their log-sum-exp


@dataclass
class _Pending:
    sids: list
    plans: list                 # (old_table, dst, new_table)
    event: torch.cuda.Event
    buffers: list = field(default_factory=list)   # keep tensors alive until the event


class Compressor:
    """Enqueues compressions (Zipage Sec. 4.2 scoring, then top-k and
    compaction, App. C.6) of a batch of requests, layer_stride layers per
    launch (App. C.1), on a side stream that first waits for the work already
    enqueued on the current stream (Sec. 4.5)."""

    def __init__(self, cache: zp.PagedKVCache, params: zp.ScoreParams, layer_stride,
                 stream=None, device="cuda"):
        self.cache = cache
        self.geom = cache.geom
        self.params = params
        self.layer_stride = max(1, min(layer_stride, cache.geom.num_layers))
        self.stream = stream
        self.device = device
        # Buffers reused by every launch (grown when a launch needs more):
        # device ones are used in stream order on the compression stream; the
        # pinned metadata buffers form a ring, each rewritten only after the
        # copy that last read it has run.
        self._dev = {}
        self._ring = [[None, None] for _ in range(4)]
        self._ring_i = 0

    def _device_buf(self, name, numel, dtype, zero, old):
        """Flat device buffer of at least numel elements; a replaced one goes
        to `old` so that it outlives the launches already enqueued on it."""
        t = self._dev.get(name)
        if t is None or t.numel() < numel:
            if t is not None:
                old.append(t)
            make = torch.zeros if zero else torch.empty
            t = make(max(numel, 1), dtype=dtype, device=self.device)
            self._dev[name] = t
        return t

    def _pinned_meta(self, numel):
        slot = self._ring[self._ring_i]
        self._ring_i = (self._ring_i + 1) % len(self._ring)
        buf, ev = slot
        if ev is not None:
            ev.synchronize()          # the copy that last read this buffer has run
        if buf is None or buf.numel() < numel:
            buf = torch.zeros(max(numel, 1), dtype=torch.int32).pin_memory()
            slot[0] = buf
        slot[1] = torch.cuda.Event()
        return buf, slot

    def launch(self, src, dst, nblocks, slots, first, lse_ok, record=False, n_max=None):
        """src [nreq][maxb] / dst [nreq][n_max-1] block tables, nblocks, query
        slots, first-compression and window-LSE flags per request (host
        values); every request of the call keeps (n_max - 1) b tokens
        (n_max defaults to the geometry's). Returns (done event, buffers to
        keep alive until it, scores, kept indices); scores and kept cover
        every layer only when record."""
        G = self.geom
        n_max = G.n_max if n_max is None else n_max
        b, keep = G.block_size, (n_max - 1) * G.block_size
        nreq, maxb = src.shape
        nd = n_max - 1
        assert np.shape(dst) == (nreq, nd)
        # one pinned int32 staging buffer: src tables | dst tables | N | slot |
        # first | window log-sum-exp valid
        nmeta = nreq * (maxb + nd + 4)
        meta_all, ring_slot = self._pinned_meta(nmeta)
        meta = meta_all[:nmeta]
        m = meta.numpy()
        m[:nreq * maxb] = np.asarray(src, np.int32).reshape(-1)
        m[nreq * maxb:nreq * (maxb + nd)] = np.asarray(dst, np.int32).reshape(-1)
        tail = m[nreq * (maxb + nd):].reshape(4, nreq)
        tail[0] = nblocks
        tail[1] = slots
        tail[2] = [1 if f else 0 for f in first]
        tail[3] = [1 if f else 0 for f in lse_ok]
        stream = self.stream or torch.cuda.current_stream()
        ready = torch.cuda.Event()
        ready.record()
        bufs = []
        with torch.cuda.stream(stream):
            stream.wait_event(ready)
            meta_d = self._device_buf("meta", nmeta, torch.int32, False, bufs)[:nmeta]
            meta_d.copy_(meta, non_blocking=True)
            ring_slot[1].record(stream)
            o = nreq * maxb
            src_d = meta_d[:o].view(nreq, maxb)
            dst_d = meta_d[o:o + nreq * nd].view(nreq, nd)
            o += nreq * nd
            nblk_d = meta_d[o:o + nreq]
            qslot_d = meta_d[o + nreq:o + 2 * nreq]
            first_d = meta_d[o + 2 * nreq:o + 3 * nreq].to(torch.uint8)
            lse_d = (meta_d[o + 3 * nreq:o + 4 * nreq].to(torch.uint8)
                     if self.cache.qwin_lse is not None else None)
            # every request's window rows carry their log-sum-exp: the scoring
            # call skips its statistics pass altogether
            lse_all = lse_d is not None and all(bool(f) for f in lse_ok)
            ls = self.layer_stride
            use_f = self.params.use_global and self.cache.gscore is not None
            shape = (G.num_layers if record else ls, nreq, G.num_kv_heads, maxb * b)
            if record:
                # recording keeps every layer's scores and kept lists (read by tests)
                scores = torch.empty(shape, dtype=torch.float32, device=self.device)
                f_new = torch.empty_like(scores) if use_f else None
                kept = torch.empty((G.num_layers, nreq, G.num_kv_heads, keep), dtype=torch.int32,
                                   device=self.device)
            else:
                ns = int(np.prod(shape))
                scores = self._device_buf("scores", ns, torch.float32, False, bufs)[:ns].view(shape)
                f_new = (self._device_buf("f_new", ns, torch.float32, False, bufs)[:ns].view(shape)
                         if use_f else None)
                kept = None
            # workspaces: zero-filled once; the kernels leave their counters at zero
            sws = self._device_buf("score_ws", max(zp.zp_score_workspace_size(G, ls, nreq, maxb),
                                                   256), torch.uint8, True, bufs)
            cws = self._device_buf("select_ws", max(zp.zp_select_workspace_size(G, ls, nreq, keep),
                                                    256), torch.uint8, True, bufs)
            for lb in range(0, G.num_layers, ls):
                lc = min(ls, G.num_layers - lb)
                sl = slice(lb, lb + lc) if record else slice(0, lc)
                sc, fn = scores[sl], (f_new[sl] if use_f else None)
                zp.zp_score_tokens(self.cache, self.params, lb, lc, src_d, nblk_d, maxb, qslot_d,
                                   first_d, sc, fn, sws, stream=stream, window_lse_valid=lse_d,
                                   window_lse_all=lse_all)
                zp.zp_select_compact(self.cache, lb, lc, sc, src_d, nblk_d, maxb, dst_d, keep,
                                     kept[sl] if kept is not None else None, cws,
                                     stream=stream, f_new=fn)
            done = torch.cuda.Event()
            done.record(stream)
            bufs += [first_d, lse_d]
            if record:
                bufs += [scores, f_new, kept]
        return done, bufs, scores, kept


class DecodeEngine:
    """Batch of requests decoding layer by layer over a paged cache."""

    def __init__(self, geom: zp.CacheGeometry, params: zp.ScoreParams, max_seqs, table_cap,
                 layer_stride=8, async_compress=True, with_global=True, device="cuda",
                 cache_init=None, record=False, window_lse=True):
        self.geom = geom
        self.params = params
        self.B = max_seqs
        self.cap = table_cap
        self.layer_stride = max(1, min(layer_stride, geom.num_layers))
        self.async_compress = async_compress
        self.device = device
        # window_lse: the attention kernels keep each window query's
        # log-sum-exp, and scoring reuses it instead of a statistics pass
        self.window_lse = window_lse
        self.cache = zp.PagedKVCache(geom, device=device, with_global=with_global, init=cache_init,
                                     with_window_lse=window_lse)
        self.alloc = zp.BlockAllocator(geom.num_blocks)
        self.reqs: dict[int, Request] = {}
        # Host master copies, staged through a ring of pinned buffers: a
        # buffer is rewritten only after the copy that last read it finished.
        self.tables_np = np.zeros((max_seqs, table_cap), np.int32)
        self.lens_np = np.zeros(max_seqs, np.int32)
        self._ring = [(torch.zeros((max_seqs, table_cap), dtype=torch.int32).pin_memory(),
                       torch.zeros(max_seqs, dtype=torch.int32).pin_memory(),
                       torch.cuda.Event()) for _ in range(4)]
        self._ring_i = 0
        self.tables_d = torch.zeros((max_seqs, table_cap), dtype=torch.int32, device=device)
        self.lens_d = torch.zeros(max_seqs, dtype=torch.int32, device=device)
        self.qslot_d = torch.arange(max_seqs, dtype=torch.int32, device=device)
        self.max_seq_len = table_cap * geom.block_size
        self.dec_ws = zp.new_workspace(zp.zp_decode_workspace_size(geom, max_seqs,
                                                                    self.max_seq_len), device)
        self.side = torch.cuda.Stream(device=device)
        self.compressor = Compressor(self.cache, params, self.layer_stride,
                                     self.side if async_compress else None, device)
        self.pending: list[_Pending] = []
        self.compressions = 0
        self.compressions_lse = 0   # of which the window rows carried their log-sum-exp
        self.decoded_tokens = 0
        # optional per-layer timing of the decode kernel (start, end) events
        self.layer_events = None
        # with record=True every compression keeps its scores and kept indices
        # (device tensors, read by tests): list of (sids, first, scores, kept)
        self.record = record
        self.log = []

    # ------------------------------------------------------------------ setup
    def add_request(self, sid, n_tokens, prefix_table=None):
        """Registers request `sid` holding n_tokens resident tokens. Blocks
        are allocated here (after sharing `prefix_table`, if given); the
        caller fills their contents. Returns the block table."""
        assert 0 <= sid < self.B and sid not in self.reqs
        b = self.geom.block_size
        nb = -(-n_tokens // b)
        table = []
        if prefix_table:
            self.alloc.share(prefix_table)
            table = list(prefix_table)
        table += self.alloc.alloc(nb - len(table))
        assert len(table) <= self.cap
        # tokens written by the caller come without window log-sum-exp
        self.reqs[sid] = Request(sid, table, n_tokens, lse_from=n_tokens)
        return table

    def prefill(self, sids, chunk_lens, q, k_new, v_new, out, lse=None):
        """Prompt chunks of requests `sids` through every layer with
        zp_paged_prefill (Zipage Sec. 4.1: the prompt is written in full and
        may exceed N_max blocks until its first compression). Request sids[i]
        must have been added with the length it has after its chunk of
        chunk_lens[i] tokens; the tokens before the chunk (a shared prefix,
        say) are already resident. Chunk i occupies rows cu[i]..cu[i+1]-1
        (cu = running sum of chunk_lens) of q/out [L][T][h_q][d] and
        k_new/v_new [L][T][h_kv][d]. Window rows of each chunk's final block
        get their log-sum-exp. Compressions whose trigger the prompt meets
        are launched at the end."""
        G = self.geom
        lens = [int(x) for x in chunk_lens]
        assert len(lens) == len(sids) and q.shape[1] == sum(lens)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ctx = np.array([self.reqs[s].n - n for s, n in zip(sids, lens)], np.int32)
        assert (ctx >= 0).all()
        stride = max(len(self.reqs[s].table) for s in sids)
        tab = np.zeros((len(sids), stride), np.int32)
        for i, s in enumerate(sids):
            tab[i, :len(self.reqs[s].table)] = self.reqs[s].table
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(self.device)
        cu_d, ctx_d, tab_d = dev(cu), dev(ctx), dev(tab)
        slot_d = dev(np.array(sids, np.int32))
        ws = zp.new_workspace(zp.zp_prefill_workspace_size(G, len(sids)), self.device)
        for l in range(G.num_layers):
            zp.zp_paged_prefill(self.cache, l, q[l], k_new[l], v_new[l], cu_d, ctx_d, max(lens),
                                tab_d, slot_d, out[l], None if lse is None else lse[l], ws)
        for s, c in zip(sids, ctx):
            self.reqs[s].lse_from = int(c)
        self.prefill_ws = ws      # device error bits of the last prefill
        self.compress_due_now()

    def write_tokens(self, sid, layer, start, k, v):
        """Copies K/V rows [h_kv][t][d] of request `sid` into its pages from
        logical position `start` (prompt ingest; plain device copies)."""
        r = self.reqs[sid]
        b = self.geom.block_size
        t_total = k.shape[1]
        t = 0
        while t < t_total:
            pos = start + t
            blk, off = divmod(pos, b)
            cnt = min(b - off, t_total - t)
            pg = r.table[blk]
            self.cache.k[layer, pg, :, off:off + cnt] = k[:, t:t + cnt]
            self.cache.v[layer, pg, :, off:off + cnt] = v[:, t:t + cnt]
            t += cnt

    def write_window_queries(self, sid, layer, qw):
        """Query-cache rows [h_kv][g][w][d] of request `sid` (prompt window)."""
        self.cache.qwin[layer, sid] = qw

    # ------------------------------------------------------------------ step
    def active(self):
        return [s for s, r in self.reqs.items() if not r.compressing and not r.done]

    def prepare_step(self):
        """Reserves a block for each active request's next token and uploads
        tables and lengths. Returns the list of active sids."""
        self.poll()
        b = self.geom.block_size
        act = self.active()
        self.lens_np[:] = 0
        for s in act:
            r = self.reqs[s]
            if r.n // b >= len(r.table):
                r.table += self.alloc.alloc(1)
            nt = len(r.table)
            if not np.array_equal(self.tables_np[s, :nt], r.table):
                self.tables_np[s, :nt] = r.table
            self.lens_np[s] = r.n + 1
        tab_h, len_h, ev = self._ring[self._ring_i]
        self._ring_i = (self._ring_i + 1) % len(self._ring)
        ev.synchronize()
        np.copyto(tab_h.numpy(), self.tables_np)
        np.copyto(len_h.numpy(), self.lens_np)
        self.tables_d.copy_(tab_h, non_blocking=True)
        self.lens_d.copy_(len_h, non_blocking=True)
        ev.record()
        self._calls = zp.LayerCalls(self.cache, "decode", self.tables_d, self.lens_d, self.dec_ws,
                                    qslot=self.qslot_d, max_seq_len=self.max_seq_len)
        return act

    def decode_layer(self, layer, q, k_new, v_new, out, lse=None):
        self._calls(layer, q, k_new, v_new, out, lse)

    def finish_step(self, act):
        """Advances lengths and launches compressions that became due."""
        for s in act:
            self.reqs[s].n += 1
        self.decoded_tokens += len(act)
        due = [s for s in act if self._due(self.reqs[s])]
        if due:
            self.compress(due)

    def step(self, q, k_new, v_new, out):
        """One decode step of every active request through all layers.
        q/out: [L][B][h_q][d]; k_new/v_new: [L][B][h_kv][d] (rows of requests
        that are not active are ignored)."""
        act = self.prepare_step()
        for l in range(self.geom.num_layers):
            ev = self.layer_events[l] if self.layer_events else None
            if ev:
                ev[0].record()
            self.decode_layer(l, q[l], k_new[l], v_new[l], out[l])
            if ev:
                ev[1].record()
        self.finish_step(act)
        return act

    # ------------------------------------------------------------ compression
    def _due(self, r: Request):
        b, n_max = self.geom.block_size, self.geom.n_max
        N = -(-r.n // b)
        return N >= n_max and r.n % b == 0 and r.n > 0

    def compress_due_now(self):
        """Compresses requests whose prompt already meets the trigger."""
        due = [s for s, r in self.reqs.items()
               if not r.compressing and not r.done and self._due(r)]
        if due:
            self.compress(due)

    def compress(self, sids):
        G = self.geom
        plans, ok = [], []
        for s in sids:
            r = self.reqs[s]
            try:
                dst, new, _ = self.alloc.plan_compress(r.table, G.n_max)
            except zp.NoBlocks:
                continue          # stays uncompressed; a scheduler would preempt
            plans.append((list(r.table), dst, new))
            ok.append(s)
            r.compressing = True
        if not ok:
            return
        nreq = len(ok)
        maxb = max(len(p[0]) for p in plans)
        src = np.zeros((nreq, maxb), np.int32)
        for i, p in enumerate(plans):
            src[i, :len(p[0])] = p[0]
        # every window row (the last w positions) carries its log-sum-exp
        lse_ok = [self.reqs[s].n - G.window >= self.reqs[s].lse_from for s in ok]
        first = [self.reqs[s].first for s in ok]
        done, bufs, scores, kept = self.compressor.launch(
            src, np.array([p[1] for p in plans], np.int32), [len(p[0]) for p in plans], ok,
            first, lse_ok, record=self.record)
        if self.record:
            self.log.append((list(ok), np.array(first, np.uint8), scores, kept))
        self.pending.append(_Pending(ok, plans, done, bufs))
        self.compressions += nreq
        self.compressions_lse += sum(1 for f in lse_ok if f)
        if not self.async_compress:
            self.poll(wait=True)

    def poll(self, wait=False):
        """Commits finished compressions (all of them if wait)."""
        keep = self.geom.keep
        still = []
        for p in self.pending:
            if wait:
                p.event.synchronize()
            elif not p.event.query():
                still.append(p)
                continue
            for s, (old, _dst, new) in zip(p.sids, p.plans):
                self.alloc.commit_compress(old, new)
                r = self.reqs[s]
                r.table = list(new)
                r.n = keep
                r.first = False
                r.compressing = False
                r.lse_from = keep     # the next window rows come from decode
        self.pending = still

    def wait_compressions(self):
        self.poll(wait=True)

    def resident_kv(self, sid, layer, head):
        """K, V rows [n][d] of a request read back through its block table
        (test helper)."""
        r = self.reqs[sid]
        b = self.geom.block_size
        idx = torch.tensor(r.table, device=self.device)
        K = self.cache.k[layer, idx, head].reshape(-1, self.geom.head_dim)[:r.n]
        V = self.cache.v[layer, idx, head].reshape(-1, self.geom.head_dim)[:r.n]
        return K, V


class ServingEngine:
    """Requests driven by the library's scheduler (zp_sched: constrained or
    hybrid scheduling with query slots, preemption and shared prefixes,
    Zipage Sec. 4.3 / Fig. 2 / Sec. 4.4) through the prefill, decode and
    compression kernels.

    One call of step() asks the scheduler for a step and enqueues its work:
    first the compressions it planned (on the side stream, after the kernels
    of earlier steps, Sec. 4.5), then either one prefill of the admitted
    prompt chunks or one decode token of every scheduled request, layer by
    layer. Compressions whose event has completed are committed at the start
    of the next step. There are no weights: `inputs` supplies each layer's
    q / k / v rows for a step (see step()), and attention outputs go to
    buffers owned here (`out_prefill`, `out_decode`, the last step's values).
    """

    def __init__(self, geom: zp.CacheGeometry, params: zp.ScoreParams, max_running, table_cap,
                 max_prefill_tokens, policy="hybrid", prefix_sharing=False, layer_stride=8,
                 async_compress=True, with_global=True, device="cuda", keep_layer_outputs=False,
                 nmax_growth=0):
        G = geom
        self.geom = G
        self.device = device
        self.R, self.cap = max_running, table_cap
        self.max_seq_len = table_cap * G.block_size
        self.max_prefill = max_prefill_tokens
        self.cache = zp.PagedKVCache(G, device=device, with_global=with_global,
                                     with_window_lse=True)
        self.sched = zp.Scheduler(G.num_blocks, G.block_size, G.window, G.n_max, G.max_slots,
                                  max_running, max_prefill_tokens, policy,
                                  prefix_sharing=prefix_sharing, table_cap=table_cap,
                                  nmax_growth=nmax_growth)
        self.async_compress = async_compress
        self.side = torch.cuda.Stream(device=device)
        self.compressor = Compressor(self.cache, params, layer_stride,
                                     self.side if async_compress else None, device)
        # the decode batch varies step by step and smaller batches split the
        # sequences further: size the workspace for the largest need
        ws = max(zp.zp_decode_workspace_size(G, nb, self.max_seq_len)
                 for nb in range(1, max_running + 1))
        self.dec_ws = zp.new_workspace(ws, device)
        self.pf_ws = zp.new_workspace(zp.zp_prefill_workspace_size(G, max_running), device)
        # pinned staging ring for step metadata: tables [R][cap] | a [R] | slot [R] | cu [R+1]
        n_meta = max_running * (table_cap + 3) + 1
        self._ring = [(torch.zeros(n_meta, dtype=torch.int32).pin_memory(), torch.cuda.Event())
                      for _ in range(4)]
        self._ring_i = 0
        self.meta_d = torch.zeros(n_meta, dtype=torch.int32, device=device)
        dt = G.torch_dtype()
        nl = G.num_layers if keep_layer_outputs else 1
        # a request longer than max_prefill_tokens is prefilled alone
        self.max_chunk = max(max_prefill_tokens, self.max_seq_len)
        self.out_prefill = torch.empty((nl, self.max_chunk, G.num_q_heads, G.head_dim),
                                       dtype=dt, device=device)
        self.out_decode = torch.empty((nl, max_running, G.num_q_heads, G.head_dim), dtype=dt,
                                      device=device)
        self.pending = []           # (rids, event, buffers)
        self.generated = 0          # output tokens produced
        self.steps = 0

    # ---------------------------------------------------------------- intake
    def add(self, rid, prompt_len, max_new, prefix_group=-1, prefix_len=0, n_max=0):
        """Queues a request; n_max = its own N_max (0: the geometry's, which
        is also the largest allowed). With nmax_growth > 0 the scheduler
        raises it as the request's sequence grows (adaptive N_max)."""
        self.sched.add(rid, prompt_len, max_new, prefix_group, prefix_len, n_max)

    def unfinished(self):
        return self.sched.unfinished()

    # ------------------------------------------------------------------ step
    def _stage(self, st, first_col):
        """Uploads the step's tables, per-entry values and slots; returns the
        device views (tables [n][cap], a [n], slot [n], cu [n+1])."""
        n, cap = st.n, self.cap
        buf, ev = self._ring[self._ring_i]
        self._ring_i = (self._ring_i + 1) % len(self._ring)
        ev.synchronize()
        m = buf.numpy()
        m[:n * cap] = st.tables.reshape(-1)
        m[n * cap:n * cap + n] = first_col
        m[n * cap + n:n * cap + 2 * n] = st.slot
        cu = m[n * cap + 2 * n:n * cap + 3 * n + 1]
        cu[0] = 0
        np.cumsum(st.len, out=cu[1:])
        tot = n * (cap + 3) + 1
        self.meta_d[:tot].copy_(buf[:tot], non_blocking=True)
        ev.record()
        d = self.meta_d
        return (d[:n * cap].view(n, cap), d[n * cap:n * cap + n],
                d[n * cap + n:n * cap + 2 * n], d[n * cap + 2 * n:n * cap + 3 * n + 1])

    def _compress(self, st):
        # one launch per distinct N_max (requests may carry their own)
        for nm in sorted(set(st.c_nmax.tolist())):
            sel = np.nonzero(st.c_nmax == nm)[0]
            maxb = int(st.c_nblocks[sel].max())
            src = np.ascontiguousarray(st.c_src[sel, :maxb])
            dst = np.ascontiguousarray(st.c_dst[sel, :nm - 1])
            # every window row is written by a kernel that holds the
            # request's slot, so the window log-sum-exp is always valid here
            done, bufs, _s, _k = self.compressor.launch(
                src, dst, st.c_nblocks[sel].copy(), st.c_slot[sel].copy(),
                st.c_first[sel].astype(bool), [True] * len(sel), n_max=nm)
            self.pending.append((st.c_rid[sel].tolist(), done, bufs))
        if not self.async_compress:
            self.poll(wait=True)

    def poll(self, wait=False):
        """Commits compressions whose kernels have finished (all if wait)."""
        still = []
        for rids, ev, bufs in self.pending:
            if wait:
                ev.synchronize()
            elif not ev.query():
                still.append((rids, ev, bufs))
                continue
            for r in rids:
                self.sched.compress_done(r)
        self.pending = still

    def step(self, inputs):
        """One scheduler step. inputs(kind, st, layer) returns (q, k, v) for
        the step's tokens in batch-entry order: [T][h_q][d], [T][h_kv][d],
        [T][h_kv][d] with T = sum(st.len) (prefill) or st.n (decode).
        Returns the scheduler's Step."""
        self.poll()
        st = self.sched.step()
        self.steps += 1
        if st.n_comp:
            self._compress(st)
        G = self.geom
        if st.kind == zp.ZP_STEP_PREFILL:
            tab, ctx, slot, cu = self._stage(st, st.ctx)
            T = int(st.len.sum())
            mq = int(st.len.max())
            if T > self.max_chunk:
                raise RuntimeError(f"prefill of {T} tokens exceeds {self.max_chunk}")
            call = zp.LayerCalls(self.cache, "prefill", tab, ctx, self.pf_ws, qslot=slot,
                                 cu_seqlens=cu, max_q_len=mq)
            for l in range(G.num_layers):
                q, k, v = inputs(st.kind, st, l)
                call(l, q, k, v, self.out_prefill[l if self.out_prefill.shape[0] > 1 else 0, :T])
            self.generated += st.n
        elif st.kind == zp.ZP_STEP_DECODE:
            tab, lens, slot, _cu = self._stage(st, st.ctx + 1)
            call = zp.LayerCalls(self.cache, "decode", tab, lens, self.dec_ws, qslot=slot,
                                 max_seq_len=self.max_seq_len)
            for l in range(G.num_layers):
                q, k, v = inputs(st.kind, st, l)
                call(l, q, k, v, self.out_decode[l if self.out_decode.shape[0] > 1 else 0, :st.n])
            self.generated += st.n
        elif self.pending:
            # nothing to run until a compression commits
            self.pending[0][1].synchronize()
        elif st.n_comp == 0 and self.sched.unfinished() > 0:
            raise RuntimeError("scheduler made no progress: every request waits")
        return st

    def run(self, inputs, max_steps=1 << 30):
        """Steps until every request has finished; returns the step count."""
        n = 0
        while (self.sched.unfinished() > 0 or self.pending) and n < max_steps:
            if self.sched.unfinished() == 0:
                self.poll(wait=True)
                break
            self.step(inputs)
            n += 1
        return n

    def device_errors(self):
        """Device error bits of the decode and prefill workspaces."""
        return zp.zp_workspace_errors(self.dec_ws) | zp.zp_workspace_errors(self.pf_ws)
