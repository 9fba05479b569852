"""Host runtime around libzp: per-step decode of a batch of requests, the
compression trigger, target planning, and asynchronous compression on a side
HIP stream.

Zipage (arXiv 2603.08743): Sec. 4.1 (cap of N_max blocks, trigger after a
step that leaves N >= N_max full blocks, reserved N_max-th block), Sec. 4.2
(query-cache slot per request), Sec. 4.4 (shared prefix blocks and their
target blocks), Sec. 4.5 (decoding requests do not wait for compression; a
compressing request rejoins decode once its compression has finished),
App. C.1 (compression runs layer_stride layers per launch).

Every numeric step runs in the library's kernels; this module only keeps
block tables and per-request state and enqueues work (torch supplies device
memory and streams). Scheduling policies (admission, preemption, hybrid query
slots) are out of scope: requests are added explicitly.
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
        self.pending: list[_Pending] = []
        self.compressions = 0
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
        return act

    def decode_layer(self, layer, q, k_new, v_new, out, lse=None):
        zp.zp_paged_decode(self.cache, layer, q, k_new, v_new, self.tables_d, self.lens_d,
                           self.max_seq_len, self.qslot_d, out, lse, self.dec_ws)

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
        b, n_max = G.block_size, G.n_max
        keep = G.keep
        plans, ok = [], []
        for s in sids:
            r = self.reqs[s]
            try:
                dst, new, _ = self.alloc.plan_compress(r.table, n_max)
            except zp.NoBlocks:
                continue          # stays uncompressed; a scheduler would preempt
            plans.append((list(r.table), dst, new))
            ok.append(s)
            r.compressing = True
        if not ok:
            return
        nreq = len(ok)
        maxb = max(len(p[0]) for p in plans)
        nd = n_max - 1
        # one pinned int32 staging buffer: src tables | dst tables | N | slot |
        # first | window log-sum-exp valid
        meta = torch.zeros(nreq * (maxb + nd + 4), dtype=torch.int32).pin_memory()
        m = meta.numpy()
        src = m[:nreq * maxb].reshape(nreq, maxb)
        dst = m[nreq * maxb:nreq * (maxb + nd)].reshape(nreq, nd)
        tail = m[nreq * (maxb + nd):].reshape(4, nreq)
        for i, p in enumerate(plans):
            src[i, :len(p[0])] = p[0]
            dst[i] = p[1]
        tail[0] = [len(p[0]) for p in plans]
        tail[1] = ok
        tail[2] = [1 if self.reqs[s].first else 0 for s in ok]
        # every window row (the last w positions) carries its log-sum-exp
        tail[3] = [1 if self.reqs[s].n - G.window >= self.reqs[s].lse_from else 0 for s in ok]
        first = tail[2].astype(np.uint8)
        stream = self.side if self.async_compress else torch.cuda.current_stream()
        ready = torch.cuda.Event()
        ready.record()
        bufs = [meta]
        with torch.cuda.stream(stream):
            stream.wait_event(ready)
            meta_d = meta.to(self.device, non_blocking=True)
            o = nreq * maxb
            src_d = meta_d[:o].view(nreq, maxb)
            dst_d = meta_d[o:o + nreq * nd].view(nreq, nd)
            o += nreq * nd
            nblk_d = meta_d[o:o + nreq]
            qslot_d = meta_d[o + nreq:o + 2 * nreq]
            first_d = meta_d[o + 2 * nreq:o + 3 * nreq].to(torch.uint8)
            lse_d = (meta_d[o + 3 * nreq:o + 4 * nreq].to(torch.uint8) if self.window_lse
                     else None)
            ls = self.layer_stride
            nl = G.num_layers if self.record else ls     # recording keeps every layer
            scores = torch.empty((nl, nreq, G.num_kv_heads, maxb * b), dtype=torch.float32,
                                 device=self.device)
            use_f = self.params.use_global and self.cache.gscore is not None
            f_new = torch.empty_like(scores) if use_f else None
            kept = (torch.empty((G.num_layers, nreq, G.num_kv_heads, keep), dtype=torch.int32,
                                device=self.device) if self.record else None)
            sws = zp.new_workspace(zp.zp_score_workspace_size(G, ls, nreq, maxb), self.device)
            cws = zp.new_workspace(zp.zp_select_workspace_size(G, ls, nreq, keep), self.device)
            for lb in range(0, G.num_layers, ls):
                lc = min(ls, G.num_layers - lb)
                sl = slice(lb, lb + lc) if self.record else slice(0, lc)
                sc, fn = scores[sl], (f_new[sl] if use_f else None)
                zp.zp_score_tokens(self.cache, self.params, lb, lc, src_d, nblk_d, maxb, qslot_d,
                                   first_d, sc, fn, sws, stream=stream, window_lse_valid=lse_d)
                zp.zp_select_compact(self.cache, lb, lc, sc, src_d, nblk_d, maxb, dst_d, keep,
                                     kept[sl] if kept is not None else None, cws,
                                     stream=stream, f_new=fn)
            done = torch.cuda.Event()
            done.record(stream)
            bufs += [meta_d, first_d, lse_d, scores, f_new, sws, cws]
            if self.record:
                self.log.append((list(ok), first.copy(), scores, kept))
        self.pending.append(_Pending(ok, plans, done, bufs))
        self.compressions += nreq
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
