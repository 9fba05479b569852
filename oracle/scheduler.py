"""Constrained and hybrid scheduling of Compressed PagedAttention, as a plain
Python state machine.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Integer logic: the
product's C++ scheduler must make exactly the same decisions, step by step.

Source: "Zipage: Maintain High Request Concurrency for LLM Reasoning through
Compressed PagedAttention" (arXiv 2603.08743):
  Sec. 4.1  cap of N_max blocks, compression once N >= N_max full blocks,
            the reserved N_max-th block;
  Sec. 4.2  one query-cache slot per compressing request, M slots in all;
  Sec. 4.3  constrained scheduling (at most M running requests, a request
            that finds no free block waits, no preemption) and hybrid
            scheduling (its four rules), Fig. 2 (request states);
  Sec. 4.4  shared prefix blocks, target blocks of a compression, and the
            preemption of the last uncompressed request when prefixes are
            shared.

Readings where the pages leave a step open (the product follows the same):
  R1  A step is either a prefill step or a decode step: requests at the head
      of the waiting queue are admitted first (first come, first served; the
      admission stops at the first request that cannot be admitted), and
      only when none is admitted do the running requests decode.
  R2  Token accounting: a prefill of L tokens produces one output token; a
      decode step appends the K/V of the previous output token and produces
      the next one. A request finishes when it has produced max_new tokens.
      A preempted request keeps its outputs and is prefilled again over
      prompt + outputs (recomputation), at the front of the waiting queue.
      A batch entry carries ctx (tokens resident before it: its cache
      position) and pos (its first token's index in the request's token
      sequence); they differ once the request has been compressed.
  R3  "Needs a query slot": writing the token at position p (0-based) needs
      a slot iff p lies in block N_max - 1 or later and in the last w slots
      of its block (its query is a window query of a block whose end can
      trigger a compression). A request without a slot decodes only while
      its next position needs none, and is admitted without a slot only
      if its last prompt position needs none.
  R4  Slot holders are always among the first M running requests (slots go
      to requests there, and the queue only shrinks ahead of them), so a
      request admitted at a position below M always finds a free slot.
  R5  Victims of a block shortage: with shared prefixes, the last running
      request that has never been compressed and is not being compressed;
      otherwise, under hybrid scheduling, the last running request without
      a slot; under constrained scheduling, none (the request waits).
      Victims are taken one at a time, from the back, until a block is
      free; the requester itself may be the victim.
  R6  A request whose step leaves n = N b tokens with N >= N_max is due.
      Compressions of due requests are planned at the start of the next
      step, before anything else, and run before that step's kernels; while
      compressing, a request does not decode. A due request whose targets
      cannot be allocated (shared prefixes only) preempts per R5, or waits.
  R7  Shared prefixes: requests of one prefix group share their first
      floor(prefix_len / b) blocks. The first member admitted writes them;
      later members (admitted in a later step) take a reference instead of
      prefilling them. A member stops holding the group's blocks when its
      compression is planned, when it finishes or when it is preempted; a
      group whose last holder stopped is forgotten.
  R8  Ids (blocks, slots) are taken lowest first.
  R9  Per-request N_max (the pages name it as a per-request attribute and
      leave the choice open): each request may carry its own N_max, at most
      the configured one, which every rule above then uses for it (slot
      need, trigger, targets, kept tokens). Slots are also reserved
      blockwise: a slot goes to a request only while the N_max of all slot
      holders, its own included, sums to at most the pool size, the
      per-request form of M <= N_total / N_max (Sec. 4.2), so the slot
      holders can always reach their caps. With one N_max for all and a pool
      sized by that rule the reservation never binds.
  R10 Adaptive N_max (the pages' Limitations section names an N_max set per
      request from its actual sequence length, with no rule): with a growth
      step A > 0, a request's N_max is raised, after each of its steps,
      to min(N_cap, N_base + floor(L / A)), where N_base is the N_max it was
      added with, N_cap the configured one and L = prompt + outputs so far
      (its actual sequence length). It never falls. A slot holder's raise is
      cut so that the slot holders' N_max still sum to at most the pool
      (R9); the rest of the raise waits for a later step. The raise comes
      before the trigger check, so a longer request is compressed later and
      keeps more blocks. A = 0 turns the rule off.
"""
from __future__ import annotations

from collections import deque

from .planner import plan_targets

WAITING, RUNNING, COMPRESSING, FINISHED = "waiting", "running", "compressing", "finished"
CONSTRAINED, HYBRID = "constrained", "hybrid"


class Req:
    def __init__(self, rid, prompt, max_new, group, prefix_len, n_max):
        self.rid = rid
        self.n_max = n_max
        self.base_n_max = n_max      # R10: the N_max it was added with
        self.prompt = prompt
        self.max_new = max_new
        self.group = group
        self.prefix_len = prefix_len
        self.gen = 0                 # output tokens produced so far
        self.n = 0                   # tokens resident in the cache
        self.table = []
        self.slot = None
        self.state = WAITING
        self.compressed = False      # at least one compression committed
        self.due = False
        self.holds_prefix = False
        self.plan = None             # (old table, dst, new table) while compressing


class Scheduler:
    def __init__(self, num_blocks, block_size, window, n_max, num_slots, max_running,
                 max_prefill_tokens, policy=HYBRID, prefix_sharing=False, table_cap=None,
                 nmax_growth=0):
        assert policy in (CONSTRAINED, HYBRID) and nmax_growth >= 0
        self.growth = nmax_growth
        self.b = block_size
        self.w = window
        self.n_max = n_max
        self.M = num_slots
        self.max_running = max_running
        self.max_prefill = max_prefill_tokens
        self.policy = policy
        self.prefix = prefix_sharing
        self.table_cap = table_cap
        self.num_blocks = num_blocks
        self.refcount = [0] * num_blocks
        self.reqs = {}
        self.waiting = deque()
        self.running = []
        self.groups = {}             # group -> dict(blocks, holders, step)
        self.group_len = {}
        self.t = 0

    # ------------------------------------------------------------ resources
    def num_free(self):
        return sum(1 for c in self.refcount if c == 0)

    def _alloc(self, k):
        ids = [i for i, c in enumerate(self.refcount) if c == 0][:k]
        assert len(ids) == k
        for i in ids:
            self.refcount[i] = 1
        return ids

    def _decref(self, ids):
        for i in ids:
            assert self.refcount[i] > 0
            self.refcount[i] -= 1

    def _lowest_free(self, used, limit):
        for i in range(limit):
            if i not in used:
                return i
        raise AssertionError("no free id")

    def _free_slot(self):
        return self._lowest_free({r.slot for r in self.running if r.slot is not None}, self.M)

    def _slot_fits(self, r):
        """R9: a free slot exists and the holders' N_max still fit the pool."""
        holders = [x for x in self.running if x.slot is not None]
        return (len(holders) < self.M and
                sum(x.n_max for x in holders) + r.n_max <= self.num_blocks)

    # ---------------------------------------------------------------- rules
    def needs_slot(self, p, n_max=None):
        """R3: writing position p needs a query-cache slot."""
        n_max = self.n_max if n_max is None else n_max
        return p // self.b >= n_max - 1 and p % self.b >= self.b - self.w

    def _is_due(self, r):
        return r.n > 0 and r.n % self.b == 0 and r.n // self.b >= r.n_max

    def _share_count(self, r):
        return r.prefix_len // self.b if (self.prefix and r.group >= 0) else 0

    def _leave_group(self, r):
        if r.holds_prefix:
            g = self.groups[r.group]
            g["holders"] -= 1
            if g["holders"] == 0:
                del self.groups[r.group]
            r.holds_prefix = False

    def _release(self, r):
        self._decref(r.table)
        self._leave_group(r)
        r.table, r.slot, r.n, r.due = [], None, 0, False
        self.running.remove(r)

    def _preempt(self, v, out):
        self._release(v)
        v.state = WAITING
        self.waiting.appendleft(v)
        out["preempted"].append(v.rid)

    def _victim(self):
        """R5."""
        for v in reversed(self.running):
            if self.prefix:
                if v.state == RUNNING and not v.compressed:
                    return v
            elif self.policy == HYBRID:
                if v.slot is None:
                    return v
        return None

    def _finish(self, r, out):
        self._release(r)
        r.state = FINISHED
        out["finished"].append(r.rid)

    # ------------------------------------------------------------------ api
    def add(self, rid, prompt_len, max_new, prefix_group=-1, prefix_len=0, n_max=0):
        assert rid not in self.reqs and prompt_len >= 1 and max_new >= 1
        n_max = n_max or self.n_max
        assert 2 <= n_max <= self.n_max
        if prefix_group >= 0:
            assert 0 <= prefix_len < prompt_len
            assert self.group_len.setdefault(prefix_group, prefix_len) == prefix_len
        r = Req(rid, prompt_len, max_new, prefix_group, prefix_len if prefix_group >= 0 else 0,
                n_max)
        self.reqs[rid] = r
        self.waiting.append(r)

    def compress_done(self, rid):
        """The compaction of `rid` has finished: its table becomes the target
        table, blocks it no longer lists lose its reference (Sec. 4.4)."""
        r = self.reqs[rid]
        assert r.state == COMPRESSING
        old, _dst, new = r.plan
        self._decref([p for p in old if p not in new])
        r.table = list(new)
        r.n = (r.n_max - 1) * self.b
        r.compressed = True
        r.state = RUNNING
        r.plan = None

    def unfinished(self):
        return sum(1 for r in self.reqs.values() if r.state != FINISHED)

    def step(self):
        self.t += 1
        out = dict(kind="idle", batch=[], comp=[], finished=[], preempted=[], blocked=0)
        # (a) R6: plan the compressions of due requests, in queue order
        for r in list(self.running):
            if r in self.running and r.state == RUNNING and r.due:
                self._try_compress(r, out)
        # (b) Sec. 4.3: free slots go to the foremost of the first M
        for r in self.running[:self.M]:
            if r.slot is None:
                if not self._slot_fits(r):
                    break                    # first come first served: no overtaking
                r.slot = self._free_slot()
        # (c) R1: admission
        if self._admit(out):
            out["kind"] = "prefill"
            for e in out["batch"]:
                r = self.reqs[e["rid"]]
                r.n = r.prompt + r.gen
                r.gen += 1
                self._advance(r, out)
        else:
            self._decode(out)
            if out["batch"]:
                out["kind"] = "decode"
                for e in out["batch"]:
                    r = self.reqs[e["rid"]]
                    r.n += 1
                    r.gen += 1
                    self._advance(r, out)
        return out

    # ---------------------------------------------------------------- steps
    def _grow(self, r):
        """R10: raise r's N_max with its actual sequence length."""
        if not self.growth:
            return
        want = min(self.n_max, r.base_n_max + (r.prompt + r.gen) // self.growth)
        if want <= r.n_max:
            return
        if r.slot is not None:
            held = sum(x.n_max for x in self.running if x.slot is not None)   # r's included
            want = min(want, r.n_max + self.num_blocks - held)
        r.n_max = max(r.n_max, want)

    def _advance(self, r, out):
        if r.gen >= r.max_new:
            self._finish(r, out)
            return
        self._grow(r)
        if self._is_due(r):
            r.due = True

    def _try_compress(self, r, out):
        while True:
            shared = {p for p in r.table if self.refcount[p] > 1}
            plan = plan_targets(r.table, {p: self.refcount[p] for p in r.table}, r.n_max)
            if plan["n_new"] <= self.num_free():
                break
            v = self._victim()
            if v is None:
                return                      # waits (R6)
            self._preempt(v, out)
            if v is r:
                return
        fresh = self._alloc(plan["n_new"])
        names = {f"new{i}": fresh[i] for i in range(plan["n_new"])}
        dst = [names.get(p, p) for p in plan["dst"]]
        new = [names.get(p, p) for p in plan["new_table"]]
        assert not (shared & set(new))
        self._leave_group(r)
        r.plan = (list(r.table), dst, new)
        r.state = COMPRESSING
        r.due = False
        out["comp"].append(dict(rid=r.rid, slot=r.slot, first=not r.compressed, n_max=r.n_max,
                                src=list(r.table), dst=dst, new=new))

    def _admit(self, out):
        tokens = 0
        while self.waiting and len(self.running) < self.max_running:
            r = self.waiting[0]
            L = r.prompt + r.gen
            g = self.groups.get(r.group) if self._share_count(r) > 0 else None
            if g is not None and g["step"] >= self.t:
                g = None                     # written in this very step
            nshare = len(g["blocks"]) if g else 0
            chunk = L - nshare * self.b
            if out["batch"] and tokens + chunk > self.max_prefill:
                break
            need = -(-L // self.b) - nshare
            if self.table_cap is not None:
                assert nshare + need <= self.table_cap, "table_cap exceeded"
            if self.num_free() < need:
                break
            with_slot = len(self.running) < self.M and self._slot_fits(r)
            if not with_slot and (self.policy == CONSTRAINED or self.needs_slot(L - 1, r.n_max)):
                break
            self.waiting.popleft()
            table = []
            if g:
                for p in g["blocks"]:
                    self.refcount[p] += 1
                g["holders"] += 1
                table = list(g["blocks"])
                r.holds_prefix = True
            table += self._alloc(need)
            k = self._share_count(r)
            if g is None and k > 0 and r.group not in self.groups:
                self.groups[r.group] = dict(blocks=table[:k], holders=1, step=self.t)
                r.holds_prefix = True
            r.table = table
            r.slot = self._free_slot() if with_slot else None
            r.state = RUNNING
            self.running.append(r)
            out["batch"].append(dict(rid=r.rid, slot=r.slot, ctx=nshare * self.b,
                                     pos=nshare * self.b, len=chunk, table=list(table)))
            tokens += chunk
        return bool(out["batch"])

    def _decode(self, out):
        sched = []
        for r in list(self.running):
            if r not in self.running or r.state != RUNNING or r.due:
                continue
            if r.slot is None and self.needs_slot(r.n, r.n_max):
                out["blocked"] += 1
                continue
            if r.n == len(r.table) * self.b:
                gone = False
                while self.num_free() == 0:
                    v = self._victim()
                    if v is None:
                        break
                    self._preempt(v, out)
                    if v in sched:
                        sched.remove(v)
                    if v is r:
                        gone = True
                        break
                if gone:
                    continue
                if self.num_free() == 0:
                    out["blocked"] += 1
                    continue
                if self.table_cap is not None:
                    assert len(r.table) < self.table_cap, "table_cap exceeded"
                r.table.append(self._alloc(1)[0])
            sched.append(r)
        for r in sched:
            out["batch"].append(dict(rid=r.rid, slot=r.slot, ctx=r.n, pos=r.prompt + r.gen - 1,
                                     len=1, table=list(r.table)))
