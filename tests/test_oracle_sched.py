"""Pins of the oracle's constrained / hybrid scheduler (no GPU).

Zipage (arXiv 2603.08743) Sec. 4.3 (constrained scheduling, the four rules of
hybrid scheduling, Fig. 2), Sec. 4.1 (trigger at N >= N_max full blocks,
N_max - 1 blocks kept plus the reserved block), Sec. 4.4 (shared prefix
blocks, targets, preemption of the last uncompressed request).

The step-by-step traces below were worked out by hand from those rules and
the readings stated in the oracle module; the random-stream tests check
invariants that hold for any correct scheduler.
"""
import numpy as np
import pytest

from oracle.scheduler import CONSTRAINED, HYBRID, Scheduler


def _brief(o):
    return (o["kind"], [(e["rid"], e["slot"], e["ctx"], e["len"], e["table"]) for e in o["batch"]],
            [(c["rid"], c["src"], c["dst"], c["new"]) for c in o["comp"]],
            o["finished"], o["preempted"], o["blocked"])


def test_constrained_admits_at_most_m():
    """M = 2: the third request waits for a slot, gets the freed slot and the
    lowest free block once the second request finishes."""
    s = Scheduler(100, 16, 4, 4, 2, 8, 1000, CONSTRAINED)
    s.add(0, 10, 3)
    s.add(1, 20, 2)
    s.add(2, 5, 2)
    want = [
        ("prefill", [(0, 0, 0, 10, [0]), (1, 1, 0, 20, [1, 2])], [], [], [], 0),
        ("decode", [(0, 0, 10, 1, [0]), (1, 1, 20, 1, [1, 2])], [], [1], [], 0),
        ("prefill", [(2, 1, 0, 5, [1])], [], [], [], 0),
        ("decode", [(0, 0, 11, 1, [0]), (2, 1, 5, 1, [1])], [], [0, 2], [], 0),
        ("idle", [], [], [], [], 0),
    ]
    for w in want:
        assert _brief(s.step()) == w
    assert s.unfinished() == 0 and s.num_free() == 100


def test_hybrid_slotless_request_blocks_at_the_window_then_takes_the_slot():
    """M = 1, N_max = 2, b = 16, w = 4: positions 28..31 need a slot. The
    second request is admitted without one, stops before position 28, takes
    slot 0 when the first request finishes, is compressed at n = 32 (targets:
    its own first block, reserved: its second) and resumes with n = 16."""
    s = Scheduler(100, 16, 4, 2, 1, 8, 1000, HYBRID)
    s.add(0, 8, 5)
    s.add(1, 26, 10)
    want = [
        ("prefill", [(0, 0, 0, 8, [0]), (1, None, 0, 26, [1, 2])], [], [], [], 0),
        ("decode", [(0, 0, 8, 1, [0]), (1, None, 26, 1, [1, 2])], [], [], [], 0),
        ("decode", [(0, 0, 9, 1, [0]), (1, None, 27, 1, [1, 2])], [], [], [], 0),
        ("decode", [(0, 0, 10, 1, [0])], [], [], [], 1),
        ("decode", [(0, 0, 11, 1, [0])], [], [0], [], 1),
        ("decode", [(1, 0, 28, 1, [1, 2])], [], [], [], 0),
        ("decode", [(1, 0, 29, 1, [1, 2])], [], [], [], 0),
        ("decode", [(1, 0, 30, 1, [1, 2])], [], [], [], 0),
        ("decode", [(1, 0, 31, 1, [1, 2])], [], [], [], 0),
        ("idle", [], [(1, [1, 2], [1], [1, 2])], [], [], 0),
        ("decode", [(1, 0, 16, 1, [1, 2])], [], [], [], 0),
        ("decode", [(1, 0, 17, 1, [1, 2])], [], [], [], 0),
        ("decode", [(1, 0, 18, 1, [1, 2])], [], [1], [], 0),
    ]
    pos = []
    for w in want:
        o = s.step()
        assert _brief(o) == w, s.t
        pos += [(e["rid"], e["pos"]) for e in o["batch"]]
        for c in o["comp"]:
            s.compress_done(c["rid"])
    assert s.unfinished() == 0
    # token indices run on across the compression (cache position 16 holds
    # token 32), and the prefill of request 1 starts at token 0
    assert [p for r, p in pos if r == 1] == [0, 26, 27] + list(range(28, 35))


def test_constrained_waits_for_blocks_released_by_compression():
    """Four blocks = M N_max. A 40-token prompt holds three blocks; the short
    request finds no free block at n = 16 and waits (no preemption) until the
    long one is compressed into two blocks and its third block is released."""
    s = Scheduler(4, 16, 4, 2, 2, 8, 1000, CONSTRAINED)
    s.add(0, 40, 30)
    s.add(1, 10, 30)
    trace = []
    for _ in range(11):
        o = s.step()
        trace.append(_brief(o))
        for c in o["comp"]:
            s.compress_done(c["rid"])
    assert all(t[4] == [] for t in trace)                     # never preempts
    assert [t[5] for t in trace] == [0] * 7 + [1, 1, 1, 0]
    assert trace[7][1] == [(0, 0, 46, 1, [0, 1, 2])]
    assert trace[9] == ("idle", [], [(0, [0, 1, 2], [0], [0, 1])], [], [], 1)
    assert trace[10][1] == [(0, 0, 16, 1, [0, 1]), (1, 1, 16, 1, [3, 2])]


def test_hybrid_preempts_the_last_slotless_request():
    """M = 1 and four blocks. The slot-less second request needs its third
    block when none is free; being the last request without a slot it is
    itself preempted, and re-enters the waiting queue with its outputs."""
    s = Scheduler(4, 16, 4, 4, 1, 8, 1000, HYBRID)
    s.add(0, 16, 40)
    s.add(1, 20, 40)
    o = s.step()
    assert _brief(o)[1] == [(0, 0, 0, 16, [0]), (1, None, 0, 20, [1, 2])]
    o = s.step()
    assert _brief(o)[1] == [(0, 0, 16, 1, [0, 3]), (1, None, 20, 1, [1, 2])]
    for t in range(3, 14):
        o = s.step()
        assert o["preempted"] == []
    o = s.step()                                               # step 14
    assert o["preempted"] == [1] and [e["rid"] for e in o["batch"]] == [0]
    assert s.reqs[1].gen == 13 and s.reqs[1].table == [] and list(s.waiting) == [s.reqs[1]]
    assert s.num_free() == 2
    o = s.step()                                               # 33 tokens need 3 blocks
    assert o["kind"] == "decode" and [e["rid"] for e in o["batch"]] == [0]


def test_prefix_sharing_and_preemption_of_the_last_uncompressed_request():
    """Shared prefixes (Sec. 4.4), four blocks, M = 2. The second member of
    the group shares block 0 and prefills only 4 tokens. When the first
    member is due, its shared position needs a fresh target block and none
    is free: the last uncompressed request (the second member, which holds
    a slot) is preempted; block 0 is then private and compressed in place."""
    s = Scheduler(4, 16, 4, 2, 2, 8, 1000, HYBRID, prefix_sharing=True)
    s.add(0, 40, 20, 1, 16)
    assert _brief(s.step())[1] == [(0, 0, 0, 40, [0, 1, 2])]
    s.add(1, 20, 20, 1, 16)
    assert _brief(s.step())[1] == [(1, 1, 16, 4, [0, 3])]
    assert s.refcount == [2, 1, 1, 1]
    for _ in range(8):
        assert s.step()["kind"] == "decode"
    o = s.step()                                               # step 11
    assert _brief(o) == ("idle", [], [(0, [0, 1, 2], [0], [0, 1])], [], [1], 0)
    assert s.refcount == [1, 1, 1, 0] and s.groups == {}
    assert s.step()["kind"] == "idle"                         # 29 tokens need 2 blocks
    s.compress_done(0)
    assert s.refcount == [1, 1, 0, 0]
    o = s.step()
    assert _brief(o)[1] == [(1, 1, 0, 29, [2, 3])]


def test_prefix_members_of_one_step_do_not_share():
    """Members admitted in the step that writes the prefix prefill it
    themselves; a member admitted later shares it."""
    s = Scheduler(16, 16, 4, 2, 4, 8, 1000, HYBRID, prefix_sharing=True)
    s.add(0, 40, 10, 7, 32)
    s.add(1, 36, 10, 7, 32)
    o = s.step()
    assert _brief(o)[1] == [(0, 0, 0, 40, [0, 1, 2]), (1, 1, 0, 36, [3, 4, 5])]
    s.add(2, 34, 10, 7, 32)
    o = s.step()
    assert _brief(o)[1] == [(2, 2, 32, 2, [0, 1, 6])]
    assert s.refcount[:7] == [2, 2, 1, 1, 1, 1, 1] and s.groups[7]["holders"] == 2


def test_prefix_target_is_a_fresh_block_when_shared():
    s = Scheduler(16, 16, 4, 2, 4, 8, 1000, HYBRID, prefix_sharing=True)
    s.add(0, 40, 20, 7, 32)
    s.step()
    s.add(2, 34, 20, 7, 32)
    o = s.step()                                               # shares blocks 0, 1
    assert _brief(o)[1] == [(2, 1, 32, 2, [0, 1, 3])]
    for _ in range(8):
        s.step()                                               # request 0 reaches 48
    o = s.step()
    assert [(c["rid"], c["src"], c["dst"], c["new"]) for c in o["comp"]] == [(0, [0, 1, 2], [4], [4, 2])]
    s.compress_done(0)
    assert s.refcount[:6] == [1, 1, 1, 1, 1, 0]                # request 0 dropped blocks 0 and 1


# ----------------------------------------------------------------- invariants
def random_stream(seed, n, b, short=False, nmax_choices=None):
    """Prompts of 1..10 blocks (1..4 when short), outputs of 1..16 blocks
    (1..3 when short); 60 % of the requests in one of two prefix groups
    (prefix lengths 2b and b + 1). With nmax_choices, each request also draws
    its own N_max from them (0 = the configured one)."""
    rng = np.random.default_rng(seed)
    nm = np.random.default_rng(seed + 77)
    out = []
    for rid in range(n):
        prompt = int(rng.integers(1, 4 * b if short else 10 * b))
        new = int(rng.integers(1, 3 * b if short else 16 * b))
        grp, plen = -1, 0
        if rng.random() < 0.6:
            grp = int(rng.integers(0, 2))
            plen = b + 1 if grp else 2 * b          # one prefix length per group
            if plen >= prompt:
                grp, plen = -1, 0
        out.append((rid, prompt, new, grp, plen,
                    int(nm.choice(nmax_choices)) if nmax_choices else 0))
    return out


def drive(s, stream, seed, max_steps=200000, arrivals=True, check=None):
    """Adds requests over time, completes compressions after 0-3 steps."""
    rng = np.random.default_rng(seed + 1000)
    pend = []
    pos = 0
    steps = []
    for _ in range(max_steps):
        if pos < len(stream):
            k = len(stream) - pos if not arrivals else int(rng.integers(0, 4))
            for rid, p, m, g, pl, nm in stream[pos:pos + k]:
                s.add(rid, p, m, g, pl, nm)
            pos = min(pos + k, len(stream))
        o = s.step()
        steps.append(o)
        if check:
            check(s, o)
        pend += [[c["rid"], int(rng.integers(0, 4))] for c in o["comp"]]
        in_flight = bool(pend)
        keep = []
        for x in pend:
            if x[1] == 0:
                s.compress_done(x[0])
            else:
                x[1] -= 1
                keep.append(x)
        pend = keep
        if pos == len(stream) and s.unfinished() == 0 and not pend:
            return steps
        if o["kind"] == "idle" and not in_flight and pos == len(stream):
            raise AssertionError(f"no progress at step {s.t}")
    raise AssertionError("did not finish")


def _invariants(s, o):
    b = s.b
    # every block's count equals the number of tables (and pending plans) that hold it
    held = [0] * len(s.refcount)
    for r in s.reqs.values():
        for p in r.table:
            held[p] += 1
        if r.plan:
            for p in r.plan[2]:
                if p not in r.plan[0]:
                    held[p] += 1
    assert held == s.refcount
    slots = [r.slot for r in s.running if r.slot is not None]
    assert len(slots) == len(set(slots)) and all(0 <= x < s.M for x in slots)
    assert all(r.slot is not None for r in s.running if r.compressed or r.state == "compressing")
    # R4: slot holders sit among the first M running requests
    assert all(r.slot is None for r in s.running[s.M:])
    # per-request form of M <= N_total / N_max
    assert sum(r.n_max for r in s.running if r.slot is not None) <= len(s.refcount)
    if s.policy == CONSTRAINED:
        assert len(s.running) <= s.M
    assert len(s.running) <= s.max_running
    for e in o["batch"]:
        r = s.reqs[e["rid"]]
        if not r.compressed:
            assert e["pos"] == e["ctx"]
        if o["kind"] == "decode":
            assert e["pos"] == r.prompt + r.gen - 2          # gen counts this step's output
            assert e["slot"] is not None or not s.needs_slot(e["ctx"], r.n_max)
            assert e["ctx"] < len(e["table"]) * b
        else:
            last = e["ctx"] + e["len"] - 1
            assert e["slot"] is not None or not s.needs_slot(last, r.n_max)
            assert len(e["table"]) == -(-(last + 1) // b)
    for r in s.running:
        if r.compressed and r.state == "running":
            # the reserved block completes the table, unless N_max has grown
            # since (R10): the table then grows block by block up to it
            assert len(r.table) <= r.n_max and r.n <= r.n_max * b
            assert len(r.table) == r.n_max or r.n_max > r.base_n_max
    for c in o["comp"]:
        nm = c["n_max"]
        assert len(c["dst"]) == nm - 1 and len(c["new"]) == nm and c["slot"] is not None


@pytest.mark.parametrize("policy", [CONSTRAINED, HYBRID])
@pytest.mark.parametrize("prefix", [False, True])
@pytest.mark.parametrize("extra", [0, 6])
@pytest.mark.parametrize("seed", range(4))
def test_random_streams_finish_with_invariants(policy, prefix, extra, seed):
    b, nmax, M = 16, 3, 4
    stream = random_stream(seed, 40, b, short=seed % 2 == 1)
    if not prefix:
        stream = [(r, p, m, -1, 0, nm) for r, p, m, _g, _pl, nm in stream]
    # the longest prompt (10 blocks) fits; M N_max <= blocks (Sec. 4.2)
    nb = max(M * nmax, 10) + extra
    s = Scheduler(nb, b, 4, nmax, M, 8, 256, policy, prefix_sharing=prefix, table_cap=64)
    drive(s, stream, seed, check=_invariants)
    out = {r.rid: r.gen for r in s.reqs.values()}
    assert out == {x[0]: x[2] for x in stream}
    assert s.num_free() == nb


@pytest.mark.parametrize("policy", [CONSTRAINED, HYBRID])
@pytest.mark.parametrize("prefix", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_per_request_n_max_streams_finish_with_invariants(policy, prefix, seed):
    """Requests with their own N_max (2, 3 or the configured 4) on a pool
    smaller than M times the largest N_max: the slot reservation keeps the
    holders within the pool and every request finishes."""
    b, nmax, M = 16, 4, 4
    stream = random_stream(seed, 40, b, short=seed % 2 == 1, nmax_choices=[2, 3, 0])
    if not prefix:
        stream = [(r, p, m, -1, 0, nm) for r, p, m, _g, _pl, nm in stream]
    nb = 12
    s = Scheduler(nb, b, 4, nmax, M, 8, 256, policy, prefix_sharing=prefix, table_cap=64)
    steps = drive(s, stream, seed, check=_invariants)
    assert {r.rid: r.gen for r in s.reqs.values()} == {x[0]: x[2] for x in stream}
    assert s.num_free() == nb
    kept = {c["n_max"] for o in steps for c in o["comp"]}
    assert kept >= {2, 3}


def test_per_request_n_max_compresses_to_its_own_cap():
    """N_max = 2 for one request, 3 for the other (b = 16): the first is due
    at 32 tokens and keeps 16, the second at 48 and keeps 32."""
    s = Scheduler(100, 16, 4, 3, 2, 8, 1000, HYBRID)
    s.add(0, 30, 20, n_max=2)
    s.add(1, 46, 20)
    comps = []
    for _ in range(6):
        o = s.step()
        comps += [(c["rid"], c["n_max"], c["src"], c["dst"], c["new"]) for c in o["comp"]]
        for c in o["comp"]:
            s.compress_done(c["rid"])
    assert comps == [(0, 2, [0, 1], [0], [0, 1]), (1, 3, [2, 3, 4], [2, 3], [2, 3, 4])]
    # both were due after step 3, compressed in step 4, decoded in steps 5, 6
    assert (s.reqs[0].n, s.reqs[1].n) == (16 + 2, 32 + 2)


def test_slot_reservation_holds_back_a_large_n_max():
    """Pool of 6 blocks, M = 2: a request with N_max 4 holds a slot, a second
    with N_max 4 would push the reserved caps to 8 > 6 and is admitted
    without a slot (hybrid) or not at all (constrained); one with N_max 2
    fits beside the first."""
    for pol, want in ((HYBRID, [0, None]), (CONSTRAINED, [0])):
        s = Scheduler(6, 16, 4, 4, 2, 8, 1000, pol)
        s.add(0, 10, 5)
        s.add(1, 10, 5)
        o = s.step()
        assert [e["slot"] for e in o["batch"]] == want
    s = Scheduler(6, 16, 4, 4, 2, 8, 1000, CONSTRAINED)
    s.add(0, 10, 5)
    s.add(1, 10, 5, n_max=2)
    o = s.step()
    assert [e["slot"] for e in o["batch"]] == [0, 1]


def test_constrained_never_preempts_and_hybrid_runs_more_requests():
    """Short requests (fewer than N_max blocks each): constrained scheduling
    keeps at most M requests running; hybrid scheduling fills the idle
    blocks with requests that need no slot (Sec. 4.3)."""
    b, nmax, M = 16, 4, 2
    stream = [(r, 20, 20, -1, 0, 0) for r in range(24)]
    res = {}
    for pol in (CONSTRAINED, HYBRID):
        s = Scheduler(M * nmax + 8, b, 4, nmax, M, 16, 10000, pol)
        steps = drive(s, stream, 0, arrivals=False)
        dec = [len(o["batch"]) for o in steps if o["kind"] == "decode"]
        res[pol] = (len(steps), max(dec), sum(len(o["preempted"]) for o in steps))
    assert res[CONSTRAINED][1] == M and res[CONSTRAINED][2] == 0
    assert res[HYBRID][1] > M
    assert res[HYBRID][0] < res[CONSTRAINED][0]


# ------------------------------------------------------------ adaptive N_max
def test_adaptive_n_max_raises_the_cap_with_the_sequence_length():
    """R10 by hand: b = 16, w = 4, N_cap = 4, growth step A = 24, one request
    added with N_max 2 (prompt 30, 40 outputs). L = prompt + outputs:
    after the prefill L = 31 -> N_max 2 + 31 // 24 = 3; at L = 48 (step 18)
    -> 4, the cap. With N_max 2 it would have been due at n = 32 (step 3);
    now it is due at n = 64 (step 35, 35 outputs), compressed in step 36 to
    (4 - 1) * 16 = 48 tokens with its own blocks as targets, and finishes
    after 5 more outputs in step 41."""
    s = Scheduler(100, 16, 4, 4, 1, 8, 1000, HYBRID, nmax_growth=24)
    s.add(0, 30, 40, n_max=2)
    r = s.reqs[0]
    nm, comps, fin = [], [], None
    for t in range(1, 45):
        o = s.step()
        nm.append(r.n_max)
        for c in o["comp"]:
            comps.append((t, c["n_max"], c["src"], c["dst"], c["new"], r.n))
            s.compress_done(c["rid"])
        if o["finished"]:
            fin = t
            break
    assert nm[:17] == [3] * 17 and nm[17:35] == [4] * 18
    assert comps == [(36, 4, [0, 1, 2, 3], [0, 1, 2], [0, 1, 2, 3], 64)]
    assert fin == 41 and r.gen == 40


def test_adaptive_n_max_raise_is_cut_by_the_slot_reservation():
    """Pool of 7 blocks, M = 2, N_cap 4, A = 8; two requests added with
    N_max 2 (prompts 10; 30 and 60 outputs). After the prefill (L = 11) each
    wants 3: holders' sum 4 -> 5 -> 6 <= 7. At L = 16 (step 6) each wants 4:
    request 0 gets it (sum 7); request 1 is cut to 3 (7 - 7 leaves no room)
    and stays there until request 0 finishes in step 30: request 0 comes
    first in that step's batch, so its slot is free when request 1's raise is
    taken, in the same step. Request 1 is due at n = 64 (step 55), compressed
    in step 56 to 48 tokens, and finishes after 5 more outputs (step 61)."""
    s = Scheduler(7, 16, 4, 4, 2, 8, 1000, HYBRID, nmax_growth=8)
    s.add(0, 10, 30, n_max=2)
    s.add(1, 10, 60, n_max=2)
    r0, r1 = s.reqs[0], s.reqs[1]
    traj, comps, fin = [], [], {}
    for t in range(1, 70):
        o = s.step()
        traj.append((r0.n_max, r1.n_max))
        for c in o["comp"]:
            comps.append((t, c["rid"], c["n_max"], r1.n))
            s.compress_done(c["rid"])
        for x in o["finished"]:
            fin[x] = t
        assert not o["preempted"]
        if s.unfinished() == 0:
            break
    assert traj[:5] == [(3, 3)] * 5
    assert traj[5:29] == [(4, 3)] * 24
    assert traj[29] == (4, 4)
    assert fin == {0: 30, 1: 61}
    assert comps == [(56, 1, 4, 64)]


def test_adaptive_n_max_off_keeps_the_given_cap():
    s = Scheduler(100, 16, 4, 4, 1, 8, 1000, HYBRID)
    s.add(0, 30, 5, n_max=2)
    for _ in range(5):
        o = s.step()
        assert s.reqs[0].n_max == 2 or s.reqs[0].state == "finished"
        for c in o["comp"]:
            assert c["n_max"] == 2
            s.compress_done(c["rid"])


@pytest.mark.parametrize("policy", [CONSTRAINED, HYBRID])
@pytest.mark.parametrize("prefix", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_adaptive_n_max_streams_finish_with_invariants(policy, prefix, seed):
    """Random streams with N_base in {2, 3} and a growth step of 3 blocks on
    a pool where the reservation binds: invariants hold at every step, every
    request finishes, and compressions happen at more than one N_max."""
    b, nmax, M = 16, 5, 4
    stream = random_stream(seed, 40, b, short=seed % 2 == 1, nmax_choices=[2, 3])
    if not prefix:
        stream = [(r, p, m, -1, 0, nm) for r, p, m, _g, _pl, nm in stream]
    nb = 14
    s = Scheduler(nb, b, 4, nmax, M, 8, 256, policy, prefix_sharing=prefix, table_cap=64,
                  nmax_growth=3 * b)

    def check(s, o):
        _invariants(s, o)
        for r in s.reqs.values():
            assert r.base_n_max <= r.n_max <= s.n_max

    steps = drive(s, stream, seed, check=check)
    assert {r.rid: r.gen for r in s.reqs.values()} == {x[0]: x[2] for x in stream}
    assert s.num_free() == nb
    kept = {c["n_max"] for o in steps for c in o["comp"]}
    assert len(kept) >= 2
    assert any(r.n_max > r.base_n_max for r in s.reqs.values())
