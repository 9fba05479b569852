"""The C++ scheduler (zp_sched_*, through the C ABI) against the oracle's
state machine, step by step (no GPU).

Zipage (arXiv 2603.08743) Sec. 4.3 (constrained / hybrid scheduling, Fig. 2)
and Sec. 4.4 (shared prefixes, preemption of the last uncompressed request).
Bar: integer decisions, so every step's output (kind, batch entries with
their slots, contexts, lengths and block tables, planned compressions with
source / target / new tables, finished and preempted ids, blocked count)
and every request's state and the pool's reference counts are identical.
"""
import numpy as np
import pytest

from compressed_paged_kv_gqa_amd import zp
from oracle.scheduler import Scheduler as OracleScheduler

from test_oracle_sched import random_stream

STATE = {"waiting": zp.ZP_REQ_WAITING, "running": zp.ZP_REQ_RUNNING,
         "compressing": zp.ZP_REQ_COMPRESSING, "finished": zp.ZP_REQ_FINISHED}


def _pair(num_blocks, b, w, nmax, M, R, max_prefill, policy, prefix=False, cap=64, growth=0):
    o = OracleScheduler(num_blocks, b, w, nmax, M, R, max_prefill, policy,
                        prefix_sharing=prefix, table_cap=cap, nmax_growth=growth)
    c = zp.Scheduler(num_blocks, b, w, nmax, M, R, max_prefill, policy, prefix_sharing=prefix,
                     table_cap=cap, nmax_growth=growth)
    return o, c


def _same_state(o, c):
    for rid, r in o.reqs.items():
        got = c.request(rid)
        want = dict(state=STATE[r.state], n=r.n, gen=r.gen,
                    slot=-1 if r.slot is None else r.slot, compressed=int(r.compressed),
                    ntable=len(r.table), n_max=r.n_max, table=r.table)
        assert got == want, (rid, got, want)
    assert [c.refcount(i) for i in range(len(o.refcount))] == o.refcount
    assert c.unfinished() == o.unfinished()


def lockstep(o, c, stream, seed, arrivals=True, max_steps=100000, state_every=1):
    rng = np.random.default_rng(seed + 1000)
    pend, pos, steps = [], 0, 0
    counts = dict(pre=0, blocked=0, slotless=0, shared=0, fresh=0, comp=0)
    while steps < max_steps:
        if pos < len(stream):
            k = len(stream) - pos if not arrivals else int(rng.integers(0, 4))
            for rid, p, m, g, pl, nm in stream[pos:pos + k]:
                o.add(rid, p, m, g, pl, nm)
                c.add(rid, p, m, g, pl, nm)
            pos = min(pos + k, len(stream))
        a = o.step()
        got = c.step().as_dict()
        steps += 1
        assert got == a, f"step {o.t}"
        if steps % state_every == 0:
            _same_state(o, c)
        counts["pre"] += len(a["preempted"])
        counts["blocked"] += a["blocked"]
        counts["slotless"] += sum(e["slot"] is None for e in a["batch"])
        counts["shared"] += sum(e["ctx"] > 0 for e in a["batch"] if a["kind"] == "prefill")
        counts["fresh"] += sum(bool(set(x["new"]) - set(x["src"])) for x in a["comp"])
        counts["comp"] += len(a["comp"])
        pend += [[x["rid"], int(rng.integers(0, 4))] for x in a["comp"]]
        keep = []
        for x in pend:
            if x[1] == 0:
                o.compress_done(x[0])
                c.compress_done(x[0])
            else:
                x[1] -= 1
                keep.append(x)
        pend = keep
        if steps % state_every == 0:
            _same_state(o, c)
        if pos == len(stream) and o.unfinished() == 0 and not pend:
            break
    assert o.unfinished() == 0
    st = c.stats()
    assert st["finished"] == len(stream) and st["free_blocks"] == len(o.refcount)
    assert st["preemptions"] == counts["pre"] and st["compressions"] == counts["comp"]
    return counts


@pytest.mark.parametrize("policy", ["constrained", "hybrid"])
@pytest.mark.parametrize("prefix", [False, True])
@pytest.mark.parametrize("extra", [0, 6])
@pytest.mark.parametrize("seed", range(4))
def test_random_streams_match_the_oracle(policy, prefix, extra, seed):
    b, nmax, M = 16, 3, 4
    stream = random_stream(seed, 40, b, short=seed % 2 == 1)
    if not prefix:
        stream = [(r, p, m, -1, 0, nm) for r, p, m, _g, _pl, nm in stream]
    o, c = _pair(max(M * nmax, 10) + extra, b, 4, nmax, M, 8, 256, policy, prefix)
    lockstep(o, c, stream, seed)


@pytest.mark.parametrize("policy", ["constrained", "hybrid"])
@pytest.mark.parametrize("prefix", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_per_request_n_max_matches_the_oracle(policy, prefix, seed):
    """Requests with their own N_max (2, 3, or the configured 4) on a pool
    where the slot reservation binds."""
    b, nmax, M = 16, 4, 4
    stream = random_stream(seed, 40, b, short=seed % 2 == 1, nmax_choices=[2, 3, 0])
    if not prefix:
        stream = [(r, p, m, -1, 0, nm) for r, p, m, _g, _pl, nm in stream]
    o, c = _pair(12, b, 4, nmax, M, 8, 256, policy, prefix)
    lockstep(o, c, stream, seed)


@pytest.mark.parametrize("policy", ["constrained", "hybrid"])
@pytest.mark.parametrize("prefix", [False, True])
@pytest.mark.parametrize("seed", range(3))
def test_adaptive_n_max_matches_the_oracle(policy, prefix, seed):
    """Adaptive N_max (growth step 3 blocks, N_base 2 or 3, cap 5) on a pool
    where the slot reservation cuts raises: same decisions, same caps."""
    b = 16
    stream = random_stream(seed, 40, b, short=seed % 2 == 1, nmax_choices=[2, 3])
    if not prefix:
        stream = [(r, p, m, -1, 0, nm) for r, p, m, _g, _pl, nm in stream]
    o, c = _pair(14, b, 4, 5, 4, 8, 256, policy, prefix, growth=3 * b)
    lockstep(o, c, stream, seed)
    assert any(r.n_max > r.base_n_max for r in o.reqs.values())


def test_adaptive_n_max_hand_scenarios_match():
    """The two hand-derived traces of the oracle's pins, through the C ABI."""
    for args, adds in (((100, 16, 4, 4, 1, 8, 1000, "hybrid"), [(0, 30, 40, -1, 0, 2)]),
                       ((7, 16, 4, 4, 2, 8, 1000, "hybrid"), [(0, 10, 30, -1, 0, 2),
                                                              (1, 10, 60, -1, 0, 2)])):
        o, c = _pair(*args, growth=24 if args[0] == 100 else 8)
        lockstep(o, c, adds, 0, arrivals=False)


def test_the_random_streams_reach_every_branch():
    """Across the parity streams: preemptions, waits, slot-less decoding,
    shared prefixes and fresh target blocks all occur."""
    tot = dict(pre=0, blocked=0, slotless=0, shared=0, fresh=0, comp=0)
    for policy in ("constrained", "hybrid"):
        for seed in range(4):
            stream = random_stream(seed, 40, 16, short=seed % 2 == 1)
            o, c = _pair(12, 16, 4, 3, 4, 8, 256, policy, True)
            for k, v in lockstep(o, c, stream, seed).items():
                tot[k] += v
    assert all(v > 0 for v in tot.values()), tot


@pytest.mark.parametrize("seed", range(3))
def test_larger_geometry_matches_the_oracle(seed):
    """b = 256, w = 16, N_max = 8, M = 8 over 64 requests arriving at once
    (the shape of the decode workload, scaled down)."""
    b = 256
    rng = np.random.default_rng(seed)
    stream = [(r, int(rng.integers(64, 3000)), int(rng.integers(1, 3000)), -1, 0, 0)
              for r in range(64)]
    o, c = _pair(8 * 8 + 24, b, 16, 8, 8, 32, 16384, "hybrid")
    lockstep(o, c, stream, seed, arrivals=False, state_every=16)
    _same_state(o, c)


def test_hand_scenario_matches():
    o, c = _pair(100, 16, 4, 2, 1, 8, 1000, "hybrid")
    lockstep(o, c, [(0, 8, 5, -1, 0, 0), (1, 26, 10, -1, 0, 0)], 0, arrivals=False)


# ------------------------------------------------------------------- errors
def test_bad_configuration_and_arguments():
    with pytest.raises(zp.ZpError):
        zp.Scheduler(16, 12, 4, 2, 1, 8, 100)            # block size not a power of two
    with pytest.raises(zp.ZpError):
        zp.Scheduler(16, 16, 4, 4, 1, 8, 100, table_cap=3)
    c = zp.Scheduler(16, 16, 4, 2, 1, 8, 100, table_cap=4)
    c.add(0, 10, 5)
    with pytest.raises(zp.ZpError):
        c.add(0, 10, 5)                                  # repeated id
    with pytest.raises(zp.ZpError):
        c.add(1, 0, 5)
    with pytest.raises(zp.ZpError):
        c.add(2, 10, 5, 3, 10)                           # prefix_len must be < prompt_len
    with pytest.raises(zp.ZpError):
        c.add(4, 65, 5)                                  # 5 blocks > table_cap
    c.add(5, 30, 5, 3, 16)
    with pytest.raises(zp.ZpError):
        c.add(6, 40, 5, 3, 17)                           # one prefix length per group
    with pytest.raises(zp.ZpError):
        c.add(7, 10, 5, n_max=3)                         # above the configured N_max
    with pytest.raises(zp.ZpError):
        c.add(8, 10, 5, n_max=1)
    with pytest.raises(zp.ZpError) as e:
        c.compress_done(0)                               # not compressing
    assert e.value.status == zp.ZP_ESTATE
    assert c.request(99)["state"] == zp.ZP_REQ_UNKNOWN


def test_table_cap_overflow_is_reported():
    """Shared prefixes, table_cap = N_max = 2: two due members, the second
    finds no block for its fresh target and preempts itself; recomputed over
    33 tokens it would need three blocks. Both schedulers refuse in the same
    step (the C++ one with ZP_ESTATE)."""
    o, c = _pair(4, 16, 4, 2, 2, 8, 1000, "hybrid", prefix=True, cap=2)
    for x in (o, c):
        x.add(0, 20, 100, 1, 16)
    o.step()
    c.step()
    for x in (o, c):
        x.add(1, 20, 100, 1, 16)
    for _ in range(13):
        a = o.step()
        assert c.step().as_dict() == a
    assert a["batch"][1]["ctx"] == 31                    # both due after this step
    # step 15: request 0 takes the last block as its fresh target, request 1
    # preempts itself and its recomputation is refused
    with pytest.raises(AssertionError, match="table_cap"):
        o.step()
    with pytest.raises(zp.ZpError) as e:
        c.step()
    assert e.value.status == zp.ZP_ESTATE and "table_cap" in str(e.value)
