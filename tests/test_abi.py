"""CPU tests of the C ABI: the library loads and exports every declared
symbol, host-side validation rejects bad calls before touching the GPU, and the
host block allocator / compression planner / capacity helper agree with the
oracle's integer rules (Zipage Sec. 4.1, Sec. 4.2 eq. (1), Sec. 4.4,
App. C.3 eq. (2)). No GPU work is launched here.
"""
import ctypes as C
import itertools
import random

import pytest

from compressed_paged_kv_gqa_amd import zp
from oracle import planner as PL


def test_library_exports_every_header_symbol():
    names = zp.header_symbols()
    assert len(names) >= 20
    lib = C.CDLL(zp.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert zp.lib().zp_version().decode().startswith("zp")


def _geom(**kw):
    g = dict(num_layers=1, num_blocks=16, block_size=16, num_kv_heads=1, num_q_heads=4,
             head_dim=64, window=8, max_slots=1, n_max=4, dtype="f32")
    g.update(kw)
    return zp.CacheGeometry(**g)


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(block_size=24), dict(block_size=512),
                                 dict(num_q_heads=6), dict(window=0), dict(window=3),
                                 dict(n_max=1), dict(num_q_heads=12, num_kv_heads=4)])
def test_bad_geometry_is_rejected_on_the_host(bad):
    g = _geom(**bad).c()
    cache = zp.Cache(1, 1, 1, None)   # never dereferenced: validation fails first
    st = zp.lib().zp_paged_decode(C.byref(g), C.byref(cache), 0, 1, 1, 1, 1, 1, 1, 1, 16, None,
                                  1, None, 1, 1 << 20, None)
    assert st == zp.ZP_EINVAL
    assert zp.lib().zp_last_error().decode()
    assert zp.lib().zp_decode_workspace_size(C.byref(g), 1, 16) == 0


@pytest.mark.parametrize("batch,split", [(64, False), (96, False), (97, True), (107, True),
                                         (108, False), (128, False), (256, False)])
def test_decode_launch_splits_only_just_past_one_round(batch, split):
    """At the Qwen3-8B decode shape (3 resident 4-wavefront workgroups per
    CU, 768 in all) a batch whose (sequence, kv-head) items fill more than
    one round but at most 1.125 rounds is split in two (the split partials
    then need workspace); below one round and from 108 sequences on it is
    not."""
    g = _geom(num_layers=36, num_blocks=4096, block_size=256, num_kv_heads=8, num_q_heads=32,
              head_dim=128, window=16, max_slots=batch, n_max=8, dtype="bf16").c()
    need = zp.lib().zp_decode_workspace_size(C.byref(g), batch, 2048)
    assert (need > 256) == split


def test_short_workspace_and_null_buffers_are_rejected():
    g = _geom().c()
    cache = zp.Cache(1, 1, 1, None)
    need = zp.lib().zp_decode_workspace_size(C.byref(g), 2, 3000)
    assert need > 256                       # split partials of long rows
    st = zp.lib().zp_paged_decode(C.byref(g), C.byref(cache), 0, 2, 1, 1, 1, 1, 1, 1, 3000, None,
                                  1, None, 1, need - 1, None)
    assert st == zp.ZP_EINVAL and "workspace" in zp.lib().zp_last_error().decode()
    st = zp.lib().zp_paged_decode(C.byref(g), C.byref(cache), 3, 2, 1, 1, 1, 1, 1, 1, 3000, None,
                                  1, None, 1, need, None)
    assert st == zp.ZP_EINVAL  # layer out of range
    sp = zp.ScoreParams(tau=0.0).c()
    st = zp.lib().zp_score_tokens(C.byref(g), C.byref(cache), C.byref(sp), 0, 1, 1, 1, 4, 1, 4, 1,
                                  1, None, 1, None, 64, 1, 1 << 20, None)
    assert st == zp.ZP_EINVAL  # global flag without F, or tau = 0
    st = zp.lib().zp_select_compact(C.byref(g), C.byref(cache), 0, 1, 1, 1, None, 64, 1, 4, 1, 4,
                                    1, 4, 0, None, 0, 1, 256, None)
    assert st == zp.ZP_EINVAL  # keep = 0


def test_score_redundancy_variant_is_validated():
    assert zp.ScoreParams(redundancy="flash").c().flags & zp.ZP_SCORE_REDUNDANCY_FLASH
    assert not zp.ScoreParams().c().flags & zp.ZP_SCORE_REDUNDANCY_FLASH
    with pytest.raises(ValueError):
        zp.ScoreParams(redundancy="original").c()


def test_score_global_reduce_is_validated():
    assert zp.ScoreParams(global_reduce="sum").c().flags & zp.ZP_SCORE_GLOBAL_SUM
    assert not zp.ScoreParams().c().flags & zp.ZP_SCORE_GLOBAL_SUM
    # no history, no reduce: the sum flag is only set with the global score
    assert not zp.ScoreParams(global_reduce="sum", use_global=False).c().flags & zp.ZP_SCORE_GLOBAL_SUM
    with pytest.raises(ValueError):
        zp.ScoreParams(global_reduce="mean").c()
    # the C ABI refuses the sum flag without the global score (host-side,
    # before anything is enqueued)
    g = _geom().c()
    cache = zp.Cache(1, 1, 1, None)
    sp = zp.ScoreParams(use_global=False).c()
    sp.flags |= zp.ZP_SCORE_GLOBAL_SUM
    st = zp.lib().zp_score_tokens(C.byref(g), C.byref(cache), C.byref(sp), 0, 1, 1, 1, 4, 1, 4, 1,
                                  1, None, 1, None, 64, 1, 1 << 20, None)
    assert st == zp.ZP_EINVAL and "GLOBAL_SUM" in zp.lib().zp_last_error().decode()


def test_score_window_lse_all_needs_the_lse_table():
    # the flag promises every window row's log-sum-exp: refused on the host
    # when the cache has no log-sum-exp table, and unknown bits stay refused
    g = _geom().c()
    cache = zp.Cache(1, 1, 1, None, None)
    sp = zp.ScoreParams(use_global=False).c()
    sp.flags |= zp.ZP_SCORE_WINDOW_LSE_ALL
    st = zp.lib().zp_score_tokens(C.byref(g), C.byref(cache), C.byref(sp), 0, 1, 1, 1, 4, 1, 4, 1,
                                  1, None, 1, None, 64, 1, 1 << 20, None)
    assert st == zp.ZP_EINVAL and "WINDOW_LSE_ALL" in zp.lib().zp_last_error().decode()
    sp.flags = zp.ZP_SCORE_WINDOW_LSE_ALL << 1
    st = zp.lib().zp_score_tokens(C.byref(g), C.byref(cache), C.byref(sp), 0, 1, 1, 1, 4, 1, 4, 1,
                                  1, None, 1, None, 64, 1, 1 << 20, None)
    assert st == zp.ZP_EINVAL and "unknown flags" in zp.lib().zp_last_error().decode()


# --- allocator ------------------------------------------------------------

def test_alloc_all_or_nothing_and_conservation():
    a = zp.BlockAllocator(10)
    x = a.alloc(4)
    assert x == [0, 1, 2, 3] and a.num_free == 6
    with pytest.raises(zp.NoBlocks):
        a.alloc(7)
    assert a.num_free == 6                          # unchanged
    a.share(x[:2])
    assert [a.refcount(i) for i in x] == [2, 2, 1, 1]
    a.free(x)
    assert [a.refcount(i) for i in x] == [1, 1, 0, 0] and a.num_free == 8
    with pytest.raises(zp.ZpError) as e:
        a.free([2])                                 # double free
    assert e.value.status == zp.ZP_ESTATE and a.num_free == 8
    with pytest.raises(zp.ZpError) as e:
        a.free([0, 0])                              # would underflow: state unchanged
    assert e.value.status == zp.ZP_ESTATE and a.refcount(0) == 1
    assert a.alloc(2) == [2, 3]                     # lowest ids first
    assert a.refcount(99) == -1


def _map_plan(oracle_plan, fresh):
    """Replaces the oracle's symbolic new blocks by allocator ids."""
    m = {f"new{i}": f for i, f in enumerate(fresh)}
    f = lambda xs: [m.get(x, x) for x in xs]
    return f(oracle_plan["dst"]), f(oracle_plan["new_table"])


@pytest.mark.parametrize("n_blocks,n_prefix,n_max", [
    (8, 0, 8), (10, 0, 8), (13, 0, 4), (8, 4, 8), (8, 7, 8), (9, 8, 8), (4, 4, 4), (6, 5, 4)])
def test_planner_matches_oracle_and_commit_releases(n_blocks, n_prefix, n_max):
    total = 64
    a = zp.BlockAllocator(total)
    prefix = a.alloc(n_prefix) if n_prefix else []
    a.share(prefix)                                  # another request holds them too
    own = a.alloc(n_blocks - n_prefix)
    table = prefix + own
    rc = {p: a.refcount(p) for p in table}
    ref = PL.plan_targets(table, rc, n_max)
    free_before = a.num_free
    dst, new, rel = a.plan_compress(table, n_max)
    fresh = [p for p in new if p not in table]
    assert len(fresh) == ref["n_new"] and a.num_free == free_before - ref["n_new"]
    assert (dst, new) == _map_plan(ref, sorted(fresh))
    assert rel == ref["release"]
    # in-place safety: each target is the source block at that position or fresh
    for i, p in enumerate(dst):
        assert p == table[i] or p not in table
    a.commit_compress(table, new)
    for p in ref["decref"]:
        assert a.refcount(p) == rc[p] - 1            # shared blocks drop by one
    for p in rel:
        assert a.refcount(p) == 0
    for p in new:
        assert a.refcount(p) == 1
    held = sum(a.refcount(i) for i in range(total))
    assert a.num_free + len([i for i in range(total) if a.refcount(i) > 0]) == total
    assert held >= len(new)


def test_plan_without_free_blocks_changes_nothing_and_abort_frees():
    a = zp.BlockAllocator(9)
    table = a.alloc(8)
    a.share(table[:4])
    assert a.num_free == 1
    before = [a.refcount(i) for i in range(9)]
    with pytest.raises(zp.NoBlocks):
        a.plan_compress(table, 8)                    # needs 4 fresh blocks
    assert [a.refcount(i) for i in range(9)] == before
    b = zp.BlockAllocator(20)
    t = b.alloc(8)
    b.share(t[:2])
    dst, new, rel = b.plan_compress(t, 8)
    b.abort_compress(t, new)
    assert b.num_free == 12 and [b.refcount(p) for p in t[:2]] == [2, 2]


def test_plan_rejects_non_prefix_sharing_and_bad_tables():
    a = zp.BlockAllocator(20)
    t = a.alloc(8)
    a.share([t[3]])
    with pytest.raises(zp.ZpError) as e:
        a.plan_compress(t, 8)
    assert e.value.status == zp.ZP_EINVAL
    with pytest.raises(zp.ZpError):
        a.plan_compress(t[:5], 8)                    # fewer than n_max blocks
    with pytest.raises(zp.ZpError):
        a.plan_compress([t[0], t[0]] + t[2:], 8)     # repeated block


def test_random_allocator_sequences_conserve_blocks():
    rng = random.Random(0)
    a = zp.BlockAllocator(50)
    held = {}
    for _ in range(400):
        op = rng.random()
        if op < 0.4:
            n = rng.randint(0, 6)
            try:
                for i in a.alloc(n):
                    held[i] = held.get(i, 0) + 1
            except zp.NoBlocks:
                assert a.num_free < n
        elif op < 0.6 and held:
            i = rng.choice(list(held))
            a.share([i])
            held[i] += 1
        elif held:
            i = rng.choice(list(held))
            a.free([i])
            held[i] -= 1
            if held[i] == 0:
                del held[i]
        assert all(a.refcount(i) == held.get(i, 0) for i in range(50))
        assert a.num_free == 50 - len(held)


@pytest.mark.parametrize("m_avail,m_kv,m_f,m_q,n_max", [
    (1000, 10, 0, 5, 4), (124, 10, 0, 5, 2), (97, 3, 0, 7, 8), (5000, 64, 1, 3, 8),
    (10, 20, 0, 1, 4), (999, 7, 2, 0, 3),
    (288 * 2**30, 2 * 256 * 8 * 128 * 2 * 36, 256 * 8 * 4 * 36, 16 * 32 * 128 * 2 * 36, 8)])
def test_capacity_matches_oracle(m_avail, m_kv, m_f, m_q, n_max):
    assert zp.zp_capacity(m_avail, m_kv, m_f, m_q, n_max) == PL.capacity(m_avail, m_kv, m_q,
                                                                         n_max, m_f)
