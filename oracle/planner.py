"""Block-level rules of Compressed PagedAttention, as plain Python.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Integer logic: the
product's C++ allocator/planner must agree with these functions exactly.

Source: "Zipage: Maintain High Request Concurrency for LLM Reasoning through
Compressed PagedAttention" (arXiv 2603.08743), Sec. 4.1 (cap and reserved
block), Sec. 4.2 eq. (1) (capacity), Sec. 4.4 (shared-prefix target blocks and
reference counts), App. C.3 eq. (2) (capacity with a global-score cache).
"""
from __future__ import annotations

from fractions import Fraction


def plan_targets(table, refcount, n_max):
    """Target blocks of one compression (Sec. 4.1 and Sec. 4.4).

    ``table`` is the request's block table (N >= n_max entries), ``refcount``
    maps a block id to its reference count; blocks with a count above one are
    shared. Shared blocks must form a prefix of the table.

    Rule: kept tokens go to N_max - 1 target blocks and the N_max-th block is
    reserved for later decoding. With N_prefix shared blocks, if
    N_prefix >= N_max - 1 all N_max - 1 targets are new blocks; otherwise the
    N_prefix shared positions get new blocks and the remaining positions reuse
    the request's own blocks. Reading (the figure that shows this is
    garbled): new blocks take the logical positions of the shared blocks,
    reused own blocks keep their own positions, and the reserved block is the
    first own block not used as a target (a new block if there is none).

    New blocks are written as the strings "new0", "new1", ... in allocation
    order. Returns dict(dst [n_max-1], new_table [n_max], n_new, release
    (own blocks that go back to the pool), decref (shared blocks that lose
    this request's reference)).
    """
    N = len(table)
    assert N >= n_max >= 2
    shared = [refcount[p] > 1 for p in table]
    n_prefix = sum(shared)
    assert all(shared[:n_prefix]) and not any(shared[n_prefix:]), \
        "shared blocks must form a prefix"
    n_new = 0
    dst = []
    for i in range(n_max - 1):
        if i < n_prefix:
            dst.append(f"new{n_new}")
            n_new += 1
        else:
            dst.append(table[i])
    own_unused = [p for i, p in enumerate(table) if not shared[i] and p not in dst]
    if own_unused:
        reserved = own_unused[0]
    else:
        reserved = f"new{n_new}"
        n_new += 1
    new_table = dst + [reserved]
    release = [p for p in own_unused if p != reserved]
    decref = [p for i, p in enumerate(table) if shared[i]]
    return dict(dst=dst, new_table=new_table, n_new=n_new, release=release,
                decref=decref)


def capacity(m_avail, m_kv, m_q, n_max, m_f=0):
    """Maximum concurrency M and block count N_total (eq. (1), eq. (2)).

    The paper's linear program: maximise M subject to
    m_blk * N_total + M * m_q <= m_avail and M <= N_total / N_max, with
    m_blk = m_kv (eq. (1)) or m_kv plus the per-block global-score bytes
    (eq. (2) writes it as (1 + 1/(2d)) m_kv when F has the KV element size;
    here the extra bytes per block are given directly as ``m_f``). The
    optimum sits on M = N_total / N_max; its closed form, floored, is
    M = floor(m_avail / (m_blk N_max + m_q)) and
    N_total = floor(m_avail / (m_blk + m_q / N_max)).
    """
    m_blk = Fraction(m_kv) + Fraction(m_f)
    M = Fraction(m_avail) / (m_blk * n_max + m_q)
    Nt = Fraction(m_avail) / (m_blk + Fraction(m_q) / n_max)
    return int(M.__floor__()), int(Nt.__floor__())
