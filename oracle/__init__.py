"""CPU oracle for Compressed PagedAttention (Zipage, arXiv 2603.08743).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, float64 NumPy statement
of what the hot path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The product library
(``compressed_paged_kv_gqa_amd``) never imports it, and it never imports the
product library: the two share no code.

Modules
-------
zipage   decode attention, window attention score, global score, pooling,
         redundancy scores (original / flash / lightning), window mask, top-k,
         compaction, and a whole compression event.
planner  block-level target rule for shared prefixes and the capacity
         formulas (Zipage paper, Sec. 4.2 eq. (1), Sec. 4.4, App. C.3 eq. (2)).
scheduler constrained and hybrid scheduling with query slots, preemption and
         shared prefixes (Sec. 4.3, Fig. 2, Sec. 4.4), as a state machine.

Parity status of each function is stated in its docstring; every function is
pinned by a ``-m "not gpu"`` test except where it says "parity unpinned".
"""
from . import zipage, planner, scheduler  # noqa: F401
