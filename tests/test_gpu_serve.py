"""GPU: the serving loop (zp_sched driving prefill, decode and compression
kernels) on seeded request streams.

Zipage (arXiv 2603.08743) Sec. 4.3 / Fig. 2 (constrained and hybrid
scheduling, preemption), Sec. 4.4 (shared prefix blocks), Sec. 4.5
(asynchronous compression), Sec. 6 (attention over the resident tokens is
ordinary softmax attention).

Every token's q, k, v come from per-position tables (a request's prefix
positions from its group's table), so the cache can be read back and each
resident row traced to the token it came from. Checks, at every step:
  - each decode / prefill output equals the oracle's softmax attention over
    the request's resident K/V read back through the step's block table
    (tolerance 1e-5 relative for fp32, 2e-2 for bf16);
  - a request never compressed holds exactly tokens
    0..n-1, one compressed holds a strictly increasing subsequence whose last
    rows (the window of its last compression and every token since) are
    consecutive; K and V rows equal the table rows of their tokens, bit for
    bit;
and at the end: every request produced max_new tokens, no device error bit.
"""
import numpy as np
import pytest
import torch

from compressed_paged_kv_gqa_amd import engine as E
from compressed_paged_kv_gqa_amd import synth, zp
from oracle import zipage as Z

from gpu_cases import announce, tol_for

pytestmark = pytest.mark.gpu


class TableModel:
    """q, k, v of every (source, position, layer) drawn once from a seed."""

    def __init__(self, geom, stream, seed):
        G = self.G = geom
        self.nreq = len(stream)
        self.P = max(p + m for _r, p, m, _g, _pl, _nm in stream) + 1
        groups = sorted({g for _r, _p, _m, g, _pl, _nm in stream if g >= 0})
        self.src_of_group = {g: self.nreq + i for i, g in enumerate(groups)}
        self.meta = {r: (g, pl) for r, _p, _m, g, pl, _nm in stream}
        self.n_max = {r: nm or geom.n_max for r, _p, _m, _g, _pl, nm in stream}
        S = self.nreq + len(groups)
        gen = synth.rng(seed, 7, 0, "serve")
        L, P = G.num_layers, self.P
        K = gen.standard_normal((L, S, P, G.num_kv_heads, G.head_dim))
        K *= np.where(gen.random((L, S, P, G.num_kv_heads)) < 0.02, 4.0, 1.0)[..., None]
        V = gen.standard_normal((L, S, P, G.num_kv_heads, G.head_dim))
        Q = gen.standard_normal((L, S, P, G.num_q_heads, G.head_dim))
        self.K = synth.cast(K, G.dtype).reshape(L, S * P, G.num_kv_heads, G.head_dim)
        self.V = synth.cast(V, G.dtype).reshape(L, S * P, G.num_kv_heads, G.head_dim)
        self.Q = synth.cast(Q, G.dtype).reshape(L, S * P, G.num_q_heads, G.head_dim)
        dt = G.torch_dtype()
        self.Kd = torch.from_numpy(self.K).to(dt).cuda()
        self.Vd = torch.from_numpy(self.V).to(dt).cuda()
        self.Qd = torch.from_numpy(self.Q).to(dt).cuda()
        self._idx = None

    def row(self, rid, pos):
        g, pl = self.meta[rid]
        src = self.src_of_group[g] if (g >= 0 and pos < pl) else rid
        return src * self.P + pos

    def rows(self, st, kind):
        """Rows of the step's tokens, by their index in the request's token
        sequence (pos), which differs from the cache position after a
        compression."""
        out = []
        for i in range(st.n):
            r, p0 = int(st.rid[i]), int(st.pos[i])
            ln = int(st.len[i]) if kind == zp.ZP_STEP_PREFILL else 1
            out += [self.row(r, p) for p in range(p0, p0 + ln)]
        return np.array(out, np.int64)

    def __call__(self, kind, st, layer):
        if layer == 0:
            self._idx = torch.from_numpy(self.rows(st, kind)).cuda()
        return (self.Qd[layer].index_select(0, self._idx), self.Kd[layer].index_select(0, self._idx),
                self.Vd[layer].index_select(0, self._idx))


def _resident(Kc, Vc, layer, h, table, n, b):
    return (Z.gather_sequence(Kc[layer, :, h], table, n, b),
            Z.gather_sequence(Vc[layer, :, h], table, n, b))


def _check_outputs(eng, model, st, kind, tol):
    G = eng.geom
    g = G.group
    Kc = eng.cache.k.float().cpu().numpy()
    Vc = eng.cache.v.float().cpu().numpy()
    worst = 0.0
    t0 = 0
    for i in range(st.n):
        r, ctx, p0 = int(st.rid[i]), int(st.ctx[i]), int(st.pos[i])
        ln = int(st.len[i]) if kind == zp.ZP_STEP_PREFILL else 1
        n = ctx + ln
        tab = st.tables[i][st.tables[i] >= 0]
        rows = sorted({0, ln - 1, ln // 2}) if kind == zp.ZP_STEP_PREFILL else [0]
        for l in range(G.num_layers):
            out = (eng.out_prefill if kind == zp.ZP_STEP_PREFILL else eng.out_decode)[l]
            for h in range(G.num_kv_heads):
                K, V = _resident(Kc, Vc, l, h, tab, n, G.block_size)
                for x in rows:
                    q = model.Q[l, model.row(r, p0 + x), h * g:(h + 1) * g]
                    ref, _ = Z.decode_attention(q, K[None, :ctx + x + 1], V[None, :ctx + x + 1])
                    got = out[t0 + x, h * g:(h + 1) * g].float().cpu().numpy()
                    err = np.abs(got - ref).max() / np.abs(ref).max()
                    worst = max(worst, err)
                    assert err <= tol, (kind, r, x, l, h, err)
        t0 += ln
    return worst


def _check_resident(eng, model, last_nmax):
    """Traces every resident K/V row of every running request back to the
    token it came from (rows are matched bit for bit against the request's
    table rows; seeded normal rows do not repeat). last_nmax: the N_max each
    request's last compression kept (N_max - 1 blocks)."""
    G = eng.geom
    b = G.block_size
    Kc = eng.cache.k.float().cpu().numpy()
    Vc = eng.cache.v.float().cpu().numpy()
    checked = 0
    for r in range(model.nreq):
        info = eng.sched.request(r)
        if info["state"] != zp.ZP_REQ_RUNNING:
            continue
        n, tab = info["n"], info["table"]
        for l in range(G.num_layers):
            for h in range(G.num_kv_heads):
                K, V = _resident(Kc, Vc, l, h, tab, n, b)
                assert np.isfinite(K).all() and np.isfinite(V).all(), (r, l, h, "non-finite rows")
                idx = np.array([model.row(r, p) for p in range(model.P)])
                where = {model.K[l, i, h].tobytes(): p for p, i in enumerate(idx)}
                pos = np.array([where.get(k.astype(np.float32).tobytes(), -1) for k in K])
                assert (pos >= 0).all(), (r, l, h, "resident K row from nowhere", np.where(pos < 0))
                if not info["compressed"]:
                    np.testing.assert_array_equal(pos, np.arange(n))
                else:
                    # kept rows in token order; the window of the last
                    # compression and every token since are consecutive
                    assert np.all(np.diff(pos) > 0)
                    tail = pos[(last_nmax[r] - 1) * b - G.window:]
                    np.testing.assert_array_equal(tail, np.arange(tail[0], tail[0] + len(tail)))
                np.testing.assert_array_equal(V, model.V[l, idx[pos], h])
        checked += 1
    return checked


def _stream(seed, n, b, prefix, nmax_choices=None):
    rng = np.random.default_rng(seed)
    out = []
    for r in range(n):
        p = int(rng.integers(5, 4 * b))
        m = int(rng.integers(8, 6 * b))
        g, pl = -1, 0
        if prefix and rng.random() < 0.6 and p > 20:
            g, pl = 0, 20
        nm = int(rng.choice(nmax_choices)) if nmax_choices else 0
        out.append((r, p, m, g, pl, nm))
    return out


CASES = [
    # dtype, policy, prefix, blocks, async, per-request N_max choices (0 = the
    # geometry's), geometry N_max, adaptive N_max growth step (tokens, 0 = off);
    # a request arrives every third step
    ("f32", "hybrid", True, 14, True, None, 3, 0),
    ("f32", "hybrid", True, 11, False, None, 3, 0),
    ("f32", "hybrid", False, 11, True, None, 3, 0),
    ("f32", "constrained", True, 12, True, None, 3, 0),
    ("f32", "constrained", False, 9, False, None, 3, 0),
    ("bf16", "hybrid", True, 14, True, None, 3, 0),
    ("f32", "hybrid", True, 12, True, [2, 0], 3, 0),
    ("bf16", "constrained", False, 8, True, [2, 0], 3, 0),
    ("f32", "hybrid", True, 14, True, [2], 4, 24),
    ("bf16", "constrained", False, 12, True, [2], 4, 24),
]


@pytest.mark.parametrize("case", CASES, ids=[
    f"{c[0]}-{c[1]}-{'prefix' if c[2] else 'noprefix'}-nb{c[3]}{'-nmax' if c[5] else ''}"
    f"{'-grow' if c[7] else ''}" for c in CASES])
def test_serving_loop(case):
    dtype, policy, prefix, nblocks, async_c, nmax_choices, nmax, growth = case
    b, M = 16, 3
    announce(f"serve dtype={dtype} policy={policy} prefix={prefix} blocks={nblocks} "
             f"async={async_c} nmax={nmax_choices} cap={nmax} growth={growth}")
    geom = zp.CacheGeometry(num_layers=2, num_blocks=nblocks, block_size=b, num_kv_heads=2,
                            num_q_heads=4, head_dim=64, window=8, max_slots=M, n_max=nmax,
                            dtype=dtype)
    stream = _stream(11, 14, b, prefix, nmax_choices)
    model = TableModel(geom, stream, 3)
    eng = E.ServingEngine(geom, zp.ScoreParams(), max_running=8, table_cap=24,
                          max_prefill_tokens=128, policy=policy, prefix_sharing=prefix,
                          layer_stride=1, async_compress=async_c, keep_layer_outputs=True,
                          nmax_growth=growth)
    last_nmax = {}
    kept_caps = set()
    tol = tol_for(dtype)
    worst, kinds = 0.0, {}
    n = added = 0
    while eng.unfinished() > 0 or added < len(stream):
        if n % 3 == 0 and added < len(stream):
            eng.add(*stream[added])
            added += 1
        st = eng.step(model)
        n += 1
        assert n < 5000
        for i in range(st.n_comp):
            last_nmax[int(st.c_rid[i])] = int(st.c_nmax[i])
            kept_caps.add(int(st.c_nmax[i]))
        torch.cuda.synchronize()
        kinds[st.kind] = kinds.get(st.kind, 0) + 1
        if st.kind in (zp.ZP_STEP_PREFILL, zp.ZP_STEP_DECODE):
            try:
                worst = max(worst, _check_outputs(eng, model, st, st.kind, tol))
            except AssertionError:
                print(f"[serve] step {n} kind {st.kind} rids {st.rid.tolist()} "
                      f"ctx {st.ctx.tolist()} pos {st.pos.tolist()} errors {eng.device_errors()}")
                _check_resident(eng, model, last_nmax)
                raise
        # running requests only: in-flight compactions touch none of their blocks
        _check_resident(eng, model, last_nmax)
    eng.poll(wait=True)
    torch.cuda.synchronize()
    assert eng.device_errors() == 0
    stats = eng.sched.stats()
    assert stats["finished"] == len(stream)
    assert eng.generated == sum(x[2] for x in stream)
    assert stats["compressions"] > 0
    if policy == "constrained" and not prefix:
        assert stats["preemptions"] == 0
    if growth:
        # the caps grew with the sequences: compressions kept more than N_base
        assert max(kept_caps) > 2, kept_caps
    print(f"[serve] steps={n} kinds={kinds} worst={worst:.3g} stats={stats}")
