"""ctypes binding of libzp (the C ABI declared in include/zp.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels. Functions keep the C names and take torch tensors for device
buffers (PyTorch provides device memory and streams, nothing else). The
library must be built (``python -m compressed_paged_kv_gqa_amd._build``);
importing the binding without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzp.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "zp.h")

ZP_OK, ZP_EINVAL, ZP_ENOBLOCKS, ZP_EHIP, ZP_ESTATE = 0, -1, -2, -3, -4
ZP_DTYPE_F32, ZP_DTYPE_BF16 = 0, 1
ZP_DEVERR_BLOCK_ID, ZP_DEVERR_SEQ_LEN, ZP_DEVERR_SLOT, ZP_DEVERR_KEEP = 1, 2, 4, 8
ZP_SCORE_GLOBAL, ZP_SCORE_POOL, ZP_SCORE_POOL_FIRST_ONLY, ZP_SCORE_REDUNDANCY = 1, 2, 4, 8
ZP_SCORE_REDUNDANCY_FLASH = 0x10
ZP_SCORE_GLOBAL_SUM = 0x20
ZP_SCORE_WINDOW_LSE_ALL = 0x40
ZP_SELECT_NO_COMPACT = 1


class ZpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"zp status {status}: {msg}")
        self.status = status


class NoBlocks(ZpError):
    pass


class Geom(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "num_layers", "num_blocks", "block_size", "num_kv_heads", "num_q_heads",
        "head_dim", "window", "max_slots", "n_max", "dtype")]


class Cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("qwin", C.c_void_p),
                ("gscore", C.c_void_p), ("qwin_lse", C.c_void_p)]


class ScoreParamsC(C.Structure):
    _fields_ = [("alpha", C.c_float), ("lambda_", C.c_float), ("tau", C.c_float),
                ("sim_threshold", C.c_float), ("pool_kernel", C.c_int32),
                ("flags", C.c_uint32)]


ZP_SCHED_CONSTRAINED, ZP_SCHED_HYBRID = 0, 1
ZP_STEP_IDLE, ZP_STEP_PREFILL, ZP_STEP_DECODE = 0, 1, 2
ZP_REQ_WAITING, ZP_REQ_RUNNING, ZP_REQ_COMPRESSING, ZP_REQ_FINISHED, ZP_REQ_UNKNOWN = 0, 1, 2, 3, -1


class SchedConfig(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "num_blocks", "block_size", "window", "n_max", "num_slots", "max_running",
        "max_prefill_tokens", "table_cap", "policy", "prefix_sharing", "nmax_growth")]


_OUT_ARRAYS = ("rid", "slot", "ctx", "pos", "len", "tables", "c_rid", "c_slot", "c_first",
               "c_nblocks", "c_nmax", "c_src", "c_dst", "c_new", "finished", "preempted")
_OUT_COUNTS = ("kind", "n", "n_comp", "n_finished", "n_preempted", "n_blocked")


class SchedStepOut(C.Structure):
    _fields_ = ([(n, C.POINTER(C.c_int32)) for n in _OUT_ARRAYS] +
                [(n, C.c_int32) for n in _OUT_COUNTS])


class SchedStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "steps", "prefill_steps", "decode_steps", "idle_steps", "waiting", "running",
        "compressing", "finished", "free_blocks", "slots_in_use", "prefill_tokens",
        "decode_tokens", "compressions", "preemptions", "blocked")]


class SchedReqInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("state", "n", "gen", "slot", "compressed", "ntable",
                                         "n_max")]


_lib = None
_P = C.c_void_p
_I32P = C.POINTER(C.c_int32)


def _declare(lib):
    g, c, sp = C.POINTER(Geom), C.POINTER(Cache), C.POINTER(ScoreParamsC)
    i32, i64, sz, u32 = C.c_int32, C.c_int64, C.c_size_t, C.c_uint32
    sigs = {
        "zp_last_error": (C.c_char_p, []),
        "zp_version": (C.c_char_p, []),
        "zp_decode_workspace_size": (sz, [g, i32, i32]),
        "zp_paged_decode": (C.c_int, [g, c, i32, i32, _P, _P, _P, _P, i32, _P, i32, _P, _P,
                                      _P, _P, sz, _P]),
        "zp_paged_decode_noalloc": (C.c_int, [g, c, i32, i32, _P, _P, _P, _P, i32, _P, i32, _P,
                                              _P, _P, _P, _P]),
        "zp_prefill_workspace_size": (sz, [g, i32]),
        "zp_paged_prefill": (C.c_int, [g, c, i32, i32, _P, _P, _P, _P, _P, i32, _P, i32, _P, _P,
                                       _P, _P, sz, _P]),
        "zp_score_workspace_size": (sz, [g, i32, i32, i32]),
        "zp_score_tokens": (C.c_int, [g, c, sp, i32, i32, i32, _P, i32, _P, i32, _P, _P, _P,
                                      _P, _P, i64, _P, sz, _P]),
        "zp_select_workspace_size": (sz, [g, i32, i32, i32]),
        "zp_select_compact": (C.c_int, [g, c, i32, i32, i32, _P, _P, i64, _P, i32, _P, i32, _P,
                                        i32, i32, _P, u32, _P, sz, _P]),
        "zp_workspace_errors": (C.c_int, [_P, C.POINTER(C.c_uint32), _P]),
        "zp_workspace_clear_errors": (C.c_int, [_P, _P]),
        "zp_alloc_create": (_P, [i32]),
        "zp_alloc_destroy": (None, [_P]),
        "zp_block_alloc": (C.c_int, [_P, i32, _I32P]),
        "zp_block_free": (C.c_int, [_P, _I32P, i32]),
        "zp_block_share": (C.c_int, [_P, _I32P, i32]),
        "zp_block_refcount": (i32, [_P, i32]),
        "zp_num_free": (i32, [_P]),
        "zp_num_blocks": (i32, [_P]),
        "zp_plan_compress": (C.c_int, [_P, _I32P, i32, i32, _I32P, _I32P, _I32P, _I32P]),
        "zp_commit_compress": (C.c_int, [_P, _I32P, i32, _I32P, i32]),
        "zp_abort_compress": (C.c_int, [_P, _I32P, i32, _I32P, i32]),
        "zp_capacity": (C.c_int, [i64, i64, i64, i64, i32, C.POINTER(i64), C.POINTER(i64)]),
        "zp_sched_create": (_P, [C.POINTER(SchedConfig)]),
        "zp_sched_destroy": (None, [_P]),
        "zp_sched_add": (C.c_int, [_P, i32, i32, i32, i32, i32, i32]),
        "zp_sched_step": (C.c_int, [_P, C.POINTER(SchedStepOut)]),
        "zp_sched_compress_done": (C.c_int, [_P, i32]),
        "zp_sched_get_stats": (C.c_int, [_P, C.POINTER(SchedStats)]),
        "zp_sched_request": (C.c_int, [_P, i32, C.POINTER(SchedReqInfo), _P]),
        "zp_sched_unfinished": (i32, [_P]),
        "zp_sched_allocator": (_P, [_P]),
    }
    host_only = bool(os.environ.get("ZP_LIBRARY"))
    for name, (res, args) in sigs.items():
        if host_only and not hasattr(lib, name):
            continue          # a host-only build (see lib()) has no GPU entry points
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def lib():
    """The loaded libzp (raises ImportError if it has not been built).

    The environment variable ZP_LIBRARY names another build to load instead,
    for instance a host-only sanitizer build of the allocator, planner and
    scheduler (tests); its missing GPU entry points are left undeclared."""
    global _lib
    if _lib is None:
        path = os.environ.get("ZP_LIBRARY") or LIB_PATH
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with "
                "`python -m compressed_paged_kv_gqa_amd._build` (there is no fallback path)")
        _lib = _declare(C.CDLL(path))
    return _lib


def header_symbols():
    """Function names declared in include/zp.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zp_[a-z0-9_]+)\s*\(", text)))


def _check(status, what=""):
    if status == ZP_OK:
        return
    msg = lib().zp_last_error().decode()
    if status == ZP_ENOBLOCKS:
        raise NoBlocks(status, msg)
    raise ZpError(status, f"{what}: {msg}" if what else msg)


# --------------------------------------------------------------------------
# Geometry and caches
# --------------------------------------------------------------------------

@dataclass
class CacheGeometry:
    num_layers: int
    num_blocks: int
    block_size: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    window: int
    max_slots: int
    n_max: int
    dtype: str = "bf16"        # "bf16" or "f32"

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def keep(self):
        """Tokens kept per compression, k = (N_max - 1) b."""
        return (self.n_max - 1) * self.block_size

    def c(self):
        return Geom(self.num_layers, self.num_blocks, self.block_size, self.num_kv_heads,
                    self.num_q_heads, self.head_dim, self.window, self.max_slots, self.n_max,
                    ZP_DTYPE_BF16 if self.dtype == "bf16" else ZP_DTYPE_F32)

    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


class PagedKVCache:
    """Device buffers of K, V, the window query cache and the global-score
    cache F, in the layouts include/zp.h documents. Allocated with torch."""

    def __init__(self, geom: CacheGeometry, device="cuda", with_global=True, init=None,
                 with_window_lse=False):
        import torch
        self.geom = geom
        dt = geom.torch_dtype()
        G = geom
        shape = (G.num_layers, G.num_blocks, G.num_kv_heads, G.block_size, G.head_dim)
        alloc = torch.zeros if init == "zeros" else torch.empty
        self.k = alloc(shape, dtype=dt, device=device)
        self.v = alloc(shape, dtype=dt, device=device)
        self.qwin = alloc((G.num_layers, max(G.max_slots, 1), G.num_kv_heads, G.group,
                           G.window, G.head_dim), dtype=dt, device=device)
        self.gscore = (alloc((G.num_layers, G.num_blocks, G.num_kv_heads, G.block_size),
                             dtype=torch.float32, device=device) if with_global else None)
        self.qwin_lse = (torch.zeros((G.num_layers, max(G.max_slots, 1), G.num_kv_heads, G.group,
                                      G.window), dtype=torch.float32, device=device)
                         if with_window_lse else None)

    def c(self):
        return Cache(self.k.data_ptr(), self.v.data_ptr(), self.qwin.data_ptr(),
                     self.gscore.data_ptr() if self.gscore is not None else None,
                     self.qwin_lse.data_ptr() if self.qwin_lse is not None else None)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, dtype, name, device=True):
    import torch
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")


# --------------------------------------------------------------------------
# GPU entry points
# --------------------------------------------------------------------------

def zp_decode_workspace_size(geom: CacheGeometry, batch, max_seq_len):
    return lib().zp_decode_workspace_size(C.byref(geom.c()), batch, max_seq_len)


def zp_score_workspace_size(geom: CacheGeometry, layer_count, nreq, max_blocks):
    return lib().zp_score_workspace_size(C.byref(geom.c()), layer_count, nreq, max_blocks)


def zp_select_workspace_size(geom: CacheGeometry, layer_count, nreq, keep):
    return lib().zp_select_workspace_size(C.byref(geom.c()), layer_count, nreq, int(keep))


def new_workspace(nbytes, device="cuda"):
    """A zero-filled device workspace (uint8), as the ABI expects on first use."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def zp_paged_decode(cache: PagedKVCache, layer, q, k_new, v_new, block_tables, seq_lens,
                    max_seq_len, qslot, out, lse, workspace, stream=None):
    import torch
    geom = cache.geom
    dt = geom.torch_dtype()
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(qslot, torch.int32, "qslot")
    _need(lse, torch.float32, "lse")
    batch, hq, hkv, d = q.shape[0], geom.num_q_heads, geom.num_kv_heads, geom.head_dim
    for t, n, h in ((q, "q", hq), (out, "out", hq), (k_new, "k_new", hkv), (v_new, "v_new", hkv)):
        if tuple(t.shape) != (batch, h, d) or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous [{batch}][{h}][{d}] tensor, got {tuple(t.shape)}")
    if block_tables.shape[0] < batch or seq_lens.shape[0] < batch or (
            qslot is not None and qslot.shape[0] < batch):
        raise ValueError("block_tables, seq_lens and qslot need a row per batch entry")
    if lse is not None and (tuple(lse.shape) != (batch, hq) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous [{batch}][{hq}] tensor")
    _check(lib().zp_paged_decode(
        C.byref(geom.c()), C.byref(cache.c()), layer, batch, q.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(),
        int(max_seq_len), _ptr(qslot), out.data_ptr(), _ptr(lse), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)), "zp_paged_decode")


ZP_DECODE_SCRATCH_BYTES = 16 * 1024 * 1024


def zp_paged_decode_noalloc(cache: PagedKVCache, layer, q, k_new, v_new, block_tables, seq_lens,
                            max_seq_len, qslot, out, lse, errors=None, stream=None):
    """zp_paged_decode with the library's static scratch instead of a
    workspace; `errors` is an optional zero-filled int32/uint32 device
    tensor of one element that collects the device error bits."""
    import torch
    geom = cache.geom
    dt = geom.torch_dtype()
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(qslot, torch.int32, "qslot")
    _need(lse, torch.float32, "lse")
    if errors is not None and (errors.dtype not in (torch.int32, torch.uint32)
                               or errors.numel() < 1 or errors.device.type != "cuda"):
        raise ValueError("errors must be a device tensor of one 32-bit integer")
    batch, hq, hkv, d = q.shape[0], geom.num_q_heads, geom.num_kv_heads, geom.head_dim
    for t, n, h in ((q, "q", hq), (out, "out", hq), (k_new, "k_new", hkv), (v_new, "v_new", hkv)):
        if tuple(t.shape) != (batch, h, d) or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous [{batch}][{h}][{d}] tensor, got {tuple(t.shape)}")
    if block_tables.shape[0] < batch or seq_lens.shape[0] < batch or (
            qslot is not None and qslot.shape[0] < batch):
        raise ValueError("block_tables, seq_lens and qslot need a row per batch entry")
    if lse is not None and (tuple(lse.shape) != (batch, hq) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous [{batch}][{hq}] tensor")
    _check(lib().zp_paged_decode_noalloc(
        C.byref(geom.c()), C.byref(cache.c()), layer, batch, q.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(),
        int(max_seq_len), _ptr(qslot), out.data_ptr(), _ptr(lse), _ptr(errors), _stream(stream)),
        "zp_paged_decode_noalloc")


class LayerCalls:
    """zp_paged_decode / zp_paged_prefill for every layer of one step, with
    the per-step arguments (tables, lengths, slots, workspace, stream)
    validated and converted once. Each layer then passes only its q / k / v /
    out tensors, checked for shape and dtype against the first layer's.
    Argument marshalling only, as the functions above."""

    def __init__(self, cache: PagedKVCache, kind, block_tables, lens, workspace, qslot=None,
                 max_seq_len=None, cu_seqlens=None, max_q_len=None, stream=None):
        import torch
        geom = cache.geom
        self._g = geom.c()
        self._c = cache.c()
        self._gp, self._cp = C.byref(self._g), C.byref(self._c)
        self._dt = geom.torch_dtype()
        self._hq, self._hkv, self._d = geom.num_q_heads, geom.num_kv_heads, geom.head_dim
        for t, n in ((block_tables, "block_tables"), (lens, "lens"), (qslot, "qslot"),
                     (cu_seqlens, "cu_seqlens")):
            _need(t, torch.int32, n)
        _need(workspace, torch.uint8, "workspace")
        self._ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size())
        self._st = _stream(stream)
        self._tab, self._stride = block_tables.data_ptr(), block_tables.shape[1]
        self._lens, self._slot = lens.data_ptr(), _ptr(qslot)
        if kind == "decode":
            self._n = block_tables.shape[0]
            if lens.shape[0] < self._n or (qslot is not None and qslot.shape[0] < self._n):
                raise ValueError("lens and qslot need a row per batch entry")
            self._max = int(max_seq_len)
            self._fn = lib().zp_paged_decode
        elif kind == "prefill":
            self._n = lens.shape[0]
            if cu_seqlens is None or cu_seqlens.shape[0] != self._n + 1:
                raise ValueError("cu_seqlens must hold nreq + 1 offsets")
            if block_tables.shape[0] != self._n:
                raise ValueError("block_tables needs a row per chunk")
            self._cu, self._mq = cu_seqlens.data_ptr(), int(max_q_len)
            self._fn = lib().zp_paged_prefill
        else:
            raise ValueError(kind)
        self.kind = kind
        self._T = None
        self._f32 = torch.float32

    def _check_rows(self, q, k, v, out, lse):
        T = q.shape[0]
        if self._T is None:
            for t, n, h in ((q, "q", self._hq), (out, "out", self._hq), (k, "k_new", self._hkv),
                            (v, "v_new", self._hkv)):
                if (tuple(t.shape) != (T, h, self._d) or not t.is_contiguous()
                        or t.dtype != self._dt or t.device.type != "cuda"):
                    raise ValueError(f"{n} must be a contiguous [{T}][{h}][{self._d}] "
                                     f"{self._dt} device tensor")
            if self.kind == "decode" and T != self._n:
                raise ValueError("q must hold one row per batch entry")
            self._T = T
            self._shapes = (q.shape, k.shape, out.shape)
        elif (q.shape, k.shape, out.shape) != self._shapes or v.shape != k.shape or \
                q.dtype != self._dt or k.dtype != self._dt or v.dtype != self._dt or \
                out.dtype != self._dt or not (q.is_contiguous() and k.is_contiguous() and
                                              v.is_contiguous() and out.is_contiguous()):
            raise ValueError("every layer's tensors must match the first layer's")
        if lse is not None and (tuple(lse.shape) != (T, self._hq) or lse.dtype != self._f32
                                or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous [T][h_q] float32 tensor")

    def __call__(self, layer, q, k, v, out, lse=None):
        self._check_rows(q, k, v, out, lse)
        if self.kind == "decode":
            st = self._fn(self._gp, self._cp, layer, self._n, q.data_ptr(), k.data_ptr(),
                          v.data_ptr(), self._tab, self._stride, self._lens, self._max, self._slot,
                          out.data_ptr(), _ptr(lse), self._ws[0], self._ws[1], self._st)
        else:
            st = self._fn(self._gp, self._cp, layer, self._n, q.data_ptr(), k.data_ptr(),
                          v.data_ptr(), self._cu, self._lens, self._mq, self._tab, self._stride,
                          self._slot, out.data_ptr(), _ptr(lse), self._ws[0], self._ws[1],
                          self._st)
        _check(st, "zp_paged_" + self.kind)


def zp_prefill_workspace_size(geom: CacheGeometry, nreq):
    return lib().zp_prefill_workspace_size(C.byref(geom.c()), nreq)


def zp_paged_prefill(cache: PagedKVCache, layer, q, k_new, v_new, cu_seqlens, ctx_lens,
                     max_q_len, block_tables, qslot, out, lse, workspace, stream=None):
    """q/out [T][h_q][d], k_new/v_new [T][h_kv][d]; cu_seqlens [nreq+1],
    ctx_lens [nreq], block_tables [nreq][stride] int32 device tensors."""
    import torch
    geom = cache.geom
    dt = geom.torch_dtype()
    for t, n in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (out, "out")):
        _need(t, dt, n)
    for t, n in ((cu_seqlens, "cu_seqlens"), (ctx_lens, "ctx_lens"),
                 (block_tables, "block_tables"), (qslot, "qslot")):
        _need(t, torch.int32, n)
    _need(lse, torch.float32, "lse")
    nreq = ctx_lens.shape[0]
    if cu_seqlens.shape[0] != nreq + 1:
        raise ValueError("cu_seqlens must hold nreq + 1 offsets")
    T, hq, hkv, d = q.shape[0], geom.num_q_heads, geom.num_kv_heads, geom.head_dim
    # the kernels take cu_seqlens[nreq] == T on trust: the buffers must agree
    for t, n, h in ((q, "q", hq), (out, "out", hq), (k_new, "k_new", hkv), (v_new, "v_new", hkv)):
        if tuple(t.shape) != (T, h, d) or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous [{T}][{h}][{d}] tensor, got {tuple(t.shape)}")
    if lse is not None and (tuple(lse.shape) != (T, hq) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous [{T}][{hq}] tensor")
    _check(lib().zp_paged_prefill(
        C.byref(geom.c()), C.byref(cache.c()), layer, nreq, q.data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), cu_seqlens.data_ptr(), ctx_lens.data_ptr(), int(max_q_len),
        block_tables.data_ptr(), block_tables.shape[1], _ptr(qslot), out.data_ptr(), _ptr(lse),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)),
        "zp_paged_prefill")


@dataclass
class ScoreParams:
    """Scoring hyper-parameters (defaults: Zipage App. C.8's recommendation,
    lambda 0.2, tau 0.4, alpha 0.8, pooling at the first compression only,
    lightning redundancy; p and the pooling width are readings: 0.9 and 7).
    ``redundancy`` picks the lightning (App. C.7, within each block) or the
    flash (Alg. 3, over the whole sequence) row sums; ``global_reduce`` the
    max-reduce of Alg. 2 or App. C.3's decayed sum-reduce."""
    alpha: float = 0.8
    lam: float = 0.2
    tau: float = 0.4
    p: float = 0.9
    pool_kernel: int = 7
    use_global: bool = True
    global_reduce: str = "max"
    use_pool: bool = True
    pool_first_only: bool = True
    use_redundancy: bool = True
    redundancy: str = "lightning"

    def c(self):
        if self.redundancy not in ("lightning", "flash"):
            raise ValueError(f"redundancy must be 'lightning' or 'flash', not {self.redundancy!r}")
        if self.global_reduce not in ("max", "sum"):
            raise ValueError(f"global_reduce must be 'max' or 'sum', not {self.global_reduce!r}")
        flags = ((ZP_SCORE_GLOBAL if self.use_global else 0)
                 | (ZP_SCORE_GLOBAL_SUM if self.use_global and self.global_reduce == "sum" else 0)
                 | (ZP_SCORE_POOL if self.use_pool else 0)
                 | (ZP_SCORE_POOL_FIRST_ONLY if self.pool_first_only else 0)
                 | (ZP_SCORE_REDUNDANCY if self.use_redundancy else 0)
                 | (ZP_SCORE_REDUNDANCY_FLASH if self.redundancy == "flash" else 0))
        return ScoreParamsC(self.alpha, self.lam, self.tau, self.p, self.pool_kernel, flags)


def zp_score_tokens(cache: PagedKVCache, params: ScoreParams, layer_begin, layer_count,
                    block_tables, num_blocks, max_blocks, qslot, first_compression, scores,
                    f_new, workspace, stream=None, window_lse_valid=None, window_lse_all=False):
    """window_lse_all: every request's window rows carry their log-sum-exp
    (window_lse_valid is then not read); the statistics pass is skipped."""
    import torch
    _need(block_tables, torch.int32, "block_tables")
    _need(num_blocks, torch.int32, "num_blocks")
    _need(qslot, torch.int32, "qslot")
    _need(first_compression, torch.uint8, "first_compression")
    _need(window_lse_valid, torch.uint8, "window_lse_valid")
    _need(scores, torch.float32, "scores")
    _need(f_new, torch.float32, "f_new")
    if f_new is not None and f_new.shape != scores.shape:
        raise ValueError("f_new must have the shape of scores")
    nreq = block_tables.shape[0]
    pc = params.c()
    if window_lse_all:
        pc.flags |= ZP_SCORE_WINDOW_LSE_ALL
    _check(lib().zp_score_tokens(
        C.byref(cache.geom.c()), C.byref(cache.c()), C.byref(pc), layer_begin,
        layer_count, nreq, block_tables.data_ptr(), block_tables.shape[1],
        num_blocks.data_ptr(), int(max_blocks), qslot.data_ptr(), first_compression.data_ptr(),
        _ptr(window_lse_valid), scores.data_ptr(), _ptr(f_new), scores.shape[-1],
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)),
        "zp_score_tokens")


def zp_select_compact(cache: PagedKVCache, layer_begin, layer_count, scores, src_tables,
                      num_blocks, max_blocks, dst_tables, keep, kept_idx, workspace,
                      flags=0, stream=None, f_new=None):
    import torch
    _need(scores, torch.float32, "scores")
    _need(f_new, torch.float32, "f_new")
    if f_new is not None and f_new.shape != scores.shape:
        raise ValueError("f_new must have the shape of scores")
    _need(src_tables, torch.int32, "src_tables")
    _need(num_blocks, torch.int32, "num_blocks")
    _need(dst_tables, torch.int32, "dst_tables")
    _need(kept_idx, torch.int32, "kept_idx")
    nreq = src_tables.shape[0]
    _check(lib().zp_select_compact(
        C.byref(cache.geom.c()), C.byref(cache.c()), layer_begin, layer_count, nreq,
        scores.data_ptr(), _ptr(f_new), scores.shape[-1], src_tables.data_ptr(),
        src_tables.shape[1],
        num_blocks.data_ptr(), int(max_blocks), _ptr(dst_tables),
        dst_tables.shape[1] if dst_tables is not None else 0, int(keep), _ptr(kept_idx),
        int(flags), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)), "zp_select_compact")


def zp_workspace_errors(workspace, stream=None):
    flags = C.c_uint32(0)
    _check(lib().zp_workspace_errors(workspace.data_ptr(), C.byref(flags), _stream(stream)),
           "zp_workspace_errors")
    return flags.value


def zp_workspace_clear_errors(workspace, stream=None):
    _check(lib().zp_workspace_clear_errors(workspace.data_ptr(), _stream(stream)),
           "zp_workspace_clear_errors")


# --------------------------------------------------------------------------
# Host allocator and planner
# --------------------------------------------------------------------------

def _arr(xs):
    xs = list(xs)
    return (C.c_int32 * max(len(xs), 1))(*xs)


class BlockAllocator:
    """Refcounted block pool (zp_alloc_*, zp_block_*, zp_plan/commit/abort)."""

    def __init__(self, num_blocks):
        self._h = lib().zp_alloc_create(num_blocks)
        if not self._h:
            raise ZpError(ZP_EINVAL, lib().zp_last_error().decode())

    def close(self):
        if self._h:
            lib().zp_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n):
        ids = (C.c_int32 * max(n, 1))()
        _check(lib().zp_block_alloc(self._h, n, ids), "zp_block_alloc")
        return list(ids[:n])

    def free(self, ids):
        ids = list(ids)
        _check(lib().zp_block_free(self._h, _arr(ids), len(ids)), "zp_block_free")

    def share(self, ids):
        ids = list(ids)
        _check(lib().zp_block_share(self._h, _arr(ids), len(ids)), "zp_block_share")

    def refcount(self, i):
        return lib().zp_block_refcount(self._h, i)

    @property
    def num_free(self):
        return lib().zp_num_free(self._h)

    @property
    def num_blocks(self):
        return lib().zp_num_blocks(self._h)

    def plan_compress(self, table, n_max):
        """Returns (dst_table [n_max-1], new_table [n_max], release list)."""
        table = list(table)
        dst = (C.c_int32 * (n_max - 1))()
        new = (C.c_int32 * n_max)()
        rel = (C.c_int32 * max(len(table), 1))()
        nrel = C.c_int32(0)
        _check(lib().zp_plan_compress(self._h, _arr(table), len(table), n_max, dst, new, rel,
                                      C.byref(nrel)), "zp_plan_compress")
        return list(dst), list(new), list(rel[:nrel.value])

    def commit_compress(self, old_table, new_table):
        _check(lib().zp_commit_compress(self._h, _arr(old_table), len(old_table),
                                        _arr(new_table), len(new_table)), "zp_commit_compress")

    def abort_compress(self, old_table, new_table):
        _check(lib().zp_abort_compress(self._h, _arr(old_table), len(old_table),
                                       _arr(new_table), len(new_table)), "zp_abort_compress")


def zp_capacity(m_avail, m_kv, m_f, m_q, n_max):
    M = C.c_int64(0)
    N = C.c_int64(0)
    _check(lib().zp_capacity(m_avail, m_kv, m_f, m_q, n_max, C.byref(M), C.byref(N)),
           "zp_capacity")
    return M.value, N.value


# --------------------------------------------------------------------------
# Scheduler (zp_sched_*)
# --------------------------------------------------------------------------

class Step:
    """Output of one zp_sched_step: numpy views of the caller-owned arrays
    (valid until the next step) and the counts."""

    def __init__(self, bufs, raw, table_cap, n_max):
        self.kind = raw.kind
        self.n = raw.n
        self.n_comp = raw.n_comp
        self.n_blocked = raw.n_blocked
        n, nc = raw.n, raw.n_comp
        self.rid, self.slot = bufs["rid"][:n], bufs["slot"][:n]
        self.ctx, self.len = bufs["ctx"][:n], bufs["len"][:n]
        self.pos = bufs["pos"][:n]
        self.tables = bufs["tables"].reshape(-1, table_cap)[:n]
        self.c_rid, self.c_slot = bufs["c_rid"][:nc], bufs["c_slot"][:nc]
        self.c_first, self.c_nblocks = bufs["c_first"][:nc], bufs["c_nblocks"][:nc]
        self.c_nmax = bufs["c_nmax"][:nc]
        self.c_src = bufs["c_src"].reshape(-1, table_cap)[:nc]
        self.c_dst = bufs["c_dst"].reshape(-1, n_max - 1)[:nc]
        self.c_new = bufs["c_new"].reshape(-1, n_max)[:nc]
        self.finished = bufs["finished"][:raw.n_finished]
        self.preempted = bufs["preempted"][:raw.n_preempted]

    def as_dict(self):
        """Plain-Python form (lists; slot None for no slot)."""
        kinds = {ZP_STEP_IDLE: "idle", ZP_STEP_PREFILL: "prefill", ZP_STEP_DECODE: "decode"}
        sl = lambda x: None if x < 0 else int(x)
        batch = []
        for i in range(self.n):
            nt = int((self.tables[i] >= 0).sum())
            batch.append(dict(rid=int(self.rid[i]), slot=sl(self.slot[i]), ctx=int(self.ctx[i]),
                              pos=int(self.pos[i]), len=int(self.len[i]),
                              table=self.tables[i, :nt].tolist()))
        comp = []
        for i in range(self.n_comp):
            nb, nm = int(self.c_nblocks[i]), int(self.c_nmax[i])
            comp.append(dict(rid=int(self.c_rid[i]), slot=sl(self.c_slot[i]),
                             first=bool(self.c_first[i]), n_max=nm,
                             src=self.c_src[i, :nb].tolist(), dst=self.c_dst[i, :nm - 1].tolist(),
                             new=self.c_new[i, :nm].tolist()))
        return dict(kind=kinds[self.kind], batch=batch, comp=comp,
                    finished=self.finished.tolist(), preempted=self.preempted.tolist(),
                    blocked=int(self.n_blocked))


class Scheduler:
    """Binding of zp_sched (constrained / hybrid scheduling, Zipage Sec. 4.3
    and Sec. 4.4). Arrays of the step output are allocated once, here."""

    def __init__(self, num_blocks, block_size, window, n_max, num_slots, max_running,
                 max_prefill_tokens, policy="hybrid", prefix_sharing=False, table_cap=64,
                 nmax_growth=0):
        import numpy as np
        pol = {"constrained": ZP_SCHED_CONSTRAINED, "hybrid": ZP_SCHED_HYBRID}[policy]
        self.cfg = SchedConfig(num_blocks, block_size, window, n_max, num_slots, max_running,
                               max_prefill_tokens, table_cap, pol, 1 if prefix_sharing else 0,
                               nmax_growth)
        self._h = lib().zp_sched_create(C.byref(self.cfg))
        if not self._h:
            raise ZpError(ZP_EINVAL, lib().zp_last_error().decode())
        R, cap = max_running, table_cap
        sizes = dict(rid=R, slot=R, ctx=R, pos=R, len=R, tables=R * cap, c_rid=R, c_slot=R, c_first=R,
                     c_nblocks=R, c_nmax=R, c_src=R * cap, c_dst=R * (n_max - 1), c_new=R * n_max,
                     finished=R, preempted=R)
        self._bufs = {k: np.zeros(v, np.int32) for k, v in sizes.items()}
        self._out = SchedStepOut()
        for k, a in self._bufs.items():
            setattr(self._out, k, a.ctypes.data_as(C.POINTER(C.c_int32)))
        self.table_cap, self.n_max = table_cap, n_max

    def close(self):
        if self._h:
            lib().zp_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, rid, prompt_len, max_new, prefix_group=-1, prefix_len=0, n_max=0):
        _check(lib().zp_sched_add(self._h, rid, prompt_len, max_new, prefix_group, prefix_len,
                                  n_max), "zp_sched_add")

    def step(self) -> Step:
        _check(lib().zp_sched_step(self._h, C.byref(self._out)), "zp_sched_step")
        return Step(self._bufs, self._out, self.table_cap, self.n_max)

    def compress_done(self, rid):
        _check(lib().zp_sched_compress_done(self._h, rid), "zp_sched_compress_done")

    def stats(self):
        st = SchedStats()
        _check(lib().zp_sched_get_stats(self._h, C.byref(st)), "zp_sched_get_stats")
        return {k: getattr(st, k) for k, _ in SchedStats._fields_}

    def request(self, rid):
        info = SchedReqInfo()
        tab = (C.c_int32 * self.table_cap)()
        _check(lib().zp_sched_request(self._h, rid, C.byref(info), tab), "zp_sched_request")
        d = {k: getattr(info, k) for k, _ in SchedReqInfo._fields_}
        d["table"] = list(tab[:info.ntable])
        return d

    def unfinished(self):
        return lib().zp_sched_unfinished(self._h)

    def refcount(self, block):
        return lib().zp_block_refcount(lib().zp_sched_allocator(self._h), block)

    def num_free(self):
        return lib().zp_num_free(lib().zp_sched_allocator(self._h))
