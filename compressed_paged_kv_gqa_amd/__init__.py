"""MI355X-native compressed paged KV cache hot path (Zipage, arXiv 2603.08743).

The compute path is libzp (HIP kernels for gfx950 behind the C ABI in
include/zp.h); ``zp`` is its ctypes binding, ``engine`` the host runtime that
drives decode steps and asynchronous compressions, ``synth`` the seeded
synthetic inputs. Build the library with ``python -m
compressed_paged_kv_gqa_amd._build``.
"""
from . import zp  # noqa: F401

__all__ = ["zp"]
