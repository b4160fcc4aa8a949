"""KVMem hot path on MI355X: Mean-K index, query-conditioned block selection,
re-RoPE view materialisation and split-K decode attention as HIP kernels for
gfx950 behind the C ABI in include/kvmem.h.

The Python side only marshals arguments (``_lib``) and holds device buffers
(``pipeline``); it fails loudly when libkvmem.so has not been built.
"""
from . import _lib  # noqa: F401
from ._lib import (KVMemError, kvmem_attend, kvmem_attend_scratch_bytes, kvmem_build_index,  # noqa: F401
                   kvmem_materialize, kvmem_score_select, kvmem_score_select_scratch_bytes, kvmem_version,
                   load)
