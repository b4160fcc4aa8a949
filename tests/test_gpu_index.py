"""GPU parity of the Mean-K index build over block ranges, through the C ABI.

The bf16 build gives each workgroup 512 consecutive blocks of one head,
starting from the tile (64-block) boundary at or below the range's first block,
and writes only the rows inside the range.  These cases check the range logic
against the oracle, bit for bit: a full build of sessions whose lengths end
mid-tile and mid-group, and kvmem_update_index from first blocks in the middle
of a tile, on tile and group boundaries, at the last block and past it (empty
range).  Rows below each range must keep the sentinel they were overwritten
with, rows inside must equal the oracle's rounded means.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_sparse_decode_amd.pipeline import DeviceWorkspace, index_rows
from oracle import kvmem_oracle as O
from tests.helpers import make_workload, oracle_ws, small_cfg
import block_sparse_decode_amd._lib as L

pytestmark = pytest.mark.gpu

SENTINEL = 0x7A7A   # a bf16 bit pattern no mean of these inputs produces


def _index_bits(dw) -> np.ndarray:
    return index_rows(dw.index, dw.max_blocks).contiguous().view(torch.int16).cpu().numpy()


def _oracle_bits(ws, s: int, h: int, blocks) -> np.ndarray:
    rows = O.mean_k_rows(ws, s, h, list(blocks))          # rounded to bf16, as float64
    return (rows.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


@pytest.mark.parametrize("firsts", [
    (700, 600, 0),        # mid-tile, mid-group; a whole session
    (512, 64, 18),        # on a group boundary, on a tile boundary, mid-tile
    (1499, 1099, 618),    # the last block of each session
    (1500, 1100, 619),    # empty ranges
])
def test_update_index_ranges(firsts):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # lengths end mid-tile and mid-group: 1500, 1100 and 619 complete blocks (+ partial blocks)
    cfg = small_cfg("index_ranges", "bf16", S=3, Hq=16, Hkv=2, n_tokens=(32 * 1500 + 7, 32 * 1100, 32 * 619 + 31),
                    k=8, R=2, n_planted=4, seed=29)
    wl = make_workload(cfg)
    print(f"[gpu] index ranges N={list(wl.n_tokens)} first={firsts}", flush=True)
    dw = DeviceWorkspace(wl, "cuda")
    dw.build_index()
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0
    ws = oracle_ws(wl)
    full = _index_bits(dw)
    nbs = [int(n) // 32 for n in wl.n_tokens]
    for s in range(cfg.n_sessions):
        for h in range(cfg.n_kv_heads):
            assert np.array_equal(full[s, h, :nbs[s]], _oracle_bits(ws, s, h, range(nbs[s]))), (s, h, "full build")

    dw.index.view(torch.int16).fill_(SENTINEL)
    first = np.asarray(firsts, np.int32)
    L.kvmem_update_index(dw.geom, dw.ws, first, dw.index)
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0
    got = _index_bits(dw)
    for s in range(cfg.n_sessions):
        f, nb = int(first[s]), nbs[s]
        for h in range(cfg.n_kv_heads):
            assert bool((got[s, h, :f] == SENTINEL).all()), (s, h, "rows below the range were written")
            assert bool((got[s, h, nb:] == SENTINEL).all()), (s, h, "rows past the complete blocks were written")
            assert np.array_equal(got[s, h, f:nb], full[s, h, f:nb]), (s, h, "range rows")
