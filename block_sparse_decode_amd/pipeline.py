"""Device buffers for one KV workspace and the library calls in order.

Plumbing only: torch allocates device memory; every computation is a call
into libkvmem.so.  Used by the tests, the benchmark and the smoke check.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L

BLOCK = 32


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host array (bf16 as raw uint16 bits, or fp32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def v_view_token_major(v_view: torch.Tensor) -> torch.Tensor:
    """[S][Hkv][nblk][d][32 slots] dimension-major V view -> [S][Hkv][nblk*32][d]
    token-major (inverse of the slot order documented in kvmem.h)."""
    sigma = [8 * ((u & 15) >> 2) + 4 * (u >> 4) + (u & 3) for u in range(BLOCK)]
    idx = torch.tensor(sigma, device=v_view.device)
    x = v_view.index_select(-1, idx).transpose(-1, -2)          # [..][nblk][32][d]
    S, H, nb = x.shape[:3]
    return x.reshape(S, H, nb * BLOCK, x.shape[-1])


INDEX_TILE = 64


def index_tile_shape(S: int, H: int, max_blocks: int, d: int, dtype: str) -> tuple:
    """Shape of the tiled Mean-K index as documented in kvmem.h:
    [S][H][tiles of 64 blocks][16-byte word][64 rows][elements per word]."""
    E = 8 if dtype == "bf16" else 4
    return (S, H, -(-max_blocks // INDEX_TILE), d // E, INDEX_TILE, E)


def index_rows(index: torch.Tensor, max_blocks: int) -> torch.Tensor:
    """Tiled index [S][H][NT][W][64][E] -> row-major [S][H][max_blocks][d]."""
    S, H, NT, W, T, E = index.shape
    x = index.permute(0, 1, 2, 4, 3, 5).reshape(S, H, NT * T, W * E)
    return x[:, :, :max_blocks]


class DeviceWorkspace:
    """Inputs of a workload on the GPU plus every buffer the four calls use."""

    def __init__(self, wl, device="cuda", k_select=None, n_recent=None, max_view=None, with_v=True,
                 device_pools=None, host_pools=False):
        cfg = wl.cfg
        self.cfg = cfg
        self.device = torch.device(device)
        self.dtype = cfg.dtype
        self.tdtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.k_select = cfg.k_select if k_select is None else k_select
        self.n_recent = cfg.n_recent if n_recent is None else n_recent
        self.T = cfg.T
        S, H, d = cfg.n_sessions, cfg.n_kv_heads, cfg.head_dim
        self.S, self.H, self.d = S, H, d
        if device_pools is not None:           # pools the caller has already put on the device
            self.k_pool, self.v_pool = device_pools
        elif host_pools:                        # the host tier: pinned host memory the GPU reads in place
            self.k_pool = to_device(wl.k_pool, cfg.dtype, "cpu").pin_memory()
            self.v_pool = to_device(wl.v_pool, cfg.dtype, "cpu").pin_memory() if with_v else None
        elif wl.k_pool is not None:
            self.k_pool = to_device(wl.k_pool, cfg.dtype, self.device)
            self.v_pool = to_device(wl.v_pool, cfg.dtype, self.device) if with_v else None
        else:                                   # pools too large for the host: drawn chunk by chunk
            self.k_pool = self._stream_pool(wl, "k")
            self.v_pool = self._stream_pool(wl, "v") if with_v else None
        self.block_table = torch.from_numpy(np.ascontiguousarray(wl.block_table, dtype=np.int32)).to(self.device)
        self.n_tokens = np.array(wl.n_tokens, dtype=np.int32, copy=True)   # own copy: append advances it
        self.dev_error = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.max_blocks = int(wl.block_table.shape[1])
        self.q = to_device(wl.q, cfg.dtype, self.device)
        self.q_norm_w = torch.from_numpy(np.ascontiguousarray(wl.q_norm_w, dtype=np.float32)).to(self.device)
        self.geom = L.make_geom(cfg.n_q_heads, H, cfg.dtype, d)
        self.ws = L.make_workspace(self.k_pool, self.v_pool, self.block_table, self.n_tokens, self.dev_error)

        shape = index_tile_shape(S, H, self.max_blocks, d, cfg.dtype)
        assert int(np.prod(shape)) * (2 if cfg.dtype == "bf16" else 4) == \
            L.kvmem_index_bytes(self.geom, S, self.max_blocks)
        self.index = torch.empty(shape, dtype=self.tdtype, device=self.device)
        self.n_list = self.k_select + self.n_recent
        self.view_blocks = torch.empty((S, H, max(1, self.n_list)), dtype=torch.int32, device=self.device)
        self.view_tokens = np.zeros(S, np.int32)
        need = int(L.kvmem_view_tokens(self.n_tokens, self.k_select, self.n_recent).max())
        mv = max(BLOCK, -(-need // BLOCK) * BLOCK)
        self.max_view = mv if max_view is None else max_view
        self.k_view = torch.empty((S, H, self.max_view, d), dtype=self.tdtype, device=self.device)
        self.v_view = torch.empty((S, H, self.max_view // BLOCK, d, BLOCK), dtype=self.tdtype, device=self.device)
        self.out = torch.empty((S, self.T, cfg.n_q_heads, d), dtype=torch.float32, device=self.device)
        nb = L.kvmem_score_select_scratch_bytes(self.geom, S, self.max_blocks, self.T)
        na = L.kvmem_attend_scratch_bytes(self.geom, S, self.T, self.max_view)
        self.score_scratch = torch.empty(max(nb, 1), dtype=torch.uint8, device=self.device)
        self.attend_scratch = torch.empty(max(na, 1), dtype=torch.uint8, device=self.device)
        self.eps = cfg.eps
        self.theta = cfg.rope_theta

    @staticmethod
    def view_length_of(wl, k_select=None, n_recent=None) -> list:
        """View tokens of every session of a workload (the library's host-side query)."""
        k = wl.cfg.k_select if k_select is None else k_select
        r = wl.cfg.n_recent if n_recent is None else n_recent
        return [int(v) for v in L.kvmem_view_tokens(wl.n_tokens, k, r)]

    def _stream_pool(self, wl, which: str) -> torch.Tensor:
        from workloads import pool_chunks
        cfg = wl.cfg
        shape = (wl.n_pages, cfg.n_kv_heads, BLOCK, cfg.head_dim)
        pool = torch.empty(shape, dtype=self.tdtype, device=self.device)
        for _, _, pages, x in pool_chunks(wl, which):
            idx = torch.from_numpy(np.ascontiguousarray(pages, dtype=np.int64)).to(self.device)
            pool[idx] = to_device(x, cfg.dtype, self.device)
        return pool

    # --- the four calls ---------------------------------------------------
    def build_index(self, stream=None):
        L.kvmem_build_index(self.geom, self.ws, self.index, stream)

    def update_index(self, first_block: np.ndarray, stream=None):
        """Index rows of blocks first_block[s] .. of every session (host array)."""
        L.kvmem_update_index(self.geom, self.ws, np.ascontiguousarray(first_block, dtype=np.int32), self.index,
                             stream)

    def score_select(self, stream=None, scores=None, agg=None):
        L.kvmem_score_select(self.geom, self.ws, self.index, self.q, self.T, self.q_norm_w, self.eps,
                             self.k_select, self.n_recent, self.view_blocks, self.view_tokens,
                             scores=scores, agg=agg, scratch=self.score_scratch, stream=stream)

    def materialize(self, stream=None):
        L.kvmem_materialize(self.geom, self.ws, self.view_blocks, self.n_list, self.view_tokens,
                            self.max_view, self.theta, self.k_view, self.v_view, stream)

    def attend(self, stream=None):
        L.kvmem_attend(self.geom, self.S, self.q, self.T, self.q_norm_w, self.eps, self.k_view, self.v_view,
                       self.view_tokens, self.max_view, self.theta, self.out, scratch=self.attend_scratch,
                       stream=stream)

    # --- decoding over the reused view ---------------------------------------
    def append(self, k_new, v_new, stream=None):
        """Append T_new tokens per session ([S][T_new][Hkv][d] device tensors,
        pre-RoPE) to the pools and the view, then index the blocks they
        completed.  Advances the host lengths in place (the workspace struct
        points at them)."""
        T_new = int(k_new.shape[1])
        L.kvmem_append(self.geom, self.ws, self.k_pool, self.v_pool, k_new, v_new, T_new, self.view_tokens,
                       self.max_view, self.theta, self.k_view, self.v_view, stream)
        first = (self.n_tokens // BLOCK).astype(np.int32)
        self.n_tokens += T_new
        self.view_tokens += T_new
        if np.any(self.n_tokens // BLOCK > first):
            L.kvmem_update_index(self.geom, self.ws, first, self.index, stream)

    def attend_append(self, k_new, v_new, stream=None):
        """One decode token in one call: the attention over the current view
        (into self.out), then the append of k_new / v_new as append() does
        (the append rides on the attention's merge launch)."""
        T_new = int(k_new.shape[1])
        L.kvmem_attend_append(self.geom, self.ws, self.q, self.T, self.q_norm_w, self.eps, self.k_view, self.v_view,
                              self.view_tokens, self.max_view, self.theta, self.out, self.k_pool, self.v_pool, k_new,
                              v_new, T_new, scratch=self.attend_scratch, stream=stream)
        first = (self.n_tokens // BLOCK).astype(np.int32)
        self.n_tokens += T_new
        self.view_tokens += T_new
        if np.any(self.n_tokens // BLOCK > first):
            L.kvmem_update_index(self.geom, self.ws, first, self.index, stream)

    # --- attention straight from the pages ----------------------------------
    def attend_paged(self, out=None, stream=None):
        """The attention of kvmem_attend over the current lists, read from the
        pages (no materialised view)."""
        if not hasattr(self, "paged_scratch"):
            nbytes = L.kvmem_attend_paged_scratch_bytes(self.geom, self.S, self.T, max(1, self.n_list))
            self.paged_scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        L.kvmem_attend_paged(self.geom, self.ws, self.q, self.T, self.q_norm_w, self.eps, self.view_blocks,
                             self.n_list, self.view_tokens, self.theta, self.out if out is None else out,
                             scratch=self.paged_scratch, stream=stream)

    def materialize_attend(self, out=None, stream=None):
        """kvmem_materialize and kvmem_attend in one pass over the selected
        blocks: the view is written and the step's attention computed."""
        if not hasattr(self, "paged_scratch"):
            nbytes = L.kvmem_attend_paged_scratch_bytes(self.geom, self.S, self.T, max(1, self.n_list))
            self.paged_scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        L.kvmem_materialize_attend(self.geom, self.ws, self.q, self.T, self.q_norm_w, self.eps, self.view_blocks,
                                   self.n_list, self.view_tokens, self.max_view, self.theta, self.k_view,
                                   self.v_view, self.out if out is None else out, scratch=self.paged_scratch,
                                   stream=stream)

    # --- host-tier paging ----------------------------------------------------
    def stage(self, staged: "StagedView", stream=None):
        """Copy the current lists' blocks from this workspace's pools (pinned
        host memory for the host tier) into the staging pool."""
        L.kvmem_stage_view(self.geom, self.ws, self.view_blocks, self.n_list, self.view_tokens, staged.k, staged.v,
                           staged.table, staged.list, stream)

    def materialize_attend_staged(self, staged: "StagedView", out=None, stream=None):
        """kvmem_materialize_attend over the staged pool (its identity list)."""
        if not hasattr(self, "paged_scratch"):
            nbytes = L.kvmem_attend_paged_scratch_bytes(self.geom, self.S, self.T, max(1, self.n_list))
            self.paged_scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        L.kvmem_materialize_attend(self.geom, staged.ws, self.q, self.T, self.q_norm_w, self.eps, staged.list,
                                   self.n_list, self.view_tokens, self.max_view, self.theta, self.k_view,
                                   self.v_view, self.out if out is None else out, scratch=self.paged_scratch,
                                   stream=stream)

    # --- selection-quality diagnostic ---------------------------------------
    def attention_mass(self, mass, lse=None, view_blocks=None, n_list=None, stream=None):
        """Share of full attention over the history that the listed blocks
        carry (default: the current selection's lists)."""
        vb = self.view_blocks if view_blocks is None else view_blocks
        nl = self.n_list if n_list is None else n_list
        if not hasattr(self, "mass_scratch"):
            nbytes = L.kvmem_attention_mass_scratch_bytes(self.geom, self.S, self.T, self.max_blocks)
            self.mass_scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        L.kvmem_attention_mass(self.geom, self.ws, self.q, self.T, self.q_norm_w, self.eps, vb, nl, self.theta,
                               mass, lse, scratch=self.mass_scratch, stream=stream)

    def run(self, stream=None):
        self.build_index(stream)
        self.score_select(stream)
        self.materialize(stream)
        self.attend(stream)


class StagedView:
    """Device staging pool of a workspace's views (kvmem_stage_view): page
    s * n_list + m holds every KV head's m-th listed block; with its block
    table and identity list it is a workspace whose history is the view."""

    def __init__(self, dw: DeviceWorkspace):
        S, H, d, n = dw.S, dw.H, dw.d, max(1, dw.n_list)
        self.k = torch.empty((S * n, H, BLOCK, d), dtype=dw.tdtype, device=dw.device)
        self.v = torch.empty((S * n, H, BLOCK, d), dtype=dw.tdtype, device=dw.device)
        self.table = torch.empty((S, n), dtype=torch.int32, device=dw.device)
        self.list = torch.empty((S, H, n), dtype=torch.int32, device=dw.device)
        # the staged history lengths are the view lengths (the array the
        # selection writes in place)
        self.ws = L.make_workspace(self.k, self.v, self.table, dw.view_tokens, dw.dev_error)
