"""Test-side glue: build oracle workspaces from generated workloads."""
from __future__ import annotations

import numpy as np

from oracle import kvmem_oracle as O
from workloads import Config, Workload, make_workload


def oracle_ws(wl: Workload) -> O.Workspace:
    c = wl.cfg
    return O.Workspace(wl.k_pool, wl.v_pool, wl.block_table, wl.n_tokens, c.dtype,
                       c.n_q_heads, c.n_kv_heads, c.head_dim)


def small_cfg(name: str = "small", dtype: str = "bf16", S: int = 1, Hq: int = 16, Hkv: int = 2,
              n_tokens=(4096,), T: int = 1, k: int = 16, R: int = 4, n_planted: int = 8,
              seed: int = 11, **kw) -> Config:
    if len(n_tokens) != S:
        n_tokens = tuple(n_tokens) * S if len(n_tokens) == 1 else tuple(n_tokens)
    return Config(name, dtype, S, Hq, Hkv, n_tokens=tuple(n_tokens), T=T, k_select=k,
                  n_recent=R, plant="fixed", n_planted=n_planted, seed=seed, **kw)


def logical_tokens(wl: Workload, pool: np.ndarray, s: int, h: int) -> np.ndarray:
    """All history tokens of (s, h) in logical order, gathered straight from
    the page table (independent of the oracle's accessors): [N][d] float64."""
    n = int(wl.n_tokens[s])
    nb = -(-n // 32)
    pages = wl.block_table[s, :nb]
    raw = pool[pages, h].reshape(nb * 32, pool.shape[-1])[:n]
    if wl.cfg.dtype == "bf16":
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return raw.astype(np.float64)


__all__ = ["oracle_ws", "small_cfg", "logical_tokens", "make_workload"]
