"""Seeded, chunk-addressable synthetic KV workspaces.

Every input of the KVMem hot path is drawn here: paged pre-RoPE keys and
values, the logical-block -> page table, the per-session history lengths, the
decode queries and the q-RMSNorm weight.  The shapes follow the pages' setting
(32-token blocks per the KVMem review's 'Summary'; histories up to one million
tokens per the KVMEM reproduction README's 'Offline and online results', and up
to ten million per the review's 'Key claims under review'; a 256K native window
bounds the view, same section).

Recipe (one seed per workload):
  * q_hat[s, h]   : a unit direction per (session, KV head), N(0, I) normalised.
  * q[s, t, g]    : q_scale * q_hat[s, g // G] + q_noise * N(0, 1) per element.
  * K, V          : N(0, 1) per element, drawn in fp32 and rounded once to the
                    storage dtype (round-to-nearest-even for bf16).
  * planting      : keys of a planted block get + m * q_hat[s, h] on all 32
                    tokens before rounding.  "fixed": n_planted blocks per
                    (session, KV head) drawn among the selection candidates,
                    m = plant_offset.  "fraction": the same with
                    round(fraction * candidates) blocks.  "pareto": every
                    complete block gets m = min(0.05 * U**(-1/1.5), 20),
                    U ~ Uniform(0, 1].
  * block table   : logical blocks of all sessions map to a seeded random
                    permutation of the physical pages; unused entries are -1.
                    Spare pages (never referenced) hold NaN so that a stray
                    read shows up in the results.
Random streams come from numpy's SeedSequence([seed, stream, ...]) with
1024-block chunks, so any chunk can be regenerated on its own (pool_chunks
yields them one by one, for workspaces too large to hold on the host).
A workload may carry a key repair log (Workload.extra["repairs"]: ordered
(session, KV head, block, dim, delta) entries): after a key chunk is drawn,
each entry adds delta to that coordinate of the block's 32 keys in fp32 and
re-rounds to the storage dtype, in log order.

Decoding over a reused view (with_decode_capacity, draw_decode_tokens): the
block table gains pages for the blocks the histories grow into (new pages
appended to the pools, NaN-filled, mapped in a seeded order), and each decode
step's new tokens have K, V ~ N(0, 1) per element, rounded once, from the
streams (seed, decode K or V, step).

Nothing in this module computes any part of the method itself.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK_TOKENS = 32
CHUNK_BLOCKS = 1024

# stream ids
_S_K, _S_V, _S_QHAT, _S_Q, _S_PLANT, _S_TABLE, _S_W, _S_LEN, _S_DEC_K, _S_DEC_V, _S_DEC_TABLE = range(1, 12)


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits (uint16) to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str                       # "f32" | "bf16"
    n_sessions: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int = 128
    n_tokens: tuple = ()             # per-session history lengths (fixed)
    ragged_blocks: tuple = ()        # (lo, hi): block counts ~ U{lo..hi} per session
    T: int = 1                       # query tokens per step
    k_select: int = 8
    n_recent: int = 8
    plant: str = "fixed"             # "fixed" | "fraction" | "pareto" | "none"
    n_planted: int = 0
    plant_fraction: float = 0.0
    plant_offset: float = 2.0
    rope_theta: float = 1e6
    eps: float = 1e-6
    seed: int = 1
    q_scale: float = 4.0
    q_noise: float = 0.1
    w_mode: str = "unit"             # "unit" | "random"
    spare_pages: int = 0
    max_blocks: int = 0              # block-table capacity; 0 = just enough

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads.  Sizes follow the scope of the hot path (tiny fp32 layer,
# 27B-class GQA layer at 256K and 1M tokens, 16 ragged sessions with 4-token
# MTP-style queries, and a 10M-token index with a 512-token prefill chunk).
CONFIGS = {
    "c1": Config("c1_tiny_fp32", "f32", 1, 4, 1, n_tokens=(4096,), T=1,
                 k_select=8, n_recent=8, plant="fixed", n_planted=8, seed=1),
    "c2": Config("c2_256k_bf16", "bf16", 1, 64, 8, n_tokens=(262144,), T=1,
                 k_select=1024, n_recent=64, plant="fixed", n_planted=64, seed=2),
    "c3": Config("c3_1m_bf16", "bf16", 1, 64, 8, n_tokens=(1048576,), T=1,
                 k_select=7936, n_recent=256, plant="pareto", seed=3),
    "c4": Config("c4_16x64k_t4_bf16", "bf16", 16, 64, 8, ragged_blocks=(1024, 2048), T=4,
                 k_select=96, n_recent=32, plant="fixed", n_planted=16, seed=4,
                 max_blocks=2048),
    "c5": Config("c5_10m_t512_bf16", "bf16", 1, 64, 8, n_tokens=(10_000_000,), T=512,
                 k_select=2048, n_recent=0, plant="fraction", plant_fraction=0.01, seed=5),
}


@dataclass
class Workload:
    cfg: Config
    k_pool: np.ndarray        # [n_pages][Hkv][32][d], uint16 bf16 bits or float32
    v_pool: np.ndarray
    block_table: np.ndarray   # int32 [S][max_blocks], -1 = unused
    n_tokens: np.ndarray      # int32 [S]
    q: np.ndarray             # [S][T][Hq][d], uint16 bf16 bits or float32
    q_norm_w: np.ndarray      # float32 [d]
    qhat: np.ndarray          # float64 [S][Hkv][d]
    plant_mag: np.ndarray     # float32 [S][Hkv][max_blocks]
    extra: dict = field(default_factory=dict)

    @property
    def n_pages(self) -> int:
        return int(self.k_pool.shape[0]) if self.k_pool is not None else int(self.extra["n_pages"])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def session_lengths(cfg: Config) -> np.ndarray:
    if cfg.n_tokens:
        assert len(cfg.n_tokens) == cfg.n_sessions
        return np.asarray(cfg.n_tokens, dtype=np.int64)
    lo, hi = cfg.ragged_blocks
    nb = _rng(cfg.seed, _S_LEN).integers(lo, hi + 1, size=cfg.n_sessions)
    return (nb * BLOCK_TOKENS).astype(np.int64)


def _candidate_count(n_tok: int, n_recent: int) -> int:
    """Complete blocks that are not among the last n_recent blocks."""
    nb_full = n_tok // BLOCK_TOKENS
    nb_all = -(-n_tok // BLOCK_TOKENS)
    return max(0, min(nb_full, nb_all - n_recent))


def _plant_magnitudes(cfg: Config, lens: np.ndarray, max_blocks: int) -> np.ndarray:
    S, H = cfg.n_sessions, cfg.n_kv_heads
    mag = np.zeros((S, H, max_blocks), np.float32)
    for s in range(S):
        n_tok = int(lens[s])
        nb_full = n_tok // BLOCK_TOKENS
        nc = _candidate_count(n_tok, cfg.n_recent)
        rng = _rng(cfg.seed, _S_PLANT, s)
        for h in range(H):
            if cfg.plant == "none" or nb_full == 0:
                continue
            if cfg.plant == "pareto":
                u = 1.0 - rng.random(nb_full)             # U ~ (0, 1]
                mag[s, h, :nb_full] = np.minimum(0.05 * u ** (-1.0 / 1.5), 20.0)
            else:
                n = cfg.n_planted if cfg.plant == "fixed" else int(round(cfg.plant_fraction * nc))
                n = min(n, nc)
                if n > 0:
                    idx = rng.choice(nc, size=n, replace=False)
                    mag[s, h, idx] = cfg.plant_offset
    return mag


def _make_table(cfg: Config, lens: np.ndarray, max_blocks: int):
    nblk = [-(-int(n) // BLOCK_TOKENS) for n in lens]
    total = int(sum(nblk))
    n_pages = total + cfg.spare_pages
    perm = _rng(cfg.seed, _S_TABLE).permutation(n_pages)[:total].astype(np.int32)
    table = np.full((cfg.n_sessions, max_blocks), -1, np.int32)
    off = 0
    for s, nb in enumerate(nblk):
        table[s, :nb] = perm[off:off + nb]
        off += nb
    return table, n_pages


def _chunk_jobs(cfg: Config, lens: np.ndarray) -> list:
    jobs = []
    for s in range(cfg.n_sessions):
        nblk = -(-int(lens[s]) // BLOCK_TOKENS)
        for c0 in range(0, nblk, CHUNK_BLOCKS):
            jobs.append((s, c0, min(nblk, c0 + CHUNK_BLOCKS)))
    return jobs


def _draw_chunk(cfg: Config, job, lens: np.ndarray, stream: int, mag: np.ndarray | None, qhat: np.ndarray,
                repairs=()) -> np.ndarray:
    """Blocks [b0, b1) of session s for all KV heads, in storage form: [nb][H][32][d]."""
    H, d, Bt = cfg.n_kv_heads, cfg.head_dim, BLOCK_TOKENS
    s, b0, b1 = job
    nb = b1 - b0
    x = np.empty((nb, H, Bt, d), np.float32)
    _rng(cfg.seed, stream, s, b0 // CHUNK_BLOCKS).standard_normal(out=x, dtype=np.float32)
    if mag is not None:
        m = mag[s, :, b0:b1].T.astype(np.float32)                       # [nb][H]
        x += m[:, :, None, None] * qhat[s][None, :, None, :].astype(np.float32)
    n_tok = int(lens[s])
    last_valid = n_tok - (b1 - 1) * Bt                                 # tokens in the last block
    if last_valid < Bt:                                                # partial tail: zero the rest
        x[-1, :, last_valid:, :] = 0.0
    out = f32_to_bf16_bits(x) if cfg.dtype == "bf16" else x
    for (rs, rh, rb, ri, delta) in repairs:
        if rs == s and b0 <= rb < b1:
            if cfg.dtype == "bf16":
                col = bf16_bits_to_f32(out[rb - b0, rh, :, ri])
                out[rb - b0, rh, :, ri] = f32_to_bf16_bits(col + np.float32(delta))
            else:
                out[rb - b0, rh, :, ri] += np.float32(delta)
    return out


def _fill_pool(cfg: Config, pool: np.ndarray, table: np.ndarray, lens: np.ndarray,
               stream: int, mag: np.ndarray | None, qhat: np.ndarray, threads: int, repairs=()):
    jobs = _chunk_jobs(cfg, lens)

    def work(job):
        s, b0, b1 = job
        pool[table[s, b0:b1]] = _draw_chunk(cfg, job, lens, stream, mag, qhat, repairs)

    if threads <= 1 or len(jobs) <= 1:
        for j in jobs:
            work(j)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, jobs))


def pool_chunks(wl: "Workload", which: str = "k", threads: int | None = None, jobs=None):
    """Yield (session, first block, pages, chunk) for every 1024-block chunk of
    the K ("k") or V ("v") pool, drawn exactly as make_workload draws them
    (chunk = [nb][H][32][d] in storage form).  Chunks are drawn on a thread
    pool and yielded in order; `jobs` restricts the walk to given
    (session, first block, end block) chunks."""
    cfg = wl.cfg
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    lens = wl.n_tokens.astype(np.int64)
    stream, mag = (_S_K, wl.plant_mag) if which == "k" else (_S_V, None)
    repairs = tuple(wl.extra.get("repairs", ())) if which == "k" else ()
    jobs = _chunk_jobs(cfg, lens) if jobs is None else list(jobs)
    draw = lambda job: _draw_chunk(cfg, job, lens, stream, mag, wl.qhat, repairs)
    with _cf.ThreadPoolExecutor(max(1, threads)) as ex:
        futs = [ex.submit(draw, j) for j in jobs[:2 * threads]]
        for i, job in enumerate(jobs):
            x = futs[i].result()
            futs[i] = None
            if i + 2 * threads < len(jobs):
                futs.append(ex.submit(draw, jobs[i + 2 * threads]))
            s, b0, b1 = job
            yield s, b0, wl.block_table[s, b0:b1], x


def make_workload(cfg: Config, threads: int | None = None, with_v: bool = True, pools: bool = True,
                  repairs=()) -> Workload:
    """Draw the full workspace of `cfg` (host arrays).  With pools=False the K
    and V pools are left out (None) and can be drawn chunk by chunk with
    pool_chunks; `repairs` is a key repair log (see the module notes)."""
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    S, Hq, H, d, T = cfg.n_sessions, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.T
    assert Hq % H == 0
    lens = session_lengths(cfg)
    need = max(1, max(-(-int(n) // BLOCK_TOKENS) for n in lens))
    max_blocks = max(need, cfg.max_blocks)

    qhat = np.empty((S, H, d), np.float64)
    for s in range(S):
        v = _rng(cfg.seed, _S_QHAT, s).standard_normal((H, d))
        qhat[s] = v / np.linalg.norm(v, axis=1, keepdims=True)

    G = Hq // H
    qf = np.empty((S, T, Hq, d), np.float32)
    for s in range(S):
        noise = _rng(cfg.seed, _S_Q, s).standard_normal((T, Hq, d)).astype(np.float32)
        base = np.repeat(qhat[s], G, axis=0).astype(np.float32)        # [Hq][d]
        qf[s] = cfg.q_scale * base[None] + cfg.q_noise * noise
    q = f32_to_bf16_bits(qf) if cfg.dtype == "bf16" else qf

    if cfg.w_mode == "unit":
        w = np.ones(d, np.float32)
    else:
        w = (0.5 + _rng(cfg.seed, _S_W).random(d)).astype(np.float32)

    mag = _plant_magnitudes(cfg, lens, max_blocks)
    table, n_pages = _make_table(cfg, lens, max_blocks)
    extra = {"repairs": list(repairs)} if repairs else {}
    if not pools:
        wl = Workload(cfg, None, None, table, lens.astype(np.int32), q, w, qhat, mag, extra)
        wl.extra["n_pages"] = n_pages
        return wl
    pdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    nan = np.uint16(0x7FC0) if cfg.dtype == "bf16" else np.float32(np.nan)
    shape = (n_pages, H, BLOCK_TOKENS, d)
    k_pool = np.empty(shape, pdt)
    v_pool = np.empty(shape if with_v else (0, H, BLOCK_TOKENS, d), pdt)
    if cfg.spare_pages:
        used = np.zeros(n_pages, bool)
        used[table[table >= 0]] = True
        k_pool[~used] = nan
        if with_v:
            v_pool[~used] = nan
    _fill_pool(cfg, k_pool, table, lens, _S_K, mag, qhat, threads, tuple(repairs))
    if with_v:
        _fill_pool(cfg, v_pool, table, lens, _S_V, None, qhat, threads)
    return Workload(cfg, k_pool, v_pool, table, lens.astype(np.int32), q, w, qhat, mag, extra)


def with_decode_capacity(wl: Workload, extra_tokens: int) -> Workload:
    """A copy of wl whose histories can each grow by extra_tokens: the blocks
    they grow into get new pages (appended to the pools, NaN-filled) mapped in
    the block table, whose width grows as needed."""
    cfg = wl.cfg
    S = cfg.n_sessions
    lens = wl.n_tokens.astype(np.int64)
    have = [-(-int(n) // BLOCK_TOKENS) for n in lens]
    need = [-(-(int(n) + extra_tokens) // BLOCK_TOKENS) for n in lens]
    n_new = int(sum(b - a for a, b in zip(have, need)))
    max_blocks = max(wl.max_blocks, max(need) if need else 1)
    table = np.full((S, max_blocks), -1, np.int32)
    table[:, :wl.max_blocks] = wl.block_table
    base = wl.n_pages
    pages = base + _rng(cfg.seed, _S_DEC_TABLE).permutation(n_new).astype(np.int32)
    off = 0
    for s in range(S):
        k = need[s] - have[s]
        table[s, have[s]:need[s]] = pages[off:off + k]
        off += k
    nan = np.uint16(0x7FC0) if cfg.dtype == "bf16" else np.float32(np.nan)

    def grow(pool):
        if pool is None:
            return None
        extra = np.full((n_new,) + pool.shape[1:], nan, pool.dtype)
        return np.concatenate([pool, extra], axis=0)

    mag = np.zeros((S, cfg.n_kv_heads, max_blocks), np.float32)
    mag[:, :, :wl.max_blocks] = wl.plant_mag
    out = Workload(cfg, grow(wl.k_pool), grow(wl.v_pool) if wl.v_pool is not None and len(wl.v_pool) else wl.v_pool,
                   table, wl.n_tokens.copy(), wl.q, wl.q_norm_w, wl.qhat, mag, dict(wl.extra))
    if wl.k_pool is None:
        out.extra["n_pages"] = base + n_new
    return out


def draw_decode_tokens(cfg: Config, step: int, T_new: int):
    """K and V of decode step `step`'s T_new new tokens per session, pre-RoPE:
    [S][T_new][Hkv][d] in the storage dtype (bf16 as raw uint16 bits)."""
    shape = (cfg.n_sessions, T_new, cfg.n_kv_heads, cfg.head_dim)
    k = _rng(cfg.seed, _S_DEC_K, step).standard_normal(shape).astype(np.float32)
    v = _rng(cfg.seed, _S_DEC_V, step).standard_normal(shape).astype(np.float32)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return k, v
