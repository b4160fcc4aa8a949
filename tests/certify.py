"""Selection-margin certification of generated workloads (test-side, uses the oracle).

Bit-exact comparison of the selected block set is only well posed when the
aggregated scores at the top-k cut are separated.  For every (session, KV
head) with a cut, this module computes A with the oracle and checks
    (A_(k) - A_(k+1)) / A_(k) >= tau
where A_(k) is the smallest selected and A_(k+1) the largest unselected
candidate.  When the gap is short it repairs the input: selected blocks whose
A lies within a few tau of the cut get their keys moved along the query
direction on the single coordinate where the group's normalised query is
largest (on all 32 tokens, so the block mean moves by the same amount), the
keys are re-rounded to the storage dtype, and the check is repeated on the
oracle's recomputed index.  It also checks that every candidate's A is at
least 1e-30, so that no denormal flush on either side can change a ranking.
"""
from __future__ import annotations

import numpy as np

from oracle import kvmem_oracle as O
from tests.helpers import oracle_ws
from workloads import Workload, f32_to_bf16_bits, bf16_bits_to_f32

TAU = 1e-3
A_FLOOR = 1e-30


def _cut_gap(A: np.ndarray, nc: int, k_eff: int):
    a = A[:nc]
    order = np.lexsort((np.arange(nc), -a))
    ak, ak1 = a[order[k_eff - 1]], a[order[k_eff]]
    return (ak - ak1) / ak, order, ak, ak1


def _shift_block_keys(wl: Workload, s: int, h: int, beta: int, i_star: int, delta: float):
    page = wl.block_table[s, beta]
    if wl.cfg.dtype == "bf16":
        x = bf16_bits_to_f32(wl.k_pool[page, h, :, i_star])
        wl.k_pool[page, h, :, i_star] = f32_to_bf16_bits(x + np.float32(delta))
    else:
        wl.k_pool[page, h, :, i_star] += np.float32(delta)


def certify(wl: Workload, tau: float = TAU, max_rounds: int = 40, t_chunk: int = 0) -> dict:
    """Repair `wl` in place until every cut is separated by tau.  Returns a
    report {(s, h): (rounds, blocks_moved, final_gap)}."""
    cfg = wl.cfg
    ws = oracle_ws(wl)
    G, H, d = cfg.group, cfg.n_kv_heads, cfg.head_dim
    report = {}
    for s in range(cfg.n_sessions):
        n_tok = int(wl.n_tokens[s])
        nc, _, _ = O.recent_split(n_tok, cfg.n_recent)
        k_eff = min(cfg.k_select, nc)
        qn = O.q_rmsnorm(O.decode(wl.q[s], cfg.dtype), wl.q_norm_w, cfg.eps)
        for h in range(H):
            if nc == 0:
                continue
            index = O.mean_k_index(ws, s, h)
            qg = qn[:, h * G:(h + 1) * G]
            qbar = qg.reshape(-1, d).mean(axis=0)
            i_star = int(np.argmax(np.abs(qbar)))
            sign = 1.0 if qbar[i_star] > 0 else -1.0
            base = 4.0 * tau * np.sqrt(d) / abs(qbar[i_star])          # shift of the block mean
            moved, rounds, gap = 0, 0, np.inf
            for rounds in range(max_rounds):
                A = O.head_aggregate(qg, index, t_chunk)
                assert A[:nc].min() >= A_FLOOR, (s, h, A[:nc].min())
                if k_eff == 0 or k_eff == nc:
                    break
                gap, order, ak, ak1 = _cut_gap(A, nc, k_eff)
                if gap >= tau:
                    break
                sel = order[:k_eff]
                near = sel[A[sel] <= ak1 * (1 + 3 * tau)]
                delta = sign * base * (1.5 ** rounds)
                for beta in near:
                    _shift_block_keys(wl, s, h, int(beta), i_star, delta)
                moved += len(near)
                index[near] = O.mean_k_rows(ws, s, h, near)
            else:
                raise RuntimeError(f"certify: no margin after {max_rounds} rounds at s={s} h={h}")
            report[(s, h)] = (rounds, moved, gap)
    return report


def chunk_workspace(wl: Workload, s: int, b0: int, chunk: np.ndarray) -> O.Workspace:
    """Oracle view of one drawn pool chunk (blocks b0 .. b0 + len(chunk) of
    session s as logical blocks 0 .. len(chunk) - 1 on pages 0 ..)."""
    c = wl.cfg
    nb = chunk.shape[0]
    n_tok = min(int(wl.n_tokens[s]) - 32 * b0, 32 * nb)
    return O.Workspace(chunk, None, np.arange(nb, dtype=np.int32)[None, :], np.array([n_tok]), c.dtype,
                       c.n_q_heads, c.n_kv_heads, c.head_dim)


def streamed_index(wl: Workload, threads: int | None = None) -> np.ndarray:
    """The oracle Mean-K index of session 0, every KV head, drawn chunk by
    chunk (for workspaces whose pools do not fit on the host): [H][Nb][d]."""
    from workloads import pool_chunks
    cfg = wl.cfg
    nb_full = int(wl.n_tokens[0]) // 32
    index = np.empty((cfg.n_kv_heads, nb_full, cfg.head_dim), np.float64)
    for s, b0, _, x in pool_chunks(wl, "k", threads):
        if s != 0:
            continue
        ws = chunk_workspace(wl, 0, b0, x)
        n = min(x.shape[0], nb_full - b0)
        for h in range(cfg.n_kv_heads):
            index[h, b0:b0 + n] = O.mean_k_rows(ws, 0, h, range(n))
    return index


def certify_streaming(wl: Workload, index: np.ndarray, tau: float = TAU, max_rounds: int = 40,
                      t_chunk: int = 16, log=print) -> tuple[list, dict, list]:
    """certify() for a single-session workload whose pools are drawn chunk by
    chunk: the repairs are appended to wl.extra["repairs"] (the generator
    replays them) and the repaired index rows are recomputed from redrawn
    chunks.  Returns (repair log, report, A per KV head)."""
    from workloads import pool_chunks
    cfg = wl.cfg
    G, H, d = cfg.group, cfg.n_kv_heads, cfg.head_dim
    n_tok = int(wl.n_tokens[0])
    nc, _, _ = O.recent_split(n_tok, cfg.n_recent)
    k_eff = min(cfg.k_select, nc)
    qn = O.q_rmsnorm(O.decode(wl.q[0], cfg.dtype), wl.q_norm_w, cfg.eps)
    wl.extra.setdefault("repairs", [])
    report, A_all = {}, []
    for h in range(H):
        qg = qn[:, h * G:(h + 1) * G]
        qbar = qg.reshape(-1, d).mean(axis=0)
        i_star = int(np.argmax(np.abs(qbar)))
        sign = 1.0 if qbar[i_star] > 0 else -1.0
        base = 4.0 * tau * np.sqrt(d) / abs(qbar[i_star])
        moved, gap = 0, np.inf
        for rounds in range(max_rounds):
            A = O.head_aggregate(qg, index[h], t_chunk)
            assert A[:nc].min() >= A_FLOOR, (h, A[:nc].min())
            if k_eff == 0 or k_eff == nc:
                break
            gap, order, ak, ak1 = _cut_gap(A, nc, k_eff)
            log(f"  head {h} round {rounds}: cut gap {gap:.3e}")
            if gap >= tau:
                break
            sel = order[:k_eff]
            near = [int(b) for b in sel[A[sel] <= ak1 * (1 + 3 * tau)]]
            delta = float(np.float32(sign * base * (1.5 ** rounds)))
            wl.extra["repairs"].extend((0, h, b, i_star, delta) for b in near)
            moved += len(near)
            jobs = sorted({(0, (b // 1024) * 1024, min((b // 1024 + 1) * 1024, -(-n_tok // 32))) for b in near})
            for s, b0, _, x in pool_chunks(wl, "k", jobs=jobs):
                ws = chunk_workspace(wl, 0, b0, x)
                loc = [b - b0 for b in near if b0 <= b < b0 + x.shape[0]]
                index[h, [b0 + i for i in loc]] = O.mean_k_rows(ws, 0, h, loc)
        else:
            raise RuntimeError(f"certify_streaming: no margin after {max_rounds} rounds at h={h}")
        report[h] = (rounds, moved, gap)
        A_all.append(A)
    return wl.extra["repairs"], report, A_all
