"""Writes tests/golden/c5_10m_golden.npz: oracle results for the 10M-token,
512-query-token workload (too large to recompute inside a test).

Run from the repository root:  python -m tests.golden.make_c5_golden
It draws the workload chunk by chunk, builds the oracle Mean-K index,
certifies a selection margin at every top-k cut (logging the key repairs the
certification makes, which the generator replays), and stores: the repair
log, the view block list of every KV head, the view length, and the oracle's
aggregated score A on every selected block and on a seeded sample of the
other candidates.  Only oracle/, workloads/ and tests/certify.py are used.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

from oracle import kvmem_oracle as O
from tests.certify import TAU, certify_streaming, streamed_index
from workloads import CONFIGS, make_workload

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c5_10m_golden.npz")


def main():
    cfg = CONFIGS["c5"]
    t0 = time.time()
    wl = make_workload(cfg, pools=False)
    n_tok = int(wl.n_tokens[0])
    index = streamed_index(wl)
    print(f"index {index.shape} in {time.time() - t0:.0f} s", flush=True)
    repairs, report, A_all = certify_streaming(wl, index, TAU, log=lambda m: print(m, flush=True))
    print(f"certified in {time.time() - t0:.0f} s: {report}", flush=True)
    lists, samples, a_samp = [], [], []
    nc, _, _ = O.recent_split(n_tok, cfg.n_recent)
    rng = np.random.default_rng(12345)
    for h, A in enumerate(A_all):
        lst, V = O.view_list(A, n_tok, cfg.k_select, cfg.n_recent)
        lists.append(lst)
        other = np.setdiff1d(np.arange(nc), lst)
        pick = np.concatenate([lst[lst < nc], rng.choice(other, size=2048, replace=False)])
        samples.append(pick)
        a_samp.append(A[pick])
    np.savez_compressed(OUT, repairs=np.array(repairs, dtype=np.float64).reshape(-1, 5),
                        lists=np.stack(lists).astype(np.int32), view_tokens=np.int64(V),
                        a_blocks=np.stack(samples).astype(np.int32), a_values=np.stack(a_samp),
                        a_sums=np.array([A[:nc].sum() for A in A_all]),
                        gaps=np.array([report[h][2] for h in range(len(A_all))]))
    print(f"wrote {OUT} ({os.path.getsize(OUT)} bytes) in {time.time() - t0:.0f} s")


if __name__ == "__main__":
    sys.exit(main())
