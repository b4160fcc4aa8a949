"""Benchmark of the KVMem hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

(--workload c5 times the 10M-token, 512-token-chunk stress instead: one
workspace drawn on the device, score_select -> update_index -> materialize,
no attention; the scorer is reported against the bf16 matrix-core peak.)

One step is one recall step of the method over the 1M-token workspace
(1,048,576 tokens = 32,768 blocks; 64 query / 8 KV heads; d = 128; bf16):
    kvmem_score_select -> kvmem_update_index -> kvmem_materialize_attend
i.e. scoring and selection, the Mean-K index maintenance a step does (the
rows of the newest complete block), and the gather + re-RoPE with the step's
attention in one pass (it writes the same view as kvmem_materialize and
returns the attention over it; with more than 16 query rows per KV head,
kvmem_materialize -> kvmem_attend, which is faster there).  The step with the
two separate calls is timed as well ("separate_calls"), and so is a full
index build (stage "build_index_full", outside the steps).
Two independent copies of the workspace are used in turn, so the index a
scorer reads was last touched two steps earlier, with the gathers and
attentions of both copies (>4 GB of traffic, far beyond the 256 MB MALL) in
between.  Inputs are resident in HBM before the timed region.

Prints ONE JSON line.  `value` is blocks scored per second: the workspace's
complete blocks over the mean time of kvmem_score_select (HIP events recorded
on the stream the library launches on); whole-step throughput is
`step_blocks_per_s`.  `roofline` reports the dominant stage against the 8 TB/s
HBM peak using the algorithmic bytes of the method; `cpu_baseline` times the
CPU oracle stage by stage on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blocks scored/s + view decode-step latency (µs) at 1M-token workspace; % HBM peak"
HBM_PEAK = 8.0e12   # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15   # flop/s, MI355X dense bf16 matrix cores

# HBM bytes per launch of each stage's main kernel at the 1M-token workspace,
# from rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by a plain 1 GiB device
# copy (fetch x2.0, write x1.0); the summary and commands are in
# profiles/c3_1m_hbm_traffic.md.  Valid only for the kernel sources they were
# taken on (sha256 over block_sparse_decode_amd/csrc/* and build.py); otherwise reported null.
COUNTER_SOURCES_SHA = "0e7508d320a8fd8f53c0be728ecb56e0648b56baba751384cdcf3797966dc3cd"
MEASURED_TRAFFIC = {"build_index_full": 2.216e+09, "materialize_attend": 2.172e+09, "materialize": 2.156e+09,
                    "attend": 1.076e+09, "score_select": 9.208e+07}


def kernel_sources_sha() -> str:
    """sha256 over the kernel sources and the build script (its flags shape the code)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "block_sparse_decode_amd", "csrc", "*"))) + \
            [os.path.join(ROOT, "block_sparse_decode_amd", "build.py")]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def alg_bytes(cfg, n_blocks: int, view_tokens: int) -> dict:
    """Algorithmic bytes per call: what the method must move."""
    b = 2 if cfg.dtype == "bf16" else 4
    H, d = cfg.n_kv_heads, cfg.head_dim
    return {
        # read 32 keys, write one index row, per (block, KV head)
        "build_index": (32 + 1) * H * d * b * n_blocks,
        "build_index_full": (32 + 1) * H * d * b * n_blocks,
        # the newest complete block of every session
        "update_index": (32 + 1) * H * d * b * cfg.n_sessions,
        # read the index row of every (block, KV head), write A
        "score_select": (H * d * b + H * 4) * n_blocks,
        # read K and V of the selected tokens, write both into the view
        "materialize": 4 * H * d * b * view_tokens,
        # read K and V of the view once
        "attend": 2 * H * d * b * view_tokens,
        # the gather's bytes; the attention reads nothing more
        "materialize_attend": 4 * H * d * b * view_tokens,
    }


def alg_flops(cfg, n_blocks: int) -> float:
    """Scoring flops the method needs per call: 2 T Hq d per block."""
    return 2.0 * cfg.T * cfg.n_q_heads * cfg.head_dim * n_blocks


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_stages(wl, heads, threads=None) -> dict:
    """Seconds per stage of the oracle for the given KV heads of session 0
    (index, score + select, materialize, attend), BLAS threads limited to
    `threads` when given."""
    import contextlib

    from oracle import kvmem_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(threads) if threads else contextlib.nullcontext()
    except Exception:  # pragma: no cover
        lim = contextlib.nullcontext()
    cfg = wl.cfg
    ws = O.Workspace(wl.k_pool, wl.v_pool, wl.block_table, wl.n_tokens, cfg.dtype, cfg.n_q_heads,
                     cfg.n_kv_heads, cfg.head_dim)
    G = cfg.group
    n_tok = int(wl.n_tokens[0])
    t = {"index": 0.0, "score_select": 0.0, "materialize": 0.0, "attend": 0.0}
    with lim:
        qn = O.q_rmsnorm(O.decode(wl.q[0], cfg.dtype), wl.q_norm_w, cfg.eps)
        for h in heads:
            t0 = time.perf_counter()
            idx = O.mean_k_index(ws, 0, h)
            t1 = time.perf_counter()
            A = O.head_aggregate(qn[:, h * G:(h + 1) * G], idx)
            lst, V = O.view_list(A, n_tok, cfg.k_select, cfg.n_recent)
            t2 = time.perf_counter()
            kv, vv = O.materialize(ws, 0, h, lst, V, cfg.rope_theta)
            t3 = time.perf_counter()
            O.attend(qn[:, h * G:(h + 1) * G], kv, vv, cfg.rope_theta)
            t4 = time.perf_counter()
            for k, a, b in (("index", t0, t1), ("score_select", t1, t2), ("materialize", t2, t3),
                            ("attend", t3, t4)):
                t[k] += b - a
    return t


def cpu_baseline(wl, heads=None, small=("c1", "c2")) -> dict:
    """The oracle as it stands, timed stage by stage on a sample: the whole
    path for every KV head of session 0 (by default), with all BLAS threads
    and with one, scaled to the full workload; the same for the small
    workloads (two heads of c1 and of c2, scaled)."""
    from workloads import CONFIGS, make_workload
    if heads is None:
        heads = tuple(range(wl.cfg.n_kv_heads))
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    cfg = wl.cfg
    scale = cfg.n_kv_heads / len(heads)
    nb = int(wl.n_tokens[0]) // 32
    t_all = _oracle_stages(wl, heads)
    t_one = _oracle_stages(wl, heads, threads=1)
    per_all = {k: round(v * scale, 4) for k, v in t_all.items()}
    per_one = {k: round(v * scale, 4) for k, v in t_one.items()}
    sample_s = sum(t_all.values()) + sum(t_one.values())
    others = {}
    for name in small:
        c = CONFIGS[name]
        if c.name == cfg.name:
            continue
        w2 = make_workload(c)
        hs = tuple(range(min(2, c.n_kv_heads)))
        sc = c.n_kv_heads / len(hs)
        a = _oracle_stages(w2, hs)
        o = _oracle_stages(w2, hs, threads=1)
        sample_s += sum(a.values()) + sum(o.values())
        nb2 = int(w2.n_tokens[0]) // 32
        others[c.name] = {"seconds_per_stage": {k: round(v * sc, 5) for k, v in a.items()},
                          "seconds_per_stage_1_thread": {k: round(v * sc, 5) for k, v in o.items()},
                          "blocks_scored_per_s": round(nb2 / (a["score_select"] * sc), 1),
                          "heads_sampled": list(hs)}
    return {"value": nb / per_all["score_select"], "unit": "blocks/s", "cores": int(threads), "kind": "oracle",
            "cpu": cpu_model(), "host_cpus_available": len(os.sched_getaffinity(0)),
            "sample": f"oracle stages (index, score + select, view, attention) for KV heads {list(heads)} of "
                      f"{cfg.n_kv_heads} of session 0, with {threads} BLAS threads and with 1, scaled "
                      f"x{scale:.2f}; value = complete blocks / (score + select seconds per step) with all "
                      f"threads; numpy float64, elementwise work single-threaded; plus {', '.join(others)} "
                      f"({sample_s:.1f} s of CPU work in all)",
            "seconds_per_stage": per_all, "seconds_per_stage_1_thread": per_one,
            "blocks_scored_per_s_1_thread": nb / per_one["score_select"],
            "seconds_per_step": round(sum(per_all.values()), 4), "other_workloads": others}


def decode_loop(wl, dev, stream, n_dec: int) -> dict:
    """Decoding over a reused view: one selection and gather, then n_dec
    decode steps of (attention of one query token over the view, append of
    that token's K/V to the history and the view, Mean-K row of each block the
    history completes).  Timed per step with HIP events on the library's
    stream, after the view is built, in thirds: the first with events before
    the attention, between it and the append, and after the append (the
    attention / append breakdown); the second with the two calls and one event
    per step; the last with kvmem_attend_append (the attention, then the
    append on the attention's merge launch) and one event per step, the
    reported step latency.  (Each recorded event leaves the GPU idle for a few
    µs between the kernels it separates, so the step latencies take one event
    per interval, as the main step loop does.)"""
    import torch

    from block_sparse_decode_amd.pipeline import DeviceWorkspace, to_device
    from workloads import draw_decode_tokens, with_decode_capacity

    cfg = wl.cfg
    wd = with_decode_capacity(wl, n_dec)
    V_start = DeviceWorkspace.view_length_of(wd)
    V0 = int(max(V_start))
    dw = DeviceWorkspace(wd, dev, max_view=-(-(V0 + n_dec) // 32) * 32)
    kn, vn = draw_decode_tokens(cfg, 0, n_dec)
    kd, vd = to_device(kn, cfg.dtype, dev), to_device(vn, cfg.dtype, dev)
    toks = [(kd[:, t:t + 1].contiguous(), vd[:, t:t + 1].contiguous()) for t in range(n_dec)]
    dw.build_index(stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    dw.score_select(stream)
    ev[1].record(stream)
    dw.materialize(stream)
    ev[2].record(stream)
    # thirds: the breakdown (two calls, events between them); two calls with
    # one event per step; the fused call (kvmem_attend_append) with one event
    # per step
    n_two = n_dec // 3
    n_br = n_dec - 2 * n_two
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_br)]
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_two + 2)]
    for t in range(n_dec):
        if t < n_br:
            evs[t][0].record(stream)
            dw.attend(stream)
            evs[t][1].record(stream)
            dw.append(*toks[t], stream=stream)
            evs[t][2].record(stream)
        elif t < n_br + n_two:
            sev[t - n_br].record(stream)
            dw.attend(stream)
            dw.append(*toks[t], stream=stream)
        else:
            if t == n_br + n_two:
                sev[n_two].record(stream)             # end of the two-call third
            sev[t - n_br + 1].record(stream)
            dw.attend_append(*toks[t], stream=stream)
    sev[-1].record(stream)
    torch.cuda.synchronize()
    att = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    app_all = np.array([e[1].elapsed_time(e[2]) * 1e3 for e in evs])
    step_marked = att + app_all
    step_two = np.array([sev[i].elapsed_time(sev[i + 1]) * 1e3 for i in range(n_two)]) if n_two else step_marked
    step_us = np.array([sev[i].elapsed_time(sev[i + 1]) * 1e3 for i in range(n_two + 1, 2 * n_two + 1)]) \
        if n_two else step_marked
    recall = ev[0].elapsed_time(ev[2]) * 1e3
    # steps at which some session's history completes a block (index rows added)
    blocks_done = [t for t in range(n_br) if any((int(n) + t + 1) % 32 == 0 for n in wl.n_tokens)]
    plain = [t for t in range(n_br) if t not in blocks_done]
    app = app_all
    return {"tokens": n_dec, "view_tokens_start": int(np.sum(V_start)),
            "step_us_median": round(float(np.median(step_us)), 2),
            "step_us_median_two_calls": round(float(np.median(step_two)), 2),
            "step_us_median_three_events": round(float(np.median(step_marked)), 2),
            "attend_us_median": round(float(np.median(att)), 2),
            "append_us_median": round(float(np.median(app[plain])), 2),
            "append_with_index_update_us_median": round(float(np.median(app[blocks_done])), 2) if blocks_done else None,
            "attend_hbm_frac": round(2 * cfg.n_kv_heads * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)
                                     * int(np.sum(V_start)) / (np.median(att) * 1e-6) / HBM_PEAK, 4),
            "recall_us": round(recall, 2),
            "tokens_per_s_view_reused": round(n_dec / ((recall + float(np.median(step_us)) * n_dec) * 1e-6), 1),
            "tokens_per_s_reselect_each_token": round(1.0 / ((recall + float(np.median(att))) * 1e-6), 1)}


def paged_vs_view(wl, dev, stream, reps: int = 10) -> dict:
    """Attention straight from the pages against gather + attention over the
    view, on the same selection (HIP events, medians).  A view serving n
    decode tokens costs materialize + n * attend; reading the pages costs
    n * paged."""
    import torch

    from block_sparse_decode_amd.pipeline import DeviceWorkspace

    cfg = wl.cfg
    dw = DeviceWorkspace(wl, dev)
    dw.build_index(stream)
    dw.score_select(stream)
    dw.materialize(stream)
    dw.attend(stream)
    dw.attend_paged(stream=stream)
    torch.cuda.synchronize()

    def timed(fn):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    t_mat = timed(dw.materialize)
    t_att = timed(dw.attend)
    t_pg = timed(lambda st: dw.attend_paged(stream=st))
    t_fu = timed(lambda st: dw.materialize_attend(stream=st))
    V = int(np.sum(dw.view_tokens))
    nbytes = 2 * cfg.n_kv_heads * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4) * V
    breakeven = t_mat / (t_pg - t_att) if t_pg > t_att else None
    # n tokens over a view made in one pass: t_fu + (n - 1) t_att, against n t_pg
    breakeven_fu = (t_fu - t_att) / (t_pg - t_att) if t_pg > t_att else None
    return {"paged_us": round(t_pg, 2), "paged_hbm_frac": round(nbytes / (t_pg * 1e-6) / HBM_PEAK, 4),
            "view_attend_us": round(t_att, 2), "materialize_us": round(t_mat, 2),
            "materialize_attend_us": round(t_fu, 2),
            "tokens_per_view_breakeven": None if breakeven is None else round(breakeven, 1),
            "tokens_per_view_breakeven_one_pass": None if breakeven_fu is None else round(breakeven_fu, 1)}


HOST_LINK_PEAK = 64.0e9   # B/s per direction, PCIe Gen5 x16 (the MI355X host interface)


def host_tier(wl, dev, stream, reps: int = 5) -> dict:
    """Host-tier paging: the K/V pools in pinned host memory (read by the GPU
    in place), the Mean-K index built from them into HBM, then per recall step
    score_select -> kvmem_stage_view (the listed tiles over the host link into
    an HBM staging pool) -> the one-pass gather + attention on the staged pool.
    Reports the staged bytes per second against the link's peak, and the copy
    overlapped with decode attention of a device-resident copy of the
    workspace on another stream (normal priority) against the two back to
    back."""
    import torch

    from block_sparse_decode_amd.pipeline import DeviceWorkspace, StagedView

    cfg = wl.cfg
    dw = DeviceWorkspace(wl, dev, host_pools=True)

    def timed(fn, n=reps):
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    t_idx = timed(lambda: dw.build_index(stream), 2)
    t_ss = timed(lambda: dw.score_select(stream))
    st = StagedView(dw)
    t_st = timed(lambda: dw.stage(st, stream))
    t_ma = timed(lambda: dw.materialize_attend_staged(st, stream=stream))
    b = 2 if cfg.dtype == "bf16" else 4
    V = int(np.sum(dw.view_tokens))
    staged = 2 * cfg.n_kv_heads * cfg.head_dim * b * V
    idx_bytes = 32 * cfg.n_kv_heads * cfg.head_dim * b * int(np.sum(np.asarray(wl.n_tokens) // 32))
    # overlap: decode attention of a device-resident copy on another stream
    hb = DeviceWorkspace(wl, dev)
    hb.build_index(stream)
    hb.score_select(stream)
    hb.materialize(stream)
    torch.cuda.synchronize()
    t_att = timed(lambda: hb.attend(stream))
    n_att = max(1, int(t_st / t_att))
    t_atts = timed(lambda: [hb.attend(stream) for _ in range(n_att)], 3)
    s2 = torch.cuda.Stream(dev)
    tog = []
    for _ in range(3):
        torch.cuda.synchronize()
        a = time.perf_counter()
        dw.stage(st, s2)
        for _ in range(n_att):
            hb.attend(stream)
        torch.cuda.synchronize()
        tog.append((time.perf_counter() - a) * 1e6)
    return {"stage_us": round(t_st, 1), "staged_bytes": staged, "staged_GB/s": round(staged / t_st / 1e3, 2),
            "link_peak_GB/s": HOST_LINK_PEAK / 1e9, "link_frac": round(staged / (t_st * 1e-6) / HOST_LINK_PEAK, 4),
            "index_build_from_host_us": round(t_idx, 1),
            "index_build_from_host_GB/s": round(idx_bytes / t_idx / 1e3, 2),
            "score_select_us": round(t_ss, 2), "materialize_attend_staged_us": round(t_ma, 2),
            "recall_from_host_us": round(t_ss + t_st + t_ma, 1),
            "overlap": {"decode_attentions": n_att, "attention_us": round(t_att, 2),
                        "stage_alone_us": round(t_st, 1), "attentions_alone_us": round(t_atts, 1),
                        "back_to_back_us": round(t_st + t_atts, 1), "together_us": round(float(np.median(tog)), 1)}}


def mass_diagnostic(wl, dev, stream, reps: int = 5) -> dict:
    """Selection-quality diagnostic: share of full attention over the history
    that the selected blocks carry, and that the recent-only control (the
    recent blocks alone, same list length) carries.  Timed with HIP events;
    the kernel streams every history key once."""
    import torch

    from block_sparse_decode_amd.pipeline import DeviceWorkspace

    cfg = wl.cfg
    dw = DeviceWorkspace(wl, dev, with_v=False)
    dw.build_index(stream)
    dw.score_select(stream)
    S, H, T, Hq = cfg.n_sessions, cfg.n_kv_heads, cfg.T, cfg.n_q_heads
    rec = torch.full((S, H, dw.n_list), -1, dtype=torch.int32, device=dev)
    for s in range(S):                                  # each session's recent blocks, partial tail included
        nb_all = -(-int(wl.n_tokens[s]) // 32)
        r0 = max(0, nb_all - cfg.n_recent)
        rec[s, :, :nb_all - r0] = torch.arange(r0, nb_all, dtype=torch.int32, device=dev)
    mass = torch.empty((S, T, Hq), device=dev)
    m_rec = torch.empty((S, T, Hq), device=dev)
    dw.attention_mass(mass, stream=stream)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dw.attention_mass(mass, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    dw.attention_mass(m_rec, view_blocks=rec, stream=stream)
    torch.cuda.synchronize()
    t = float(np.median(ts))
    nbytes = int(np.sum(wl.n_tokens)) * H * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)
    return {"mass_selected_mean": round(float(mass.mean()), 4), "mass_selected_min": round(float(mass.min()), 4),
            "mass_recent_only_mean": round(float(m_rec.mean()), 4),
            "blocks_selected": cfg.k_select, "blocks_recent": cfg.n_recent,
            "us": round(t * 1e6, 2), "alg_bytes": nbytes, "hbm_frac": round(nbytes / t / HBM_PEAK, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-diagnostic", action="store_true",
                    help="skip the selection-quality diagnostic after the timed steps")
    ap.add_argument("--no-host-tier", action="store_true",
                    help="skip the host-tier paging measurement after the timed steps")
    ap.add_argument("--decode-tokens", type=int, default=256,
                    help="decode steps over one reused view after the timed steps (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run one plain 1 GiB device copy (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X here "
              "(sharding by KV head is a design note, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_sparse_decode_amd.pipeline import DeviceWorkspace
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    long_chunk = cfg.T * cfg.group > 32
    if long_chunk:
        # 41 GB of K/V: drawn chunk by chunk on the device, one copy (the 640 MB
        # index already exceeds the 256 MB MALL)
        wl = make_workload(cfg, pools=False)
        wss = [DeviceWorkspace(wl, dev)]
        stages = ["score_select", "update_index", "materialize"]
    else:
        wl = make_workload(cfg)
        wss = [DeviceWorkspace(wl, dev), DeviceWorkspace(wl, dev)]
        separate = ["score_select", "update_index", "materialize", "attend"]
        one_pass = cfg.dtype == "bf16" and cfg.T * cfg.group <= 16
        stages = ["score_select", "update_index", "materialize_attend"] if one_pass else separate
    print(f"[bench] workload {cfg.name} ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)
    for w in wss:
        w.build_index(stream)
    torch.cuda.synchronize()

    # the per-step index maintenance: rows of each session's newest complete block
    newest = np.maximum(np.asarray(wl.n_tokens) // 32 - 1, 0).astype(np.int32)

    def step(i, evs=None, stage_list=None):
        a = wss[i % len(wss)]
        calls = {"score_select": a.score_select, "materialize": a.materialize, "attend": a.attend,
                 "update_index": lambda st: a.update_index(newest, st),
                 "materialize_attend": lambda st: a.materialize_attend(stream=st)}
        stage_list = stages if stage_list is None else stage_list
        for j, name in enumerate(stage_list):
            if evs is not None:
                evs[j].record(stream)
            calls[name](stream)
        if evs is not None:
            evs[len(stage_list)].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {wall:.3f}s", file=sys.stderr, flush=True)

    # the full Mean-K index build (done once per workspace, not per step),
    # the copies alternating
    n_full = 10 if not long_chunk else 2
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_full)]
    for i in range(n_full):
        fev[i][0].record(stream)
        wss[i % len(wss)].build_index(stream)
        fev[i][1].record(stream)
    torch.cuda.synchronize()
    t_full = [e[0].elapsed_time(e[1]) * 1e-3 for e in fev]

    sep_rep = None
    if not long_chunk and stages != separate:
        # the same step with kvmem_materialize + kvmem_attend, for comparison
        n_sep = max(10, args.steps // 5)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(separate) + 1)] for _ in range(n_sep)]
        for i in range(3):
            step(i, stage_list=separate)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(n_sep):
            step(i, sev[i], stage_list=separate)
        torch.cuda.synchronize()
        wall_sep = time.perf_counter() - t1
        sep_rep = {"ms_per_step": round(wall_sep / n_sep * 1e3, 4), "steps": n_sep}
        for j, s in enumerate(separate):
            sep_rep[s + "_us"] = round(float(np.mean([e[j].elapsed_time(e[j + 1]) for e in sev])) * 1e3, 2)

    per = {s: [] for s in stages}
    for ev in events:
        for j, s in enumerate(stages):
            per[s].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)
    mean = {s: float(np.mean(v)) for s, v in per.items()}

    # every session of the step: complete blocks scored, view tokens gathered
    n_tok_all = int(np.sum(wl.n_tokens))
    nb = int(np.sum(np.asarray(wl.n_tokens) // 32))
    V = int(np.sum(wss[0].view_tokens))
    ab = alg_bytes(cfg, nb, V)
    stage_rep = {}
    for s in stages:
        gbs = ab[s] / mean[s] / 1e9
        stage_rep[s] = {"us": round(mean[s] * 1e6, 2), "us_median": round(float(np.median(per[s])) * 1e6, 2),
                        "us_p10": round(float(np.percentile(per[s], 10)) * 1e6, 2),
                        "us_p90": round(float(np.percentile(per[s], 90)) * 1e6, 2), "alg_bytes": int(ab[s]),
                        "GB/s": round(gbs, 1), "hbm_frac": round(gbs * 1e9 / HBM_PEAK, 4)}
    mf = float(np.mean(t_full))
    stage_rep["build_index_full"] = {"us": round(mf * 1e6, 2), "us_median": round(float(np.median(t_full)) * 1e6, 2),
                                     "launches": n_full, "alg_bytes": int(ab["build_index_full"]),
                                     "GB/s": round(ab["build_index_full"] / mf / 1e9, 1),
                                     "hbm_frac": round(ab["build_index_full"] / mf / HBM_PEAK, 4),
                                     "note": "outside the steps: the whole index of a copy, once per workspace"}
    fl = alg_flops(cfg, nb)
    stage_rep["score_select"]["alg_flops"] = fl
    stage_rep["score_select"]["TFLOP/s"] = round(fl / mean["score_select"] / 1e12, 2)
    dom = max(stages, key=lambda s: mean[s])
    ms_per_step = wall / args.steps * 1e3
    res = {
        "metric": METRIC,
        "value": nb / mean["score_select"],
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.n_sessions} session{'s' if cfg.n_sessions > 1 else ''}, "
                               f"{n_tok_all:,} tokens ({nb:,} blocks of 32), {cfg.n_q_heads} q heads / "
                               f"{cfg.n_kv_heads} KV heads, d={cfg.head_dim}, {cfg.dtype}, top-{cfg.k_select} + "
                               f"{cfg.n_recent} recent blocks per session -> {V:,} view tokens, T={cfg.T}",
                   "blocks": nb, "view_tokens": V, "query_tokens": cfg.T},
        "decode_step_latency_us": None,
        "recall_latency_us": round(stage_rep["score_select"]["us"] + stage_rep[stages[2]]["us"], 2),
        "step_blocks_per_s": nb / (wall / args.steps),
        "score_select_hbm_frac": stage_rep["score_select"]["hbm_frac"],
        "stages": stage_rep,
    }
    if sep_rep is not None:
        res["separate_calls"] = sep_rep
    if long_chunk:
        # prefill-style chunk: the scorer is a matrix-core contraction
        res["roofline"] = {"bound": "mfma", "kernel": "score_select", "achieved": round(fl / mean["score_select"] / 1e12, 2),
                           "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                           "frac": round(fl / mean["score_select"] / MFMA_BF16_PEAK, 4), "traffic": None}
    else:
        res["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(ab[dom] / mean[dom] / 1e9, 1),
                           "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": round(ab[dom] / mean[dom] / HBM_PEAK, 4),
                           "traffic": (MEASURED_TRAFFIC.get(dom) if args.workload == "c3"
                                       and kernel_sources_sha() == COUNTER_SOURCES_SHA else None)}
    if not long_chunk and args.decode_tokens > 0:
        wss.clear()                                   # frees the two timed workspaces
        torch.cuda.empty_cache()
        print(f"[bench] decode loop over one reused view ({args.decode_tokens} tokens) ...", file=sys.stderr, flush=True)
        dec = decode_loop(wl, dev, stream, args.decode_tokens)
        res["decode"] = dec
        res["decode_step_latency_us"] = dec["step_us_median"]
    if not long_chunk and not args.no_host_tier:
        print("[bench] host-tier paging (pinned host pools, staging over the host link) ...", file=sys.stderr,
              flush=True)
        res["host_tier"] = host_tier(wl, dev, stream)
        torch.cuda.empty_cache()
    if not long_chunk and not args.no_diagnostic:
        print("[bench] attention from the pages vs gather + view attention ...", file=sys.stderr, flush=True)
        res["paged_attend"] = paged_vs_view(wl, dev, stream)
        print("[bench] selection-quality diagnostic ...", file=sys.stderr, flush=True)
        res["selection_quality"] = mass_diagnostic(wl, dev, stream)
    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y
    if not args.no_cpu_baseline and not long_chunk:
        print("[bench] cpu baseline (oracle sample) ...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


if __name__ == "__main__":
    main()
