"""GPU parity of attention straight from the pages (kvmem_attend_paged)
against the oracle's gather + attention and against the library's own view
attention, through the C ABI; and of the one-pass gather + attention
(kvmem_materialize_attend), whose view must equal kvmem_materialize's bit for
bit (slots past the last view block untouched) and whose output must equal
kvmem_attend_paged's bit for bit (same kernel, same keys, same order).

Bars: the attention bar against the oracle (2e-2 max-abs for bf16) and the
regression bar of the parity tests (1e-3 of the head's largest output plus
2e-6) against the oracle and against the view attention; against
kvmem_materialize + kvmem_attend on the same lists <= 5e-5 max-abs: the same
rounded keys and operands, only the split structure, hence the order of the
fp32 sums, differs (over up to 2^18 terms: ~sqrt(n) * 2^-24 * |o| ~ 3e-5).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import kvmem_oracle as O
from tests.certify import certify
from tests.helpers import make_workload, oracle_ws, small_cfg
from tests.test_gpu_parity import ATT_TOL, SMALL, reg_bar
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

CASES = {n: SMALL[n] for n in ("bf16_ragged", "bf16_t2_g8", "bf16_t4_g8", "bf16_g1", "recent_only",
                               "budget_covers_all", "r0_partial", "empty_and_tiny")}
# fp32 workspaces (the vector-ALU kernel): ragged with a partial tail, three
# query tokens, and the tiny fp32 workload
CASES.update({n: SMALL[n] for n in ("f32_ragged", "f32_t3_g4")})
CASES["c1"] = CONFIGS["c1"]
CASES["nine_heads"] = small_cfg("paged_nine_heads", "bf16", S=2, Hq=18, Hkv=9, n_tokens=(32 * 210 + 3, 32 * 90),
                                k=30, R=3, n_planted=4, seed=111)
# workgroups hold the largest divisor of Hkv up to 8 wavefronts: one (Hkv = 1),
# five (a prime), and two groups of six (Hkv = 12)
CASES["one_head"] = small_cfg("paged_one_head", "bf16", S=2, Hq=8, Hkv=1, n_tokens=(32 * 150 + 9, 32 * 40),
                              k=20, R=2, n_planted=4, seed=112)
CASES["five_heads"] = small_cfg("paged_five_heads", "bf16", S=2, Hq=10, Hkv=5, n_tokens=(32 * 95 + 30, 32 * 61),
                                k=14, R=3, n_planted=3, seed=113)
CASES["twelve_heads"] = small_cfg("paged_twelve_heads", "bf16", S=1, Hq=48, Hkv=12, n_tokens=(32 * 120 + 1,),
                                  k=16, R=2, n_planted=3, seed=114)
# two list blocks per split, strided over the view (workgroup j: blocks j,
# j + n_splits, ...): session 0 has 96 splits, which the kernel permutes across
# XCDs (96 = the launch's width, a multiple of 8), session 1 has 75 (no
# permutation) and takes every candidate (budget above its history)
CASES["strided_splits"] = small_cfg("paged_strided", "bf16", S=2, Hq=64, Hkv=8, n_tokens=(32 * 400 + 5, 32 * 150),
                                    k=188, R=4, n_planted=6, seed=115)


def _run(wl, heads=None):
    from block_sparse_decode_amd.pipeline import DeviceWorkspace
    cfg = wl.cfg
    print(f"[gpu] paged {cfg.name} N={list(wl.n_tokens)[:4]} T={cfg.T} k={cfg.k_select} R={cfg.n_recent}", flush=True)
    dw = DeviceWorkspace(wl, "cuda")
    dw.build_index()
    dw.score_select()
    dw.materialize()
    dw.attend()
    torch.cuda.synchronize()
    out_view = dw.out.cpu().numpy().astype(np.float64)
    out_p = torch.full_like(dw.out, float("nan"))
    dw.attend_paged(out=out_p)
    torch.cuda.synchronize()
    out_paged = out_p.cpu().numpy().astype(np.float64)
    assert int(dw.dev_error.item()) == 0
    d = float(np.abs(out_paged - out_view).max())
    assert d <= 5e-5, (cfg.name, "paged vs view", d)
    for s in range(cfg.n_sessions):
        for h in range(cfg.n_kv_heads):
            o_v = out_view[s, :, h * cfg.group:(h + 1) * cfg.group]
            dd = float(np.abs(out_paged[s, :, h * cfg.group:(h + 1) * cfg.group] - o_v).max())
            assert dd <= reg_bar(o_v), (cfg.name, s, h, "paged vs view, regression bar", dd)

    # one pass: the view as the gather writes it, the output as the paged attention's
    k_ref, v_ref = dw.k_view.clone(), dw.v_view.clone()
    sentinel = 0x5A5A
    dw.k_view.view(torch.int16).fill_(sentinel)
    dw.v_view.view(torch.int16).fill_(sentinel)
    out_f = torch.full_like(dw.out, float("nan"))
    dw.materialize_attend(out=out_f)
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0
    assert torch.equal(out_f.view(torch.int32), out_p.view(torch.int32)), (cfg.name, "fused vs paged output")
    for s in range(cfg.n_sessions):
        nb = (int(dw.view_tokens[s]) + 31) // 32
        kf, vf = dw.k_view[s].view(torch.int16), dw.v_view[s].view(torch.int16)
        assert torch.equal(kf[:, :32 * nb], k_ref[s].view(torch.int16)[:, :32 * nb]), (cfg.name, s, "fused K view")
        assert torch.equal(vf[:, :nb], v_ref[s].view(torch.int16)[:, :nb]), (cfg.name, s, "fused V view")
        assert bool((kf[:, 32 * nb:] == sentinel).all()) and bool((vf[:, nb:] == sentinel).all()), (cfg.name, s)
    ws = oracle_ws(wl)
    G = cfg.group
    vb = dw.view_blocks.cpu().numpy()
    heads = range(cfg.n_kv_heads) if heads is None else heads
    worst = 0.0
    for s in range(cfg.n_sessions):
        qn = O.q_rmsnorm(O.decode(wl.q[s], cfg.dtype), wl.q_norm_w, cfg.eps)
        V = int(dw.view_tokens[s])
        for h in heads:
            lst = vb[s, h][vb[s, h] >= 0].astype(np.int64)
            kv, vv = O.materialize(ws, s, h, lst, V, cfg.rope_theta)
            o_ref = O.attend(qn[:, h * G:(h + 1) * G], kv, vv, cfg.rope_theta)
            err = float(np.abs(out_paged[s, :, h * G:(h + 1) * G] - o_ref).max()) if V else \
                float(np.abs(out_paged[s, :, h * G:(h + 1) * G]).max())
            worst = max(worst, err / reg_bar(o_ref))
            assert err <= ATT_TOL[cfg.dtype], (cfg.name, s, h, err)
            assert err <= reg_bar(o_ref), (cfg.name, s, h, "regression bar", err, reg_bar(o_ref))
    print(f"[gpu] paged {cfg.name}: |paged - view| {d:.2e}, |paged - oracle| / regression bar {worst:.3f}; one-pass view and output"
          " bit-identical", flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_paged_parity(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = make_workload(CASES[name])
    certify(wl)
    _run(wl)


def test_paged_c3_full():
    """The 1M-token workspace: 8192-block lists, 256 splits per head; two
    heads against the oracle, all heads against the view attention."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = make_workload(CONFIGS["c3"])
    _run(wl, heads=(0, 7))
