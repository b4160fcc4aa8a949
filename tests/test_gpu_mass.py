"""GPU parity of the selection-quality diagnostic (kvmem_attention_mass)
against the CPU oracle, through the C ABI.

Lists: the selection's own, the recent blocks only (the pages' control), all
blocks (mass 1) and none (mass 0).  Keys for the oracle are read straight
from the page table.  Bars: |mass - ref| <= 2e-4 + 1e-3 * ref (the logits
carry the query's hi/lo bf16 split and fp32 accumulation, ~1e-5 relative);
|lse - ref| <= 2e-3.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import kvmem_oracle as O
from tests.certify import certify
from tests.helpers import logical_tokens, make_workload, small_cfg
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

CASES = {
    "g8_ragged": small_cfg("mass_g8", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 300 + 5, 32 * 64),
                           k=24, R=3, n_planted=6, seed=101),
    "t2_g8": small_cfg("mass_t2", "bf16", S=1, Hq=16, Hkv=2, T=2, n_tokens=(32 * 500 + 17,),
                       k=40, R=4, n_planted=8, seed=102),
    "t4_g8_nine_heads": small_cfg("mass_t4", "bf16", S=1, Hq=72, Hkv=9, T=4, n_tokens=(32 * 130,),
                                  k=12, R=2, n_planted=3, seed=103),
    # fp32 workspaces (the vector-ALU kernel)
    "f32_t3_g4": small_cfg("mass_f32", "f32", S=2, Hq=8, Hkv=2, T=3, n_tokens=(32 * 200 + 9, 32 * 33),
                           k=12, R=2, n_planted=4, seed=104),
    "c1": CONFIGS["c1"],
}


def _lists(n_tok, H, n_list, kind):
    """[H][n_list] int32 lists of one session: the recent blocks only (the
    pages' control, 8 blocks) or every block."""
    nb_all = -(-n_tok // 32)
    out = np.full((H, n_list), -1, np.int32)
    if kind == "recent":
        r0 = max(0, nb_all - 8)
        out[:, :nb_all - r0] = np.arange(r0, nb_all)
    elif kind == "all":
        out[:, :nb_all] = np.arange(nb_all)
    return out


def _check(wl, dw, kinds=("selected", "recent", "all", "none"), heads=None):
    cfg = wl.cfg
    S, H, T, Hq, G = cfg.n_sessions, cfg.n_kv_heads, cfg.T, cfg.n_q_heads, cfg.group
    heads = range(H) if heads is None else heads
    gpu_sel = dw.view_blocks.cpu().numpy()
    for kind in kinds:
        n_list = 0 if kind == "none" else max(dw.n_list, max(-(-int(n) // 32) for n in wl.n_tokens))
        lists = np.full((S, H, max(1, n_list)), -1, np.int32)
        for s in range(S):
            if not n_list:
                continue
            if kind == "selected":
                lists[s, :, :gpu_sel.shape[2]] = gpu_sel[s]
            else:
                lists[s] = _lists(int(wl.n_tokens[s]), H, n_list, kind)
        vb = torch.from_numpy(lists).cuda()
        mass = torch.full((S, T, Hq), float("nan"), device="cuda")
        lse = torch.full((S, T, Hq), float("nan"), device="cuda")
        dw.attention_mass(mass, lse, view_blocks=vb, n_list=n_list)
        torch.cuda.synchronize()
        m_gpu, l_gpu = mass.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        for s in range(S):
            qn = O.q_rmsnorm(O.decode(wl.q[s], cfg.dtype), wl.q_norm_w, cfg.eps)
            for h in heads:
                keys = logical_tokens(wl, wl.k_pool, s, h)
                listed = [b for b in lists[s, h, :n_list] if b >= 0] if n_list else []
                m_ref, l_ref = O.attention_mass(qn[:, h * G:(h + 1) * G], keys, listed, cfg.rope_theta, cfg.dtype)
                mg, lg = m_gpu[s, :, h * G:(h + 1) * G], l_gpu[s, :, h * G:(h + 1) * G]
                assert np.all(np.abs(mg - m_ref) <= 2e-4 + 1e-3 * m_ref), (cfg.name, kind, s, h, mg, m_ref)
                assert np.all(np.abs(lg - l_ref) <= 2e-3), (cfg.name, kind, s, h, lg, l_ref)
        print(f"[gpu] mass {cfg.name} {kind}: mean {m_gpu.mean():.4f}", flush=True)
    assert int(dw.dev_error.item()) == 0


@pytest.mark.parametrize("name", list(CASES))
def test_mass_parity(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd.pipeline import DeviceWorkspace
    wl = make_workload(CASES[name])
    certify(wl)
    print(f"[gpu] mass {name} N={list(wl.n_tokens)}", flush=True)
    dw = DeviceWorkspace(wl, "cuda")
    dw.build_index()
    dw.score_select()
    torch.cuda.synchronize()
    _check(wl, dw)


def test_mass_c2_full():
    """The 256K-token workload (8 KV heads, one per wavefront of a
    workgroup); heads 0 and 7 checked against the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd.pipeline import DeviceWorkspace
    wl = make_workload(CONFIGS["c2"])
    print(f"[gpu] mass c2 N={list(wl.n_tokens)}", flush=True)
    dw = DeviceWorkspace(wl, "cuda")
    dw.build_index()
    dw.score_select()
    torch.cuda.synchronize()
    _check(wl, dw, kinds=("selected", "recent"), heads=(0, 7))
