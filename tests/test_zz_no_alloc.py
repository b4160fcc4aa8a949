"""kvmem_attend_noalloc (kvmem_attend with the library's own scratch array,
for callers that cannot allocate) against kvmem_attend, through the C ABI:
two calls in a row, the second with a smaller input (fewer sessions, shorter
views, other heads), each output bit for bit equal to kvmem_attend's on the
same views (same kernels, same split structure), and within the attention
bars against the oracle on a head of each case."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import kvmem_oracle as O
from tests.certify import certify
from tests.helpers import make_workload, oracle_ws, small_cfg
from tests.test_gpu_parity import ATT_TOL, reg_bar
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

CASES = [CONFIGS["c2"],
         small_cfg("noalloc_small", "bf16", S=3, Hq=16, Hkv=2, T=2, n_tokens=(32 * 300 + 5, 32 * 64, 7),
                   k=24, R=3, n_planted=6, seed=121)]


def _views(cfg):
    from block_sparse_decode_amd.pipeline import DeviceWorkspace
    wl = make_workload(cfg)
    certify(wl)
    dw = DeviceWorkspace(wl, "cuda")
    dw.build_index()
    dw.score_select()
    dw.materialize()
    dw.attend()
    torch.cuda.synchronize()
    return wl, dw


def test_noalloc_attend_matches_attend():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd import _lib as L
    for cfg in CASES:
        wl, dw = _views(cfg)
        need = L.kvmem_attend_scratch_bytes(dw.geom, dw.S, dw.T, dw.max_view)
        assert 0 < need <= L.NOALLOC_SCRATCH_BYTES
        print(f"[gpu] noalloc {cfg.name}: S={dw.S} T={dw.T} V={list(dw.view_tokens)} scratch {need} B", flush=True)
        out = torch.full_like(dw.out, float("nan"))
        L.kvmem_attend_noalloc(dw.geom, dw.S, dw.q, dw.T, dw.q_norm_w, dw.eps, dw.k_view, dw.v_view,
                               dw.view_tokens, dw.max_view, dw.theta, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), dw.out.view(torch.int32)), cfg.name
        # the attention bars against the oracle, one head per session
        ws = oracle_ws(wl)
        G = cfg.group
        vb = dw.view_blocks.cpu().numpy()
        o = out.cpu().numpy().astype(np.float64)
        for s in range(cfg.n_sessions):
            h = s % cfg.n_kv_heads
            qn = O.q_rmsnorm(O.decode(wl.q[s], cfg.dtype), wl.q_norm_w, cfg.eps)
            lst = vb[s, h][vb[s, h] >= 0].astype(np.int64)
            kv, vv = O.materialize(ws, s, h, lst, int(dw.view_tokens[s]), cfg.rope_theta)
            o_ref = O.attend(qn[:, h * G:(h + 1) * G], kv, vv, cfg.rope_theta)
            err = float(np.abs(o[s, :, h * G:(h + 1) * G] - o_ref).max()) if len(kv) else float(np.abs(o[s]).max())
            assert err <= ATT_TOL[cfg.dtype] and err <= reg_bar(o_ref), (cfg.name, s, h, err)
        del dw
        torch.cuda.empty_cache()
