"""More sessions than one launch takes (64): every entry point splits the
batch into launches of at most 64 sessions with a session offset.  70 ragged
sessions (empty, partial-tail and multi-block histories) through the whole
path, checked against the oracle on sessions on both sides of the split,
including the last one."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import kvmem_oracle as O
from tests.helpers import logical_tokens, make_workload, oracle_ws, small_cfg
from tests.test_gpu_parity import ATT_TOL, reg_bar

pytestmark = pytest.mark.gpu

S = 70
CHECK = (0, 1, 62, 63, 64, 65, 69)


def _lengths():
    rng = np.random.default_rng(141)
    n = rng.integers(0, 32 * 40, S)
    n[[0, 63, 64, 69]] = [0, 32 * 33 + 7, 5, 32 * 40]
    return tuple(int(x) for x in n)


def test_seventy_sessions():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd import _lib as L
    from block_sparse_decode_amd.pipeline import DeviceWorkspace, index_rows, v_view_token_major
    cfg = small_cfg("seventy", "bf16", S=S, Hq=8, Hkv=2, n_tokens=_lengths(), k=6, R=2, n_planted=3, seed=142)
    wl = make_workload(cfg)
    print(f"[gpu] {S} sessions, lengths {list(wl.n_tokens)[:8]} ...", flush=True)
    dw = DeviceWorkspace(wl, "cuda")
    ag = torch.full((S, cfg.n_kv_heads, dw.max_blocks), float("nan"), device="cuda")
    dw.build_index()
    dw.score_select(agg=ag)
    dw.materialize()
    dw.attend()
    torch.cuda.synchronize()
    out_view = dw.out.clone()
    out_p = torch.full_like(dw.out, float("nan"))
    dw.attend_paged(out=out_p)
    mass = torch.full((S, cfg.T, cfg.n_q_heads), float("nan"), device="cuda")
    dw.attention_mass(mass)
    out_na = torch.full_like(dw.out, float("nan"))
    L.kvmem_attend_noalloc(dw.geom, dw.S, dw.q, dw.T, dw.q_norm_w, dw.eps, dw.k_view, dw.v_view, dw.view_tokens,
                           dw.max_view, dw.theta, out_na)
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0
    assert torch.equal(out_na.view(torch.int32), out_view.view(torch.int32))
    assert float((out_p - out_view).abs().max()) <= 5e-5
    # the one-pass gather + attention: the same view, the paged attention's output
    k_ref, v_ref = dw.k_view.clone(), dw.v_view.clone()
    dw.k_view.view(torch.int16).fill_(0x5A5A)
    dw.v_view.view(torch.int16).fill_(0x5A5A)
    out_f = torch.full_like(dw.out, float("nan"))
    dw.materialize_attend(out=out_f)
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0
    assert torch.equal(out_f.view(torch.int32), out_p.view(torch.int32))
    for s in range(S):
        nb = (int(dw.view_tokens[s]) + 31) // 32
        assert torch.equal(dw.k_view[s].view(torch.int16)[:, :32 * nb], k_ref[s].view(torch.int16)[:, :32 * nb]), s
        assert torch.equal(dw.v_view[s].view(torch.int16)[:, :nb], v_ref[s].view(torch.int16)[:, :nb]), s
    ws = oracle_ws(wl)
    G = cfg.group
    idx = index_rows(dw.index, dw.max_blocks)
    kview = dw.k_view.view(torch.int16).cpu().numpy().view(np.uint16)
    vview = v_view_token_major(dw.v_view).contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    vb = dw.view_blocks.cpu().numpy()
    A = ag.cpu().numpy().astype(np.float64)
    o = out_view.cpu().numpy().astype(np.float64)
    m = mass.cpu().numpy().astype(np.float64)
    for s in CHECK:
        n_tok = int(wl.n_tokens[s])
        nb = n_tok // 32
        qn = O.q_rmsnorm(O.decode(wl.q[s], cfg.dtype), wl.q_norm_w, cfg.eps)
        assert int(dw.view_tokens[s]) == O.view_tokens(n_tok, cfg.k_select, cfg.n_recent), s
        for h in range(cfg.n_kv_heads):
            index = O.mean_k_index(ws, s, h)
            got = O.decode(idx[s, h, :nb].contiguous().view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
            assert np.array_equal(got, index), (s, h, "index")
            A_ref = O.head_aggregate(qn[:, h * G:(h + 1) * G], index)
            assert np.all(np.abs(A[s, h, :nb] - A_ref) <= 1e-3 * A_ref + 1e-30), (s, h, "A")
            lst, V = O.view_list(A_ref, n_tok, cfg.k_select, cfg.n_recent)
            want = np.full(dw.n_list, -1)
            want[:len(lst)] = lst
            assert np.array_equal(vb[s, h], want), (s, h, "list")
            kv, vv = O.materialize(ws, s, h, lst, V, cfg.rope_theta)
            assert np.array_equal(O.decode(vview[s, h, :V], "bf16"), vv), (s, h, "V view")
            kg = O.decode(kview[s, h, :V], "bf16")
            ulp = np.ldexp(1.0, np.frexp(np.abs(kv))[1] - 8)
            assert np.all(np.abs(kg - kv) <= ulp + 1e-6 * np.abs(kv).max(axis=-1, keepdims=True)), (s, h, "K view")
            o_ref = O.attend(qn[:, h * G:(h + 1) * G], kv, vv, cfg.rope_theta)
            err = float(np.abs(o[s, :, h * G:(h + 1) * G] - o_ref).max()) if V else float(np.abs(o[s]).max())
            assert err <= ATT_TOL["bf16"] and err <= reg_bar(o_ref), (s, h, "attend", err)
            keys = logical_tokens(wl, wl.k_pool, s, h)
            m_ref, _ = O.attention_mass(qn[:, h * G:(h + 1) * G], keys, list(lst), cfg.rope_theta, "bf16")
            mg = m[s, :, h * G:(h + 1) * G]
            assert np.all(np.abs(mg - m_ref) <= 2e-4 + 1e-3 * m_ref), (s, h, "mass", mg, m_ref)
    print(f"[gpu] {S} sessions: index, A, lists, view, attention (view, pages, one pass, scratch-free) and mass match "
          f"on sessions {CHECK}", flush=True)
