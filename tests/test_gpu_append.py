"""GPU parity of decoding over a reused view (append + incremental index),
through the C ABI, against the CPU oracle.

After one selection and gather, three appends (45, 35, 3 tokens: the first two cross
history-block and view-block boundaries, the third does not) each followed by
attention.  Bars:
pools bit-exact (every page, spare pages included), index rows bit-exact, V
view bit-exact, K view within one bf16 ulp (the gather's bar), the view's tail
slots zero, attention within the attention bar and the regression bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import kvmem_oracle as O
from tests.certify import certify
from tests.helpers import make_workload, oracle_ws, small_cfg
from tests.test_gpu_parity import ATT_TOL, _bits_to_f64, reg_bar
from workloads import draw_decode_tokens, with_decode_capacity

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_g8": small_cfg("dec_bf16_g8", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 300 + 5, 32 * 64),
                         k=24, R=3, n_planted=6, seed=81),
    "f32_g4": small_cfg("dec_f32_g4", "f32", S=2, Hq=8, Hkv=2, n_tokens=(32 * 200 + 31, 32 * 40),
                        k=10, R=2, n_planted=4, seed=82),
}
STEPS = (45, 35, 3)             # the third stays inside a view block the second opened


def _raw_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _raw_np(a: np.ndarray) -> np.ndarray:
    return a.view(np.int16) if a.dtype == np.uint16 else a.view(np.int32)


@pytest.mark.parametrize("name", list(CASES))
def test_append_parity(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd.pipeline import DeviceWorkspace, index_rows, to_device, v_view_token_major
    cfg = CASES[name]
    wl0 = make_workload(cfg)
    certify(wl0)
    extra = sum(STEPS)
    wl = with_decode_capacity(wl0, extra)
    V0 = [O.view_tokens(int(n), cfg.k_select, cfg.n_recent) for n in wl.n_tokens]
    max_view = -(-(max(V0) + extra) // 32) * 32
    print(f"[gpu] append {name} N={list(wl.n_tokens)} V={V0} steps={STEPS}", flush=True)
    dw = DeviceWorkspace(wl, "cuda", max_view=max_view)
    dw.build_index()
    dw.score_select()
    dw.materialize()
    torch.cuda.synchronize()

    ws = oracle_ws(wl)
    S, H, G = cfg.n_sessions, cfg.n_kv_heads, cfg.group
    views = {}
    vb = dw.view_blocks.cpu().numpy()
    for s in range(S):
        index = [O.mean_k_index(ws, s, h) for h in range(H)]
        _, A_all, _ = O.session_scores(ws, s, wl.q[s], wl.q_norm_w, cfg.eps, index, keep_scores=False)
        for h in range(H):
            lst, V = O.view_list(A_all[h], int(wl.n_tokens[s]), cfg.k_select, cfg.n_recent)
            assert np.array_equal(vb[s, h, :len(lst)], lst), (name, s, h, "list")
            views[s, h] = O.materialize(ws, s, h, lst, V, cfg.rope_theta)

    for step, T_new in enumerate(STEPS):
        kn, vn = draw_decode_tokens(cfg, step, T_new)
        dw.append(to_device(kn, cfg.dtype, "cuda"), to_device(vn, cfg.dtype, "cuda"))
        dw.attend()
        torch.cuda.synchronize()
        for s in range(S):
            ws = O.append_history(ws, s, kn[s], vn[s])
            for h in range(H):
                kv, vv = views[s, h]
                views[s, h] = O.append_view(kv, vv, O.decode(kn[s, :, h], cfg.dtype), O.decode(vn[s, :, h], cfg.dtype),
                                            cfg.rope_theta, cfg.dtype)
        assert np.array_equal(dw.n_tokens, ws.n_tokens), (name, step)
        # pools: every page, bit for bit
        assert np.array_equal(_raw_bits(dw.k_pool), _raw_np(ws.k_pool)), (name, step, "K pool")
        assert np.array_equal(_raw_bits(dw.v_pool), _raw_np(ws.v_pool)), (name, step, "V pool")
        idx = _bits_to_f64(index_rows(dw.index, dw.max_blocks).contiguous(), cfg.dtype)
        kview = _bits_to_f64(dw.k_view, cfg.dtype)
        vview = _bits_to_f64(v_view_token_major(dw.v_view).contiguous(), cfg.dtype)
        out = dw.out.cpu().numpy().astype(np.float64)
        for s in range(S):
            qn = O.q_rmsnorm(O.decode(wl.q[s], cfg.dtype), wl.q_norm_w, cfg.eps)
            nb = int(ws.n_tokens[s]) // 32
            for h in range(H):
                assert np.array_equal(idx[s, h, :nb], O.mean_k_index(ws, s, h)), (name, step, s, h, "index")
                kv, vv = views[s, h]
                V = kv.shape[0]
                assert V == int(dw.view_tokens[s])
                assert np.array_equal(vview[s, h, :V], vv), (name, step, s, h, "V view")
                rot = 1e-6 * np.abs(kv).max(axis=-1, keepdims=True)
                if cfg.dtype == "bf16":
                    ulp = np.ldexp(1.0, np.frexp(np.abs(kv))[1] - 8)
                    assert np.all(np.abs(kview[s, h, :V] - kv) <= ulp + rot), (name, step, s, h, "K view")
                else:
                    assert np.all(np.abs(kview[s, h, :V] - kv) <= 2e-7 * np.abs(kv) + rot), (name, step, s, h, "K view")
                end = -(-V // 32) * 32
                assert np.all(kview[s, h, V:end] == 0) and np.all(vview[s, h, V:end] == 0), (name, step, "tail")
                o_ref = O.attend(qn[:, h * G:(h + 1) * G], kv, vv, cfg.rope_theta)
                err = float(np.abs(out[s, :, h * G:(h + 1) * G] - o_ref).max())
                assert err <= ATT_TOL[cfg.dtype], (name, step, s, h, "attend", err)
                assert err <= reg_bar(o_ref), (name, step, s, h, "attend regression bar", err, reg_bar(o_ref))
    assert int(dw.dev_error.item()) == 0


# kvmem_attend_append against kvmem_attend + kvmem_append: the same kernels'
# results, so every output, pool, view and index word must match bit for bit.
# The wide case has 51 splits, so its append rides on the merge that folds
# split groups (the small ones on the narrow merge).
FUSED = dict(CASES)
FUSED["bf16_wide"] = small_cfg("dec_bf16_wide", "bf16", S=1, Hq=8, Hkv=1, n_tokens=(32 * 600 + 7,),
                               k=200, R=4, n_planted=6, seed=83)


@pytest.mark.parametrize("name", list(FUSED))
def test_attend_append_matches_two_calls(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd.pipeline import DeviceWorkspace, to_device
    cfg = FUSED[name]
    extra = sum(STEPS)
    wl = with_decode_capacity(make_workload(cfg), extra)
    V0 = [O.view_tokens(int(n), cfg.k_select, cfg.n_recent) for n in wl.n_tokens]
    max_view = -(-(max(V0) + extra) // 32) * 32
    print(f"[gpu] attend_append {name} N={list(wl.n_tokens)} V={V0} steps={STEPS}", flush=True)
    two, one = DeviceWorkspace(wl, "cuda", max_view=max_view), DeviceWorkspace(wl, "cuda", max_view=max_view)
    for dw in (two, one):
        # equal starting contents everywhere the comparison looks (the views
        # and the index are allocated uninitialised past what the calls write)
        for buf in (dw.k_view, dw.v_view, dw.index):
            buf.zero_()
        dw.build_index()
        dw.score_select()
        dw.materialize()
    torch.cuda.synchronize()
    for step, T_new in enumerate(STEPS):
        kn, vn = draw_decode_tokens(cfg, step, T_new)
        kd, vd = to_device(kn, cfg.dtype, "cuda"), to_device(vn, cfg.dtype, "cuda")
        two.attend()
        two.append(kd, vd)
        one.attend_append(kd, vd)
        torch.cuda.synchronize()
        assert int(one.dev_error.item()) == 0
        assert np.array_equal(one.n_tokens, two.n_tokens) and np.array_equal(one.view_tokens, two.view_tokens)
        for what in ("out", "k_pool", "v_pool", "k_view", "v_view", "index"):
            a, b = getattr(one, what), getattr(two, what)
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                               b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32)), \
                (name, step, what)
    print(f"[gpu] attend_append {name}: outputs, pools, views and index bit-identical to attend + append", flush=True)
