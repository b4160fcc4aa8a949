"""GPU parity of host-tier paging (kvmem_stage_view), through the C ABI.

The K/V pools live in pinned host memory that the GPU reads over the host
link; the Mean-K index is built from them into device memory; after the
selection, the listed tiles are staged into a device pool in view order and
the one-pass gather + attention runs on the staged pool.  Bars:
  * index and lists from the host pools: bit-identical to the same workload's
    device-resident path;
  * staged tiles: bit for bit the oracle's stored K and V of each listed
    block (tokens past the view zero), staged table and identity list exact;
  * view and attention from the staged pool: bit for bit those of the
    device-resident one-pass call (the keys and the list structure are the
    same), and the attention within the bars against the oracle.
"""
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

CASES = {
    "ragged": small_cfg("stage_ragged", "bf16", S=3, Hq=16, Hkv=2, n_tokens=(32 * 300 + 5, 32 * 64, 7),
                        k=24, R=3, n_planted=6, spare_pages=5, seed=131),
    "t2": small_cfg("stage_t2", "bf16", S=2, Hq=16, Hkv=2, T=2, n_tokens=(32 * 700, 32 * 257 + 1),
                    k=50, R=5, n_planted=8, seed=132),
    "c2": CONFIGS["c2"],
}


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _require_addressable(dw):
    """The library's own check that the GPU reads the host pools in place,
    through a staging call whose views are empty (it reads no pool data)."""
    from block_sparse_decode_amd import _lib as L
    from block_sparse_decode_amd.pipeline import StagedView
    st = StagedView(dw)
    zero = np.zeros(dw.S, np.int32)
    rc = L.kvmem_stage_view(dw.geom, dw.ws, dw.view_blocks, dw.n_list, zero, st.k, st.v, st.table, st.list,
                            check=False)
    torch.cuda.synchronize()
    assert rc == L.KVMEM_OK, f"pinned host pools not addressable by the GPU (status {rc})"


@pytest.mark.parametrize("name", list(CASES))
def test_stage_parity(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd.pipeline import DeviceWorkspace, StagedView, index_rows
    cfg = CASES[name]
    wl = make_workload(cfg)
    certify(wl)
    print(f"[gpu] stage {cfg.name} N={list(wl.n_tokens)[:4]} T={cfg.T} k={cfg.k_select} R={cfg.n_recent}", flush=True)
    ref = DeviceWorkspace(wl, "cuda")                  # device-resident pools
    ref.build_index()
    ref.score_select()
    ref.materialize_attend()
    torch.cuda.synchronize()

    dw = DeviceWorkspace(wl, "cuda", host_pools=True)  # pinned host pools
    assert dw.k_pool.device.type == "cpu" and dw.k_pool.is_pinned()
    _require_addressable(dw)
    dw.build_index()
    dw.score_select()
    torch.cuda.synchronize()
    rows_h, rows_d = index_rows(dw.index, dw.max_blocks), index_rows(ref.index, ref.max_blocks)
    for s in range(cfg.n_sessions):                     # the written rows: each session's complete blocks
        nb = int(wl.n_tokens[s]) // 32
        assert torch.equal(_bits(rows_h[s, :, :nb]), _bits(rows_d[s, :, :nb])), (name, s, "index from the host tier")
    assert torch.equal(dw.view_blocks, ref.view_blocks), "lists"
    assert np.array_equal(dw.view_tokens, ref.view_tokens)

    st = StagedView(dw)
    st.k.view(torch.int16).fill_(0x5A5A)
    st.v.view(torch.int16).fill_(0x5A5A)
    dw.stage(st)
    out = torch.full_like(dw.out, float("nan"))
    dw.materialize_attend_staged(st, out=out)
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0

    # staged table, identity list and tiles against the oracle's stored blocks
    ws = oracle_ws(wl)
    S, H, n_list = cfg.n_sessions, cfg.n_kv_heads, dw.n_list
    vb = dw.view_blocks.cpu().numpy()
    table = st.table.cpu().numpy()
    lst = st.list.cpu().numpy()
    sk = _bits(st.k).cpu().numpy().view(np.uint16)
    sv = _bits(st.v).cpu().numpy().view(np.uint16)
    for s in range(S):
        V = int(dw.view_tokens[s])
        nvb = -(-V // 32)
        want_t = np.where(np.arange(n_list) < nvb, s * n_list + np.arange(n_list), -1)
        assert np.array_equal(table[s], want_t), (name, s)
        for h in range(H):
            assert np.array_equal(lst[s, h], np.where(np.arange(n_list) < nvb, np.arange(n_list), -1)), (name, s, h)
            if nvb == 0:
                continue
            blocks = vb[s, h, :nvb].astype(np.int64)
            kref = O.block_tokens_of(ws, ws.k_pool, s, h, blocks)        # [nvb][32][d] float64
            vref = O.block_tokens_of(ws, ws.v_pool, s, h, blocks)
            valid = (np.arange(nvb * 32) < V).reshape(nvb, 32)[..., None]
            kref = np.where(valid, kref, 0.0)
            vref = np.where(valid, vref, 0.0)
            pages = s * n_list + np.arange(nvb)
            assert np.array_equal(O.decode(sk[pages, h], "bf16"), kref), (name, s, h, "staged K")
            assert np.array_equal(O.decode(sv[pages, h], "bf16"), vref), (name, s, h, "staged V")

    # view and attention: bit for bit the device-resident one-pass call's
    for s in range(S):
        nb = -(-int(dw.view_tokens[s]) // 32)
        assert torch.equal(_bits(dw.k_view[s, :, :32 * nb]), _bits(ref.k_view[s, :, :32 * nb])), (name, s, "K view")
        assert torch.equal(_bits(dw.v_view[s, :, :nb]), _bits(ref.v_view[s, :, :nb])), (name, s, "V view")
    assert torch.equal(out.view(torch.int32), ref.out.view(torch.int32)), (name, "attention")
    # and the attention against the oracle, one head per session
    G = cfg.group
    o = out.cpu().numpy().astype(np.float64)
    for s in range(S):
        h = s % H
        qn = O.q_rmsnorm(O.decode(wl.q[s], cfg.dtype), wl.q_norm_w, cfg.eps)
        kv, vv = O.materialize(ws, s, h, vb[s, h][vb[s, h] >= 0].astype(np.int64), int(dw.view_tokens[s]),
                               cfg.rope_theta)
        o_ref = O.attend(qn[:, h * G:(h + 1) * G], kv, vv, cfg.rope_theta)
        err = float(np.abs(o[s, :, h * G:(h + 1) * G] - o_ref).max())
        assert err <= ATT_TOL[cfg.dtype] and err <= reg_bar(o_ref), (name, s, h, err)
    print(f"[gpu] stage {cfg.name}: index, lists, staged tiles, view and attention match", flush=True)


def test_stage_bad_entries_are_flagged_and_zero():
    """A listed block whose page is outside the pool: flagged, staged as a zero
    tile, and the staged view equals the device-resident gather's (which
    writes zeros for it)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_decode_amd import _lib as L
    from block_sparse_decode_amd.pipeline import DeviceWorkspace, StagedView
    cfg = small_cfg("stage_bad", "bf16", S=1, Hq=16, Hkv=2, n_tokens=(32 * 64 + 9,), k=8, R=2, seed=133)
    wl = make_workload(cfg)
    dw = DeviceWorkspace(wl, "cuda", host_pools=True)
    _require_addressable(dw)
    dw.build_index()
    dw.score_select()
    torch.cuda.synchronize()
    beta = int(dw.view_blocks[0, 1, 3].item())
    bt = dw.block_table.clone()
    dw.block_table[0, beta] = wl.n_pages + 7            # outside the pool, after the selection
    st = StagedView(dw)
    dw.stage(st)
    dw.materialize()                                     # the gather straight from the host pools
    torch.cuda.synchronize()
    k_direct, v_direct = dw.k_view.clone(), dw.v_view.clone()
    assert int(dw.dev_error.item()) & L.KVMEM_DEVERR_PAGE
    assert bool((_bits(st.k[3, 1]) == 0).all()) and bool((_bits(st.v[3, 1]) == 0).all())
    dw.dev_error.zero_()
    L.kvmem_materialize(dw.geom, st.ws, st.list, dw.n_list, dw.view_tokens, dw.max_view, dw.theta, dw.k_view,
                        dw.v_view)
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0
    nb = -(-int(dw.view_tokens[0]) // 32)
    assert torch.equal(_bits(dw.k_view[0, :, :32 * nb]), _bits(k_direct[0, :, :32 * nb]))
    assert torch.equal(_bits(dw.v_view[0, :, :nb]), _bits(v_direct[0, :, :nb]))
    dw.block_table.copy_(bt)
