"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes scratch buffers, and rejects every invalid argument
before it enqueues anything (so these calls never reach the device)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import __graft_entry__  # noqa: F401  (puts the repo root on sys.path)
from block_sparse_decode_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvmem.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        __graft_entry__.build()
    return L.load()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(kvmem_[a-z_]+)\s*\(", src)))


def test_exports_match_header(lib):
    decl = _declared()
    assert set(decl) == set(L.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in decl:
        assert name in syms, name
        assert hasattr(lib, name)


def test_status_strings_and_version(lib):
    assert L.status_string(0) == "ok"
    assert "scratch" in L.status_string(3)
    assert L.kvmem_version() >= 200


def _geom(dtype="bf16", Hq=64, Hkv=8, d=128, bt=32):
    return L.make_geom(Hq, Hkv, dtype, d, bt)


def _ws(S=2, max_blocks=64, n_tok=(100, 2048), n_pages=70):
    n = np.asarray(n_tok, np.int32)
    ws = L.Workspace(0x1000, 0x2000, 0x3000, n.ctypes.data, S, max_blocks, n_pages, None)
    return ws, n


def test_scratch_sizes(lib):
    g = _geom()
    a = L.kvmem_score_select_scratch_bytes(g, 1, 32768, 1)
    # per-head scores + per-chunk stats + aggregated scores
    assert a >= 64 * 32768 * 4 + 8 * 32768 * 4
    assert L.kvmem_score_select_scratch_bytes(g, 0, 32768, 1) == 0
    assert L.kvmem_score_select_scratch_bytes(_geom(d=64), 1, 32768, 1) == 0
    # tiled index: whole tiles of 64 blocks per (session, KV head)
    assert L.kvmem_index_bytes(g, 1, 32768) == 8 * 32768 * 128 * 2
    assert L.kvmem_index_bytes(g, 3, 65) == 3 * 8 * 128 * 128 * 2
    assert L.kvmem_index_bytes(_geom("f32", 4, 1), 2, 1) == 2 * 64 * 128 * 4
    assert L.kvmem_index_bytes(g, 0, 64) == 0 and L.kvmem_index_bytes(g, 1, 0) == 0
    assert L.kvmem_index_bytes(_geom(d=64), 1, 64) == 0
    b = L.kvmem_attend_scratch_bytes(g, 1, 1, 262144)
    assert b > 0 and b % 256 == 0
    assert L.kvmem_attend_scratch_bytes(g, 1, 1, 100) == 0          # not a multiple of 32


def test_build_index_rejects(lib):
    ws, n = _ws()
    assert L.kvmem_build_index(_geom(), ws, None, check=False) == L.KVMEM_E_ARG
    assert L.kvmem_build_index(_geom(d=64), ws, 0x10, check=False) == L.KVMEM_E_UNSUPPORTED
    assert L.kvmem_build_index(_geom(bt=16), ws, 0x10, check=False) == L.KVMEM_E_UNSUPPORTED
    assert L.kvmem_build_index(_geom(Hq=63), ws, 0x10, check=False) == L.KVMEM_E_ARG
    g = _geom()
    g.kv_dtype = 7
    assert L.kvmem_build_index(g, ws, 0x10, check=False) == L.KVMEM_E_UNSUPPORTED
    ws2, n2 = _ws(n_tok=(100, 64 * 32 + 1))                           # longer than the table
    assert L.kvmem_build_index(_geom(), ws2, 0x10, check=False) == L.KVMEM_E_ARG
    ws3, n3 = _ws(n_tok=(-1, 5))
    assert L.kvmem_build_index(_geom(), ws3, 0x10, check=False) == L.KVMEM_E_ARG
    st = L.load().kvmem_build_index(None, ctypes.byref(ws), 0x10, None)
    assert st == L.KVMEM_E_ARG
    st = L.load().kvmem_build_index(ctypes.byref(_geom()), None, 0x10, None)
    assert st == L.KVMEM_E_ARG


def test_score_select_rejects(lib):
    ws, n = _ws()
    vt = np.zeros(2, np.int32)
    g = _geom()
    need = L.kvmem_score_select_scratch_bytes(g, 2, 64, 1)
    common = dict(view_tokens_host=vt, scratch=0x4000, scratch_bytes=need, check=False)
    call = lambda **kw: L.kvmem_score_select(**{**dict(geom=g, ws=ws, index=0x10, q=0x20, T=1, q_norm_w=0x30,
                                                      eps=1e-6, k_select=8, n_recent=4, view_blocks=0x40),
                                              **common, **kw})
    assert call(T=0) == L.KVMEM_E_ARG
    assert call(k_select=-1) == L.KVMEM_E_ARG
    assert call(n_recent=-2) == L.KVMEM_E_ARG
    assert call(index=None) == L.KVMEM_E_ARG
    assert call(q=None) == L.KVMEM_E_ARG
    assert call(q_norm_w=None) == L.KVMEM_E_ARG
    assert call(view_blocks=None) == L.KVMEM_E_ARG
    assert call(eps=float("nan")) == L.KVMEM_E_ARG
    assert call(eps=-1.0) == L.KVMEM_E_ARG
    assert call(scratch_bytes=need - 1) == L.KVMEM_E_WORKSPACE
    assert call(scratch=None) == L.KVMEM_E_WORKSPACE
    assert call(geom=_geom(d=256)) == L.KVMEM_E_UNSUPPORTED


def test_materialize_rejects(lib):
    ws, n = _ws()
    g = _geom()
    vt = np.array([64, 96], np.int32)
    call = lambda **kw: L.kvmem_materialize(**{**dict(geom=g, ws=ws, view_blocks=0x10, n_list=4,
                                                     view_tokens_host=vt, max_view=128, rope_theta=1e6,
                                                     k_view=0x20, v_view=0x30, check=False), **kw})
    assert call(max_view=100) == L.KVMEM_E_ARG             # not a multiple of 32
    assert call(max_view=64) == L.KVMEM_E_ARG              # shorter than a view
    assert call(n_list=2) == L.KVMEM_E_ARG                 # view longer than the list allows
    assert call(view_blocks=None) == L.KVMEM_E_ARG
    assert call(k_view=None) == L.KVMEM_E_ARG
    assert call(rope_theta=0.5) == L.KVMEM_E_ARG
    assert call(rope_theta=float("inf")) == L.KVMEM_E_ARG
    ws_nov = L.Workspace(0x1000, None, 0x3000, n.ctypes.data, 2, 64, 70, None)
    assert call(ws=ws_nov) == L.KVMEM_E_ARG                # V pool needed
    assert call(view_tokens_host=np.array([-1, 0], np.int32)) == L.KVMEM_E_ARG


def test_attend_rejects(lib):
    g = _geom()
    vt = np.array([64, 96], np.int32)
    need = L.kvmem_attend_scratch_bytes(g, 2, 1, 128)
    call = lambda **kw: L.kvmem_attend(**{**dict(geom=g, n_sessions=2, q=0x10, T=1, q_norm_w=0x20, eps=1e-6,
                                                k_view=0x30, v_view=0x40, view_tokens_host=vt, max_view=128,
                                                rope_theta=1e6, out=0x50, scratch=0x60, scratch_bytes=need,
                                                check=False), **kw})
    assert call(T=0) == L.KVMEM_E_ARG
    assert call(n_sessions=0) == L.KVMEM_E_ARG
    assert call(out=None) == L.KVMEM_E_ARG
    assert call(view_tokens_host=np.array([64, 160], np.int32)) == L.KVMEM_E_ARG
    assert call(scratch_bytes=need - 1) == L.KVMEM_E_WORKSPACE
    assert call(T=8) == L.KVMEM_E_UNSUPPORTED               # 64 query rows per KV head in bf16
    assert call(geom=_geom(bt=64)) == L.KVMEM_E_UNSUPPORTED


def test_materialize_attend_rejects(lib):
    ws, n = _ws()
    g = _geom()
    vt = np.array([64, 96], np.int32)
    need = L.kvmem_attend_paged_scratch_bytes(g, 2, 1, 4)
    assert need > 0
    call = lambda **kw: L.kvmem_materialize_attend(**{**dict(
        geom=g, ws=ws, q=0x10, T=1, q_norm_w=0x20, eps=1e-6, view_blocks=0x30, n_list=4, view_tokens_host=vt,
        max_view=128, rope_theta=1e6, k_view=0x40, v_view=0x50, out=0x60, scratch=0x70, scratch_bytes=need,
        check=False), **kw})
    assert call(k_view=None) == L.KVMEM_E_ARG
    assert call(v_view=None) == L.KVMEM_E_ARG
    assert call(max_view=100) == L.KVMEM_E_ARG             # not a multiple of 32
    assert call(max_view=64) == L.KVMEM_E_ARG              # shorter than a view
    assert call(n_list=2) == L.KVMEM_E_ARG                 # view longer than the list allows
    assert call(view_blocks=None) == L.KVMEM_E_ARG
    assert call(T=0) == L.KVMEM_E_ARG
    assert call(q=None) == L.KVMEM_E_ARG
    assert call(out=None) == L.KVMEM_E_ARG
    assert call(rope_theta=1.0) == L.KVMEM_E_ARG
    assert call(scratch_bytes=need - 1) == L.KVMEM_E_WORKSPACE
    assert call(T=8) == L.KVMEM_E_UNSUPPORTED               # 64 query rows per KV head
    assert call(geom=_geom("f32"), T=16) == L.KVMEM_E_UNSUPPORTED   # fp32: at most 64 rows
    assert call(geom=_geom("f32"), T=8, scratch_bytes=L.kvmem_attend_paged_scratch_bytes(
        _geom("f32"), 2, 8, 4) - 1) == L.KVMEM_E_WORKSPACE  # fp32 with 64 rows gets past the row check


def test_update_index_rejects(lib):
    g = _geom()
    ws, n = _ws()
    first = np.array([0, 64], np.int32)          # session 1 has 2048 // 32 = 64 complete blocks
    bad = lambda *a, **k: L.kvmem_update_index(*a, check=False, **k)
    assert bad(g, ws, np.array([-1, 0], np.int32), 0x4000) == L.KVMEM_E_ARG
    assert bad(g, ws, np.array([0, 65], np.int32), 0x4000) == L.KVMEM_E_ARG     # past the complete blocks
    assert bad(g, ws, np.array([4, 0], np.int32), 0x4000) == L.KVMEM_E_ARG      # session 0 has 3 blocks
    assert bad(g, ws, first, None) == L.KVMEM_E_ARG
    assert bad(_geom(d=64), ws, first, 0x4000) == L.KVMEM_E_UNSUPPORTED


def test_append_rejects(lib):
    g = _geom()
    ws, n = _ws(n_tok=(100, 2000))
    vt = np.array([64, 96], np.int32)
    kp, vp = 0x1000, 0x2000                      # the workspace's own pools

    def bad(geom=g, ws_=ws, k_pool=kp, v_pool=vp, k_new=0x5000, v_new=0x6000, T_new=4, view=vt, max_view=256,
            theta=1e6, kv=0x7000, vv=0x8000):
        return L.kvmem_append(geom, ws_, k_pool, v_pool, k_new, v_new, T_new, view, max_view, theta, kv, vv,
                              check=False)

    assert bad(k_pool=0x1100) == L.KVMEM_E_ARG            # not the workspace's pool
    assert bad(v_pool=None) == L.KVMEM_E_ARG
    assert bad(k_new=None) == L.KVMEM_E_ARG
    assert bad(kv=None) == L.KVMEM_E_ARG
    assert bad(T_new=-1) == L.KVMEM_E_ARG
    assert bad(max_view=250) == L.KVMEM_E_ARG             # not a multiple of 32
    assert bad(theta=1.0) == L.KVMEM_E_ARG
    assert bad(view=np.array([64, 253], np.int32)) == L.KVMEM_E_ARG     # view would overflow max_view
    assert bad(T_new=49) == L.KVMEM_E_ARG                 # 2000 + 49 > 64 blocks of 32
    assert bad(geom=_geom(bt=16)) == L.KVMEM_E_UNSUPPORTED
    ws_nov = L.Workspace(0x1000, None, 0x3000, n.ctypes.data, 2, 64, 70, None)
    assert bad(ws_=ws_nov, v_pool=None) == L.KVMEM_E_ARG  # V pool required
    assert bad(T_new=0) == L.KVMEM_OK                     # nothing to do, nothing enqueued


def test_view_tokens_query(lib):
    """The host-only view-length query equals the oracle's view length (the
    selected whole blocks plus the recent range, partial tail included)."""
    from oracle import kvmem_oracle as O
    rng = np.random.default_rng(12)
    n = np.concatenate([[0, 1, 31, 32, 33, 64, 32 * 100 + 7], rng.integers(0, 32 * 5000, 40)]).astype(np.int32)
    for k, r in ((0, 0), (8, 8), (7936, 256), (3, 0), (0, 5), (10_000, 2), (1, 1000)):
        got = L.kvmem_view_tokens(n, k, r)
        want = [O.view_tokens(int(x), k, r) for x in n]
        assert got.tolist() == want, (k, r)
    out = np.zeros(2, np.int32)
    q = L.load().kvmem_view_tokens
    nn = np.array([64, 100], np.int32)
    assert q(0, nn.ctypes.data, 1, 1, out.ctypes.data) == L.KVMEM_E_ARG
    assert q(2, None, 1, 1, out.ctypes.data) == L.KVMEM_E_ARG
    assert q(2, nn.ctypes.data, 1, 1, None) == L.KVMEM_E_ARG
    assert q(2, nn.ctypes.data, -1, 1, out.ctypes.data) == L.KVMEM_E_ARG
    assert q(2, nn.ctypes.data, 1, -1, out.ctypes.data) == L.KVMEM_E_ARG
    neg = np.array([64, -1], np.int32)
    assert q(2, neg.ctypes.data, 1, 1, out.ctypes.data) == L.KVMEM_E_ARG


def test_attention_mass_rejects(lib):
    ws, n = _ws()
    g = _geom()
    need = L.kvmem_attention_mass_scratch_bytes(g, 2, 1, 64)
    assert need > 0 and need % 256 == 0
    assert L.kvmem_attention_mass_scratch_bytes(g, 0, 1, 64) == 0
    assert L.kvmem_attention_mass_scratch_bytes(g, 2, 0, 64) == 0
    assert L.kvmem_attention_mass_scratch_bytes(_geom(d=64), 2, 1, 64) == 0
    call = lambda **kw: L.kvmem_attention_mass(**{**dict(
        geom=g, ws=ws, q=0x10, T=1, q_norm_w=0x20, eps=1e-6, view_blocks=0x30, n_list=4, rope_theta=1e6,
        mass=0x40, lse=None, scratch=0x50, scratch_bytes=need, check=False), **kw})
    assert call(q=None) == L.KVMEM_E_ARG
    assert call(q_norm_w=None) == L.KVMEM_E_ARG
    assert call(mass=None) == L.KVMEM_E_ARG
    assert call(T=0) == L.KVMEM_E_ARG
    assert call(n_list=-1) == L.KVMEM_E_ARG
    assert call(view_blocks=None) == L.KVMEM_E_ARG          # a list of 4 entries without a buffer
    assert call(eps=float("nan")) == L.KVMEM_E_ARG
    assert call(eps=-1.0) == L.KVMEM_E_ARG
    assert call(rope_theta=1.0) == L.KVMEM_E_ARG
    assert call(rope_theta=float("inf")) == L.KVMEM_E_ARG
    assert call(scratch_bytes=need - 1) == L.KVMEM_E_WORKSPACE
    assert call(scratch=None) == L.KVMEM_E_WORKSPACE
    assert call(T=8) == L.KVMEM_E_UNSUPPORTED               # 64 query rows per KV head
    assert call(geom=_geom("f32"), T=16) == L.KVMEM_E_UNSUPPORTED   # fp32: at most 64 rows
    assert call(geom=_geom("f32"), T=8, scratch_bytes=L.kvmem_attention_mass_scratch_bytes(
        _geom("f32"), 2, 8, 64) - 1) == L.KVMEM_E_WORKSPACE # fp32 with 64 rows gets past the row check
    assert call(geom=_geom(d=64)) == L.KVMEM_E_UNSUPPORTED
    ws2, n2 = _ws(n_tok=(100, 64 * 32 + 1))                  # longer than the table
    assert call(ws=ws2) == L.KVMEM_E_ARG
    st = L.load().kvmem_attention_mass(ctypes.byref(g), None, 0x10, 1, 0x20, 1e-6, 0x30, 4, 1e6, 0x40, None,
                                       0x50, need, None)
    assert st == L.KVMEM_E_ARG


def test_attend_noalloc_rejects(lib):
    """The scratch-free attention checks its arguments like kvmem_attend and
    refuses a call whose scratch would exceed its array, all before any HIP
    call."""
    g = _geom()
    vt = np.array([64, 96], np.int32)
    call = lambda **kw: L.kvmem_attend_noalloc(**{**dict(geom=g, n_sessions=2, q=0x10, T=1, q_norm_w=0x20,
                                                         eps=1e-6, k_view=0x30, v_view=0x40, view_tokens_host=vt,
                                                         max_view=128, rope_theta=1e6, out=0x50, check=False),
                                                  **kw})
    assert call(T=0) == L.KVMEM_E_ARG
    assert call(n_sessions=0) == L.KVMEM_E_ARG
    assert call(out=None) == L.KVMEM_E_ARG
    assert call(q=None) == L.KVMEM_E_ARG
    assert call(view_tokens_host=np.array([64, 160], np.int32)) == L.KVMEM_E_ARG
    assert call(max_view=100) == L.KVMEM_E_ARG
    assert call(eps=float("nan")) == L.KVMEM_E_ARG
    assert call(rope_theta=1.0) == L.KVMEM_E_ARG
    assert call(T=8) == L.KVMEM_E_UNSUPPORTED               # 64 query rows per KV head in bf16
    assert call(geom=_geom(bt=64)) == L.KVMEM_E_UNSUPPORTED
    # beyond the array: 32 sessions of 262,144-token views
    S, mv = 32, 262144
    assert L.kvmem_attend_scratch_bytes(g, S, 1, mv) > L.NOALLOC_SCRATCH_BYTES
    big = np.full(S, mv, np.int32)
    assert call(n_sessions=S, view_tokens_host=big, max_view=mv) == L.KVMEM_E_WORKSPACE
    assert L.kvmem_attend_scratch_bytes(g, 1, 1, mv) <= L.NOALLOC_SCRATCH_BYTES


def test_stage_view_rejects(lib):
    ws, n = _ws()
    g = _geom()
    vt = np.array([64, 96], np.int32)
    call = lambda **kw: L.kvmem_stage_view(**{**dict(geom=g, ws=ws, view_blocks=0x10, n_list=4,
                                                    view_tokens_host=vt, stage_k=0x20, stage_v=0x30,
                                                    stage_table=0x40, stage_list=0x50, check=False), **kw})
    assert call(stage_k=None) == L.KVMEM_E_ARG
    assert call(stage_v=None) == L.KVMEM_E_ARG
    assert call(stage_table=None) == L.KVMEM_E_ARG
    assert call(stage_list=None) == L.KVMEM_E_ARG
    assert call(n_list=0) == L.KVMEM_E_ARG
    assert call(n_list=2) == L.KVMEM_E_ARG                 # a view longer than the list allows
    assert call(view_blocks=None) == L.KVMEM_E_ARG
    assert call(view_tokens_host=np.array([-1, 0], np.int32)) == L.KVMEM_E_ARG
    assert call(geom=_geom(d=64)) == L.KVMEM_E_UNSUPPORTED
    ws_nov = L.Workspace(0x1000, None, 0x3000, n.ctypes.data, 2, 64, 70, None)
    assert call(ws=ws_nov) == L.KVMEM_E_ARG                # V pool needed
    ws2, n2 = _ws(n_tok=(100, 64 * 32 + 1))                  # longer than the table
    assert call(ws=ws2) == L.KVMEM_E_ARG


def test_attend_append_rejects(lib):
    """The decode call (attention, then the append on the merge launch) makes
    every check of kvmem_attend and of kvmem_append before enqueuing."""
    ws, n = _ws(n_tok=(100, 1000))
    g = _geom()
    vt = np.array([64, 96], np.int32)
    need = L.kvmem_attend_scratch_bytes(g, 2, 1, 128)
    call = lambda **kw: L.kvmem_attend_append(**{**dict(
        geom=g, ws=ws, q=0x10, T=1, q_norm_w=0x20, eps=1e-6, k_view=0x30, v_view=0x40, view_tokens_host=vt,
        max_view=128, rope_theta=1e6, out=0x50, k_pool=0x1000, v_pool=0x2000, k_new=0x60, v_new=0x70, T_new=1,
        scratch=0x80, scratch_bytes=need, check=False), **kw})
    assert call(T=0) == L.KVMEM_E_ARG
    assert call(out=None) == L.KVMEM_E_ARG
    assert call(k_new=None) == L.KVMEM_E_ARG
    assert call(T_new=-1) == L.KVMEM_E_ARG
    assert call(k_pool=0x1001) == L.KVMEM_E_ARG                   # not the workspace's pool
    assert call(T_new=33) == L.KVMEM_E_ARG                        # session 1's view would pass max_view
    assert call(T_new=64 * 32 - 1000 + 1, max_view=2048) == L.KVMEM_E_ARG   # session 1's history would pass the table
    assert call(T_new=64 * 32 - 1000, max_view=2048) == L.KVMEM_E_WORKSPACE  # fits; the scratch was sized for 128
    ws_nov = L.Workspace(0x1000, None, 0x3000, n.ctypes.data, 2, 64, 70, None)
    assert call(ws=ws_nov, v_pool=None) == L.KVMEM_E_ARG          # V pool needed
    assert call(scratch_bytes=need - 1) == L.KVMEM_E_WORKSPACE
    assert call(T=8) == L.KVMEM_E_UNSUPPORTED                     # 64 query rows per KV head in bf16
