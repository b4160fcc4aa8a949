"""The seeded generators: determinism, chunk addressability, layout, planting,
and the margin certifier."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import kvmem_oracle as O
from tests.certify import TAU, certify
from tests.helpers import make_workload, oracle_ws, small_cfg
from workloads import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits
from workloads.synth import session_lengths


def test_deterministic_and_threads_independent():
    cfg = small_cfg(n_tokens=(32 * 2500 + 3,), Hkv=2, Hq=4)
    a = make_workload(cfg, threads=1)
    b = make_workload(cfg, threads=4)
    for f in ("k_pool", "v_pool", "block_table", "n_tokens", "q", "q_norm_w", "qhat", "plant_mag"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_table_is_a_permutation_and_tail_zeroed():
    cfg = small_cfg(S=3, n_tokens=(100, 64, 1), Hkv=2, Hq=4, spare_pages=5)
    wl = make_workload(cfg)
    used = wl.block_table[wl.block_table >= 0]
    assert sorted(used.tolist()) == sorted(set(used.tolist()))
    assert len(used) == 4 + 2 + 1 and wl.n_pages == 12
    # tokens past the end of the history are zero in the partial tail page
    tail = wl.k_pool[wl.block_table[0, 3]]
    assert np.all(tail[:, 4:] == 0) and np.any(tail[:, :4] != 0)
    spare = np.setdiff1d(np.arange(wl.n_pages), used)
    assert np.all(np.isnan(bf16_bits_to_f32(wl.k_pool[spare])))


def test_bf16_helpers_roundtrip():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 0.0], np.float32)
    b = f32_to_bf16_bits(x)
    assert bf16_bits_to_f32(b).tolist() == [1.0, 1.0, 1 + 2 ** -6, -2.5, 0.0]


def test_config_catalog_shapes():
    c4 = CONFIGS["c4"]
    lens = session_lengths(c4)
    assert len(lens) == 16 and np.all(lens % 32 == 0)
    assert lens.min() >= 1024 * 32 and lens.max() <= 2048 * 32
    assert CONFIGS["c5"].n_tokens[0] // 32 == 312_500
    assert CONFIGS["c3"].n_tokens[0] == 1 << 20


def test_planting_adds_along_qhat():
    cfg = small_cfg(dtype="f32", n_tokens=(32 * 50,), Hkv=1, Hq=2, n_planted=5, R=2)
    wl = make_workload(cfg)
    planted = np.nonzero(wl.plant_mag[0, 0])[0]
    assert len(planted) == 5 and planted.max() < 48
    ws = oracle_ws(wl)
    idx = O.mean_k_index(ws, 0, 0)
    proj = idx @ wl.qhat[0, 0]
    assert proj[planted].min() > 1.0 and np.delete(proj, planted).max() < 1.0


def test_certify_opens_the_cut():
    cfg = small_cfg(dtype="bf16", n_tokens=(32 * 3000,), Hkv=2, Hq=16, k=300, R=8,
                    n_planted=20, seed=21)
    wl = make_workload(cfg)
    rep = certify(wl)
    ws = oracle_ws(wl)
    for h in range(2):
        qn = O.q_rmsnorm(O.decode(wl.q[0], "bf16"), wl.q_norm_w, cfg.eps)
        A = O.head_aggregate(qn[:, h * 8:(h + 1) * 8], O.mean_k_index(ws, 0, h))
        nc = 3000 - 8
        a = np.sort(A[:nc])[::-1]
        assert (a[299] - a[300]) / a[299] >= TAU
    assert any(v[1] > 0 for v in rep.values())      # this seed needs repairs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_chunks_match_full_draw_with_repairs(dtype):
    """Chunk-by-chunk drawing (used for workspaces too large for the host)
    gives the same pools as the full draw, repair log included."""
    from workloads import pool_chunks
    cfg = CONFIGS["c1"].replace(dtype=dtype, n_tokens=(2 * 1024 * 32 + 100,), k_select=8, n_recent=4)
    rep = [(0, 0, 5, 3, 0.25), (0, 0, 5, 3, -0.125), (0, 0, 1500, 7, 1.0)]
    full = make_workload(cfg, repairs=rep)
    lite = make_workload(cfg, pools=False, repairs=rep)
    assert lite.k_pool is None and lite.n_pages == full.n_pages
    assert np.array_equal(lite.block_table, full.block_table) and np.array_equal(lite.q, full.q)
    for which, pool in (("k", full.k_pool), ("v", full.v_pool)):
        n = 0
        for s, b0, pages, x in pool_chunks(lite, which, threads=2):
            assert np.array_equal(pool[pages], x), (which, b0)
            n += len(pages)
        assert n == -(-int(full.n_tokens[0]) // 32)
    # the repairs moved exactly the logged coordinates
    plain = make_workload(cfg)
    diff = np.argwhere(plain.k_pool != full.k_pool)
    pages = {int(full.block_table[0, b]) for b in (5, 1500)}
    assert {int(p) for p in diff[:, 0]} <= pages and len(diff) > 0


def test_certify_streaming_matches_in_memory():
    """The chunk-by-chunk certification (used for the 10M-token workload) logs
    repairs that, replayed by the generator, give the same separated cut as
    the in-memory certification of the same workload."""
    from tests.certify import certify_streaming, streamed_index
    # (5% planted, k = 100: head 0's cut needs one repair round on this seed)
    cfg = CONFIGS["c5"].replace(name="c5_small", n_tokens=(3 * 1024 * 32,), T=4, k_select=100,
                                plant_fraction=0.05, n_q_heads=8, n_kv_heads=2)
    wl_mem = make_workload(cfg)
    rep_mem = certify(wl_mem, t_chunk=2)
    lite = make_workload(cfg, pools=False)
    index = streamed_index(lite, threads=2)
    ws = oracle_ws(wl_mem)
    repairs, rep, A_all = certify_streaming(lite, index, t_chunk=2, log=lambda m: None)
    assert {h: r[1] for h, r in rep.items()} == {h: r[1] for (s, h), r in rep_mem.items()}
    assert len(repairs) > 0
    replay = make_workload(cfg, repairs=repairs)
    assert np.array_equal(replay.k_pool, wl_mem.k_pool)
    for h in range(cfg.n_kv_heads):
        assert np.array_equal(index[h], O.mean_k_index(ws, 0, h))
        assert rep[h][2] >= TAU
