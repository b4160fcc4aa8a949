"""GPU parity of every step against the CPU oracle, through the C ABI.

Bars (from the scope of the hot path):
  * Mean-K index            : bit-exact (fp64 sums, one rounding on both sides)
  * raw block scores s      : |d| <= 1e-3 * max(|s_ref|, rms of the row)
  * aggregated scores A     : |d| <= 1e-3 * A_ref
  * selected blocks, view   : bit-exact (inputs certified with a 1e-3 cut margin)
  * V view                  : bit-exact;  K view: <= 1 bf16 ulp / 2e-6 relative fp32
  * attention output        : <= 2e-2 max-abs for bf16, <= 1e-4 for fp32, and
                              the regression bar below
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from oracle import kvmem_oracle as O
from tests.certify import certify
from tests.helpers import make_workload, oracle_ws, small_cfg
from workloads import CONFIGS

pytestmark = pytest.mark.gpu

ATT_TOL = {"bf16": 2e-2, "f32": 1e-4}

# Regression bar, applied beside ATT_TOL to every attention output of a (session,
# KV head): |o_gpu - o_ref| <= REG_REL * max|o_ref| + REG_ABS.  The kernels form
# each logit from bf16 hi + lo query operands (~2^-16 relative) and accumulate
# every product, exponential and weighted sum in fp32; their keys differ from the
# oracle's by one bf16 ulp only on the elements whose exact rotated value lies
# within the fp32 rotation error of a rounding boundary (a fraction ~1e-5 of
# them).  Together that moves an output, a convex combination of value rows,
# by far less than 1e-3 of its largest coordinate, while a 32-token tile that a
# kernel drops or counts twice in a diffuse 262,144-token view moves it by about
# p_tile * |v_tile - o| ~ 1.2e-4 * 0.5, several times the bar there.
REG_REL, REG_ABS = 1e-3, 2e-6


def reg_bar(o_ref: np.ndarray) -> float:
    return REG_REL * (float(np.abs(o_ref).max()) if o_ref.size else 0.0) + REG_ABS


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits_to_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    with np.errstate(invalid="ignore"):          # buffers hold unwritten slots past the views
        if dtype == "bf16":
            b = t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
            return b.view(np.float32).astype(np.float64)
        return t.cpu().numpy().astype(np.float64)


def run_gpu(wl, scores=True, attend=True):
    from block_sparse_decode_amd.pipeline import DeviceWorkspace, index_rows, v_view_token_major
    cfg = wl.cfg
    print(f"[gpu] {cfg.name} S={cfg.n_sessions} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} T={cfg.T} "
          f"N={list(wl.n_tokens)[:4]} k={cfg.k_select} R={cfg.n_recent}", flush=True)
    dw = DeviceWorkspace(wl, "cuda")
    S, H, T, Hq = cfg.n_sessions, cfg.n_kv_heads, cfg.T, cfg.n_q_heads
    sc = torch.full((S, T, Hq, dw.max_blocks), float("nan"), device="cuda") if scores else None
    ag = torch.full((S, H, dw.max_blocks), float("nan"), device="cuda")
    dw.build_index()
    dw.score_select(scores=sc, agg=ag)
    dw.materialize()
    if attend:
        dw.attend()
    torch.cuda.synchronize()
    res = dict(dw=dw, index=_bits_to_f64(index_rows(dw.index, dw.max_blocks).contiguous(), cfg.dtype), agg=ag.cpu().numpy().astype(np.float64),
               scores=None if sc is None else sc.cpu().numpy().astype(np.float64),
               vb=dw.view_blocks.cpu().numpy(), vt=dw.view_tokens.copy(),
               kview=_bits_to_f64(dw.k_view, cfg.dtype),
               vview=_bits_to_f64(v_view_token_major(dw.v_view).contiguous(), cfg.dtype),
               out=dw.out.cpu().numpy().astype(np.float64) if attend else None, err=int(dw.dev_error.item()))
    return res


def check_session(wl, res, s, heads=None, att_heads=None, check_scores=True, tag=""):
    cfg = wl.cfg
    ws = oracle_ws(wl)
    G = cfg.group
    heads = range(cfg.n_kv_heads) if heads is None else heads
    att_heads = heads if att_heads is None else att_heads
    n_tok = int(wl.n_tokens[s])
    nb = n_tok // 32
    index = [O.mean_k_index(ws, s, h) for h in range(cfg.n_kv_heads)]
    S_all, A_all, qn = O.session_scores(ws, s, wl.q[s], wl.q_norm_w, cfg.eps, index,
                                        keep_scores=check_scores)
    V_ref = O.view_tokens(n_tok, cfg.k_select, cfg.n_recent)
    assert int(res["vt"][s]) == V_ref, (tag, s)
    worst_att = 0.0
    for h in heads:
        # index: bit-exact
        assert np.array_equal(res["index"][s, h, :nb], index[h]), (tag, s, h, "index")
        # aggregated scores
        A_ref = A_all[h]
        A_gpu = res["agg"][s, h, :nb]
        assert np.all(np.abs(A_gpu - A_ref) <= 1e-3 * A_ref + 1e-30), (tag, s, h, "A")
        if check_scores and nb > 0:
            s_ref = S_all[h]                                      # [T][G][nb]
            s_gpu = res["scores"][s, :, h * G:(h + 1) * G, :nb]
            scale = np.maximum(np.abs(s_ref), np.sqrt(np.mean(s_ref ** 2, axis=-1, keepdims=True)))
            assert np.all(np.abs(s_gpu - s_ref) <= 1e-3 * scale), (tag, s, h, "scores")
        # selection: bit-exact list incl. recent and padding
        lst, V = O.view_list(A_ref, n_tok, cfg.k_select, cfg.n_recent)
        n_list = cfg.k_select + cfg.n_recent
        want = np.full(n_list, -1, np.int64)
        want[:len(lst)] = lst
        assert np.array_equal(res["vb"][s, h, :n_list], want), (tag, s, h, "view_blocks")
        if h not in att_heads:
            continue
        kv, vv = O.materialize(ws, s, h, lst, V, cfg.rope_theta)
        assert np.array_equal(res["vview"][s, h, :V], vv), (tag, s, h, "V view")
        kg = res["kview"][s, h, :V]
        # one storage rounding plus the fp32 rotation error, which is relative to
        # the rotated pair's magnitude (cancellation can make a result tiny)
        rot = 1e-6 * np.abs(kv).max(axis=-1, keepdims=True)
        if cfg.dtype == "bf16":
            ulp = np.ldexp(1.0, np.frexp(np.abs(kv))[1] - 8)
            assert np.all(np.abs(kg - kv) <= ulp + rot), (tag, s, h, "K view")
        else:
            assert np.all(np.abs(kg - kv) <= 2e-7 * np.abs(kv) + rot), (tag, s, h, "K view")
        # the padded tail of the last view block is zero
        if V % 32:
            end = -(-V // 32) * 32
            assert np.all(res["kview"][s, h, V:end] == 0) and np.all(res["vview"][s, h, V:end] == 0)
        if res["out"] is None:                                    # attention not run (long query chunks)
            continue
        o_ref = O.attend(qn[:, h * G:(h + 1) * G], kv, vv, cfg.rope_theta)
        o_gpu = res["out"][s, :, h * G:(h + 1) * G]
        err = float(np.abs(o_gpu - o_ref).max()) if V else float(np.abs(o_gpu).max())
        bar = reg_bar(o_ref)
        worst_att = max(worst_att, err / bar)
        assert err <= ATT_TOL[cfg.dtype], (tag, s, h, "attend", err)
        assert err <= bar, (tag, s, h, "attend regression bar", err, bar)
    return worst_att


def _full_check(wl, attend=True, **kw):
    res = run_gpu(wl, attend=attend)
    assert res["err"] == 0
    worst = 0.0
    for s in range(wl.cfg.n_sessions):
        worst = max(worst, check_session(wl, res, s, tag=wl.cfg.name, **kw))
    print(f"[gpu] {wl.cfg.name}: worst attention |err| / regression bar = {worst:.3f}", flush=True)
    return res


# ---------------------------------------------------------------------------
# small and edge-case workloads (several tiles, ragged tails)
# ---------------------------------------------------------------------------

SMALL = {
    "bf16_ragged": small_cfg("bf16_ragged", "bf16", S=3, Hq=16, Hkv=2, n_tokens=(32 * 300 + 5, 32 * 64, 7),
                             k=24, R=3, n_planted=6, spare_pages=5, seed=31),
    "f32_ragged": small_cfg("f32_ragged", "f32", S=2, Hq=8, Hkv=2, n_tokens=(32 * 513 + 31, 32 * 40),
                            k=17, R=2, n_planted=5, spare_pages=2, seed=32),
    "bf16_t2_g8": small_cfg("bf16_t2_g8", "bf16", S=2, Hq=16, Hkv=2, T=2, n_tokens=(32 * 700, 32 * 257 + 1),
                            k=50, R=5, n_planted=8, seed=33),
    "bf16_t4_g8": small_cfg("bf16_t4_g8", "bf16", S=3, Hq=16, Hkv=2, T=4, n_tokens=(32 * 1100, 32 * 600, 32 * 90),
                            k=40, R=8, n_planted=10, seed=34),
    "bf16_g4": small_cfg("bf16_g4", "bf16", S=1, Hq=8, Hkv=2, n_tokens=(32 * 1000,), k=64, R=4, seed=35),
    "bf16_g1": small_cfg("bf16_g1", "bf16", S=1, Hq=4, Hkv=4, n_tokens=(32 * 777 + 3,), k=32, R=2, seed=36),
    "f32_t3_g4": small_cfg("f32_t3_g4", "f32", S=2, Hq=8, Hkv=2, T=3, n_tokens=(32 * 200 + 9, 32 * 33),
                           k=12, R=2, seed=37),
    "recent_only": small_cfg("recent_only", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 50 + 3, 32 * 8),
                             k=0, R=6, seed=38),
    "budget_covers_all": small_cfg("budget_covers_all", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 60 + 3, 32 * 11),
                             k=10_000, R=2, seed=39),
    "r0_partial": small_cfg("r0_partial", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 90 + 17, 32 * 33),
                            k=20, R=0, seed=40),
    "empty_and_tiny": small_cfg("empty_and_tiny", "bf16", S=4, Hq=16, Hkv=2, n_tokens=(0, 5, 32, 32 * 40),
                                k=8, R=2, n_planted=2, seed=41),
    # more candidates than one 32768-key register tile of the selection kernel
    "multi_tile_select": small_cfg("multi_tile_select", "bf16", S=1, Hq=4, Hkv=1, n_tokens=(32 * 36000 + 9,),
                                   k=500, R=16, n_planted=300, seed=61),
    # a list of more than 16384 entries
    "two_list_windows": small_cfg("two_list_windows", "bf16", S=1, Hq=4, Hkv=1, n_tokens=(32 * 18000 + 7,),
                                  k=16_500, R=8, n_planted=100, seed=62),
    # budget extremes: one block, and every candidate but one
    "select_one": small_cfg("select_one", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 400 + 9, 32 * 75),
                            k=1, R=3, n_planted=1, seed=67),
    "select_all_but_one": small_cfg("select_all_but_one", "bf16", S=1, Hq=16, Hkv=2, n_tokens=(32 * 60 + 3,),
                                    k=58, R=2, n_planted=4, seed=68),
    # chunk edges of the chunk-parallel selection (1024 candidates per chunk):
    # one candidate in the last chunk, and whole chunks only
    "select_chunk_plus_one": small_cfg("select_chunk_plus_one", "bf16", S=1, Hq=16, Hkv=2,
                                       n_tokens=(32 * 1029 + 5,), k=300, R=5, n_planted=40, seed=71),
    "select_three_chunks": small_cfg("select_three_chunks", "bf16", S=2, Hq=16, Hkv=2,
                                     n_tokens=(32 * (3072 + 2), 32 * 2048 + 31), k=1500, R=2, n_planted=40,
                                     seed=72),
    # exactly one full 32768-key selection tile (no padding keys), and one key
    # more (the multi-tile selection kernel)
    "full_select_tile": small_cfg("full_select_tile", "bf16", S=1, Hq=4, Hkv=1, n_tokens=(32 * (32768 + 4),),
                                  k=3000, R=4, n_planted=200, seed=65),
    "select_tile_plus_one": small_cfg("select_tile_plus_one", "bf16", S=1, Hq=4, Hkv=1,
                                      n_tokens=(32 * (32769 + 4) + 1,), k=3000, R=5, n_planted=200, seed=66),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(name):
    _need_gpu()
    wl = make_workload(SMALL[name])
    certify(wl)
    _full_check(wl)


# Exact ties in the aggregated scores: every block's keys are a copy of one of
# four template blocks, so a head's index rows, scores and aggregated scores
# take four values, identical bit for bit within a class on both sides, and the
# budget cuts through a class: the kept blocks of that class are the ones with
# the lowest block indices.  One case per selection kernel (up to one 32768-key
# tile; more than that, with a list longer than the 16384 entries that kernel
# stages at a time); the second session of "ties" keeps every candidate.
TIES = {
    "ties": small_cfg("ties", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 3000 + 5, 32 * 700), k=1000, R=4,
                      seed=63),
    "ties_multi_tile": small_cfg("ties_multi_tile", "bf16", S=1, Hq=4, Hkv=1, n_tokens=(32 * 34000 + 3,), k=17_000,
                                 R=4, seed=64),
}


@pytest.mark.parametrize("name", list(TIES))
def test_selection_exact_ties(name):
    _need_gpu()
    cfg = TIES[name]
    wl = make_workload(cfg)
    rng = np.random.default_rng(cfg.seed)
    for s in range(cfg.n_sessions):
        nb = int(wl.n_tokens[s]) // 32
        cls = rng.integers(0, 4, nb)
        cls[:4] = np.arange(4)
        tmpl = wl.block_table[s, :4].copy()
        for b in range(4, nb):
            wl.k_pool[wl.block_table[s, b]] = wl.k_pool[tmpl[cls[b]]]
    # the four classes must be well apart, so only the ties are at stake
    ws = oracle_ws(wl)
    for s in range(cfg.n_sessions):
        index = [O.mean_k_index(ws, s, h) for h in range(cfg.n_kv_heads)]
        _, A_all, _ = O.session_scores(ws, s, wl.q[s], wl.q_norm_w, cfg.eps, index, keep_scores=False)
        for h in range(cfg.n_kv_heads):
            v = np.sort(A_all[h][:4])
            assert np.all(np.diff(v) > 1e-3 * v[1:]), (name, s, h, v)
    _full_check(wl, check_scores=False)


# Ties by selection chunk: every block of 1024-block chunk c carries the keys
# of the chunk's first block, so a head's A takes one value per chunk (the
# four well apart) and the budget cuts through one chunk's tied class, whose
# kept blocks are its lowest ones.  For the seed used, head 0 ranks the chunks
# 1 > 0 > 2 > 3 and head 1 ranks them 1 > 0 > 3 > 2, so k = 1500 cuts inside
# chunk 0 with the later chunk 1 taken whole, and k = 2500 and 3500 cut inside
# later chunks after two and three whole ones.
@pytest.mark.parametrize("k", [1500, 2500, 3500])
def test_selection_ties_by_chunk(k):
    _need_gpu()
    cfg = small_cfg(f"ties_by_chunk_{k}", "bf16", S=1, Hq=16, Hkv=2, n_tokens=(32 * (4096 + 3),), k=k, R=3,
                    seed=73)
    wl = make_workload(cfg)
    tmpl = [wl.block_table[0, 1024 * c] for c in range(4)]
    for b in range(4096):
        if b % 1024:
            wl.k_pool[wl.block_table[0, b]] = wl.k_pool[tmpl[b // 1024]]
    ws = oracle_ws(wl)
    index = [O.mean_k_index(ws, 0, h) for h in range(cfg.n_kv_heads)]
    _, A_all, _ = O.session_scores(ws, 0, wl.q[0], wl.q_norm_w, cfg.eps, index, keep_scores=False)
    for h in range(cfg.n_kv_heads):
        v = np.sort([A_all[h][1024 * c] for c in range(4)])
        assert np.all(np.diff(v) > 1e-3 * v[1:]), (k, h, v)
    _full_check(wl, check_scores=False)


# Every block's keys identical: all candidates tie, all of them fall into the
# selection's boundary bin (the tile kernel's LDS list holds all 32768), and the
# kept blocks are the lowest block indices.
EQUAL = {
    "all_equal_full_tile": small_cfg("all_equal_full_tile", "bf16", S=1, Hq=4, Hkv=1,
                                     n_tokens=(32 * (32768 + 4),), k=20_000, R=4, seed=69),
    "all_equal_two_sessions": small_cfg("all_equal_two_sessions", "bf16", S=2, Hq=16, Hkv=2,
                                        n_tokens=(32 * 500 + 7, 32 * 90), k=77, R=3, seed=70),
}


@pytest.mark.parametrize("name", list(EQUAL))
def test_selection_all_equal(name):
    _need_gpu()
    cfg = EQUAL[name]
    wl = make_workload(cfg)
    for s in range(cfg.n_sessions):
        nb = int(wl.n_tokens[s]) // 32
        tmpl = wl.block_table[s, 0]
        for b in range(1, nb):
            wl.k_pool[wl.block_table[s, b]] = wl.k_pool[tmpl]
    res = _full_check(wl, check_scores=False)
    for s in range(cfg.n_sessions):
        nb = int(wl.n_tokens[s]) // 32
        nc, _, _ = O.recent_split(int(wl.n_tokens[s]), cfg.n_recent)
        k_eff = min(cfg.k_select, nc)
        for h in range(cfg.n_kv_heads):
            assert np.array_equal(res["vb"][s, h, :k_eff], np.arange(k_eff)), (name, s, h)


# Long query chunks (more than 32 query rows per KV head): the two-pass
# matrix-core scorer.  One 64-row chunk; padded operand sets (40 rows); a
# partial second chunk (80 rows, G = 2); ragged block counts leave partial
# index tiles and 256-block groups.  Attention is not run for such steps.
LONG = {
    "long_t8_g8": small_cfg("long_t8_g8", "bf16", S=2, Hq=16, Hkv=2, T=8, n_tokens=(32 * 700 + 5, 32 * 300),
                            k=40, R=4, n_planted=8, seed=51),
    "long_t5_g8": small_cfg("long_t5_g8", "bf16", S=1, Hq=16, Hkv=2, T=5, n_tokens=(32 * 1000,),
                            k=64, R=0, n_planted=12, seed=52),
    "long_t40_g2": small_cfg("long_t40_g2", "bf16", S=2, Hq=4, Hkv=2, T=40, n_tokens=(32 * 513, 32 * 64 + 3),
                             k=32, R=2, n_planted=6, seed=53),
}


@pytest.mark.parametrize("name", list(LONG))
def test_long_chunk_parity(name):
    _need_gpu()
    wl = make_workload(LONG[name])
    certify(wl)
    _full_check(wl, attend=False)


def _bound_far_workload():
    """Long chunk whose queries have no component in dims 64..127 while the
    keys of four blocks (two 64-block tiles) are large there: those blocks'
    index rows have a large norm and no effect on any score, so the
    statistics pass's Cauchy-Schwarz shift |q~| max|k_bar| lies far above the
    rows' scores in those tiles (its exact-maximum path) and close to them in
    the rest."""
    cfg = small_cfg("long_bound_far", "bf16", S=1, Hq=16, Hkv=2, T=8, n_tokens=(32 * 600 + 7,), k=40, R=3,
                    n_planted=8, seed=54)
    wl = make_workload(cfg)
    wl.q[..., 64:] = 0
    wl.k_pool[wl.block_table[0, [70, 80, 200, 210]], :, :, 64:] = 0x41C0   # bf16 24.0
    certify(wl)
    return wl


def test_long_chunk_shift_far_above_scores():
    _need_gpu()
    wl = _bound_far_workload()
    cfg = wl.cfg
    ws = oracle_ws(wl)
    G, d = cfg.group, cfg.head_dim
    c = np.log2(np.e) / np.sqrt(d)
    qn = O.q_rmsnorm(O.decode(wl.q[0], cfg.dtype), wl.q_norm_w, cfg.eps)
    for h in range(cfg.n_kv_heads):                       # the case is what it claims to be
        idx = O.mean_k_index(ws, 0, h)
        qg = qn[:, h * G:(h + 1) * G].reshape(-1, d)
        s, kn, qnorm = qg @ idx.T * c, np.linalg.norm(idx, axis=1), np.linalg.norm(qg, axis=1) * c
        for t in range(len(idx) // 64):
            gap = qnorm * kn[64 * t:64 * t + 64].max() - s[:, 64 * t:64 * t + 64].max(axis=1)
            assert (gap.min() > 100) if t in (1, 3) else (gap.max() < 50), (h, t, gap.min(), gap.max())
    _full_check(wl, attend=False)


def test_scorer_wavefront_spans_keys():
    """The matrix-core scorer (9-32 query rows per KV head) with more items
    than it has wavefronts: 9 sessions x 8 KV heads x 33 index tiles (the
    longest history is 2,100 blocks) is 2,376 (session, head, tile) items for
    2,048 wavefronts, two items each, so a wavefront's two items often belong
    to different (session, head) keys: it builds the operands of a second key,
    flushes one statistics slot per key, and its look-ahead past a key's last
    tile reads the empty resource.  Ragged lengths, partial last blocks and
    partial last tiles; T = 2 (16 rows)."""
    _need_gpu()
    lens = (32 * 2100 - 5, 32 * 2050 + 17, 32 * 2003, 32 * 1999 + 1, 32 * 1500, 32 * 2100, 32 * 1800 + 31,
            32 * 2088, 32 * 2011 + 8)
    cfg = small_cfg("scorer_spans_keys", "bf16", S=9, Hq=64, Hkv=8, T=2, n_tokens=lens, k=24, R=4, n_planted=6,
                    seed=81)
    wl = make_workload(cfg)
    ntl = -(-max(n // 32 for n in lens) // 64)
    items = cfg.n_sessions * cfg.n_kv_heads * ntl
    print(f"[gpu] {items} scorer items over {ntl} tiles per key", flush=True)
    assert ntl == 33 and items > 2048
    certify(wl)
    _full_check(wl, attend=True)


def test_c1_parity():
    _need_gpu()
    wl = make_workload(CONFIGS["c1"])
    certify(wl)
    res = _full_check(wl)
    # the planted blocks are the selected ones
    planted = set(np.nonzero(wl.plant_mag[0, 0])[0].tolist())
    assert set(res["vb"][0, 0, :8].tolist()) == planted


def test_random_qnorm_weight():
    _need_gpu()
    cfg = small_cfg("w_random", "bf16", S=1, Hq=16, Hkv=2, n_tokens=(32 * 400,), k=30, R=4, seed=42,
                    w_mode="random")
    wl = make_workload(cfg)
    certify(wl)
    _full_check(wl)


# ---------------------------------------------------------------------------
# properties
# ---------------------------------------------------------------------------

def _defined(wl, res):
    """The parts of every output the library defines (buffers also hold
    never-written slots past each session's blocks and view)."""
    out = {"out": res["out"], "vb": res["vb"]}
    for s in range(wl.cfg.n_sessions):
        nb = int(wl.n_tokens[s]) // 32
        V = int(res["vt"][s])
        out[f"index{s}"] = res["index"][s, :, :nb]
        out[f"agg{s}"] = res["agg"][s, :, :nb]
        out[f"kview{s}"] = res["kview"][s, :, :V]
        out[f"vview{s}"] = res["vview"][s, :, :V]
    return out


def test_deterministic_and_page_permutation_invariant():
    _need_gpu()
    cfg = small_cfg("perm", "bf16", S=2, Hq=16, Hkv=2, n_tokens=(32 * 500 + 7, 32 * 100), k=40, R=3, seed=43,
                    spare_pages=3)
    wl = make_workload(cfg)
    a = _defined(wl, run_gpu(wl))
    b = _defined(wl, run_gpu(wl))
    for k in a:
        assert np.array_equal(a[k], b[k]), k                       # run-to-run bitwise
    perm = np.random.default_rng(5).permutation(wl.n_pages)
    wl2 = make_workload(cfg)
    wl2.k_pool = np.empty_like(wl.k_pool)
    wl2.v_pool = np.empty_like(wl.v_pool)
    wl2.k_pool[perm] = wl.k_pool
    wl2.v_pool[perm] = wl.v_pool
    wl2.block_table = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    c = _defined(wl2, run_gpu(wl2))
    for k in a:
        assert np.array_equal(a[k], c[k]), k


def test_split_count_invariance():
    # a larger view buffer changes the split-K partition; the merge must agree
    _need_gpu()
    from block_sparse_decode_amd.pipeline import DeviceWorkspace
    cfg = small_cfg("splits", "bf16", S=1, Hq=64, Hkv=8, n_tokens=(32 * 4000,), k=1000, R=8, seed=44)
    wl = make_workload(cfg)
    outs = []
    for mv in (None, 32 * 1008 * 8, 32 * 1008 * 64):
        dw = DeviceWorkspace(wl, "cuda", max_view=mv)
        dw.run()
        torch.cuda.synchronize()
        outs.append(dw.out.cpu().numpy())
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-5


def test_bad_page_is_flagged_not_read():
    _need_gpu()
    cfg = small_cfg("badpage", "bf16", S=1, Hq=16, Hkv=2, n_tokens=(32 * 64,), k=8, R=2, seed=45)
    wl = make_workload(cfg)
    wl.block_table[0, 5] = wl.n_pages + 100          # outside the pool: kernels must skip it
    res = run_gpu(wl, scores=False)
    assert res["err"] & 1
    assert np.all(res["index"][0, :, 5] == 0)


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

def test_c2_full():
    _need_gpu()
    wl = make_workload(CONFIGS["c2"])
    certify(wl)
    _full_check(wl, check_scores=True)


def test_c3_full():
    _need_gpu()
    wl = make_workload(CONFIGS["c3"])
    certify(wl)
    res = run_gpu(wl, scores=False)
    assert res["err"] == 0
    # selection for every head; materialise + attention on two heads
    check_session(wl, res, 0, att_heads=(0, 5), check_scores=False, tag="c3")


def test_c4_full():
    _need_gpu()
    wl = make_workload(CONFIGS["c4"])
    certify(wl)
    res = run_gpu(wl)
    assert res["err"] == 0
    for s in range(16):
        check_session(wl, res, s, att_heads=(s % 8,), tag=f"c4 s={s}")


C5_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "c5_10m_golden.npz")


def _c5_device_pools_and_views(wl, lists, cfg):
    """Draws the K and V pools chunk by chunk straight onto the device and,
    from the same chunks, the oracle's view of every listed block (its keys
    rotated at the view positions and rounded, its values as stored), plus the
    oracle's index rows of a sample of chunks.  Returns the device pools, the
    expected views [H][V][d] (float32, exact bf16 values) and the sampled rows."""
    from block_sparse_decode_amd.pipeline import to_device
    from tests.certify import chunk_workspace
    from workloads import pool_chunks
    H, d = cfg.n_kv_heads, cfg.head_dim
    n_tok = int(wl.n_tokens[0])
    last = -(-n_tok // 32)
    V = 32 * lists.shape[1]
    shape = (wl.n_pages, H, 32, d)
    exp = {"k": np.full((H, V, d), np.nan, np.float32), "v": np.full((H, V, d), np.nan, np.float32)}
    sample = {0, ((last - 1) // 1024) * 1024, (int(lists[0, 0]) // 1024) * 1024, 100 * 1024, 200 * 1024}
    rows = {}
    pools = {}
    for which in ("k", "v"):
        pool = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        for _, b0, pages, x in pool_chunks(wl, which):
            idx = torch.from_numpy(np.ascontiguousarray(pages, dtype=np.int64)).to("cuda")
            pool[idx] = to_device(x, "bf16", "cuda")
            cws = chunk_workspace(wl, 0, b0, x)
            b1 = b0 + x.shape[0]
            if which == "k" and b0 in sample:
                n = min(b1, n_tok // 32) - b0
                rows[b0] = [O.mean_k_rows(cws, 0, h, range(n)) for h in range(H)]
            for h in range(H):
                ms = np.nonzero((lists[h] >= b0) & (lists[h] < b1))[0]
                if len(ms) == 0:
                    continue
                toks = O.block_tokens_of(cws, cws.k_pool, 0, h, [int(lists[h, m]) - b0 for m in ms])  # [n][32][d]
                if which == "k":
                    pos = (32 * ms[:, None] + np.arange(32)[None, :]).reshape(-1)
                    rot = O.round_store(O.rope(toks.reshape(-1, d), pos, cfg.rope_theta), "bf16")
                    exp["k"][h, pos] = rot.astype(np.float32)
                else:
                    pos = (32 * ms[:, None] + np.arange(32)[None, :]).reshape(-1)
                    exp["v"][h, pos] = toks.reshape(-1, d).astype(np.float32)
        pools[which] = pool
        print(f"[gpu] c5: {which.upper()} pool drawn on the device, views of its listed blocks computed", flush=True)
    return (pools["k"], pools["v"]), exp, rows


def test_c5_full():
    """10,000,000 tokens (312,500 blocks), a 512-token query chunk x 64 heads,
    top-2048 per KV head, 65,536-token view: the two-pass matrix-core scorer
    at full size.  The oracle's scoring at this size takes minutes, so its
    results (the certified view lists, A on every selected block and on a
    sample of the others, and the key repair log the certification made) come
    from tests/golden/make_c5_golden.py.  The pools are drawn here chunk by
    chunk, and from the same chunks the oracle gives every listed block's view
    (all 16,384 view blocks are compared) and the index rows of a sample of
    chunks."""
    _need_gpu()
    from block_sparse_decode_amd.pipeline import DeviceWorkspace, index_rows, v_view_token_major
    if not os.path.exists(C5_GOLDEN):
        pytest.skip("tests/golden/c5_10m_golden.npz not generated")
    g = np.load(C5_GOLDEN)
    repairs = [(int(a), int(b), int(c), int(d), float(e)) for a, b, c, d, e in g["repairs"]]
    cfg = CONFIGS["c5"]
    wl = make_workload(cfg, pools=False, repairs=repairs)
    lists = g["lists"]
    print(f"[gpu] c5: drawing {wl.n_pages} pages of K and V on the device ({len(repairs)} key repairs)", flush=True)
    pools, exp, rows = _c5_device_pools_and_views(wl, lists, cfg)
    dw = DeviceWorkspace(wl, "cuda", device_pools=pools)
    H, G, mb = cfg.n_kv_heads, cfg.group, dw.max_blocks
    ag = torch.full((1, H, mb), float("nan"), device="cuda")
    dw.build_index()
    dw.score_select(agg=ag)
    dw.materialize()
    torch.cuda.synchronize()
    assert int(dw.dev_error.item()) == 0
    n_tok = int(wl.n_tokens[0])
    nc, _, _ = O.recent_split(n_tok, cfg.n_recent)
    # selection (bit-exact) and view length
    vb = dw.view_blocks.cpu().numpy()[0]
    assert np.array_equal(vb, lists)
    V = int(dw.view_tokens[0])
    assert V == int(g["view_tokens"]) == 65536
    # aggregated scores on the sampled blocks; every head's A sums to T * G
    A = ag.cpu().numpy()[0].astype(np.float64)
    for h in range(H):
        a_ref = g["a_values"][h]
        a_gpu = A[h, g["a_blocks"][h]]
        assert np.all(np.abs(a_gpu - a_ref) <= 1e-3 * a_ref + 1e-30), (h, "A")
        assert abs(A[h, :nc].sum() - g["a_sums"][h]) <= 1e-3 * g["a_sums"][h], (h, "sum A")
        assert abs(g["a_sums"][h] - cfg.T * G) <= 1e-6 * cfg.T * G
    # index rows of the sampled chunks
    idx_dev = index_rows(dw.index, mb)
    for b0, want in rows.items():
        n = want[0].shape[0]
        for h in range(H):
            got = _bits_to_f64(idx_dev[0, h, b0:b0 + n].contiguous(), "bf16")
            assert np.array_equal(got, want[h]), (b0, h, "index")
    # every view block: V bit for bit, K within one bf16 ulp
    kg = _bits_to_f64(dw.k_view[0, :, :V].contiguous(), "bf16")
    vg = _bits_to_f64(v_view_token_major(dw.v_view)[0, :, :V].contiguous(), "bf16")
    kv = exp["k"].astype(np.float64)
    assert not np.isnan(kv).any() and not np.isnan(exp["v"]).any()
    assert np.array_equal(vg, exp["v"].astype(np.float64)), "V view"
    ulp = np.ldexp(1.0, np.frexp(np.abs(kv))[1] - 8)
    rot = 1e-6 * np.abs(kv).max(axis=-1, keepdims=True)
    bad = np.abs(kg - kv) > ulp + rot
    assert not bad.any(), ("K view", np.argwhere(bad)[:4])
    print(f"[gpu] c5: selection, A samples, index rows of {len(rows)} chunks and all "
          f"{H * V // 32} view blocks match", flush=True)
