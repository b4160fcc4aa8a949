"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a closed form, an invariant, a
brute-force enumeration, an independent library routine or a hand-derived
fixture under tests/golden/.  A plausible slip in the oracle (a dropped term,
a wrong sign, index or pairing, a transposed operand, a wrong tie rule) fails
at least one of them.
"""
from __future__ import annotations

import itertools
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

from oracle import kvmem_oracle as O
from tests.helpers import logical_tokens, make_workload, oracle_ws, small_cfg
from workloads import CONFIGS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def _golden_pairs(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        # two expressions separated by 2+ spaces
        parts = [p for p in line.split("  ") if p.strip()]
        out.append((parts[0].strip(), parts[1].strip()))
    return out


def test_round_bf16_golden_cases():
    env = {"inf": math.inf}
    for a, b in _golden_pairs("bf16_rounding.txt"):
        x = float(eval(a, {}, env))
        want = float(eval(b, {}, env))
        got = float(O.round_bf16(np.array([x]))[0])
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (a, got, want)


def test_round_bf16_matches_torch_on_fp32_inputs():
    # torch's fp32 -> bf16 cast is an independent implementation; on fp32
    # inputs there is no double rounding, so the two must agree bit for bit.
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-30).astype(np.float32),
        (rng.standard_normal(50_000) * 1e30).astype(np.float32),
        # exact ties: bf16 value + half quantum
        ((rng.integers(0x3F00, 0x4100, 20_000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_f32_ties():
    assert O.round_f32(np.array([1 + 2.0 ** -24]))[0] == 1.0
    assert O.round_f32(np.array([1 + 3 * 2.0 ** -24]))[0] == 1 + 2.0 ** -22
    assert O.round_f32(np.array([1 + 2.0 ** -24 + 2.0 ** -50]))[0] == 1 + 2.0 ** -23


def test_decode_bf16_bits():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127]
    assert list(O.decode(bits, "bf16")) == want
    # and back: every finite bf16 pattern survives decode -> bf16_bits
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (allbits & 0x7F80) != 0x7F80
    assert np.array_equal(O.bf16_bits(O.decode(allbits[finite], "bf16")), allbits[finite])


# ---------------------------------------------------------------------------
# O1 Mean-K index
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mean_k_identity(dtype):
    # <q, k_bar> equals the mean of the per-token scores (linearity), up to the
    # single storage rounding of k_bar.
    cfg = small_cfg(dtype=dtype, n_tokens=(32 * 40 + 7,), Hkv=2, Hq=4, spare_pages=3)
    wl = make_workload(cfg)
    ws = oracle_ws(wl)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, cfg.head_dim))
    for h in range(cfg.n_kv_heads):
        idx = O.mean_k_index(ws, 0, h)
        assert idx.shape == (40, cfg.head_dim)                     # partial tail not indexed
        toks = logical_tokens(wl, wl.k_pool, 0, h)[: 40 * 32]
        per_token = toks @ q.T                                     # [N][6]
        want = per_token.reshape(40, 32, -1).mean(axis=1)          # [40][6]
        got = idx @ q.T
        ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
        mean_abs = np.abs(toks.reshape(40, 32, -1).mean(axis=1))   # |k_bar| before rounding
        bound = (mean_abs @ np.abs(q).T) * ulp + 1e-12
        assert np.all(np.abs(got - want) <= bound)
        assert np.all(np.isfinite(idx))                            # spare NaN pages never read


def test_mean_k_page_permutation_invariance():
    cfg = small_cfg(dtype="bf16", n_tokens=(32 * 64,), Hkv=1, Hq=2)
    wl = make_workload(cfg)
    ws = oracle_ws(wl)
    base = O.mean_k_index(ws, 0, 0)
    # move every page to a new physical slot and rewrite the table
    perm = np.random.default_rng(1).permutation(wl.n_pages)
    k2 = np.empty_like(wl.k_pool)
    k2[perm] = wl.k_pool
    t2 = perm[wl.block_table]
    ws2 = O.Workspace(k2, wl.v_pool, t2, wl.n_tokens, "bf16", 2, 1, 128)
    assert np.array_equal(O.mean_k_index(ws2, 0, 0), base)


def test_mean_k_constant_block():
    # a block whose 32 keys are all equal indexes to that key
    cfg = small_cfg(dtype="f32", n_tokens=(64,), Hkv=1, Hq=1, n_planted=0, R=0)
    wl = make_workload(cfg)
    page = wl.block_table[0, 1]
    v = np.linspace(-3, 3, 128).astype(np.float32)
    wl.k_pool[page, 0, :, :] = v
    idx = O.mean_k_index(oracle_ws(wl), 0, 0)
    assert np.array_equal(idx[1], v.astype(np.float64))


# ---------------------------------------------------------------------------
# O2 q-RMSNorm
# ---------------------------------------------------------------------------

def test_rmsnorm_invariants():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((5, 128)) * 3
    w = 0.5 + rng.random(128)
    qn = O.q_rmsnorm(q, w, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean((qn / w) ** 2, axis=-1)), 1.0, rtol=1e-14)
    for c in (1e-3, 7.0, 1e4):
        np.testing.assert_allclose(O.q_rmsnorm(c * q, w, 0.0), qn, rtol=1e-13)
    # eps shrinks the output by sqrt(ms / (ms + eps))
    ms = np.mean(q * q, axis=-1, keepdims=True)
    np.testing.assert_allclose(O.q_rmsnorm(q, w, 0.25), qn * np.sqrt(ms / (ms + 0.25)), rtol=1e-13)
    # direction preserved (for unit weight)
    qn1 = O.q_rmsnorm(q, np.ones(128), 0.0)
    cos = np.sum(qn1 * q, -1) / np.linalg.norm(qn1, axis=-1) / np.linalg.norm(q, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)


# ---------------------------------------------------------------------------
# O3 scores
# ---------------------------------------------------------------------------

def test_block_scores_closed_forms():
    d = 128
    rng = np.random.default_rng(3)
    qn = rng.standard_normal((2, 3, d))
    index = np.zeros((d + 2, d))
    index[:d] = np.eye(d)                       # basis rows pick one coordinate
    index[d] = 2.5 * qn[1, 2] / np.linalg.norm(qn[1, 2])
    v = rng.standard_normal(d)
    index[d + 1] = v - (v @ qn[0, 0]) / (qn[0, 0] @ qn[0, 0]) * qn[0, 0]   # orthogonal to q[0,0]
    s = O.block_scores(qn, index)
    assert s.shape == (2, 3, d + 2)
    np.testing.assert_allclose(s[:, :, :d], qn / math.sqrt(d), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(s[1, 2, d], 2.5 * np.linalg.norm(qn[1, 2]) / math.sqrt(d), rtol=1e-13)
    assert abs(s[0, 0, d + 1]) < 1e-12


# ---------------------------------------------------------------------------
# O4/O5 softmax + GQA sum
# ---------------------------------------------------------------------------

def test_gqa_regression_fixture():
    rows, exp = [], {}
    for line in open(os.path.join(GOLDEN, "gqa_regression.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0].startswith("head"):
            rows.append([float(x) for x in line[1:]])
        else:
            exp[line[0]] = int(line[1])
    s = np.array(rows)[None]                          # [T=1][G=2][3]
    A = O.gqa_sum(O.softmax_blocks(s))
    e = math.exp
    z0 = e(10) + 2
    z1 = e(-10) + e(1) + 1
    closed = [e(10) / z0 + e(-10) / z1, 1 / z0 + e(1) / z1, 1 / z0 + 1 / z1]
    np.testing.assert_allclose(A, closed, rtol=1e-14)
    assert int(np.argmax(A)) == exp["expect_top1_softmax_then_sum"]
    avg = s.mean(axis=1)
    assert int(np.argmax(avg[0])) == exp["expect_top1_average_first"]
    assert O.select_topk(A, 3, 1).tolist() == [exp["expect_top1_softmax_then_sum"]]


def test_softmax_against_scipy_and_mass():
    from scipy.special import softmax
    rng = np.random.default_rng(4)
    s = rng.standard_normal((3, 8, 500)) * 4
    p = O.softmax_blocks(s)
    np.testing.assert_allclose(p, softmax(s, axis=-1), rtol=1e-13, atol=1e-300)
    A = O.gqa_sum(p)
    assert abs(A.sum() - 3 * 8) < 1e-11                # sum_beta A = T * G
    # shift invariance per head
    np.testing.assert_allclose(O.softmax_blocks(s + rng.standard_normal((3, 8, 1)) * 50), p, rtol=1e-12)


@pytest.mark.parametrize("T,t_chunk,G,nb", [(7, 3, 4, 50), (512, 16, 8, 96), (5, 1, 2, 7), (9, 20, 8, 33),
                                            (6, 6, 3, 40)])
def test_head_aggregate_chunked(T, t_chunk, G, nb):
    """The chunked aggregation (it wrote the 10M-token golden, 16 query tokens
    at a time) against scipy's softmax over the same scores, summed over all
    tokens and heads, for chunk sizes that do and do not divide T; and the
    closed form sum_beta A = T * G."""
    from scipy.special import softmax
    rng = np.random.default_rng(T * 1000 + t_chunk)
    d = 128
    qg = rng.standard_normal((T, G, d)) * 3
    index = rng.standard_normal((nb, d))
    s = np.einsum("tgi,bi->tgb", qg, index) / math.sqrt(d)
    want = softmax(s, axis=-1).sum(axis=(0, 1))
    got = O.head_aggregate(qg, index, t_chunk)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)
    assert abs(got.sum() - T * G) <= 1e-10 * T * G
    # a chunk that the loop dropped or counted twice changes the sum by G * t_chunk
    if 0 < t_chunk < T:
        assert abs(O.head_aggregate(qg[:T - 1], index, t_chunk).sum() - (T - 1) * G) <= 1e-10 * T * G


# ---------------------------------------------------------------------------
# O6/O7 selection
# ---------------------------------------------------------------------------

def _brute_topk(A, k):
    """Max-sum subset of size k; among ties the lexicographically smallest
    sorted index vector (ties -> lower block index)."""
    best = None
    for sub in itertools.combinations(range(len(A)), k):
        key = (-sum(A[i] for i in sub), sub)
        if best is None or key < best:
            best = key
    return list(best[1])


def test_select_topk_brute_force():
    rng = np.random.default_rng(6)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        if trial % 2:
            A = rng.integers(0, 4, n).astype(float)          # tie heavy
        else:
            A = rng.random(n)
        k = int(rng.integers(0, n + 2))
        got = O.select_topk(A, n, k).tolist()
        want = _brute_topk(list(A), min(k, n)) if min(k, n) > 0 else []
        assert got == want, (A, k, got, want)


def test_view_list_recent_and_tail():
    A = np.arange(20, dtype=float)[::-1].copy()          # block 0 best
    # 20 complete blocks + partial tail of 5 tokens; R = 3 -> recent = blocks 18, 19, 20
    lst, V = O.view_list(A, 20 * 32 + 5, k=4, n_recent=3)
    assert lst.tolist() == [0, 1, 2, 3, 18, 19, 20]
    assert V == 4 * 32 + 2 * 32 + 5
    # k = 0: recent-only control (README 'Local reproduction')
    lst, V = O.view_list(A, 20 * 32 + 5, k=0, n_recent=3)
    assert lst.tolist() == [18, 19, 20] and V == 69
    # budget covers everything: whole history in order (full-attention control)
    lst, V = O.view_list(A, 20 * 32 + 5, k=1000, n_recent=3)
    assert lst.tolist() == list(range(21)) and V == 20 * 32 + 5
    # R = 0 with a partial tail: the tail is neither recent nor indexed
    lst, V = O.view_list(A, 20 * 32 + 5, k=2, n_recent=0)
    assert lst.tolist() == [0, 1] and V == 64
    # empty history
    lst, V = O.view_list(np.zeros(0), 0, k=5, n_recent=5)
    assert lst.tolist() == [] and V == 0
    # more recent blocks than history
    lst, V = O.view_list(A[:2], 2 * 32, k=5, n_recent=9)
    assert lst.tolist() == [0, 1] and V == 64
    assert O.view_tokens(20 * 32 + 5, 4, 3) == 4 * 32 + 2 * 32 + 5


def test_budget_constants_from_the_pages():
    # 1M workspace: 7,936 selected + 256 recent blocks of 32 tokens fill exactly
    # the 256K native window (review, 'Key claims under review'); 256K workspace:
    # 1,024 + 64 blocks -> 34,816 tokens.
    c3, c2 = CONFIGS["c3"], CONFIGS["c2"]
    assert O.view_tokens(c3.n_tokens[0], c3.k_select, c3.n_recent) == 256 * 1024
    assert O.view_tokens(c2.n_tokens[0], c2.k_select, c2.n_recent) == 34816
    assert O.BLOCK_TOKENS == 32


# ---------------------------------------------------------------------------
# O8 RoPE + materialise
# ---------------------------------------------------------------------------

def test_rope_complex_form_and_properties():
    d, theta = 128, 1e6
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, d))
    pos = np.array([0, 1, 2, 17, 4096, 65535, 100000, 262143, 262144], float)
    y = O.rope(x, pos, theta)
    # independent complex formulation: z_i = x_i + i x_{i+d/2}, z_i * e^{i phi_i}
    i = np.arange(d // 2)
    phi = pos[:, None] * np.exp(-(2 * i / d) * np.log(theta))
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * phi)
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-9)
    np.testing.assert_array_equal(O.rope(x, np.zeros(9), theta), x)          # RoPE(x, 0) = x
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # re-RoPE: RoPE(RoPE(x, p), j - p) = RoPE(x, j)
    p = np.array([5.0, 1000.0, 77777.0])
    j = np.array([0.0, 262143.0, 12.0])
    np.testing.assert_allclose(O.rope(O.rope(x[:3], p, theta), j - p, theta), O.rope(x[:3], j, theta),
                               atol=1e-10)
    # <RoPE(q, a), RoPE(k, b)> depends on a - b only
    q, k = x[0], x[1]
    v1 = O.rope(q, 1000.0, theta) @ O.rope(k, 300.0, theta)
    v2 = O.rope(q, 250700.0, theta) @ O.rope(k, 250000.0, theta)
    assert abs(v1 - v2) < 1e-9


def test_rope_angle_exact_against_decimal():
    # phi = p * theta^(-2i/d) to float64 accuracy at the largest view positions
    getcontext().prec = 50
    d, theta = 128, 1e6
    for p in (262143, 1048575, 9_999_999):
        got = O.rope_angles(np.array([float(p)]), d, theta)[0]
        for i in (0, 1, 7, 31, 63):
            want = Decimal(p) * (Decimal(theta).ln() * Decimal(-2 * i) / Decimal(d)).exp()
            assert abs(Decimal(float(got[i])) - want) <= abs(want) * Decimal(2.0 ** -51)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_materialize_full_budget_is_full_history(dtype):
    cfg = small_cfg(dtype=dtype, n_tokens=(32 * 12 + 9,), Hkv=2, Hq=4, k=100, R=2)
    wl = make_workload(cfg)
    ws = oracle_ws(wl)
    A = np.ones(12)
    lst, V = O.view_list(A, int(wl.n_tokens[0]), cfg.k_select, cfg.n_recent)
    assert V == int(wl.n_tokens[0])
    for h in range(2):
        kv, vv = O.materialize(ws, 0, h, lst, V, cfg.rope_theta)
        toks_k = logical_tokens(wl, wl.k_pool, 0, h)
        toks_v = logical_tokens(wl, wl.v_pool, 0, h)
        np.testing.assert_array_equal(vv, toks_v)                       # V copied bit for bit
        direct = O.round_store(O.rope(toks_k, np.arange(V), cfg.rope_theta), dtype)
        np.testing.assert_array_equal(kv, direct)


def test_materialize_reorders_by_list():
    cfg = small_cfg(dtype="f32", n_tokens=(32 * 10,), Hkv=1, Hq=2, k=3, R=1)
    wl = make_workload(cfg)
    ws = oracle_ws(wl)
    lst = np.array([2, 5, 7, 9])
    kv, vv = O.materialize(ws, 0, 0, lst, 128, 1e6)
    toks_k = logical_tokens(wl, wl.k_pool, 0, 0)
    toks_v = logical_tokens(wl, wl.v_pool, 0, 0)
    for m, b in enumerate(lst):
        np.testing.assert_array_equal(vv[32 * m:32 * m + 32], toks_v[32 * b:32 * b + 32])
        # re-RoPE: the block's keys sit at view positions 32m.., not at 32b..
        np.testing.assert_array_equal(
            kv[32 * m:32 * m + 32],
            O.round_f32(O.rope(toks_k[32 * b:32 * b + 32], np.arange(32 * m, 32 * m + 32), 1e6)))


# ---------------------------------------------------------------------------
# O9 attention
# ---------------------------------------------------------------------------

def test_attend_against_torch_sdpa():
    rng = np.random.default_rng(8)
    T, G, d, V = 3, 4, 128, 300
    qn = rng.standard_normal((T, G, d))
    kv = rng.standard_normal((V, d))
    vv = rng.standard_normal((V, d))
    got = O.attend(qn, kv, vv, 1e6)
    # independent: complex-form RoPE of q at V + t, then torch SDPA in float64
    i = np.arange(d // 2)
    pos = (V + np.arange(T))[:, None, None].astype(float)
    phi = pos * np.exp(-(2 * i / d) * np.log(1e6))
    z = (qn[..., : d // 2] + 1j * qn[..., d // 2:]) * np.exp(1j * phi)
    qr = np.concatenate([z.real, z.imag], -1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr.reshape(1, T * G, d)), torch.from_numpy(kv[None]), torch.from_numpy(vv[None]))
    np.testing.assert_allclose(got.reshape(T * G, d), ref[0].numpy(), rtol=1e-10, atol=1e-12)
    # convex combination of the value rows
    assert np.all(got <= vv.max(0) + 1e-12) and np.all(got >= vv.min(0) - 1e-12)
    assert np.array_equal(O.attend(qn, kv[:0], vv[:0], 1e6), np.zeros((T, G, d)))


def test_full_budget_pipeline_is_full_attention():
    # README 'Local reproduction': with a budget covering every block the view
    # is the whole history and attention over it is plain full attention.
    cfg = small_cfg(dtype="f32", n_tokens=(32 * 20 + 3,), Hkv=2, Hq=8, k=10_000, R=1, T=2)
    wl = make_workload(cfg)
    ws = oracle_ws(wl)
    r = O.run_session(ws, 0, wl.q[0], wl.q_norm_w, cfg.eps, cfg.k_select, cfg.n_recent, cfg.rope_theta)
    N = int(wl.n_tokens[0])
    d, G = 128, 4
    qf = wl.q[0].astype(np.float64)
    qn = qf / np.sqrt(np.mean(qf ** 2, -1, keepdims=True) + cfg.eps)
    i = np.arange(d // 2)
    for h in range(2):
        toks_k = logical_tokens(wl, wl.k_pool, 0, h)
        toks_v = logical_tokens(wl, wl.v_pool, 0, h)
        phik = np.arange(N)[:, None] * np.exp(-(2 * i / d) * np.log(1e6))
        zk = (toks_k[:, :64] + 1j * toks_k[:, 64:]) * np.exp(1j * phik)
        kr = np.concatenate([zk.real, zk.imag], -1).astype(np.float32).astype(np.float64)
        q_g = qn[:, h * G:(h + 1) * G]
        phiq = (N + np.arange(2))[:, None, None] * np.exp(-(2 * i / d) * np.log(1e6))
        zq = (q_g[..., :64] + 1j * q_g[..., 64:]) * np.exp(1j * phiq)
        qr = np.concatenate([zq.real, zq.imag], -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr.reshape(1, 2 * G, d)), torch.from_numpy(kr[None]),
            torch.from_numpy(toks_v[None]))
        np.testing.assert_allclose(r["out"][h].reshape(2 * G, d), ref[0].numpy(), rtol=1e-9, atol=1e-11)


def test_recent_only_control_pipeline():
    cfg = small_cfg(dtype="bf16", n_tokens=(32 * 30,), Hkv=1, Hq=4, k=0, R=5)
    wl = make_workload(cfg)
    r = O.run_session(oracle_ws(wl), 0, wl.q[0], wl.q_norm_w, cfg.eps, 0, 5, cfg.rope_theta)
    assert r["lists"][0].tolist() == [25, 26, 27, 28, 29] and r["V"] == 160


def test_planted_blocks_are_found():
    # with strong planted offsets along q_hat, the planted blocks carry the
    # largest aggregated scores (a sanity pin of the whole score chain)
    cfg = CONFIGS["c1"]
    wl = make_workload(cfg)
    ws = oracle_ws(wl)
    idx = [O.mean_k_index(ws, 0, 0)]
    _, A, _ = O.session_scores(ws, 0, wl.q[0], wl.q_norm_w, cfg.eps, idx)
    nc, _, _ = O.recent_split(int(wl.n_tokens[0]), cfg.n_recent)
    planted = set(np.nonzero(wl.plant_mag[0, 0] > 0)[0].tolist())
    assert set(O.select_topk(A[0], nc, cfg.k_select).tolist()) == planted


# ---------------------------------------------------------------------------
# step-level view reuse: append and incremental index
# ---------------------------------------------------------------------------

def _decode_wl(dtype, n_tokens, extra, seed):
    from workloads import draw_decode_tokens, with_decode_capacity
    cfg = small_cfg(f"dec_{dtype}", dtype, S=len(n_tokens), Hq=4, Hkv=2, n_tokens=n_tokens, k=3, R=2,
                    n_planted=2, seed=seed)
    return with_decode_capacity(make_workload(cfg), extra), draw_decode_tokens


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_history_lands_at_history_positions(dtype):
    """The appended tokens read back, through the page table directly, at
    positions N .. N + T_new - 1; every earlier token is unchanged; the
    blocks the append completed index to the mean of their keys."""
    wl, draw = _decode_wl(dtype, (32 * 5 + 7, 32 * 3), 80, 71)
    ws = oracle_ws(wl)
    kn, vn = draw(wl.cfg, 0, 45)
    for s in range(2):
        n0 = int(ws.n_tokens[s])
        ws2 = O.append_history(ws, s, kn[s], vn[s])
        assert int(ws2.n_tokens[s]) == n0 + 45
        wl2 = type(wl)(wl.cfg, ws2.k_pool, ws2.v_pool, wl.block_table, ws2.n_tokens, wl.q, wl.q_norm_w,
                       wl.qhat, wl.plant_mag)
        for h in range(2):
            before = logical_tokens(wl, wl.k_pool, s, h)
            after_k = logical_tokens(wl2, ws2.k_pool, s, h)
            after_v = logical_tokens(wl2, ws2.v_pool, s, h)
            assert np.array_equal(after_k[:n0], before)
            assert np.array_equal(after_k[n0:], O.decode(kn[s, :, h], dtype))
            assert np.array_equal(after_v[n0:], O.decode(vn[s, :, h], dtype))
            # newly completed blocks: the rounded mean of their 32 keys
            first = n0 // 32
            rows = O.update_index_rows(ws2, s, h, first)
            nb2 = (n0 + 45) // 32
            assert rows.shape[0] == nb2 - first
            for i, b in enumerate(range(first, nb2)):
                want = O.round_store(after_k[32 * b:32 * b + 32].mean(axis=0), dtype)
                assert np.array_equal(rows[i], want)
            # and rows of untouched blocks equal the full index
            full = O.mean_k_index(ws2, s, h)
            assert np.array_equal(full[first:], rows)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_view_equals_gathering_the_block(dtype):
    """Appending the 32 tokens of a block to a view of whole blocks gives
    exactly the view that lists that block last (positions continue at V)."""
    wl, _ = _decode_wl(dtype, (32 * 9,), 0, 72)
    ws = oracle_ws(wl)
    lst = np.array([1, 4, 6], np.int64)
    theta = 1e6
    for h in range(2):
        kv, vv = O.materialize(ws, 0, h, lst, 96, theta)
        blk = O.block_tokens_of(ws, ws.k_pool, 0, h, [7])[0]
        vblk = O.block_tokens_of(ws, ws.v_pool, 0, h, [7])[0]
        k2, v2 = O.append_view(kv, vv, blk, vblk, theta, dtype)
        kw, vw = O.materialize(ws, 0, h, np.append(lst, 7), 128, theta)
        assert np.array_equal(k2, kw) and np.array_equal(v2, vw)
        # an off-by-one position would rotate the block differently
        k_wrong = O.round_store(O.rope(blk, 97 + np.arange(32), theta), dtype)
        assert not np.array_equal(k_wrong, kw[96:])


def test_append_one_at_a_time_equals_all_at_once():
    """Position bookkeeping: appending tokens one per step gives the same
    history and view as appending them in one call."""
    wl, draw = _decode_wl("bf16", (32 * 4 + 30,), 40, 73)
    ws = oracle_ws(wl)
    kn, vn = draw(wl.cfg, 1, 5)
    theta = 1e6
    kv0 = np.zeros((0, 128)); vv0 = np.zeros((0, 128))
    ws_all = O.append_history(ws, 0, kn[0], vn[0])
    k_all, v_all = O.append_view(kv0, vv0, O.decode(kn[0, :, 1], "bf16"), O.decode(vn[0, :, 1], "bf16"), theta, "bf16")
    ws_one, k_one, v_one = ws, kv0, vv0
    for t in range(5):
        ws_one = O.append_history(ws_one, 0, kn[0, t:t + 1], vn[0, t:t + 1])
        k_one, v_one = O.append_view(k_one, v_one, O.decode(kn[0, t:t + 1, 1], "bf16"),
                                     O.decode(vn[0, t:t + 1, 1], "bf16"), theta, "bf16")
    assert np.array_equal(ws_one.k_pool, ws_all.k_pool) and np.array_equal(ws_one.v_pool, ws_all.v_pool)
    assert np.array_equal(k_one, k_all) and np.array_equal(v_one, v_all)


# ---------------------------------------------------------------------------
# selection-quality diagnostic
# ---------------------------------------------------------------------------

def _mass_case(seed=91, n_tok=32 * 37 + 11, T=2):
    rng = np.random.default_rng(seed)
    d = 128
    keys = O.round_bf16(rng.standard_normal((n_tok, d)))
    q = rng.standard_normal((T, 4, d)) * 0.3 + 1.0
    qn = O.q_rmsnorm(q, np.ones(d), 1e-6)
    return qn, keys


def test_attention_mass_closed_forms_and_additivity():
    qn, keys = _mass_case()
    nb_all = -(-keys.shape[0] // 32)
    full, lse = O.attention_mass(qn, keys, np.arange(nb_all), 1e6, "bf16")
    assert np.allclose(full, 1.0, atol=1e-13)
    empty, lse2 = O.attention_mass(qn, keys, [], 1e6, "bf16")
    assert np.all(empty == 0) and np.array_equal(lse, lse2)
    a, _ = O.attention_mass(qn, keys, [0, 5, 9, nb_all - 1], 1e6, "bf16")
    b, _ = O.attention_mass(qn, keys, [1, 2, 30], 1e6, "bf16")
    ab, _ = O.attention_mass(qn, keys, [0, 1, 2, 5, 9, 30, nb_all - 1], 1e6, "bf16")
    assert np.allclose(a + b, ab, atol=1e-14)
    ign, _ = O.attention_mass(qn, keys, [0, 5, 9, nb_all - 1, nb_all + 3, -1], 1e6, "bf16")
    assert np.array_equal(ign, a)                              # entries outside the history are ignored
    assert np.all(O.attention_mass(np.zeros((1, 1, 128)), np.zeros((0, 128)), [0], 1e6, "bf16")[0] == 0)


def test_attention_mass_against_complex_rope_and_torch():
    """Independent weights: RoPE written with complex numbers, softmax and
    logsumexp from torch in float64."""
    qn, keys = _mass_case(seed=92, n_tok=32 * 21 + 5, T=3)
    T, G, d = qn.shape
    N = keys.shape[0]
    theta = 1e6
    freq = theta ** (-np.arange(64) * 2.0 / d)

    def crope(x, pos):
        z = (x[..., :64] + 1j * x[..., 64:]) * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * freq)
        return np.concatenate([z.real, z.imag], axis=-1)

    kr = O.round_bf16(crope(keys, np.arange(N)))
    qr = crope(qn, (N + np.arange(T))[:, None] * np.ones((1, G)))
    logits = torch.from_numpy(np.einsum("tgd,jd->tgj", qr, kr) / np.sqrt(d))
    p = torch.softmax(logits, dim=-1).numpy()
    listed = [0, 3, 4, 11, 21]
    tok = np.concatenate([np.arange(32 * b, min(N, 32 * b + 32)) for b in listed])
    mass, lse = O.attention_mass(qn, keys, listed, theta, "bf16")
    assert np.allclose(mass, p[..., tok].sum(axis=-1), atol=1e-12)
    assert np.allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), atol=1e-10)


def test_attention_mass_is_attention_over_the_full_view():
    """Mass of one block = the attention output over a full-budget view whose
    values are that block's indicator (same query position N + t)."""
    wl = make_workload(small_cfg("mass_view", "bf16", S=1, Hq=8, Hkv=2, n_tokens=(32 * 12 + 9,), T=2, k=2, R=1,
                                 n_planted=2, seed=93))
    ws = oracle_ws(wl)
    N = int(wl.n_tokens[0])
    nb_all = -(-N // 32)
    qn = O.q_rmsnorm(O.decode(wl.q[0], "bf16"), wl.q_norm_w, wl.cfg.eps)
    for h in range(2):
        kv, _ = O.materialize(ws, 0, h, np.arange(nb_all), N, 1e6)
        keys = logical_tokens(wl, wl.k_pool, 0, h)
        for b in (0, 4, nb_all - 1):
            vv = np.zeros((N, 128))
            vv[32 * b:min(N, 32 * b + 32), 0] = 1.0
            o = O.attend(qn[:, 4 * h:4 * h + 4], kv, vv, 1e6)
            mass, _ = O.attention_mass(qn[:, 4 * h:4 * h + 4], keys, [b], 1e6, "bf16")
            assert np.allclose(o[..., 0], mass, atol=1e-13)
