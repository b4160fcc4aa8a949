"""Plain CPU oracle of the KVMem hot path (NumPy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check in __graft_entry__ and the
cpu_baseline leg of bench.py use it.  It shares no code with the HIP library.

Sources (web pages, cited by title and section):
  [README]  "KVMEM: Virtualizing a million-token agent workspace with paged KV"
            (reproduction README, daiwk.github.io auto-research) -- sections
            'Background and main changes', 'Core equation',
            '2026-09-08 validation correction', 'Local reproduction'.
  [REVIEW]  "KVMem: Virtualizing Million-Token Agent Workspaces on a Consumer
            GPU" (evolve.pub review) -- sections 'Summary',
            'Key claims under review', 'Strengths', 'Scope & Claims'.

Every step is the plain definition evaluated in float64; values are rounded
to the storage dtype exactly where the library stores them (the Mean-K index
and the materialised K view).  Where the pages leave a step open the reading
taken is stated in the function's docstring.

Pins: every function here is checked by tests/test_oracle_pins.py against a
closed form, an invariant, a brute-force enumeration, an independent library
routine or a hand-derived fixture.  No function is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK_TOKENS = 32          # [REVIEW 'Summary']: selection works on 32-token blocks
BF16_OVERFLOW = 2.0 ** 128


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64.  bf16 arrives as raw uint16 bits."""
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(raw, dtype=np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even), as float64.

    Written from the format: for |x| >= 2**-126 the quantum is 2**(e-8) with
    x = m * 2**e, 0.5 <= |m| < 1; below that the subnormal quantum 2**-133
    applies.  Results of magnitude >= 2**128 overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    quantum = np.ldexp(np.ones_like(x), e - 8)
    r = np.rint(x / quantum) * quantum
    big = np.abs(r) >= BF16_OVERFLOW
    if np.any(big):
        r = np.where(big, np.copysign(np.inf, x), r)
    return r


def round_f32(x: np.ndarray) -> np.ndarray:
    """Nearest fp32 value (IEEE cast, ties to even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else round_f32(x)


def bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 values that are exactly bf16 -> raw uint16 bits."""
    f = np.asarray(x64, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# the paged workspace ([README 'Background and main changes']: history is kept
# as paged KV; [README 'Core equation']: address space and execution window
# are separate)
# ---------------------------------------------------------------------------

@dataclass
class Workspace:
    k_pool: np.ndarray        # [n_pages][Hkv][32][d] stored keys (pre-RoPE)
    v_pool: np.ndarray        # [n_pages][Hkv][32][d] stored values
    block_table: np.ndarray   # [S][max_blocks] logical block -> page
    n_tokens: np.ndarray      # [S] history lengths
    dtype: str                # "f32" | "bf16"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def block_counts(n_tok: int) -> tuple[int, int]:
    """(complete blocks, all blocks incl. a partial tail)."""
    return n_tok // BLOCK_TOKENS, -(-n_tok // BLOCK_TOKENS)


def block_tokens_of(ws: Workspace, pool: np.ndarray, s: int, h: int, blocks) -> np.ndarray:
    """Stored K or V of logical blocks `blocks` of session s, head h: [nb][32][d] float64."""
    pages = ws.block_table[s, np.asarray(blocks, dtype=np.int64)]
    return decode(pool[pages, h], ws.dtype)


# ---------------------------------------------------------------------------
# O1  Mean-K index  ([README 'Core equation']: index vector k_bar_b per block;
#     [REVIEW 'Summary']: position-independent Mean-K index over 32-token
#     blocks -> the mean of the block's pre-RoPE keys)
# ---------------------------------------------------------------------------

def mean_k_rows(ws: Workspace, s: int, h: int, blocks) -> np.ndarray:
    """k_bar[beta] = round_store(sum_u K_pre[32*beta + u] / 32) for the given
    complete blocks; the sum is taken in float64."""
    keys = block_tokens_of(ws, ws.k_pool, s, h, blocks)
    return round_store(keys.sum(axis=1) / BLOCK_TOKENS, ws.dtype)


def mean_k_index(ws: Workspace, s: int, h: int, chunk: int = 4096) -> np.ndarray:
    """Mean-K index of every complete block of session s, KV head h: [Nb][d].

    Reading taken: the partial tail block is not indexed (it is not a complete
    32-token block).  The loop over block ranges only bounds memory; blocks
    are independent.
    """
    nb, _ = block_counts(int(ws.n_tokens[s]))
    out = np.empty((nb, ws.head_dim), np.float64)
    for b0 in range(0, nb, chunk):
        b1 = min(nb, b0 + chunk)
        out[b0:b1] = mean_k_rows(ws, s, h, range(b0, b1))
    return out


# ---------------------------------------------------------------------------
# O2  q-RMSNorm  ([README '2026-09-08 validation correction']: the query is
#     normalised before scoring; omitting it was a withdrawn bug)
# ---------------------------------------------------------------------------

def q_rmsnorm(q: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """q_tilde = w * q / sqrt(mean_i q_i^2 + eps) over the last axis.

    Reading taken: RMSNorm with the weight applied after normalisation and no
    intermediate rounding; eps = 1e-6 unless stated.
    """
    q = np.asarray(q, dtype=np.float64)
    rms = np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + float(eps))
    return q / rms * np.asarray(w, dtype=np.float64)


# ---------------------------------------------------------------------------
# O3  block scores  ([README 'Core equation']: s_b = <q, k_bar_b> / sqrt(d))
# ---------------------------------------------------------------------------

def block_scores(qn_group: np.ndarray, index: np.ndarray) -> np.ndarray:
    """s[t, g, beta] = <q_tilde[t, g], k_bar[beta]> / sqrt(d).

    qn_group: [T][G][d] normalised (un-rotated) queries of the KV head's group;
    index: [Nb][d].  Reading taken: scoring uses the pre-RoPE query against the
    pre-RoPE index, so the score does not depend on positions.
    """
    T, G, d = qn_group.shape
    return (qn_group.reshape(T * G, d) @ index.T).reshape(T, G, -1) / np.sqrt(d)


# ---------------------------------------------------------------------------
# O4/O5  per-head softmax over blocks, then GQA sum
#     ([README '2026-09-08 validation correction']: averaging GQA query heads
#     before the softmax was a withdrawn bug -> softmax per query head first)
# ---------------------------------------------------------------------------

def softmax_blocks(s: np.ndarray) -> np.ndarray:
    """p = exp(s - max) / sum exp(s - max) along the block axis (last)."""
    if s.shape[-1] == 0:
        return s.copy()
    z = np.exp(s - s.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def gqa_sum(p: np.ndarray) -> np.ndarray:
    """A[beta] = sum over query tokens t and group heads g of p[t, g, beta].

    Reading taken for multi-token steps: the per-(token, head) softmaxes are
    summed, which keeps a fixed block budget.
    """
    return p.sum(axis=(0, 1))


# ---------------------------------------------------------------------------
# O6/O7  budgeted selection plus recent blocks
#     ([README 'Core equation']: selected KV is concatenated within the block
#     budget; [README 'Local reproduction']: the recent-only control uses the
#     same block budget)
# ---------------------------------------------------------------------------

def recent_split(n_tok: int, n_recent: int) -> tuple[int, int, int]:
    """(n_candidates, recent_start, n_blocks_all).

    Recent = the last n_recent logical blocks, a partial tail counting as one.
    Candidates = complete blocks before the recent range.
    """
    nb_full, nb_all = block_counts(n_tok)
    r_start = max(0, nb_all - n_recent)
    return min(nb_full, r_start), r_start, nb_all


def select_topk(A: np.ndarray, n_cand: int, k: int) -> np.ndarray:
    """The min(k, n_cand) candidates with the largest A, ties to the lower
    block index, returned in ascending block order."""
    k_eff = min(k, n_cand)
    if k_eff <= 0:
        return np.zeros(0, np.int64)
    a = np.asarray(A[:n_cand], dtype=np.float64)
    beta = np.arange(n_cand)
    order = np.lexsort((beta, -a))          # primary: A descending, then beta ascending
    return np.sort(order[:k_eff])


def view_list(A: np.ndarray, n_tok: int, k: int, n_recent: int) -> tuple[np.ndarray, int]:
    """Selected blocks ascending, then the recent blocks ascending; and the
    number of view tokens V (32 per block except a partial tail)."""
    n_cand, r_start, nb_all = recent_split(n_tok, n_recent)
    sel = select_topk(A, n_cand, k)
    lst = np.concatenate([sel, np.arange(r_start, nb_all)]).astype(np.int64)
    V = BLOCK_TOKENS * len(sel) + max(0, n_tok - BLOCK_TOKENS * r_start)
    return lst, V


def view_tokens(n_tok: int, k: int, n_recent: int) -> int:
    """V without needing the scores (it depends only on the lengths)."""
    n_cand, r_start, _ = recent_split(n_tok, n_recent)
    return BLOCK_TOKENS * min(k, n_cand) + max(0, n_tok - BLOCK_TOKENS * r_start)


# ---------------------------------------------------------------------------
# O8  RoPE and materialisation  ([REVIEW 'Summary', 'Scope & Claims']: the
#     selected blocks are restored with position-consistent re-RoPE into a
#     bounded execution view; [README 'Background and main changes']: the view
#     lies within the native window)
# ---------------------------------------------------------------------------

def rope_angles(pos: np.ndarray, d: int, theta: float) -> np.ndarray:
    """phi[..., i] = pos * theta**(-2i/d), i < d/2, in float64."""
    inv_freq = float(theta) ** (-(2.0 * np.arange(d // 2, dtype=np.float64)) / d)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE over the full head dim: pairs (i, i + d/2).

    Reading taken: NeoX pairing, all d dims rotated, exact float64 angle.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    phi = rope_angles(np.broadcast_to(np.asarray(pos, dtype=np.float64), x.shape[:-1]), d, theta)
    c, s = np.cos(phi), np.sin(phi)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def materialize(ws: Workspace, s: int, h: int, lst: np.ndarray, V: int, theta: float):
    """View slot j = 32*m + u takes token u of the m-th listed block.

    K_view[j] = round_store(RoPE(K_pre[token], j)); V_view[j] = V[token]
    exactly.  Returns (K_view, V_view) as float64 arrays [V][d].
    """
    d = ws.head_dim
    kv = np.zeros((V, d)); vv = np.zeros((V, d))
    if V == 0:
        return kv, vv
    nblk = -(-V // BLOCK_TOKENS)
    keys = block_tokens_of(ws, ws.k_pool, s, h, lst[:nblk]).reshape(-1, d)[:V]
    vals = block_tokens_of(ws, ws.v_pool, s, h, lst[:nblk]).reshape(-1, d)[:V]
    kv = round_store(rope(keys, np.arange(V), theta), ws.dtype)
    return kv, vals


# ---------------------------------------------------------------------------
# O9  decode attention over the view ([README 'Local reproduction']: the view
#     replaces full attention; "attention replacement")
# ---------------------------------------------------------------------------

def attend(qn_group: np.ndarray, k_view: np.ndarray, v_view: np.ndarray, theta: float) -> np.ndarray:
    """o[t, g] = sum_j softmax_j(<RoPE(q_tilde[t, g], V + t), K_view[j]> / sqrt(d)) V_view[j].

    Reading taken: query token t sits at view position V + t and attends to the
    whole view only (no mask among the step's own tokens).  An empty view
    gives a zero output.
    """
    T, G, d = qn_group.shape
    V = k_view.shape[0]
    if V == 0:
        return np.zeros((T, G, d))
    pos = (V + np.arange(T, dtype=np.float64))[:, None]
    qr = rope(qn_group, np.broadcast_to(pos, (T, G)), theta)            # [T][G][d]
    logits = (qr.reshape(T * G, d) @ k_view.T) / np.sqrt(d)
    p = softmax_blocks(logits)
    return (p @ v_view).reshape(T, G, d)


# ---------------------------------------------------------------------------
# F1  step-level view reuse ([REVIEW 'Scope & Claims']: recall is scheduled per
#     agent step; [REVIEW 'Strengths']: attention is stable within a step and
#     shifts across step boundaries -> the view selected at a step boundary
#     serves the step's decode tokens, which are appended to it)
# ---------------------------------------------------------------------------

def append_history(ws: Workspace, s: int, k_new_raw: np.ndarray, v_new_raw: np.ndarray) -> Workspace:
    """History of session s after T_new new tokens: token t is stored (bit
    copy) at history position N + t, i.e. slot (N + t) % 32 of the page the
    block table names for block (N + t) // 32.  k_new_raw, v_new_raw: stored
    values [T_new][Hkv][d].  Returns a new Workspace (pools copied) with
    n_tokens[s] advanced by T_new."""
    kp, vp = ws.k_pool.copy(), ws.v_pool.copy()
    n0 = int(ws.n_tokens[s])
    for t in range(k_new_raw.shape[0]):
        pos = n0 + t
        page = int(ws.block_table[s, pos // BLOCK_TOKENS])
        kp[page, :, pos % BLOCK_TOKENS] = k_new_raw[t]
        vp[page, :, pos % BLOCK_TOKENS] = v_new_raw[t]
    n_tok = np.array(ws.n_tokens, copy=True)
    n_tok[s] = n0 + k_new_raw.shape[0]
    return Workspace(kp, vp, ws.block_table, n_tok, ws.dtype, ws.n_q_heads, ws.n_kv_heads, ws.head_dim)


def append_view(k_view: np.ndarray, v_view: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                theta: float, dtype: str):
    """View of one KV head after appending T_new tokens: with V = len(k_view),
    position V + t takes round_store(RoPE(k_new[t], V + t)) and v_new[t]
    exactly (the same rule as materialisation at that position).  k_new,
    v_new: float64 [T_new][d]."""
    V = k_view.shape[0]
    pos = V + np.arange(k_new.shape[0])
    k_add = round_store(rope(k_new, pos, theta), dtype)
    return np.concatenate([k_view, k_add]), np.concatenate([v_view, np.asarray(v_new, dtype=np.float64)])


def update_index_rows(ws: Workspace, s: int, h: int, first_block: int) -> np.ndarray:
    """Mean-K rows of the complete blocks first_block .. Nb - 1 (the blocks a
    decode step completed): [Nb - first_block][d]."""
    nb, _ = block_counts(int(ws.n_tokens[s]))
    return mean_k_rows(ws, s, h, range(first_block, nb)) if nb > first_block else np.zeros((0, ws.head_dim))


# ---------------------------------------------------------------------------
# F3  selection-quality diagnostic ([REVIEW 'Strengths']: a few top blocks
#     carry most of the attention mass; [README 'Local reproduction']: the
#     selection is compared with full attention and the recent-only control)
# ---------------------------------------------------------------------------

def attention_mass(qn_group: np.ndarray, keys: np.ndarray, listed_blocks, theta: float, dtype: str):
    """Share of full attention over the history that the listed blocks carry.

    Full attention = attention over a full-budget view: history token j's key
    rotated at position j and stored-rounded, query token t at position N + t
    (N = len(keys)).  keys: pre-RoPE keys [N][d] float64 of one KV head, in
    history order; listed_blocks: block indices (entries outside the history
    are ignored).  Returns (mass [T][G], lse [T][G]) with lse the natural
    log-sum-exp of the logits.  An empty history gives mass 0, lse -inf.
    """
    T, G, d = qn_group.shape
    N = keys.shape[0]
    if N == 0:
        return np.zeros((T, G)), np.full((T, G), -np.inf)
    kfull = round_store(rope(keys, np.arange(N), theta), dtype)
    pos = (N + np.arange(T, dtype=np.float64))[:, None]
    qr = rope(qn_group, np.broadcast_to(pos, (T, G)), theta)
    logits = (qr.reshape(T * G, d) @ kfull.T) / np.sqrt(d)
    mx = logits.max(axis=-1, keepdims=True)
    z = np.exp(logits - mx)
    tot = z.sum(axis=-1)
    in_list = np.zeros(N, bool)
    for b in np.asarray(listed_blocks, dtype=np.int64):
        if 0 <= b and BLOCK_TOKENS * b < N:
            in_list[BLOCK_TOKENS * b:BLOCK_TOKENS * (b + 1)] = True
    mass = z[:, in_list].sum(axis=-1) / tot
    lse = mx[:, 0] + np.log(tot)
    return mass.reshape(T, G), lse.reshape(T, G)


# ---------------------------------------------------------------------------
# whole path for one session
# ---------------------------------------------------------------------------

def head_aggregate(qn_group: np.ndarray, index: np.ndarray, t_chunk: int = 0) -> np.ndarray:
    """A[beta] for one KV head: per-(token, head) softmax over blocks, summed.

    With t_chunk > 0 the query tokens are taken t_chunk at a time and their
    contributions added; each softmax row is still taken whole, so this only
    bounds memory for long query chunks.
    """
    T = qn_group.shape[0]
    if t_chunk <= 0 or t_chunk >= T:
        return gqa_sum(softmax_blocks(block_scores(qn_group, index)))
    A = np.zeros(index.shape[0])
    for t0 in range(0, T, t_chunk):
        A += gqa_sum(softmax_blocks(block_scores(qn_group[t0:t0 + t_chunk], index)))
    return A


def session_scores(ws: Workspace, s: int, q_raw: np.ndarray, w: np.ndarray, eps: float,
                   index_by_head: list[np.ndarray], keep_scores: bool = True, t_chunk: int = 0):
    """Per-head scores s [Hkv][T][G][Nb] (optional) and aggregated A [Hkv][Nb]
    of session s.  q_raw: stored queries [T][Hq][d] of session s.
    """
    G = ws.group
    qn = q_rmsnorm(decode(q_raw, ws.dtype), w, eps)                      # [T][Hq][d]
    S_all, A_all = [], []
    for h in range(ws.n_kv_heads):
        qg = qn[:, h * G:(h + 1) * G]
        if keep_scores:
            sc = block_scores(qg, index_by_head[h])
            S_all.append(sc)
            A_all.append(gqa_sum(softmax_blocks(sc)))
        else:
            A_all.append(head_aggregate(qg, index_by_head[h], t_chunk))
    return S_all, A_all, qn


def run_session(ws: Workspace, s: int, q_raw: np.ndarray, w: np.ndarray, eps: float,
                k: int, n_recent: int, theta: float, heads=None, with_attend: bool = True):
    """Index -> scores -> selection -> view -> attention for session s.

    Returns a dict of per-KV-head results (lists indexed by head).
    """
    H, G = ws.n_kv_heads, ws.group
    n_tok = int(ws.n_tokens[s])
    index = [mean_k_index(ws, s, h) for h in range(H)]
    scores, A, qn = session_scores(ws, s, q_raw, w, eps, index)
    heads = range(H) if heads is None else heads
    out = {"index": index, "scores": scores, "A": A, "lists": {}, "V": None,
           "k_view": {}, "v_view": {}, "out": {}}
    for h in heads:
        lst, V = view_list(A[h], n_tok, k, n_recent)
        out["lists"][h] = lst
        out["V"] = V
        kv, vv = materialize(ws, s, h, lst, V, theta)
        out["k_view"][h] = kv
        out["v_view"][h] = vv
        if with_attend:
            out["out"][h] = attend(qn[:, h * G:(h + 1) * G], kv, vv, theta)
    return out
