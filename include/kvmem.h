/*
 * kvmem.h -- C ABI of the KVMem hot path on MI355X (gfx950).
 *
 * KVMem keeps a long agent history as paged KV and runs each step over a
 * bounded, query-selected execution view.  The library implements the
 * data-parallel path of that method as these calls:
 *
 *   kvmem_build_index    Mean-K index: mean of each 32-token block's pre-RoPE
 *                        keys, per KV head.
 *   kvmem_score_select   q-RMSNorm, block scores s_b = <q, k_bar_b>/sqrt(d),
 *                        per-query-head softmax over blocks, sum per KV head,
 *                        top-k under the block budget plus the recent blocks.
 *   kvmem_materialize    gather of the selected blocks in their original
 *                        order, re-RoPE'd to contiguous view positions.
 *   kvmem_attend         decode attention of the step's queries over the view.
 *   kvmem_attend_paged   the same attention computed straight from the pages
 *                        through the view lists (no materialised view).
 *   kvmem_materialize_attend  the gather and the attention in one pass: the
 *                        view as kvmem_materialize writes it, and the
 *                        attention over it, reading each selected block once.
 *
 * and, for decoding many tokens over one view (step-level reuse):
 *
 *   kvmem_append         new tokens' K/V into the paged history and the view.
 *   kvmem_update_index   Mean-K rows of the blocks completed since the last
 *                        index build.
 *
 * and, for workspaces whose pages live in pinned host memory:
 *
 *   kvmem_stage_view     the listed blocks of every view, copied over the
 *                        host link into a device staging pool in view order.
 *
 * and a selection-quality diagnostic:
 *
 *   kvmem_attention_mass share of full attention over the whole history that
 *                        the listed blocks capture.
 *
 * Sources, cited by page title and section:
 *   [README] "KVMEM: Virtualizing a million-token agent workspace with paged
 *            KV" (reproduction README): 'Background and main changes',
 *            'Core equation', '2026-09-08 validation correction',
 *            'Local reproduction'.
 *   [REVIEW] "KVMem: Virtualizing Million-Token Agent Workspaces on a Consumer
 *            GPU" (evolve.pub review): 'Summary', 'Key claims under review',
 *            'Strengths', 'Scope & Claims'.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers are DEVICE pointers owned by the caller unless the name ends in
 *    _host.  The library allocates nothing and keeps no state between calls
 *    (it only caches the device's compute-unit count to size its grids).
 *  - Every call validates its arguments on the host first; on any invalid
 *    argument it returns an error status and enqueues nothing.  Otherwise it
 *    enqueues its kernels on `stream` (a hipStream_t; NULL = the default
 *    stream) and returns KVMEM_OK without synchronising.  Faults inside a
 *    kernel surface at the caller's next synchronisation, as usual in HIP.
 *  - A failed kernel launch returns KVMEM_E_HIP (work enqueued before it in
 *    the same call may already be running).
 *  - Geometry: head_dim must be 128 and block_tokens 32; n_q_heads must be a
 *    multiple of n_kv_heads (query head g belongs to KV head g / G with
 *    G = n_q_heads / n_kv_heads).  kv_dtype is KVMEM_F32 or KVMEM_BF16 and
 *    applies to the K/V pools, the index, the queries and the view.
 *  - Calls on the same stream are ordered; concurrent calls on different
 *    streams that write the same buffers race.  The library itself is
 *    thread-safe (its only cached value is a device property).
 */
#ifndef KVMEM_H_
#define KVMEM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVMEM_OK = 0,
  KVMEM_E_ARG = 1,          /* null pointer, negative size, inconsistent sizes  */
  KVMEM_E_UNSUPPORTED = 2,  /* geometry or dtype the kernels do not implement   */
  KVMEM_E_WORKSPACE = 3,    /* scratch buffer smaller than the queried size     */
  KVMEM_E_HIP = 4           /* a HIP launch failed                              */
} kvmem_status;

typedef enum { KVMEM_F32 = 0, KVMEM_BF16 = 1 } kvmem_dtype;

/* Bits a kernel ORs into kvmem_workspace.dev_error when it meets a bad table
 * entry.  The offending block is not read; its outputs are written as zeros. */
#define KVMEM_DEVERR_PAGE  1   /* block_table entry outside [0, n_pages)            */
#define KVMEM_DEVERR_BLOCK 2   /* view_blocks entry outside the session's history   */

typedef struct {
  int32_t n_q_heads;     /* Hq                                  */
  int32_t n_kv_heads;    /* Hkv                                 */
  int32_t head_dim;      /* d, must be 128                      */
  int32_t block_tokens;  /* tokens per block, must be 32        */
  int32_t kv_dtype;      /* kvmem_dtype                         */
} kvmem_geom;

/* The paged workspace ([README 'Background and main changes']: the history is
 * kept as paged KV; [README 'Core equation']: address space and execution
 * window are separate).
 *
 * k_pool, v_pool : [n_pages][Hkv][32][d] in kv_dtype.  A page holds one
 *                  32-token block of one session for all KV heads; keys are
 *                  stored BEFORE RoPE.  Tokens of a partial last block beyond
 *                  the history are never read.
 * block_table    : [n_sessions][max_blocks] int32, logical block -> page.
 *                  Entries past a session's history are never read.
 * n_tokens_host  : HOST array [n_sessions] of history lengths, each in
 *                  [0, 32 * max_blocks].
 * dev_error      : optional device int32 (may be NULL) that kernels OR
 *                  KVMEM_DEVERR_* bits into.                                 */
typedef struct {
  const void *k_pool;
  const void *v_pool;
  const int32_t *block_table;
  const int32_t *n_tokens_host;
  int32_t n_sessions;
  int32_t max_blocks;
  int32_t n_pages;
  int32_t *dev_error;
} kvmem_workspace;

/* ---------------------------------------------------------------------------
 * Mean-K index ([README 'Core equation']: each block b has an index vector
 * k_bar_b; [REVIEW 'Summary']: a position-independent Mean-K index over
 * 32-token blocks, i.e. the mean of the block's pre-RoPE keys).
 *
 * For every session s, KV head h and complete block beta < n_tokens[s] / 32:
 *   row(s, h, beta) = round( (1/32) * sum_{u<32} K[page(s,beta)][h][u][:] )
 * The sum is accumulated in fp64 and rounded once (to nearest, ties to even)
 * to kv_dtype.  Rows for beta >= n_tokens[s] / 32 are not written.  v_pool
 * is not used and may be NULL.
 *
 * index : kvmem_index_bytes() bytes in kv_dtype, TILED: the rows of each
 *         (s, h) are grouped in tiles of 64 consecutive blocks, and inside a
 *         tile the 16-byte word w (elements [E*w, E*w + E) of a row, E = 8 for
 *         bf16 and 4 for fp32) of all 64 rows is stored contiguously:
 *           element i of row(s, h, beta) is at element offset
 *             ((((s * Hkv + h) * NT + beta / 64) * (d / E) + i / E) * 64
 *               + beta % 64) * E + i % E,        NT = ceil(max_blocks / 64).
 *         (One load instruction of a 64-lane wavefront then reads one word of
 *         64 rows as a single contiguous 1 KiB access, with every lane
 *         holding its own row.)
 * ------------------------------------------------------------------------- */
size_t kvmem_index_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t max_blocks);
kvmem_status kvmem_build_index(const kvmem_geom *geom, const kvmem_workspace *ws,
                               void *index, void *stream);

/* Incremental form: writes the rows of blocks first_block_host[s] <= beta <
 * n_tokens[s] / 32 only (same values as kvmem_build_index), e.g. the blocks a
 * decode step completed.  first_block_host: HOST [n_sessions], each in
 * [0, n_tokens[s] / 32]; NULL means 0 (then this is kvmem_build_index).     */
kvmem_status kvmem_update_index(const kvmem_geom *geom, const kvmem_workspace *ws,
                                const int32_t *first_block_host, void *index, void *stream);

/* ---------------------------------------------------------------------------
 * Query-conditioned block selection ([README 'Core equation']:
 * s_b = <q, k_bar_b>/sqrt(d), selected KV within the block budget;
 * [README '2026-09-08 validation correction']: the query is RMS-normalised
 * and GQA query heads are softmaxed per head, not averaged before the
 * softmax; [README 'Local reproduction']: recent blocks share the budget).
 *
 * For session s, with N = n_tokens[s], Nb = N / 32 complete blocks,
 * Nall = ceil(N / 32) blocks, recent range [r0, Nall) with
 * r0 = max(0, Nall - n_recent), candidates beta < nc = min(Nb, r0), and
 * k_eff = min(k_select, nc):
 *   q~[t][g]   = w * q[t][g] / sqrt(mean_i q[t][g][i]^2 + eps)      (fp32)
 *   s[t][g][b] = <q~[t][g], index[h(g)][b]> / sqrt(d),  b < Nb       (fp32)
 *   p[t][g][b] = softmax over b < Nb of s[t][g][:]
 *   A[h][b]    = sum_t sum_{g in group h} p[t][g][b]
 * with index rows read from the tiled layout of kvmem_build_index.
 * The k_eff candidates with the largest A (ties: lower block index) are
 * listed in ascending order, followed by the recent blocks ascending, then
 * -1 padding:
 *   view_blocks[s][h][0 .. k_select + n_recent)
 * view_tokens_host[s] receives the view length
 *   V = 32 * k_eff + max(0, N - 32 * r0)
 * (computed on the host: it depends on the lengths only).
 *
 * q            : [n_sessions][T][Hq][d] in kv_dtype.
 * q_norm_w     : [d] fp32.
 * scores_opt   : optional [n_sessions][T][Hq][max_blocks] fp32, receives s.
 * agg_opt      : optional [n_sessions][Hkv][max_blocks] fp32, receives A.
 * scratch      : device buffer of at least kvmem_score_select_scratch_bytes().
 * Requires T >= 1, k_select >= 0, n_recent >= 0.
 * ------------------------------------------------------------------------- */
/* The view lengths kvmem_score_select will report, computed on the host
 * from the history lengths alone (the selection always fills its budget up to
 * the candidates there are), for sizing the view buffers before the first
 * selection.  For each session s < n_sessions, with N = n_tokens_host[s] and
 * r0, nc, k_eff as above:
 *   view_tokens_host[s] = 32 * k_eff + max(0, N - 32 * r0).
 * Enqueues nothing and touches no device memory.  KVMEM_E_ARG for
 * n_sessions <= 0, a NULL array, k_select < 0, n_recent < 0 or a negative
 * length.                                                                  */
kvmem_status kvmem_view_tokens(int32_t n_sessions, const int32_t *n_tokens_host, int32_t k_select,
                               int32_t n_recent, int32_t *view_tokens_host);

size_t kvmem_score_select_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions,
                                        int32_t max_blocks, int32_t T);
kvmem_status kvmem_score_select(const kvmem_geom *geom, const kvmem_workspace *ws,
                                const void *index, const void *q, int32_t T,
                                const float *q_norm_w, float eps,
                                int32_t k_select, int32_t n_recent,
                                int32_t *view_blocks, int32_t *view_tokens_host,
                                float *scores_opt, float *agg_opt,
                                void *scratch, size_t scratch_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Materialisation of the bounded execution view ([REVIEW 'Summary' and
 * 'Scope & Claims']: selected blocks are restored with position-consistent
 * re-RoPE into a bounded view; [README 'Background and main changes']: the
 * view is materialised within the native window).
 *
 * View slot j = 32*m + u (m < ceil(V/32), u < 32, j < V) holds token u of
 * block beta = view_blocks[s][h][m]:
 *   K_view[j] = round( RoPE(K[page(s,beta)][h][u], position j) )
 *   V_view[j] = V[page(s,beta)][h][u]        (bit copy)
 * RoPE rotates pairs (i, i + d/2) by angle j * theta^(-2i/d).  Its cosine and
 * sine are formed from the block angle 32*m*theta_i and the in-block angle
 * u*theta_i (each reduced modulo 2*pi and evaluated in fp64; the in-block pair
 * rounded to fp32) by the angle-addition identities in fp64, rounded to fp32
 * once; the rotation is in fp32 and the result rounded to nearest even.
 * kvmem_append and kvmem_attend_paged form view keys the same way, bit for
 * bit.
 * Slots j in [V, 32 * ceil(V/32)) are written as zeros; later slots are not
 * written.
 *
 * view_blocks      : as written by kvmem_score_select, row stride n_list.
 * view_tokens_host : HOST [n_sessions] view lengths V (<= 32 * n_list and
 *                    <= max_view).
 * k_view           : [n_sessions][Hkv][max_view][d] in kv_dtype, token-major.
 * v_view           : [n_sessions][Hkv][max_view/32][d][32] in kv_dtype: each
 *                    32-token view block is stored dimension-major, and token
 *                    u of the block sits at slot
 *                      sigma(u) = 8*((u & 15) >> 2) + 4*(u >> 4) + (u & 3).
 *                    (This is the operand order of the attention kernel's
 *                    matrix-core tiles, so kvmem_attend reads it directly.)
 * max_view must be a positive multiple of 32.
 * ------------------------------------------------------------------------- */
kvmem_status kvmem_materialize(const kvmem_geom *geom, const kvmem_workspace *ws,
                               const int32_t *view_blocks, int32_t n_list,
                               const int32_t *view_tokens_host, int32_t max_view,
                               float rope_theta, void *k_view, void *v_view, void *stream);

/* ---------------------------------------------------------------------------
 * Host-tier paging ([README 'Background and main changes']: the history is
 * kept as paged KV across GPU memory, host memory and NVMe, and the selected
 * blocks are brought into the bounded view on demand; [REVIEW 'Summary']).
 *
 * The workspace's K/V pools may be pinned host memory (hipHostMalloc, e.g.
 * torch's pinned allocator: the GPU reads it in place over the host link;
 * memory merely registered with hipHostRegister is not supported) or device
 * memory; the Mean-K index, built by kvmem_build_index from either, stays in
 * device memory, so kvmem_score_select never touches the host tier.  After a
 * selection, this call copies exactly the listed (block, KV head) tiles of
 * every session's view into a device staging pool laid out in view order:
 *   stage page s * n_list + m, KV head h  <-  K and V of head h's m-th listed
 *                                             block, view_blocks[s][h][m]
 * and writes the staged workspace's block table and list:
 *   stage_table[s][m]   = s * n_list + m   for m < ceil(V/32), else -1
 *   stage_list[s][h][m] = m                for m < ceil(V/32), else -1
 * A workspace { stage_k, stage_v, stage_table, view_tokens_host (as history
 * lengths), n_sessions, n_list (as max_blocks), n_sessions * n_list pages }
 * with stage_list as its view list then gives kvmem_materialize,
 * kvmem_materialize_attend and kvmem_attend_paged exactly the view and the
 * attention the original workspace gives with view_blocks (a view position
 * depends only on the list slot).  Tokens past V in the last block are not
 * read and are zero in the staged pool; a bad list entry or page sets the
 * KVMEM_DEVERR_* bit and is staged as a zero tile, as the gather writes it.
 * KVMEM_E_ARG (checked last, with HIP's pointer query) if a pool is not
 * readable by the GPU at its own address (e.g. pageable host memory).
 *
 * view_blocks, n_list, view_tokens_host : as for kvmem_materialize.
 * stage_k, stage_v : device, [n_sessions * n_list][Hkv][32][d] in kv_dtype.
 * stage_table      : device int32 [n_sessions][n_list].
 * stage_list       : device int32 [n_sessions][Hkv][n_list].
 * ------------------------------------------------------------------------- */
kvmem_status kvmem_stage_view(const kvmem_geom *geom, const kvmem_workspace *ws,
                              const int32_t *view_blocks, int32_t n_list,
                              const int32_t *view_tokens_host,
                              void *stage_k, void *stage_v, int32_t *stage_table,
                              int32_t *stage_list, void *stream);

/* ---------------------------------------------------------------------------
 * Decode attention over the view ([README 'Local reproduction']: attention
 * over the selected view replaces full attention).
 *
 * For session s with view length V, query token t < T and query head g:
 *   q_r       = RoPE(q~[t][g], position V + t)       (q~ as in score_select)
 *   l_j       = <q_r, K_view[h(g)][j]> / sqrt(d),  j < V
 *   out[t][g] = sum_j softmax_j(l) * V_view[h(g)][j]
 * The step's own tokens attend to the view only (no mask among them).  An
 * empty view (V = 0) gives a zero output.  Accumulation is fp32; the
 * split-K partials are merged by log-sum-exp in a fixed order, so results are
 * deterministic run to run.
 *
 * q, q_norm_w, eps : as for kvmem_score_select.
 * k_view, v_view   : as written by kvmem_materialize.
 * out              : [n_sessions][T][Hq][d] fp32.
 * scratch          : at least kvmem_attend_scratch_bytes() bytes.
 * ------------------------------------------------------------------------- */
size_t kvmem_attend_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t T,
                                  int32_t max_view);
kvmem_status kvmem_attend(const kvmem_geom *geom, int32_t n_sessions,
                          const void *q, int32_t T, const float *q_norm_w, float eps,
                          const void *k_view, const void *v_view,
                          const int32_t *view_tokens_host, int32_t max_view,
                          float rope_theta, float *out,
                          void *scratch, size_t scratch_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * kvmem_attend for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no scratch argument and calls no allocating routine; otherwise it is
 * kvmem_attend (same checks, same kernels, the same output bits).
 *
 * Its scratch is the library's own device array of
 * KVMEM_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends.  A
 * call that needs more (kvmem_attend_scratch_bytes() above the constant, e.g.
 * more than fifteen sessions of 262,144-token views at 64 query / 8 KV heads)
 * returns KVMEM_E_WORKSPACE and enqueues nothing.  The call runs on the
 * current device (stream must belong to it).  The array's device address is
 * looked up once per device, on the first call made with that device
 * current: make one call before capturing a graph.  Every call on a GPU
 * shares that GPU's array and leaves its partial results there; nothing in
 * it needs to start at zero (a call reads only partials it wrote itself), but
 * calls that overlap on one GPU (other streams, other host threads) race:
 * serialise them, e.g. on one stream.  KVMEM_E_HIP if the device or the
 * array's address cannot be obtained.
 * ------------------------------------------------------------------------- */
#define KVMEM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
kvmem_status kvmem_attend_noalloc(const kvmem_geom *geom, int32_t n_sessions,
                                  const void *q, int32_t T, const float *q_norm_w, float eps,
                                  const void *k_view, const void *v_view,
                                  const int32_t *view_tokens_host, int32_t max_view,
                                  float rope_theta, float *out, void *stream);

/* ---------------------------------------------------------------------------
 * Attention straight from the paged history ([README 'Core equation']: the
 * address space and the execution window are separate; [REVIEW 'Summary']:
 * the view is the selected blocks re-RoPE'd to contiguous positions).
 *
 * Computes exactly what kvmem_materialize followed by kvmem_attend computes
 * with the same view_blocks and view lengths, without writing the view: the
 * m-th listed block of (s, h) is read from its page, its keys rotated at view
 * positions 32m .. 32m + 31 and rounded to kv_dtype there, its values used
 * as stored; view positions at or past V are masked.  A bad list entry or
 * page sets the KVMEM_DEVERR_* bit and counts as a zero block (as the gather
 * writes it).  Worth it when a view serves few decode tokens: it reads the
 * selected K/V once per call, where the gather reads them and writes the
 * view once per step.
 *
 * view_blocks, n_list : as written by kvmem_score_select.
 * view_tokens_host    : HOST [n_sessions] view lengths V (<= 32 * n_list).
 * q, q_norm_w, eps, out, rope_theta : as for kvmem_attend (T * G <= 32 for
 *                       bf16, <= 64 for fp32; KVMEM_E_UNSUPPORTED beyond).
 * scratch             : at least kvmem_attend_paged_scratch_bytes() bytes.
 * ------------------------------------------------------------------------- */
size_t kvmem_attend_paged_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t T,
                                        int32_t n_list);
kvmem_status kvmem_attend_paged(const kvmem_geom *geom, const kvmem_workspace *ws,
                                const void *q, int32_t T, const float *q_norm_w, float eps,
                                const int32_t *view_blocks, int32_t n_list,
                                const int32_t *view_tokens_host, float rope_theta, float *out,
                                void *scratch, size_t scratch_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Gather + re-RoPE and the step's attention in one pass ([REVIEW 'Summary']:
 * the selected blocks are restored with position-consistent re-RoPE into the
 * bounded view; [README 'Local reproduction']: attention over that view).
 *
 * Writes k_view and v_view exactly as kvmem_materialize does (same bits, same
 * zeros past V), and computes into out the attention kvmem_attend computes
 * over them, reading each selected K/V block once: the attention is that of
 * kvmem_attend_paged (its keys are the view's keys, bit for bit).  The view is
 * then ready for kvmem_attend / kvmem_append over the step's later tokens.
 * Slots at or past 32 * ceil(V/32) are not written.
 *
 * Arguments as for kvmem_attend_paged, plus max_view, k_view, v_view as for
 * kvmem_materialize (V <= max_view).  scratch: at least
 * kvmem_attend_paged_scratch_bytes() bytes.
 * ------------------------------------------------------------------------- */
kvmem_status kvmem_materialize_attend(const kvmem_geom *geom, const kvmem_workspace *ws,
                                      const void *q, int32_t T, const float *q_norm_w, float eps,
                                      const int32_t *view_blocks, int32_t n_list,
                                      const int32_t *view_tokens_host, int32_t max_view,
                                      float rope_theta, void *k_view, void *v_view, float *out,
                                      void *scratch, size_t scratch_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Step-level view reuse ([REVIEW 'Scope & Claims']: recall is scheduled per
 * agent step; [REVIEW 'Strengths']: attention is stable within a step and
 * shifts across step boundaries).  The view selected and materialised at a
 * step boundary serves all of the step's decode tokens; each new token's K/V
 * is appended to both the paged history and the view, and blocks are indexed
 * as they complete (kvmem_update_index), so the next selection sees them.
 *
 * For session s with history length N = n_tokens_host[s] (BEFORE the append)
 * and view length V = view_tokens_host[s], new token t < T_new, KV head h:
 *   K[page(s, (N+t)/32)][h][(N+t) % 32] = k_new[s][t][h]       (bit copy)
 *   V[page(s, (N+t)/32)][h][(N+t) % 32] = v_new[s][t][h]       (bit copy)
 *   K_view[s][h][V+t] = round( RoPE(k_new[s][t][h], position V + t) )
 *   V_view[s][h][V+t] = v_new[s][t][h]        (at its slot, bit copy)
 * with RoPE and rounding exactly as in kvmem_materialize, so an appended
 * token equals the same token gathered into view position V + t.  View slots
 * from V + T_new to the end of that 32-token view block are zero afterwards:
 * a view block the append opens is cleared past the new end, and a block
 * already holding view tokens keeps the zeros kvmem_materialize (or an
 * earlier append) left after the view's last token.  Afterwards the
 * caller advances n_tokens_host[s] and view_tokens_host[s] by T_new; the
 * decode queries of later steps then attend to the appended tokens.
 *
 * k_pool, v_pool : the workspace's pools (must equal ws->k_pool and
 *                  ws->v_pool), written.  The block table must map the
 *                  blocks holding positions [N, N + T_new) to pages; a bad
 *                  page sets KVMEM_DEVERR_PAGE and skips that pool write.
 * k_new, v_new   : [n_sessions][T_new][Hkv][d] in kv_dtype, keys pre-RoPE.
 * k_view, v_view : as for kvmem_materialize.
 * Requires N + T_new <= 32 * max_blocks and V + T_new <= max_view for every
 * session; T_new = 0 does nothing.
 * ------------------------------------------------------------------------- */
kvmem_status kvmem_append(const kvmem_geom *geom, const kvmem_workspace *ws,
                          void *k_pool, void *v_pool,
                          const void *k_new, const void *v_new, int32_t T_new,
                          const int32_t *view_tokens_host, int32_t max_view,
                          float rope_theta, void *k_view, void *v_view, void *stream);

/* -------------------------------------------------------------------------
 * kvmem_attend_append: one decode token over a reused view in one call --
 * kvmem_attend over the current view (lengths view_tokens_host, BEFORE the
 * append), then kvmem_append of the step's new tokens, with exactly the
 * results of those two calls made in that order ([REVIEW 'Scope & Claims']:
 * the view serves every decode token of a step; [README 'Core equation']:
 * attention over the bounded view).  The append runs as extra workgroups of
 * the attention's split-merge launch, which follows the attention kernel on
 * the stream, so the appended view slots are written after every read of the
 * view and the append costs no launch of its own.
 *
 * n_sessions is ws->n_sessions.  q, T, q_norm_w, eps, k_view, v_view,
 * max_view, rope_theta, out, scratch, scratch_bytes: as for kvmem_attend
 * (scratch sized by kvmem_attend_scratch_bytes).  k_pool, v_pool, k_new,
 * v_new, T_new: as for kvmem_append.  Every check of both calls is made
 * before anything is enqueued.  As with kvmem_append, the caller then
 * advances n_tokens_host[s] and view_tokens_host[s] by T_new and indexes the
 * blocks the append completed (kvmem_update_index).
 * ------------------------------------------------------------------------- */
kvmem_status kvmem_attend_append(const kvmem_geom *geom, const kvmem_workspace *ws, const void *q, int32_t T,
                                 const float *q_norm_w, float eps, void *k_view, void *v_view,
                                 const int32_t *view_tokens_host, int32_t max_view, float rope_theta, float *out,
                                 void *k_pool, void *v_pool, const void *k_new, const void *v_new, int32_t T_new,
                                 void *scratch, size_t scratch_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Selection-quality diagnostic ([REVIEW 'Strengths']: a few top blocks carry
 * most of the attention mass, which motivates block selection; [README 'Local
 * reproduction']: selection is compared with full attention and with the
 * recent-only control at the same budget).
 *
 * Full attention over the history is attention over a full-budget view:
 * every history token j < N = n_tokens[s] with its key rotated at its own
 * position and rounded to kv_dtype, the query token t at position N + t
 * (q~ and RoPE as in kvmem_attend, the step's tokens attend to the history
 * only).  For session s, query token t and query head g:
 *   l_j         = <RoPE(q~[t][g], N + t), round(RoPE(K[j], j))> / sqrt(d)
 *   mass[t][g]  = sum over tokens j of the blocks listed in
 *                 view_blocks[s][h(g)][0 .. n_list) of softmax_j(l)
 *   lse[t][g]   = log sum_j exp(l_j)                  (natural log)
 * with the partial tail block's valid tokens included.  Listed entries must
 * ascend and be followed only by -1 padding (the layout kvmem_score_select
 * writes); entries outside [0, ceil(N/32)) are ignored.  mass is 0 for an
 * empty history or list.  Pass the selection's list for the method's mass and
 * a list of the recent blocks only for the recent-only control.
 *
 * q, q_norm_w, eps : as for kvmem_score_select (T * G <= 32 for bf16, <= 64
 *                    for fp32; KVMEM_E_UNSUPPORTED beyond).
 * mass, lse_opt    : [n_sessions][T][Hq] fp32 (lse_opt may be NULL).
 * scratch          : at least kvmem_attention_mass_scratch_bytes() bytes.
 * Reads the K pool only (v_pool may be NULL).
 * ------------------------------------------------------------------------- */
size_t kvmem_attention_mass_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t T,
                                          int32_t max_blocks);
kvmem_status kvmem_attention_mass(const kvmem_geom *geom, const kvmem_workspace *ws,
                                  const void *q, int32_t T, const float *q_norm_w, float eps,
                                  const int32_t *view_blocks, int32_t n_list, float rope_theta,
                                  float *mass, float *lse_opt,
                                  void *scratch, size_t scratch_bytes, void *stream);

/* Static text for a status code. */
const char *kvmem_status_string(kvmem_status status);

/* Library version as 10000*major + 100*minor + patch. */
int32_t kvmem_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVMEM_H_ */
