// Host-side launchers of the KVMem kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvmem_device.h"

namespace kvmem {

// --- Mean-K index -----------------------------------------------------------
// The index is stored in tiles of kIdxTile consecutive blocks of one (session,
// KV head).  Inside a tile, 16-byte word w (elements [w*E, w*E + E) of a row,
// E = 16 / sizeof(element)) of all kIdxTile rows is contiguous:
//   element (row r, dim i) of a tile sits at ((i / E) * kIdxTile + r) * E + i % E.
// A tile is kIdxTile * kD elements; (session s, head h) owns n_tiles tiles,
// n_tiles = ceil(max_blocks / kIdxTile).
constexpr int kIdxTile = 64;
__host__ __device__ constexpr int idx_tiles(int max_blocks) { return (max_blocks + kIdxTile - 1) / kIdxTile; }

// Rows of blocks [first_block, n_blocks) of each session.
hipError_t launch_build_index(int bf16, const void *k_pool, const int32_t *table, void *index,
                              int32_t *dev_err, const SessI32 &first_block, const SessI32 &n_blocks, int s0,
                              int n_sess, int Hkv, int max_blocks, int n_pages, hipStream_t st);

// --- scoring ------------------------------------------------------------------
constexpr int kAggChunk = 1024;      // blocks per aggregation workgroup (one per thread)

// Selection histogram per (session, KV head): the candidates' A counted by
// the top digit of their fp32 bits (A >= 0, so bits 30..20: the exponent and
// three significand bits).  Top-k starts its radix select from these counts.
constexpr int kSelBins = 2048;
constexpr int kSelShift = 20;

struct ScoreGeom {
  int Tq, Hq, Hkv, G, max_blocks;
  int n_tiles;       // index tiles per (session, head)
  int slot_stride;   // softmax-statistics slots per query row (n_tiles + 1)
};

// How one scoring launch split its work: items are (session, row group of
// rpg query rows, KV head, index tile), tile fastest, and wavefront w owns
// items [w * per, (w + 1) * per).  The softmax statistics of a (session, row
// group, head) key are written by every wavefront whose range meets the key,
// one slot each, in wavefront order.
struct ScoreSplit {
  int n_sess, rpg, n_rg, ntl, per;
};

// Work item = (session, row group, KV head, index tile), tile fastest.  The
// key (session, row group, head) = item / ntl = (sl * n_rg + rg) * Hkv + h.
struct ScoreItem {
  int sl, h, r0, t, nb, key;
};
__device__ __forceinline__ ScoreItem decode_score_item(int item, const ScoreSplit &sp, int Hkv, const SessI32 &n_blocks) {
  ScoreItem it;
  it.t = item % sp.ntl;
  it.key = item / sp.ntl;
  it.h = it.key % Hkv;
  const int y = it.key / Hkv;
  it.r0 = (y % sp.n_rg) * sp.rpg;
  it.sl = y / sp.n_rg;
  it.nb = n_blocks.v[it.sl];
  return it;
}
// First softmax-statistics slot of a key and the number of slots it has.
__host__ __device__ __forceinline__ int score_slot0(int key, const ScoreSplit &sp) { return (key * sp.ntl) / sp.per; }
__host__ __device__ __forceinline__ int score_n_slots(int key, const ScoreSplit &sp) {
  return ((key + 1) * sp.ntl - 1) / sp.per - score_slot0(key, sp) + 1;
}

// Both scorers below also clear zero[0 .. n_zero) (the selection histograms
// of the launch's sessions, which the aggregation kernel then fills).
hipError_t launch_score_gemv(int bf16, const void *index, const void *q, const float *qw, float eps, float *scores,
                             float2 *part, uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, ScoreSplit *split, hipStream_t st);

// Matrix-core scorers for bf16 steps: at most kGemvMaxRows rows per KV head
// (one wavefront per index tile), and more (row groups of 32).
constexpr int kGemvMaxRows = 8;
hipError_t launch_score_r8(const void *index, const void *q, const float *qw, float eps, float *scores, float2 *part,
                          uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess, const ScoreGeom &g,
                          ScoreSplit *split, hipStream_t st);
hipError_t launch_score_mfma(const void *index, const void *q, const float *qw, float eps, float *scores,
                             float2 *part, uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, ScoreSplit *split, hipStream_t st);

// Long query chunks (bf16, more than kMfmaMaxRows rows per KV head): two passes
// over the index on the matrix cores without storing the score matrix; writes
// A directly (no aggregation kernel).  Scratch per LongScratch.
constexpr int kMfmaMaxRows = 32;
struct LongScratch {
  size_t qf_bytes, part_bytes, lse_bytes;
};
LongScratch long_scratch_layout(int S, int Hkv, int T, int G, int max_blocks);
hipError_t launch_score_long(const void *index, const void *q, const float *qw, float eps, uint4 *qf, float2 *part,
                             float *lse, float *A, float *scores_opt, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, hipStream_t st);

// --- selection ------------------------------------------------------------------
struct TopkMeta {
  SessI32 n_cand, k_eff, r_start, n_all;
};

// A for every complete block of the scored sessions, and the candidates
// (blocks below n_cand) counted into hist[(s * Hkv + h) * kSelBins + digit]
// (cleared by the scorer of the same call).  Per chunk c of kAggChunk blocks
// of a (session, KV head), c < sel_chunks(max_blocks), the chunk's candidate
// keys (A's bits without the sign bit) are also written grouped by digit,
// highest digit first, to skey[((s * Hkv + h) * n_chunks + c) * kAggChunk
// ...], and the number of its candidates whose digit is >= b to
// sincl[((s * Hkv + h) * n_chunks + c) * kSelBins + b].
hipError_t launch_aggregate(const float *scores, const float2 *part, float *A, uint32_t *hist, uint32_t *skey,
                            uint16_t *sincl, const SessI32 &n_blocks, const SessI32 &n_cand, int s0, int n_sess,
                            const ScoreGeom &g, const ScoreSplit &split, hipStream_t st);
__host__ __device__ constexpr int sel_chunks(int max_blocks) { return (max_blocks + kAggChunk - 1) / kAggChunk; }

// Selection from A; hist, skey, sincl: the aggregation's selection histograms
// and grouped keys, or all null.
hipError_t launch_topk(const float *A, const uint32_t *hist, const uint32_t *skey, const uint16_t *sincl,
                       int32_t *view_blocks, const TopkMeta &meta, int s0, int n_sess, int Hkv, int max_blocks,
                       int n_list, hipStream_t st);

// --- materialise ------------------------------------------------------------------
hipError_t launch_materialize(int bf16, const void *k_pool, const void *v_pool, const int32_t *table,
                              const int32_t *view_blocks, void *k_view, void *v_view, int32_t *dev_err,
                              const SessI32 &view_tok, const SessI32 &n_all, int s0, int n_sess,
                              int Hkv, int max_blocks, int n_pages, int n_list, int max_view,
                              double theta, hipStream_t st);

// --- host-tier staging ------------------------------------------------------------
// The listed (block, KV head) tiles of every session's view, read from the
// pools (pinned host memory or HBM) into staged page s * n_list + m, with the
// staged block table and identity list (see k_stage.hip).
hipError_t launch_stage(int bf16, const void *k_pool, const void *v_pool, const int32_t *table,
                        const int32_t *view_blocks, void *stage_k, void *stage_v, int32_t *stage_table,
                        int32_t *stage_list, int32_t *dev_err, const SessI32 &view_tok, const SessI32 &n_all,
                        int s0, int n_sess, int Hkv, int max_blocks, int n_pages, int n_list, hipStream_t st);

// --- append ---------------------------------------------------------------------
// Writes T_new new tokens per session into the pools at history positions
// n_tok + t and into the view at positions view_tok + t (K re-RoPE'd there).
hipError_t launch_append(int bf16, void *k_pool, void *v_pool, const int32_t *table, const void *k_new,
                         const void *v_new, int T_new, void *k_view, void *v_view, int32_t *dev_err,
                         const SessI32 &n_tok, const SessI32 &view_tok, int s0, int n_sess, int Hkv, int max_blocks,
                         int n_pages, int max_view, double theta, hipStream_t st);

// --- attend ---------------------------------------------------------------------
struct AttendGeom {
  int Tq, Hq, Hkv, G, rows, max_view, max_splits, tpw;
};
int attend_tokens_per_wave(int n_sessions, int Hkv, int max_view, int rows);
int attend_max_splits(int max_view, int tpw);

// New tokens appended by the merge launch of an attention (kvmem_attend_append):
// T_new extra workgroups per session, each running the append of one token
// (the k_append routine) while the other workgroups merge the splits.  The
// merge runs after the attention kernel on the same stream, so the tokens'
// view slots are written after every read of the view.  T_new = 0: none.
struct AppendArgs {
  void *kpool, *vpool;
  const int32_t *table;
  const void *knew, *vnew;
  void *kview, *vview;
  int32_t *dev_err;
  SessI32 n_tok;                  // history lengths before the append
  int T_new, Hkv, max_blocks, n_pages, max_view, bf16;
  double theta;
};

hipError_t launch_attend(int bf16, const void *q, const float *qw, float eps, const void *k_view,
                         const void *v_view, float *part_o, float2 *part_ml, float *out,
                         const SessI32 &view_tok, int s0, int n_sess, const AttendGeom &g, double theta,
                         hipStream_t st, const AppendArgs *ap = nullptr);

// Merge of split partials (layout of the view attention) into out; with ap,
// also the append of ap->T_new tokens per session (view lengths view_tok).
hipError_t launch_attend_combine(const float *part_o, const float2 *part_ml, float *out, const SessI32 &view_tok,
                                 int s0, int n_sess, const AttendGeom &g, hipStream_t st,
                                 const AppendArgs *ap = nullptr);

// --- attention straight from the pages ------------------------------------------
// query rows per KV head of the fp32 kernels (attention from the pages, the
// one-pass call and the diagnostic on fp32 workspaces)
constexpr int kF32PagedMaxRows = 64;
struct PagedGeom {
  int Tq, Hq, Hkv, G, rows, max_blocks, n_pages, n_list;
  int bps;          // list blocks per split
  int max_splits;   // split slots per (session, head) in the partials
};
int paged_blocks_per_split(int n_sessions, int Hkv, int n_list);
hipError_t launch_attend_paged(int bf16, const void *q, const float *qw, float eps, const void *k_pool,
                               const void *v_pool, const int32_t *table, const int32_t *view_blocks, float *part_o,
                               float2 *part_ml, float *out, int32_t *dev_err, const SessI32 &view_tok,
                               const SessI32 &n_all, int s0, int n_sess, const PagedGeom &g, double theta,
                               void *k_view, void *v_view, int max_view, hipStream_t st);

// --- selection-quality diagnostic ------------------------------------------------
struct MassGeom {
  int Tq, Hq, Hkv, G, rows, max_blocks, n_pages, n_list;
  int chunk;      // history blocks per workgroup
  int n_chunks;   // chunk slots per (session, head) in the partials
};
int mass_chunk(int n_sessions, int Hkv, int max_blocks);
hipError_t launch_mass(int bf16, const void *q, const float *qw, float eps, const void *k_pool, const int32_t *table,
                       const int32_t *view_blocks, float4 *part, float *mass, float *lse, int32_t *dev_err,
                       const SessI32 &n_tok, int s0, int n_sess, const MassGeom &g, double theta, hipStream_t st);

}  // namespace kvmem
