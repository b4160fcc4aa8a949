// Host-side launchers of the KVMem kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvmem_device.h"

namespace kvmem {

// --- Mean-K index -----------------------------------------------------------
hipError_t launch_build_index(int bf16, const void *k_pool, const int32_t *table, void *index,
                              int32_t *dev_err, const SessI32 &n_blocks, int s0, int n_sess,
                              int Hkv, int max_blocks, int n_pages, hipStream_t st);

// --- scoring ------------------------------------------------------------------
constexpr int kScoreChunk = 128;     // index rows per scoring work item
constexpr int kAggChunk = 256;       // blocks per aggregation workgroup (one per thread)

struct ScoreGeom {
  int Tq, Hq, Hkv, G, max_blocks, n_chunks;
};

hipError_t launch_score_gemv(int bf16, const void *index, const void *q, const float *qw, float eps,
                             float *scores, float2 *part, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, hipStream_t st);

hipError_t launch_aggregate(const float *scores, const float2 *part, float *A, const SessI32 &n_blocks,
                            int s0, int n_sess, const ScoreGeom &g, hipStream_t st);

// --- selection ------------------------------------------------------------------
struct TopkMeta {
  SessI32 n_cand, k_eff, r_start, n_all;
};
hipError_t launch_topk(const float *A, int32_t *view_blocks, const TopkMeta &meta, int s0, int n_sess,
                       int Hkv, int max_blocks, int n_list, hipStream_t st);

// --- materialise ------------------------------------------------------------------
hipError_t launch_materialize(int bf16, const void *k_pool, const void *v_pool, const int32_t *table,
                              const int32_t *view_blocks, void *k_view, void *v_view, int32_t *dev_err,
                              const SessI32 &view_tok, const SessI32 &n_all, int s0, int n_sess,
                              int Hkv, int max_blocks, int n_pages, int n_list, int max_view,
                              double theta, hipStream_t st);

// --- attend ---------------------------------------------------------------------
struct AttendGeom {
  int Tq, Hq, Hkv, G, rows, max_view, max_splits, tpw;
};
int attend_tokens_per_wave(int n_sessions, int Hkv, int max_view);
int attend_max_splits(int max_view, int tpw);

hipError_t launch_attend(int bf16, const void *q, const float *qw, float eps, const void *k_view,
                         const void *v_view, float *part_o, float2 *part_ml, uint4 *qop, float *out,
                         const SessI32 &view_tok, int s0, int n_sess, const AttendGeom &g, double theta,
                         hipStream_t st);

}  // namespace kvmem
