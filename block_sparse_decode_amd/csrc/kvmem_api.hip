// Host side of the C ABI declared in include/kvmem.h: argument validation,
// scratch layout, launch geometry and the per-session launch loop.  No call
// allocates, synchronises or keeps state; every invalid argument is rejected
// before anything is enqueued.
#include <math.h>
#include <string.h>

#include <atomic>

#include "../../include/kvmem.h"
#include "kvmem_internal.h"

using namespace kvmem;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

kvmem_status check_geom(const kvmem_geom *g) {
  if (!g) return KVMEM_E_ARG;
  if (g->n_q_heads <= 0 || g->n_kv_heads <= 0 || g->n_q_heads % g->n_kv_heads != 0) return KVMEM_E_ARG;
  if (g->head_dim != kD || g->block_tokens != kBT) return KVMEM_E_UNSUPPORTED;
  if (g->kv_dtype != KVMEM_F32 && g->kv_dtype != KVMEM_BF16) return KVMEM_E_UNSUPPORTED;
  return KVMEM_OK;
}

kvmem_status check_ws(const kvmem_workspace *w, bool need_v) {
  if (!w) return KVMEM_E_ARG;
  if (w->n_sessions <= 0 || w->max_blocks <= 0 || w->n_pages <= 0) return KVMEM_E_ARG;
  if (!w->k_pool || !w->block_table || !w->n_tokens_host) return KVMEM_E_ARG;
  if (need_v && !w->v_pool) return KVMEM_E_ARG;
  const long cap = (long)w->max_blocks * kBT;
  for (int s = 0; s < w->n_sessions; ++s)
    if (w->n_tokens_host[s] < 0 || (long)w->n_tokens_host[s] > cap) return KVMEM_E_ARG;
  return KVMEM_OK;
}

kvmem_status hip_status(hipError_t e) { return e == hipSuccess ? KVMEM_OK : KVMEM_E_HIP; }

// True when the GPU can read p at address p: device memory, or pinned host
// memory mapped into the device's address space (hipHostMalloc).  A pointer
// HIP does not know (pageable memory) is refused; its lookup error is cleared
// so that it does not surface at a later launch check.
bool gpu_addressable(const void *p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.devicePointer == p;
}

struct Split {
  int n_cand, r_start, n_all, n_full;
};
Split recent_split(int n_tok, int n_recent) {
  Split r;
  r.n_full = n_tok / kBT;
  r.n_all = (n_tok + kBT - 1) / kBT;
  r.r_start = r.n_all - n_recent > 0 ? r.n_all - n_recent : 0;
  r.n_cand = r.n_full < r.r_start ? r.n_full : r.r_start;
  return r;
}

// View tokens of a history of n_tok tokens: k_eff selected whole blocks plus
// the recent range (its partial tail block counts its valid tokens only).
int view_length(int n_tok, int k_select, int n_recent) {
  const Split sp = recent_split(n_tok, n_recent);
  const int k_eff = k_select < sp.n_cand ? k_select : sp.n_cand;
  const long tail = (long)n_tok - (long)kBT * sp.r_start;
  return kBT * k_eff + (int)(tail > 0 ? tail : 0);
}

// Steps with many query rows per KV head (bf16) take the two-pass long-chunk
// scorer, which never stores the score matrix.
bool long_chunk(const kvmem_geom *g, int T) {
  return g->kv_dtype == KVMEM_BF16 && (long)T * (g->n_q_heads / g->n_kv_heads) > kMfmaMaxRows;
}

// score_select scratch.  Short steps: per-head scores, per-(row, slot)
// softmax statistics, A.  Long chunks: query operands, per-(row, block group)
// statistics, per-row log-sum-exp, A.
struct ScoreScratch {
  size_t scores, part, agg, qf, lse, hist, skey, sincl, total;
};
ScoreScratch score_scratch(const kvmem_geom *g, int S, int max_blocks, int T) {
  ScoreScratch r;
  const size_t a_bytes = align_up((size_t)S * g->n_kv_heads * max_blocks * sizeof(float));
  if (long_chunk(g, T)) {
    const LongScratch L = long_scratch_layout(S, g->n_kv_heads, T, g->n_q_heads / g->n_kv_heads, max_blocks);
    r.scores = 0;
    r.part = 0;
    r.qf = align_up(L.part_bytes);
    r.lse = r.qf + align_up(L.qf_bytes);
    r.agg = r.lse + align_up(L.lse_bytes);
    r.hist = r.skey = r.sincl = 0;
    r.total = r.agg + a_bytes;
    return r;
  }
  const size_t rows = (size_t)S * T * g->n_q_heads;
  const size_t n_slots = (size_t)idx_tiles(max_blocks) + 1;   // softmax-statistics slots per row
  r.scores = 0;
  r.part = align_up(rows * max_blocks * sizeof(float));
  r.agg = r.part + align_up(rows * n_slots * sizeof(float2));
  r.qf = r.lse = r.agg;
  r.hist = r.agg + a_bytes;
  // each aggregation chunk's keys grouped by top digit, and its counts per digit
  const size_t chunks = (size_t)S * g->n_kv_heads * sel_chunks(max_blocks);
  r.skey = r.hist + align_up((size_t)S * g->n_kv_heads * kSelBins * sizeof(uint32_t));
  r.sincl = r.skey + align_up(chunks * kAggChunk * sizeof(uint32_t));
  r.total = r.sincl + align_up(chunks * kSelBins * sizeof(uint16_t));
  return r;
}

struct AttendScratch {
  size_t part_o, part_ml, total;
  int tpw, max_splits;
};
AttendScratch attend_scratch(const kvmem_geom *g, int S, int T, int max_view) {
  AttendScratch r;
  r.tpw = attend_tokens_per_wave(S, g->n_kv_heads, max_view, T * (g->n_q_heads / g->n_kv_heads));
  r.max_splits = attend_max_splits(max_view, r.tpw);
  const size_t rows = (size_t)T * (g->n_q_heads / g->n_kv_heads);
  const size_t n = (size_t)S * g->n_kv_heads * r.max_splits * rows;
  r.part_o = 0;
  r.part_ml = align_up(n * kD * sizeof(float));
  r.total = r.part_ml + align_up(n * sizeof(float2));
  return r;
}

// Scratch of kvmem_attend_noalloc: the library's own device array, one per
// GPU (each device holds its own copy of a __device__ variable), kept until
// the process ends.  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, looked up once per device on
// the first call made with that device current, and cached here.
constexpr size_t kNoAllocBytes = KVMEM_NOALLOC_SCRATCH_BYTES;
constexpr int kNoAllocDevices = 64;
std::atomic<void *> g_noalloc_ptr[kNoAllocDevices];

}  // namespace

static __device__ __align__(256) unsigned char kvmem_noalloc_scratch[kNoAllocBytes];

// Device address of the current device's copy of kvmem_noalloc_scratch.
static kvmem_status noalloc_scratch(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocDevices) return KVMEM_E_HIP;
  void *p = g_noalloc_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(kvmem_noalloc_scratch)) != hipSuccess || p == nullptr) return KVMEM_E_HIP;
    g_noalloc_ptr[dev].store(p, std::memory_order_release);   // the same address if two threads race here
  }
  *ptr = p;
  return KVMEM_OK;
}

extern "C" {

const char *kvmem_status_string(kvmem_status st) {
  switch (st) {
    case KVMEM_OK: return "ok";
    case KVMEM_E_ARG: return "invalid argument";
    case KVMEM_E_UNSUPPORTED: return "unsupported geometry or dtype";
    case KVMEM_E_WORKSPACE: return "scratch buffer too small";
    case KVMEM_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t kvmem_version(void) { return 300; }

kvmem_status kvmem_view_tokens(int32_t n_sessions, const int32_t *n_tokens_host, int32_t k_select,
                               int32_t n_recent, int32_t *view_tokens_host) {
  if (n_sessions <= 0 || !n_tokens_host || !view_tokens_host || k_select < 0 || n_recent < 0) return KVMEM_E_ARG;
  for (int s = 0; s < n_sessions; ++s)
    if (n_tokens_host[s] < 0) return KVMEM_E_ARG;
  for (int s = 0; s < n_sessions; ++s) view_tokens_host[s] = view_length(n_tokens_host[s], k_select, n_recent);
  return KVMEM_OK;
}

size_t kvmem_index_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t max_blocks) {
  if (check_geom(geom) != KVMEM_OK || n_sessions <= 0 || max_blocks <= 0) return 0;
  const size_t elem = geom->kv_dtype == KVMEM_BF16 ? 2 : 4;
  return (size_t)n_sessions * geom->n_kv_heads * idx_tiles(max_blocks) * kIdxTile * kD * elem;
}

kvmem_status kvmem_update_index(const kvmem_geom *geom, const kvmem_workspace *ws, const int32_t *first_block_host,
                                void *index, void *stream) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if ((st = check_ws(ws, false)) != KVMEM_OK) return st;
  if (!index) return KVMEM_E_ARG;
  if (first_block_host)
    for (int s = 0; s < ws->n_sessions; ++s)
      if (first_block_host[s] < 0 || first_block_host[s] > ws->n_tokens_host[s] / kBT) return KVMEM_E_ARG;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  for (int s0 = 0; s0 < ws->n_sessions; s0 += kMaxSess) {
    const int n = ws->n_sessions - s0 < kMaxSess ? ws->n_sessions - s0 : kMaxSess;
    SessI32 nb, first;
    memset(&nb, 0, sizeof(nb));
    memset(&first, 0, sizeof(first));
    for (int i = 0; i < n; ++i) {
      nb.v[i] = ws->n_tokens_host[s0 + i] / kBT;
      first.v[i] = first_block_host ? first_block_host[s0 + i] : 0;
    }
    st = hip_status(launch_build_index(bf16, ws->k_pool, ws->block_table, index, ws->dev_error, first, nb, s0, n,
                                       geom->n_kv_heads, ws->max_blocks, ws->n_pages, (hipStream_t)stream));
    if (st != KVMEM_OK) return st;
  }
  return KVMEM_OK;
}

kvmem_status kvmem_build_index(const kvmem_geom *geom, const kvmem_workspace *ws, void *index, void *stream) {
  return kvmem_update_index(geom, ws, nullptr, index, stream);
}

kvmem_status kvmem_append(const kvmem_geom *geom, const kvmem_workspace *ws, void *k_pool, void *v_pool,
                          const void *k_new, const void *v_new, int32_t T_new, const int32_t *view_tokens_host,
                          int32_t max_view, float rope_theta, void *k_view, void *v_view, void *stream) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if ((st = check_ws(ws, true)) != KVMEM_OK) return st;
  // the pools are the workspace's own, named writable here
  if (!k_pool || !v_pool || k_pool != ws->k_pool || v_pool != ws->v_pool) return KVMEM_E_ARG;
  if (!k_new || !v_new || !view_tokens_host || !k_view || !v_view || T_new < 0) return KVMEM_E_ARG;
  if (max_view <= 0 || max_view % kBT != 0 || !(rope_theta > 1.0f) || !isfinite(rope_theta)) return KVMEM_E_ARG;
  for (int s = 0; s < ws->n_sessions; ++s) {
    if ((long)ws->n_tokens_host[s] + T_new > (long)ws->max_blocks * kBT) return KVMEM_E_ARG;
    if (view_tokens_host[s] < 0 || (long)view_tokens_host[s] + T_new > max_view) return KVMEM_E_ARG;
  }
  if (T_new == 0) return KVMEM_OK;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  for (int s0 = 0; s0 < ws->n_sessions; s0 += kMaxSess) {
    const int n = ws->n_sessions - s0 < kMaxSess ? ws->n_sessions - s0 : kMaxSess;
    SessI32 nt, vt;
    memset(&nt, 0, sizeof(nt));
    memset(&vt, 0, sizeof(vt));
    for (int i = 0; i < n; ++i) {
      nt.v[i] = ws->n_tokens_host[s0 + i];
      vt.v[i] = view_tokens_host[s0 + i];
    }
    st = hip_status(launch_append(bf16, k_pool, v_pool, ws->block_table, k_new, v_new, T_new, k_view, v_view,
                                  ws->dev_error, nt, vt, s0, n, geom->n_kv_heads, ws->max_blocks, ws->n_pages,
                                  max_view, (double)rope_theta, (hipStream_t)stream));
    if (st != KVMEM_OK) return st;
  }
  return KVMEM_OK;
}

size_t kvmem_score_select_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t max_blocks, int32_t T) {
  if (check_geom(geom) != KVMEM_OK || n_sessions <= 0 || max_blocks <= 0 || T <= 0) return 0;
  return score_scratch(geom, n_sessions, max_blocks, T).total;
}

kvmem_status kvmem_score_select(const kvmem_geom *geom, const kvmem_workspace *ws, const void *index,
                                const void *q, int32_t T, const float *q_norm_w, float eps, int32_t k_select,
                                int32_t n_recent, int32_t *view_blocks, int32_t *view_tokens_host,
                                float *scores_opt, float *agg_opt, void *scratch, size_t scratch_bytes,
                                void *stream) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if ((st = check_ws(ws, false)) != KVMEM_OK) return st;
  if (!index || !q || !q_norm_w || !view_tokens_host || T <= 0 || k_select < 0 || n_recent < 0) return KVMEM_E_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return KVMEM_E_ARG;
  const long n_list_l = (long)k_select + n_recent;
  if (n_list_l > (1L << 30)) return KVMEM_E_ARG;
  const int n_list = (int)n_list_l;
  if (n_list > 0 && !view_blocks) return KVMEM_E_ARG;
  const int S = ws->n_sessions;
  // 32-bit indexing of the query rows and of the scoring work items
  const long q_rows = (long)S * T * geom->n_q_heads;
  const long n_rg = ((long)T * (geom->n_q_heads / geom->n_kv_heads) + 7) / 8;
  if (q_rows * kD >= (1L << 31) || (long)S * geom->n_kv_heads * n_rg * idx_tiles(ws->max_blocks) >= (1L << 31))
    return KVMEM_E_UNSUPPORTED;
  const ScoreScratch sc = score_scratch(geom, S, ws->max_blocks, T);
  if (!scratch || scratch_bytes < sc.total) return KVMEM_E_WORKSPACE;

  for (int s = 0; s < S; ++s) view_tokens_host[s] = view_length(ws->n_tokens_host[s], k_select, n_recent);

  char *base = (char *)scratch;
  float *scores = scores_opt ? scores_opt : (float *)(base + sc.scores);
  float2 *part = (float2 *)(base + sc.part);
  float *A = agg_opt ? agg_opt : (float *)(base + sc.agg);
  ScoreGeom g;
  g.Tq = T;
  g.Hq = geom->n_q_heads;
  g.Hkv = geom->n_kv_heads;
  g.G = g.Hq / g.Hkv;
  g.max_blocks = ws->max_blocks;
  g.n_tiles = idx_tiles(ws->max_blocks);
  g.slot_stride = g.n_tiles + 1;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  const hipStream_t hs = (hipStream_t)stream;

  for (int s0 = 0; s0 < S; s0 += kMaxSess) {
    const int n = S - s0 < kMaxSess ? S - s0 : kMaxSess;
    SessI32 nb;
    TopkMeta tm;
    memset(&nb, 0, sizeof(nb));
    memset(&tm, 0, sizeof(tm));
    for (int i = 0; i < n; ++i) {
      const Split sp = recent_split(ws->n_tokens_host[s0 + i], n_recent);
      nb.v[i] = sp.n_full;
      tm.n_cand.v[i] = sp.n_cand;
      tm.k_eff.v[i] = k_select < sp.n_cand ? k_select : sp.n_cand;
      tm.r_start.v[i] = sp.r_start;
      tm.n_all.v[i] = sp.n_all;
    }
    int max_nb = 0;
    for (int i = 0; i < n; ++i) max_nb = nb.v[i] > max_nb ? nb.v[i] : max_nb;
    if (long_chunk(geom, T)) {
      if ((st = hip_status(launch_score_long(index, q, q_norm_w, eps, (uint4 *)(base + sc.qf), part,
                                             (float *)(base + sc.lse), A, scores_opt, nb, s0, n, g, hs))) != KVMEM_OK)
        return st;
      if (n_list > 0 &&
          (st = hip_status(launch_topk(A, nullptr, nullptr, nullptr, view_blocks, tm, s0, n, g.Hkv, ws->max_blocks,
                                       n_list, hs))) != KVMEM_OK)
        return st;
    } else if (max_nb == 0) {
      // nothing to score: the lists hold the recent (partial) blocks only
      if (n_list > 0 &&
          (st = hip_status(launch_topk(A, nullptr, nullptr, nullptr, view_blocks, tm, s0, n, g.Hkv, ws->max_blocks,
                                       n_list, hs))) != KVMEM_OK)
        return st;
    } else {
      // the scorer clears this launch's selection histograms, the aggregation
      // kernel fills them and top-k starts from them
      uint32_t *hist = (uint32_t *)(base + sc.hist);
      uint32_t *zero = hist + (size_t)s0 * g.Hkv * kSelBins;
      const int n_zero = n * g.Hkv * kSelBins;
      ScoreSplit split;
      // bf16: matrix cores (one tile per wavefront up to 8 rows, row groups of
      // 32 above); fp32: the vector-ALU GEMV
      const hipError_t e =
          !bf16 ? launch_score_gemv(bf16, index, q, q_norm_w, eps, scores, part, zero, n_zero, nb, s0, n, g, &split, hs)
          : T * g.G > kGemvMaxRows
              ? launch_score_mfma(index, q, q_norm_w, eps, scores, part, zero, n_zero, nb, s0, n, g, &split, hs)
              : launch_score_r8(index, q, q_norm_w, eps, scores, part, zero, n_zero, nb, s0, n, g, &split, hs);
      if ((st = hip_status(e)) != KVMEM_OK) return st;
      uint32_t *skey = (uint32_t *)(base + sc.skey);
      uint16_t *sincl = (uint16_t *)(base + sc.sincl);
      if ((st = hip_status(launch_aggregate(scores, part, A, hist, skey, sincl, nb, tm.n_cand, s0, n, g, split, hs))) !=
          KVMEM_OK)
        return st;
      if (n_list > 0 && (st = hip_status(launch_topk(A, hist, skey, sincl, view_blocks, tm, s0, n, g.Hkv,
                                                     ws->max_blocks, n_list, hs))) != KVMEM_OK)
        return st;
    }
  }
  return KVMEM_OK;
}

struct PagedScratch {
  size_t part_o, part_ml, total;
  int bps, max_splits;
};
PagedScratch paged_scratch(const kvmem_geom *g, int S, int T, int n_list) {
  PagedScratch r;
  r.bps = paged_blocks_per_split(S, g->n_kv_heads, n_list);
  r.max_splits = (n_list + r.bps - 1) / r.bps;
  const size_t rows = (size_t)T * (g->n_q_heads / g->n_kv_heads);
  const size_t n = (size_t)S * g->n_kv_heads * r.max_splits * rows;
  r.part_o = 0;
  r.part_ml = align_up(n * kD * sizeof(float));
  r.total = r.part_ml + align_up(n * sizeof(float2));
  return r;
}

size_t kvmem_attend_paged_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t T, int32_t n_list) {
  if (check_geom(geom) != KVMEM_OK || n_sessions <= 0 || T <= 0 || n_list <= 0) return 0;
  return paged_scratch(geom, n_sessions, T, n_list).total;
}

// Attention from the pages; with k_view / v_view also the view's K and V
// (max_view is then the view's capacity).
static kvmem_status paged_attend(const kvmem_geom *geom, const kvmem_workspace *ws, const void *q, int32_t T,
                                 const float *q_norm_w, float eps, const int32_t *view_blocks, int32_t n_list,
                                 const int32_t *view_tokens_host, float rope_theta, float *out, void *scratch,
                                 size_t scratch_bytes, void *stream, void *k_view, void *v_view, int32_t max_view) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if ((st = check_ws(ws, true)) != KVMEM_OK) return st;
  if (!q || !q_norm_w || !out || !view_tokens_host || T <= 0 || n_list < 0 || (n_list > 0 && !view_blocks))
    return KVMEM_E_ARG;
  if (!(eps >= 0.f) || !isfinite(eps) || !(rope_theta > 1.0f) || !isfinite(rope_theta)) return KVMEM_E_ARG;
  const bool wv = k_view != nullptr || v_view != nullptr;
  if (wv && (!k_view || !v_view || max_view <= 0 || max_view % kBT != 0)) return KVMEM_E_ARG;
  const int G = geom->n_q_heads / geom->n_kv_heads;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  if ((long)T * G > (bf16 ? kMfmaMaxRows : kF32PagedMaxRows)) return KVMEM_E_UNSUPPORTED;
  const int S = ws->n_sessions;
  for (int s = 0; s < S; ++s) {
    const int V = view_tokens_host[s];
    if (V < 0 || (long)V > (long)kBT * n_list || (wv && V > max_view)) return KVMEM_E_ARG;
  }
  if ((long)S * geom->n_kv_heads * n_list >= (1L << 31)) return KVMEM_E_UNSUPPORTED;
  const PagedScratch sc = paged_scratch(geom, S, T, n_list > 0 ? n_list : 1);
  if (!scratch || scratch_bytes < sc.total) return KVMEM_E_WORKSPACE;
  PagedGeom g;
  g.Tq = T;
  g.Hq = geom->n_q_heads;
  g.Hkv = geom->n_kv_heads;
  g.G = G;
  g.rows = T * G;
  g.max_blocks = ws->max_blocks;
  g.n_pages = ws->n_pages;
  g.n_list = n_list;
  g.bps = sc.bps;
  g.max_splits = sc.max_splits;
  char *base = (char *)scratch;
  for (int s0 = 0; s0 < S; s0 += kMaxSess) {
    const int n = S - s0 < kMaxSess ? S - s0 : kMaxSess;
    SessI32 vt, na;
    memset(&vt, 0, sizeof(vt));
    memset(&na, 0, sizeof(na));
    for (int i = 0; i < n; ++i) {
      vt.v[i] = view_tokens_host[s0 + i];
      na.v[i] = (ws->n_tokens_host[s0 + i] + kBT - 1) / kBT;
    }
    st = hip_status(launch_attend_paged(bf16, q, q_norm_w, eps, ws->k_pool, ws->v_pool, ws->block_table, view_blocks,
                                        (float *)(base + sc.part_o), (float2 *)(base + sc.part_ml), out,
                                        ws->dev_error, vt, na, s0, n, g, (double)rope_theta, wv ? k_view : nullptr,
                                        wv ? v_view : nullptr, wv ? max_view : 0, (hipStream_t)stream));
    if (st != KVMEM_OK) return st;
  }
  return KVMEM_OK;
}

kvmem_status kvmem_attend_paged(const kvmem_geom *geom, const kvmem_workspace *ws, const void *q, int32_t T,
                                const float *q_norm_w, float eps, const int32_t *view_blocks, int32_t n_list,
                                const int32_t *view_tokens_host, float rope_theta, float *out, void *scratch,
                                size_t scratch_bytes, void *stream) {
  return paged_attend(geom, ws, q, T, q_norm_w, eps, view_blocks, n_list, view_tokens_host, rope_theta, out, scratch,
                      scratch_bytes, stream, nullptr, nullptr, 0);
}

kvmem_status kvmem_materialize_attend(const kvmem_geom *geom, const kvmem_workspace *ws, const void *q, int32_t T,
                                      const float *q_norm_w, float eps, const int32_t *view_blocks, int32_t n_list,
                                      const int32_t *view_tokens_host, int32_t max_view, float rope_theta,
                                      void *k_view, void *v_view, float *out, void *scratch, size_t scratch_bytes,
                                      void *stream) {
  if (!k_view || !v_view) return KVMEM_E_ARG;
  return paged_attend(geom, ws, q, T, q_norm_w, eps, view_blocks, n_list, view_tokens_host, rope_theta, out, scratch,
                      scratch_bytes, stream, k_view, v_view, max_view);
}

size_t kvmem_attention_mass_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t T, int32_t max_blocks) {
  if (check_geom(geom) != KVMEM_OK || n_sessions <= 0 || max_blocks <= 0 || T <= 0) return 0;
  const int chunk = mass_chunk(n_sessions, geom->n_kv_heads, max_blocks);
  const size_t n_chunks = (size_t)((max_blocks + chunk - 1) / chunk);
  const size_t rows = (size_t)T * (geom->n_q_heads / geom->n_kv_heads);
  return align_up((size_t)n_sessions * geom->n_kv_heads * n_chunks * rows * sizeof(float4));
}

kvmem_status kvmem_attention_mass(const kvmem_geom *geom, const kvmem_workspace *ws, const void *q, int32_t T,
                                  const float *q_norm_w, float eps, const int32_t *view_blocks, int32_t n_list,
                                  float rope_theta, float *mass, float *lse_opt, void *scratch, size_t scratch_bytes,
                                  void *stream) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if ((st = check_ws(ws, false)) != KVMEM_OK) return st;
  if (!q || !q_norm_w || !mass || T <= 0 || n_list < 0 || (n_list > 0 && !view_blocks)) return KVMEM_E_ARG;
  if (!(eps >= 0.f) || !isfinite(eps) || !(rope_theta > 1.0f) || !isfinite(rope_theta)) return KVMEM_E_ARG;
  const int G = geom->n_q_heads / geom->n_kv_heads;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  if ((long)T * G > (bf16 ? kMfmaMaxRows : kF32PagedMaxRows)) return KVMEM_E_UNSUPPORTED;
  const int S = ws->n_sessions;
  if ((long)S * geom->n_kv_heads * n_list >= (1L << 31)) return KVMEM_E_UNSUPPORTED;
  const size_t need = kvmem_attention_mass_scratch_bytes(geom, S, T, ws->max_blocks);
  if (!scratch || scratch_bytes < need) return KVMEM_E_WORKSPACE;
  MassGeom g;
  g.Tq = T;
  g.Hq = geom->n_q_heads;
  g.Hkv = geom->n_kv_heads;
  g.G = G;
  g.rows = T * G;
  g.max_blocks = ws->max_blocks;
  g.n_pages = ws->n_pages;
  g.n_list = n_list;
  g.chunk = mass_chunk(S, geom->n_kv_heads, ws->max_blocks);
  g.n_chunks = (ws->max_blocks + g.chunk - 1) / g.chunk;
  for (int s0 = 0; s0 < S; s0 += kMaxSess) {
    const int n = S - s0 < kMaxSess ? S - s0 : kMaxSess;
    SessI32 nt;
    memset(&nt, 0, sizeof(nt));
    for (int i = 0; i < n; ++i) nt.v[i] = ws->n_tokens_host[s0 + i];
    st = hip_status(launch_mass(bf16, q, q_norm_w, eps, ws->k_pool, ws->block_table, view_blocks, (float4 *)scratch, mass,
                                lse_opt, ws->dev_error, nt, s0, n, g, (double)rope_theta, (hipStream_t)stream));
    if (st != KVMEM_OK) return st;
  }
  return KVMEM_OK;
}

kvmem_status kvmem_stage_view(const kvmem_geom *geom, const kvmem_workspace *ws, const int32_t *view_blocks,
                              int32_t n_list, const int32_t *view_tokens_host, void *stage_k, void *stage_v,
                              int32_t *stage_table, int32_t *stage_list, void *stream) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if ((st = check_ws(ws, true)) != KVMEM_OK) return st;
  if (!view_tokens_host || !stage_k || !stage_v || !stage_table || !stage_list || n_list <= 0) return KVMEM_E_ARG;
  bool any = false;
  for (int s = 0; s < ws->n_sessions; ++s) {
    const int V = view_tokens_host[s];
    if (V < 0 || (long)V > (long)kBT * n_list) return KVMEM_E_ARG;
    any = any || V > 0;
  }
  if (any && !view_blocks) return KVMEM_E_ARG;
  // staged pages and list entries are indexed in 32 bits
  if ((long)ws->n_sessions * n_list * geom->n_kv_heads >= (1L << 31)) return KVMEM_E_UNSUPPORTED;
  // the kernel reads the pools in place: they must be device memory or host
  // memory mapped for the GPU at the same address (pageable memory would fault)
  if (!gpu_addressable(ws->k_pool) || !gpu_addressable(ws->v_pool)) return KVMEM_E_ARG;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  for (int s0 = 0; s0 < ws->n_sessions; s0 += kMaxSess) {
    const int n = ws->n_sessions - s0 < kMaxSess ? ws->n_sessions - s0 : kMaxSess;
    SessI32 vt, na;
    memset(&vt, 0, sizeof(vt));
    memset(&na, 0, sizeof(na));
    for (int i = 0; i < n; ++i) {
      vt.v[i] = view_tokens_host[s0 + i];
      na.v[i] = (ws->n_tokens_host[s0 + i] + kBT - 1) / kBT;
    }
    st = hip_status(launch_stage(bf16, ws->k_pool, ws->v_pool, ws->block_table, view_blocks, stage_k, stage_v,
                                 stage_table, stage_list, ws->dev_error, vt, na, s0, n, geom->n_kv_heads,
                                 ws->max_blocks, ws->n_pages, n_list, (hipStream_t)stream));
    if (st != KVMEM_OK) return st;
  }
  return KVMEM_OK;
}

kvmem_status kvmem_materialize(const kvmem_geom *geom, const kvmem_workspace *ws, const int32_t *view_blocks,
                               int32_t n_list, const int32_t *view_tokens_host, int32_t max_view, float rope_theta,
                               void *k_view, void *v_view, void *stream) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if ((st = check_ws(ws, true)) != KVMEM_OK) return st;
  if (!view_tokens_host || !k_view || !v_view || n_list < 0) return KVMEM_E_ARG;
  if (max_view <= 0 || max_view % kBT != 0) return KVMEM_E_ARG;
  if (!(rope_theta > 1.0f) || !isfinite(rope_theta)) return KVMEM_E_ARG;
  bool any = false;
  for (int s = 0; s < ws->n_sessions; ++s) {
    const int V = view_tokens_host[s];
    if (V < 0 || V > max_view || (long)V > (long)kBT * n_list) return KVMEM_E_ARG;
    any = any || V > 0;
  }
  if (any && !view_blocks) return KVMEM_E_ARG;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  for (int s0 = 0; s0 < ws->n_sessions; s0 += kMaxSess) {
    const int n = ws->n_sessions - s0 < kMaxSess ? ws->n_sessions - s0 : kMaxSess;
    SessI32 vt, na;
    memset(&vt, 0, sizeof(vt));
    memset(&na, 0, sizeof(na));
    for (int i = 0; i < n; ++i) {
      vt.v[i] = view_tokens_host[s0 + i];
      na.v[i] = (ws->n_tokens_host[s0 + i] + kBT - 1) / kBT;
    }
    st = hip_status(launch_materialize(bf16, ws->k_pool, ws->v_pool, ws->block_table, view_blocks, k_view, v_view,
                                       ws->dev_error, vt, na, s0, n, geom->n_kv_heads, ws->max_blocks, ws->n_pages,
                                       n_list, max_view, (double)rope_theta, (hipStream_t)stream));
    if (st != KVMEM_OK) return st;
  }
  return KVMEM_OK;
}

size_t kvmem_attend_scratch_bytes(const kvmem_geom *geom, int32_t n_sessions, int32_t T, int32_t max_view) {
  if (check_geom(geom) != KVMEM_OK || n_sessions <= 0 || T <= 0 || max_view <= 0 || max_view % kBT) return 0;
  return attend_scratch(geom, n_sessions, T, max_view).total;
}

// Argument checks of kvmem_attend (all of them, before any HIP call); on
// success *sc holds the scratch layout the call needs.
static kvmem_status attend_check(const kvmem_geom *geom, int32_t n_sessions, const void *q, int32_t T,
                                 const float *q_norm_w, float eps, const void *k_view, const void *v_view,
                                 const int32_t *view_tokens_host, int32_t max_view, float rope_theta, float *out,
                                 AttendScratch *sc) {
  kvmem_status st = check_geom(geom);
  if (st != KVMEM_OK) return st;
  if (n_sessions <= 0 || !q || !q_norm_w || !k_view || !v_view || !view_tokens_host || !out || T <= 0)
    return KVMEM_E_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return KVMEM_E_ARG;
  if (max_view <= 0 || max_view % kBT != 0) return KVMEM_E_ARG;
  if (!(rope_theta > 1.0f) || !isfinite(rope_theta)) return KVMEM_E_ARG;
  for (int s = 0; s < n_sessions; ++s)
    if (view_tokens_host[s] < 0 || view_tokens_host[s] > max_view) return KVMEM_E_ARG;
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  const long rows = (long)T * (geom->n_q_heads / geom->n_kv_heads);
  if ((bf16 && rows > 32) || (!bf16 && rows > 64)) return KVMEM_E_UNSUPPORTED;
  *sc = attend_scratch(geom, n_sessions, T, max_view);
  return KVMEM_OK;
}

// The launches of kvmem_attend over a checked call, with its scratch at `base`.
static kvmem_status attend_launch(const kvmem_geom *geom, int32_t n_sessions, const void *q, int32_t T,
                                  const float *q_norm_w, float eps, const void *k_view, const void *v_view,
                                  const int32_t *view_tokens_host, int32_t max_view, float rope_theta, float *out,
                                  const AttendScratch &sc, char *base, void *stream,
                                  AppendArgs *ap = nullptr, const int32_t *n_tokens_host = nullptr) {
  const int bf16 = geom->kv_dtype == KVMEM_BF16;
  AttendGeom g;
  g.Tq = T;
  g.Hq = geom->n_q_heads;
  g.Hkv = geom->n_kv_heads;
  g.G = g.Hq / g.Hkv;
  g.rows = T * g.G;
  g.max_view = max_view;
  g.max_splits = sc.max_splits;
  g.tpw = sc.tpw;
  for (int s0 = 0; s0 < n_sessions; s0 += kMaxSess) {
    const int n = n_sessions - s0 < kMaxSess ? n_sessions - s0 : kMaxSess;
    SessI32 vt;
    memset(&vt, 0, sizeof(vt));
    for (int i = 0; i < n; ++i) vt.v[i] = view_tokens_host[s0 + i];
    if (ap != nullptr) {
      memset(&ap->n_tok, 0, sizeof(ap->n_tok));
      for (int i = 0; i < n; ++i) ap->n_tok.v[i] = n_tokens_host[s0 + i];
    }
    const kvmem_status st = hip_status(launch_attend(bf16, q, q_norm_w, eps, k_view, v_view,
                                                     (float *)(base + sc.part_o), (float2 *)(base + sc.part_ml),
                                                     out, vt, s0, n, g, (double)rope_theta, (hipStream_t)stream, ap));
    if (st != KVMEM_OK) return st;
  }
  return KVMEM_OK;
}

kvmem_status kvmem_attend(const kvmem_geom *geom, int32_t n_sessions, const void *q, int32_t T,
                          const float *q_norm_w, float eps, const void *k_view, const void *v_view,
                          const int32_t *view_tokens_host, int32_t max_view, float rope_theta, float *out,
                          void *scratch, size_t scratch_bytes, void *stream) {
  AttendScratch sc;
  const kvmem_status st = attend_check(geom, n_sessions, q, T, q_norm_w, eps, k_view, v_view, view_tokens_host,
                                       max_view, rope_theta, out, &sc);
  if (st != KVMEM_OK) return st;
  if (!scratch || scratch_bytes < sc.total) return KVMEM_E_WORKSPACE;
  return attend_launch(geom, n_sessions, q, T, q_norm_w, eps, k_view, v_view, view_tokens_host, max_view,
                       rope_theta, out, sc, (char *)scratch, stream);
}

kvmem_status kvmem_attend_append(const kvmem_geom *geom, const kvmem_workspace *ws, const void *q, int32_t T,
                                 const float *q_norm_w, float eps, void *k_view, void *v_view,
                                 const int32_t *view_tokens_host, int32_t max_view, float rope_theta, float *out,
                                 void *k_pool, void *v_pool, const void *k_new, const void *v_new, int32_t T_new,
                                 void *scratch, size_t scratch_bytes, void *stream) {
  if (!ws) return KVMEM_E_ARG;
  AttendScratch sc;
  kvmem_status st = attend_check(geom, ws->n_sessions, q, T, q_norm_w, eps, k_view, v_view, view_tokens_host,
                                 max_view, rope_theta, out, &sc);
  if (st != KVMEM_OK) return st;
  // the checks of kvmem_append
  if ((st = check_ws(ws, true)) != KVMEM_OK) return st;
  if (!k_pool || !v_pool || k_pool != ws->k_pool || v_pool != ws->v_pool) return KVMEM_E_ARG;
  if (!k_new || !v_new || T_new < 0) return KVMEM_E_ARG;
  for (int s = 0; s < ws->n_sessions; ++s) {
    if ((long)ws->n_tokens_host[s] + T_new > (long)ws->max_blocks * kBT) return KVMEM_E_ARG;
    if ((long)view_tokens_host[s] + T_new > max_view) return KVMEM_E_ARG;
  }
  if (!scratch || scratch_bytes < sc.total) return KVMEM_E_WORKSPACE;
  AppendArgs ap;
  memset(&ap, 0, sizeof(ap));
  ap.kpool = k_pool;
  ap.vpool = v_pool;
  ap.table = ws->block_table;
  ap.knew = k_new;
  ap.vnew = v_new;
  ap.kview = k_view;
  ap.vview = v_view;
  ap.dev_err = ws->dev_error;
  ap.T_new = T_new;
  ap.Hkv = geom->n_kv_heads;
  ap.max_blocks = ws->max_blocks;
  ap.n_pages = ws->n_pages;
  ap.max_view = max_view;
  ap.bf16 = geom->kv_dtype == KVMEM_BF16;
  ap.theta = (double)rope_theta;
  return attend_launch(geom, ws->n_sessions, q, T, q_norm_w, eps, k_view, v_view, view_tokens_host, max_view,
                       rope_theta, out, sc, (char *)scratch, stream, &ap, ws->n_tokens_host);
}

kvmem_status kvmem_attend_noalloc(const kvmem_geom *geom, int32_t n_sessions, const void *q, int32_t T,
                                  const float *q_norm_w, float eps, const void *k_view, const void *v_view,
                                  const int32_t *view_tokens_host, int32_t max_view, float rope_theta, float *out,
                                  void *stream) {
  AttendScratch sc;
  kvmem_status st = attend_check(geom, n_sessions, q, T, q_norm_w, eps, k_view, v_view, view_tokens_host, max_view,
                                 rope_theta, out, &sc);
  if (st != KVMEM_OK) return st;
  if (sc.total > kNoAllocBytes) return KVMEM_E_WORKSPACE;
  void *base = nullptr;
  if ((st = noalloc_scratch(&base)) != KVMEM_OK) return st;
  return attend_launch(geom, n_sessions, q, T, q_norm_w, eps, k_view, v_view, view_tokens_host, max_view,
                       rope_theta, out, sc, (char *)base, stream);
}

}  // extern "C"
