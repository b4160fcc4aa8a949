// Block scoring and GQA aggregation for short query steps (T * G rows per KV head).
//
// KVMem scores every indexed block with s_b = <q, k_bar_b>/sqrt(d) (reproduction
// README, 'Core equation') after RMS-normalising the query, then softmaxes each
// query head over the blocks and sums the heads of a KV group (README,
// '2026-09-08 validation correction': averaging GQA heads before the softmax was
// the withdrawn bug).
//
// k_score_gemv: a memory-bound GEMV on the vector ALUs.  LPR lanes share one
// 256-byte index row, each lane holding DPL = 128/LPR of its dimensions and the
// matching slice of all LPR query rows in registers, so every index element is
// loaded once and feeds LPR FMAs.  The LPR partial sums are then combined with a
// DPP reduce-scatter: lane p keeps its partials in a lane-specific row order
// (row = register ^ x(p)), chosen so that at every step each lane adds the
// partner's register that holds the same row -- log2(LPR) fused add+DPP moves and
// no selects.  After the last step lane p owns the full score of row x(p).
// Scores go through LDS to coalesced stores; per (row, chunk) the kernel also
// writes the chunk's max and sum of exp, so the softmax needs no second pass over
// the index.
//
// k_aggregate: merges the chunk statistics into each row's max and normaliser,
// then A[b] = sum_rows exp(s[row][b] - M_row) / Z_row, summed in row order.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

// Reduce-scatter schedule for LPR lanes per index row.  Step i exchanges with
// lane p ^ mask_i (DPP pattern) and keeps registers [0, LPR >> (i+1)).  x(p) is
// the linear map over the bits of p with x(p) ^ x(p ^ mask_i) = LPR >> (i+1).
template <int LPR>
struct RS;

template <>
struct RS<4> {  // masks 2, 1
  static __device__ __forceinline__ int x(int p) { return p & 3; }
  template <int N>
  static __device__ __forceinline__ void reduce(float (&a)[N]) {
    a[0] += dpp_f32<kDppXor2>(a[2]);
    a[1] += dpp_f32<kDppXor2>(a[3]);
    a[0] += dpp_f32<kDppXor1>(a[1]);
  }
};

template <>
struct RS<8> {  // masks 7, 2, 1
  static __device__ __forceinline__ int x(int p) {
    return (p & 1) ^ (p & 2) ^ ((p & 4) ? 7 : 0);
  }
  template <int N>
  static __device__ __forceinline__ void reduce(float (&a)[N]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += dpp_f32<kDppMirror8>(a[k + 4]);
    a[0] += dpp_f32<kDppXor2>(a[2]);
    a[1] += dpp_f32<kDppXor2>(a[3]);
    a[0] += dpp_f32<kDppXor1>(a[1]);
  }
};

template <>
struct RS<16> {  // masks 15, 7, 2, 1
  static __device__ __forceinline__ int x(int p) {
    return (p & 1) ^ (p & 2) ^ ((p & 4) ? 7 : 0) ^ ((p & 8) ? 12 : 0);
  }
  template <int N>
  static __device__ __forceinline__ void reduce(float (&a)[N]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] += dpp_f32<kDppMirror16>(a[k + 8]);
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += dpp_f32<kDppMirror8>(a[k + 4]);
    a[0] += dpp_f32<kDppXor2>(a[2]);
    a[1] += dpp_f32<kDppXor2>(a[3]);
    a[0] += dpp_f32<kDppXor1>(a[1]);
  }
};

template <typename T, int N>
struct LoadRow;

template <int N>
struct LoadRow<uint16_t, N> {  // N bf16 (N multiple of 8) -> fp32
  static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[N]) {
#pragma unroll
    for (int c = 0; c < N / 8; ++c) {
      const uint4 w = *reinterpret_cast<const uint4 *>(p + 8 * c);
      const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * c + 2 * k] = bf16_lo(e[k]);
        v[8 * c + 2 * k + 1] = bf16_hi(e[k]);
      }
    }
  }
};

template <int N>
struct LoadRow<float, N> {  // N fp32 (N multiple of 4)
  static __device__ __forceinline__ void load(const float *p, float (&v)[N]) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const float4 w = reinterpret_cast<const float4 *>(p)[c];
      v[4 * c] = w.x; v[4 * c + 1] = w.y; v[4 * c + 2] = w.z; v[4 * c + 3] = w.w;
    }
  }
};

__device__ __forceinline__ float load_elem(const uint16_t *p) { return bf16_lo(*p); }
__device__ __forceinline__ float load_elem(const float *p) { return *p; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
  return v;
}

// q~ = w * q / sqrt(mean(q^2) + eps), pre-scaled by 1/sqrt(d), for rows
// [r0, r0 + NR) of KV head h, into LDS.  Rows past n_rows are zero.
template <typename T, int NR>
__device__ __forceinline__ void norm_rows_to_lds(float (*qs)[kD], const T *q, const float *qw, float eps,
                                                 int s, int h, int r0, int n_rows, int Tq, int Hq, int G) {
  const int lane16 = threadIdx.x & 15;
  for (int rr = threadIdx.x >> 4; rr < NR; rr += blockDim.x >> 4) {
    const int r = r0 + rr;
    float x[8];
    float ss = 0.f;
    if (r < n_rows) {
      const int t = r / G, g = r % G;
      const T *src = q + (((size_t)s * Tq + t) * Hq + (size_t)h * G + g) * kD + lane16 * 8;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] = load_elem(src + k);
        ss += x[k] * x[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = 0.f;
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) ss += shfl_xor_f(ss, m);
    const float rs = (1.0f / sqrtf(ss * (1.0f / kD) + eps)) * 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
    for (int k = 0; k < 8; ++k) qs[rr][lane16 * 8 + k] = (r < n_rows) ? x[k] * rs * qw[lane16 * 8 + k] : 0.f;
  }
}

// Raw 16-byte words of the index slice one lane reads for one work item.
template <typename T, int LPR>
struct ItemRaw {
  static constexpr int kWords = (kD / LPR) * (int)sizeof(T) / 16;   // per index row and lane
  static constexpr int kRows = kScoreChunk / (4 * (64 / LPR));         // rows per lane per item
  uint4 w[kRows][kWords];
};

// Work item = (session, KV head x row group, chunk of kScoreChunk blocks).
struct Item {
  int sl, h, r0, b0, nb, key;
  bool valid;
};

__device__ __forceinline__ Item decode_item(int item, int n_chunks_launch, int ny, int Hkv, int rows_per_group,
                                            int n_rows, const SessI32 &n_blocks) {
  Item it;
  const int chunk = item % n_chunks_launch;
  it.key = item / n_chunks_launch;
  const int y = it.key % ny;
  it.sl = it.key / ny;
  it.h = y % Hkv;
  it.r0 = (y / Hkv) * rows_per_group;
  it.nb = n_blocks.v[it.sl];
  it.b0 = chunk * kScoreChunk;
  it.valid = it.b0 < it.nb && it.r0 < n_rows;
  return it;
}

template <typename T, int LPR>
__device__ __forceinline__ void load_item(ItemRaw<T, LPR> &raw, const T *index, const Item &it, int s0,
                                          const ScoreGeom &g, int lane, int wave) {
  constexpr int DPL = kD / LPR;
  constexpr int RPW = 64 / LPR;
  constexpr int RPI = 4 * RPW;
  const T *base = index + ((size_t)((s0 + it.sl) * g.Hkv + it.h) * g.max_blocks) * kD + (lane % LPR) * DPL;
#pragma unroll
  for (int r = 0; r < ItemRaw<T, LPR>::kRows; ++r) {
    // rows past the history re-read the last row (their scores are never
    // stored): no branch around the loads, so they all stay in flight
    const int b = min(it.b0 + r * RPI + wave * RPW + lane / LPR, it.nb - 1);
    const T *src = base + (size_t)b * kD;
#pragma unroll
    for (int w = 0; w < ItemRaw<T, LPR>::kWords; ++w) raw.w[r][w] = load_nt16(src + w * (16 / sizeof(T)));
  }
}

template <int N>
__device__ __forceinline__ void unpack_row(const uint4 *w, float (&v)[N], uint16_t) {
#pragma unroll
  for (int c = 0; c < N / 8; ++c) {
    const uint32_t e[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * c + 2 * k] = bf16_lo(e[k]);
      v[8 * c + 2 * k + 1] = bf16_hi(e[k]);
    }
  }
}
template <int N>
__device__ __forceinline__ void unpack_row(const uint4 *w, float (&v)[N], float) {
#pragma unroll
  for (int c = 0; c < N / 4; ++c) {
    v[4 * c] = __uint_as_float(w[c].x);
    v[4 * c + 1] = __uint_as_float(w[c].y);
    v[4 * c + 2] = __uint_as_float(w[c].z);
    v[4 * c + 3] = __uint_as_float(w[c].w);
  }
}

// Persistent over work items, chunk fastest.  Workgroup b takes the contiguous
// items [b * per, (b + 1) * per), so the grid is one round of resident
// workgroups and the query rows are normalised again only when (session, head)
// changes.  The next item's index rows are requested before the current item's
// scores are written out.
template <typename T, int LPR>
__global__ __launch_bounds__(256) void k_score_gemv(const T *__restrict__ index, const T *__restrict__ q,
                                                    const float *__restrict__ qw, float eps,
                                                    float *__restrict__ scores, float2 *__restrict__ part,
                                                    SessI32 n_blocks, int s0, ScoreGeom g, int n_sess,
                                                    int n_rg, int n_chunks_launch, int per) {
  constexpr int ROWS = LPR;
  constexpr int DPL = kD / LPR;
  constexpr int RPW = 64 / LPR;
  constexpr int RPI = 4 * RPW;
  constexpr int NIT = kScoreChunk / RPI;
  __shared__ float qs[ROWS][kD];
  __shared__ float st[ROWS][kScoreChunk];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int p = lane % LPR;
  const int xl = RS<LPR>::x(p);
  const int n_rows = g.Tq * g.G;
  const int ny = g.Hkv * n_rg;
  const int total = n_sess * ny * n_chunks_launch;
  const int item0 = blockIdx.x * per;
  const int item1 = min(total, item0 + per);
  int loaded = -1;
  float qr[ROWS][DPL];
  ItemRaw<T, LPR> raw;

  int item = item0;
  Item cur;
  for (; item < item1; ++item) {                       // first valid item
    cur = decode_item(item, n_chunks_launch, ny, g.Hkv, ROWS, n_rows, n_blocks);
    if (cur.valid) break;
  }
  if (item < item1) load_item<T, LPR>(raw, index, cur, s0, g, lane, wave);

  while (item < item1) {
    const int s = s0 + cur.sl;
    if (cur.key != loaded) {
      __syncthreads();
      norm_rows_to_lds<T, ROWS>(qs, q, qw, eps, s, cur.h, cur.r0, n_rows, g.Tq, g.Hq, g.G);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < ROWS; ++k)
#pragma unroll
        for (int j = 0; j < DPL; ++j) qr[k][j] = qs[k ^ xl][p * DPL + j];
      loaded = cur.key;
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float kv[DPL];
      unpack_row(raw.w[it], kv, T());
      float acc[ROWS];
#pragma unroll
      for (int k = 0; k < ROWS; ++k) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) a = fmaf(qr[k][j], kv[j], a);
        acc[k] = a;
      }
      RS<LPR>::reduce(acc);
      st[xl][it * RPI + wave * RPW + lane / LPR] = acc[0];
    }
    // next valid item: request its rows now
    int nxt = item + 1;
    Item next = cur;
    for (; nxt < item1; ++nxt) {
      next = decode_item(nxt, n_chunks_launch, ny, g.Hkv, ROWS, n_rows, n_blocks);
      if (next.valid) break;
    }
    if (nxt < item1) load_item<T, LPR>(raw, index, next, s0, g, lane, wave);
    __syncthreads();

    const int nvalid = min(kScoreChunk, cur.nb - cur.b0);
    const int chunk = cur.b0 / kScoreChunk;
    for (int rr = wave; rr < ROWS; rr += 4) {
      const int r = cur.r0 + rr;
      if (r >= n_rows) break;
      const int t = r / g.G, gg = r % g.G;
      const size_t row_id = ((size_t)s * g.Tq + t) * g.Hq + (size_t)cur.h * g.G + gg;
      float *dst = scores + row_id * g.max_blocks + cur.b0;
      float m = -INFINITY;
      for (int j = lane; j < nvalid; j += 64) {
        const float v = st[rr][j];
        dst[j] = v;
        m = fmaxf(m, v);
      }
      m = wave_max(m);
      float l = 0.f;
      for (int j = lane; j < nvalid; j += 64) l += expf(st[rr][j] - m);
      l = wave_sum(l);
      if (lane == 0) part[row_id * g.n_chunks + chunk] = make_float2(m, l);
    }
    __syncthreads();
    item = nxt;
    cur = next;
  }
}

__device__ __forceinline__ float2 merge_ml(float2 a, float2 b) {
  const float M = fmaxf(a.x, b.x);
  if (M == -INFINITY) return make_float2(-INFINITY, 0.f);
  return make_float2(M, a.y * expf(a.x - M) + b.y * expf(b.x - M));
}

constexpr int kAggRowsPerPass = 64;

// One workgroup per (session, KV head, 256 blocks).  Each wavefront first
// merges the chunk statistics of some rows into the row's max M and 1/Z
// (log-sum-exp merge), then every thread owns one block and sums
// exp(s - M) / Z over the rows in a fixed order.
__global__ __launch_bounds__(256) void k_aggregate(const float *__restrict__ scores,
                                                   const float2 *__restrict__ part, float *__restrict__ A,
                                                   SessI32 n_blocks, int s0, ScoreGeom g) {
  __shared__ float sM[kAggRowsPerPass];
  __shared__ float sInvZ[kAggRowsPerPass];
  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int nb = n_blocks.v[sl];
  const int b0 = blockIdx.x * kAggChunk;
  if (b0 >= nb) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n_rows = g.Tq * g.G;
  const int nch = (nb + kScoreChunk - 1) / kScoreChunk;
  const int b = b0 + threadIdx.x;
  const bool valid = b < nb;
  float acc = 0.f;

  for (int rb = 0; rb < n_rows; rb += kAggRowsPerPass) {
    const int nr = min(kAggRowsPerPass, n_rows - rb);
    for (int rr = wave; rr < nr; rr += 4) {
      const int r = rb + rr;
      const int t = r / g.G, gg = r % g.G;
      const size_t row_id = ((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg;
      float2 ml = make_float2(-INFINITY, 0.f);
      for (int c = lane; c < nch; c += 64) ml = merge_ml(ml, part[row_id * g.n_chunks + c]);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        float2 o;
        o.x = shfl_xor_f(ml.x, m);
        o.y = shfl_xor_f(ml.y, m);
        ml = merge_ml(ml, o);
      }
      if (lane == 0) {
        sM[rr] = ml.x;
        sInvZ[rr] = 1.0f / ml.y;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int rr = 0; rr < nr; ++rr) {
      const int r = rb + rr;
      const int t = r / g.G, gg = r % g.G;
      const size_t row_id = ((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg;
      const float v = valid ? scores[row_id * g.max_blocks + b] : 0.f;
      acc += expf(v - sM[rr]) * sInvZ[rr];
    }
    __syncthreads();
  }
  if (valid) A[((size_t)s * g.Hkv + h) * g.max_blocks + b] = acc;
}

template <typename T, int LPR>
hipError_t launch_gemv_lpr(const void *index, const void *q, const float *qw, float eps, float *scores,
                           float2 *part, const SessI32 &n_blocks, int s0, int n_sess, const ScoreGeom &g,
                           int max_nb, hipStream_t st) {
  const int n_rows = g.Tq * g.G;
  const int n_rg = (n_rows + LPR - 1) / LPR;
  const int n_chunks = (max_nb + kScoreChunk - 1) / kScoreChunk;
  const long total = (long)n_sess * g.Hkv * n_rg * n_chunks;
  static int res = 0;                                   // resident workgroups (device property)
  if (res == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_score_gemv<T, LPR>, 256, 0) != hipSuccess) per_cu = 1;
    res = (cus > 0 ? cus : 256) * (per_cu > 0 ? per_cu : 1);
  }
  const long grid0 = total < res ? total : res;
  const int per = (int)((total + grid0 - 1) / grid0);
  const int grid = (int)((total + per - 1) / per);
  hipLaunchKernelGGL((k_score_gemv<T, LPR>), dim3(grid), dim3(256), 0, st, (const T *)index, (const T *)q, qw, eps,
                     scores, part, n_blocks, s0, g, n_sess, n_rg, n_chunks, per);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemv_t(const void *index, const void *q, const float *qw, float eps, float *scores,
                         float2 *part, const SessI32 &n_blocks, int s0, int n_sess, const ScoreGeom &g,
                         hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  if (max_nb == 0) return hipSuccess;
  const int n_rows = g.Tq * g.G;
  if (n_rows <= 4) return launch_gemv_lpr<T, 4>(index, q, qw, eps, scores, part, n_blocks, s0, n_sess, g, max_nb, st);
  if (n_rows <= 8) return launch_gemv_lpr<T, 8>(index, q, qw, eps, scores, part, n_blocks, s0, n_sess, g, max_nb, st);
  return launch_gemv_lpr<T, 16>(index, q, qw, eps, scores, part, n_blocks, s0, n_sess, g, max_nb, st);
}

}  // namespace

hipError_t launch_score_gemv(int bf16, const void *index, const void *q, const float *qw, float eps,
                             float *scores, float2 *part, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, hipStream_t st) {
  return bf16 ? launch_gemv_t<uint16_t>(index, q, qw, eps, scores, part, n_blocks, s0, n_sess, g, st)
              : launch_gemv_t<float>(index, q, qw, eps, scores, part, n_blocks, s0, n_sess, g, st);
}

hipError_t launch_aggregate(const float *scores, const float2 *part, float *A, const SessI32 &n_blocks,
                            int s0, int n_sess, const ScoreGeom &g, hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  if (max_nb == 0) return hipSuccess;
  dim3 grid((unsigned)((max_nb + kAggChunk - 1) / kAggChunk), (unsigned)g.Hkv, (unsigned)n_sess);
  hipLaunchKernelGGL(k_aggregate, grid, dim3(256), 0, st, scores, part, A, n_blocks, s0, g);
  return hipGetLastError();
}

}  // namespace kvmem
