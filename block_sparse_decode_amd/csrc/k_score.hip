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

template <typename T, int LPR>
__global__ __launch_bounds__(256) void k_score_gemv(const T *__restrict__ index, const T *__restrict__ q,
                                                    const float *__restrict__ qw, float eps,
                                                    float *__restrict__ scores, float2 *__restrict__ part,
                                                    SessI32 n_blocks, int s0, ScoreGeom g) {
  constexpr int ROWS = LPR;
  constexpr int DPL = kD / LPR;
  constexpr int RPW = 64 / LPR;          // index rows per wave per step
  constexpr int RPI = 4 * RPW;           // index rows per workgroup per step
  constexpr int NIT = kScoreChunk / RPI;
  __shared__ float qs[ROWS][kD];
  __shared__ float st[ROWS][kScoreChunk];

  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y % g.Hkv;
  const int rg = blockIdx.y / g.Hkv;
  const int chunk = blockIdx.x;
  const int nb = n_blocks.v[sl];
  const int b0 = chunk * kScoreChunk;
  const int n_rows = g.Tq * g.G;
  const int r0 = rg * ROWS;
  if (b0 >= nb || r0 >= n_rows) return;

  norm_rows_to_lds<T, ROWS>(qs, q, qw, eps, s, h, r0, n_rows, g.Tq, g.Hq, g.G);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int p = lane % LPR;
  const int xl = RS<LPR>::x(p);
  float qr[ROWS][DPL];
#pragma unroll
  for (int k = 0; k < ROWS; ++k)
#pragma unroll
    for (int j = 0; j < DPL; ++j) qr[k][j] = qs[k ^ xl][p * DPL + j];

  const T *base = index + ((size_t)(s * g.Hkv + h) * g.max_blocks) * kD + p * DPL;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int bl = it * RPI + wave * RPW + lane / LPR;
    const int b = b0 + bl;
    float kv[DPL];
    if (b < nb) {
      LoadRow<T, DPL>::load(base + (size_t)b * kD, kv);
    } else {
#pragma unroll
      for (int j = 0; j < DPL; ++j) kv[j] = 0.f;
    }
    float acc[ROWS];
#pragma unroll
    for (int k = 0; k < ROWS; ++k) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) a = fmaf(qr[k][j], kv[j], a);
      acc[k] = a;
    }
    RS<LPR>::reduce(acc);
    st[xl][bl] = acc[0];
  }
  __syncthreads();

  const int nvalid = min(kScoreChunk, nb - b0);
  for (int rr = wave; rr < ROWS; rr += 4) {
    const int r = r0 + rr;
    if (r >= n_rows) break;
    const int t = r / g.G, gg = r % g.G;
    const size_t row_id = ((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg;
    float *dst = scores + row_id * g.max_blocks + b0;
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
}

__device__ __forceinline__ float2 merge_ml(float2 a, float2 b) {
  const float M = fmaxf(a.x, b.x);
  if (M == -INFINITY) return make_float2(-INFINITY, 0.f);
  return make_float2(M, a.y * expf(a.x - M) + b.y * expf(b.x - M));
}

constexpr int kAggRowsPerPass = 64;
constexpr int kAggPerThread = kAggChunk / 256;

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

  float acc[kAggPerThread];
#pragma unroll
  for (int k = 0; k < kAggPerThread; ++k) acc[k] = 0.f;

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
    for (int rr = 0; rr < nr; ++rr) {
      const int r = rb + rr;
      const int t = r / g.G, gg = r % g.G;
      const size_t row_id = ((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg;
      const float *src = scores + row_id * g.max_blocks;
      const float M = sM[rr], iz = sInvZ[rr];
#pragma unroll
      for (int k = 0; k < kAggPerThread; ++k) {
        const int b = b0 + threadIdx.x + 256 * k;
        if (b < nb) acc[k] += expf(src[b] - M) * iz;
      }
    }
    __syncthreads();
  }
  float *dst = A + ((size_t)s * g.Hkv + h) * g.max_blocks;
#pragma unroll
  for (int k = 0; k < kAggPerThread; ++k) {
    const int b = b0 + threadIdx.x + 256 * k;
    if (b < nb) dst[b] = acc[k];
  }
}

template <typename T>
hipError_t launch_gemv_t(const void *index, const void *q, const float *qw, float eps, float *scores,
                         float2 *part, const SessI32 &n_blocks, int s0, int n_sess, const ScoreGeom &g,
                         hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  if (max_nb == 0) return hipSuccess;
  const int n_rows = g.Tq * g.G;
  const int lpr = n_rows <= 4 ? 4 : (n_rows <= 8 ? 8 : 16);
  const int n_rg = (n_rows + lpr - 1) / lpr;
  dim3 grid((unsigned)((max_nb + kScoreChunk - 1) / kScoreChunk), (unsigned)(g.Hkv * n_rg), (unsigned)n_sess);
  const T *ip = (const T *)index;
  const T *qp = (const T *)q;
  if (lpr == 4)
    hipLaunchKernelGGL((k_score_gemv<T, 4>), grid, dim3(256), 0, st, ip, qp, qw, eps, scores, part, n_blocks, s0, g);
  else if (lpr == 8)
    hipLaunchKernelGGL((k_score_gemv<T, 8>), grid, dim3(256), 0, st, ip, qp, qw, eps, scores, part, n_blocks, s0, g);
  else
    hipLaunchKernelGGL((k_score_gemv<T, 16>), grid, dim3(256), 0, st, ip, qp, qw, eps, scores, part, n_blocks, s0, g);
  return hipGetLastError();
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
