// Block scoring and aggregation for long query chunks (prefill-style steps).
//
// With hundreds of query tokens per step (T * G rows per KV head, e.g. 512
// tokens x 8 heads = 4096 rows) scoring every index block is a large dense
// contraction, and the per-(token, head) softmax of the reproduction README
// ('2026-09-08 validation correction') needs each row's normaliser over all
// blocks before any block's aggregate A[b] = sum_rows p[row][b] can be formed.
// The score matrix (rows x blocks) is far too large to keep, so it is
// computed twice on the matrix cores:
//
//   k_long_qprep : q~ * log2(e)/sqrt(d) of every row as bf16 hi + lo B-operand
//                  fragments (16 rows per operand set), and each row's |q~|.
//   k_long_pass  : one workgroup per (session, KV head, group of 256 blocks);
//                  each of its 4 wavefronts holds one 64-block index tile as
//                  A operands in registers for the whole kernel, and the rows
//                  stream through LDS in chunks of 64 (double-buffered).
//                  STATS: per-row (M, sum of 2^(s - M)) over the group's
//                  blocks -> part[row][group].  AGG: 2^(s - lse[row]) summed
//                  over all rows into per-lane block sums, reduced across the
//                  16 lanes of each block at the end -> A[b].
//   k_long_lse   : lse[row] = log2 of the row's normaliser from its partials.
//
// Scores are in log2 units throughout (the constant is folded into the query),
// so every exponential is a single exp2.  Each exponential's shift enters the
// products as the accumulator's initial value (-lse[row] in AGG; in STATS,
// -|q~| max|k_bar| over the tile, an upper bound of the row's scores there by
// Cauchy-Schwarz that stands for the row maximum M, with the exact maximum
// taken only when the bound lies so far above the scores that the sum would
// lose its terms), which leaves one exp2 and one add per score.  Output order
// is fixed everywhere (deterministic).
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr float kLog2eRsqrtD = 0.12751743074480953f;   // log2(e) / sqrt(128)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kLongBlocks = 4 * kIdxTile;              // blocks per workgroup (4 wavefronts x 1 tile)
constexpr int kLongChunkSets = 4;                      // operand sets (16 rows each) per LDS chunk
constexpr int kLongChunkRows = 16 * kLongChunkSets;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// qf[((s * Hkv + h) * n_sets + cs) * 8 + 2k + hl][lane]: lane (qq, col) holds
// dims 32k + 8qq .. + 7 of row 16cs + col, q~ * log2(e)/sqrt(d), bf16 hi (hl=0)
// or lo (hl=1).  Rows past T * G are zero.  One wavefront per (s, h, cs).
__global__ __launch_bounds__(64) void k_long_qprep(const uint16_t *__restrict__ q, const float *__restrict__ qw,
                                                   float eps, uint4 *__restrict__ qf, float *__restrict__ qn, int s0,
                                                   ScoreGeom g, int n_sets) {
  const int lane = threadIdx.x;
  const int qq = lane >> 4, col = lane & 15;
  const int cs = blockIdx.x % n_sets;
  const int h = blockIdx.x / n_sets;
  const int s = s0 + blockIdx.y;
  const int n_rows = g.Tq * g.G;
  const int r = cs * 16 + col;
  const bool valid = r < n_rows;
  const int t = valid ? r / g.G : 0, gg = valid ? r % g.G : 0;
  const uint16_t *src = q + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD + 8 * qq;
  float x[4][8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint4 w = *reinterpret_cast<const uint4 *>(src + 32 * k);
    const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[k][2 * j] = bf16_lo(e[j]);
      x[k][2 * j + 1] = bf16_hi(e[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[k][j] * x[k][j];
  }
  ss = sum_xor16(ss);
  ss = sum_xor32(ss);
  const float rs = valid ? (1.0f / sqrtf(ss * (1.0f / kD) + eps)) * kLog2eRsqrtD : 0.f;
  uint4 *dst = qf + (((size_t)s * g.Hkv + h) * n_sets + cs) * 8 * 64 + lane;
  float nn = 0.f;                                       // |q~|^2 of the row (this lane's 32 dims)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint32_t h0, l0, h1, l1;
      const float v0 = x[k][j] * rs * qw[32 * k + 8 * qq + j];
      const float v1 = x[k][j + 1] * rs * qw[32 * k + 8 * qq + j + 1];
      nn += v0 * v0 + v1 * v1;
      split_hi_lo(v0, h0, l0);
      split_hi_lo(v1, h1, l1);
      hw[j / 2] = h0 | (h1 << 16);
      lw[j / 2] = l0 | (l1 << 16);
    }
    dst[(2 * k) * 64] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    dst[(2 * k + 1) * 64] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  nn = sum_xor16(nn);
  nn = sum_xor32(nn);
  if (qq == 0) qn[((size_t)s * g.Hkv + h) * (16 * n_sets) + r] = sqrtf(nn);
}

struct LongGeom {
  int n_rows;     // T * G
  int n_sets;     // ceil(n_rows / 16)
  int n_chunks;   // ceil(n_sets / kLongChunkSets)
  int rows_pad;   // 16 * n_sets
  int n_groups;   // workgroups (block groups) per (session, head) slot row: ceil(max_blocks / 256)
};

template <bool AGG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_long_pass(const uint16_t *__restrict__ index, const uint4 *__restrict__ qf,
                                                   float2 *__restrict__ part, const float *__restrict__ lse,
                                                   float *__restrict__ A, float *__restrict__ scores,
                                                   SessI32 n_blocks, int s0, ScoreGeom g, LongGeom L) {
  __shared__ uint4 sb[2][kLongChunkSets * 8 * 64];     // B fragments of one chunk, double-buffered (64 KiB)
  __shared__ float slse[2][kLongChunkRows];
  __shared__ float2 sst[4][kLongChunkRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int qq = lane >> 4, col = lane & 15;
  const int sl = blockIdx.z, s = s0 + sl;
  const int h = blockIdx.y;
  const int grp = blockIdx.x;
  const int nb = n_blocks.v[sl];
  if (grp * kLongBlocks >= nb) return;                  // whole group past the history (uniform)
  const int tile = grp * 4 + wave;
  const bool live = tile * kIdxTile < nb;               // this wavefront's tile holds blocks
  const size_t sh = (size_t)s * g.Hkv + h;

  // the wavefront's 64 index blocks as A operands: a[4m + k] = word 4k + qq of block 16m + col
  uint4 a[16];
  {
    const uint16_t *t = index + (sh * g.n_tiles + (live ? tile : 0)) * (size_t)(kIdxTile * kD);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int k = 0; k < 4; ++k) a[4 * m + k] = load_nt16(t + ((4 * k + qq) * kIdxTile + 16 * m + col) * 8);
  }
  // block b = tile * 64 + 16m + 4qq + i is valid when below nb; only the last
  // tile of a history is partial, so the masked path is rare (`full` is the
  // same for the whole wavefront)
  const bool full = live && (tile + 1) * kIdxTile <= nb;
  int vmask = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) vmask |= (live && tile * kIdxTile + 16 * m + 4 * qq + i < nb) ? 1 << (4 * m + i) : 0;

  // STATS: the largest |index row| of the wavefront's valid blocks.  A row's
  // scores over the tile are at most |q~| kmax (Cauchy-Schwarz), which shifts
  // its exponentials in place of the row maximum.
  float kmax = 0.f;
  if (!AGG) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float nn = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t e[4] = {a[4 * m + k].x, a[4 * m + k].y, a[4 * m + k].z, a[4 * m + k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = bf16_lo(e[j]), hi = bf16_hi(e[j]);
          nn += lo * lo + hi * hi;
        }
      }
      nn = sum_xor16(nn);
      nn = sum_xor32(nn);                               // block 16m + col, in all 4 lanes of the column
      if (live && tile * kIdxTile + 16 * m + col < nb) kmax = fmaxf(kmax, nn);
    }
    kmax = sqrtf(wave_max_dpp(kmax));
  }

  float acc[16];                                        // AGG: sum over rows of 2^(s - lse) per own block
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  // Staging a chunk of query fragments (and, for AGG, its rows' lse) into LDS
  // is split in two: the global loads of chunk c + 1 are issued into
  // registers before chunk c is multiplied, and written to LDS after it, so
  // their latency hides behind the products.  (Plain code, no lambdas: the
  // staging registers must stay registers.)
  const uint4 *qsrc = qf + sh * L.n_sets * 8 * 64;
  constexpr int kPer = kLongChunkSets * 8 * 64 / 256;   // uint4 per thread per chunk
  u32x4 pre[kPer];                                       // native vectors: HIP's uint4 here stays in scratch
  float pre_lse = INFINITY;
#define KVMEM_LONG_FETCH(CHUNK)                                                        \
  {                                                                                   \
    const int fset0 = (CHUNK) * kLongChunkSets;                                       \
    const int fn = min(kLongChunkSets, L.n_sets - fset0) * 8 * 64;                    \
    _Pragma("unroll") for (int j = 0; j < kPer; ++j) {                                \
      const int i = j * 256 + tid;                                                    \
      pre[j] = reinterpret_cast<const u32x4 *>(qsrc)[(size_t)fset0 * 8 * 64 + (i < fn ? i : 0)]; \
    }                                                                                 \
    if (tid < kLongChunkRows) {                                                       \
      const int r = fset0 * 16 + tid;                                                 \
      pre_lse = r < L.rows_pad ? lse[sh * L.rows_pad + r] : (AGG ? INFINITY : 0.f);   \
    }                                                                                 \
  }
#define KVMEM_LONG_STORE(BUF)                                                          \
  {                                                                                   \
    _Pragma("unroll") for (int j = 0; j < kPer; ++j)                                 \
        reinterpret_cast<u32x4 *>(sb[(BUF)])[j * 256 + tid] = pre[j];                 \
    if (tid < kLongChunkRows) slse[(BUF)][tid] = pre_lse;                             \
  }

  KVMEM_LONG_FETCH(0)
  KVMEM_LONG_STORE(0)
  for (int chunk = 0; chunk < L.n_chunks; ++chunk) {
    const int buf = chunk & 1;
    __syncthreads();                                    // chunk staged; the other buffer is free
    const bool more = chunk + 1 < L.n_chunks;
    if (more) KVMEM_LONG_FETCH(chunk + 1)
    const int set0 = chunk * kLongChunkSets;
    const int nset = min(kLongChunkSets, L.n_sets - set0);
    for (int cs = 0; cs < nset; ++cs) {
      bf16x8 b[4][2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        b[k][0] = as_bf16x8(sb[buf][(cs * 8 + 2 * k) * 64 + lane]);
        b[k][1] = as_bf16x8(sb[buf][(cs * 8 + 2 * k + 1) * 64 + lane]);
      }
      // the shift of this lane's row enters as the accumulator's initial value,
      // so the products come out as s - shift: STATS, the bound |q~| kmax of a
      // full tile (0 otherwise); AGG, the row's lse (+inf for padding rows)
      const float shift = AGG ? slse[buf][cs * 16 + col] : (full ? slse[buf][cs * 16 + col] * kmax : 0.f);
      floatx4 d[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        d[m] = floatx4{-shift, -shift, -shift, -shift};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          d[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[4 * m + k]), b[k][0], d[m], 0, 0, 0);
          d[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[4 * m + k]), b[k][1], d[m], 0, 0, 0);
        }
      }
      const int row = (set0 + cs) * 16 + col;          // this lane's query row
      if (!AGG) {
        // the row's (max, sum of 2^(s - max)) over the wavefront's blocks, with
        // the bound standing for the max (v_exp_f32: results below 2^-126
        // flush to zero; a bound so far above a row's scores that its sum
        // falls below 2^-60 sends the set down the exact path)
        float mx = shift, sum = 0.f;
        bool exact = !full;
        if (full) {
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(d[m][i]);
          sum = sum_xor16(sum);
          sum = sum_xor32(sum);
          if (__ballot(!(sum >= 0x1p-60f)) != 0) {       // rare: the products again, unshifted
            exact = true;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              d[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                d[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[4 * m + k]), b[k][0], d[m], 0, 0, 0);
                d[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[4 * m + k]), b[k][1], d[m], 0, 0, 0);
              }
            }
          }
        }
        if (exact) {
          mx = -INFINITY;
          sum = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = (vmask >> (4 * m + i)) & 1 ? fmaxf(mx, d[m][i]) : mx;
          mx = max_xor16(mx);
          mx = max_xor32(mx);
          if (mx != -INFINITY) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
              for (int i = 0; i < 4; ++i) sum += (vmask >> (4 * m + i)) & 1 ? __builtin_amdgcn_exp2f(d[m][i] - mx) : 0.f;
          }
          sum = sum_xor16(sum);
          sum = sum_xor32(sum);
        }
        if (qq == 0) sst[wave][cs * 16 + col] = make_float2(mx, sum);
        if (scores != nullptr && row < L.n_rows) {
          // optional score output, natural-log units: scores[s][t][query head][block]
          const int t = row / g.G, gg = row % g.G;
          float *dst = scores + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * g.max_blocks;
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((vmask >> (4 * m + i)) & 1) dst[tile * kIdxTile + 16 * m + 4 * qq + i] = (d[m][i] + (exact ? 0.f : shift)) * kLn2;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[4 * m + i] += __builtin_amdgcn_exp2f(d[m][i]);
      }
    }
    if (more) KVMEM_LONG_STORE(buf ^ 1)
    if (!AGG) {
      __syncthreads();                                  // the 4 wavefronts' row statistics
      if (tid < nset * 16) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sst[w][tid].x);
        float S = 0.f;
        if (M != -INFINITY) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if (sst[w][tid].x != -INFINITY) S += sst[w][tid].y * exp2f(sst[w][tid].x - M);
        }
        part[(sh * L.rows_pad + set0 * 16 + tid) * L.n_groups + grp] = make_float2(M, S);
      }
    }
  }
  if (AGG) {
    // sum each block over the 16 lanes (rows) of its 16-lane row; all lanes get it
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = acc[i];
      v += dpp_f32<kDppXor1>(v);
      v += dpp_f32<kDppXor2>(v);
      v += dpp_f32<kDppMirror8>(v);
      v += dpp_f32<kDppMirror16>(v);
      acc[i] = v;
    }
    if (col == 0) {
      float *dst = A + sh * g.max_blocks;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((vmask >> (4 * m + i)) & 1) dst[tile * kIdxTile + 16 * m + 4 * qq + i] = acc[4 * m + i];
    }
  }
}

#undef KVMEM_LONG_FETCH
#undef KVMEM_LONG_STORE

// lse[row] = M + log2(sum_g S_g 2^(M_g - M)) over the row's block-group
// partials, M = max_g M_g; padding rows get +inf.  One wavefront per row,
// partials folded in a fixed order (lane-strided, then a fixed tree).
__global__ __launch_bounds__(256) void k_long_lse(const float2 *__restrict__ part, float *__restrict__ lse,
                                                  SessI32 n_blocks, int s0, int n_sess, ScoreGeom g, LongGeom L) {
  const int lane = threadIdx.x & 63;
  const long gid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gid >= (long)n_sess * g.Hkv * L.rows_pad) return;
  const int row = (int)(gid % L.rows_pad);
  const long shl = gid / L.rows_pad;                    // (session in launch) * Hkv + h
  const int sl = (int)(shl / g.Hkv);
  const size_t sh = (size_t)(s0 + sl) * g.Hkv + shl % g.Hkv;
  const int ng = (n_blocks.v[sl] + kLongBlocks - 1) / kLongBlocks;
  const float2 *p = part + (sh * L.rows_pad + row) * L.n_groups;
  float M = -INFINITY, S = 0.f;
  for (int i = lane; i < ng; i += 64) {
    const float2 v = p[i];
    if (v.x == -INFINITY) continue;
    const float mn = fmaxf(M, v.x);
    S = S * exp2f(M - mn) + v.y * exp2f(v.x - mn);
    M = mn;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float Mo = shfl_xor_f(M, off), So = shfl_xor_f(S, off);
    const float mn = fmaxf(M, Mo);
    if (mn != -INFINITY) {
      S = (M == -INFINITY ? 0.f : S * exp2f(M - mn)) + (Mo == -INFINITY ? 0.f : So * exp2f(Mo - mn));
      M = mn;
    }
  }
  if (lane == 0) lse[sh * L.rows_pad + row] = (row < L.n_rows && S > 0.f) ? M + log2f(S) : INFINITY;
}

LongGeom long_geom(const ScoreGeom &g) {
  LongGeom L;
  L.n_rows = g.Tq * g.G;
  L.n_sets = (L.n_rows + 15) / 16;
  L.n_chunks = (L.n_sets + kLongChunkSets - 1) / kLongChunkSets;
  L.rows_pad = 16 * L.n_sets;
  L.n_groups = (g.max_blocks + kLongBlocks - 1) / kLongBlocks;
  return L;
}

}  // namespace

LongScratch long_scratch_layout(int S, int Hkv, int T, int G, int max_blocks) {
  ScoreGeom g;
  g.Tq = T;
  g.G = G;
  g.Hkv = Hkv;
  g.max_blocks = max_blocks;
  const LongGeom L = long_geom(g);
  LongScratch r;
  r.qf_bytes = (size_t)S * Hkv * L.n_sets * 8 * 64 * sizeof(uint4);
  r.part_bytes = (size_t)S * Hkv * L.rows_pad * L.n_groups * sizeof(float2);
  r.lse_bytes = (size_t)S * Hkv * L.rows_pad * sizeof(float);
  return r;
}

hipError_t launch_score_long(const void *index, const void *q, const float *qw, float eps, uint4 *qf, float2 *part,
                             float *lse, float *A, float *scores_opt, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  if (max_nb == 0) return hipSuccess;
  const LongGeom L = long_geom(g);
  // the rows' |q~| go into the lse array, which the statistics pass reads
  // and k_long_lse then overwrites
  hipLaunchKernelGGL(k_long_qprep, dim3((unsigned)(g.Hkv * L.n_sets), (unsigned)n_sess), dim3(64), 0, st,
                     (const uint16_t *)q, qw, eps, qf, lse, s0, g, L.n_sets);
  const dim3 grid((unsigned)((max_nb + kLongBlocks - 1) / kLongBlocks), (unsigned)g.Hkv, (unsigned)n_sess);
  hipLaunchKernelGGL(k_long_pass<false>, grid, dim3(256), 0, st, (const uint16_t *)index, (const uint4 *)qf, part,
                     (const float *)lse, (float *)nullptr, scores_opt, n_blocks, s0, g, L);
  const long rows = (long)n_sess * g.Hkv * L.rows_pad;
  hipLaunchKernelGGL(k_long_lse, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, (const float2 *)part, lse,
                     n_blocks, s0, n_sess, g, L);
  hipLaunchKernelGGL(k_long_pass<true>, grid, dim3(256), 0, st, (const uint16_t *)index, (const uint4 *)qf,
                     (float2 *)nullptr, (const float *)lse, A, (float *)nullptr, n_blocks, s0, g, L);
  return hipGetLastError();
}

}  // namespace kvmem
