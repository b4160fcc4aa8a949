// Block scoring on the matrix cores, for query chunks of several tokens.
//
// With T query tokens per step every KV head scores its blocks against T * G
// query rows (the per-head softmax of the reproduction README,
// '2026-09-08 validation correction', is taken per query token and head), so
// scoring is a real dense contraction: S = index_tile (64 blocks x 128) * Q^T.
// The index tile is the A operand of v_mfma_f32_16x16x32_bf16 as it sits in
// HBM (bf16, exact); the normalised query rows q~/sqrt(d) (fp32) are split into
// bf16 hi + lo parts and both are accumulated into the same fp32 result, which
// keeps ~16 significant bits of the query, the same as an fp32 FMA product
// with a bf16 index element would need.
//
// k_score_mfma: one wavefront per run of (row group, head, index tile) items;
//               builds the query operands itself when a key starts, and
//               writes the scores and per-row softmax statistics in the same
//               form as the vector-ALU scorer, so the same aggregation kernel
//               follows.
// k_score_r8:   at most 8 query rows per KV head (the T = 1 decode step with
//               G <= 8): one wavefront per run of up to four index tiles.  The
//               8 rows' hi and lo parts form one 16-column B operand (hi in
//               columns 0..7, lo in 8..15) and the two halves of the product
//               are added with one DPP rotation, so a tile is 16 products.  A
//               wavefront keeps two whole 16 KiB tiles in flight: the registers
//               of a tile take the tile after next as soon as its products are
//               issued, so the scoring of one tile overlaps the loads of the
//               next two, where the vector-ALU GEMV for the same 8 rows is
//               bound by its FMAs and their overlap with the loads.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kMfmaRowGroup = 32;   // query rows per pass over the index: two 16-column operand sets

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4 *>(p);
  const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = bf16_lo(e[k]);
    x[2 * k + 1] = bf16_hi(e[k]);
  }
}

// The 16 A-operand words of a 64-block index tile: a.w[4m + c] is word
// 4c + qq of block 16m + col (dims 32c + 8qq .. + 7), i.e. A rows = blocks
// 16m .. 16m + 15 and k = dims 32c .. 32c + 31.  Each load reads four
// contiguous 256-byte runs of the tiled index.
struct TileA {
  uint4 w[16];
};
__device__ __forceinline__ void load_tile_a(TileA &a, const uint16_t *tile, int lane) {
  const int qq = lane >> 4, col = lane & 15;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      a.w[4 * m + c] = load_nt16(tile + ((4 * c + qq) * kIdxTile + 16 * m + col) * 8);
}

// The same 16 words through a buffer resource over the one tile: the tile's
// address stays in scalar registers (each lane adds only its own offset), and
// a resource of no records (`valid` false) answers zeros without a memory
// access, which keeps a look-ahead past the last tile free.
constexpr int kRawBufferWord3 = 0x00020000;   // resource word 3: 32-bit data format (raw byte offsets)
constexpr int kNtLoad = 2;                     // cache policy of the loads: non-temporal (streamed once)
__device__ __forceinline__ void load_tile_a_buf(TileA &a, const uint16_t *tile, bool valid, int lane) {
  const int qq = lane >> 4, col = lane & 15;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void *)tile, (short)0, valid ? kIdxTile * kD * 2 : 0, kRawBufferWord3);
  const int v = (qq * kIdxTile + col) * 16;              // bytes: word qq of block col
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c)                          // + word 4c (c * 4096 bytes) of block 16m + col
      a.w[4 * m + c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, v + m * 256, c * 4096, kNtLoad));
}

// Scores of the T * G query rows of a row group against every index row, on
// the matrix cores.  Work items and statistics slots are those of the
// vector-ALU scorer (ScoreSplit, rows per group = 32).  Per item the wavefront
// computes D[cs][m] = A(blocks 16m..) * B(rows 16cs..): lane (qq, col) holds
// the scores of blocks 16m + 4qq + i, i < 4, for row 16cs + col.  Running
// per-lane softmax statistics of its row are merged over the four lanes of a
// row at the end of each key.  A key's operands are built from its query
// words before any of its tiles is requested (the words arrive quickly while
// the memory system is idle, and the registers they held are free again),
// then its first two tiles go out together, and each tile's registers take
// the tile after next as soon as its products are done (two tiles in flight).
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_score_mfma(const uint16_t *__restrict__ index, const uint16_t *__restrict__ q,
                                                   const float *__restrict__ qw, float eps,
                                                   float *__restrict__ scores, float2 *__restrict__ part,
                                                   uint32_t *__restrict__ zero, int n_zero,
                                                   SessI32 n_blocks, int s0, ScoreGeom g, ScoreSplit sp) {
  const int lane = threadIdx.x;
  const int qq = lane >> 4, col = lane & 15;
  for (int i = blockIdx.x * 64 + lane; i < n_zero; i += gridDim.x * 64) zero[i] = 0u;
  const int n_rows = g.Tq * g.G;
  const int total = sp.n_sess * g.Hkv * sp.n_rg * sp.ntl;
  const int i0 = blockIdx.x * sp.per;                   // < total (grid = ceil(total / per))
  const int i1 = min(total, i0 + sp.per);
  const bool vec = (g.max_blocks & 3) == 0 && (((uintptr_t)scores) & 15) == 0;

  int key, key_r0;
  bf16x8 b[2][4][2];                                    // [cs][c][hi, lo]
  size_t row_id[2];
  bool row_ok[2];
  float m[2], l[2];
  uint4 qraw[2][4];                                     // the key's query words: row 16cs + col, dims 32k + 8qq ..
  float4 wraw[4][2];                                    // the norm weights of the same dims

  auto tile_of = [&](int item) {
    const ScoreItem it = decode_score_item(item, sp, g.Hkv, n_blocks);
    return index + ((size_t)((s0 + it.sl) * g.Hkv + it.h) * g.n_tiles + it.t) * (size_t)(kIdxTile * kD);
  };

  auto flush = [&]() {
    const int slot = blockIdx.x - score_slot0(key, sp);
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      float M = fmaxf(m[cs], shfl_xor_f(m[cs], 16));
      M = fmaxf(M, shfl_xor_f(M, 32));
      float x = m[cs] == -INFINITY ? 0.f : l[cs] * __expf(m[cs] - M);
      x += shfl_xor_f(x, 16);
      x += shfl_xor_f(x, 32);
      if (qq == 0 && row_ok[cs]) part[row_id[cs] * g.slot_stride + slot] = make_float2(M, x);
    }
  };

  // A key's rows (rows past T * G read row 0 and get zero operands) and the
  // loads of their words and weights.
  auto load_key = [&](const ScoreItem &c) {
    key = c.key;
    key_r0 = c.r0;
    const int s = s0 + c.sl;
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      const int r = c.r0 + cs * 16 + col;
      row_ok[cs] = r < n_rows;
      const int rr = row_ok[cs] ? r : 0;
      row_id[cs] = ((size_t)s * g.Tq + rr / g.G) * g.Hq + (size_t)c.h * g.G + rr % g.G;
      m[cs] = -INFINITY;
      l[cs] = 0.f;
      const uint16_t *src = q + row_id[cs] * kD + 8 * qq;
#pragma unroll
      for (int k = 0; k < 4; ++k) qraw[cs][k] = *reinterpret_cast<const uint4 *>(src + 32 * k);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wraw[k][0] = reinterpret_cast<const float4 *>(qw + 32 * k + 8 * qq)[0];
      wraw[k][1] = reinterpret_cast<const float4 *>(qw + 32 * k + 8 * qq)[1];
    }
  };

  // B operands of a key: lane (qq, col) holds dims 32k + 8qq .. + 7 of query
  // row r0 + 16cs + col, as q~/sqrt(d) split into bf16 hi and lo.  The row's
  // mean square is summed over the four lanes that share it.
  auto build_key = [&]() {
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t e[4] = {qraw[cs][k].x, qraw[cs][k].y, qraw[cs][k].z, qraw[cs][k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = bf16_lo(e[j]), x1 = bf16_hi(e[j]);
          ss += x0 * x0;
          ss += x1 * x1;
        }
      }
      ss += shfl_xor_f(ss, 16);
      ss += shfl_xor_f(ss, 32);
      const float rs = row_ok[cs] ? (1.0f / sqrtf(ss * (1.0f / kD) + eps)) * 0.08838834764831845f : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t e[4] = {qraw[cs][k].x, qraw[cs][k].y, qraw[cs][k].z, qraw[cs][k].w};
        const float w[8] = {wraw[k][0].x, wraw[k][0].y, wraw[k][0].z, wraw[k][0].w,
                            wraw[k][1].x, wraw[k][1].y, wraw[k][1].z, wraw[k][1].w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t h0, l0, h1, l1;
          split_hi_lo(bf16_lo(e[j]) * rs * w[2 * j], h0, l0);
          split_hi_lo(bf16_hi(e[j]) * rs * w[2 * j + 1], h1, l1);
          hw[j] = h0 | (h1 << 16);
          lw[j] = l0 | (l1 << 16);
        }
        b[cs][k][0] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
        b[cs][k][1] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
    }
  };

  auto compute = [&](const TileA &a, int item) {
    const ScoreItem c = decode_score_item(item, sp, g.Hkv, n_blocks);
    if (c.t * kIdxTile >= c.nb) return;                 // tile past this session's history
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
      if (key_r0 + cs * 16 >= n_rows) break;            // operand set wholly past the rows
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.w[4 * mm + k]), b[cs][k][0], d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.w[4 * mm + k]), b[cs][k][1], d, 0, 0, 0);
        }
        if (row_ok[cs]) {
          const int bb = c.t * kIdxTile + 16 * mm + 4 * qq;
          float *dst = scores + row_id[cs] * g.max_blocks + bb;
          if (vec && bb + 3 < c.nb) {
            *reinterpret_cast<floatx4 *>(dst) = d;     // 16-byte aligned
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (bb + i < c.nb) dst[i] = d[i];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (bb + i < c.nb) {
              const float dd = d[i] - m[cs];
              const float e = __expf(-fabsf(dd));
              l[cs] = dd > 0.f ? fmaf(l[cs], e, 1.f) : l[cs] + e;
              m[cs] = fmaxf(m[cs], d[i]);
            }
          }
        }
      }
    }
  };

  // One segment per key in the range: the key's operands, then its tiles
  // with two in flight.  Past the last item the look-ahead loads from an
  // empty resource: the loads stay unconditional (so every wait counts
  // exactly) without touching memory.
  for (int it = i0; it < i1;) {
    const ScoreItem c0 = decode_score_item(it, sp, g.Hkv, n_blocks);
    const int end = min(i1, (c0.key + 1) * sp.ntl);
    TileA ta, tb;
    load_key(c0);
    build_key();
    load_tile_a_buf(ta, tile_of(it), true, lane);
    load_tile_a_buf(tb, tile_of(min(it + 1, end - 1)), it + 1 < end, lane);
    while (true) {
      compute(ta, it);
      if (++it >= end) break;
      load_tile_a_buf(ta, tile_of(min(it + 1, end - 1)), it + 1 < end, lane);
      compute(tb, it);
      if (++it >= end) break;
      load_tile_a_buf(tb, tile_of(min(it + 1, end - 1)), it + 1 < end, lane);
    }
    flush();
  }
}

// Scores of at most 8 query rows against NTILE consecutive index tiles of one
// (session, KV head) per wavefront.  Items are (session, KV head, tile)
// (ScoreSplit with rpg = 8, one row group, per = NTILE, NTILE dividing the
// tiles per head), so each wavefront writes one statistics slot per row.
// Lane (qq, col) holds B column col: query row col & 7, dims 32c + 8qq .. +7
// of chunk c, the hi part for col < 8 and the lo part for col >= 8.  D[m]
// holds, for lane (qq, col), blocks 16m + 4qq + i of column col; after adding
// the rotation by 8 lanes, lanes col < 8 hold the full scores of row col.
// Two tiles are in flight: the registers of a multiplied tile take the tile
// after next.
template <int NTILE>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NTILE == 1 ? 4 : 2))) void k_score_r8(
    const uint16_t *__restrict__ index, const uint16_t *__restrict__ q, const float *__restrict__ qw, float eps,
    float *__restrict__ scores, float2 *__restrict__ part, uint32_t *__restrict__ zero, int n_zero,
    SessI32 n_blocks, int s0, ScoreGeom g, ScoreSplit sp) {
  const int lane = threadIdx.x;
  const int qq = lane >> 4, col = lane & 15;
  for (int i = blockIdx.x * 64 + lane; i < n_zero; i += gridDim.x * 64) zero[i] = 0u;
  const ScoreItem it = decode_score_item(blockIdx.x * NTILE, sp, g.Hkv, n_blocks);
  const int s = s0 + it.sl;
  const int n_rows = g.Tq * g.G;
  const int r = col & 7;
  const bool row_ok = r < n_rows;
  const int t = row_ok ? r / g.G : 0, gg = row_ok ? r % g.G : 0;
  const size_t row_id = ((size_t)s * g.Tq + t) * g.Hq + (size_t)it.h * g.G + gg;
  const int slot = blockIdx.x - score_slot0(it.key, sp);
  const int b0 = it.t * kIdxTile;
  if (b0 >= it.nb) {                                   // tiles past this session's history: empty slot
    if (col < 8 && qq == 0 && row_ok) part[row_id * g.slot_stride + slot] = make_float2(-INFINITY, 0.f);
    return;
  }

  // query loads first, then the tiles (vector loads complete in order)
  float x[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c) load8(q + row_id * kD + 32 * c + 8 * qq, x[c]);
  constexpr int NB = NTILE < 2 ? NTILE : 2;   // tiles in flight
  TileA a[NB];
  const uint16_t *tile0 = index + ((size_t)((size_t)s * g.Hkv + it.h) * g.n_tiles + it.t) * (size_t)(kIdxTile * kD);
  // a tile past the history reads the first one (its scores are not used)
  auto tile_ptr = [&](int k) { return b0 + k * kIdxTile < it.nb ? tile0 + (size_t)k * (kIdxTile * kD) : tile0; };
#pragma unroll
  for (int k = 0; k < NB; ++k) load_tile_a(a[k], tile_ptr(k), lane);

  // q~ / sqrt(d): the row's sum of squares over the four lanes holding it
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[c][j] * x[c][j];
  ss = sum_xor32(sum_xor16(ss));
  const float rs = (1.0f / sqrtf(ss * (1.0f / kD) + eps)) * 0.08838834764831845f;   // 1/sqrt(128)
  // columns 0..7 take bf16(y), columns 8..15 take bf16(y - bf16(y))
  const float rsv = row_ok ? rs : 0.f;
  bf16x8 bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float y0 = x[c][j] * rsv * qw[32 * c + 8 * qq + j];
      const float y1 = x[c][j + 1] * rsv * qw[32 * c + 8 * qq + j + 1];
      const uint32_t hi = pack_bf16x2(y0, y1);
      const uint32_t lo = pack_bf16x2(y0 - bf16_lo(hi), y1 - bf16_hi(hi));
      w[j / 2] = col < 8 ? hi : lo;
    }
    bq[c] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
  }

  const bool vec = (g.max_blocks & 3) == 0 && (((uintptr_t)scores) & 15) == 0;
  constexpr float kLog2e = 1.4426950408889634f;
  float Mrun = -INFINITY, Lrun = 0.f;
#pragma unroll
  for (int k = 0; k < NTILE; ++k) {
    const int bt = b0 + k * kIdxTile;
    float sc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[k % NB].w[4 * m + c]), bq[c], d, 0, 0, 0);
      const int b = bt + 16 * m + 4 * qq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = d[i] + dpp_f32<kDppRor8>(d[i]);
        sc[m][i] = b + i < it.nb ? v : -INFINITY;
      }
      if (col < 8 && row_ok && bt < it.nb) {
        float *dst = scores + row_id * g.max_blocks + b;
        if (vec && b + 3 < it.nb) {
          *reinterpret_cast<float4 *>(dst) = make_float4(sc[m][0], sc[m][1], sc[m][2], sc[m][3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (b + i < it.nb) dst[i] = sc[m][i];
        }
      }
    }
    // the freed registers take tile k + NB
    if (k + NB < NTILE) load_tile_a(a[k % NB], tile_ptr(k + NB), lane);
    // the tile's softmax statistics per row: its maximum over the four lanes
    // holding the row, then one exponential per score (log2 units,
    // v_exp_f32), folded into the wavefront's running pair
    float M = -INFINITY;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) M = fmaxf(M, sc[m][i]);
    M = max_xor32(max_xor16(M));
    if (M == -INFINITY) continue;                      // tile past the history (uniform)
    const float Ml = M * kLog2e;
    float L = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) L += __builtin_amdgcn_exp2f(fmaf(sc[m][i], kLog2e, -Ml));
    L = sum_xor32(sum_xor16(L));
    const float Mn = fmaxf(Mrun, M);
    Lrun = Lrun * __builtin_amdgcn_exp2f((Mrun - Mn) * kLog2e) + L * __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
    Mrun = Mn;
  }
  if (col < 8 && qq == 0 && row_ok) part[row_id * g.slot_stride + slot] = make_float2(Mrun, Lrun);
}

constexpr int kMfmaWavesPerSimd = 2;

}  // namespace

hipError_t launch_score_r8(const void *index, const void *q, const float *qw, float eps, float *scores, float2 *part,
                          uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess, const ScoreGeom &g,
                          ScoreSplit *split, hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  split->n_sess = n_sess;
  split->ntl = 0;
  if (max_nb == 0) return hipSuccess;
  ScoreSplit sp;
  sp.n_sess = n_sess;
  sp.rpg = kGemvMaxRows;
  sp.n_rg = 1;
  sp.ntl = idx_tiles(max_nb);
  // four (else two) tiles per wavefront when they divide a head's tiles (a
  // wavefront then never meets two keys); two are in flight at a time
  sp.per = (sp.ntl % 4 == 0) ? 4 : (sp.ntl % 2 == 0) ? 2 : 1;
  *split = sp;
  const int grid = n_sess * g.Hkv * sp.ntl / sp.per;
  if (sp.per == 4)
    hipLaunchKernelGGL(k_score_r8<4>, dim3(grid), dim3(64), 0, st, (const uint16_t *)index, (const uint16_t *)q, qw,
                       eps, scores, part, zero, n_zero, n_blocks, s0, g, sp);
  else if (sp.per == 2)
    hipLaunchKernelGGL(k_score_r8<2>, dim3(grid), dim3(64), 0, st, (const uint16_t *)index, (const uint16_t *)q, qw,
                       eps, scores, part, zero, n_zero, n_blocks, s0, g, sp);
  else
    hipLaunchKernelGGL(k_score_r8<1>, dim3(grid), dim3(64), 0, st, (const uint16_t *)index, (const uint16_t *)q, qw,
                       eps, scores, part, zero, n_zero, n_blocks, s0, g, sp);
  return hipGetLastError();
}

hipError_t launch_score_mfma(const void *index, const void *q, const float *qw, float eps, float *scores,
                             float2 *part, uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, ScoreSplit *split, hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  split->n_sess = n_sess;
  split->ntl = 0;
  if (max_nb == 0) return hipSuccess;
  ScoreSplit sp;
  sp.n_sess = n_sess;
  sp.rpg = kMfmaRowGroup;
  sp.n_rg = (g.Tq * g.G + kMfmaRowGroup - 1) / kMfmaRowGroup;
  sp.ntl = idx_tiles(max_nb);
  static int cus = 0;                                   // compute units (device property)
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  const long total = (long)n_sess * g.Hkv * sp.n_rg * sp.ntl;
  const long target = (long)cus * 4 * kMfmaWavesPerSimd;
  sp.per = (int)((total + target - 1) / target);
  const int grid = (int)((total + sp.per - 1) / sp.per);
  *split = sp;
  hipLaunchKernelGGL(k_score_mfma, dim3(grid), dim3(64), 0, st, (const uint16_t *)index, (const uint16_t *)q, qw, eps,
                     scores, part, zero, n_zero, n_blocks, s0, g, sp);
  return hipGetLastError();
}

}  // namespace kvmem
