// Mean-K index build: one index row per (session, complete block, KV head).
//
// KVMem scores each 32-token block through an index vector k_bar_b (reproduction
// README, 'Core equation'), the position-independent mean of the block's pre-RoPE
// keys (KVMem review, 'Summary').  The kernels stream the K pool once; every
// (block, head) tile is 32 x 128 contiguous elements.  Sums are kept in fp64,
// so the mean of 32 bf16 or fp32 keys is exact before the single rounding to
// the storage type.  Rows are written in the index's tiled layout (16-byte
// word w of 64 consecutive blocks contiguous), which the scorer reads fully
// coalesced.  A launch covers blocks [first_block, n_blocks) of each session:
// the whole history, or only the blocks completed since the last update.
//
// bf16 pools (k_build_index_bf16): a workgroup owns 512 consecutive blocks of
// one head, a wavefront sums one tile at a time with the next tile's loads in
// flight, and the rows collect in LDS and leave as one contiguous run at the
// end of the workgroup (writes spread between the reads cost far more HBM time
// than their 1/32 share of the bytes).  fp32 pools (k_build_index<float>): 16
// lanes per tile, each lane 8 dimensions over the 32 tokens.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kJobsPerWG = 16;   // (block, head) tiles per 256-thread workgroup (fp32 pools)

template <typename T>
struct Ld8;

template <>
struct Ld8<float> {  // 8 fp32 -> 8 doubles
  static __device__ __forceinline__ void add(const float *p, double (&acc)[8]) {
    const float4 a = load_nt16f(p);
    const float4 b = load_nt16f(p + 4);
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
  // dims [8*j, 8*j + 8) of row r of a tile: words 2j and 2j + 1
  static __device__ __forceinline__ float4 *at(float *tile, int r, int w) {
    return reinterpret_cast<float4 *>(tile + (w * kIdxTile + r) * 4);
  }
  static __device__ __forceinline__ void store(float *tile, int r, int j, const double (&m)[8]) {
    *at(tile, r, 2 * j) = make_float4((float)m[0], (float)m[1], (float)m[2], (float)m[3]);
    *at(tile, r, 2 * j + 1) = make_float4((float)m[4], (float)m[5], (float)m[6], (float)m[7]);
  }
  static __device__ __forceinline__ void zero(float *tile, int r, int j) {
    *at(tile, r, 2 * j) = make_float4(0, 0, 0, 0);
    *at(tile, r, 2 * j + 1) = make_float4(0, 0, 0, 0);
  }
};

template <typename T>
__global__ __launch_bounds__(256) void k_build_index(const T *__restrict__ kpool,
                                                     const int32_t *__restrict__ table,
                                                     T *__restrict__ index, int32_t *dev_err,
                                                     SessI32 first_block, SessI32 n_blocks, int s0, int Hkv,
                                                     int max_blocks, int n_pages) {
  const int sl = blockIdx.y;
  const int s = s0 + sl;
  const int lane16 = threadIdx.x & 15;
  // workgroup = (16 consecutive blocks, one head): each 16-byte word of the
  // 16 rows it writes is one contiguous 256-byte run of the tiled index
  const int h = (int)(blockIdx.x % Hkv);
  const long beta = first_block.v[sl] + (long)(blockIdx.x / Hkv) * kJobsPerWG + (threadIdx.x >> 4);
  if (beta >= n_blocks.v[sl]) return;

  T *tile = index + (((size_t)s * Hkv + h) * idx_tiles(max_blocks) + beta / kIdxTile) * (size_t)(kIdxTile * kD);
  const int r = (int)(beta % kIdxTile);
  const int page = table[(size_t)s * max_blocks + beta];
  if (page < 0 || page >= n_pages) {
    dev_flag(dev_err, 1);
    Ld8<T>::zero(tile, r, lane16);
    return;
  }
  const T *src = kpool + ((size_t)page * Hkv + h) * (size_t)(kBT * kD) + lane16 * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
  for (int u = 0; u < kBT; ++u) Ld8<T>::add(src + u * kD, acc);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] *= (1.0 / kBT);   // exact: power of two
  Ld8<T>::store(tile, r, lane16, acc);
}

// ---------------------------------------------------------------------------
// bf16 pools.  Index rows are 1/32 of the bytes the build reads, but written a
// few hundred bytes at a time between the reads they cost far more than their
// share of HBM time (read/write turnarounds).  So a workgroup takes NB
// consecutive blocks of one head, keeps their rows in LDS in the index's tiled
// layout and writes them at the end as one contiguous run.  One wavefront per
// (block, head) tile at a time: lane (tg, c) reads tokens tg + 4j (j < 8),
// dims 8c..8c+7, so each load instruction covers 1 KiB of the tile; the next
// tile's loads are issued before the current one is summed.
// ---------------------------------------------------------------------------
constexpr int kBuildWaves = 4;
constexpr int kBuildGroup = 512;   // blocks per workgroup: 8 tiles, 128 KiB of LDS

// Halving exchange across lane l ^ 16 (ROW32 = false) or l ^ 32 (true) with the
// VALU lane swaps of gfx950: each lane passes the value its partner keeps and
// receives the partner's copy of the value it keeps.  r[0] of the swap holds
// the value of the lane in the even 16-row (lower half), r[1] that of the odd
// row (upper half).
template <bool ROW32>
__device__ __forceinline__ double give_take(double give, double keep, bool low) {
  const uint64_t b = (uint64_t)__double_as_longlong(give);
  const auto lo = ROW32 ? __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false)
                        : __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto hi = ROW32 ? __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false)
                        : __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  const uint64_t t = low ? (((uint64_t)hi[1] << 32) | lo[1]) : (((uint64_t)hi[0] << 32) | lo[0]);
  return keep + __longlong_as_double((long long)t);
}

template <int NB>   // blocks of one head per workgroup, a multiple of kIdxTile
__global__ __launch_bounds__(64 * kBuildWaves) void k_build_index_bf16(
    const uint16_t *__restrict__ kpool, const int32_t *__restrict__ table, uint16_t *__restrict__ index,
    int32_t *dev_err, SessI32 first_block, SessI32 n_blocks, int s0, int Hkv, int max_blocks, int n_pages) {
  static_assert(NB % kIdxTile == 0 && NB % (64 * kBuildWaves) == 0, "NB");
  constexpr int kPer = NB / kBuildWaves;   // blocks per wavefront
  constexpr int kPid = kPer / 64;          // page-id registers per lane
  __shared__ uint32_t rows[NB * kD / 2];   // NB index rows, tiled as in the index
  const int sl = blockIdx.y, s = s0 + sl;
  const int lane = threadIdx.x & 63, c = lane & 15, tg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = (int)(blockIdx.x % Hkv);
  const long b_first = first_block.v[sl], b_end = n_blocks.v[sl];
  // groups start on tile boundaries, so the run a workgroup writes is whole tiles
  const long g0 = (b_first / kIdxTile) * kIdxTile + (long)(blockIdx.x / Hkv) * NB;
  if (g0 >= b_end) return;   // uniform over the workgroup
  const long lo = g0 > b_first ? g0 : b_first, hi = g0 + NB < b_end ? g0 + NB : b_end;
  const long wb = g0 + (long)wv * kPer;
  const int i0 = (int)(lo - wb > 0 ? lo - wb : 0);
  const int i1 = (int)(hi - wb < kPer ? hi - wb : kPer);   // i0 >= i1: nothing for this wavefront

  int pid[kPid];
#pragma unroll
  for (int q = 0; q < kPid; ++q) {
    const int i = q * 64 + lane;
    pid[q] = (i >= i0 && i < i1) ? table[(size_t)s * max_blocks + wb + i] : 0;
  }
  const uint16_t *head = kpool + (size_t)h * (kBT * kD) + tg * kD + c * 8;
  auto page_of = [&](int i) {   // i is wavefront-uniform
    int page = pid[0];
#pragma unroll
    for (int q = 1; q < kPid; ++q)
      if (i / 64 == q) page = pid[q];
    return __builtin_amdgcn_readlane(page, i % 64);
  };
  // every tile issues the same 8 loads (a page outside the pool reads page 0 and
  // is zeroed after the sums), so the waits for a tile never depend on the path
  auto issue = [&](int page, uint4 (&w)[8]) {
    const uint16_t *src = head + (size_t)(page >= 0 && page < n_pages ? page : 0) * Hkv * (kBT * kD);
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = load_nt16(src + 4 * j * kD);
  };
  bool bad = false;
  auto fold = [&](const uint4 (&w)[8], int page, int i) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t e[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += (double)bf16_lo(e[k]);
        acc[2 * k + 1] += (double)bf16_hi(e[k]);
      }
    }
    // fold the four token groups: lanes tg < 2 keep dims 0-3 of the slice, tg >= 2
    // dims 4-7 (exchange with l ^ 32); then even tg keeps the first two of those,
    // odd tg the last two (l ^ 16).  Lane (tg, c) ends with dims 8c + 2tg, 8c + 2tg + 1.
    const bool low32 = tg < 2, low16 = (tg & 1) == 0;
    double h4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) h4[k] = give_take<true>(low32 ? acc[4 + k] : acc[k], low32 ? acc[k] : acc[4 + k], low32);
    double m0 = give_take<false>(low16 ? h4[2] : h4[0], low16 ? h4[0] : h4[2], low16);
    double m1 = give_take<false>(low16 ? h4[3] : h4[1], low16 ? h4[1] : h4[3], low16);
    const bool ok = page >= 0 && page < n_pages;
    bad |= !ok;
    m0 = ok ? m0 * (1.0 / kBT) : 0.0;   // exact scaling: power of two
    m1 = ok ? m1 * (1.0 / kBT) : 0.0;
    const int L = wv * kPer + i;   // row within the group
    rows[(((L / kIdxTile) * 16 + c) * kIdxTile + L % kIdxTile) * 4 + tg] = f64_to_bf16(m0) | (f64_to_bf16(m1) << 16);
  };
  if (i0 < i1) {
    // the next tile's loads are in flight while this one is summed (a deeper
    // look-ahead, two tiles, measured slower)
    uint4 cur[8], nxt[8];
    int pg = page_of(i0);
    issue(pg, cur);
    for (int i = i0; i < i1 - 1; ++i) {
      const int pn = page_of(i + 1);
      issue(pn, nxt);
      __builtin_amdgcn_sched_barrier(0);   // keep the next tile's loads ahead of this tile's waits
      fold(cur, pg, i);
#pragma unroll
      for (int j = 0; j < 8; ++j) cur[j] = nxt[j];
      pg = pn;
    }
    fold(cur, pg, i1 - 1);
  }
  if (bad && lane == 0) dev_flag(dev_err, 1);
  __syncthreads();
  // the group's tiles are consecutive in the index: 16-byte word wi of the LDS
  // copy is word wi of the run; only rows in [lo, hi) are written
  const uint4 *rows4 = reinterpret_cast<const uint4 *>(rows);
  uint16_t *dst = index + (((size_t)s * Hkv + h) * idx_tiles(max_blocks) + g0 / kIdxTile) * (size_t)(kIdxTile * kD);
  for (int wi = threadIdx.x; wi < NB * 16; wi += 64 * kBuildWaves) {
    const long b = g0 + (wi / (16 * kIdxTile)) * kIdxTile + wi % kIdxTile;
    if (b >= lo && b < hi) store_nt16(dst + (size_t)wi * 8, rows4[wi]);
  }
}

}  // namespace

hipError_t launch_build_index(int bf16, const void *k_pool, const int32_t *table, void *index,
                              int32_t *dev_err, const SessI32 &first_block, const SessI32 &n_blocks, int s0,
                              int n_sess, int Hkv, int max_blocks, int n_pages, hipStream_t st) {
  int max_nb = 0;   // most blocks any session has to (re)build
  for (int i = 0; i < n_sess; ++i) {
    const int n = n_blocks.v[i] - first_block.v[i];
    max_nb = n > max_nb ? n : max_nb;
  }
  if (max_nb == 0) return hipSuccess;
  if (bf16) {
    constexpr int NB = kBuildGroup;
    long groups = 0;   // most tile-aligned groups any session spans
    for (int i = 0; i < n_sess; ++i) {
      if (n_blocks.v[i] <= first_block.v[i]) continue;
      const long a = (long)(first_block.v[i] / kIdxTile) * kIdxTile;
      const long g = (n_blocks.v[i] - a + NB - 1) / NB;
      groups = g > groups ? g : groups;
    }
    hipLaunchKernelGGL(k_build_index_bf16<NB>, dim3((unsigned)(groups * Hkv), (unsigned)n_sess),
                       dim3(64 * kBuildWaves), 0, st, (const uint16_t *)k_pool, table, (uint16_t *)index, dev_err,
                       first_block, n_blocks, s0, Hkv, max_blocks, n_pages);
  } else {
    dim3 grid((unsigned)(((long)max_nb + kJobsPerWG - 1) / kJobsPerWG * Hkv), (unsigned)n_sess);
    hipLaunchKernelGGL(k_build_index<float>, grid, dim3(256), 0, st, (const float *)k_pool, table,
                       (float *)index, dev_err, first_block, n_blocks, s0, Hkv, max_blocks, n_pages);
  }
  return hipGetLastError();
}

}  // namespace kvmem
