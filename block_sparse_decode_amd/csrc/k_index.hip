// Mean-K index build: one index row per (session, complete block, KV head).
//
// KVMem scores each 32-token block through an index vector k_bar_b (reproduction
// README, 'Core equation'), the position-independent mean of the block's pre-RoPE
// keys (KVMem review, 'Summary').  The kernel streams the K pool once: every
// (block, head) tile is 32 x 128 contiguous elements; 16 lanes own one tile, each
// lane 8 dimensions, and walk the 32 tokens with 16-byte loads (a wavefront reads
// four 256-byte rows per instruction).  Sums are kept in fp64, so the mean of 32
// bf16 or fp32 keys is exact before the single rounding to the storage type.
// Rows are written in the index's tiled layout (16-byte word w of 64
// consecutive blocks contiguous), which the scorer reads fully coalesced.
// A launch covers blocks [first_block, n_blocks) of each session: the whole
// history, or only the blocks completed since the last update.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kJobsPerWG = 16;   // (block, head) tiles per 256-thread workgroup

template <typename T>
struct Ld8;

template <>
struct Ld8<uint16_t> {  // 8 bf16 -> 8 doubles
  static __device__ __forceinline__ void add(const uint16_t *p, double (&acc)[8]) {
    const uint4 w = load_nt16(p);
    const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] += (double)bf16_lo(e[k]);
      acc[2 * k + 1] += (double)bf16_hi(e[k]);
    }
  }
  // dims [8*j, 8*j + 8) of row r of a tile: word j
  static __device__ __forceinline__ uint16_t *at(uint16_t *tile, int r, int j) { return tile + (j * kIdxTile + r) * 8; }
  static __device__ __forceinline__ void store(uint16_t *tile, int r, int j, const double (&m)[8]) {
    uint4 w;
    w.x = f64_to_bf16(m[0]) | (f64_to_bf16(m[1]) << 16);
    w.y = f64_to_bf16(m[2]) | (f64_to_bf16(m[3]) << 16);
    w.z = f64_to_bf16(m[4]) | (f64_to_bf16(m[5]) << 16);
    w.w = f64_to_bf16(m[6]) | (f64_to_bf16(m[7]) << 16);
    *reinterpret_cast<uint4 *>(at(tile, r, j)) = w;
  }
  static __device__ __forceinline__ void zero(uint16_t *tile, int r, int j) {
    *reinterpret_cast<uint4 *>(at(tile, r, j)) = make_uint4(0, 0, 0, 0);
  }
};

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
  dim3 grid((unsigned)(((long)max_nb + kJobsPerWG - 1) / kJobsPerWG * Hkv), (unsigned)n_sess);
  if (bf16)
    hipLaunchKernelGGL(k_build_index<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)k_pool, table,
                       (uint16_t *)index, dev_err, first_block, n_blocks, s0, Hkv, max_blocks, n_pages);
  else
    hipLaunchKernelGGL(k_build_index<float>, grid, dim3(256), 0, st, (const float *)k_pool, table,
                       (float *)index, dev_err, first_block, n_blocks, s0, Hkv, max_blocks, n_pages);
  return hipGetLastError();
}

}  // namespace kvmem
