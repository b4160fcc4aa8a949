// Budgeted top-k block selection plus the recent blocks, per (session, KV head).
//
// KVMem concatenates the selected KV within the block budget (reproduction
// README, 'Core equation'), and its recent-only control shares that budget
// (README, 'Local reproduction').  Here: the k_eff candidates with the largest
// aggregated score A (ties to the lower block index) are listed in ascending
// block order, then the recent blocks, then -1 padding.
//
// One 1024-thread workgroup per (session, KV head).  A >= 0, so its fp32 bit
// patterns order like the values.  Candidates are processed in tiles of 32768
// keys held in registers (thread t owns keys t, t+1024, ... of the tile, so every
// load instruction is coalesced); a tile that covers all candidates is loaded
// once for the whole kernel.  An MSB-first radix select with 11/11/10-bit digits
// (LDS histograms, the digit found by one block-wide scan over the bins) gives
// the exact k-th largest key t and how many keys equal to t are taken.  The
// ordered compaction then needs two block-wide scans per tile: per (key slot,
// wavefront) counts of ties and of kept keys come from ballots, and one
// exclusive scan over those counts in index order places every kept block, so
// the output is ascending and deterministic.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kEPT = 32;                              // keys per thread per tile
constexpr int kTile = kTopkThreads * kEPT;            // 32768 keys
constexpr int kBins = 2048;
constexpr uint32_t kNoKey = 0xffffffffu;              // above every finite non-negative key

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// Exclusive scan of one value per thread over the whole workgroup (thread order).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wsum, uint32_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t c = wsum[w];
    before += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

__device__ __forceinline__ void load_tile(const float *a, int nc, int base, uint32_t (&key)[kEPT]) {
#pragma unroll
  for (int j = 0; j < kEPT; ++j) {
    const int i = base + j * kTopkThreads + threadIdx.x;
    key[j] = i < nc ? __float_as_uint(a[i]) : kNoKey;
  }
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float *__restrict__ A, int32_t *__restrict__ view_blocks,
                                                       TopkMeta meta, int s0, int Hkv, int max_blocks, int n_list) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t cnt_eq[kEPT * kTopkWaves];
  __shared__ uint32_t cnt_sel[kEPT * kTopkWaves];
  __shared__ uint32_t wsum[kTopkWaves];
  __shared__ uint32_t sh_digit, sh_above;

  const int sl = blockIdx.y;
  const int s = s0 + sl;
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nc = meta.n_cand.v[sl];
  const int k = meta.k_eff.v[sl];
  const int r0 = meta.r_start.v[sl];
  const int nall = meta.n_all.v[sl];
  const float *a = A + ((size_t)s * Hkv + h) * max_blocks;
  int32_t *out = view_blocks + ((size_t)s * Hkv + h) * n_list;
  const bool take_all = k >= nc;
  const int n_tiles = (nc + kTile - 1) / kTile;

  uint32_t key[kEPT];
  if (n_tiles == 1) load_tile(a, nc, 0, key);

  uint32_t thr = 0, krem = 0;
  if (k > 0 && !take_all) {
    uint32_t prefix = 0;
    krem = (uint32_t)k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int bits = pass == 2 ? 10 : 11;
      const uint32_t mask = (1u << bits) - 1u;
      for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll 1
      for (int tile = 0; tile < n_tiles; ++tile) {
        if (n_tiles > 1) load_tile(a, nc, tile * kTile, key);
#pragma unroll
        for (int j = 0; j < kEPT; ++j) {
          const uint32_t u = key[j];
          const bool match = u != kNoKey && (pass == 0 || (u >> (shift + bits)) == prefix);
          if (match) atomicAdd(&hist[(u >> shift) & mask], 1u);
        }
      }
      __syncthreads();
      // bins in descending order: thread t owns bins 2047-2t and 2046-2t
      const uint32_t c0 = hist[kBins - 1 - 2 * tid], c1 = hist[kBins - 2 - 2 * tid];
      uint32_t total;
      const uint32_t before = block_excl_scan(c0 + c1, wsum, total);
      if (before < krem && krem <= before + c0) {
        sh_digit = kBins - 1 - 2 * tid;
        sh_above = before;
      } else if (before + c0 < krem && krem <= before + c0 + c1) {
        sh_digit = kBins - 2 - 2 * tid;
        sh_above = before + c0;
      }
      __syncthreads();
      prefix = (prefix << bits) | (sh_digit & mask);
      krem -= sh_above;
      __syncthreads();
    }
    thr = prefix;
  }

  if (k > 0) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t run_eq = 0, run_sel = 0;
#pragma unroll 1
    for (int tile = 0; tile < n_tiles; ++tile) {
      if (n_tiles > 1) load_tile(a, nc, tile * kTile, key);
      // ties before each key, in index order (slot j, wave, lane)
#pragma unroll
      for (int j = 0; j < kEPT; ++j) {
        const uint64_t b = __ballot(!take_all && key[j] == thr);
        if (lane == 0) cnt_eq[j * kTopkWaves + wave] = popc64(b);
      }
      __syncthreads();
      uint32_t tot_eq;
      {
        const uint32_t c = tid < kEPT * kTopkWaves ? cnt_eq[tid] : 0u;
        const uint32_t ex = block_excl_scan(c, wsum, tot_eq);
        if (tid < kEPT * kTopkWaves) cnt_eq[tid] = ex;
      }
      __syncthreads();
      uint32_t selmask = 0;
#pragma unroll
      for (int j = 0; j < kEPT; ++j) {
        const uint32_t u = key[j];
        const bool eq = !take_all && u == thr;
        const uint64_t b = __ballot(eq);
        const uint32_t eq_rank = run_eq + cnt_eq[j * kTopkWaves + wave] + popc64(b & lt);
        const bool sel = u != kNoKey && (take_all || u > thr || (eq && eq_rank < krem));
        selmask |= sel ? (1u << j) : 0u;
        const uint64_t bs = __ballot(sel);
        if (lane == 0) cnt_sel[j * kTopkWaves + wave] = popc64(bs);
      }
      __syncthreads();
      uint32_t tot_sel;
      {
        const uint32_t c = tid < kEPT * kTopkWaves ? cnt_sel[tid] : 0u;
        const uint32_t ex = block_excl_scan(c, wsum, tot_sel);
        if (tid < kEPT * kTopkWaves) cnt_sel[tid] = ex;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kEPT; ++j) {
        const bool sel = (selmask >> j) & 1u;
        const uint64_t bs = __ballot(sel);
        if (sel) {
          const uint32_t pos = run_sel + cnt_sel[j * kTopkWaves + wave] + popc64(bs & lt);
          if (pos < (uint32_t)k) out[pos] = tile * kTile + j * kTopkThreads + tid;
        }
      }
      run_eq += tot_eq;
      run_sel += tot_sel;
      __syncthreads();
    }
  }
  const int n_rec = nall - r0;
  for (int j = tid; j < n_list - k; j += kTopkThreads) out[k + j] = (j < n_rec) ? r0 + j : -1;
}

}  // namespace

hipError_t launch_topk(const float *A, int32_t *view_blocks, const TopkMeta &meta, int s0, int n_sess,
                       int Hkv, int max_blocks, int n_list, hipStream_t st) {
  dim3 grid((unsigned)Hkv, (unsigned)n_sess);
  hipLaunchKernelGGL(k_topk, grid, dim3(kTopkThreads), 0, st, A, view_blocks, meta, s0, Hkv, max_blocks, n_list);
  return hipGetLastError();
}

}  // namespace kvmem
