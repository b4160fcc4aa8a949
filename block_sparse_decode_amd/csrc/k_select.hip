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
// keys held in registers, thread t owning the 32 consecutive keys 32t .. 32t+31
// of a tile; a tile that covers all candidates is loaded once for the whole
// kernel.  The exact k-th largest key t and the number of keys equal to t that
// are taken come from an MSB-first radix select whose digits start at the
// highest bit in which the candidates differ (found by an AND/OR reduction
// first): A spans few binades, so digits taken from the top of the word would
// put nearly all keys in a handful of bins and serialise the LDS histogram
// atomics.  Ordered compaction: per thread the counts of keys above t and equal
// to t, one block-wide scan of both (packed), then each thread writes its kept
// blocks in index order; the output is ascending and deterministic.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kEPT = 32;                              // keys per thread per tile
constexpr int kTile = kTopkThreads * kEPT;            // 32768 keys
constexpr int kBins = 2048;
constexpr uint32_t kNoKey = 0xffffffffu;              // above every finite non-negative key

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
  const int i0 = base + threadIdx.x * kEPT;
  if (i0 + kEPT <= nc && ((reinterpret_cast<uintptr_t>(a + i0) & 15) == 0)) {
#pragma unroll
    for (int j = 0; j < kEPT; j += 4) {
      const uint4 w = *reinterpret_cast<const uint4 *>(a + i0 + j);
      key[j] = w.x; key[j + 1] = w.y; key[j + 2] = w.z; key[j + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kEPT; ++j) key[j] = i0 + j < nc ? __float_as_uint(a[i0 + j]) : kNoKey;
  }
}

// Workgroup-wide AND / OR of one value per thread.
__device__ __forceinline__ void block_and_or(uint32_t &vand, uint32_t &vor, uint32_t *wa, uint32_t *wo) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    vand &= (uint32_t)__shfl_xor((int)vand, off, 64);
    vor |= (uint32_t)__shfl_xor((int)vor, off, 64);
  }
  if (lane == 0) {
    wa[wave] = vand;
    wo[wave] = vor;
  }
  __syncthreads();
  vand = ~0u;
  vor = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    vand &= wa[w];
    vor |= wo[w];
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float *__restrict__ A, int32_t *__restrict__ view_blocks,
                                                       TopkMeta meta, int s0, int Hkv, int max_blocks, int n_list) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wsum[kTopkWaves];
  __shared__ uint32_t wand[kTopkWaves];
  __shared__ uint32_t sh_digit, sh_above;

  const int sl = blockIdx.y;
  const int s = s0 + sl;
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
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
    // bits in which the candidates differ: the select only has to decide those
    uint32_t vand = ~0u, vor = 0u;
#pragma unroll 1
    for (int tile = 0; tile < n_tiles; ++tile) {
      if (n_tiles > 1) load_tile(a, nc, tile * kTile, key);
#pragma unroll
      for (int j = 0; j < kEPT; ++j)
        if (key[j] != kNoKey) {
          vand &= key[j];
          vor |= key[j];
        }
    }
    block_and_or(vand, vor, wand, wsum);
    const uint32_t diff = vand ^ vor;
    uint32_t prefix = vand & ~((diff == 0u) ? 0u : (0xffffffffu >> __clz(diff)));   // common high bits
    krem = (uint32_t)k;
    // digits of up to 11 bits from the highest differing bit down
    int hi = diff == 0u ? -1 : 31 - __clz(diff);
#pragma unroll 1
    while (hi >= 0) {
      const int bits = hi + 1 < 11 ? hi + 1 : 11;
      const int shift = hi + 1 - bits;
      const uint32_t mask = (1u << bits) - 1u;
      const uint32_t hmask = (hi == 31) ? 0u : ~((2u << hi) - 1u);   // bits above the digit
      for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll 1
      for (int tile = 0; tile < n_tiles; ++tile) {
        if (n_tiles > 1) load_tile(a, nc, tile * kTile, key);
#pragma unroll
        for (int j = 0; j < kEPT; ++j) {
          const uint32_t u = key[j];
          if (u != kNoKey && (u & hmask) == prefix) atomicAdd(&hist[(u >> shift) & mask], 1u);
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
      prefix |= (sh_digit & mask) << shift;
      krem -= sh_above;
      __syncthreads();
      hi = shift - 1;
    }
    thr = prefix;
  }

  if (k > 0) {
    uint32_t run_gt = 0, run_eq = 0;
#pragma unroll 1
    for (int tile = 0; tile < n_tiles; ++tile) {
      if (n_tiles > 1) load_tile(a, nc, tile * kTile, key);
      // keys above the threshold and ties, per thread, in one packed scan
      uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
      for (int j = 0; j < kEPT; ++j) {
        const uint32_t u = key[j];
        const bool valid = u != kNoKey;
        n_gt += valid && (take_all || u > thr) ? 1u : 0u;
        n_eq += valid && !take_all && u == thr ? 1u : 0u;
      }
      uint32_t tot;
      const uint32_t ex = block_excl_scan((n_eq << 16) | n_gt, wsum, tot);
      const uint32_t gt_before = run_gt + (ex & 0xffffu), eq_before = run_eq + (ex >> 16);
      uint32_t eq_rank = eq_before;
      uint32_t pos = gt_before + (eq_before < krem ? eq_before : krem);
      const int base = tile * kTile + tid * kEPT;
#pragma unroll
      for (int j = 0; j < kEPT; ++j) {
        const uint32_t u = key[j];
        if (u == kNoKey) continue;
        bool sel;
        if (take_all || u > thr) {
          sel = true;
        } else if (u == thr) {
          sel = eq_rank < krem;
          ++eq_rank;
        } else {
          sel = false;
        }
        if (sel) {
          if (pos < (uint32_t)k) out[pos] = base + j;
          ++pos;
        }
      }
      run_gt += tot & 0xffffu;
      run_eq += tot >> 16;
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
