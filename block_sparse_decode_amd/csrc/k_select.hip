// Budgeted top-k block selection plus the recent blocks, per (session, KV head).
//
// KVMem concatenates the selected KV within the block budget (reproduction
// README, 'Core equation'), and its recent-only control shares that budget
// (README, 'Local reproduction').  Here: the k_eff candidates with the largest
// aggregated score A (ties to the lower block index) are listed in ascending
// block order, then the recent blocks, then -1 padding.
//
// One 1024-thread workgroup per (session, KV head).  A >= 0, so its fp32 bit
// patterns order like the values; an MSB-first radix select with 8-bit digits
// (four histogram passes in LDS, the digit found by a one-wavefront suffix scan)
// yields the exact k-th largest key t and how many elements equal to t are
// taken.  A final ascending sweep keeps every key > t plus the first such ties,
// placing each kept block by two block-wide prefix counts (wavefront ballots +
// per-wave totals in LDS), so the output is already sorted and deterministic.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float *__restrict__ A, int32_t *__restrict__ view_blocks,
                                                       TopkMeta meta, int s0, int Hkv, int max_blocks, int n_list) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t cnt_a[kTopkWaves];
  __shared__ uint32_t cnt_b[kTopkWaves];
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

  uint32_t thr = 0, krem = 0;
  if (k > 0 && !take_all) {
    uint32_t prefix = 0;
    krem = (uint32_t)k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += kTopkThreads) {
        const uint32_t u = __float_as_uint(a[i]);
        if (pass == 0 || (u >> (shift + 8)) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // lane L owns bins 255-4L .. 252-4L (descending); exclusive scan over lanes
        uint32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = hist[255 - 4 * lane - j];
        const uint32_t tot = c[0] + c[1] + c[2] + c[3];
        uint32_t incl = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t v = __shfl_up(incl, off, 64);
          if (lane >= off) incl += v;
        }
        uint32_t before = incl - tot;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (before < krem && krem <= before + c[j]) {
            sh_digit = 255u - 4u * lane - j;
            sh_above = before;
          }
          before += c[j];
        }
      }
      __syncthreads();
      prefix = (prefix << 8) | sh_digit;
      krem -= sh_above;
      __syncthreads();
    }
    thr = prefix;
  }

  if (k > 0) {
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t run_sel = 0, run_eq = 0;
    for (int base = 0; base < nc; base += kTopkThreads) {
      const int i = base + tid;
      const bool valid = i < nc;
      const uint32_t u = valid ? __float_as_uint(a[i]) : 0u;
      const bool gt = valid && (take_all || u > thr);
      const bool eq = valid && !take_all && u == thr;
      const uint64_t beq = __ballot(eq);
      if (lane == 0) cnt_a[wave] = popc64(beq);
      __syncthreads();
      uint32_t off_eq = 0, tot_eq = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) {
        const uint32_t c = cnt_a[w];
        off_eq += (w < wave) ? c : 0u;
        tot_eq += c;
      }
      const uint32_t eq_rank = run_eq + off_eq + popc64(beq & lt);
      const bool sel = gt || (eq && eq_rank < krem);
      const uint64_t bsel = __ballot(sel);
      if (lane == 0) cnt_b[wave] = popc64(bsel);
      __syncthreads();
      uint32_t off_sel = 0, tot_sel = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) {
        const uint32_t c = cnt_b[w];
        off_sel += (w < wave) ? c : 0u;
        tot_sel += c;
      }
      const uint32_t pos = run_sel + off_sel + popc64(bsel & lt);
      if (sel && pos < (uint32_t)k) out[pos] = i;
      run_sel += tot_sel;
      run_eq += tot_eq;
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
