// GQA aggregation and budgeted selection.
//
// KVMem softmaxes each query head over the blocks and sums the heads of a KV
// group (reproduction README, '2026-09-08 validation correction'), then keeps
// the selected KV within the block budget (README, 'Core equation'); its
// recent-only control shares that budget (README, 'Local reproduction').  Per
// (session, KV head): the k_eff candidates with the largest aggregated score A
// (ties to the lower block index) are listed in ascending block order, then
// the recent blocks, then -1 padding.
//
// k_aggregate: A[b] = sum_rows exp(s[row][b] - M_row) / Z_row for every
//   complete block (1024 blocks per workgroup), and the candidates counted by
//   the top digit of A's bits into the (session, head)'s selection histogram;
//   each chunk's keys are also written grouped by that digit.
// k_topk_chunk: the selection when every session has at most 32768
//   candidates and the histogram is there, one workgroup per aggregation
//   chunk (described with the kernel).
// k_topk: the selection otherwise, one workgroup per (session, head),
//   starting from that histogram when there is one.
//
// Selection of k_topk (select_head), one 1024-thread workgroup.  A >= 0, so its fp32 bit
// patterns order like the values.  Candidates are processed in tiles of 32768
// keys held in registers, thread t owning the 32 consecutive keys 32t .. 32t+31
// of a tile; a tile that covers all candidates is loaded once.  The exact k-th
// largest key t and the number of keys equal to t that are taken come from an
// MSB-first radix select.  When the candidates have already been counted by
// their top digit (bits 30..20), the select starts from those counts and only
// the keys of the boundary bin take part in the remaining passes.  Otherwise
// its digits start at the highest bit in which the candidates differ (found by
// an AND/OR reduction first): A spans few binades, so digits taken from the top
// of the word would put nearly all keys in a handful of bins and serialise the
// LDS histogram atomics.  Ordered compaction: per thread the counts of keys
// above t and equal to t, one block-wide scan of both (packed), then each
// thread places its kept blocks in index order into an LDS window of the list,
// which is written out coalesced; the output is ascending and deterministic.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kEPT = 32;                              // keys per thread per tile
constexpr int kTile = kTopkThreads * kEPT;            // 32768 keys
constexpr int kBins = 2048;
constexpr int kOutLds = 16384;                        // list entries staged in LDS at a time
constexpr uint32_t kNoKey = 0xffffffffu;              // above every finite non-negative key
static_assert(kBins == kSelBins && 31 - kSelShift == 11, "selection histogram digit");
static_assert(kAggChunk == kTopkThreads, "one aggregated block per thread");

struct SelSmem {
  uint32_t hist[kBins];
  uint32_t wsum[kTopkWaves];
  uint32_t wand[kTopkWaves];
  uint32_t digit, above;
  int32_t out[kOutLds];
};

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

// Finds the bin of the k-th largest key from bin counts in descending order:
// thread t owns bins kBins-1-2t and kBins-2-2t.  Sets sm.digit to the bin and
// sm.above to the number of keys in the bins above it.
__device__ __forceinline__ void find_bin(uint32_t c0, uint32_t c1, uint32_t krem, SelSmem &sm) {
  const int tid = threadIdx.x;
  uint32_t total;
  const uint32_t before = block_excl_scan(c0 + c1, sm.wsum, total);
  if (before < krem && krem <= before + c0) {
    sm.digit = kBins - 1 - 2 * tid;
    sm.above = before;
  } else if (before + c0 < krem && krem <= before + c0 + c1) {
    sm.digit = kBins - 2 - 2 * tid;
    sm.above = before + c0;
  }
  __syncthreads();
}

// Selection for one (session, KV head) by the whole workgroup.  a: A of the
// candidates [0, nc); hc: their counts by top digit, or null; out: the head's
// list of n_list entries.
__device__ __forceinline__ void select_head(const float *a, const uint32_t *hc, int32_t *out, int nc, int k, int r0, int nall,
                            int n_list, SelSmem &sm) {
  const int tid = threadIdx.x;
  const bool take_all = k >= nc;
  const int n_tiles = (nc + kTile - 1) / kTile;

  const bool use_hc = hc != nullptr && k > 0 && !take_all;
  // the counts first: the bin search then overlaps the key loads
  const uint32_t c0 = use_hc ? hc[kBins - 1 - 2 * tid] : 0u;
  const uint32_t c1 = use_hc ? hc[kBins - 2 - 2 * tid] : 0u;
  uint32_t key[kEPT];
  if (n_tiles == 1) load_tile(a, nc, 0, key);

  uint32_t thr = 0, krem = 0;
  if (k > 0 && !take_all) {
    uint32_t prefix;
    int hi;
    krem = (uint32_t)k;
    if (use_hc) {
      // the first digit's counts are given
      if (tid == 0) sm.digit = sm.above = 0u;
      find_bin(c0, c1, krem, sm);
      prefix = sm.digit << kSelShift;
      krem -= sm.above;
      hi = kSelShift - 1;
      __syncthreads();
    } else {
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
      block_and_or(vand, vor, sm.wand, sm.wsum);
      const uint32_t diff = vand ^ vor;
      prefix = vand & ~((diff == 0u) ? 0u : (0xffffffffu >> __clz(diff)));   // common high bits
      // digits of up to 11 bits from the highest differing bit down
      hi = diff == 0u ? -1 : 31 - __clz(diff);
    }
#pragma unroll 1
    while (hi >= 0) {
      const int bits = hi + 1 < 11 ? hi + 1 : 11;
      const int shift = hi + 1 - bits;
      const uint32_t mask = (1u << bits) - 1u;
      const uint32_t hmask = (hi == 31) ? 0u : ~((2u << hi) - 1u);   // bits above the digit
      for (int i = tid; i < kBins; i += kTopkThreads) sm.hist[i] = 0;
      __syncthreads();
#pragma unroll 1
      for (int tile = 0; tile < n_tiles; ++tile) {
        if (n_tiles > 1) load_tile(a, nc, tile * kTile, key);
#pragma unroll
        for (int j = 0; j < kEPT; ++j) {
          const uint32_t u = key[j];
          if (u != kNoKey && (u & hmask) == prefix) atomicAdd(&sm.hist[(u >> shift) & mask], 1u);
        }
      }
      __syncthreads();
      find_bin(sm.hist[kBins - 1 - 2 * tid], sm.hist[kBins - 2 - 2 * tid], krem, sm);
      prefix |= (sm.digit & mask) << shift;
      krem -= sm.above;
      __syncthreads();
      hi = shift - 1;
    }
    thr = prefix;
  }

  // list windows of kOutLds entries: positions are recomputed per window
#pragma unroll 1
  for (int w0 = 0; w0 < k; w0 += kOutLds) {
    const uint32_t wn = (uint32_t)min(kOutLds, k - w0);
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
      const uint32_t ex = block_excl_scan((n_eq << 16) | n_gt, sm.wsum, tot);
      const uint32_t gt_before = run_gt + (ex & 0xffffu), eq_before = run_eq + (ex >> 16);
      uint32_t eq_rank = eq_before;
      // list position of the thread's next kept key, relative to the window
      // (wraps above wn while before it)
      uint32_t p = gt_before + (eq_before < krem ? eq_before : krem) - (uint32_t)w0;
      const int base = tile * kTile + tid * kEPT;
#pragma unroll
      for (int j = 0; j < kEPT; ++j) {
        const uint32_t u = key[j];
        const bool valid = u != kNoKey;
        const bool eq = valid && u == thr;
        const bool sel = valid && (take_all || u > thr || (eq && eq_rank < krem));
        eq_rank += eq ? 1u : 0u;
        if (sel && p < wn) sm.out[p] = base + j;
        p += sel ? 1u : 0u;
      }
      run_gt += tot & 0xffffu;
      run_eq += tot >> 16;
    }
    __syncthreads();
    for (int i = tid; i < (int)wn; i += kTopkThreads) out[w0 + i] = sm.out[i];
    __syncthreads();
  }
  const int n_rec = nall - r0;
  for (int j = tid; j < n_list - k; j += kTopkThreads) out[k + j] = (j < n_rec) ? r0 + j : -1;
}

__global__ __launch_bounds__(kTopkThreads) void k_topk(const float *__restrict__ A, const uint32_t *__restrict__ hist,
                                                       int32_t *__restrict__ view_blocks, TopkMeta meta, int s0,
                                                       int Hkv, int max_blocks, int n_list) {
  __shared__ SelSmem sm;
  const int sl = blockIdx.y;
  const int s = s0 + sl;
  const int h = blockIdx.x;
  const uint32_t *hc = hist ? hist + ((size_t)s * Hkv + h) * kSelBins : nullptr;
  select_head(A + ((size_t)s * Hkv + h) * max_blocks, hc, view_blocks + ((size_t)s * Hkv + h) * n_list,
              meta.n_cand.v[sl], meta.k_eff.v[sl], meta.r_start.v[sl], meta.n_all.v[sl], n_list, sm);
}

// ---------------------------------------------------------------------------
// Selection spread over the aggregation chunks: one workgroup per (session,
// KV head, chunk of kAggChunk candidates), thread t owning block
// chunk * kAggChunk + t, when a session has at most kTile candidates.  The
// aggregation left the head's histogram by top digit (bits 30..20 of the key,
// the key being A's bit pattern without the sign bit) and, per chunk, the
// chunk's keys grouped by digit (highest first) with its counts of keys at or
// above every digit.  Every workgroup of a head finds the same exact
// threshold independently, reading only the keys of the boundary digit:
//  1. The boundary bin b0 of the k-th largest key from the histogram (a
//     prefix sum over the bins in descending order).
//  2. Per chunk j: the keys above b0 and in b0 (two counts), and the run of
//     b0's keys in j's grouped keys, fetched as one list in chunk order
//     (held in registers, or in LDS when longer than 8192 keys).
//  3. Two LDS histogram passes over the list fix bits 19..9 and 8..0: the
//     exact threshold key and how many keys equal to it are taken (ties to
//     the lower block index, so to the lower chunk first).
//  4. This chunk's first list position: the keys above b0 in earlier chunks
//     plus their boundary keys taken (counted over the list's earlier
//     chunks).  Its own keys, read from A in block order, are placed by one
//     workgroup scan, which also totals that count (three scans when only
//     some keys equal to the threshold are taken).
// The first chunk's workgroup also writes the recent blocks and the padding.
// ---------------------------------------------------------------------------
constexpr int kMaxSelChunks = kTile / kAggChunk;   // 32
constexpr int kCopyBatch = 8;                      // boundary keys fetched per thread at a time
constexpr uint32_t kKeyMask = 0x7fffffffu;

struct ChunkSmem {
  uint32_t hist[kBins];              // bits 19..9 of the boundary keys
  uint32_t hist2[kBins];             // bits 8..0 of those sharing the threshold's bits 19..9
  uint32_t wsum[kTopkWaves];
  uint32_t digit, above, before_above;
  uint32_t cab[kMaxSelChunks];       // per chunk: keys in bins above b0
  uint32_t cin[kMaxSelChunks];       // per chunk: keys in b0
  uint32_t coff[kMaxSelChunks + 1];  // per chunk: first list position of its b0 keys
  uint32_t list[kTile];
};

// Inclusive prefix sum over the wavefront on the DPP network: shifts by 1, 2,
// 4 and 8 lanes inside each 16-lane row, then row 0 into row 1 and row 2 into
// row 3 (row_bcast:15), then rows 0-1 into rows 2-3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast15, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast31, 0xc, 0xf, false);
  return v;
}

__device__ __forceinline__ uint32_t wave_total(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
}

// Exclusive prefix sum of one value per thread over a 1024-thread workgroup
// (thread order); *total gets the sum.  wsum: kTopkWaves words of LDS.
__device__ __forceinline__ uint32_t wg_excl_scan(uint32_t v, uint32_t *wsum, uint32_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = incl - v, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t c = wsum[w];
    before += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before;
}

// Bin of the krem-th largest key from counts in descending bin order (thread
// t owns bins kBins-1-2t and kBins-2-2t); sets sm.digit and sm.above (keys in
// the bins above it).  The counts must total at least krem.
__device__ __forceinline__ void find_bin_dpp(uint32_t c0, uint32_t c1, uint32_t krem, ChunkSmem &sm) {
  uint32_t total;
  const uint32_t before = wg_excl_scan(c0 + c1, sm.wsum, total);
  if (before < krem && krem <= before + c0) {
    sm.digit = kBins - 1 - 2 * threadIdx.x;
    sm.above = before;
  } else if (before + c0 < krem && krem <= before + c0 + c1) {
    sm.digit = kBins - 2 - 2 * threadIdx.x;
    sm.above = before + c0;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void k_topk_chunk(const float *__restrict__ A,
                                                             const uint32_t *__restrict__ hist,
                                                             const uint32_t *__restrict__ skey,
                                                             const uint16_t *__restrict__ sincl,
                                                             int32_t *__restrict__ view_blocks, TopkMeta meta,
                                                             int s0, int Hkv, int max_blocks, int n_chunks,
                                                             int n_list) {
  __shared__ ChunkSmem sm;
  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int ci = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = meta.n_cand.v[sl], k = meta.k_eff.v[sl];
  const size_t hk = (size_t)s * Hkv + h;
  int32_t *out = view_blocks + hk * n_list;

  if (ci == 0) {
    const int r0 = meta.r_start.v[sl], n_rec = meta.n_all.v[sl] - r0;
    for (int j = tid; j < n_list - k; j += kTopkThreads) out[k + j] = (j < n_rec) ? r0 + j : -1;
  }
  if (k == 0 || ci * kAggChunk >= nc) return;          // (uniform over the workgroup)
  const int b = ci * kAggChunk + tid;
  const bool valid = b < nc;
  if (k >= nc) {                                       // every candidate is taken
    if (valid) out[b] = b;
    return;
  }

  // the histogram's counts and this thread's key
  const uint32_t *hc = hist + hk * kSelBins;
  const uint32_t c0 = hc[kBins - 1 - 2 * tid];
  const uint32_t c1 = hc[kBins - 2 - 2 * tid];
  const uint32_t key = valid ? __float_as_uint(A[hk * max_blocks + b]) & kKeyMask : 0u;
  // the refinement histograms are cleared here, ordered before their use by
  // the barriers below
  for (int i = tid; i < kBins; i += kTopkThreads) {
    sm.hist[i] = 0u;
    sm.hist2[i] = 0u;
  }
  find_bin_dpp(c0, c1, (uint32_t)k, sm);
  const uint32_t b0 = sm.digit;
  uint32_t krem = (uint32_t)k - sm.above;

  // per chunk: keys above b0 and in b0
  const int nch = (nc + kAggChunk - 1) / kAggChunk;
  if (tid < nch) {
    const uint16_t *inc = sincl + (hk * n_chunks + tid) * kSelBins;
    const uint32_t ab = b0 + 1 < (uint32_t)kBins ? inc[b0 + 1] : 0u;
    sm.cab[tid] = ab;
    sm.cin[tid] = inc[b0] - ab;
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t vin = lane < nch ? sm.cin[lane] : 0u;
    const uint32_t vab = lane < ci ? sm.cab[lane] : 0u;
    const uint32_t incl = wave_incl_scan(vin);
    if (lane < nch) sm.coff[lane] = incl - vin;
    if (lane == 63) sm.coff[nch] = incl;               // keys of b0 over the head
    const uint32_t ab_total = wave_total(vab);
    if (lane == 0) sm.before_above = ab_total;
  }
  __syncthreads();
  // b0's keys of every chunk, in chunk order: thread t fetches list
  // positions t + 1024 u.  Up to kCopyBatch * 1024 keys (one batch) stay in
  // registers for the passes below; a longer list is read back from LDS.
  const int nl = (int)sm.coff[nch];
  const bool in_regs = nl <= kCopyBatch * kTopkThreads;
  uint32_t v[kCopyBatch];
  for (int p0 = 0; p0 < nl; p0 += kCopyBatch * kTopkThreads) {
    // every position's chunk first (the last j with coff[j] <= p, coff
    // ascending), then all loads back to back; positions past the list
    // read its last key
    uint32_t src[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      const int p = min(p0 + u * kTopkThreads + tid, nl - 1);
      int j = 0;
#pragma unroll
      for (int step = kMaxSelChunks / 2; step >= 1; step >>= 1) {
        const int jj = min(j + step, nch);               // coff[nch] = nl > p
        j = (int)sm.coff[jj] <= p ? jj : j;
      }
      src[u] = (uint32_t)j * kAggChunk + sm.cab[j] + (uint32_t)p - sm.coff[j];
    }
    const uint32_t *hs = skey + hk * n_chunks * kAggChunk;
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) v[u] = hs[src[u]];
    if (!in_regs) {
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int p = p0 + u * kTopkThreads + tid;
        if (p < nl) sm.list[p] = v[u];
      }
    }
  }
  // visits every listed key once: f(key, list position)
  auto for_each_listed = [&](auto f) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int p = u * kTopkThreads + tid;
        if (p < nl) f(v[u], p);
      }
    } else {
      for (int p = tid; p < nl; p += kTopkThreads) f(sm.list[p], p);
    }
  };
  if (!in_regs) __syncthreads();                       // the list in LDS
  // bits 19..9 of the listed keys
  for_each_listed([&](uint32_t u, int) { atomicAdd(&sm.hist[(u >> 9) & (kBins - 1)], 1u); });
  __syncthreads();
  find_bin_dpp(sm.hist[kBins - 1 - 2 * tid], sm.hist[kBins - 2 - 2 * tid], krem, sm);
  const uint32_t b1 = sm.digit;
  krem -= sm.above;
  // bits 8..0 of the listed keys that share bits 19..9
  for_each_listed([&](uint32_t u, int) {
    if (((u >> 9) & (kBins - 1)) == b1) atomicAdd(&sm.hist2[u & 511u], 1u);
  });
  __syncthreads();
  find_bin_dpp(sm.hist2[kBins - 1 - 2 * tid], sm.hist2[kBins - 2 - 2 * tid], krem, sm);
  const uint32_t b2 = sm.digit;
  krem -= sm.above;                                    // keys equal to the threshold that are taken
  const uint32_t thr = (b0 << kSelShift) | (b1 << 9) | b2;
  const uint32_t n_eq = sm.hist2[b2];

  // This chunk's kept blocks in block order.  Its first list position is
  // the keys above b0 in earlier chunks plus their boundary keys that are
  // kept (the listed keys before position coff[ci]).
  const int lim = (int)sm.coff[ci];
  uint32_t p;
  bool sel;
  if (krem == n_eq) {
    // every key equal to the threshold is kept: one scan, whose low half
    // places this chunk's kept keys and whose high half's total counts the
    // earlier chunks' kept boundary keys (each at most kTile)
    uint32_t c = 0;
    for_each_listed([&](uint32_t u, int q) { c += (q < lim && u >= thr) ? 1u : 0u; });
    sel = valid && key >= thr;
    uint32_t tot;
    const uint32_t ex = wg_excl_scan((c << 16) | (sel ? 1u : 0u), sm.wsum, tot);
    p = sm.before_above + (tot >> 16) + (ex & 0xffffu);
  } else {
    // only the first krem keys equal to the threshold, in block order
    uint32_t g = 0, e = 0;
    for_each_listed([&](uint32_t u, int q) {
      if (q < lim) {
        g += u > thr ? 1u : 0u;
        e += u == thr ? 1u : 0u;
      }
    });
    uint32_t ge;
    wg_excl_scan((e << 16) | g, sm.wsum, ge);          // each count at most kTile / 2 per half
    const uint32_t gt_before = ge & 0xffffu, eq_before = ge >> 16;
    const bool eq = valid && key == thr;
    uint32_t n_eq_chunk, n_sel;
    const uint32_t eq_rank = eq_before + wg_excl_scan(eq ? 1u : 0u, sm.wsum, n_eq_chunk);
    sel = (valid && key > thr) || (eq && eq_rank < krem);
    p = sm.before_above + gt_before + min(eq_before, krem) + wg_excl_scan(sel ? 1u : 0u, sm.wsum, n_sel);
  }
  if (sel && p < (uint32_t)k) out[p] = b;
}

__device__ __forceinline__ float2 merge_ml(float2 a, float2 b) {
  const float M = fmaxf(a.x, b.x);
  if (M == -INFINITY) return make_float2(-INFINITY, 0.f);
  return make_float2(M, a.y * expf(a.x - M) + b.y * expf(b.x - M));
}

constexpr int kAggRowsPerPass = 8;    // rows whose scores a thread holds at once

// One workgroup per (session, KV head, kAggChunk blocks); thread t owns block
// b0 + t.  Rows are taken eight at a time: every thread first requests its
// scores of those rows, then each of eight wavefronts merges the statistics
// slots of one row into the row's max M and 1/Z (each lane folds its slots,
// then one DPP max and one DPP sum over the wavefront), and every thread adds
// exp(s - M) / Z of the rows to its block in row order.  (Holding 16 or 32
// rows per pass measured slower at 32 query rows per KV head.)  The candidates' A are
// counted by top digit in LDS and the non-empty bins added to the selection
// histogram with one global atomic each (the histogram was cleared by the
// scorer earlier in the same call).  A scan of the chunk's counts in
// descending digit order gives its counts at or above every digit and each
// digit's first position; the keys are then grouped by digit in LDS (in any
// order inside a digit) and written out as one run.
__global__ __launch_bounds__(kAggChunk) void k_aggregate(const float *__restrict__ scores,
                                                         const float2 *__restrict__ part, float *__restrict__ A,
                                                         uint32_t *__restrict__ hist, uint32_t *__restrict__ skey,
                                                         uint16_t *__restrict__ sincl, SessI32 n_blocks,
                                                         SessI32 n_cand, int s0, ScoreGeom g, ScoreSplit sp) {
  __shared__ uint32_t shist[kBins];
  __shared__ uint32_t swsum[kTopkWaves];
  __shared__ uint32_t sgrouped[kAggChunk];
  __shared__ float sM[kAggRowsPerPass];
  __shared__ float sInvZ[kAggRowsPerPass];
  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int nb = n_blocks.v[sl];
  const int nc = n_cand.v[sl];
  if ((int)blockIdx.x * kAggChunk >= nb) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n_rows = g.Tq * g.G;
  const int b = blockIdx.x * kAggChunk + tid;
  const bool valid = b < nb;
  uint32_t *gh = hist + ((size_t)s * g.Hkv + h) * kSelBins;
  for (int i = tid; i < kBins; i += kAggChunk) shist[i] = 0u;
  float acc = 0.f;

  for (int rb = 0; rb < n_rows; rb += kAggRowsPerPass) {
    const int nr = min(kAggRowsPerPass, n_rows - rb);
    float sv[kAggRowsPerPass];
#pragma unroll
    for (int rr = 0; rr < kAggRowsPerPass; ++rr) {
      if (rr >= nr) break;
      const int r = rb + rr;
      const size_t row_id = ((size_t)s * g.Tq + r / g.G) * g.Hq + (size_t)h * g.G + r % g.G;
      sv[rr] = valid ? scores[row_id * g.max_blocks + b] : 0.f;
    }
    for (int rw = wave; rw < nr; rw += kAggChunk / 64) {
      const int r = rb + rw;
      const size_t row_id = ((size_t)s * g.Tq + r / g.G) * g.Hq + (size_t)h * g.G + r % g.G;
      // the scoring wavefronts that met this row's key, in order
      const int key = (sl * sp.n_rg + r / sp.rpg) * g.Hkv + h;
      const int n_slots = score_n_slots(key, sp);
      float2 ml = make_float2(-INFINITY, 0.f);
      for (int c = lane; c < n_slots; c += 64) ml = merge_ml(ml, part[row_id * g.slot_stride + c]);
      const float M = wave_max_dpp(ml.x);
      const float Z = wave_sum_dpp(ml.x == -INFINITY ? 0.f : ml.y * expf(ml.x - M));
      if (lane == 0) {
        sM[rw] = M;
        sInvZ[rw] = 1.0f / Z;
      }
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < kAggRowsPerPass; ++rr) {
      if (rr >= nr) break;
      // v_exp_f32 on log2 units: ~1e-6 relative on A; terms below 2^-126
      // flush, far below every candidate's A
      acc += __builtin_amdgcn_exp2f((sv[rr] - sM[rr]) * 1.4426950408889634f) * sInvZ[rr];
    }
    __syncthreads();
  }

  if (valid) A[((size_t)s * g.Hkv + h) * g.max_blocks + b] = acc;
  const uint32_t key = __float_as_uint(acc) & kKeyMask;
  const uint32_t digit = key >> kSelShift;
  if (b < nc) atomicAdd(&shist[digit], 1u);
  __syncthreads();
  for (int i = tid; i < kBins; i += kAggChunk) {
    const uint32_t c = shist[i];
    if (c) atomicAdd(&gh[i], c);
  }
  // thread t: digits kBins-1-2t and kBins-2-2t
  const uint32_t c0 = shist[kBins - 1 - 2 * tid], c1 = shist[kBins - 2 - 2 * tid];
  uint32_t n_in;
  const uint32_t above = wg_excl_scan(c0 + c1, swsum, n_in);   // (its barriers order the reads above)
  const size_t chunk = ((size_t)s * g.Hkv + h) * sel_chunks(g.max_blocks) + blockIdx.x;
  // counts at or above digits kBins-2-2t (low half) and kBins-1-2t (high half)
  reinterpret_cast<uint32_t *>(sincl + chunk * kSelBins)[(kBins - 2) / 2 - tid] =
      (above + c0 + c1) | ((above + c0) << 16);
  shist[kBins - 1 - 2 * tid] = above;
  shist[kBins - 2 - 2 * tid] = above + c0;
  __syncthreads();
  if (b < nc) sgrouped[atomicAdd(&shist[digit], 1u)] = key;
  __syncthreads();
  if (tid < (int)n_in) skey[chunk * kAggChunk + tid] = sgrouped[tid];
}

}  // namespace

hipError_t launch_topk(const float *A, const uint32_t *hist, const uint32_t *skey, const uint16_t *sincl,
                       int32_t *view_blocks, const TopkMeta &meta, int s0, int n_sess, int Hkv, int max_blocks,
                       int n_list, hipStream_t st) {
  int max_nc = 0;
  for (int i = 0; i < n_sess; ++i) max_nc = meta.n_cand.v[i] > max_nc ? meta.n_cand.v[i] : max_nc;
  if (hist != nullptr && max_nc <= kTile) {
    // the first chunk's workgroup always runs (it writes the recent blocks)
    const int nch = max_nc > 0 ? (max_nc + kAggChunk - 1) / kAggChunk : 1;
    dim3 grid((unsigned)nch, (unsigned)Hkv, (unsigned)n_sess);
    hipLaunchKernelGGL(k_topk_chunk, grid, dim3(kTopkThreads), 0, st, A, hist, skey, sincl, view_blocks, meta, s0,
                       Hkv, max_blocks, sel_chunks(max_blocks), n_list);
  } else {
    dim3 grid((unsigned)Hkv, (unsigned)n_sess);
    hipLaunchKernelGGL(k_topk, grid, dim3(kTopkThreads), 0, st, A, hist, view_blocks, meta, s0, Hkv, max_blocks,
                       n_list);
  }
  return hipGetLastError();
}

hipError_t launch_aggregate(const float *scores, const float2 *part, float *A, uint32_t *hist, uint32_t *skey,
                            uint16_t *sincl, const SessI32 &n_blocks, const SessI32 &n_cand, int s0, int n_sess,
                            const ScoreGeom &g, const ScoreSplit &split, hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  if (max_nb == 0) return hipSuccess;
  dim3 grid((unsigned)((max_nb + kAggChunk - 1) / kAggChunk), (unsigned)g.Hkv, (unsigned)n_sess);
  hipLaunchKernelGGL(k_aggregate, grid, dim3(kAggChunk), 0, st, scores, part, A, hist, skey, sincl, n_blocks, n_cand,
                     s0, g, split);
  return hipGetLastError();
}

}  // namespace kvmem
