// Host-tier paging: staging of a selection's blocks into an HBM page pool.
//
// KVMem keeps the agent's history as paged KV across GPU memory, host memory
// and NVMe, and brings the selected blocks into the bounded execution view on
// demand (reproduction README, 'Background and main changes'; KVMem review,
// 'Summary').  Here the K/V pages may live in pinned host memory, which the GPU
// reads directly over the host link; the Mean-K index stays in HBM, so scoring
// and selection never touch the host tier.  Once a selection is made, k_stage
// moves exactly the listed (block, KV head) tiles over the link into an HBM
// staging pool laid out in view order: staged page s * n_list + m holds, for
// every KV head h, head h's m-th listed block.  With the staged block table
// (logical block m -> page s * n_list + m) and the identity list (m at slot m),
// the staged pool is an ordinary workspace whose "history" is the view itself,
// so the gather and attention kernels run on it unchanged and write the same
// view bits: view position 32m + u depends only on the list slot, never on
// the original block index.
//
// A fixed, small grid of workgroups strides over the (session, list slot)
// pairs; a workgroup copies a slot's tiles for all KV heads, 16 bytes per lane
// per non-temporal load, with a head's K and V tiles in flight together.  Tokens past the view's end (the partial tail block) are
// not read and are zero in the staged tile; a bad list entry or page is
// flagged (KVMEM_DEVERR_*) and staged as a zero tile, which is what the gather
// would have written for it.
#include "../../include/kvmem.h"
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kStageGroups = 8;     // workgroups of one staging launch

template <int EB>   // bytes per element
__global__ __launch_bounds__(256) void k_stage(const uint4 *__restrict__ kpool, const uint4 *__restrict__ vpool,
                                               const int32_t *__restrict__ table,
                                               const int32_t *__restrict__ vblocks, uint4 *__restrict__ sk,
                                               uint4 *__restrict__ sv, int32_t *__restrict__ stable,
                                               int32_t *__restrict__ slist, int32_t *dev_err, SessI32 view_tok,
                                               SessI32 n_all, int s0, int n_sess, int Hkv, int max_blocks,
                                               int n_pages, int n_list) {
  constexpr int kWordsPerTok = kD * EB / 16;          // 16-byte words per token row
  constexpr int kTileWords = kBT * kWordsPerTok;      // one (block, head) tile
  constexpr int kPer = kTileWords / 256;              // words per thread per tile
  const int t = threadIdx.x;
  // workgroups stride over the (session, list slot) pairs, slots fastest
  for (int job = blockIdx.x; job < n_sess * n_list; job += gridDim.x) {
    const int sl = job / n_list;
    const int m = job % n_list;
    const int s = s0 + sl;
    const int V = view_tok.v[sl];
    const int nvb = (V + kBT - 1) / kBT;              // listed blocks in the view
    const size_t slot = (size_t)s * n_list + m;
    if (m >= nvb) {                                   // past the view: empty slot
      if (t == 0) stable[slot] = -1;
      for (int h = t; h < Hkv; h += 256) slist[((size_t)s * Hkv + h) * n_list + m] = -1;
      continue;
    }
    if (t == 0) stable[slot] = (int32_t)slot;
    for (int h = t; h < Hkv; h += 256) slist[((size_t)s * Hkv + h) * n_list + m] = m;
    const int nv = min(kBT, V - kBT * m);             // valid tokens of this block
    const int nall = n_all.v[sl];
    for (int h = 0; h < Hkv; ++h) {
      const int beta = vblocks[((size_t)s * Hkv + h) * n_list + m];
      const bool beta_ok = beta >= 0 && beta < nall;
      const int page = beta_ok ? table[(size_t)s * max_blocks + beta] : -1;
      const bool ok = beta_ok && page >= 0 && page < n_pages;
      if (!ok && t == 0) dev_flag(dev_err, beta_ok ? KVMEM_DEVERR_PAGE : KVMEM_DEVERR_BLOCK);
      const size_t src = ((size_t)(ok ? page : 0) * Hkv + h) * kTileWords;
      const size_t dst = (slot * Hkv + h) * kTileWords;
      uint4 kw[kPer], vw[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int w = t + 256 * i;
        const bool have = ok && w / kWordsPerTok < nv;
        kw[i] = have ? load_nt16(kpool + src + w) : make_uint4(0u, 0u, 0u, 0u);
        vw[i] = have ? load_nt16(vpool + src + w) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        sk[dst + t + 256 * i] = kw[i];
        sv[dst + t + 256 * i] = vw[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_stage(int bf16, const void *k_pool, const void *v_pool, const int32_t *table,
                        const int32_t *view_blocks, void *stage_k, void *stage_v, int32_t *stage_table,
                        int32_t *stage_list, int32_t *dev_err, const SessI32 &view_tok, const SessI32 &n_all,
                        int s0, int n_sess, int Hkv, int max_blocks, int n_pages, int n_list, hipStream_t st) {
  // the host link, not the GPU, bounds the copy: eight workgroups keep it
  // full (56.6 GB/s against 57.0 with 128 or 512 at 256K tokens; four drop to
  // 38), and fewer of them in flight interfere far less with device-memory
  // work on other streams (a copy beside 51 attention launches: 3.1 ms
  // together against 4.7 back to back with 8 workgroups, 4.5 with 128)
  const long jobs = (long)n_sess * n_list;
  const dim3 grid((unsigned)(jobs < kStageGroups ? jobs : kStageGroups));
  if (bf16)
    hipLaunchKernelGGL(k_stage<2>, grid, dim3(256), 0, st, (const uint4 *)k_pool, (const uint4 *)v_pool, table,
                       view_blocks, (uint4 *)stage_k, (uint4 *)stage_v, stage_table, stage_list, dev_err, view_tok,
                       n_all, s0, n_sess, Hkv, max_blocks, n_pages, n_list);
  else
    hipLaunchKernelGGL(k_stage<4>, grid, dim3(256), 0, st, (const uint4 *)k_pool, (const uint4 *)v_pool, table,
                       view_blocks, (uint4 *)stage_k, (uint4 *)stage_v, stage_table, stage_list, dev_err, view_tok,
                       n_all, s0, n_sess, Hkv, max_blocks, n_pages, n_list);
  return hipGetLastError();
}

}  // namespace kvmem
