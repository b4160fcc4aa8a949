// Step-level view reuse: append new tokens to the history and to the view.
//
// KVMem schedules recall per agent step (KVMem review, 'Scope & Claims'),
// because attention barely moves within a step and shifts across step
// boundaries (review, 'Strengths'): the view is selected and materialised once
// and the step's tokens decode over it.  Each generated token's K/V then has
// to land in two places:
// the paged history (pre-RoPE, at its history position, so later index builds
// and selections see it) and the live view (K rotated at the next view
// position, V in the view's slot-permuted layout), so the following decode
// steps attend to it without a new selection.
//
// One workgroup per (new token, session) covers every KV head: eight threads
// per head, thread j owning dimension pairs (8j..8j+7, 64+8j..64+8j+7), so the
// rotation needs no cross-lane data; the token's 64 (cos, sin) pairs are formed
// once per workgroup and shared by every head.  The angles are formed exactly as the gather
// forms them, so an appended token is bit-identical to the same token
// gathered into that view position.
#include "append_common.h"

namespace kvmem {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void k_append(T *__restrict__ kpool, T *__restrict__ vpool,
                                                const int32_t *__restrict__ table, const T *__restrict__ knew,
                                                const T *__restrict__ vnew, int T_new, T *__restrict__ kview,
                                                T *__restrict__ vview, int32_t *dev_err, SessI32 n_tok,
                                                SessI32 view_tok, int s0, int Hkv, int max_blocks, int n_pages,
                                                int max_view, double theta) {
  __shared__ float2 cs_tok[kD / 2];   // (cos, sin) of the token's view position
  const int sl = blockIdx.y;
  append_token<T>(kpool, vpool, table, knew, vnew, T_new, kview, vview, dev_err, n_tok.v[sl], view_tok.v[sl], s0 + sl,
                  (int)blockIdx.x, Hkv, max_blocks, n_pages, max_view, theta, cs_tok);
}

}  // namespace

hipError_t launch_append(int bf16, void *k_pool, void *v_pool, const int32_t *table, const void *k_new,
                         const void *v_new, int T_new, void *k_view, void *v_view, int32_t *dev_err,
                         const SessI32 &n_tok, const SessI32 &view_tok, int s0, int n_sess, int Hkv, int max_blocks,
                         int n_pages, int max_view, double theta, hipStream_t st) {
  dim3 grid((unsigned)T_new, (unsigned)n_sess);
  if (bf16)
    hipLaunchKernelGGL(k_append<uint16_t>, grid, dim3(256), 0, st, (uint16_t *)k_pool, (uint16_t *)v_pool, table,
                       (const uint16_t *)k_new, (const uint16_t *)v_new, T_new, (uint16_t *)k_view,
                       (uint16_t *)v_view, dev_err, n_tok, view_tok, s0, Hkv, max_blocks, n_pages, max_view, theta);
  else
    hipLaunchKernelGGL(k_append<float>, grid, dim3(256), 0, st, (float *)k_pool, (float *)v_pool, table,
                       (const float *)k_new, (const float *)v_new, T_new, (float *)k_view, (float *)v_view,
                       dev_err, n_tok, view_tok, s0, Hkv, max_blocks, n_pages, max_view, theta);
  return hipGetLastError();
}

}  // namespace kvmem
