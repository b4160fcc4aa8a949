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
#include "kvmem_internal.h"

namespace kvmem {

namespace {

// 8 elements (16 or 32 bytes, 16-byte aligned) copied bit for bit.
template <typename T>
__device__ __forceinline__ void copy8(T *dst, const T *src) {
#pragma unroll
  for (int k = 0; k < (int)sizeof(T) / 2; ++k)
    reinterpret_cast<uint4 *>(dst)[k] = reinterpret_cast<const uint4 *>(src)[k];
}

template <typename T>
__global__ __launch_bounds__(256) void k_append(T *__restrict__ kpool, T *__restrict__ vpool,
                                                const int32_t *__restrict__ table, const T *__restrict__ knew,
                                                const T *__restrict__ vnew, int T_new, T *__restrict__ kview,
                                                T *__restrict__ vview, int32_t *dev_err, SessI32 n_tok,
                                                SessI32 view_tok, int s0, int Hkv, int max_blocks, int n_pages,
                                                int max_view, double theta) {
  __shared__ float2 cs_tok[kD / 2];   // (cos, sin) of the token's view position
  const int t = blockIdx.x;
  const int sl = blockIdx.y;
  const int s = s0 + sl;
  const int j = threadIdx.x & 7;
  const int hist = n_tok.v[sl] + t;                     // < 32 * max_blocks (checked on the host)
  const int vpos = view_tok.v[sl] + t;                  // < max_view (checked on the host)
  const int beta = hist / kBT;
  const int page = table[(size_t)s * max_blocks + beta];
  const bool page_ok = page >= 0 && page < n_pages;
  if (!page_ok && threadIdx.x == 0) dev_flag(dev_err, 1);

  // the angles of view position vpos = 32 (vpos / 32) + vpos % 32, composed
  // as the gather composes them, once per frequency for every head
  if (threadIdx.x < kD / 2) {
    const double f = rope_inv_freq(threadIdx.x, theta);
    double ca, sa;
    rope_angle_f64((double)(vpos - vpos % kBT), f, ca, sa);
    float cb, sb, c, sn;
    rope_offset_pair(vpos % kBT, f, cb, sb);
    rope_compose(ca, sa, cb, sb, c, sn);
    cs_tok[threadIdx.x] = make_float2(c, sn);
  }
  __syncthreads();
  float cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    cs[e] = cs_tok[8 * j + e].x;
    sn[e] = cs_tok[8 * j + e].y;
  }

  const int m = vpos / kBT;
  const int slot = v_slot(vpos % kBT);
  for (int h = threadIdx.x >> 3; h < Hkv; h += blockDim.x / 8) {
    const size_t src = (((size_t)s * T_new + t) * Hkv + h) * kD;
    T v1[8], v2[8];
    Row8<T>::load_raw(vnew + src + 8 * j, v1);
    Row8<T>::load_raw(vnew + src + 64 + 8 * j, v2);
    // history: bit copies at (page, head, token of the block), 16 bytes a time
    if (page_ok) {
      const size_t dst = (((size_t)page * Hkv + h) * kBT + hist % kBT) * kD;
      copy8(kpool + dst + 8 * j, knew + src + 8 * j);
      copy8(kpool + dst + 64 + 8 * j, knew + src + 64 + 8 * j);
      copy8(vpool + dst + 8 * j, vnew + src + 8 * j);
      copy8(vpool + dst + 64 + 8 * j, vnew + src + 64 + 8 * j);
    }
    // view: K rotated at position vpos and rounded; V at its slot
    float x1[8], x2[8], y1[8], y2[8];
    Row8<T>::load(knew + src + 8 * j, x1);
    Row8<T>::load(knew + src + 64 + 8 * j, x2);
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(x1[e], x2[e], cs[e], sn[e], y1[e], y2[e]);
    T *kd = kview + (((size_t)s * Hkv + h) * max_view + vpos) * kD;
    Row8<T>::store(kd + 8 * j, y1);
    Row8<T>::store(kd + 64 + 8 * j, y2);
    T *vb = vview + (((size_t)s * Hkv + h) * (size_t)(max_view / kBT) + m) * (size_t)(kD * kBT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vb[(size_t)(8 * j + e) * kBT + slot] = v1[e];
      vb[(size_t)(64 + 8 * j + e) * kBT + slot] = v2[e];
    }
    // The slots after the new view length up to the end of its 32-token view
    // block must be zero, as the gather leaves them (the attention masks their
    // logits, and zero V keeps the masked products finite).  They already are
    // unless this append opened that view block; then the last token's
    // workgroup clears them (no other workgroup touches those slots).
    if (t == T_new - 1 && m * kBT >= view_tok.v[sl]) {
      const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int z = vpos + 1; z < (m + 1) * kBT; ++z) {
        T *kz = kview + (((size_t)s * Hkv + h) * max_view + z) * kD;
        Row8<T>::store(kz + 8 * j, zero);
        Row8<T>::store(kz + 64 + 8 * j, zero);
        const int zs = v_slot(z % kBT);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vb[(size_t)(8 * j + e) * kBT + zs] = (T)0;
          vb[(size_t)(64 + 8 * j + e) * kBT + zs] = (T)0;
        }
      }
    }
  }
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
