// Appending new tokens to the history and to the view: the per-token routine
// shared by k_append and by the attention's merge launch (which appends the
// step's token beside the merge, kvmem_attend_append).  Angles are formed
// exactly as the gather forms them, so an appended token is bit-identical to
// the same token gathered into that view position.
#pragma once
#include "kvmem_internal.h"

namespace kvmem {

// 8 elements (16 or 32 bytes, 16-byte aligned) copied bit for bit.
template <typename T>
__device__ __forceinline__ void copy8(T *dst, const T *src) {
#pragma unroll
  for (int k = 0; k < (int)sizeof(T) / 2; ++k)
    reinterpret_cast<uint4 *>(dst)[k] = reinterpret_cast<const uint4 *>(src)[k];
}

__device__ __forceinline__ float elem_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float elem_f32(float x) { return x; }

// The append of new token t of session s (history length n_tok_s and view
// length view_tok_s before the append) by one 256-thread workgroup; cs_tok is
// a 64-entry LDS array of the workgroup.
template <typename T>
__device__ __forceinline__ void append_token(T *__restrict__ kpool, T *__restrict__ vpool,
                                             const int32_t *__restrict__ table, const T *__restrict__ knew,
                                             const T *__restrict__ vnew, int T_new, T *__restrict__ kview,
                                             T *__restrict__ vview, int32_t *dev_err, int n_tok_s, int view_tok_s,
                                             int s, int t, int Hkv, int max_blocks, int n_pages, int max_view,
                                             double theta, float2 *cs_tok) {
  const int j = threadIdx.x & 7;
  const int hist = n_tok_s + t;                     // < 32 * max_blocks (checked on the host)
  const int vpos = view_tok_s + t;                  // < max_view (checked on the host)
  const int beta = hist / kBT;
  const int page = table[(size_t)s * max_blocks + beta];
  const bool page_ok = page >= 0 && page < n_pages;
  if (!page_ok && threadIdx.x == 0) dev_flag(dev_err, 1);

  // this thread's first head: its new K and V are requested before the
  // angles are formed, so the two latencies overlap
  const int h0 = threadIdx.x >> 3;
  T v1[8], v2[8], k1[8], k2[8];                        // raw elements (converted when used)
  auto load_head = [&](int h) {
    const size_t src = (((size_t)s * T_new + t) * Hkv + h) * kD;
    Row8<T>::load_raw(vnew + src + 8 * j, v1);
    Row8<T>::load_raw(vnew + src + 64 + 8 * j, v2);
    Row8<T>::load_raw(knew + src + 8 * j, k1);
    Row8<T>::load_raw(knew + src + 64 + 8 * j, k2);
  };
  if (h0 < Hkv) load_head(h0);

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
  for (int h = h0; h < Hkv; h += blockDim.x / 8) {
    const size_t src = (((size_t)s * T_new + t) * Hkv + h) * kD;
    if (h != h0) load_head(h);
    // history: bit copies at (page, head, token of the block), 16 bytes a time
    if (page_ok) {
      const size_t dst = (((size_t)page * Hkv + h) * kBT + hist % kBT) * kD;
      copy8(kpool + dst + 8 * j, knew + src + 8 * j);
      copy8(kpool + dst + 64 + 8 * j, knew + src + 64 + 8 * j);
      copy8(vpool + dst + 8 * j, vnew + src + 8 * j);
      copy8(vpool + dst + 64 + 8 * j, vnew + src + 64 + 8 * j);
    }
    // view: K rotated at position vpos and rounded; V at its slot
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(elem_f32(k1[e]), elem_f32(k2[e]), cs[e], sn[e], y1[e], y2[e]);
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
    if (t == T_new - 1 && m * kBT >= view_tok_s) {
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


}  // namespace kvmem
