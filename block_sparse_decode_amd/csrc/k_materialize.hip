// Materialisation of the bounded execution view: gather + re-RoPE.
//
// KVMem restores the selected blocks with position-consistent re-RoPE into a
// bounded execution view (KVMem review, 'Summary' and 'Scope & Claims'); keys are
// stored un-rotated, so block m of the list lands at view positions 32m..32m+31
// and is rotated there.  One workgroup per (session, view block) covers every KV
// head: the 32 x 64 RoPE angles are the same for all heads, so each thread forms
// its 8 (cos, sin) pairs once and reuses them for every head (the block's 64
// base angles are evaluated once per workgroup, each thread's in-block offsets
// itself, and the two composed as every kernel that touches view keys does).  Thread (u, j) owns token u and the dimension
// pairs (8j..8j+7, 64+8j..64+8j+7), so each rotation needs no cross-lane data.
// K rows are written token-major; each V block is transposed through LDS into
// the dimension-major, slot-permuted layout that the attention kernel's
// matrix-core operands read directly.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr int kVtPitch = kBT + 2;   // padded slot pitch of the LDS transpose tile

template <typename T>
__global__ __launch_bounds__(256) void k_materialize(const T *__restrict__ kpool, const T *__restrict__ vpool,
                                                     const int32_t *__restrict__ table,
                                                     const int32_t *__restrict__ vblocks, T *__restrict__ kview,
                                                     T *__restrict__ vview, int32_t *dev_err, SessI32 view_tok,
                                                     SessI32 n_all, int s0, int Hkv, int max_blocks, int n_pages,
                                                     int n_list, int max_view, double theta) {
  __shared__ double inv_freq[kD / 2];
  __shared__ double2 base_cs[kD / 2];   // (cos, sin) of the block angle 32 m * theta_i
  __shared__ T vt[kD * kVtPitch];

  const int sl = blockIdx.y;
  const int s = s0 + sl;
  const int m = blockIdx.x;
  const int V = view_tok.v[sl];
  if (kBT * m >= V) return;
  const int nv = min(kBT, V - kBT * m);
  const int t = threadIdx.x;
  const int u = t >> 3;
  const int j = t & 7;
  if (t < kD / 2) {
    const double f = rope_inv_freq(t, theta);
    inv_freq[t] = f;
    double c, sn;
    rope_angle_f64((double)(kBT * m), f, c, sn);
    base_cs[t] = make_double2(c, sn);
  }
  __syncthreads();

  float cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float cb, sb;
    rope_offset_pair(u, inv_freq[8 * j + e], cb, sb);
    const double2 a = base_cs[8 * j + e];
    rope_compose(a.x, a.y, cb, sb, cs[e], sn[e]);
  }

  const int nall = n_all.v[sl];
  const size_t view_blocks_per_head = (size_t)(max_view / kBT);
  for (int h = 0; h < Hkv; ++h) {
    const int beta = vblocks[((size_t)s * Hkv + h) * n_list + m];
    const bool beta_ok = beta >= 0 && beta < nall;
    const int page = beta_ok ? table[(size_t)s * max_blocks + beta] : -1;
    const bool ok = beta_ok && page >= 0 && page < n_pages;
    if (!ok && t == 0) dev_flag(dev_err, beta_ok ? 1 : 2);
    const bool have = ok && u < nv;

    // K: rotate pair (i, i + 64) by angle pos * theta^(-2i/d), round to storage.
    float x1[8], x2[8];
    const size_t src_off = (((size_t)(have ? page : 0) * Hkv + h) * kBT + u) * kD;
    if (have) {
      Row8<T>::load(kpool + src_off + 8 * j, x1);
      Row8<T>::load(kpool + src_off + 64 + 8 * j, x2);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x1[e] = x2[e] = 0.f;
    }
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(x1[e], x2[e], cs[e], sn[e], y1[e], y2[e]);
    T *kd = kview + (((size_t)s * Hkv + h) * max_view + (size_t)kBT * m + u) * kD;
    Row8<T>::store(kd + 8 * j, y1);
    Row8<T>::store(kd + 64 + 8 * j, y2);

    // V: bit copy, transposed to [dim][slot] through LDS.
    T v1[8], v2[8];
    if (have) {
      Row8<T>::load_raw(vpool + src_off + 8 * j, v1);
      Row8<T>::load_raw(vpool + src_off + 64 + 8 * j, v2);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v1[e] = v2[e] = (T)0;
    }
    const int slot = v_slot(u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vt[(8 * j + e) * kVtPitch + slot] = v1[e];
      vt[(64 + 8 * j + e) * kVtPitch + slot] = v2[e];
    }
    __syncthreads();
    {
      const int dim = t >> 1;
      const int half = t & 1;
      T *vd = vview + ((((size_t)s * Hkv + h) * view_blocks_per_head + m) * kD + dim) * kBT + 16 * half;
      Row8<T>::copy16(vd, vt + dim * kVtPitch + 16 * half);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_materialize(int bf16, const void *k_pool, const void *v_pool, const int32_t *table,
                              const int32_t *view_blocks, void *k_view, void *v_view, int32_t *dev_err,
                              const SessI32 &view_tok, const SessI32 &n_all, int s0, int n_sess, int Hkv,
                              int max_blocks, int n_pages, int n_list, int max_view, double theta,
                              hipStream_t st) {
  int max_v = 0;
  for (int i = 0; i < n_sess; ++i) max_v = view_tok.v[i] > max_v ? view_tok.v[i] : max_v;
  if (max_v == 0) return hipSuccess;
  dim3 grid((unsigned)((max_v + kBT - 1) / kBT), (unsigned)n_sess);
  if (bf16)
    hipLaunchKernelGGL(k_materialize<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)k_pool,
                       (const uint16_t *)v_pool, table, view_blocks, (uint16_t *)k_view, (uint16_t *)v_view,
                       dev_err, view_tok, n_all, s0, Hkv, max_blocks, n_pages, n_list, max_view, theta);
  else
    hipLaunchKernelGGL(k_materialize<float>, grid, dim3(256), 0, st, (const float *)k_pool,
                       (const float *)v_pool, table, view_blocks, (float *)k_view, (float *)v_view, dev_err,
                       view_tok, n_all, s0, Hkv, max_blocks, n_pages, n_list, max_view, theta);
  return hipGetLastError();
}

}  // namespace kvmem
