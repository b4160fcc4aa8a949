// Decode attention straight from the paged history through the view lists,
// without a materialised view.
//
// KVMem separates the address space (the paged history) from the execution
// window (reproduction README, 'Core equation'); the bounded view is the
// selected blocks re-RoPE'd to contiguous positions (KVMem review, 'Summary').
// kvmem_materialize writes that view and kvmem_attend reads it; when a view
// serves few decode tokens, writing it costs more than the attention itself.
// This kernel computes the same attention from the pages: the m-th listed
// block of a KV head occupies view positions 32m .. 32m + 31, its pre-RoPE K
// tile is rotated there in registers and rounded to bf16 exactly as the gather
// would store it, and its V tile is used as stored.
//
// One workgroup of 8 wavefronts per (session, split of the list, group of 8
// KV heads); wavefront w serves KV head 8 * group + w over the split's list
// blocks.  Per block:
//   * the 32 x 64 RoPE (cos, sin) table of the block's view positions is
//     shared by the 8 heads through LDS (double-buffered, one barrier per
//     block).  Its angles are composed from the block's 64 base angles
//     (evaluated by one wavefront the block before) and the 32 x 64 in-block
//     offsets (a table formed once per workgroup), exactly as the gather
//     composes them;
//   * S^T = K Q^T and the online softmax are those of the view attention (the
//     K tile is loaded in the A-operand layout, where a dim and its +-64
//     partner sit in one lane);
//   * V is token-major in the page, while O^T = V^T P^T needs each lane's 8
//     tokens of one dimension: the wavefront stages its V tile in its own LDS
//     tile and reads the operand from there.
// Split partials have the view attention's layout and are merged by
// k_attend_combine.
//
// With WV (kvmem_materialize_attend) the kernel also writes the view, which
// makes it the gather and the attention in one pass: a lane's rotated K
// operand for token u is a 16-byte run of the view's K row, and its V^T
// operand (8 tokens of one dimension, in the accumulator's token order) is
// exactly 8 consecutive slots of that dimension in the view's V layout, so
// both go out as 16-byte stores with no extra data movement.  Tokens at or
// past V are zeroed before the rotation and the staging, as the gather writes
// them.
#include "attend_common.h"

namespace kvmem {

namespace {

constexpr int kPgWaves = 8;
constexpr int kPgPitch = kD + 8;   // padded token pitch (elements) of a wavefront's V tile

// (cos, sin) of pos * inv_freq in fp64, kept out of line: inlined into the
// block loop its temporaries push the kernel past its register budget
__device__ __noinline__ double2 block_angle(double pos, double inv_freq) {
  double c, s;
  rope_angle_f64(pos, inv_freq, c, s);
  return make_double2(c, s);
}

// token of k-slot e (0..7) of lane group qq: the S^T accumulator order
__device__ __forceinline__ int pg_token(int qq, int e) { return e < 4 ? 4 * qq + e : 16 + 4 * qq + (e - 4); }

template <int NT, bool WV>
__global__ __launch_bounds__(512) void k_attend_paged_bf16(
    const uint16_t *__restrict__ q, const float *__restrict__ qw, float eps, const uint16_t *__restrict__ kpool,
    const uint16_t *__restrict__ vpool, const int32_t *__restrict__ table, const int32_t *__restrict__ vblocks,
    float *__restrict__ part_o, float2 *__restrict__ part_ml, float *__restrict__ out, int32_t *dev_err,
    SessI32 view_tok, SessI32 n_all, int s0, PagedGeom g, double theta, uint16_t *__restrict__ kview,
    uint16_t *__restrict__ vview, int max_view) {
  __shared__ double inv_freq[kD / 2];
  __shared__ float cs_tab[kQprepMaxT][kD / 2][2];        // query positions V + t
  // (cos, sin) of the current block's positions; rows padded by one pair so
  // that the 16 tokens one read instruction touches fall in different banks
  __shared__ float ktab[2][kBT][kD / 2 + 1][2];
  __shared__ float2 offs[kBT][kD / 2];                   // in-block angles u * theta_i
  __shared__ double2 base_cs[2][kD / 2];                 // block angles 32 m * theta_i
  __shared__ __align__(16) uint16_t vt[kPgWaves][kBT * kPgPitch];

  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qq = lane >> 4;
  const int col = lane & 15;
  const int h = blockIdx.y * kPgWaves + wave;
  const bool head_ok = h < g.Hkv;
  const int V = view_tok.v[sl];
  const int m0 = split * g.bps;
  if (kBT * m0 >= V) return;                           // uniform over the workgroup
  const int m1 = min((V + kBT - 1) / kBT, m0 + g.bps);
  const int n_splits = (V + kBT * g.bps - 1) / (kBT * g.bps);

  if (tid < kD / 2) inv_freq[tid] = rope_inv_freq(tid, theta);
  float x[NT][4][8];
  int trow[NT];
  bool rvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + col;
    rvalid[nt] = head_ok && r < g.rows;
    const int t = rvalid[nt] ? r / g.G : 0, gg = rvalid[nt] ? r % g.G : 0;
    trow[nt] = t;
    const uint16_t *src = q + (((size_t)s * g.Tq + t) * g.Hq + (size_t)(head_ok ? h : 0) * g.G + gg) * kD + 8 * qq;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 w = *reinterpret_cast<const uint4 *>(src + 32 * c);
      const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[nt][c][2 * k] = bf16_lo(e[k]);
        x[nt][c][2 * k + 1] = bf16_hi(e[k]);
      }
    }
  }

  // first tile of this wavefront's list run (a bad list entry or page gives a
  // zero tile, as the gather writes zeros for it)
  const int32_t *lst = vblocks + ((size_t)s * g.Hkv + (head_ok ? h : 0)) * g.n_list;
  auto tile_base = [&](int m, bool &ok) -> size_t {
    ok = false;
    int page = 0;
    if (head_ok) {
      const int beta = lst[m];
      const bool beta_ok = beta >= 0 && beta < n_all.v[sl];
      const int p = beta_ok ? table[(size_t)s * g.max_blocks + beta] : -1;
      ok = beta_ok && p >= 0 && p < g.n_pages;
      if (!ok && lane == 0) dev_flag(dev_err, beta_ok ? 1 : 2);
      page = ok ? p : 0;
    }
    return ((size_t)page * g.Hkv + (head_ok ? h : 0)) * (size_t)(kBT * kD);
  };
  uint4 kr[2][4], vr[2][4];
  bool ok;
  auto load_tile = [&](int m) {
    const size_t base = tile_base(m, ok);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const size_t off = base + (size_t)(16 * tt + col) * kD + 32 * c + 8 * qq;
        kr[tt][c] = load_nt16(kpool + off);
        vr[tt][c] = load_nt16(vpool + off);
      }
  };
  load_tile(m0);
  __syncthreads();                                     // inv_freq

  {
    const int n_t = (g.rows + g.G - 1) / g.G;
    for (int idx = tid; idx < n_t * (kD / 2); idx += 512) {
      const int t = idx / (kD / 2), i = idx % (kD / 2);
      rope_cos_sin((double)(V + t), inv_freq[i], cs_tab[t][i][0], cs_tab[t][i][1]);
    }
    for (int idx = tid; idx < kBT * (kD / 2); idx += 512) {
      const int u = idx / (kD / 2), i = idx % (kD / 2);
      float cb, sb;
      rope_offset_pair(u, inv_freq[i], cb, sb);
      offs[u][i] = make_float2(cb, sb);
    }
    if (tid < kD / 2) {
#pragma unroll 1
      for (int k = 0; k < 2; ++k) {
        double c, sn;
        rope_angle_f64((double)(kBT * (m0 + k)), inv_freq[tid], c, sn);
        base_cs[k][tid] = make_double2(c, sn);
      }
    }
  }
  __syncthreads();                                     // cs_tab, offs, base_cs
  bf16x8 qhi[NT][4], qlo[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) build_q_operands(x[nt], rvalid[nt], trow[nt], qq, qw, eps, cs_tab, qhi[nt], qlo[nt]);

  floatx4 o[NT][8];
  float mrun[NT], lrun[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    mrun[nt] = -INFINITY;
    lrun[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[nt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  uint16_t *myv = vt[wave];

  for (int m = m0; m < m1; ++m) {
    const int buf = (m - m0) & 1;
#pragma unroll 1
    for (int idx = tid; idx < kBT * (kD / 2); idx += 512) {
      const int u = idx / (kD / 2), i = idx % (kD / 2);
      const double2 a = base_cs[buf][i];
      const float2 b = offs[u][i];
      rope_compose(a.x, a.y, b.x, b.y, ktab[buf][u][i][0], ktab[buf][u][i][1]);
    }

    // this wavefront's V tile, token-major, into its own LDS tile (tokens at
    // or past V are zeros, as the gather writes them; their weights are 0)
    const int tb = kBT * m;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4 *>(myv + (16 * tt + col) * kPgPitch + 32 * c + 8 * qq) =
            ok && tb + 16 * tt + col < V ? vr[tt][c] : make_uint4(0, 0, 0, 0);
    __syncthreads();

    // K rotated at view positions 32m + u and rounded to bf16: A operands
    bf16x8 ka[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int u = 16 * tt + col;
      float kv[4][8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 r = ok && tb + u < V ? kr[tt][c] : make_uint4(0, 0, 0, 0);
        const uint32_t e[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          kv[c][2 * k] = bf16_lo(e[k]);
          kv[c][2 * k + 1] = bf16_hi(e[k]);
        }
      }
      uint32_t w[4][4];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          float y1[2], y2[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int ip = 32 * c + 8 * qq + j + k;
            rope_rotate(kv[c][j + k], kv[c + 2][j + k], ktab[buf][u][ip][0], ktab[buf][u][ip][1], y1[k], y2[k]);
          }
          w[c][j / 2] = pack_bf16x2(y1[0], y1[1]);
          w[c + 2][j / 2] = pack_bf16x2(y2[0], y2[1]);
        }
#pragma unroll
      for (int c = 0; c < 4; ++c) ka[tt][c] = as_bf16x8(make_uint4(w[c][0], w[c][1], w[c][2], w[c][3]));
      if (WV && head_ok) {   // the view's K row of token u: dims 32c + 8qq .. + 7 from this lane
        uint16_t *row = kview + (((size_t)s * g.Hkv + h) * max_view + tb + u) * kD + 8 * qq;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          store_nt16(row + 32 * c, make_uint4(w[c][0], w[c][1], w[c][2], w[c][3]));
      }
    }
    // writing the view, the next tile's loads go out as soon as this tile's
    // registers are free and fly during the products (479 against 491 us at
    // 1M tokens; the attention alone measured no better this way)
    if (WV && m + 1 < m1) load_tile(m + 1);

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 sc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][c], qhi[nt][c], a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][c], qlo[nt][c], a, 0, 0, 0);
        }
        sc[tt] = a;
      }
      if (tb + kBT > V) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tb + 16 * tt + 4 * qq + i >= V) sc[tt][i] = -INFINITY;
      }
      float bm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      bm = max_xor16(bm);
      bm = max_xor32(bm);
      const float mn = fmaxf(mrun[nt], bm);
      const float alpha = exp2f(mrun[nt] - mn);
      mrun[nt] = mn;
      float p[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f(sc[0][i] - mn);
        p[4 + i] = exp2f(sc[1][i] - mn);
      }
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) psum += p[i];
      lrun[nt] = lrun[nt] * alpha + psum;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t h0, l0, h1, l1;
        split_hi_lo(p[2 * k], h0, l0);
        split_hi_lo(p[2 * k + 1], h1, l1);
        ph[k] = h0 | (h1 << 16);
        pl[k] = l0 | (l1 << 16);
      }
      const bf16x8 phi = as_bf16x8(make_uint4(ph[0], ph[1], ph[2], ph[3]));
      const bf16x8 plo = as_bf16x8(make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        // V^T operand: lane (qq, col) takes dimension 16 dt + col of its 8 tokens
        const int dim = 16 * dt + col;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = (uint32_t)myv[pg_token(qq, 2 * k) * kPgPitch + dim] |
                 ((uint32_t)myv[pg_token(qq, 2 * k + 1) * kPgPitch + dim] << 16);
        const bf16x8 va = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
        if (WV && nt == 0 && head_ok)   // the lane's 8 tokens of dim are slots 8qq .. 8qq + 7 of the view's V
          store_nt16(vview + ((((size_t)s * g.Hkv + h) * (max_view / kBT) + m) * kD + dim) * kBT + 8 * qq,
                     make_uint4(w[0], w[1], w[2], w[3]));
        o[nt][dt] *= alpha;
        o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, o[nt][dt], 0, 0, 0);
        o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, o[nt][dt], 0, 0, 0);
      }
    }
    // the base angles of block m + 2 into the buffer this block's table came
    // from (every wavefront passed this block's barrier, so it is read out;
    // block m + 1's barrier orders the write before block m + 2 reads it)
    if (tid < kD / 2 && m + 2 < m1) base_cs[buf][tid] = block_angle((double)(kBT * (m + 2)), inv_freq[tid]);
    // one tile in flight per wavefront: the next tile's loads follow the
    // products (eight wavefronts per CU move 128 KiB per step between them)
    if (!WV && m + 1 < m1) load_tile(m + 1);
  }

  if (!head_ok) return;
  // the wavefront alone holds its head's rows: partials (or the output)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = sum_xor32(sum_xor16(lrun[nt]));
    const int row = nt * 16 + col;
    if (row >= g.rows) continue;
    if (n_splits == 1) {
      const int t = row / g.G, gg = row % g.G;
      float *dst = out + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD;
      const float inv = 1.0f / l;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[16 * dt + 4 * qq + i] = o[nt][dt][i] * inv;
    } else {
      const size_t pidx = (((size_t)s * g.Hkv + h) * g.max_splits + split) * g.rows + row;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) part_o[pidx * kD + 16 * dt + 4 * qq + i] = o[nt][dt][i];
      if (qq == 0) part_ml[pidx] = make_float2(mrun[nt], l);
    }
  }
}

}  // namespace

int paged_blocks_per_split(int n_sessions, int Hkv, int n_list) {
  // aim for >= 256 workgroups of 8 wavefronts; 1 .. 64 list blocks per split
  const long groups = (Hkv + kPgWaves - 1) / kPgWaves;
  long b = ((long)n_list * groups * n_sessions + 255) / 256;
  if (b < 1) b = 1;
  if (b > 64) b = 64;
  return (int)b;
}

hipError_t launch_attend_paged(const void *q, const float *qw, float eps, const void *k_pool, const void *v_pool,
                               const int32_t *table, const int32_t *view_blocks, float *part_o, float2 *part_ml,
                               float *out, int32_t *dev_err, const SessI32 &view_tok, const SessI32 &n_all, int s0,
                               int n_sess, const PagedGeom &g, double theta, void *k_view, void *v_view, int max_view,
                               hipStream_t st) {
  int max_v = 0;
  for (int i = 0; i < n_sess; ++i) max_v = view_tok.v[i] > max_v ? view_tok.v[i] : max_v;
  const int splits = (max_v + kBT * g.bps - 1) / (kBT * g.bps);
  if (splits > 0) {
    dim3 grid((unsigned)splits, (unsigned)((g.Hkv + kPgWaves - 1) / kPgWaves), (unsigned)n_sess);
#define KVMEM_PAGED(NT, WV)                                                                                     \
  hipLaunchKernelGGL((k_attend_paged_bf16<NT, WV>), grid, dim3(512), 0, st, (const uint16_t *)q, qw, eps,          \
                     (const uint16_t *)k_pool, (const uint16_t *)v_pool, table, view_blocks, part_o, part_ml, out, \
                     dev_err, view_tok, n_all, s0, g, theta, (uint16_t *)k_view, (uint16_t *)v_view, max_view)
    const bool wv = k_view != nullptr;
    if (g.rows <= 16) {
      if (wv) KVMEM_PAGED(1, true); else KVMEM_PAGED(1, false);
    } else {
      if (wv) KVMEM_PAGED(2, true); else KVMEM_PAGED(2, false);
    }
#undef KVMEM_PAGED
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  AttendGeom ag;
  ag.Tq = g.Tq;
  ag.Hq = g.Hq;
  ag.Hkv = g.Hkv;
  ag.G = g.G;
  ag.rows = g.rows;
  ag.max_view = kBT * g.n_list;
  ag.max_splits = g.max_splits;
  ag.tpw = kBT * g.bps / 4;                            // the merge's split length is 4 * tpw tokens
  return launch_attend_combine(part_o, part_ml, out, view_tok, s0, n_sess, ag, st);
}

}  // namespace kvmem
