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
// One workgroup of nw wavefronts per (session, split of the list, group of nw
// KV heads; nw is the largest divisor of Hkv up to 8); wavefront w serves KV
// head nw * group + w over the split's list blocks, which are every
// n_splits-th block of the list starting at the split's index.  Per block:
//   * the 32 x 64 RoPE (cos, sin) table of the block's view positions is
//     shared by the heads through LDS (double-buffered, one barrier per
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
// k_attend_combine.  fp32 workspaces take a vector-ALU kernel
// (k_attend_paged_f32, below) with the same splits and partials.
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

__device__ __forceinline__ uint4 and_mask(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

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
  int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qq = lane >> 4;
  const int col = lane & 15;
  const int h = blockIdx.y * (int)(blockDim.x >> 6) + wave;   // every wavefront has a head (paged_waves)
  const int nthr = (int)blockDim.x;
  const int V = view_tok.v[sl];
  const int n_splits = (V + kBT * g.bps - 1) / (kBT * g.bps);
  if (split >= n_splits) return;                       // uniform over the workgroup
  // Workgroups are dealt to the 8 XCDs in turn; this permutation of the splits
  // gives each XCD's workgroups adjacent splits.
  if ((n_splits & 7) == 0 && (int)gridDim.x == n_splits) split = (split & 7) * (n_splits >> 3) + (split >> 3);
  // This workgroup's view blocks: split, split + n_splits, split + 2 n_splits,
  // ... (at most bps of them), so that the workgroups, which run in step, read
  // and write one compact window of every head's view at a time.  One-pass
  // call at 1M tokens: 441 us with a run of bps adjacent blocks per
  // workgroup, 426 us with the blocks strided, 422 us with the XCD
  // permutation as well.
  const int nblk = (V + kBT - 1) / kBT;
  const int n_my = (nblk - split + n_splits - 1) / n_splits;
  auto blk = [&](int i) { return split + i * n_splits; };

  if (tid < kD / 2) inv_freq[tid] = rope_inv_freq(tid, theta);
  float x[NT][4][8];
  int trow[NT];
  bool rvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + col;
    rvalid[nt] = r < g.rows;
    const int t = rvalid[nt] ? r / g.G : 0, gg = rvalid[nt] ? r % g.G : 0;
    trow[nt] = t;
    const uint16_t *src = q + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD + 8 * qq;
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

  // The split's pages, resolved once (a split has at most 64 list blocks):
  // lane l holds the page of list block blk(l), or -1 for a bad list entry or
  // page (flagged here; its tile is zeros, as the gather writes zeros for it).
  // Each block then takes its page from a register with readlane instead of a
  // list load and a table load that depend on each other: resolved per block,
  // those two round trips, and a wait for every memory operation before them
  // (the view stores included), stood before each tile's loads.
  int my_page = -1;
  if (lane < n_my) {
    const int beta = vblocks[((size_t)s * g.Hkv + h) * g.n_list + blk(lane)];
    const bool beta_ok = beta >= 0 && beta < n_all.v[sl];
    const int p = beta_ok ? table[(size_t)s * g.max_blocks + beta] : -1;
    const bool okp = beta_ok && p >= 0 && p < g.n_pages;
    if (!okp) dev_flag(dev_err, beta_ok ? 1 : 2);
    my_page = okp ? p : -1;
  }
  // the tile of the workgroup's i-th block
  auto tile_base = [&](int i, bool &ok) -> size_t {
    const int page = __builtin_amdgcn_readlane(my_page, i);
    ok = page >= 0;
    return ((size_t)(ok ? page : 0) * g.Hkv + h) * (size_t)(kBT * kD);
  };
  uint4 kr[2][4], vr[2][4];
  bool ok;
  constexpr bool kKOperandLoads = WV || NT > 1;          // K loaded in the A-operand layout
  auto load_k = [&](int i) {
    bool okm;
    const size_t base = tile_base(i, okm);
    // Without the view and with one row tile: whole 128-byte lines
    // (load_k_lines; k_lines_operand before use), 190 -> 186 us per call at
    // 1M tokens.  Writing the view, or with two row tiles, the operand layout
    // directly: there the exchange's registers made the kernel spill more
    // (one-pass call 447 -> 456 us at 1M tokens).
    if (kKOperandLoads) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int c = 0; c < 4; ++c) kr[tt][c] = load_nt16(kpool + base + (size_t)(16 * tt + col) * kD + 32 * c + 8 * qq);
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) load_k_lines(kr[tt], kpool + base + (size_t)(16 * tt) * kD, qq, col);
    }
  };
  // V goes through LDS, so its loads take whole rows: instruction j, lane l
  // reads token 4j + l / 16, dims 8 (l % 16) .. + 7 (full 128-byte lines)
  auto load_v = [&](int i) {
    bool okm;
    const size_t base = tile_base(i, okm);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vr[j >> 2][j & 3] = load_nt16(vpool + base + (size_t)(4 * j + (lane >> 4)) * kD + 8 * (lane & 15));
  };
  auto load_tile = [&](int i) {
    load_k(i);
    load_v(i);
  };
  load_tile(0);
  __syncthreads();                                     // inv_freq

  {
    const int n_t = (g.rows + g.G - 1) / g.G;
    for (int idx = tid; idx < n_t * (kD / 2); idx += nthr) {
      const int t = idx / (kD / 2), i = idx % (kD / 2);
      rope_cos_sin((double)(V + t), inv_freq[i], cs_tab[t][i][0], cs_tab[t][i][1]);
    }
    for (int idx = tid; idx < kBT * (kD / 2); idx += nthr) {
      const int u = idx / (kD / 2), i = idx % (kD / 2);
      float cb, sb;
      rope_offset_pair(u, inv_freq[i], cb, sb);
      offs[u][i] = make_float2(cb, sb);
    }
    if (tid < kD / 2) {
#pragma unroll 1
      for (int k = 0; k < 2; ++k) {
        double c, sn;
        rope_angle_f64((double)(kBT * blk(k)), inv_freq[tid], c, sn);
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

  for (int i = 0; i < n_my; ++i) {
    const int m = blk(i);
    const int buf = i & 1;
#pragma unroll 1
    for (int idx = tid; idx < kBT * (kD / 2); idx += nthr) {
      const int u = idx / (kD / 2), i = idx % (kD / 2);
      const double2 a = base_cs[buf][i];
      const float2 b = offs[u][i];
      rope_compose(a.x, a.y, b.x, b.y, ktab[buf][u][i][0], ktab[buf][u][i][1]);
    }

    // this wavefront's V tile, token-major, into its own LDS tile (tokens at
    // or past V are zeros, as the gather writes them; their weights are 0)
    // (the zeroing is an AND with a lane mask, not a select: a select
    // compiles to exec-masked branches, after which the compiler no longer
    // knows the tile's loads have landed and waits for the view stores too)
    const int tb = kBT * m;
    (void)tile_base(i, ok);
    uint32_t keep[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) keep[tt] = ok && tb + 16 * tt + col < V ? 0xffffffffu : 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tok = 4 * j + (lane >> 4);
      *reinterpret_cast<uint4 *>(myv + tok * kPgPitch + 8 * (lane & 15)) =
          and_mask(vr[j >> 2][j & 3], ok && tb + tok < V ? 0xffffffffu : 0u);
    }
    // the next V tile leaves as soon as this one is staged: it flies through
    // the barrier, the rotation and both products (at 1M tokens 471 -> 458 us
    // with the view written, 258 -> 225 us without)
    if (i + 1 < n_my) load_v(i + 1);
    __syncthreads();

    // K rotated at view positions 32m + u and rounded to bf16: A operands
    bf16x8 ka[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int u = 16 * tt + col;
      uint4 kop[4];
      if (kKOperandLoads) {
#pragma unroll
        for (int c = 0; c < 4; ++c) kop[c] = kr[tt][c];
      } else {
        k_lines_operand(kr[tt], kop, col);
      }
      float kv[4][8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 r = and_mask(kop[c], keep[tt]);
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
      if (WV) {
        // The view's K rows 16tt .. 16tt + 15: this lane holds dims 32c + 8qq
        // .. + 7 of row u (16 bytes at byte 64c + 16qq).  Whole 128-byte lines
        // per store: half hf of a row (bytes 128hf ..) is pieces c = 2hf and
        // 2hf + 1 of its four qq lanes.  Lanes col and col ^ 8 swap their
        // pieces 2hf + 1 (DPP row_ror:8), then one store writes half hf of
        // rows 0..7 (col < 8: own piece 2hf; col >= 8: the partner's piece
        // 2hf + 1 of row col - 8) and the other half hf of rows 8..15.
        // (Written as 64-byte runs per store the K stream cost ~15 us more at
        // 1M tokens.)
        uint16_t *blk = kview + (((size_t)s * g.Hkv + h) * max_view + tb + 16 * tt) * kD + 8 * qq;
        const bool lo = col < 8;
        const int r_own = col, r_rcv = col ^ 8;          // rows of the own and the received piece
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          uint32_t x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[2 * hf + 1][e], kDppRor8, 0xf, 0xf, false);
          const uint4 own = make_uint4(w[2 * hf][0], w[2 * hf][1], w[2 * hf][2], w[2 * hf][3]);
          const uint4 rcv = make_uint4(x[0], x[1], x[2], x[3]);
          // rows 0..7, then rows 8..15
          store_nt16(blk + (lo ? r_own : r_rcv) * kD + 32 * (lo ? 2 * hf : 2 * hf + 1), lo ? own : rcv);
          store_nt16(blk + (lo ? r_rcv : r_own) * kD + 32 * (lo ? 2 * hf + 1 : 2 * hf), lo ? rcv : own);
        }
      }
    }
    // the next K tile: writing the view, as soon as the rotation has freed its
    // registers; without the view, once the score products have consumed the
    // rotated operands (225 -> 204 us at 1M tokens).  Any order that puts
    // this tile's K view stores behind the next loads spills ~40 registers.
    if (WV && i + 1 < n_my) load_k(i + 1);

    floatx4 scs[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][c], qhi[nt][c], a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tt][c], qlo[nt][c], a, 0, 0, 0);
        }
        scs[nt][tt] = a;
      }
    if (!WV && i + 1 < n_my) load_k(i + 1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 sc[2] = {scs[nt][0], scs[nt][1]};
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
        if (WV && nt == 0)   // the lane's 8 tokens of dim are slots 8qq .. 8qq + 7 of the view's V
          store_nt16(vview + ((((size_t)s * g.Hkv + h) * (max_view / kBT) + m) * kD + dim) * kBT + 8 * qq,
                     make_uint4(w[0], w[1], w[2], w[3]));
        o[nt][dt] *= alpha;
        o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, o[nt][dt], 0, 0, 0);
        o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, o[nt][dt], 0, 0, 0);
      }
    }
    // the base angles of block blk(i + 2) into the buffer this block's table
    // came from (every wavefront passed this block's barrier, so it is read
    // out; block i + 1's barrier orders the write before block i + 2 reads it)
    if (tid < kD / 2 && i + 2 < n_my) base_cs[buf][tid] = block_angle((double)(kBT * blk(i + 2)), inv_freq[tid]);
  }

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

// fp32 workspaces: a vector-ALU kernel with the same split structure and
// partial layout.  One 256-thread workgroup per (session, split of the list,
// KV head).  Per listed block the workgroup rotates the block's keys at their
// view positions with the gather's angle composition and rotation (so the
// keys are the view's, bit for bit), stages K and V in LDS, and runs the fp32
// logits, online softmax and weighted sum of the view attention over them.
// With WV it also writes the view exactly as the gather does (K rotated,
// token-major; V copied into its slot; zeros past V in the last block).
constexpr int kPgF32MaxRows = 64;

template <bool WV>
__global__ __launch_bounds__(256) void k_attend_paged_f32(
    const float *__restrict__ q, const float *__restrict__ qw, float eps, const float *__restrict__ kpool,
    const float *__restrict__ vpool, const int32_t *__restrict__ table, const int32_t *__restrict__ vblocks,
    float *__restrict__ part_o, float2 *__restrict__ part_ml, float *__restrict__ out, int32_t *dev_err,
    SessI32 view_tok, SessI32 n_all, int s0, PagedGeom g, double theta, float *__restrict__ kview,
    float *__restrict__ vview, int max_view) {
  __shared__ double inv_freq[kD / 2];
  __shared__ double2 base_cs[kD / 2];                  // block angles 32 m * theta_i
  __shared__ float2 offs[kBT][kD / 2];                 // in-block angles u * theta_i
  __shared__ float qs[kPgF32MaxRows][kD + 1];
  __shared__ float ks[kBT][kD + 1];
  __shared__ float vs[kBT][kD];
  __shared__ float lg[kPgF32MaxRows][kBT + 1];
  __shared__ float srs[kPgF32MaxRows], smx[kPgF32MaxRows], slsum[kPgF32MaxRows], salpha[kPgF32MaxRows];
  __shared__ int s_page;

  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int V = view_tok.v[sl];
  const int m0 = split * g.bps;
  if (kBT * m0 >= V) return;
  const int m1 = min((V + kBT - 1) / kBT, m0 + g.bps);
  const int n_splits = (V + kBT * g.bps - 1) / (kBT * g.bps);
  const int R = g.rows;
  if (tid < kD / 2) inv_freq[tid] = rope_inv_freq(tid, theta);
  if (tid < R) {
    const int t = tid / g.G, gg = tid % g.G;
    const float *src = q + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD;
    float ss = 0.f;
    for (int e = 0; e < kD; ++e) ss += src[e] * src[e];
    srs[tid] = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
    smx[tid] = -INFINITY;
    slsum[tid] = 0.f;
  }
  __syncthreads();
  for (int idx = tid; idx < kBT * (kD / 2); idx += 256) {
    float cb, sb;
    rope_offset_pair(idx / (kD / 2), inv_freq[idx % (kD / 2)], cb, sb);
    offs[idx / (kD / 2)][idx % (kD / 2)] = make_float2(cb, sb);
  }
  for (int idx = tid; idx < R * kD; idx += 256) {       // q~ rotated at V + t, in log2 units
    const int r = idx >> 7, dim = idx & (kD - 1);
    const int t = r / g.G, gg = r % g.G;
    const float *src = q + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD;
    const int i = dim & 63;
    const int pd = dim < 64 ? dim + 64 : dim - 64;
    const float x = src[dim] * srs[r] * qw[dim];
    const float px = src[pd] * srs[r] * qw[pd];
    float c, sn;
    rope_cos_sin((double)(V + t), inv_freq[i], c, sn);
    qs[r][dim] = (dim < 64 ? x * c - px * sn : x * c + px * sn) * kLog2eRsqrtD;
  }

  const int32_t *lst = vblocks + ((size_t)s * g.Hkv + h) * g.n_list;
  const int dim = tid & (kD - 1);
  const int rh = tid >> 7;                             // rows rh, rh + 2, ...
  float acc[kPgF32MaxRows / 2];
#pragma unroll
  for (int k = 0; k < kPgF32MaxRows / 2; ++k) acc[k] = 0.f;

  for (int m = m0; m < m1; ++m) {
    const int tb = kBT * m;
    if (tid < kD / 2) {
      double c, sn;
      rope_angle_f64((double)tb, inv_freq[tid], c, sn);
      base_cs[tid] = make_double2(c, sn);
    }
    if (tid == 0) {                                    // a bad entry or page is a zero block
      const int beta = lst[m];
      const bool beta_ok = beta >= 0 && beta < n_all.v[sl];
      const int page = beta_ok ? table[(size_t)s * g.max_blocks + beta] : -1;
      const bool ok = beta_ok && page >= 0 && page < g.n_pages;
      if (!ok) dev_flag(dev_err, beta_ok ? 1 : 2);
      s_page = ok ? page : -1;
    }
    __syncthreads();
    const int page = s_page;
    const size_t src = ((size_t)(page >= 0 ? page : 0) * g.Hkv + h) * (size_t)(kBT * kD);
    for (int idx = tid; idx < kBT * (kD / 2); idx += 256) {
      const int u = idx / (kD / 2), i = idx % (kD / 2);
      const bool have = page >= 0 && tb + u < V;
      const float x1 = have ? kpool[src + (size_t)u * kD + i] : 0.f;
      const float x2 = have ? kpool[src + (size_t)u * kD + 64 + i] : 0.f;
      float c, sn, y1, y2;
      rope_compose(base_cs[i].x, base_cs[i].y, offs[u][i].x, offs[u][i].y, c, sn);
      rope_rotate(x1, x2, c, sn, y1, y2);
      ks[u][i] = y1;
      ks[u][64 + i] = y2;
      if (WV) {
        float *row = kview + (((size_t)s * g.Hkv + h) * max_view + tb + u) * kD;
        row[i] = y1;
        row[64 + i] = y2;
      }
    }
    for (int idx = tid; idx < kBT * kD; idx += 256) {
      const int u = idx >> 7, d = idx & (kD - 1);
      const float v = page >= 0 && tb + u < V ? vpool[src + idx] : 0.f;
      vs[u][d] = v;
      if (WV) vview[((((size_t)s * g.Hkv + h) * (max_view / kBT) + m) * kD + d) * kBT + v_slot(u)] = v;
    }
    __syncthreads();
    for (int idx = tid; idx < R * kBT; idx += 256) {
      const int r = idx / kBT, u = idx % kBT;
      float a = -INFINITY;
      if (tb + u < V) {
        a = 0.f;
        for (int e = 0; e < kD; ++e) a = fmaf(qs[r][e], ks[u][e], a);
      }
      lg[r][u] = a;
    }
    __syncthreads();
    if (tid < R) {
      float bm = -INFINITY;
      for (int j = 0; j < kBT; ++j) bm = fmaxf(bm, lg[tid][j]);
      const float mn = fmaxf(smx[tid], bm);
      const float alpha = exp2f(smx[tid] - mn);
      float ps = 0.f;
      for (int j = 0; j < kBT; ++j) {
        const float p = exp2f(lg[tid][j] - mn);
        lg[tid][j] = p;
        ps += p;
      }
      slsum[tid] = slsum[tid] * alpha + ps;
      smx[tid] = mn;
      salpha[tid] = alpha;
    }
    __syncthreads();
    for (int k = 0; k < kPgF32MaxRows / 2; ++k) {
      const int r = rh + 2 * k;
      if (r >= R) break;
      float a = acc[k] * salpha[r];
      for (int j = 0; j < kBT; ++j) a = fmaf(lg[r][j], vs[j][dim], a);
      acc[k] = a;
    }
    __syncthreads();
  }
  for (int k = 0; k < kPgF32MaxRows / 2; ++k) {
    const int r = rh + 2 * k;
    if (r >= R) break;
    if (n_splits == 1) {
      const int t = r / g.G, gg = r % g.G;
      out[(((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD + dim] = acc[k] / slsum[r];
    } else {
      const size_t pidx = (((size_t)s * g.Hkv + h) * g.max_splits + split) * g.rows + r;
      part_o[pidx * kD + dim] = acc[k];
      if (dim == 0) part_ml[pidx] = make_float2(smx[r], slsum[r]);
    }
  }
}

}  // namespace

// Wavefronts (KV heads) per workgroup of the bf16 kernel: the largest divisor
// of Hkv up to 8, so that every wavefront has a head and no store or load in
// the block loop is guarded by one.
int paged_waves(int Hkv) {
  for (int w = kPgWaves; w > 1; --w)
    if (Hkv % w == 0) return w;
  return 1;
}

int paged_blocks_per_split(int n_sessions, int Hkv, int n_list) {
  // aim for >= 256 workgroups of 8 wavefronts; 1 .. 64 list blocks per split
  const long groups = Hkv / paged_waves(Hkv);
  long b = ((long)n_list * groups * n_sessions + 255) / 256;
  if (b < 1) b = 1;
  if (b > 64) b = 64;
  return (int)b;
}

hipError_t launch_attend_paged(int bf16, const void *q, const float *qw, float eps, const void *k_pool,
                               const void *v_pool, const int32_t *table, const int32_t *view_blocks, float *part_o,
                               float2 *part_ml, float *out, int32_t *dev_err, const SessI32 &view_tok,
                               const SessI32 &n_all, int s0, int n_sess, const PagedGeom &g, double theta,
                               void *k_view, void *v_view, int max_view, hipStream_t st) {
  int max_v = 0;
  for (int i = 0; i < n_sess; ++i) max_v = view_tok.v[i] > max_v ? view_tok.v[i] : max_v;
  const int splits = (max_v + kBT * g.bps - 1) / (kBT * g.bps);
  if (splits > 0 && !bf16) {
    const dim3 grid((unsigned)splits, (unsigned)g.Hkv, (unsigned)n_sess);
    if (k_view != nullptr)
      hipLaunchKernelGGL(k_attend_paged_f32<true>, grid, dim3(256), 0, st, (const float *)q, qw, eps,
                         (const float *)k_pool, (const float *)v_pool, table, view_blocks, part_o, part_ml, out,
                         dev_err, view_tok, n_all, s0, g, theta, (float *)k_view, (float *)v_view, max_view);
    else
      hipLaunchKernelGGL(k_attend_paged_f32<false>, grid, dim3(256), 0, st, (const float *)q, qw, eps,
                         (const float *)k_pool, (const float *)v_pool, table, view_blocks, part_o, part_ml, out,
                         dev_err, view_tok, n_all, s0, g, theta, nullptr, nullptr, max_view);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (splits > 0) {
    const int nw = paged_waves(g.Hkv);
    dim3 grid((unsigned)splits, (unsigned)(g.Hkv / nw), (unsigned)n_sess);
#define KVMEM_PAGED(NT, WV)                                                                                     \
  hipLaunchKernelGGL((k_attend_paged_bf16<NT, WV>), grid, dim3(64 * nw), 0, st, (const uint16_t *)q, qw, eps,          \
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
