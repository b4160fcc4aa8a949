// Decode attention over the materialised view: split-K flash decode.
//
// KVMem runs the model's attention over the bounded view instead of the whole
// workspace (reproduction README, 'Local reproduction': attention replacement).
// Query token t of a step sits at view position V + t, is q-RMS-normalised and
// rotated there, and attends to every view slot.
//
// bf16 path (k_attend_bf16): one workgroup of 4 wavefronts per (session, KV
// head, split of the view).  The 4 wavefronts take the split's 32-token
// blocks in turn (wavefront w: blocks w, w + 4, w + 8, ...), so that at any
// moment a workgroup reads four adjacent blocks of K and of V; each streams
// its blocks straight from HBM into matrix-core operand registers and keeps an
// online softmax; the 4 wavefronts are merged by log-sum-exp in LDS, the splits
// by k_attend_combine.  All T*G query rows of a KV head share every K/V element
// (GQA), so both products are matrix-core contractions with the rows as N:
//   S^T = K * Q^T   (v_mfma_f32_16x16x32_bf16, A = 16 tokens x 32 dims),
//   O^T = V^T * P^T (A = 16 dims x 32 tokens from the dimension-major V view).
// The S^T accumulator layout (lane = query row, 4 tokens per lane per tile) is
// exactly the P^T operand layout of the second product once the view stores
// each block's tokens in slot order sigma(u), so no shuffle or LDS transpose is
// needed between the two products, and every value a lane rescales (row max,
// row sum, O^T) belongs to that lane's own query row.  The fp32 query and the
// fp32 probabilities enter the bf16 products as a hi + lo pair of bf16 values
// (two products into one accumulator), which keeps them to ~2^-16 relative; the
// bf16 view data are exact operands.  Scores are kept in log2 units.
//
// fp32 path (k_attend_f32): a plain vector-ALU kernel with the same split and
// merge structure (logits and probabilities staged in LDS).
#include <string.h>

#include "append_common.h"
#include "attend_common.h"

namespace kvmem {

namespace {

struct KVTile {
  uint4 k[2][4];     // as load_k_lines leaves them (whole 128-byte lines per load)
  uint4 v[8];
};

__device__ __forceinline__ void load_kv_tile(KVTile &t, const uint16_t *kbase, const uint16_t *vbase, int tb,
                                             int qq, int col) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) load_k_lines(t.k[tt], kbase + (size_t)(tb + 16 * tt) * kD, qq, col);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) t.v[dt] = load_nt16(vbase + ((size_t)(tb >> 5) * kD + 16 * dt + col) * kBT + 8 * qq);
}

// One 32-token block: S^T = K Q^T, online softmax, O^T += V^T P^T.
template <int NT>
__device__ __forceinline__ void attend_tile(const KVTile &t, const bf16x8 (&qhi)[NT][4], const bf16x8 (&qlo)[NT][4],
                                            floatx4 (&o)[NT][8], float (&mrun)[NT], float (&lrun)[NT], int tb, int V,
                                            int qq, int col) {
  floatx4 sc[2][NT];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    uint4 ka[4];
    k_lines_operand(t.k[tt], ka, col);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[c]), qhi[nt][c], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[c]), qlo[nt][c], a, 0, 0, 0);
      }
      sc[tt][nt] = a;
    }
  }
  if (tb + kBT > V) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tb + 16 * tt + 4 * qq + i >= V)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sc[tt][nt][i] = -INFINITY;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float bm = fmaxf(fmaxf(fmaxf(sc[0][nt][0], sc[0][nt][1]), fmaxf(sc[0][nt][2], sc[0][nt][3])),
                     fmaxf(fmaxf(sc[1][nt][0], sc[1][nt][1]), fmaxf(sc[1][nt][2], sc[1][nt][3])));
    bm = max_xor16(bm);
    bm = max_xor32(bm);
    const float mn = fmaxf(mrun[nt], bm);
    const float alpha = exp2f(mrun[nt] - mn);
    mrun[nt] = mn;
    float p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(sc[0][nt][i] - mn);
      p[4 + i] = exp2f(sc[1][nt][i] - mn);
    }
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) psum += p[i];
    lrun[nt] = lrun[nt] * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[nt][dt] *= alpha;
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
      o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.v[dt]), phi, o[nt][dt], 0, 0, 0);
      o[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.v[dt]), plo, o[nt][dt], 0, 0, 0);
    }
  }
}

template <int NT>
__global__ __launch_bounds__(256, NT == 1 ? 2 : 1) void k_attend_bf16(
    const uint16_t *__restrict__ q, const float *__restrict__ qw, float eps, const uint16_t *__restrict__ kview,
    const uint16_t *__restrict__ vview, float *__restrict__ part_o, float2 *__restrict__ part_ml,
    float *__restrict__ out, SessI32 view_tok, int s0, AttendGeom g, double theta) {
  constexpr int RP = 16 * NT;
  constexpr int kPitch = kD + 4;
  __shared__ float cs_tab[kQprepMaxT][kD / 2][2];
  __shared__ float sm[4][RP];
  __shared__ float sls[4][RP];
  __shared__ float so[4][RP * kPitch];

  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int split = blockIdx.x;
  const int V = view_tok.v[sl];
  const int split_tok = 4 * g.tpw;
  const int start = split * split_tok;
  if (start >= V) return;
  const int n_splits = (V + split_tok - 1) / split_tok;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qq = lane >> 4;
  const int col = lane & 15;
  const size_t head = (size_t)s * g.Hkv + h;
  const uint16_t *kbase = kview + head * (size_t)g.max_view * kD;
  const uint16_t *vbase = vview + head * (size_t)g.max_view * kD;
  // this wavefront's first block, and the end of the split
  const int tok0 = start + wave * kBT;
  const int tok1 = min(V, start + split_tok);

  // Loads first, in the order they are needed: the raw query rows of this
  // lane, then the wavefront's first K/V tile.  The RoPE table is computed
  // while they are in flight.
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
  KVTile tile;
  if (tok0 < tok1) load_kv_tile(tile, kbase, vbase, tok0, qq, col);
  {
    const int n_t = (g.rows + g.G - 1) / g.G;
    for (int idx = tid; idx < n_t * (kD / 2); idx += 256) {
      const int t = idx / (kD / 2), i = idx % (kD / 2);
      rope_cos_sin((double)(V + t), rope_inv_freq(i, theta), cs_tab[t][i][0], cs_tab[t][i][1]);
    }
  }
  __syncthreads();
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
  // One 32-token tile in flight per wavefront: multiply the tile, then request
  // the wavefront's next one, four blocks on.  (Holding a second tile in flight
  // per wavefront measured markedly slower on this part.  Each wavefront
  // walking a run of its own, 64 KiB of K and of V away from its neighbours',
  // measured 191 against 168 us per call at 1M tokens.)
  for (int tb = tok0; tb < tok1; tb += 4 * kBT) {
    attend_tile<NT>(tile, qhi, qlo, o, mrun, lrun, tb, V, qq, col);
    if (tb + 4 * kBT < tok1) {
      load_kv_tile(tile, kbase, vbase, tb + 4 * kBT, qq, col);
      // keep all 16 K and V loads of the tile together (the scheduler would
      // otherwise sink the V loads below the first product and expose a
      // second memory latency per tile)
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- merge the 4 wavefronts (log-sum-exp) ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    lrun[nt] = sum_xor16(lrun[nt]);
    lrun[nt] = sum_xor32(lrun[nt]);
    const int row = nt * 16 + col;
    if (qq == 0) {
      sm[wave][row] = mrun[nt];
      sls[wave][row] = lrun[nt];
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[wave][row * kPitch + 16 * dt + 4 * qq + i] = o[nt][dt][i];
  }
  __syncthreads();
  for (int idx = tid; idx < g.rows * kD; idx += 256) {
    const int row = idx >> 7;
    const int dim = idx & (kD - 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][row]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm[w][row];
      if (mw != -INFINITY) {
        const float f = exp2f(mw - M);
        num += f * so[w][row * kPitch + dim];
        den += f * sls[w][row];
      }
    }
    if (n_splits == 1) {
      const int t = row / g.G, gg = row % g.G;
      out[(((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD + dim] = num / den;
    } else {
      const size_t pidx = (head * g.max_splits + split) * g.rows + row;
      part_o[pidx * kD + dim] = num;
      if (dim == 0) part_ml[pidx] = make_float2(M, den);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
constexpr int kF32MaxRows = 64;
constexpr int kF32Tile = 64;

__global__ __launch_bounds__(256) void k_attend_f32(const float *__restrict__ q, const float *__restrict__ qw, float eps,
                                                    const float *__restrict__ kview, const float *__restrict__ vview,
                                                    float *__restrict__ part_o, float2 *__restrict__ part_ml,
                                                    float *__restrict__ out, SessI32 view_tok, int s0, AttendGeom g,
                                                    double theta) {
  __shared__ double inv_freq[kD / 2];
  __shared__ float qs[kF32MaxRows][kD + 1];
  __shared__ float lg[kF32MaxRows][kF32Tile + 1];
  __shared__ float srs[kF32MaxRows], smx[kF32MaxRows], slsum[kF32MaxRows], salpha[kF32MaxRows];

  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int split = blockIdx.x;
  const int V = view_tok.v[sl];
  const int split_tok = 4 * g.tpw;
  const int start = split * split_tok;
  if (start >= V) return;
  const int end = min(V, start + split_tok);
  const int n_splits = (V + split_tok - 1) / split_tok;
  const int tid = threadIdx.x;
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
  for (int idx = tid; idx < R * kD; idx += 256) {
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
  __syncthreads();

  const size_t head = (size_t)s * g.Hkv + h;
  const float *kbase = kview + head * (size_t)g.max_view * kD;
  const float *vbase = vview + head * (size_t)g.max_view * kD;
  const int dim = tid & (kD - 1);
  const int rh = tid >> 7;                       // rows rh, rh + 2, ...
  float acc[kF32MaxRows / 2];
#pragma unroll
  for (int k = 0; k < kF32MaxRows / 2; ++k) acc[k] = 0.f;

  for (int tb = start; tb < end; tb += kF32Tile) {
    const int jt = tid & (kF32Tile - 1);
    const int tok = tb + jt;
    for (int r = tid >> 6; r < R; r += 4) {
      float a = -INFINITY;
      if (tok < end) {
        const float *kr = kbase + (size_t)tok * kD;
        a = 0.f;
        for (int e = 0; e < kD; ++e) a = fmaf(qs[r][e], kr[e], a);
      }
      lg[r][jt] = a;
    }
    __syncthreads();
    if (tid < R) {
      float bm = -INFINITY;
      for (int j = 0; j < kF32Tile; ++j) bm = fmaxf(bm, lg[tid][j]);
      const float mn = fmaxf(smx[tid], bm);
      const float alpha = exp2f(smx[tid] - mn);
      float ps = 0.f;
      for (int j = 0; j < kF32Tile; ++j) {
        const float p = exp2f(lg[tid][j] - mn);
        lg[tid][j] = p;
        ps += p;
      }
      slsum[tid] = slsum[tid] * alpha + ps;
      smx[tid] = mn;
      salpha[tid] = alpha;
    }
    __syncthreads();
    const int nt = min(kF32Tile, end - tb);
    for (int k = 0; k < kF32MaxRows / 2; ++k) {
      const int r = rh + 2 * k;
      if (r >= R) break;
      float a = acc[k] * salpha[r];
      for (int j = 0; j < nt; ++j) {
        const int tk = tb + j;
        a = fmaf(lg[r][j], vbase[((size_t)(tk >> 5) * kD + dim) * kBT + v_slot(tk & 31)], a);
      }
      acc[k] = a;
    }
    __syncthreads();
  }
  for (int k = 0; k < kF32MaxRows / 2; ++k) {
    const int r = rh + 2 * k;
    if (r >= R) break;
    if (n_splits == 1) {
      const int t = r / g.G, gg = r % g.G;
      out[(((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD + dim] = acc[k] / slsum[r];
    } else {
      const size_t pidx = (head * g.max_splits + split) * g.rows + r;
      part_o[pidx * kD + dim] = acc[k];
      if (dim == 0) part_ml[pidx] = make_float2(smx[r], slsum[r]);
    }
  }
}

// ---------------------------------------------------------------------------
// Selection-quality diagnostic: the share of full attention over the whole
// history that the listed blocks capture.  Full attention here is attention
// over a full-budget view: every history token j rotated at its own position
// and rounded to storage, the query token t at position N + t.
//
// k_mass_bf16: one workgroup of 8 wavefronts per (session, chunk of history
// blocks, group of 8 KV heads); wavefront w serves KV head 8 * group + w.  For
// each block the workgroup first forms the 32 x 64 RoPE (cos, sin) table of the
// block's positions (shared by the 8 heads), then each wavefront rotates the
// pre-RoPE K tile of its head, read straight from the page in the A-operand
// lane layout (a dim and its +-64 partner sit in chunks c and c ^ 2 of the same
// lane), rounds it to bf16 and forms S^T = K Q^T on the matrix cores with the
// same query operands as the view attention.  Online softmax statistics (log2
// units) are kept over all tokens and over the tokens of listed blocks; each
// wavefront writes one (m_all, l_all, m_sel, l_sel) per query row and chunk.
// k_mass_combine folds the chunks in order into mass = l_sel / l_all (after
// rescaling) and the log-sum-exp of the logits.
// ---------------------------------------------------------------------------
constexpr int kMassWaves = 8;
constexpr int kMassMaxChunk = 256;

__device__ __forceinline__ void mass_fold(float &m, float &l, float bm, float bl) {
  if (bm == -INFINITY) return;
  const float mn = fmaxf(m, bm);
  l = l * exp2f(m - mn) + bl * exp2f(bm - mn);
  m = mn;
}

template <int NT>
__global__ __launch_bounds__(512) void k_mass_bf16(const uint16_t *__restrict__ q, const float *__restrict__ qw,
                                                   float eps, const uint16_t *__restrict__ kpool,
                                                   const int32_t *__restrict__ table,
                                                   const int32_t *__restrict__ vblocks, float4 *__restrict__ part,
                                                   int32_t *dev_err, SessI32 n_tok, int s0, MassGeom g,
                                                   double theta) {
  __shared__ double inv_freq[kD / 2];
  __shared__ double step_cs[kD / 2][2];                  // cos, sin of 32 * phi_i
  __shared__ float cs_tab[kQprepMaxT][kD / 2][2];        // query positions N + t
  // (cos, sin) of the current block's positions; rows padded by one pair so
  // that the 16 tokens one read instruction touches fall in different banks
  __shared__ float ktab[2][kBT][kD / 2 + 1][2];
  __shared__ uint8_t listed[kMassWaves][kMassMaxChunk];

  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int chunk = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qq = lane >> 4;
  const int col = lane & 15;
  const int h = blockIdx.y * kMassWaves + wave;
  const bool head_ok = h < g.Hkv;
  const int N = n_tok.v[sl];
  const int n_all = (N + kBT - 1) / kBT;
  const int b0 = chunk * g.chunk;
  if (b0 >= n_all) return;                             // uniform over the workgroup
  const int b1 = min(n_all, b0 + g.chunk);

  if (tid < kD / 2) {
    inv_freq[tid] = rope_inv_freq(tid, theta);
    sincos((double)kBT * inv_freq[tid], &step_cs[tid][1], &step_cs[tid][0]);
  }
  for (int i = tid; i < kMassWaves * kMassMaxChunk; i += 512) listed[i / kMassMaxChunk][i % kMassMaxChunk] = 0;

  // raw query rows of this wavefront's head (as the view attention)
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
  __syncthreads();                                     // inv_freq, cleared flags

  // listed blocks of this chunk: the list's valid entries ascend (selected,
  // then recent, then -1), so a coarse probe per lane finds the segment that
  // holds the first entry >= b0, and the chunk's entries follow it
  if (head_ok && g.n_list > 0) {
    const int32_t *lst = vblocks + ((size_t)s * g.Hkv + h) * g.n_list;
    const int step = (g.n_list + 63) / 64;
    const int probe = lane * step;
    const uint32_t e = probe < g.n_list ? (uint32_t)lst[probe] : 0xffffffffu;   // -1 -> above every block
    const uint64_t below = __ballot(probe < g.n_list && e < (uint32_t)b0);
    const int start = below == 0 ? 0 : (63 - __clzll(below)) * step;
    for (int k = lane; k < step + g.chunk; k += 64) {
      const int idx = start + k;
      if (idx < g.n_list) {
        const int v = lst[idx];
        if (v >= b0 && v < b1) listed[wave][v - b0] = 1;
      }
    }
  }
  {
    const int n_t = (g.rows + g.G - 1) / g.G;
    for (int idx = tid; idx < n_t * (kD / 2); idx += 512) {
      const int t = idx / (kD / 2), i = idx % (kD / 2);
      rope_cos_sin((double)(N + t), inv_freq[i], cs_tab[t][i][0], cs_tab[t][i][1]);
    }
  }
  __syncthreads();
  bf16x8 qhi[NT][4], qlo[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) build_q_operands(x[nt], rvalid[nt], trow[nt], qq, qw, eps, cs_tab, qhi[nt], qlo[nt]);

  float m_all[NT], l_all[NT], m_sel[NT], l_sel[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_all[nt] = m_sel[nt] = -INFINITY;
    l_all[nt] = l_sel[nt] = 0.f;
  }
  const int32_t *trow_tab = table + (size_t)s * g.max_blocks;
  auto tile_src = [&](int beta, bool &ok) -> const uint16_t * {
    const int page = trow_tab[beta];
    ok = head_ok && page >= 0 && page < g.n_pages;
    return kpool + ((size_t)(ok ? page : 0) * g.Hkv + (head_ok ? h : 0)) * (size_t)(kBT * kD);
  };
  uint4 kr[2][4];
  bool ok_cur;
  const uint16_t *src = tile_src(b0, ok_cur);
  // (whole 128-byte lines: load_k_lines, then k_lines_operand)
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) load_k_lines(kr[tt], src + (size_t)(16 * tt) * kD, qq, col);

  // RoPE table of the current block's positions, shared by the 8 heads: each
  // thread owns 4 of its 32 x 64 entries, exact at the chunk's first block
  // and advanced one block (angle + 32 phi_i) per step by an fp64 rotation.
  constexpr int kOwn = kBT * (kD / 2) / 512;
  double tc[kOwn], ts[kOwn];
#pragma unroll
  for (int k = 0; k < kOwn; ++k) {
    const int idx = tid + 512 * k;
    const int u = idx / (kD / 2), i = idx % (kD / 2);
    float c, sn;
    rope_cos_sin((double)(kBT * b0 + u), inv_freq[i], c, sn);
    tc[k] = c;
    ts[k] = sn;
  }

  for (int beta = b0; beta < b1; ++beta) {
    const int buf = (beta - b0) & 1;
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int idx = tid + 512 * k;
      ktab[buf][idx / (kD / 2)][idx % (kD / 2)][0] = (float)tc[k];
      ktab[buf][idx / (kD / 2)][idx % (kD / 2)][1] = (float)ts[k];
      const double sc = step_cs[idx % (kD / 2)][0], ss = step_cs[idx % (kD / 2)][1];
      const double c2 = tc[k] * sc - ts[k] * ss;
      ts[k] = ts[k] * sc + tc[k] * ss;
      tc[k] = c2;
    }
    __syncthreads();
    const bool ok = ok_cur;
    if (!ok && head_ok && lane == 0) dev_flag(dev_err, 1);
    uint4 cur[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) k_lines_operand(kr[tt], cur[tt], col);
    if (beta + 1 < b1) {
      src = tile_src(beta + 1, ok_cur);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) load_k_lines(kr[tt], src + (size_t)(16 * tt) * kD, qq, col);
    }
    if (!ok) continue;                                 // per wavefront: no barrier below
    // rotate K at its own positions and round to bf16: A operands
    bf16x8 ka[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int u = 16 * tt + col;
      float kv[4][8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t e[4] = {cur[tt][c].x, cur[tt][c].y, cur[tt][c].z, cur[tt][c].w};
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
            const float cs = ktab[buf][u][ip][0], sn = ktab[buf][u][ip][1];
            y1[k] = kv[c][j + k] * cs - kv[c + 2][j + k] * sn;
            y2[k] = kv[c + 2][j + k] * cs + kv[c][j + k] * sn;
          }
          w[c][j / 2] = pack_bf16x2(y1[0], y1[1]);
          w[c + 2][j / 2] = pack_bf16x2(y2[0], y2[1]);
        }
#pragma unroll
      for (int c = 0; c < 4; ++c) ka[tt][c] = as_bf16x8(make_uint4(w[c][0], w[c][1], w[c][2], w[c][3]));
    }
    const bool sel = listed[wave][beta - b0] != 0;
    const int tb = kBT * beta;
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
      if (tb + kBT > N) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tb + 16 * tt + 4 * qq + i >= N) sc[tt][i] = -INFINITY;
      }
      float bm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      bm = max_xor16(bm);
      bm = max_xor32(bm);                              // block max of the row, in every lane of the row
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) ps += exp2f(sc[0][i] - bm) + exp2f(sc[1][i] - bm);
      mass_fold(m_all[nt], l_all[nt], bm, ps);        // lane-partial sums, common maxima
      if (sel) mass_fold(m_sel[nt], l_sel[nt], bm, ps);
    }
  }
  if (!head_ok) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float la = sum_xor32(sum_xor16(l_all[nt]));
    const float ls = sum_xor32(sum_xor16(l_sel[nt]));
    const int row = nt * 16 + col;
    if (qq == 0 && row < g.rows)
      part[(((size_t)s * g.Hkv + h) * g.n_chunks + chunk) * g.rows + row] = make_float4(m_all[nt], la, m_sel[nt], ls);
  }
}

// One wavefront per (session, KV head, query row): folds the chunks' partials
// (lane c takes chunks c, c + 64, ...; then a fixed butterfly order).
// fp32 workspaces: a vector-ALU kernel with the same chunks and partials.  One
// 256-thread workgroup per (session, chunk of history blocks, KV head); each
// history key is rotated at its own position in fp32 (the angle reduced in
// fp64, its sine and cosine in fp32, as the query angles), which is the fp32
// storage rounding, and the logits are the view attention's fp32 dot products.
__global__ __launch_bounds__(256) void k_mass_f32(const float *__restrict__ q, const float *__restrict__ qw,
                                                  float eps, const float *__restrict__ kpool,
                                                  const int32_t *__restrict__ table,
                                                  const int32_t *__restrict__ vblocks, float4 *__restrict__ part,
                                                  int32_t *dev_err, SessI32 n_tok, int s0, MassGeom g,
                                                  double theta) {
  __shared__ double inv_freq[kD / 2];
  __shared__ float qs[kF32MaxRows][kD + 1];
  __shared__ float ks[kBT][kD + 1];
  __shared__ float lg[kF32MaxRows][kBT + 1];
  __shared__ float srs[kF32MaxRows];
  __shared__ uint8_t listed[kMassMaxChunk];
  __shared__ int s_page;

  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int chunk = blockIdx.x;
  const int tid = threadIdx.x;
  const int N = n_tok.v[sl];
  const int n_all = (N + kBT - 1) / kBT;
  const int b0 = chunk * g.chunk;
  if (b0 >= n_all) return;                             // uniform over the workgroup
  const int b1 = min(n_all, b0 + g.chunk);
  const int R = g.rows;
  if (tid < kD / 2) inv_freq[tid] = rope_inv_freq(tid, theta);
  if (tid < R) {
    const int t = tid / g.G, gg = tid % g.G;
    const float *src = q + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD;
    float ss = 0.f;
    for (int e = 0; e < kD; ++e) ss += src[e] * src[e];
    srs[tid] = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  }
  for (int i = tid; i < kMassMaxChunk; i += 256) listed[i] = 0;
  __syncthreads();
  {
    const int32_t *lst = vblocks + ((size_t)s * g.Hkv + h) * g.n_list;
    for (int idx = tid; idx < g.n_list; idx += 256) {
      const int v = lst[idx];
      if (v >= b0 && v < b1) listed[v - b0] = 1;
    }
  }
  for (int idx = tid; idx < R * kD; idx += 256) {       // q~ rotated at N + t, in log2 units
    const int r = idx >> 7, dim = idx & (kD - 1);
    const int t = r / g.G, gg = r % g.G;
    const float *src = q + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD;
    const int i = dim & 63;
    const int pd = dim < 64 ? dim + 64 : dim - 64;
    const float x = src[dim] * srs[r] * qw[dim];
    const float px = src[pd] * srs[r] * qw[pd];
    float c, sn;
    rope_cos_sin((double)(N + t), inv_freq[i], c, sn);
    qs[r][dim] = (dim < 64 ? x * c - px * sn : x * c + px * sn) * kLog2eRsqrtD;
  }
  float m_all = -INFINITY, l_all = 0.f, m_sel = -INFINITY, l_sel = 0.f;   // row tid's statistics
  for (int beta = b0; beta < b1; ++beta) {
    if (tid == 0) {
      const int page = table[(size_t)s * g.max_blocks + beta];
      const bool ok = page >= 0 && page < g.n_pages;
      if (!ok) dev_flag(dev_err, 1);
      s_page = ok ? page : -1;
    }
    __syncthreads();
    const int page = s_page;
    if (page < 0) continue;                            // uniform: a bad page is skipped
    const size_t src = ((size_t)page * g.Hkv + h) * (size_t)(kBT * kD);
    for (int idx = tid; idx < kBT * (kD / 2); idx += 256) {
      const int u = idx / (kD / 2), i = idx % (kD / 2);
      const int pos = kBT * beta + u;
      const bool have = pos < N;
      const float x1 = have ? kpool[src + (size_t)u * kD + i] : 0.f;
      const float x2 = have ? kpool[src + (size_t)u * kD + 64 + i] : 0.f;
      float c, sn, y1, y2;
      rope_cos_sin((double)pos, inv_freq[i], c, sn);
      rope_rotate(x1, x2, c, sn, y1, y2);
      ks[u][i] = y1;
      ks[u][64 + i] = y2;
    }
    __syncthreads();
    for (int idx = tid; idx < R * kBT; idx += 256) {
      const int r = idx / kBT, u = idx % kBT;
      float a = -INFINITY;
      if (kBT * beta + u < N) {
        a = 0.f;
        for (int e = 0; e < kD; ++e) a = fmaf(qs[r][e], ks[u][e], a);
      }
      lg[r][u] = a;
    }
    __syncthreads();
    if (tid < R) {
      float bm = -INFINITY;
      for (int j = 0; j < kBT; ++j) bm = fmaxf(bm, lg[tid][j]);
      float bl = 0.f;
      for (int j = 0; j < kBT; ++j) bl += exp2f(lg[tid][j] - bm);
      mass_fold(m_all, l_all, bm, bl);
      if (listed[beta - b0]) mass_fold(m_sel, l_sel, bm, bl);
    }
    __syncthreads();
  }
  if (tid < R) part[(((size_t)s * g.Hkv + h) * g.n_chunks + chunk) * g.rows + tid] = make_float4(m_all, l_all, m_sel, l_sel);
}

__global__ __launch_bounds__(64) void k_mass_combine(const float4 *__restrict__ part, float *__restrict__ mass,
                                                     float *__restrict__ lse, SessI32 n_tok, int s0, MassGeom g) {
  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const int n_all = (n_tok.v[sl] + kBT - 1) / kBT;
  const int nc = (n_all + g.chunk - 1) / g.chunk;
  float ma = -INFINITY, la = 0.f, ms = -INFINITY, ls = 0.f;
  for (int c = lane; c < nc; c += 64) {
    const float4 p = part[(((size_t)s * g.Hkv + h) * g.n_chunks + c) * g.rows + row];
    mass_fold(ma, la, p.x, p.y);
    mass_fold(ms, ls, p.z, p.w);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float oma = __shfl_xor(ma, off, 64), ola = __shfl_xor(la, off, 64);
    const float oms = __shfl_xor(ms, off, 64), ols = __shfl_xor(ls, off, 64);
    // both partners fold the same two values in the same order (lower lane first)
    float am = (lane & off) ? oma : ma, al = (lane & off) ? ola : la;
    float bm = (lane & off) ? ma : oma, bl = (lane & off) ? la : ola;
    mass_fold(am, al, bm, bl);
    ma = am;
    la = al;
    float sm_ = (lane & off) ? oms : ms, sl_ = (lane & off) ? ols : ls;
    float tm = (lane & off) ? ms : oms, tl = (lane & off) ? ls : ols;
    mass_fold(sm_, sl_, tm, tl);
    ms = sm_;
    ls = sl_;
  }
  if (lane == 0) {
    const int t = row / g.G, gg = row % g.G;
    const size_t o = ((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg;
    const float m = (ms == -INFINITY || la == 0.f) ? 0.f : ls * exp2f(ms - ma) / la;
    mass[o] = m;
    if (lse) lse[o] = la == 0.f ? -INFINITY : (ma + log2f(la)) * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials of one (session, KV head, query
// row), one workgroup per quarter of the row's 128 dimensions: 256 threads =
// 32 split groups x 8 float4 slices of the quarter.  Each thread folds every
// 32nd split with an online rescale (no separate max and sum passes, eight
// splits in flight), then the 32 groups are merged by a fixed tree (three
// lane exchanges inside each wavefront, then its four wavefronts in LDS), so
// the result is deterministic.  (Folding the 32 groups in sequence in eight
// threads took ~5 us longer per call at 1M tokens.)
// ---------------------------------------------------------------------------
constexpr int kCombGroups = 32;
constexpr int kCombQuarters = 4;

// A partial softmax state (running max m, sum l, weighted values a) and the
// merge of two.  Both lanes of an exchange merge the pair (their results may
// differ in the last bit with the operands' order); the output takes the
// states of fixed lanes, so it is the same on every run.
struct CombState {
  float m, l;
  float4 a;
};
__device__ __forceinline__ CombState comb_merge(const CombState &x, const CombState &y) {
  const float M = fmaxf(x.m, y.m);
  if (M == -INFINITY) return CombState{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  const float fx = exp2f(x.m - M), fy = exp2f(y.m - M);   // exp2(-inf) = 0 for an empty side
  CombState r;
  r.m = M;
  r.l = x.l * fx + y.l * fy;
  r.a = make_float4(x.a.x * fx + y.a.x * fy, x.a.y * fx + y.a.y * fy, x.a.z * fx + y.a.z * fy,
                    x.a.w * fx + y.a.w * fy);
  return r;
}
// merge with the state of lane ^ 8 (DPP), ^ 16 or ^ 32 (lane permutes)
__device__ __forceinline__ CombState comb_xor8(const CombState &v) {
  CombState o;
  o.m = dpp_f32<kDppRor8>(v.m);
  o.l = dpp_f32<kDppRor8>(v.l);
  o.a = make_float4(dpp_f32<kDppRor8>(v.a.x), dpp_f32<kDppRor8>(v.a.y), dpp_f32<kDppRor8>(v.a.z),
                    dpp_f32<kDppRor8>(v.a.w));
  return comb_merge(v, o);
}
template <bool X32>
__device__ __forceinline__ CombState comb_xor_half(const CombState &v) {
  float p[6] = {v.m, v.l, v.a.x, v.a.y, v.a.z, v.a.w}, q[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const auto r = X32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(p[i]), __float_as_uint(p[i]), false, false)
                       : __builtin_amdgcn_permlane16_swap(__float_as_uint(p[i]), __float_as_uint(p[i]), false, false);
    p[i] = __uint_as_float(r[0]);
    q[i] = __uint_as_float(r[1]);
  }
  return comb_merge(CombState{p[0], p[1], make_float4(p[2], p[3], p[4], p[5])},
                    CombState{q[0], q[1], make_float4(q[2], q[3], q[4], q[5])});
}

// One appended token of session s0 + sl, run by a workgroup of a merge launch.
__device__ __forceinline__ void append_in_merge(const AppendArgs &ap, const SessI32 &view_tok, int s0, int sl, int t) {
  __shared__ float2 cs_tok[kD / 2];
  if (ap.bf16)
    append_token<uint16_t>((uint16_t *)ap.kpool, (uint16_t *)ap.vpool, ap.table, (const uint16_t *)ap.knew,
                           (const uint16_t *)ap.vnew, ap.T_new, (uint16_t *)ap.kview, (uint16_t *)ap.vview,
                           ap.dev_err, ap.n_tok.v[sl], view_tok.v[sl], s0 + sl, t, ap.Hkv, ap.max_blocks, ap.n_pages,
                           ap.max_view, ap.theta, cs_tok);
  else
    append_token<float>((float *)ap.kpool, (float *)ap.vpool, ap.table, (const float *)ap.knew,
                        (const float *)ap.vnew, ap.T_new, (float *)ap.kview, (float *)ap.vview, ap.dev_err,
                        ap.n_tok.v[sl], view_tok.v[sl], s0 + sl, t, ap.Hkv, ap.max_blocks, ap.n_pages, ap.max_view, ap.theta,
                        cs_tok);
}

__global__ __launch_bounds__(256) void k_attend_combine(const float *__restrict__ part_o,
                                                        const float2 *__restrict__ part_ml, float *__restrict__ out,
                                                        SessI32 view_tok, int s0, AttendGeom g, AppendArgs ap) {
  __shared__ float4 acc_s[kCombGroups][8];
  __shared__ float m_s[kCombGroups], l_s[kCombGroups];
  if (ap.T_new > 0 && (int)blockIdx.x >= (int)gridDim.x - ap.T_new) {
    if (blockIdx.y == 0) append_in_merge(ap, view_tok, s0, (int)blockIdx.z, (int)blockIdx.x - ((int)gridDim.x - ap.T_new));
    return;
  }
  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int row = blockIdx.x / kCombQuarters;
  const int quarter = blockIdx.x % kCombQuarters;
  const int tid = threadIdx.x;
  const int V = view_tok.v[sl];
  const int split_tok = 4 * g.tpw;
  const int n = (V + split_tok - 1) / split_tok;
  if (n == 1) return;                     // written by the attention kernel itself
  const int t = row / g.G, gg = row % g.G;
  float *dst = out + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD + quarter * (kD / kCombQuarters);
  if (n == 0) {
    if (tid < kD / kCombQuarters) dst[tid] = 0.f;
    return;
  }
  const size_t head = (size_t)s * g.Hkv + h;
  const size_t base = head * g.max_splits * g.rows + row;     // + i * rows
  const int sg = tid >> 3, q4 = tid & 7;
  const int slice = quarter * 8 + q4;                         // float4 slice of the row
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fold = [&](float2 ml, float4 v) {
    if (ml.x == -INFINITY) return;
    const float mn = fmaxf(m, ml.x);
    const float a = exp2f(m - mn), b = exp2f(ml.x - mn);
    l = l * a + ml.y * b;
    acc.x = acc.x * a + v.x * b; acc.y = acc.y * a + v.y * b;
    acc.z = acc.z * a + v.z * b; acc.w = acc.w * a + v.w * b;
    m = mn;
  };
  int i = sg;
  for (; i + 7 * kCombGroups < n; i += 8 * kCombGroups) {
    float2 ml[8];
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t pidx = base + (size_t)(i + kCombGroups * u) * g.rows;
      ml[u] = part_ml[pidx];
      v[u] = reinterpret_cast<const float4 *>(part_o + pidx * kD)[slice];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) fold(ml[u], v[u]);
  }
  for (; i + 3 * kCombGroups < n; i += 4 * kCombGroups) {
    float2 ml[4];
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t pidx = base + (size_t)(i + kCombGroups * u) * g.rows;
      ml[u] = part_ml[pidx];
      v[u] = reinterpret_cast<const float4 *>(part_o + pidx * kD)[slice];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) fold(ml[u], v[u]);
  }
  for (; i < n; i += kCombGroups) {
    const size_t pidx = base + (size_t)i * g.rows;
    fold(part_ml[pidx], reinterpret_cast<const float4 *>(part_o + pidx * kD)[slice]);
  }
  // the 32 groups of a slice: a fixed tree, eight groups per wavefront over
  // the lanes (sg = 8 wave + lane / 8), then the four wavefronts in LDS
  CombState st{m, l, acc};
  st = comb_xor8(st);
  st = comb_xor_half<false>(st);
  st = comb_xor_half<true>(st);
  const int wave = tid >> 6;
  if ((tid & 63) < 8) {
    acc_s[wave][q4] = st.a;
    if (q4 == 0) {
      m_s[wave] = st.m;
      l_s[wave] = st.l;
    }
  }
  __syncthreads();
  if (tid < 8) {
    CombState w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = CombState{m_s[j], l_s[j], acc_s[j][tid]};
    const CombState r = comb_merge(comb_merge(w[0], w[1]), comb_merge(w[2], w[3]));
    const float inv = 1.0f / r.l;
    reinterpret_cast<float4 *>(dst)[tid] = make_float4(r.a.x * inv, r.a.y * inv, r.a.z * inv, r.a.w * inv);
  }
}

// At most kCombGroups splits per row (short views, or long runs per
// wavefront): one thread per (query row, float4 slice of the row) folds the
// row's splits in split order with k_attend_combine's online rescale,
// kNarrowRows rows per workgroup.
constexpr int kNarrowRows = 8;

__global__ __launch_bounds__(256) void k_attend_combine_narrow(const float *__restrict__ part_o,
                                                               const float2 *__restrict__ part_ml,
                                                               float *__restrict__ out, SessI32 view_tok, int s0,
                                                               AttendGeom g, AppendArgs ap) {
  if (ap.T_new > 0 && (int)blockIdx.x >= (int)gridDim.x - ap.T_new) {
    if (blockIdx.y == 0) append_in_merge(ap, view_tok, s0, (int)blockIdx.z, (int)blockIdx.x - ((int)gridDim.x - ap.T_new));
    return;
  }
  const int sl = blockIdx.z;
  const int s = s0 + sl;
  const int h = blockIdx.y;
  const int row = blockIdx.x * kNarrowRows + (threadIdx.x >> 5);
  const int slice = threadIdx.x & 31;                           // float4 slice of the row
  if (row >= g.rows) return;
  const int V = view_tok.v[sl];
  const int split_tok = 4 * g.tpw;
  const int n = (V + split_tok - 1) / split_tok;
  if (n == 1) return;                     // written by the attention kernel itself
  const int t = row / g.G, gg = row % g.G;
  float4 *dst = reinterpret_cast<float4 *>(out + (((size_t)s * g.Tq + t) * g.Hq + (size_t)h * g.G + gg) * kD);
  if (n == 0) {
    dst[slice] = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const size_t base = ((size_t)s * g.Hkv + h) * g.max_splits * g.rows + row;
  float m = -INFINITY, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < n; i0 += 8) {
    float2 ml[8];
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t pidx = base + (size_t)min(i0 + u, n - 1) * g.rows;
      ml[u] = part_ml[pidx];
      v[u] = reinterpret_cast<const float4 *>(part_o + pidx * kD)[slice];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u >= n || ml[u].x == -INFINITY) continue;
      const float mn = fmaxf(m, ml[u].x);
      const float a = exp2f(m - mn), b = exp2f(ml[u].x - mn);
      l = l * a + ml[u].y * b;
      acc.x = acc.x * a + v[u].x * b; acc.y = acc.y * a + v[u].y * b;
      acc.z = acc.z * a + v[u].z * b; acc.w = acc.w * a + v[u].w * b;
      m = mn;
    }
  }
  const float inv = 1.0f / l;
  dst[slice] = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

}  // namespace

int attend_tokens_per_wave(int n_sessions, int Hkv, int max_view, int rows) {
  // Up to 16 query rows per KV head (two workgroups per CU): aim for >= 512
  // workgroups at the largest view (one round on 256 CUs), 32..1024 tokens per
  // wavefront (1M tokens: 2048 workgroups of 8 blocks per wavefront measured
  // 181 us, 1024 of 16: 174 us, 512 of 32: 168 us, 256 of 64: 176 us).  More
  // rows (one workgroup per CU, whose prologue and merge are larger): >= 256
  // workgroups, up to 512 tokens per wavefront (measured: 16 sessions of
  // 4096-token views with 32 rows, 166 us at the first sizing, 80 us here).
  const long target = rows <= 16 ? 512L : 256L;
  const long work = (long)max_view * n_sessions * Hkv;
  long tpw_blocks = (work + target * 4 * kBT - 1) / (target * 4 * kBT);
  if (tpw_blocks < 1) tpw_blocks = 1;
  if (tpw_blocks > (rows <= 16 ? 32 : 16)) tpw_blocks = rows <= 16 ? 32 : 16;
  return (int)tpw_blocks * kBT;
}

int attend_max_splits(int max_view, int tpw) { return (max_view + 4 * tpw - 1) / (4 * tpw); }

hipError_t launch_attend(int bf16, const void *q, const float *qw, float eps, const void *k_view,
                         const void *v_view, float *part_o, float2 *part_ml, float *out,
                         const SessI32 &view_tok, int s0, int n_sess, const AttendGeom &g, double theta,
                         hipStream_t st, const AppendArgs *ap) {
  int max_v = 0;
  for (int i = 0; i < n_sess; ++i) max_v = view_tok.v[i] > max_v ? view_tok.v[i] : max_v;
  const int splits = max_v > 0 ? (max_v + 4 * g.tpw - 1) / (4 * g.tpw) : 0;
  if (splits > 0) {
    dim3 grid((unsigned)splits, (unsigned)g.Hkv, (unsigned)n_sess);
    if (!bf16) {
      hipLaunchKernelGGL(k_attend_f32, grid, dim3(256), 0, st, (const float *)q, qw, eps, (const float *)k_view,
                         (const float *)v_view, part_o, part_ml, out, view_tok, s0, g, theta);
    } else if (g.rows <= 16) {
      hipLaunchKernelGGL(k_attend_bf16<1>, grid, dim3(256), 0, st, (const uint16_t *)q, qw, eps,
                         (const uint16_t *)k_view, (const uint16_t *)v_view, part_o, part_ml, out, view_tok, s0, g,
                         theta);
    } else {
      hipLaunchKernelGGL(k_attend_bf16<2>, grid, dim3(256), 0, st, (const uint16_t *)q, qw, eps,
                         (const uint16_t *)k_view, (const uint16_t *)v_view, part_o, part_ml, out, view_tok, s0, g,
                         theta);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_attend_combine(part_o, part_ml, out, view_tok, s0, n_sess, g, st, ap);
}

hipError_t launch_attend_combine(const float *part_o, const float2 *part_ml, float *out, const SessI32 &view_tok,
                                 int s0, int n_sess, const AttendGeom &g, hipStream_t st, const AppendArgs *ap) {
  AppendArgs none;
  memset(&none, 0, sizeof(none));
  const AppendArgs &a = ap != nullptr ? *ap : none;
  const unsigned extra = a.T_new > 0 ? (unsigned)a.T_new : 0u;   // append workgroups at the end of x
  int max_v = 0;
  for (int i = 0; i < n_sess; ++i) max_v = view_tok.v[i] > max_v ? view_tok.v[i] : max_v;
  const int n_max = (max_v + 4 * g.tpw - 1) / (4 * g.tpw);
  if (n_max <= kCombGroups) {
    dim3 cgrid((unsigned)((g.rows + kNarrowRows - 1) / kNarrowRows) + extra, (unsigned)g.Hkv, (unsigned)n_sess);
    hipLaunchKernelGGL(k_attend_combine_narrow, cgrid, dim3(256), 0, st, part_o, part_ml, out, view_tok, s0, g, a);
  } else {
    dim3 cgrid((unsigned)(g.rows * kCombQuarters) + extra, (unsigned)g.Hkv, (unsigned)n_sess);
    hipLaunchKernelGGL(k_attend_combine, cgrid, dim3(256), 0, st, part_o, part_ml, out, view_tok, s0, g, a);
  }
  return hipGetLastError();
}

}  // namespace kvmem

namespace kvmem {

hipError_t launch_mass(int bf16, const void *q, const float *qw, float eps, const void *k_pool, const int32_t *table,
                       const int32_t *view_blocks, float4 *part, float *mass, float *lse, int32_t *dev_err,
                       const SessI32 &n_tok, int s0, int n_sess, const MassGeom &g, double theta, hipStream_t st) {
  int max_all = 0;
  for (int i = 0; i < n_sess; ++i) {
    const int n = (n_tok.v[i] + kBT - 1) / kBT;
    max_all = n > max_all ? n : max_all;
  }
  const int groups = (g.Hkv + kMassWaves - 1) / kMassWaves;
  if (max_all > 0 && !bf16) {
    const dim3 grid((unsigned)((max_all + g.chunk - 1) / g.chunk), (unsigned)g.Hkv, (unsigned)n_sess);
    hipLaunchKernelGGL(k_mass_f32, grid, dim3(256), 0, st, (const float *)q, qw, eps, (const float *)k_pool, table,
                       view_blocks, part, dev_err, n_tok, s0, g, theta);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (max_all > 0) {
    dim3 grid((unsigned)((max_all + g.chunk - 1) / g.chunk), (unsigned)groups, (unsigned)n_sess);
    if (g.rows <= 16)
      hipLaunchKernelGGL(k_mass_bf16<1>, grid, dim3(512), 0, st, (const uint16_t *)q, qw, eps,
                         (const uint16_t *)k_pool, table, view_blocks, part, dev_err, n_tok, s0, g, theta);
    else
      hipLaunchKernelGGL(k_mass_bf16<2>, grid, dim3(512), 0, st, (const uint16_t *)q, qw, eps,
                         (const uint16_t *)k_pool, table, view_blocks, part, dev_err, n_tok, s0, g, theta);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 cgrid((unsigned)g.rows, (unsigned)g.Hkv, (unsigned)n_sess);
  hipLaunchKernelGGL(k_mass_combine, cgrid, dim3(64), 0, st, part, mass, lse, n_tok, s0, g);
  return hipGetLastError();
}

int mass_chunk(int n_sessions, int Hkv, int max_blocks) {
  // aim for >= 256 workgroups; 8 .. 256 blocks per chunk
  const long groups = (Hkv + kMassWaves - 1) / kMassWaves;
  long c = ((long)max_blocks * groups * n_sessions + 255) / 256;
  if (c < 8) c = 8;
  if (c > kMassMaxChunk) c = kMassMaxChunk;
  return (int)c;
}

}  // namespace kvmem
