// Query operands shared by the attention kernels (view attention, paged
// attention, attention-mass diagnostic).
#pragma once

#include "kvmem_internal.h"

namespace kvmem {

namespace {

constexpr float kLog2eRsqrtD = 0.12751743074480953f;   // log2(e) / sqrt(128)
constexpr int kQprepMaxT = 32;                          // query tokens per step in the bf16 path

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// K tiles read as whole 128-byte lines.  The matrix-core A operand of a
// 16-token K tile (256-byte rows) puts 16-byte piece c (dims 32c + 8qq .. +
// 7) of row col in lane (qq, col); loaded that way, each instruction reads
// 64-byte halves of 16 rows.  Here the two instructions of half hf of the row
// (pieces 2hf, 2hf + 1) each read 8 whole rows: lanes col < 8 and col + 8
// (same qq) take the two pieces of one line.
//   r[2hf]     : piece 2hf of row col (col < 8), piece 2hf + 1 of row col - 8
//   r[2hf + 1] : piece 2hf + 1 of row col + 8 (col < 8), piece 2hf of row col
// rows: the tile's first row.
__device__ __forceinline__ void load_k_lines(uint4 (&r)[4], const uint16_t *rows, int qq, int col) {
  const bool lo = col < 8;
  const int ra = lo ? col : col - 8, rb = lo ? col + 8 : col;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    r[2 * hf] = load_nt16(rows + (size_t)ra * kD + 32 * (lo ? 2 * hf : 2 * hf + 1) + 8 * qq);
    r[2 * hf + 1] = load_nt16(rows + (size_t)rb * kD + 32 * (lo ? 2 * hf + 1 : 2 * hf) + 8 * qq);
  }
}

// The A operand of row col from load_k_lines' registers: the own piece 2hf
// stays, piece 2hf + 1 comes from lane col ^ 8 (DPP row_ror:8), which holds
// it for this lane.
__device__ __forceinline__ void k_lines_operand(const uint4 (&r)[4], uint4 (&a)[4], int col) {
  const bool lo = col < 8;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const uint4 own = lo ? r[2 * hf] : r[2 * hf + 1];
    const uint4 send = lo ? r[2 * hf + 1] : r[2 * hf];
    a[2 * hf] = own;
    a[2 * hf + 1] = make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.x, kDppRor8, 0xf, 0xf, false),
                               (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.y, kDppRor8, 0xf, 0xf, false),
                               (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.z, kDppRor8, 0xf, 0xf, false),
                               (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send.w, kDppRor8, 0xf, 0xf, false));
  }
}


// Query operands of the matrix-core products for the 16 rows of operand set nt:
// q~ (RMSNorm, weight), RoPE at V + t, scaled by log2(e)/sqrt(d), split into
// bf16 hi + lo, in the B-operand lane layout.  Lane (qq, col) holds row
// 16*nt + col; its chunk c holds dims 32c + 8qq .. +7, so the RoPE partner of
// a dim (+-64) sits in chunk c ^ 2 of the same lane.  x holds the row's raw
// values, cs_tab the (cos, sin) of every (query token, frequency).
__device__ __forceinline__ void build_q_operands(const float (&x)[4][8], bool valid, int t, int qq, const float *qw,
                                                 float eps, const float (*cs_tab)[kD / 2][2], bf16x8 (&qhi)[4],
                                                 bf16x8 (&qlo)[4]) {
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[c][j] * x[c][j];
  ss = sum_xor16(ss);
  ss = sum_xor32(ss);
  const float rs = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
  float y[4][8];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) y[c][j] = x[c][j] * rs * qw[32 * c + 8 * qq + j];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint32_t h2[2], l2[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ip = 32 * (c & 1) + 8 * qq + j + k;          // pair index (dim mod 64)
        const float cs = cs_tab[t][ip][0], sn = cs_tab[t][ip][1];
        const float xo = y[c][j + k], xp = y[c ^ 2][j + k];
        const float r = (c < 2 ? xo * cs - xp * sn : xo * cs + xp * sn) * kLog2eRsqrtD;
        split_hi_lo(valid ? r : 0.f, h2[k], l2[k]);
      }
      hw[j / 2] = h2[0] | (h2[1] << 16);
      lw[j / 2] = l2[0] | (l2[1] << 16);
    }
    qhi[c] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
    qlo[c] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
  }
}

}  // namespace

}  // namespace kvmem
