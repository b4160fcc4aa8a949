// Block scoring and GQA aggregation for short query steps (T * G rows per KV head).
//
// KVMem scores every indexed block with s_b = <q, k_bar_b>/sqrt(d) (reproduction
// README, 'Core equation') after RMS-normalising the query, then softmaxes each
// query head over the blocks and sums the heads of a KV group (README,
// '2026-09-08 validation correction': averaging GQA heads before the softmax was
// the withdrawn bug).
//
// k_score_gemv:  a GEMV on the vector ALUs, one index row per lane, for steps
//                of at most 8 query rows per KV head (details at the kernel).
// Each scoring wavefront writes one (max, sum of exp) slot per query row and
// key it met; the aggregation kernel merges them.
#include "kvmem_internal.h"

namespace kvmem {

namespace {

__device__ __forceinline__ float load_elem(const uint16_t *p) { return bf16_lo(*p); }
__device__ __forceinline__ float load_elem(const float *p) { return *p; }

// One lane's index row inside a tile, as 16-byte words (16 for bf16, 32 for
// fp32).  Word w of the 64 rows of a tile is contiguous, so load w of a
// wavefront is a single coalesced 1 KiB access.
template <typename T>
struct RowRaw {
  static constexpr int kWords = kD * (int)sizeof(T) / 16;
  uint4 w[kWords];
};

template <typename T>
__device__ __forceinline__ void load_row(RowRaw<T> &r, const T *tile, int lane) {
#pragma unroll
  for (int i = 0; i < RowRaw<T>::kWords; ++i) r.w[i] = load_nt16(tile + (i * kIdxTile + lane) * (16 / (int)sizeof(T)));
}

// 8 consecutive elements of the row, starting at element 8c, as fp32.
__device__ __forceinline__ void row8(const RowRaw<uint16_t> &r, int c, float (&v)[8]) {
  const uint32_t e[4] = {r.w[c].x, r.w[c].y, r.w[c].z, r.w[c].w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = bf16_lo(e[k]);
    v[2 * k + 1] = bf16_hi(e[k]);
  }
}
__device__ __forceinline__ void row8(const RowRaw<float> &r, int c, float (&v)[8]) {
  const uint4 a = r.w[2 * c], b = r.w[2 * c + 1];
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

// acc[r] += sum_j q_j(r) * kv[j] for the eight query values q_j(r) = lane
// 8H + j of each 16-lane row of q[r] (the query rows are replicated in the four
// rows of the wavefront, so every lane sees the same q_j(r)).  Each FMA takes
// q_j(r) through a DPP row broadcast (row_newbcast) of its first operand: the
// query stays in registers and costs no extra instruction.  The FMAs are
// ordered dimension-major, so consecutive ones update different rows and do
// not wait on each other.  A DPP read of q needs two wait states after a VALU
// write of it, which the compiler does not insert for inline asm, hence the
// leading s_nop.  (Generated: one block per row count and half.)
template <int R>
struct Fma8;
template <>
struct Fma8<4> {
  static __device__ __forceinline__ void fma8_lo(float (&acc)[4], const float (&q)[4], const float (&kv)[8]) {
    asm("s_nop 1\n\t"
          "v_fmac_f32_dpp %0, %4, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(kv[0]), "v"(kv[1]), "v"(kv[2]), "v"(kv[3]), "v"(kv[4]), "v"(kv[5]), "v"(kv[6]), "v"(kv[7]));
  }

  static __device__ __forceinline__ void fma8_hi(float (&acc)[4], const float (&q)[4], const float (&kv)[8]) {
    asm("s_nop 1\n\t"
          "v_fmac_f32_dpp %0, %4, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %4, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %5, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %6, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %7, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(kv[0]), "v"(kv[1]), "v"(kv[2]), "v"(kv[3]), "v"(kv[4]), "v"(kv[5]), "v"(kv[6]), "v"(kv[7]));
  }
};
template <>
struct Fma8<8> {
  static __device__ __forceinline__ void fma8_lo(float (&acc)[8], const float (&q)[8], const float (&kv)[8]) {
    asm("s_nop 1\n\t"
          "v_fmac_f32_dpp %0, %8, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %16 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %18 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %19 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %20 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %21 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %22 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %23 row_newbcast:7 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]), "v"(kv[0]), "v"(kv[1]), "v"(kv[2]), "v"(kv[3]), "v"(kv[4]), "v"(kv[5]), "v"(kv[6]), "v"(kv[7]));
  }

  static __device__ __forceinline__ void fma8_hi(float (&acc)[8], const float (&q)[8], const float (&kv)[8]) {
    asm("s_nop 1\n\t"
          "v_fmac_f32_dpp %0, %8, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %0, %8, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %1, %9, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %2, %10, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %3, %11, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %4, %12, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %5, %13, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %6, %14, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
          "v_fmac_f32_dpp %7, %15, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]), "+v"(acc[6]), "+v"(acc[7])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]), "v"(kv[0]), "v"(kv[1]), "v"(kv[2]), "v"(kv[3]), "v"(kv[4]), "v"(kv[5]), "v"(kv[6]), "v"(kv[7]));
  }
};

// Block-scoring GEMV, one index row per lane.  A wavefront owns a contiguous
// range of items; for each it streams the 64 rows of one index tile (lane b
// holds row b whole, 16 coalesced loads), and accumulates the R query rows of
// its group against it.  The query rows sit in registers, replicated per
// 16-lane row, and reach the FMAs through DPP broadcasts: no LDS, no scalar
// loads and no cross-lane reduction in the inner loop.
//
// Softmax statistics: each lane keeps a running max m and sum l of exp(s - m)
// per query row over the blocks it has scored in the current key; at the end
// of each key the wavefront reduces them once and writes one (max, sum) slot
// per row.  Scores are stored coalesced per row.
//
// bf16: the next item's rows are requested before the current item is
// computed (two register buffers).  fp32 rows are twice as large and are
// loaded one item at a time.
template <typename T, int R>
__global__ __launch_bounds__(64) void k_score_gemv(const T *__restrict__ index, const T *__restrict__ q,
                                                   const float *__restrict__ qw, float eps,
                                                   float *__restrict__ scores, float2 *__restrict__ part,
                                                   uint32_t *__restrict__ zero, int n_zero,
                                                   SessI32 n_blocks, int s0, ScoreGeom g, ScoreSplit sp) {
  constexpr bool kPrefetch = sizeof(T) == 2;
  const int lane = threadIdx.x;
  for (int i = blockIdx.x * 64 + lane; i < n_zero; i += gridDim.x * 64) zero[i] = 0u;
  const int n_rows = g.Tq * g.G;
  const int total = sp.n_sess * g.Hkv * sp.n_rg * sp.ntl;
  const int i0 = blockIdx.x * sp.per;                   // < total (grid = ceil(total / per))
  const int i1 = min(total, i0 + sp.per);

  int key, key_r0;
  float qv[R][kD / 16];                                 // q[r][16 m + lane % 16] (see fma8)
  size_t row_id[R];                                     // (s, t, query head) rows of the key
  float m[R], l[R];

  auto tile_of = [&](int item) {
    const ScoreItem it = decode_score_item(item, sp, g.Hkv, n_blocks);
    return index + ((size_t)((s0 + it.sl) * g.Hkv + it.h) * g.n_tiles + it.t) * (size_t)(kIdxTile * kD);
  };

  // one (max, sum) slot per row of the current key
  auto flush = [&]() {
    const int slot = blockIdx.x - score_slot0(key, sp);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (key_r0 + r >= n_rows) break;
      const float M = wave_max_dpp(m[r]);
      const float x = m[r] == -INFINITY ? 0.f : l[r] * __expf(m[r] - M);
      const float L = wave_sum_dpp(x);
      if (lane == 0) part[row_id[r] * g.slot_stride + slot] = make_float2(M, L);
    }
  };

  // Query registers and fresh statistics for a new key: lane l holds
  // q~[r][16 mm + l % 16] / sqrt(d) (l % 16 = the lane's place in its 16-lane
  // row, so every row of the wavefront carries the whole query row).  The mean
  // square of a query row is summed over the 16 lanes of a row with DPP.
  auto start_key = [&](const ScoreItem &c) {
    key = c.key;
    key_r0 = c.r0;
    const int s = s0 + c.sl;
    const int i = lane & 15;
    float w[kD / 16];
#pragma unroll
    for (int mm = 0; mm < kD / 16; ++mm) w[mm] = qw[16 * mm + i];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // rows past n_rows read row r0 (their results are not stored)
      const int row = c.r0 + r < n_rows ? c.r0 + r : c.r0;
      const int t = row / g.G, gg = row % g.G;
      row_id[r] = ((size_t)s * g.Tq + t) * g.Hq + (size_t)c.h * g.G + gg;
      const T *src = q + row_id[r] * kD + i;
      float ss = 0.f;
#pragma unroll
      for (int mm = 0; mm < kD / 16; ++mm) {
        qv[r][mm] = load_elem(src + 16 * mm);
        ss += qv[r][mm] * qv[r][mm];
      }
      ss += dpp_f32<kDppXor1>(ss);
      ss += dpp_f32<kDppXor2>(ss);
      ss += dpp_f32<kDppMirror8>(ss);
      ss += dpp_f32<kDppMirror16>(ss);
      const float rs = (1.0f / sqrtf(ss * (1.0f / kD) + eps)) * 0.08838834764831845f;   // 1/sqrt(128)
#pragma unroll
      for (int mm = 0; mm < kD / 16; ++mm) qv[r][mm] *= rs * w[mm];
      m[r] = -INFINITY;
      l[r] = 0.f;
    }
  };

  auto compute = [&](const RowRaw<T> &raw, int item) {
    const ScoreItem c = decode_score_item(item, sp, g.Hkv, n_blocks);
    if (c.t * kIdxTile >= c.nb) return;                 // tile past this session's history

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int cc = 0; cc < kD / 8; cc += 2) {
      float q[R], kv[8];
#pragma unroll
      for (int r = 0; r < R; ++r) q[r] = qv[r][cc / 2];
      row8(raw, cc, kv);
      Fma8<R>::fma8_lo(acc, q, kv);
      row8(raw, cc + 1, kv);
      Fma8<R>::fma8_hi(acc, q, kv);
    }

    const int b = c.t * kIdxTile + lane;
    if (b < c.nb) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (c.r0 + r >= n_rows) break;
        scores[row_id[r] * g.max_blocks + b] = acc[r];
        // running softmax statistics: one exp per score
        const float d = acc[r] - m[r];
        const float e = __expf(-fabsf(d));
        l[r] = d > 0.f ? fmaf(l[r], e, 1.f) : l[r] + e;
        m[r] = fmaxf(m[r], acc[r]);
      }
    }
  };

  // One segment per key in the range: the key's query loads go out before its
  // first tile load (vector loads complete in order), then the tiles stream.
  // bf16 keeps one tile of look-ahead.  After the last item the look-ahead
  // reads the index's first tile instead, which every wavefront shares and the
  // caches keep: the loads stay unconditional (a branch around them makes the
  // compiler wait for both buffers) without costing HBM traffic.
  for (int it = i0; it < i1;) {
    const ScoreItem c0 = decode_score_item(it, sp, g.Hkv, n_blocks);
    const int end = min(i1, (c0.key + 1) * sp.ntl);
    start_key(c0);
    if constexpr (kPrefetch) {
      RowRaw<T> ra, rb;
      load_row(ra, tile_of(it), lane);
      while (true) {
        load_row(rb, it + 1 < end ? tile_of(it + 1) : index, lane);
        compute(ra, it);
        if (++it >= end) break;
        load_row(ra, it + 1 < end ? tile_of(it + 1) : index, lane);
        compute(rb, it);
        if (++it >= end) break;
      }
    } else {
      RowRaw<T> ra;
      for (; it < end; ++it) {
        load_row(ra, tile_of(it), lane);
        compute(ra, it);
      }
    }
    flush();
  }
}

// Wavefronts per SIMD that the scorer's grid aims for: each wavefront then
// gets several items, so its next tile streams in while it computes.
constexpr int kScoreWavesPerSimd = 2;

template <typename T, int R>
hipError_t launch_gemv_r(const void *index, const void *q, const float *qw, float eps, float *scores, float2 *part,
                         uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess, const ScoreGeom &g, int max_nb,
                         ScoreSplit *split, hipStream_t st) {
  static int cus = 0;                                   // compute units (device property)
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  ScoreSplit sp;
  sp.n_sess = n_sess;
  sp.rpg = R;
  sp.n_rg = (g.Tq * g.G + R - 1) / R;
  sp.ntl = idx_tiles(max_nb);
  const long total = (long)n_sess * g.Hkv * sp.n_rg * sp.ntl;
  const long target = (long)cus * 4 * kScoreWavesPerSimd;
  sp.per = (int)((total + target - 1) / target);
  const int grid = (int)((total + sp.per - 1) / sp.per);
  *split = sp;
  hipLaunchKernelGGL((k_score_gemv<T, R>), dim3(grid), dim3(64), 0, st, (const T *)index, (const T *)q, qw, eps,
                     scores, part, zero, n_zero, n_blocks, s0, g, sp);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemv_t(const void *index, const void *q, const float *qw, float eps, float *scores, float2 *part,
                         uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess, const ScoreGeom &g, ScoreSplit *split,
                         hipStream_t st) {
  int max_nb = 0;
  for (int i = 0; i < n_sess; ++i) max_nb = n_blocks.v[i] > max_nb ? n_blocks.v[i] : max_nb;
  split->n_sess = n_sess;
  split->ntl = 0;
  if (max_nb == 0) return hipSuccess;
  const int n_rows = g.Tq * g.G;
  if (n_rows <= 4)
    return launch_gemv_r<T, 4>(index, q, qw, eps, scores, part, zero, n_zero, n_blocks, s0, n_sess, g, max_nb, split, st);
  // more rows: groups of 8 rows, each re-reading the index rows
  return launch_gemv_r<T, 8>(index, q, qw, eps, scores, part, zero, n_zero, n_blocks, s0, n_sess, g, max_nb, split, st);
}

}  // namespace

hipError_t launch_score_gemv(int bf16, const void *index, const void *q, const float *qw, float eps, float *scores,
                             float2 *part, uint32_t *zero, int n_zero, const SessI32 &n_blocks, int s0, int n_sess,
                             const ScoreGeom &g, ScoreSplit *split, hipStream_t st) {
  return bf16 ? launch_gemv_t<uint16_t>(index, q, qw, eps, scores, part, zero, n_zero, n_blocks, s0, n_sess, g, split, st)
              : launch_gemv_t<float>(index, q, qw, eps, scores, part, zero, n_zero, n_blocks, s0, n_sess, g, split, st);
}

}  // namespace kvmem
