// Device-side helpers shared by the KVMem kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvmem {

constexpr int kD = 128;        // head dim
constexpr int kBT = 32;        // tokens per block
constexpr int kMaxSess = 64;   // sessions handled by one launch

// Per-session scalars passed by value in the kernel arguments (the lengths
// live on the host, so no device copy or synchronisation is needed).
struct SessI32 {
  int32_t v[kMaxSess];
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: data read once).  Streams that
// are read once run markedly faster with this hint on MI355X (measured ~6.4
// vs ~4.4 TB/s for the same access pattern).
__device__ __forceinline__ uint4 load_nt16(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16-byte streaming store (non-temporal hint: written once, read much later).
__device__ __forceinline__ void store_nt16(void *p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ float4 load_nt16f(const void *p) {
  const uint4 v = load_nt16(p);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32 / fp64
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, nearest with ties to even (gfx950's conversion
// instruction; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// y = hi + lo with hi = bf16(y) and lo = bf16(y - hi): a product with a bf16
// operand accumulated over both parts carries ~16 significant bits of y.
__device__ __forceinline__ void split_hi_lo(float y, uint32_t &hi, uint32_t &lo) {
  hi = f32_to_bf16(y);
  lo = f32_to_bf16(y - __uint_as_float(hi << 16));
}

// Two fp32 -> packed bf16 (lo in bits 0..15), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// fp64 -> bf16 bits with a single rounding (nearest, ties to even).  The
// significand is rounded directly on the fp64 bit pattern to the 8 bits bf16
// keeps, so no intermediate fp32 rounding can double-round.  Magnitudes below
// the bf16 normal range use the fixed 2^-133 quantum of its subnormals.  Both
// forms are evaluated and one is selected, so callers stay free of branches.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  const double ys = rint(x * 0x1p133) * 0x1p-133;               // exact multiple of 2^-133
  const uint32_t small = x != x ? 0x7fc0u : __float_as_uint((float)ys) >> 16;
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t half = 1ull << 44;
  const uint64_t rem = b & ((1ull << 45) - 1);
  const uint64_t keep = b >> 45;
  const uint64_t up = (rem > half || (rem == half && (keep & 1))) ? 1 : 0;   // carry may bump the exponent
  const double r = __longlong_as_double((long long)((keep + up) << 45));
  const uint32_t normal = __float_as_uint((float)r) >> 16;               // exact, or +-inf
  return fabs(x) >= 0x1p-126 ? normal : small;
}

// ---------------------------------------------------------------------------
// Eight consecutive elements of a row (16-byte aligned in global memory):
// load as fp32, load / copy raw, store fp32 rounded to the element type.
// ---------------------------------------------------------------------------
template <typename T>
struct Row8;

template <>
struct Row8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[8]) {
    const uint4 w = load_nt16(p);
    const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_lo(e[k]);
      v[2 * k + 1] = bf16_hi(e[k]);
    }
  }
  static __device__ __forceinline__ void load_raw(const uint16_t *p, uint16_t (&v)[8]) {
    const uint4 w = load_nt16(p);
    const uint32_t e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = (uint16_t)(e[k] & 0xffffu);
      v[2 * k + 1] = (uint16_t)(e[k] >> 16);
    }
  }
  // 16 raw elements from LDS (2-byte aligned) to global memory (32-byte aligned)
  static __device__ __forceinline__ void copy16(uint16_t *dst, const uint16_t *src) {
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = (uint32_t)src[2 * k] | ((uint32_t)src[2 * k + 1] << 16);
    reinterpret_cast<uint4 *>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4 *>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
  static __device__ __forceinline__ void store(uint16_t *p, const float (&v)[8]) {
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4 *>(p) = w;
  }
};

template <>
struct Row8<float> {
  static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
    const float4 a = load_nt16f(p);
    const float4 b = load_nt16f(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void load_raw(const float *p, float (&v)[8]) { load(p, v); }
  static __device__ __forceinline__ void copy16(float *dst, const float *src) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      reinterpret_cast<float4 *>(dst)[k] = make_float4(src[4 * k], src[4 * k + 1], src[4 * k + 2], src[4 * k + 3]);
  }
  static __device__ __forceinline__ void store(float *p, const float (&v)[8]) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// ---------------------------------------------------------------------------
// RoPE angle: phi = pos * theta^(-2i/d) formed in fp64, reduced modulo 2*pi
// in fp64 with a two-term 2*pi (Cody-Waite), then sin/cos in fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double rope_inv_freq(int i, double theta) {
  return pow(theta, -(double)(2 * i) / (double)kD);
}

__device__ __forceinline__ void rope_cos_sin(double pos, double inv_freq, float &c, float &s) {
  const double kTwoPiHi = 6.283185307179586232;      // fp64 nearest to 2*pi
  const double kTwoPiLo = 2.4492935982947064e-16;    // 2*pi - kTwoPiHi
  const double kInvTwoPi = 0.15915494309189535;
  const double phi = pos * inv_freq;
  const double n = rint(phi * kInvTwoPi);
  double r = fma(-n, kTwoPiHi, phi);
  r = fma(-n, kTwoPiLo, r);
  sincosf((float)r, &s, &c);
}

// fp64 sin and cos of pos * inv_freq, reduced modulo 2*pi as above.
__device__ __forceinline__ void rope_angle_f64(double pos, double inv_freq, double &c, double &s) {
  const double kTwoPiHi = 6.283185307179586232;
  const double kTwoPiLo = 2.4492935982947064e-16;
  const double kInvTwoPi = 0.15915494309189535;
  const double phi = pos * inv_freq;
  const double n = rint(phi * kInvTwoPi);
  double r = fma(-n, kTwoPiHi, phi);
  r = fma(-n, kTwoPiLo, r);
  sincos(r, &s, &c);
}

// RoPE (cos, sin) of a key at view position p = 32 m + u.  The angle is split
// into a block part 32 m * theta_i and an in-block part u * theta_i, each
// formed and reduced in fp64 and evaluated with fp64 sin / cos; the in-block
// pair is rounded to fp32 (kernels that reuse it across blocks keep a table of
// the 32 x 64 pairs), and the two are combined with the angle-addition
// identities in fp64 and rounded to fp32 once.  Every kernel that writes or
// reads view keys forms their angles with these two functions, so gathered,
// appended and paged keys agree bit for bit.
__device__ __forceinline__ void rope_offset_pair(int u, double inv_freq, float &cb, float &sb) {
  double c, s;
  rope_angle_f64((double)u, inv_freq, c, s);
  cb = (float)c;
  sb = (float)s;
}
__device__ __forceinline__ void rope_compose(double ca, double sa, float cb, float sb, float &c, float &s) {
  c = (float)fma(ca, (double)cb, -(sa * (double)sb));
  s = (float)fma(sa, (double)cb, ca * (double)sb);
}

// The rotated pair (x1, x2) -> (x1 c - x2 s, x2 c + x1 s) with its fused
// operations written out, so that every kernel rounds it the same way.
__device__ __forceinline__ void rope_rotate(float x1, float x2, float c, float s, float &y1, float &y2) {
  y1 = fmaf(x1, c, -(x2 * s));
  y2 = fmaf(x2, c, x1 * s);
}

// Slot of token u inside a dimension-major 32-token V view block.
__host__ __device__ __forceinline__ int v_slot(int u) {
  return 8 * ((u & 15) >> 2) + 4 * (u >> 4) + (u & 3);
}

// s_waitcnt immediate for gfx9-family: vmcnt(0), expcnt/lgkmcnt left at max.
constexpr int kWaitVmcnt0 = 0x0F70;

// ---------------------------------------------------------------------------
// cross-lane
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppMirror8 = 0x141;    // row_half_mirror: lane i <-> 7 - i within 8
constexpr int kDppMirror16 = 0x140;   // row_mirror: lane i <-> 15 - i within 16
constexpr int kDppBcast15 = 0x142;    // row_bcast:15: lane 15 of each row -> the next row
constexpr int kDppBcast31 = 0x143;    // row_bcast:31: lane 31 -> rows 2 and 3
constexpr int kDppRor8 = 0x128;       // row_ror:8: lane i <-> lane i ^ 8 within 16

// DPP move that writes only the rows in ROW_MASK; other lanes get `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32_rows(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xf, false));
}

// One butterfly step across 16-lane rows (partner lane l ^ 16) or wavefront
// halves (l ^ 32) with the VALU lane permutes of gfx950: passing v as both
// operands, the two results hold v[l] and v[l ^ m] in every lane (which is
// which depends on the lane), so a commutative op of the two is the step.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Whole-wavefront sum / max on the DPP network (no LDS round trips): reduce
// each 16-lane row (quad swaps, then the half-row and row mirrors), fold row 0
// into row 1 and row 2 into row 3 (row_bcast:15), then rows 0-1 into rows 2-3
// (row_bcast:31).  Lane 63 ends with the total, returned to every lane.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppMirror8>(v);
  v += dpp_f32<kDppMirror16>(v);
  v += dpp_f32_rows<kDppBcast15, 0xa>(0.f, v);
  v += dpp_f32_rows<kDppBcast31, 0xc>(0.f, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppMirror8>(v));
  v = fmaxf(v, dpp_f32<kDppMirror16>(v));
  v = fmaxf(v, dpp_f32_rows<kDppBcast15, 0xa>(-INFINITY, v));
  v = fmaxf(v, dpp_f32_rows<kDppBcast31, 0xc>(-INFINITY, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ void dev_flag(int32_t *err, int bits) {
  if (err) atomicOr(err, bits);
}

}  // namespace kvmem
