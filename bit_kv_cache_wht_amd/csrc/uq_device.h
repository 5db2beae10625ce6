// Device-side building blocks for libuq (gfx950, wave64).
//
// [review] = "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
//            (manon006.tistory.com/395)
//
// Rounding decisions of the write path are taken in float64 on the exact rotated
// value: the Walsh-Hadamard butterfly of bf16/f32 inputs is exact in float64 for
// any row whose nonzero exponents span at most 38 (bf16) / 22 (f32) binades, so
// its result does not depend on the order of the additions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/uq.h"
#include "uq_internal.h"

namespace uq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;    // tokens per page
constexpr int kGroup = 32;   // channels per scale group ([review] §3.1)

// sqrt(1/d) as the nearest double (0x1.6a09e667f3bcdp-4 is sqrt(2)/16 rounded once).
template <int D> __device__ __forceinline__ double wht_c() { return D == 64 ? 0.125 : 0x1.6a09e667f3bcdp-4; }
template <int D> __device__ __forceinline__ float wht_cf() { return D == 64 ? 0.125f : 0x1.6a09e6p-4f; }

// Sign bit (1u << 31, or 0) of channel ch in the rotation's sign diagonal.
__device__ __forceinline__ uint32_t sign_mask(const Rot& r, int ch) {
  const int w = ch >> 5;
  const uint32_t word = w == 0 ? r.s[0] : w == 1 ? r.s[1] : w == 2 ? r.s[2] : r.s[3];
  return ((word >> (ch & 31)) & 1u) << 31;
}
__device__ __forceinline__ bool has_signs(const Rot& r) { return (r.s[0] | r.s[1] | r.s[2] | r.s[3]) != 0u; }
// x with its sign bit XORed by m (an exact negation when m is set).
__device__ __forceinline__ double flip_sign(double x, uint32_t m) {
  return __hiloint2double(__double2hiint(x) ^ (int)m, __double2loint(x));
}
__device__ __forceinline__ float flip_sign(float x, uint32_t m) { return __uint_as_float(__float_as_uint(x) ^ m); }

// Position of KV head h's block inside FP4 page `page` of a cache with H KV
// heads: (h + 2 page) mod H, so that for an even H a pair's two blocks stay
// adjacent and pair p sits at pair position (p + page) mod (H / 2).  `mask` is
// H - 1 when H is a power of two, else -1.  Page ids are non-negative.
__device__ __forceinline__ int fp4_block_pos(int h, int page, int H, int mask) {
  if (mask >= 0) return (int)(((uint32_t)h + 2u * (uint32_t)page) & (uint32_t)mask);
  return (h + 2 * (page % H)) % H;
}

// FP8 pages rotate their bytes with the page id: byte b of the page laid out as
// blocks back to back is stored at (b + 256 (page mod units)) mod page_bytes,
// units = page_bytes / 256 (umask = units - 1 when units is a power of two,
// else -1).  Every 16-byte load or store stays inside one 256-byte unit.
__device__ __forceinline__ uint32_t fp8_rot(int page, int units, int umask) {
  return (uint32_t)(umask >= 0 ? (page & umask) : page % units) << 8;
}
__device__ __forceinline__ uint32_t fp8_wrap(uint32_t b, uint32_t rot, uint32_t page_bytes) {
  const uint32_t x = b + rot;                      // both below page_bytes
  return x >= page_bytes ? x - page_bytes : x;
}

template <int D> struct Fp4Block {
  static constexpr int kCodeBytes = kPage * D / 2;          // codes of 16 slots
  static constexpr int kBytes = kCodeBytes + kPage * D / 32; // + one scale byte per group
};

__device__ __forceinline__ double bf16_bits_to_f64(uint32_t b16) {
  return (double)__uint_as_float(b16 << 16);
}

// Value of `v` held by lane ^ XOR (XOR = 1 or 2, inside a quad) via DPP quad_perm.
template <int XOR> __device__ __forceinline__ double quad_swap(double v) {
  constexpr int ctrl = XOR == 1 ? 0xB1 /* [1,0,3,2] */ : 0x4E /* [2,3,0,1] */;
  // a quad permutation reads a lane of every quad, so no lane needs an old value
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), ctrl, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), ctrl, 0xF, 0xF, true);
  return __hiloint2double(hi, lo);
}

// Value of `v` held by lane ^ M (M = 1, 2, 4 or 8, inside the lane's 16-lane
// row) via DPP; p = the lane index modulo 16.  M = 4 takes lane + 4 (row_shl:4)
// where bit 2 of p is clear and lane - 4 (row_shr:4) where it is set; M = 8 is
// row_ror:8.
template <int M> __device__ __forceinline__ double lane_xor16(double v, int p) {
  if constexpr (M == 1 || M == 2) {
    return quad_swap<M>(v);
  } else {
    constexpr int c0 = M == 4 ? 0x104 : 0x128;
    const int lo0 = __builtin_amdgcn_mov_dpp(__double2loint(v), c0, 0xF, 0xF, true);
    const int hi0 = __builtin_amdgcn_mov_dpp(__double2hiint(v), c0, 0xF, 0xF, true);
    if constexpr (M == 8) {
      return __hiloint2double(hi0, lo0);
    } else {
      const int lo1 = __builtin_amdgcn_mov_dpp(__double2loint(v), 0x114, 0xF, 0xF, true);
      const int hi1 = __builtin_amdgcn_mov_dpp(__double2hiint(v), 0x114, 0xF, 0xF, true);
      return (p & 4) ? __hiloint2double(hi1, lo1) : __hiloint2double(hi0, lo0);
    }
  }
}

// Sylvester butterfly over the 32 values a lane holds (stages h = 1..16).
__device__ __forceinline__ void wht32_inlane(double (&x)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; i += 2 * h)
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const double a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
}

// One butterfly stage whose partner element sits in lane ^ XOR: the lane with the
// XOR bit clear keeps a + b, the other b' = a - b, each a single rounded add
// (fma with an exact +-1 product).
template <int XOR> __device__ __forceinline__ void wht_cross_stage(double (&x)[32], int lane) {
  const double sgn = (lane & XOR) ? -1.0 : 1.0;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const double other = quad_swap<XOR>(x[e]);
    x[e] = __builtin_fma(x[e], sgn, other);
  }
}

// Normalized WHT of a row of D = 32 * LPR channels spread over LPR = D/32
// consecutive lanes, lane part p holding channels 32p..32p+31.  On return the
// lane holds output channels 32p..32p+31, i.e. one quantization group.
template <int D> __device__ __forceinline__ void wht_row(double (&x)[32], int lane) {
  wht32_inlane(x);
  wht_cross_stage<1>(x, lane);                 // h = 32
  if constexpr (D == 128) wht_cross_stage<2>(x, lane);   // h = 64
  const double c = wht_c<D>();
#pragma unroll
  for (int e = 0; e < 32; ++e) x[e] = __builtin_fma(x[e], c, 0.0);   // + 0: an exact zero is +0
}

// Least integer E with m <= 6 * 2^E, clamped to [-127, 127] (m == 0 -> -127).
// With m = f * 2^ex, f in [0.5, 1): 6 * 2^(ex-3) = 0.75 * 2^ex, so E = ex - 3
// when f <= 0.75 and ex - 2 otherwise.
__device__ __forceinline__ int scale_exponent(double m) {
  if (!(m > 0.0)) return -127;
  int ex;
  const double f = frexp(m, &ex);
  int e = ex - 3 + (f > 0.75 ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// constOpt scale exponent ([review] §3.3 "constant-optimized scaling", c = 0.156;
// §6.2): the integer nearest to log2(s), s = c m rounded once to float64,
// clamped to [-127, 127] (m = 0 gives -127).  With s = M 2^e, M in [1, 2), the
// exponent rounds up when M > sqrt(2); no double equals sqrt(2), and the least
// double above it has significand bits 0x6A09E667F3BCD, so the test is a
// comparison of the significand bits.
__device__ __forceinline__ int constopt_exponent(double m) {
  const double s = 0.156 * m;
  if (!(s >= 0x1p-128)) return -127;                 // zero, or below the clamp
  const uint64_t b = (uint64_t)__double_as_longlong(s);
  const int e = (int)(b >> 52) - 1023;               // s is normal and positive here
  const int E = e + ((b & 0xFFFFFFFFFFFFFull) >= 0x6A09E667F3BCDull ? 1 : 0);
  return E > 127 ? 127 : (E < -127 ? -127 : E);      // s in [2^-128, 2^-127.5) gives -128
}

// FP4 E2M1 code of r = x / 2^E: magnitude rounded to nearest of
// {0,.5,1,1.5,2,3,4,6}, ties to the even code, |r| > 6 saturating; sign bit from r.
// The grid has quantum 0.5 on [0,2), 1 on [2,4), 2 on [4,6]: scale into integer
// steps, round half to even, and offset into the code range.
__device__ __forceinline__ uint32_t e2m1_code(double r) {
  const double a = fmin(fabs(r), 6.0);
  double s;
  int off;
  if (a < 2.0) { s = 2.0; off = 0; }
  else if (a < 4.0) { s = 1.0; off = 2; }
  else { s = 0.5; off = 4; }
  const int n = (int)__builtin_rint(a * s);
  const uint32_t sign = ((uint32_t)__double2hiint(r)) >> 31;
  return (uint32_t)(n + off) | (sign << 3);
}

// r rounded to float32 by round-to-odd (truncate, then set the last bit if any
// dropped bit was set).  Rounding that result to a format with at least two
// fewer significant bits (here E2M1 x 2^E, 2 bits, whose decision points are all
// even floats) gives the same result as rounding r itself, so the float32
// hardware converter can take the decision that is defined on the float64
// value.  Valid for |r| < 2^128; below 2^-120 it returns a float of r's sign and
// magnitude below 2^-119 (callers only need that such values round to zero).
// Integer form: the magnitude, floored at 2^-120 so that its float64 exponent
// lies in [903, 1150], has the float32 exponent 896 below it; its low nine
// exponent bits and the top 23 mantissa bits, shifted right by 29, minus 384 in
// the exponent field, are the truncated float32 magnitude.
__device__ __forceinline__ float f32_round_to_odd(double r) {
  const double a = fmax(fabs(r), 0x1p-120);
  const uint32_t ahi = (uint32_t)__double2hiint(a), alo = (uint32_t)__double2loint(a);
  const uint32_t mag = __builtin_amdgcn_alignbit(ahi, alo, 29) - (384u << 23);
  const uint32_t sticky = min(alo << 3, 1u);   // 1 if any dropped low bit is set
  return __uint_as_float(((uint32_t)__double2hiint(r) & 0x80000000u) | mag | sticky);
}

// OCP E4M3 bytes (nearest, ties to even, |v| > 448 -> 448, sign copied, also
// for zero; subnormal quantum 2^-9) of four values, byte i from the i-th.  The
// hardware converter v_cvt_pk_fp8_f32 (probed on gfx950 over every E4M3 value,
// the midpoints and one ulp either side, subnormals and signed zeros: nearest
// even, OCP encoding) takes float32 inputs within +-448.
__device__ __forceinline__ uint32_t e4m3x4_f32(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
  b = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
  c = __builtin_amdgcn_fmed3f(c, -448.f, 448.f);
  d = __builtin_amdgcn_fmed3f(d, -448.f, 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
// The same for float64 values: clamped to +-448 in float64, then rounded to
// float32 by round to odd, which keeps the nearest-even decision onto the
// 4-bit significand (and the sign of zero).
__device__ __forceinline__ uint32_t e4m3x4_f64(double a, double b, double c, double d) {
  auto f = [](double v) { return f32_round_to_odd(fmin(fmax(v, -448.0), 448.0)); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f(a), f(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f(c), f(d), lo, true);
}

// bf16 bits of a float, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Loads of cache pages, which a decode launch reads once: nontemporal, so the
// lines stream through the caches instead of being kept in them (on MI355X a
// plain streaming read runs at ~6.3 TB/s this way against ~7.0 TB/s).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load4_stream(const void* p) {
  return __builtin_nontemporal_load(static_cast<const uint32_t*>(p));
}

// 32 consecutive input values (bf16 bits or f32) starting at element `elem`, as float64.
template <int IN> __device__ __forceinline__ void load_row32(const void* base, int64_t elem, double (&x)[32]) {
  if constexpr (IN == UQ_IN_BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint4 u = p[w];
      const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * w + 2 * i] = bf16_bits_to_f64(d[i] & 0xFFFFu);
        x[8 * w + 2 * i + 1] = bf16_bits_to_f64(d[i] >> 16);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float4 f = p[w];
      x[4 * w] = f.x; x[4 * w + 1] = f.y; x[4 * w + 2] = f.z; x[4 * w + 3] = f.w;
    }
  }
}


}  // namespace uq
