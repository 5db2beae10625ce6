// FP4 write of one (token, KV head) row of K or of V ([review] §3.1;
// [commentary] footnote 2), spread over LPR consecutive lanes of a wave: lane
// part p holds channels E*p .. E*p + E - 1 (E = D / LPR).  The append kernel and
// the fused decode step both write through this code, so a token gets the same
// bytes whichever entry point stores it.
//
// [review] = "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
//            (manon006.tistory.com/395)
// [commentary] = pheeree.github.io "kv-cache-4bit-serving-residency-collapse"
//
// Butterfly stages h < E run inside the lane, stages h >= E between lanes p and
// p ^ (h / E); every sum is exact in float64, so the result does not depend on
// the split.  After the butterfly each lane owns the same channels of the rotated
// row, so group absmax, scale, rounding and packing need at most a max across the
// LPG = 32 / E lanes of a group.
#pragma once
#include "uq_device.h"

namespace uq {

// Butterfly stage between lane parts p and p ^ M (the row's lanes are aligned
// to their count, so p ^ M is lane ^ M).
template <int E, int M> __device__ __forceinline__ void cross_stage(double (&x)[E], int p) {
  const double sgn = (p & M) ? -1.0 : 1.0;
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = __builtin_fma(x[e], sgn, lane_xor16<M>(x[e], p));
}

template <int D, int IN, int LPR> struct Fp4Row {
  static constexpr int E = D / LPR;                       // channels per lane
  static constexpr int LPG = E < 32 ? 32 / E : 1;         // lanes per quantization group
  static constexpr int GPL = E > 32 ? E / 32 : 1;         // quantization groups per lane
  static constexpr int BLK = Fp4Block<D>::kBytes;
  static constexpr int CODE = Fp4Block<D>::kCodeBytes;
  static constexpr int CPL = D / 32;                      // V: channel pairs per PV lane row group
  static constexpr int NU = E * (IN == UQ_IN_BF16 ? 2 : 4) / 16;
  uint4 raw[NU];                                          // the lane's input bits
  uint32_t w[E / 8];                                      // packed codes, channel E*p + i in nibble i
  int ex[GPL];                                            // scale exponents of the lane's groups

  // Input channels E*p .. of row `row` of a [rows][D] array (bf16 bits or f32).
  __device__ __forceinline__ void load(const void* src, int64_t row, int p) {
    const uint8_t* b = static_cast<const uint8_t*>(src) + (row * D + E * p) * (IN == UQ_IN_BF16 ? 2 : 4);
#pragma unroll
    for (int i = 0; i < NU; ++i) raw[i] = load16(b + 16 * i);
  }

  // Normalized WHT, group absmax, UE8M0 exponent (the absmax rule, or constOpt
  // when `constopt`) and E2M1 codes (all lanes of the row call it together).
  // RV: the cache's rotation variant applies -- R = c_d H diag(s) with its
  // signs, and a V row of a K-only cache is quantized as it is; without RV the
  // rotation is the plain c_d H.
  template <bool RV = false>
  __device__ __forceinline__ void quantize(int p, bool constopt, const Rot& rot, bool is_v) {
    const bool rotate = !RV || !(is_v && rot.k_only != 0u);   // the same for all lanes of the row
    double x[E];
    to_f64(x);
    if (rotate) {
      if (RV && has_signs(rot)) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = flip_sign(x[e], sign_mask(rot, E * p + e));
      }
      butterfly<1, E>(x);
      // the partner lanes of a cross stage belong to the same row
      if constexpr (LPR > 1) cross_stage<E, 1>(x, p);
      if constexpr (LPR > 2) cross_stage<E, 2>(x, p);
      if constexpr (LPR > 4) cross_stage<E, 4>(x, p);
      if constexpr (LPR > 8) cross_stage<E, 8>(x, p);
    }

    codes(x, rotate ? wht_c<D>() : 1.0, constopt);
  }

  // The lane's inputs as float64, in raw order (exact).
  __device__ __forceinline__ void to_f64(double (&x)[E]) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const uint32_t d[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (IN == UQ_IN_BF16) {
          x[8 * i + 2 * j] = bf16_bits_to_f64(d[j] & 0xFFFFu);
          x[8 * i + 2 * j + 1] = bf16_bits_to_f64(d[j] >> 16);
        } else {
          x[4 * i + j] = (double)__uint_as_float(d[j]);
        }
      }
    }
  }

  // Sylvester butterfly stages h = H0, 2 H0, .. < H1 over the local index.
  template <int H0, int H1> __device__ __forceinline__ static void butterfly(double (&x)[E]) {
#pragma unroll
    for (int hh = H0; hh < H1; hh <<= 1)
#pragma unroll
      for (int i = 0; i < E; i += 2 * hh)
#pragma unroll
        for (int j = i; j < i + hh; ++j) {
          const double a0 = x[j], a1 = x[j + hh];
          x[j] = a0 + a1;
          x[j + hh] = a0 - a1;
        }
  }

  // Group absmax, UE8M0 exponent and E2M1 codes of the lane's rotated channels
  // x (not yet multiplied by c).
  __device__ __forceinline__ void codes(double (&x)[E], double c, bool constopt) {
    // The normalized channel is RN(c_d x + 0) (one float64 rounding; the + 0
    // makes an exact zero +0 whatever the butterfly's signed zeros; unrotated,
    // c = 1 and x + 0 is x with a zero of either sign made +0).  Rounding is
    // monotone, so the group absmax of those is RN(c max |x|).
    constexpr int EG = E / GPL;                           // channels of one group held by the lane
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      double m = 0.0;                                     // the same in every lane of the group
#pragma unroll
      for (int e = 0; e < EG; ++e) m = fmax(m, fabs(x[EG * g + e]));
      if constexpr (LPG > 1) m = fmax(m, quad_swap<1>(m));
      if constexpr (LPG > 2) m = fmax(m, quad_swap<2>(m));
      const int xg = constopt ? constopt_exponent(m * c) : scale_exponent(m * c);
      ex[g] = xg;
      if (xg >= -100 && xg <= 100) {
        // hardware E2M1 rounding (nearest even, saturating at 6, sign kept) of a
        // float32 image, divided by the scale 2^xg.  The image is the float32
        // nearest the value: rounding that again to E2M1 decides as the value
        // itself would unless the image is exactly an E2M1 decision point
        // ((2k + 1) 2^(xg-2) for k < 3, 2.5, 3.5 or 5 times 2^xg), and every
        // decision point has its 21 low significand bits clear.  When some
        // lane of the wave holds an image with those bits clear (exact zeros
        // included), the wave takes the round-to-odd image instead, which
        // keeps every decision.
        const float sc = __uint_as_float((uint32_t)(xg + 127) << 23);
        float f[EG];
        uint32_t low = ~0u;
#pragma unroll
        for (int i = 0; i < EG; ++i) {
          f[i] = (float)__builtin_fma(x[EG * g + i], c, 0.0);
          low = min(low, __float_as_uint(f[i]) << 11);
        }
        if (__builtin_expect(__any(low == 0u), 0)) {
#pragma unroll
          for (int i = 0; i < EG; ++i) f[i] = f32_round_to_odd(__builtin_fma(x[EG * g + i], c, 0.0));
        }
#pragma unroll
        for (int q = EG / 8 * g; q < EG / 8 * (g + 1); ++q) {
          const int i0 = 8 * q - EG * g;
          uint32_t acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[i0], f[i0 + 1], sc, 0);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, f[i0 + 2], f[i0 + 3], sc, 1);
          acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, f[i0 + 4], f[i0 + 5], sc, 2);
          w[q] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, f[i0 + 6], f[i0 + 7], sc, 3);
        }
      } else {                                            // scales beyond the float32 range: float64 rounding
#pragma unroll
        for (int q = EG / 8 * g; q < EG / 8 * (g + 1); ++q) {
          uint32_t acc = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc |= e2m1_code(ldexp(__builtin_fma(x[8 * q + i], c, 0.0), -xg)) << (4 * i);
          w[q] = acc;
        }
      }
    }
  }

  // Stores into the K head block `blk` at page slot `off`: codes [slot][D/2],
  // scales [slot % 4][group][slot / 4].
  __device__ __forceinline__ void store_k(uint8_t* blk, int off, int p) const {
    uint8_t* dst = blk + off * (D / 2) + (E / 2) * p;
    if constexpr (E >= 32) {
#pragma unroll
      for (int u = 0; u < E / 32; ++u)
        reinterpret_cast<uint4*>(dst)[u] = make_uint4(w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]);
    } else if constexpr (E == 16) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    } else {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
    }
    if (p % LPG == 0) {
#pragma unroll
      for (int g = 0; g < GPL; ++g)
        blk[CODE + 4 * ((off & 3) * (D / 32) + p / LPG * GPL + g) + (off >> 2)] = (uint8_t)(ex[g] + 127);
    }
  }

  // Stores into the V head block `blk` at page slot `off`: channel pair c in
  // code row 16 (c % CPL) + c / CPL, column `off`; scales [group][slot].
  __device__ __forceinline__ void store_v(uint8_t* blk, int off, int p) const {
    // pair c = (E/2) p + i lies in row 16 (i % CPL) + ((E/2) p + i) / CPL: a lane
    // base and constant offsets (E/2 is a multiple of CPL)
    static_assert((E / 2) % CPL == 0, "a lane's channel pairs start at a multiple of CPL");
    uint8_t* b = blk + off + kPage * ((E / 2) / CPL * p);
#pragma unroll
    for (int i = 0; i < E / 2; ++i) b[(16 * (i % CPL) + i / CPL) * kPage] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
    if (p % LPG == 0) {
#pragma unroll
      for (int g = 0; g < GPL; ++g) blk[CODE + (p / LPG * GPL + g) * kPage + off] = (uint8_t)(ex[g] + 127);
    }
  }
};

}  // namespace uq
