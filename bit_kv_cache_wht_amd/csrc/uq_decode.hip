// Split-K GQA decode attention over the paged FP4 / FP8 / BF16 cache.
//
// [review] = "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
//            (manon006.tistory.com/395)
//
// Launch sequence on one stream:
//   1. query + plan: the query is rotated and rounded to E4M3 once, outside the
//      key loop ([review] §4.2; skipped for BF16); one extra workgroup turns
//      seq_lens into the list of (sequence, split) pairs.
//   2. decode: persistent workgroups of 4 waves walk the item list; one wave
//      streams the pages of one KV head of one split, four pages per step.
//   3. reduce: merges the split partials (m, l, o), normalizes and, for FP4,
//      rotates the output back with the normalized WHT.
//
// Per step a wave covers 4 pages (64 tokens) of one KV head and up to 16 query
// heads (the GQA group, padded to the 16 MFMA columns):
//   QK  4 x v_mfma_scale_f32_16x16x128_f8f6f4.  A = K, rows = 16 tokens chosen so
//       that lane (h, j) of the result holds page j's tokens 4m..4m+3; the FP4 K
//       group scale is the A block scale, so K is never dequantized ([review] §3.2).
//       B = E4M3 query with unit scale.
//   PV  v_mfma_f32_16x16x32_f16, O^T[channel][head] += V^T[channel][token] P^T;
//       V goes through the hardware FP4 -> f16 conversion with its group scale
//       ([review] §3.2, §6.3), P is float16 (float8 P is far too coarse).
//       Lane (h, j) of the QK result already holds the P values that the B
//       operand of lane (h, j) needs, so P never moves between lanes.
// Operand layouts (verified on gfx950): for the 16x16x128 scaled MFMA, lane l
// holds row/column l%16; an FP4 operand holds k = 32(l/16)..+31 (low nibble
// first) and an FP8 operand k = 16(l/16)..+15 and 64+16(l/16)..+15; lane i+16b
// supplies the scale of row i, k-block b.  For 16x16x32 f16, lane l holds
// k = 8(l/16)..+7; results land in lane l as column l%16, rows 4(l/16)..+3.
#include <type_traits>

#include "uq_device.h"
#include "uq_internal.h"


namespace uq {

namespace {

constexpr int kTargetItems = 1024;   // decode items per launch the plan aims for
constexpr int kCUs = 256;            // MI355X compute units; one 4-wave workgroup per SIMD wave slot

struct PlanHdr {
  int32_t n_bs;   // (sequence, split) pairs
  int32_t pps;    // pages per split, multiple of 4
};

// ------------------------------------------------------------------ plan
__device__ void plan_block(const int32_t* seq_lens, int B, int target_bs, PlanHdr* hdr, int32_t* base,
                           int2* items) {
  __shared__ int32_t red[256];
  __shared__ int32_t s_pps, s_carry;
  const int tid = threadIdx.x;
  int32_t tot = 0;
  for (int b = tid; b < B; b += blockDim.x) tot += (seq_lens[b] + kPage - 1) / kPage;
  red[tid] = tot;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  if (tid == 0) {
    int pps = (red[0] + target_bs - 1) / target_bs;
    pps = pps < 4 ? 4 : (pps + 3) & ~3;
    s_pps = pps;
    s_carry = 0;
  }
  __syncthreads();
  const int pps = s_pps;
  for (int b0 = 0; b0 < B; b0 += blockDim.x) {
    const int b = b0 + tid;
    const int pages = b < B ? (seq_lens[b] + kPage - 1) / kPage : 0;
    const int ns = (pages + pps - 1) / pps;
    red[tid] = ns;
    __syncthreads();
    for (int s = 1; s < 256; s <<= 1) {       // inclusive Hillis-Steele scan
      const int v = tid >= s ? red[tid - s] : 0;
      __syncthreads();
      red[tid] += v;
      __syncthreads();
    }
    const int start = s_carry + red[tid] - ns;
    if (b < B) {
      base[b] = start;
      for (int s = 0; s < ns; ++s) items[start + s] = make_int2(b, s);
    }
    __syncthreads();
    if (tid == blockDim.x - 1) s_carry += red[tid];
    __syncthreads();
  }
  if (tid == 0) {
    base[B] = s_carry;
    hdr->n_bs = s_carry;
    hdr->pps = pps;
  }
}

template <int D, int IN, bool ROT>
__global__ __launch_bounds__(256) void query_plan_kernel(const void* q, uint8_t* qbuf, int rows, const int32_t* seq_lens,
                                                         int B, int target_bs, PlanHdr* hdr, int32_t* base, int2* items) {
  if (blockIdx.x == gridDim.x - 1) {
    plan_block(seq_lens, B, target_bs, hdr, base, items);
    return;
  }
  if (qbuf == nullptr) return;
  constexpr int LPR = D / 32;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int p = lane % LPR;
  const int64_t row0 = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * RPW;
  if (row0 >= rows) return;
  const int64_t row = row0 + lane / LPR;
  const bool in_range = row < rows;
  const int64_t r = in_range ? row : 0;
  double x[32];
  if constexpr (IN == UQ_IN_BF16) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(q) + r * D + 32 * p);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint4 u = src[w];
      const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * w + 2 * i] = bf16_bits_to_f64(d[i] & 0xFFFFu);
        x[8 * w + 2 * i + 1] = bf16_bits_to_f64(d[i] >> 16);
      }
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(q) + r * D + 32 * p);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float4 f = src[w];
      x[4 * w] = f.x; x[4 * w + 1] = f.y; x[4 * w + 2] = f.z; x[4 * w + 3] = f.w;
    }
  }
  if constexpr (ROT) wht_row<D>(x, lane);
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = e4m3_from_f64(x[4 * i]) | e4m3_from_f64(x[4 * i + 1]) << 8 | e4m3_from_f64(x[4 * i + 2]) << 16 |
           e4m3_from_f64(x[4 * i + 3]) << 24;
  if (!in_range) return;
  uint4* o = reinterpret_cast<uint4*>(qbuf + r * D + 32 * p);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// ------------------------------------------------------------------ formats
// Each policy loads one step (4 pages) into registers and provides:
//   qk(step, q, S)       S[m] = 16x16 logits for token rows of MFMA m
//   v_operand(step, t, half, A)  f16 A operand (V^T) of output tile t for the
//                        token half (slots 0..7 or 8..15) of page j
//   channel(t, j, v)     output channel of accumulator element v of tile t
// Tiles: D/16 output tiles of 16 channels.

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// PV product with P = hi + lo split into two float16 parts: float16 alone keeps
// 11 bits of each probability, which against value channels of magnitude ~50
// leaves errors near 1e-2; the split carries ~22 bits.
__device__ __forceinline__ v4f mma2(const v8h& a, const v8h (&p)[2], v4f c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p[0], c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p[1], c, 0, 0, 0);
}

// E4M3 query as the FP8 B operand: lane (h, j) holds k = 16j..16j+15 and
// 64+16j..64+16j+15 of query row h (zero rows past the GQA group).
template <int D> __device__ __forceinline__ v8i load_q_fp8(const uint8_t* qrow, bool valid, int j4) {
  uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
  if (valid) {
    lo = load16(qrow + 16 * j4);
    if constexpr (D == 128) hi = load16(qrow + 64 + 16 * j4);
  }
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// FP4.  Lane (r, j) of the PV product owns channel pairs CPL*r .. CPL*r + CPL-1
// (CPL = D/32, i.e. channels 2*CPL*r .. 2*CPL*r + 2*CPL - 1, all in group
// r*CPL/16), so one scale per token serves all of its conversions.
template <int D> struct Fp4Pol {
  static constexpr int kOcc = 2;        // waves per SIMD (256 registers each)
  static constexpr int kStages = 2;
  static constexpr int kBlk = Fp4Block<D>::kBytes;
  static constexpr int kCode = Fp4Block<D>::kCodeBytes;
  static constexpr int kGroups = D / 32;
  static constexpr int kCPL = D / 32;             // channel pairs per lane
  static constexpr int kTiles = D / 16;
  struct Step {
    uint4 kc[4];          // K codes, MFMA m: token slot 4m + (lane%16)%4, group lane/16
    uint32_t ks;          // K scale bytes of those 4 tokens (byte m)
    uint4 vc[kCPL];       // V codes of channel pair kCPL*(lane%16) + q, slots 0..15
    uint4 vs;             // V scale bytes of that group, slots 0..15
  };
  struct QOp { v8i b; };
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4) {
    qo.b = load_q_fp8<D>(qrow, valid, j4);
  }
  __device__ static void load(Step& st, const uint8_t* kb, const uint8_t* vb, int r16, int j4) {
    if (j4 < kGroups) {
#pragma unroll
      for (int m = 0; m < 4; ++m) st.kc[m] = load16(kb + (4 * m + (r16 & 3)) * (D / 2) + 16 * j4);
      // scale bytes are stored [slot % 4][group][slot / 4]: one dword per lane
      st.ks = *reinterpret_cast<const uint32_t*>(kb + kCode + 4 * ((r16 & 3) * kGroups + j4));
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) st.kc[m] = make_uint4(0, 0, 0, 0);
      st.ks = 0x7F7F7F7Fu;
    }
#pragma unroll
    for (int q = 0; q < kCPL; ++q) st.vc[q] = load16(vb + (kCPL * r16 + q) * kPage);
    st.vs = load16(vb + kCode + kPage * ((kCPL * r16) / 16));
  }
  template <int M> __device__ static v4f qk1(const Step& st, const QOp& qo) {
    const v8i a = v8i{(int)st.kc[M].x, (int)st.kc[M].y, (int)st.kc[M].z, (int)st.kc[M].w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qo.b, v4f{0, 0, 0, 0}, 4 /*A fp4*/, 0 /*B fp8*/,
                                                           M /*byte M of ks*/, (int)st.ks, 0, 127);
  }
  __device__ static void qk(const Step& st, const QOp& qo, v4f (&S)[4]) {
    S[0] = qk1<0>(st, qo);
    S[1] = qk1<1>(st, qo);
    S[2] = qk1<2>(st, qo);
    S[3] = qk1<3>(st, qo);
  }
  template <class MaskFn>
  __device__ static void pv(const Step& st, const v8h (&P)[2][2], v4f (&O)[kTiles], MaskFn mask) {
    const uint32_t s[4] = {st.vs.x, st.vs.y, st.vs.z, st.vs.w};
    float sc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) sc[t] = __uint_as_float(((s[t >> 2] >> (8 * (t & 3))) & 0xFFu) << 23);
#pragma unroll
    for (int q = 0; q < kCPL; ++q) {
      const uint32_t c[4] = {st.vc[q].x, st.vc[q].y, st.vc[q].z, st.vc[q].w};
      uint32_t X[16];      // slot t: (channel 2cp, channel 2cp + 1) scaled by 2^(byte_t - 127)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        v2h h;
        switch (t & 3) {
          case 0: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 0); break;
          case 1: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 1); break;
          case 2: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 2); break;
          default: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 3); break;
        }
        X[t] = __builtin_bit_cast(uint32_t, h);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t ev[4], od[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t x0 = X[8 * half + 2 * i], x1 = X[8 * half + 2 * i + 1];
          ev[i] = mask(half, i, __builtin_amdgcn_perm(x1, x0, 0x05040100u));   // low halves: even channel
          od[i] = mask(half, i, __builtin_amdgcn_perm(x1, x0, 0x07060302u));   // high halves: odd channel
        }
        const v8h ae = __builtin_bit_cast(v8h, make_uint4(ev[0], ev[1], ev[2], ev[3]));
        const v8h ao = __builtin_bit_cast(v8h, make_uint4(od[0], od[1], od[2], od[3]));
        O[2 * q] = mma2(ae, P[half], O[2 * q]);
        O[2 * q + 1] = mma2(ao, P[half], O[2 * q + 1]);
      }
    }
  }
  // Tile 2q + par, row 4j + v: channel pair kCPL * (4j + v) + q, channel 2 * pair + par.
  __device__ static int channel(int tile, int j4, int v) { return 2 * (kCPL * (4 * j4 + v) + (tile >> 1)) + (tile & 1); }
};

// FP8 baseline.  QK runs on f16 MFMAs after an exact E4M3 -> f16 conversion:
// the FP8 x FP8 MFMAs (16x16x128 scaled and 16x16x32) drop low-order bits of
// small products when large ones are present in the same instruction, which
// with unrotated outlier channels moves logits by ~1e-4 relative.
template <int D> struct Fp8Pol {
  static constexpr int kOcc = 1;
  static constexpr int kStages = 3;
  static constexpr int kBlk = kPage * D;
  static constexpr int kTiles = D / 16;
  static constexpr int kLanesK = D / 32;   // lane groups holding 32 channels of a row
  struct Step {
    uint4 k[4][2];          // K bytes 32j..32j+31 of token slot 4m + (lane%16)%4
    uint4 vc[kTiles];       // V bytes of channel 16t + lane%16, slots 0..15
  };
  // q as f16 B operands: MFMA kk pairs k-block j with channels 32j + 8kk..+7
  struct QOp { v8h b[4]; };
  __device__ static v8h cvt8(uint32_t w0, uint32_t w1) {
    const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4) {
    uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
    if (valid && j4 < kLanesK) {
      lo = load16(qrow + 32 * j4);
      hi = load16(qrow + 32 * j4 + 16);
    }
    qo.b[0] = cvt8(lo.x, lo.y);
    qo.b[1] = cvt8(lo.z, lo.w);
    qo.b[2] = cvt8(hi.x, hi.y);
    qo.b[3] = cvt8(hi.z, hi.w);
  }
  __device__ static void load(Step& st, const uint8_t* kb, const uint8_t* vb, int r16, int j4) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int slot = 4 * m + (r16 & 3);
      if (j4 < kLanesK) {
        st.k[m][0] = load16(kb + slot * D + 32 * j4);
        st.k[m][1] = load16(kb + slot * D + 32 * j4 + 16);
      } else {
        st.k[m][0] = st.k[m][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) st.vc[t] = load16(vb + (16 * t + r16) * kPage);
  }
  __device__ static void qk(const Step& st, const QOp& qo, v4f (&S)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4f acc = {0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cvt8(st.k[m][0].x, st.k[m][0].y), qo.b[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cvt8(st.k[m][0].z, st.k[m][0].w), qo.b[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cvt8(st.k[m][1].x, st.k[m][1].y), qo.b[2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(cvt8(st.k[m][1].z, st.k[m][1].w), qo.b[3], acc, 0, 0, 0);
      S[m] = acc;
    }
  }
  template <class MaskFn>
  __device__ static void pv(const Step& st, const v8h (&P)[2][2], v4f (&O)[kTiles], MaskFn mask) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const uint32_t c[4] = {st.vc[t].x, st.vc[t].y, st.vc[t].z, st.vc[t].w};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t word = c[2 * half + (i >> 1)];
          const v2h h = (i & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true)
                                : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
          a[i] = mask(half, i, __builtin_bit_cast(uint32_t, h));
        }
        O[t] = mma2(__builtin_bit_cast(v8h, make_uint4(a[0], a[1], a[2], a[3])), P[half], O[t]);
      }
    }
  }
  __device__ static int channel(int tile, int j4, int v) { return 16 * tile + 4 * j4 + v; }
};

template <int D> struct Bf16Pol {
  static constexpr int kOcc = 1;
  static constexpr int kStages = 2;
  static constexpr int kBlk = kPage * D * 2;
  static constexpr int kTiles = D / 16;
  static constexpr int kK = D / 32;     // 16x16x32 MFMAs per token row
  struct Step {
    uint4 k[4][kK];        // K bf16 channels 32kk + 8j..+7 of token slot 4m + (lane%16)%4
    uint4 v[kTiles][2];    // V bf16 of channel 16t + lane%16, slots 0..7 and 8..15
  };
  struct QOp { v8bf b[kK]; };
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4) {
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      const uint4 u = valid ? load16(qrow + 2 * (32 * kk + 8 * j4)) : make_uint4(0, 0, 0, 0);
      qo.b[kk] = __builtin_bit_cast(v8bf, u);
    }
  }
  __device__ static void load(Step& st, const uint8_t* kb, const uint8_t* vb, int r16, int j4) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int slot = 4 * m + (r16 & 3);
#pragma unroll
      for (int kk = 0; kk < kK; ++kk) st.k[m][kk] = load16(kb + 2 * (slot * D + 32 * kk + 8 * j4));
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      st.v[t][0] = load16(vb + 2 * ((16 * t + r16) * kPage));
      st.v[t][1] = load16(vb + 2 * ((16 * t + r16) * kPage + 8));
    }
  }
  __device__ static void qk(const Step& st, const QOp& qo, v4f (&S)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4f acc = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < kK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, st.k[m][kk]), qo.b[kk], acc, 0, 0, 0);
      S[m] = acc;
    }
  }
  template <class MaskFn>
  __device__ static void pv(const Step& st, const v8h (&P)[2][2], v4f (&O)[kTiles], MaskFn mask) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t c[4] = {st.v[t][half].x, st.v[t][half].y, st.v[t][half].z, st.v[t][half].w};
        uint32_t a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(c[i] << 16), hi = __uint_as_float(c[i] & 0xFFFF0000u);
          a[i] = mask(half, i, pack_h2((_Float16)lo, (_Float16)hi));
        }
        O[t] = mma2(__builtin_bit_cast(v8h, make_uint4(a[0], a[1], a[2], a[3])), P[half], O[t]);
      }
    }
  }
  __device__ static int channel(int tile, int j4, int v) { return 16 * tile + 4 * j4 + v; }
};

// ------------------------------------------------------------------ decode
struct KArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t page_bytes;
  const int32_t* page_table;
  int32_t max_pages;
  const int32_t* seq_lens;
  const uint8_t* q;          // E4M3 query (FP4/FP8) or the caller's bf16 query
  int64_t q_row_bytes;
  int32_t Hq, Hkv, G, n_hg;
  float scale_log2;          // sm_scale * log2(e)
  const PlanHdr* hdr;
  const int2* items;
  float2* ml;                // [bs][Hq] (m in log2 units, l)
  float* po;                 // [bs][Hq][D]
};

template <class Pol, int D>
__global__ __launch_bounds__(256, Pol::kOcc) void decode_kernel(const KArgs a, const int32_t* __restrict__ page_table,
                                                        const int2* __restrict__ items,
                                                        const int32_t* __restrict__ seq_lens) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, j4 = lane >> 4;
  const int n_items = a.hdr->n_bs * a.n_hg;
  const int pps = a.hdr->pps;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int bs = item / a.n_hg;
    const int hk = (item - bs * a.n_hg) * kWavesPerWG + wave;
    if (hk >= a.Hkv) continue;
    const int2 it2 = items[bs];
    const int b = it2.x;
    const int L = seq_lens[b];
    const int pages = (L + kPage - 1) / kPage;
    const int p_begin = it2.y * pps;
    const int p_end = min(p_begin + pps, pages);
    const int n_step = (p_end - p_begin + 3) >> 2;
    const int32_t* pt = page_table + (int64_t)b * a.max_pages;
    const int hq0 = hk * a.G;

    typename Pol::QOp qo;
    Pol::load_q(qo, a.q + (int64_t)(b * a.Hq + hq0 + r16) * a.q_row_bytes, r16 < a.G, j4);

    float m_run = -INFINITY, l_run = 0.f;
    const float m_slack = 8.0f / a.scale_log2;     // 2^8 headroom in raw logit units
    v4f O[Pol::kTiles];
#pragma unroll
    for (int t = 0; t < Pol::kTiles; ++t) O[t] = v4f{0, 0, 0, 0};

    const int64_t head_off = (int64_t)hk * Pol::kBlk;
    // The four page ids of a step are wave-uniform: scalar loads fetch them one
    // step ahead of the data loads that use them.  A vector load here would sit
    // at the back of the in-order vector-memory counter, and waiting for it
    // would also wait for every prefetch issued before it.
    struct Ids { int v[4]; };
    auto fetch_ids = [&](int s) {
      Ids r;
      const int pg = p_begin + 4 * s;
#pragma unroll
      for (int x = 0; x < 4; ++x) r.v[x] = pt[min(pg + x, p_end - 1)];
      return r;
    };
    auto pick = [](const Ids& ids, int x) {
      return x == 0 ? ids.v[0] : x == 1 ? ids.v[1] : x == 2 ? ids.v[2] : ids.v[3];
    };
    auto load_step = [&](typename Pol::Step& st, const Ids& ids) {
      const int idk = pick(ids, r16 >> 2), idv = pick(ids, j4);
      Pol::load(st, a.k_pool + (int64_t)idk * a.page_bytes + head_off, a.v_pool + (int64_t)idv * a.page_bytes + head_off,
                r16, j4);
    };
    // One step: QK, online softmax, PV.  MASKED handles a partial last step
    // (pages past the split, slots past the sequence); every other step is full.
    auto compute_step = [&](const typename Pol::Step& st, int s, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int pg = p_begin + 4 * s;
      v4f S[4];
      Pol::qk(st, qo, S);
      // tokens of page pg + j4 held by this lane: slots 4m + v
      int nvalid = kPage;
      float t[16];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) t[4 * m + v] = S[m][v];
      if constexpr (MASKED) {
        const int tok0 = (pg + j4) * kPage;
        nvalid = (pg + j4 < p_end) ? min(kPage, L - tok0) : 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = i < nvalid ? t[i] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
#pragma unroll
      for (int i = 4; i < 16; i += 2) mx = fmaxf(mx, fmaxf(t[i], t[i + 1]));
      // Conditional rescaling: exponents are taken against the running reference
      // m_run as long as no logit exceeds it by more than 8 / scale_log2 (so
      // p <= 2^8, well inside float16); only then is the reference raised,
      // which needs the cross-lane maximum and a rescale of l and O.
      if (__any(mx > m_run + m_slack)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
        l_run *= alpha;
#pragma unroll
        for (int tt = 0; tt < Pol::kTiles; ++tt) O[tt] *= alpha;
        m_run = m_new;
      }
      const float neg_mc = -m_run * a.scale_log2;
      float psum = 0.f;
      float pf[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[i], a.scale_log2, neg_mc));
        psum += pf[i];
      }
      l_run += psum;
      v8h P[2][2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const _Float16 hi = (_Float16)pf[8 * half + i];
          P[half][0][i] = hi;
          P[half][1][i] = (_Float16)__builtin_fmaf((float)hi, -1.0f, pf[8 * half + i]);   // exact p - hi
        }
      if constexpr (!MASKED) {
        Pol::pv(st, P, O, [](int, int, uint32_t x) { return x; });
      } else {
        // zero V of slots past the valid ones so garbage in unwritten slots cannot
        // turn 0 * inf into NaN; dword i of half h holds slots 8h + 2i, 8h + 2i + 1
        Pol::pv(st, P, O, [nvalid](int half, int i, uint32_t x) {
          const int s0 = 8 * half + 2 * i;
          const uint32_t keep = (s0 < nvalid ? 0xFFFFu : 0u) | (s0 + 1 < nvalid ? 0xFFFF0000u : 0u);
          return x & keep;
        });
      }
    };

    // Software pipeline: kStages register buffers, kStages - 1 steps of loads in
    // flight while one step computes (latency x bandwidth needs ~100 KB in
    // flight per CU).  Buffer indices are compile-time after unrolling.
    // Prefetches are issued unconditionally, clamped to the last step (those
    // addresses were just loaded, so the repeats hit in L2), which keeps the
    // number of outstanding loads the same on every path and lets each step
    // wait only for its own data.
    constexpr int P = Pol::kStages;
    typename Pol::Step st[P];
    const int last = n_step - 1;
    // the last step is full when its 4 pages exist and hold 64 valid tokens
    const bool last_full = (p_begin + 4 * n_step <= p_end) && ((p_begin + 4 * n_step) * kPage <= L);
#pragma unroll
    for (int i = 0; i < P - 1; ++i) load_step(st[i], fetch_ids(min(i, last)));
    Ids next = fetch_ids(min(P - 1, last));
    for (int s0 = 0;; s0 += P) {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const int cur = s0 + i;
        if (cur > last) goto steps_done;
        load_step(st[(i + P - 1) % P], next);
        next = fetch_ids(min(cur + P, last));
        if (cur < last || last_full) compute_step(st[i], cur, std::false_type{});
        else compute_step(st[i], cur, std::true_type{});
      }
    }
  steps_done:

    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (r16 < a.G) {
      const int64_t prow = (int64_t)bs * a.Hq + hq0 + r16;
      float* o = a.po + prow * D;
#pragma unroll
      for (int tt = 0; tt < Pol::kTiles; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[Pol::channel(tt, j4, v)] = O[tt][v];
      if (j4 == 0) a.ml[prow] = make_float2(m_run * a.scale_log2, l_tot);
    }
  }
}

// ------------------------------------------------------------------ reduce
template <int D, bool UNROT>
__global__ __launch_bounds__(256) void reduce_kernel(const PlanHdr* hdr, const int32_t* base, const float2* ml,
                                                     const float* po, float* out, int rows, int Hq) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int b = row / Hq, h = row - b * Hq;
  const int s0 = base[b], ns = base[b + 1] - s0;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  if (ns > 0) {
    // split headers: lane s holds (m, l) of split s (64 splits per pass)
    float mmax = -INFINITY;
    for (int c = 0; c < ns; c += 64) {
      const float m = c + lane < ns ? ml[(int64_t)(s0 + c + lane) * Hq + h].x : -INFINITY;
      mmax = fmaxf(mmax, m);
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, x));
    float l = 0.f;
    for (int c = 0; c < ns; c += 64) {
      const int n = min(64, ns - c);
      float w = 0.f, lw = 0.f;
      if (lane < n) {
        const float2 v = ml[(int64_t)(s0 + c + lane) * Hq + h];
        w = __builtin_amdgcn_exp2f(v.x - mmax);
        lw = w * v.y;
      }
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) lw += __shfl_xor(lw, x);
      l += lw;
      const float* src = po + ((int64_t)(s0 + c) * Hq + h) * D + lane;
      const int64_t stride = (int64_t)Hq * D;
      int s = 0;
      for (; s + 4 <= n; s += 4) {               // four independent split rows in flight
        float v[4][PER];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int k = 0; k < PER; ++k) v[u][k] = src[(s + u) * stride + 64 * k];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float wu = __shfl(w, s + u);
#pragma unroll
          for (int k = 0; k < PER; ++k) o[k] += wu * v[u][k];
        }
      }
      for (; s < n; ++s) {
        const float ws = __shfl(w, s);
#pragma unroll
        for (int k = 0; k < PER; ++k) o[k] += ws * src[s * stride + 64 * k];
      }
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] *= inv;
    if constexpr (UNROT) {
      if constexpr (PER == 2) {           // stage h = 64 is inside the lane
        const float x0 = o[0], x1 = o[1];
        o[0] = x0 + x1;
        o[1] = x0 - x1;
      }
#pragma unroll
      for (int hh = 32; hh >= 1; hh >>= 1) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const float other = __shfl_xor(o[k], hh);
          o[k] = (lane & hh) ? other - o[k] : o[k] + other;
        }
      }
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] *= wht_cf<D>();
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) out[(int64_t)row * D + lane + 64 * k] = o[k];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  const DecodeLayout& L = a.lay;
  PlanHdr* hdr = reinterpret_cast<PlanHdr*>(a.ws + L.hdr);
  int32_t* base = reinterpret_cast<int32_t*>(a.ws + L.base);
  int2* items = reinterpret_cast<int2*>(a.ws + L.items);
  uint8_t* qbuf = a.ws + L.qbuf;
  float2* ml = reinterpret_cast<float2*>(a.ws + L.ml);
  float* po = reinterpret_cast<float*>(a.ws + L.po);
  const int rows = a.B * a.Hq;
  const bool want_q = a.format != UQ_KV_BF16;
  const bool rot = a.format == UQ_KV_FP4;
  const unsigned qblocks = want_q ? (unsigned)(((rows + 64 / (D / 32) - 1) / (64 / (D / 32)) + 3) / 4) : 0;
  const dim3 g1(qblocks + 1), blk(256);
#define UQ_QP(II, RR) hipLaunchKernelGGL((query_plan_kernel<D, II, RR>), g1, blk, 0, s, a.q, want_q ? qbuf : nullptr, \
                                         rows, a.seq_lens, a.B, L.target_bs, hdr, base, items)
  if (a.q_dtype == UQ_IN_BF16) { if (rot) UQ_QP(UQ_IN_BF16, true); else UQ_QP(UQ_IN_BF16, false); }
  else { if (rot) UQ_QP(UQ_IN_F32, true); else UQ_QP(UQ_IN_F32, false); }
#undef UQ_QP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  KArgs k;
  k.k_pool = a.k_pool;
  k.v_pool = a.v_pool;
  k.page_bytes = a.page_bytes;
  k.page_table = a.page_table;
  k.max_pages = a.max_pages;
  k.seq_lens = a.seq_lens;
  k.q = want_q ? qbuf : static_cast<const uint8_t*>(a.q);
  k.q_row_bytes = want_q ? D : 2 * D;
  k.Hq = a.Hq;
  k.Hkv = a.Hkv;
  k.G = a.Hq / a.Hkv;
  k.n_hg = (a.Hkv + kWavesPerWG - 1) / kWavesPerWG;
  k.scale_log2 = a.sm_scale * 1.4426950408889634f;
  k.hdr = hdr;
  k.items = items;
  k.ml = ml;
  k.po = po;
  const int max_items = L.max_bs * k.n_hg;
  const int occ = a.format == UQ_KV_FP4 ? Fp4Pol<D>::kOcc : 1;
  const int wgs = kCUs * occ;
  const dim3 g2((unsigned)(max_items < wgs ? max_items : wgs));
  if (a.ev_start != nullptr) {
    e = hipEventRecord(a.ev_start, s);
    if (e != hipSuccess) return e;
  }
  if (a.format == UQ_KV_FP4)
    hipLaunchKernelGGL((decode_kernel<Fp4Pol<D>, D>), g2, blk, 0, s, k, a.page_table, items, a.seq_lens);
  else if (a.format == UQ_KV_FP8)
    hipLaunchKernelGGL((decode_kernel<Fp8Pol<D>, D>), g2, blk, 0, s, k, a.page_table, items, a.seq_lens);
  else hipLaunchKernelGGL((decode_kernel<Bf16Pol<D>, D>), g2, blk, 0, s, k, a.page_table, items, a.seq_lens);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_stop != nullptr) {
    e = hipEventRecord(a.ev_stop, s);
    if (e != hipSuccess) return e;
  }

  const dim3 g3((unsigned)((rows + 3) / 4));
  if (a.unrotate) hipLaunchKernelGGL((reduce_kernel<D, true>), g3, blk, 0, s, hdr, base, ml, po, a.out, rows, a.Hq);
  else hipLaunchKernelGGL((reduce_kernel<D, false>), g3, blk, 0, s, hdr, base, ml, po, a.out, rows, a.Hq);
  return hipGetLastError();
}

}  // namespace

DecodeLayout decode_layout(int format, int B, int Hq, int Hkv, int D) {
  DecodeLayout L;
  const int n_hg = (Hkv + kWavesPerWG - 1) / kWavesPerWG;
  L.target_bs = (kTargetItems + n_hg - 1) / n_hg;
  L.max_bs = L.target_bs + B;
  size_t off = 0;
  L.hdr = off; off = align256(off + sizeof(PlanHdr));
  L.base = off; off = align256(off + sizeof(int32_t) * (size_t)(B + 1));
  L.items = off; off = align256(off + sizeof(int2) * (size_t)L.max_bs);
  L.qbuf = off; off = align256(off + (format == UQ_KV_BF16 ? 0 : (size_t)B * Hq * D));
  L.ml = off; off = align256(off + sizeof(float2) * (size_t)L.max_bs * Hq);
  L.po = off; off = align256(off + sizeof(float) * (size_t)L.max_bs * Hq * D);
  L.total = off;
  return L;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? launch_decode_d<128>(a, s) : launch_decode_d<64>(a, s);
}

}  // namespace uq
