// Split-K GQA decode attention over the paged FP4 / FP8 / BF16 cache, one kernel.
//
// [review] = "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
//            (manon006.tistory.com/395)
//
// One launch per call.  Each workgroup derives the split plan from seq_lens in
// LDS, rotates and rounds its query rows to E4M3 once, outside the key loop
// ([review] §4.2; BF16 keeps bf16), streams the pages of its (sequence, KV head,
// split) item with its four waves, merges them in LDS and writes the output
// rotated back with the normalized WHT.  Sequences split across workgroups are
// merged by the last workgroup to finish.
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

constexpr int kTargetItems = 512;    // decode items per launch the plan aims for (one per workgroup)
constexpr int kCUs = 256;            // MI355X compute units; one 4-wave workgroup per SIMD wave slot

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
    uint4 vc[kCPL];       // V codes of channel pair kCPL*(lane%16) + q (row 16q + lane%16), slots 0..15
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
    for (int q = 0; q < kCPL; ++q) st.vc[q] = load16(vb + (16 * q + r16) * kPage);   // pair kCPL*r16 + q
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

// ------------------------------------------------------------------ plan
// Every workgroup derives the split plan from seq_lens in LDS: pages per split
// pps (a multiple of 4, sized so that the (sequence, split) pairs number about
// target_bs) and base[b] = first pair of sequence b, base[B] = number of pairs.
// A sequence of length 0 still gets one (empty) pair so that its output row is
// written.
__device__ void wg_plan(const int32_t* __restrict__ seq_lens, int B, int target_bs, int32_t* base, int32_t* red,
                        int32_t& pps_out) {
  const int tid = threadIdx.x;
  int32_t tot = 0;
  for (int b = tid; b < B; b += 256) tot += (seq_lens[b] + kPage - 1) / kPage;
  red[tid] = tot;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  int pps = (red[0] + target_bs - 1) / target_bs;
  pps = pps < 4 ? 4 : (pps + 3) & ~3;
  __syncthreads();
  int32_t carry = 0;
  for (int b0 = 0; b0 < B; b0 += 256) {
    const int b = b0 + tid;
    const int pages = b < B ? (seq_lens[b] + kPage - 1) / kPage : 0;
    const int ns = b < B ? max(1, (pages + pps - 1) / pps) : 0;
    red[tid] = ns;
    __syncthreads();
    for (int st = 1; st < 256; st <<= 1) {      // inclusive Hillis-Steele scan
      const int v = tid >= st ? red[tid - st] : 0;
      __syncthreads();
      red[tid] += v;
      __syncthreads();
    }
    if (b < B) base[b] = carry + red[tid] - ns;
    carry += red[255];
    __syncthreads();
  }
  if (tid == 0) base[B] = carry;
  __syncthreads();
  pps_out = pps;
}

// Query rows of one workgroup into LDS: E4M3 bytes of the (FP4: rotated) rows
// row0 .. row0 + n - 1 of q, zero rows up to 16; BF16 keeps the bf16 values.
// Run by one wave; D/32 lanes per row as in the write path.
template <int D, int IN, int FMT>
__device__ void query_rows(const void* q, int64_t row0, int n, uint8_t* qs, int lane) {
  if constexpr (FMT == UQ_KV_BF16) {
    // 16 rows x D bf16; 16 bytes per lane per pass
    constexpr int kChunks = 16 * D * 2 / 16;
    for (int c = lane; c < kChunks; c += 64) {
      const int r = c / (D / 8), k = c - r * (D / 8);
      const uint4 v = r < n ? load16(static_cast<const uint16_t*>(q) + (row0 + r) * D + 8 * k) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(qs + 16 * c) = v;
    }
  } else {
    constexpr int LPR = D / 32;
    const int rr = lane / LPR, p = lane % LPR;
    if (rr >= 16) return;                          // whole quads drop out together
    double x[32];
    if (rr < n) {
      load_row32<IN>(q, (row0 + rr) * D + 32 * p, x);
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = 0.0;
    }
    if constexpr (FMT == UQ_KV_FP4) wht_row<D>(x, lane);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = e4m3_from_f64(x[4 * i]) | e4m3_from_f64(x[4 * i + 1]) << 8 | e4m3_from_f64(x[4 * i + 2]) << 16 |
             e4m3_from_f64(x[4 * i + 3]) << 24;
    uint4* o = reinterpret_cast<uint4*>(qs + rr * D + 32 * p);
    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
    o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Normalizes one merged output row held as channels lane + 64k and, for FP4,
// rotates it back with the normalized WHT (stage h = 64 inside the lane, the
// others across lanes), then stores it.
template <int D, bool UNROT>
__device__ void store_row(float (&o)[D / 64], float l, float* dst, int lane) {
  constexpr int PER = D / 64;
  const float inv = l > 0.f ? 1.f / l : 0.f;      // l == 0 only for empty sequences
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] *= inv;
  if constexpr (UNROT) {
    if constexpr (PER == 2) {
      const float x0 = o[0], x1 = o[1];
      o[0] = x0 + x1;
      o[1] = x0 - x1;
    }
#pragma unroll
    for (int hh = 32; hh >= 1; hh >>= 1)
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const float other = __shfl_xor(o[k], hh);
        o[k] = (lane & hh) ? other - o[k] : o[k] + other;
      }
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] *= wht_cf<D>();
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) dst[lane + 64 * k] = o[k];
}

// ------------------------------------------------------------------ decode
struct KArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t page_bytes;
  int32_t max_pages;
  const void* q;             // caller's query [B][Hq][D], bf16 or f32
  int32_t B, Hq, Hkv, G;
  int32_t target_bs;
  float scale_log2;          // sm_scale * log2(e)
  float* out;                // [B][Hq][D]
  float2* ml;                // [bs][Hq] (m in log2 units, l) of multi-split sequences
  float* po;                 // [bs][Hq][D]
  int32_t* cnt;              // [B][Hkv] arrival counters, zero between calls
};

// LDS carve-up of one workgroup (bytes): query rows, four per-wave partial
// results (m, l, O for 16 heads), the plan scratch and base[B + 1].
template <int D, int FMT> struct Smem {
  static constexpr int kQ = 16 * D * (FMT == UQ_KV_BF16 ? 2 : 1);
  static constexpr int kO = kQ;                                // [4][16][D] float
  static constexpr int kM = kO + 4 * 16 * D * 4;               // [4][16] float
  static constexpr int kL = kM + 4 * 16 * 4;                   // [4][16] float
  static constexpr int kFlag = kL + 4 * 16 * 4;
  static constexpr int kRed = kFlag + 16;                      // [256] int
  static constexpr int kBase = kRed + 256 * 4;                 // [B + 1] int
  static size_t bytes(int B) { return (size_t)kBase + 4 * (size_t)(B + 1); }
};

// One workgroup per item (sequence b, KV head hk, split s of pps pages); its
// four waves take consecutive quarters of the split's 4-page steps and merge in
// LDS.  A sequence with one split writes its output directly; otherwise each
// split writes a partial and the last one to arrive (device-scope counter)
// merges them.
template <class Pol, int D, int IN, int FMT, bool UNROT>
__global__ __launch_bounds__(256, Pol::kOcc) void decode_kernel(const KArgs a, const int32_t* __restrict__ page_table,
                                                                const int32_t* __restrict__ seq_lens) {
  using SM = Smem<D, FMT>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* qs = smem;
  float* mo = reinterpret_cast<float*>(smem + SM::kO);
  float* mm = reinterpret_cast<float*>(smem + SM::kM);
  float* mlw = reinterpret_cast<float*>(smem + SM::kL);
  int32_t* flag = reinterpret_cast<int32_t*>(smem + SM::kFlag);
  int32_t* red = reinterpret_cast<int32_t*>(smem + SM::kRed);
  int32_t* base = reinterpret_cast<int32_t*>(smem + SM::kBase);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, j4 = lane >> 4;
  int pps;
  wg_plan(seq_lens, a.B, a.target_bs, base, red, pps);
  const int n_items = base[a.B] * a.Hkv;

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int bs = item / a.Hkv;
    const int hk = item - bs * a.Hkv;
    int lo = 0, hi = a.B;                        // b: last index with base[b] <= bs
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (base[mid] <= bs) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int n_split = base[b + 1] - base[b];
    const int L = seq_lens[b];
    const int pages = (L + kPage - 1) / kPage;
    const int p_begin = (bs - base[b]) * pps;
    const int p_end = min(p_begin + pps, pages);
    const int n_step = p_end > p_begin ? (p_end - p_begin + 3) >> 2 : 0;
    const int s_lo = wave * n_step / 4, s_hi = (wave + 1) * n_step / 4;   // this wave's steps
    const int32_t* pt = page_table + (int64_t)b * a.max_pages;
    const int hq0 = hk * a.G;
    const int64_t head_off = (int64_t)hk * Pol::kBlk;

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

    constexpr int P = Pol::kStages;
    typename Pol::Step st[P];
    const int last = s_hi - 1;
    if (s_hi > s_lo) {
#pragma unroll
      for (int i = 0; i < P - 1; ++i) load_step(st[i], fetch_ids(min(s_lo + i, last)));
    }
    if (wave == 0) query_rows<D, IN, FMT>(a.q, (int64_t)b * a.Hq + hq0, a.G, qs, lane);
    __syncthreads();
    typename Pol::QOp qo;
    Pol::load_q(qo, qs + r16 * D * (FMT == UQ_KV_BF16 ? 2 : 1), r16 < a.G, j4);

    float m_run = -INFINITY, l_run = 0.f;
    const float m_slack = 8.0f / a.scale_log2;     // 2^8 headroom in raw logit units
    v4f O[Pol::kTiles];
#pragma unroll
    for (int t = 0; t < Pol::kTiles; ++t) O[t] = v4f{0, 0, 0, 0};

    // One step: QK, online softmax, PV.  MASKED handles the split's partial last
    // step (pages past the split, slots past the sequence).
    auto compute_step = [&](const typename Pol::Step& st, int s, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int pg = p_begin + 4 * s;
      v4f S[4];
      Pol::qk(st, qo, S);
      int nvalid = kPage;                          // valid slots of page pg + j4
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
      // p <= 2^8, well inside float16); only then is the reference raised, which
      // needs the cross-lane maximum and a rescale of l and O.
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
      v8h Pm[2][2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const _Float16 hi16 = (_Float16)pf[8 * half + i];
          Pm[half][0][i] = hi16;
          Pm[half][1][i] = (_Float16)__builtin_fmaf((float)hi16, -1.0f, pf[8 * half + i]);   // exact p - hi
        }
      if constexpr (!MASKED) {
        Pol::pv(st, Pm, O, [](int, int, uint32_t x) { return x; });
      } else {
        // zero V of slots past the valid ones so garbage in unwritten slots cannot
        // turn 0 * inf into NaN; dword i of half h holds slots 8h + 2i, 8h + 2i + 1
        Pol::pv(st, Pm, O, [nvalid](int half, int i, uint32_t x) {
          const int s0 = 8 * half + 2 * i;
          const uint32_t keep = (s0 < nvalid ? 0xFFFFu : 0u) | (s0 + 1 < nvalid ? 0xFFFF0000u : 0u);
          return x & keep;
        });
      }
    };

    if (s_hi > s_lo) {
      // Software pipeline over this wave's steps: P register buffers, P - 1 steps
      // of loads in flight.  Prefetches are issued unconditionally (clamped to the
      // wave's last step, whose addresses then hit in L2) so the number of
      // outstanding loads is the same on every path and each step waits only
      // for its own data.  Page ids are wave-uniform: scalar loads fetch them one
      // step ahead, outside the in-order vector-memory counter.
      const bool last_full = (p_begin + 4 * n_step <= p_end) && ((p_begin + 4 * n_step) * kPage <= L);
      const int split_last = n_step - 1;
      Ids next = fetch_ids(min(s_lo + P - 1, last));
      for (int s0 = s_lo;; s0 += P) {
#pragma unroll
        for (int i = 0; i < P; ++i) {
          const int cur = s0 + i;
          if (cur > last) goto steps_done;
          load_step(st[(i + P - 1) % P], next);
          next = fetch_ids(min(cur + P, last));
          if (cur < split_last || last_full) compute_step(st[i], cur, std::false_type{});
          else compute_step(st[i], cur, std::true_type{});
        }
      }
    steps_done:;
    }

    // per-wave result -> LDS: m (log2 units), l (summed over the 4 lane groups), O
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (r16 < a.G) {
      float* o = mo + (wave * 16 + r16) * D;
#pragma unroll
      for (int tt = 0; tt < Pol::kTiles; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[Pol::channel(tt, j4, v)] = O[tt][v];
      if (j4 == 0) {
        mm[wave * 16 + r16] = m_run * a.scale_log2;
        mlw[wave * 16 + r16] = l_tot;
      }
    }
    __syncthreads();

    // merge the 4 waves; wave w handles heads w, w + 4, ...
    constexpr int PER = D / 64;
    for (int h = wave; h < a.G; h += 4) {
      float m = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) m = fmaxf(m, mm[w * 16 + h]);
      float o[PER], l = 0.f;
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] = 0.f;
      if (m > -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float wt = __builtin_amdgcn_exp2f(mm[w * 16 + h] - m);
          l += wt * mlw[w * 16 + h];
#pragma unroll
          for (int k = 0; k < PER; ++k) o[k] += wt * mo[(w * 16 + h) * D + lane + 64 * k];
        }
      }
      const int64_t row = (int64_t)b * a.Hq + hq0 + h;
      if (n_split == 1) {
        store_row<D, UNROT>(o, l, a.out + row * D, lane);
      } else {
        const int64_t prow = (int64_t)bs * a.Hq + hq0 + h;
#pragma unroll
        for (int k = 0; k < PER; ++k) a.po[prow * D + lane + 64 * k] = o[k];
        if (lane == 0) a.ml[prow] = make_float2(m, l);
      }
    }

    if (n_split > 1) {
      // publish the partial; the last split to arrive merges all of them
      __threadfence();
      __syncthreads();
      if (threadIdx.x == 0) {
        int32_t* c = a.cnt + (int64_t)b * a.Hkv + hk;
        const int old = __hip_atomic_fetch_add(c, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const int is_last = old == n_split - 1;
        if (is_last) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = is_last;
      }
      __syncthreads();
      if (*flag) {
        __threadfence();
        const int bs0 = base[b];
        for (int h = wave; h < a.G; h += 4) {
          const int64_t col = hq0 + h;
          float m = -INFINITY;
          for (int c0 = 0; c0 < n_split; c0 += 64) {
            const float mv = c0 + lane < n_split ? a.ml[(int64_t)(bs0 + c0 + lane) * a.Hq + col].x : -INFINITY;
            m = fmaxf(m, mv);
          }
#pragma unroll
          for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
          float o[PER], l = 0.f;
#pragma unroll
          for (int k = 0; k < PER; ++k) o[k] = 0.f;
          for (int c0 = 0; c0 < n_split; c0 += 64) {
            const int n = min(64, n_split - c0);
            float wt = 0.f, lw = 0.f;
            if (lane < n) {
              const float2 v = a.ml[(int64_t)(bs0 + c0 + lane) * a.Hq + col];
              wt = v.x > -INFINITY ? __builtin_amdgcn_exp2f(v.x - m) : 0.f;
              lw = wt * v.y;
            }
#pragma unroll
            for (int x = 32; x >= 1; x >>= 1) lw += __shfl_xor(lw, x);
            l += lw;
            for (int sidx = 0; sidx < n; ++sidx) {
              const float ws = __shfl(wt, sidx);
              const float* src = a.po + ((int64_t)(bs0 + c0 + sidx) * a.Hq + col) * D + lane;
#pragma unroll
              for (int k = 0; k < PER; ++k) o[k] += ws * src[64 * k];
            }
          }
          store_row<D, UNROT>(o, l, a.out + ((int64_t)b * a.Hq + col) * D, lane);
        }
      }
    }
    __syncthreads();                               // LDS is reused by the next item
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int D, int IN, int FMT, bool UNROT, class Pol>
hipError_t launch_one(const DecodeArgs& a, const KArgs& k, hipStream_t s) {
  const size_t lds = Smem<D, FMT>::bytes(a.B);
  const int max_items = a.lay.max_bs * a.Hkv;
  const int wgs = kCUs * Pol::kOcc;
  const dim3 grid((unsigned)(max_items < wgs ? max_items : wgs)), blk(256);
  hipLaunchKernelGGL((decode_kernel<Pol, D, IN, FMT, UNROT>), grid, blk, lds, s, k, a.page_table, a.seq_lens);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t s) {
  const DecodeLayout& L = a.lay;
  KArgs k;
  k.k_pool = a.k_pool;
  k.v_pool = a.v_pool;
  k.page_bytes = a.page_bytes;
  k.max_pages = a.max_pages;
  k.q = a.q;
  k.B = a.B;
  k.Hq = a.Hq;
  k.Hkv = a.Hkv;
  k.G = a.Hq / a.Hkv;
  k.target_bs = L.target_bs;
  k.scale_log2 = a.sm_scale * 1.4426950408889634f;
  k.out = a.out;
  k.ml = reinterpret_cast<float2*>(a.ws + L.ml);
  k.po = reinterpret_cast<float*>(a.ws + L.po);
  k.cnt = reinterpret_cast<int32_t*>(a.ws + L.cnt);
  hipError_t e;
  if (a.ev_start != nullptr && (e = hipEventRecord(a.ev_start, s)) != hipSuccess) return e;
  const bool bf = a.q_dtype == UQ_IN_BF16;
  if (a.format == UQ_KV_FP4) {
    if (a.unrotate) e = bf ? launch_one<D, UQ_IN_BF16, UQ_KV_FP4, true, Fp4Pol<D>>(a, k, s)
                           : launch_one<D, UQ_IN_F32, UQ_KV_FP4, true, Fp4Pol<D>>(a, k, s);
    else e = bf ? launch_one<D, UQ_IN_BF16, UQ_KV_FP4, false, Fp4Pol<D>>(a, k, s)
                : launch_one<D, UQ_IN_F32, UQ_KV_FP4, false, Fp4Pol<D>>(a, k, s);
  } else if (a.format == UQ_KV_FP8) {
    e = bf ? launch_one<D, UQ_IN_BF16, UQ_KV_FP8, false, Fp8Pol<D>>(a, k, s)
           : launch_one<D, UQ_IN_F32, UQ_KV_FP8, false, Fp8Pol<D>>(a, k, s);
  } else {
    e = launch_one<D, UQ_IN_BF16, UQ_KV_BF16, false, Bf16Pol<D>>(a, k, s);
  }
  if (e != hipSuccess) return e;
  if (a.ev_stop != nullptr && (e = hipEventRecord(a.ev_stop, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace

DecodeLayout decode_layout(int format, int B, int Hq, int Hkv, int D) {
  (void)format;
  DecodeLayout L;
  L.target_bs = (kTargetItems + Hkv - 1) / Hkv;
  L.max_bs = L.target_bs + B;
  size_t off = 0;
  L.cnt = off; off = align256(off + sizeof(int32_t) * (size_t)B * Hkv);
  L.ml = off; off = align256(off + sizeof(float2) * (size_t)L.max_bs * Hq);
  L.po = off; off = align256(off + sizeof(float) * (size_t)L.max_bs * Hq * D);
  L.total = off;
  return L;
}

size_t decode_lds_bytes(int format, int B, int D) {
  if (format == UQ_KV_BF16) return D == 128 ? Smem<128, UQ_KV_BF16>::bytes(B) : Smem<64, UQ_KV_BF16>::bytes(B);
  return D == 128 ? Smem<128, UQ_KV_FP4>::bytes(B) : Smem<64, UQ_KV_FP4>::bytes(B);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? launch_decode_d<128>(a, s) : launch_decode_d<64>(a, s);
}

}  // namespace uq
