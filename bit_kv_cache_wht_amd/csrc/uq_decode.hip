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
#include <atomic>
#include <type_traits>

#include "uq_device.h"
#include "uq_fp4_row.h"
#include "uq_internal.h"


namespace uq {

namespace {

constexpr int kMaxGrid = 1024;       // workgroups per launch, at most (one per compute unit)
constexpr int kMaxR = 8;             // items per round of a workgroup, at most

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

// Where an item's head blocks sit in a page: head0 = the item's first KV head
// (FP4 blocks at position (h + 2 page) mod H, see fp4_block_pos; FP8 and BF16
// blocks at position h).
struct PageGeo {
  int head0;
  int H;
  int mask;
  int units, umask;   // FP8 byte rotation (fp8_rot)
};

// One of a step's page ids (wave-uniform values) by a lane-dependent index.
__device__ __forceinline__ int pick_id(const int (&ids)[4], int x) {
  return x == 0 ? ids[0] : x == 1 ? ids[1] : x == 2 ? ids[2] : ids[3];
}

// Keep-masks for the slots of one page that are valid (slot < nvalid): bytes
// (slot t = byte t of 16) and 16-bit halves (slot t = half t of 16).
__device__ __forceinline__ uint32_t slot_bytes_kept(int nvalid, int first) {
  const int n = nvalid - first;                   // valid slots among first .. first + 3
  return n >= 4 ? 0xFFFFFFFFu : n <= 0 ? 0u : (1u << (8 * n)) - 1u;
}
__device__ __forceinline__ uint32_t slot_halves_kept(int nvalid, int first) {
  const int n = nvalid - first;                   // valid slots among first, first + 1
  return n >= 2 ? 0xFFFFFFFFu : n <= 0 ? 0u : 0xFFFFu;
}

// PV product with P = hi + lo split into two float16 parts: float16 alone keeps
// 11 bits of each probability, which against value channels of magnitude ~50
// leaves errors near 1e-2; the split carries ~22 bits.
__device__ __forceinline__ v4f mma2(const v8h& a, const v8h (&p)[2], v4f c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p[0], c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p[1], c, 0, 0, 0);
}

// p0, p1 ~= hi + lo as packed float16 pairs: hi = f16(p), lo = f16(p - hi) (the
// float32 difference is exact: hi is within 2^-11 of p), lo by v_fma_mix straight
// from the packed hi halves.  lo feeds an MFMA, which must not read a register
// sooner than two wait states after a VALU instruction writes it, and the
// compiler pads only around instructions it sees: the asm block therefore ends
// with s_nop 1 (without it the MFMA followed the last write after one wait state
// and could read the register's old high half).
__device__ __forceinline__ void split_f16x2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, v2h{(_Float16)p0, (_Float16)p1});
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "s_nop 1"
      : "=&v"(lo)
      : "v"(hi), "v"(p0), "v"(p1));
}

// p0, p1 ~= hi + lo as packed bf16 pairs: hi = bf16(p) (nearest even), lo =
// bf16(p - hi) (the float32 difference is exact: hi is within 2^-9 of p); 16
// significant bits of each probability.
__device__ __forceinline__ void split_bf16x2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
  const __bf16 l0 = (__bf16)(p0 - (float)h0), l1 = (__bf16)(p1 - (float)h1);
  hi = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  lo = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
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
// kShareAlpha: the cost, in steps, charged to each item when the steps of a call
// are divided between workgroups (the per-item share of a round's set-up,
// prologue latency, drain and merge; see share_plan).
template <int D> struct Fp4Pol {
  static constexpr int kShareAlpha = 12;
  static constexpr int kOcc = 2;        // waves per SIMD (256 registers each)
  static constexpr int kBuf = 2;        // K and V register buffers (steps of prefetch)
  // one KV head per item; a step is 4 pages; lane (r, j) holds the 16 slots of page j
  static constexpr int kNH = 1, kNP = 4, kTok = 16;
  __device__ static int lane_page(int j4) { return j4; }
  __device__ static int lane_slot0(int) { return 0; }
  static constexpr int kBlk = Fp4Block<D>::kBytes;
  static constexpr int kCode = Fp4Block<D>::kCodeBytes;
  static constexpr int kGroups = D / 32;
  static constexpr int kCPL = D / 32;             // channel pairs per lane
  static constexpr int kTiles = D / 16;
  struct KStep {
    uint4 kc[4];          // K codes, MFMA m: token slot 4m + (lane%16)%4, group lane/16
    uint32_t ks;          // K scale bytes of those 4 tokens (byte m)
  };
  struct VStep {
    uint4 vc[kCPL];       // V codes of channel pair kCPL*(lane%16) + q (row 16q + lane%16), slots 0..15
    uint4 vs;             // V scale bytes of that group, slots 0..15
  };
  struct QOp { v8i b; };
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4, int) {
    qo.b = load_q_fp8<D>(qrow, valid, j4);
  }
  __device__ static void load_k(KStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    load_k_page(st, pool, pick_id(ids, r16 >> 2), page_bytes, g, r16, j4);
  }
  // the same with the lane's page id (that of page (lane % 16) / 4 of the step)
  __device__ static void load_k_page(KStep& st, const uint8_t* pool, int pid, int64_t page_bytes, const PageGeo& g,
                                     int r16, int j4) {
    const uint8_t* kb = pool + (int64_t)pid * page_bytes + (int64_t)fp4_block_pos(g.head0, pid, g.H, g.mask) * kBlk;
    if (j4 < kGroups) {
#pragma unroll
      for (int m = 0; m < 4; ++m) st.kc[m] = load16_stream(kb + (4 * m + (r16 & 3)) * (D / 2) + 16 * j4);
      // scale bytes are stored [slot % 4][group][slot / 4]: one dword per lane
      st.ks = load4_stream(kb + kCode + 4 * ((r16 & 3) * kGroups + j4));
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) st.kc[m] = make_uint4(0, 0, 0, 0);
      st.ks = 0x7F7F7F7Fu;
    }
  }
  __device__ static void load_v(VStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const int pid = pick_id(ids, j4);
    const uint8_t* vb = pool + (int64_t)pid * page_bytes + (int64_t)fp4_block_pos(g.head0, pid, g.H, g.mask) * kBlk;
#pragma unroll
    for (int q = 0; q < kCPL; ++q) st.vc[q] = load16_stream(vb + (16 * q + r16) * kPage);   // pair kCPL*r16 + q
    st.vs = load16_stream(vb + kCode + kPage * ((kCPL * r16) / 16));
  }
  template <int M> __device__ static v4f qk1(const KStep& st, const QOp& qo) {
    const v8i a = v8i{(int)st.kc[M].x, (int)st.kc[M].y, (int)st.kc[M].z, (int)st.kc[M].w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qo.b, v4f{0, 0, 0, 0}, 4 /*A fp4*/, 0 /*B fp8*/,
                                                           M /*byte M of ks*/, (int)st.ks, 0, 127);
  }
  __device__ static void qk(const KStep& st, const QOp& qo, v4f (&S)[4]) {
    S[0] = qk1<0>(st, qo);
    S[1] = qk1<1>(st, qo);
    S[2] = qk1<2>(st, qo);
    S[3] = qk1<3>(st, qo);
  }
  // Clears the value codes of slots past nvalid and gives them scale byte 127
  // (2^0), so that whatever an unwritten slot holds converts to zero.
  __device__ static void mask_v(VStep& st, int nvalid) {
    const uint32_t k0 = slot_bytes_kept(nvalid, 0), k1 = slot_bytes_kept(nvalid, 4),
                   k2 = slot_bytes_kept(nvalid, 8), k3 = slot_bytes_kept(nvalid, 12);
#pragma unroll
    for (int q = 0; q < kCPL; ++q) {
      st.vc[q].x &= k0; st.vc[q].y &= k1; st.vc[q].z &= k2; st.vc[q].w &= k3;
    }
    st.vs.x = (st.vs.x & k0) | (~k0 & 0x7F7F7F7Fu);
    st.vs.y = (st.vs.y & k1) | (~k1 & 0x7F7F7F7Fu);
    st.vs.z = (st.vs.z & k2) | (~k2 & 0x7F7F7F7Fu);
    st.vs.w = (st.vs.w & k3) | (~k3 & 0x7F7F7F7Fu);
  }
  __device__ static void pv(const VStep& st, const v8h (&P)[2][2], v4f (&O)[kTiles], int) {
    const uint32_t s[4] = {st.vs.x, st.vs.y, st.vs.z, st.vs.w};
    // The conversion reads only the exponent field of its float scale, so byte k
    // of a scale word only has to be shifted into bits 23..30; the bits around it
    // land in the sign and mantissa and are ignored.
    float sc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int k = t & 3;
      sc[t] = __uint_as_float(k == 3 ? s[t >> 2] >> 1 : s[t >> 2] << (23 - 8 * k));
    }
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
          ev[i] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);   // low halves: even channel
          od[i] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);   // high halves: odd channel
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

// FP4 with two KV heads per item (GQA groups of up to 8 query heads, an even
// number of KV heads).  A step is 2 pages of both heads, the same bytes as a
// 4-page step of one head, and the 16 MFMA columns hold the query heads of both
// KV heads (head X in columns X*G .. X*G + G - 1) instead of 8 real columns and 8
// of padding: the softmax work per step halves, and the two heads' adjacent
// head-blocks (2 x 17*d/2 bytes, whole cache lines for d = 128) are fetched by
// the same wave at the same time.
//   QK: for each of the step's two token rows-of-16 (mm), head 0's product with
//       the query operand masked to head 0's columns plus head 1's masked to
//       head 1's, in one accumulator: 4 scaled MFMAs.  Token row i of MFMA mm is
//       page i >> 3, slot 8((i >> 2) & 1) + 4mm + (i & 3), so lane (h, j) of the
//       result holds slots 8(j & 1) .. 8(j & 1) + 7 of page j >> 1.
//   PV: per head and tile one f16 product pair over the step's 32 tokens, P
//       masked to that head's columns.
template <int D> struct Fp4PairPol {
  static constexpr int kShareAlpha = 12;
  static constexpr int kOcc = 2;
  static constexpr int kBuf = 2;
  static constexpr int kNH = 2, kNP = 2, kTok = 8;
  __device__ static int lane_page(int j4) { return j4 >> 1; }
  __device__ static int lane_slot0(int j4) { return 8 * (j4 & 1); }
  static constexpr int kBlk = Fp4Block<D>::kBytes;
  static constexpr int kCode = Fp4Block<D>::kCodeBytes;
  static constexpr int kGroups = D / 32;
  static constexpr int kCPL = D / 32;             // channel pairs per lane
  static constexpr int kTiles = D / 16;
  struct KStep {
    uint4 kc[4];          // MFMA 2X + mm: head X, token row lane%16, group lane/16
    uint32_t ks;          // byte 2X + mm: the scale of that row and group
  };
  struct VStep {
    uint2 vc[2][kCPL];    // head X, channel pair kCPL*(lane%16) + q: slots 8(j&1)..+7 of page j>>1
    uint2 vs[2];          // head X, scale bytes of that group, same slots
  };
  struct QOp { v8i b[2]; };   // the lane's query row if its column belongs to head X, else zero
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4, int lane_head) {
    const v8i q = load_q_fp8<D>(qrow, valid, j4);
    const v8i z = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    qo.b[0] = lane_head == 0 ? q : z;
    qo.b[1] = lane_head == 1 ? q : z;
  }
  __device__ static void load_k(KStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    // the pair's two blocks are adjacent (positions 2k, 2k + 1 of the page)
    const int pid = pick_id(ids, r16 >> 3);
    const uint8_t* pg = pool + (int64_t)pid * page_bytes + (int64_t)fp4_block_pos(g.head0, pid, g.H, g.mask) * kBlk;
    const int slot0 = 8 * ((r16 >> 2) & 1) + (r16 & 3);
    if (j4 < kGroups) {
      uint32_t d[2];
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        const uint8_t* kb = pg + X * kBlk;
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) st.kc[2 * X + mm] = load16_stream(kb + (slot0 + 4 * mm) * (D / 2) + 16 * j4);
        // scales are [slot % 4][group][slot / 4]; this lane needs slot / 4 = 2((r16 >> 2) & 1) + mm
        d[X] = load4_stream(kb + kCode + 4 * ((r16 & 3) * kGroups + j4));
      }
      st.ks = __builtin_amdgcn_perm(d[1], d[0], ((r16 >> 2) & 1) ? 0x07060302u : 0x05040100u);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) st.kc[m] = make_uint4(0, 0, 0, 0);
      st.ks = 0x7F7F7F7Fu;
    }
  }
  __device__ static void load_v(VStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const int pid = pick_id(ids, j4 >> 1);
    const uint8_t* pg = pool + (int64_t)pid * page_bytes + (int64_t)fp4_block_pos(g.head0, pid, g.H, g.mask) * kBlk +
                        8 * (j4 & 1);
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      const uint8_t* vb = pg + X * kBlk;
#pragma unroll
      for (int q = 0; q < kCPL; ++q) st.vc[X][q] = load8_stream(vb + (16 * q + r16) * kPage);
      st.vs[X] = load8_stream(vb + kCode + kPage * ((kCPL * r16) / 16));
    }
  }
  template <int M> __device__ static v4f qk1(const KStep& st, const v8i& b, v4f c) {
    const v8i a = v8i{(int)st.kc[M].x, (int)st.kc[M].y, (int)st.kc[M].z, (int)st.kc[M].w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4 /*A fp4*/, 0 /*B fp8*/, M, (int)st.ks, 0, 127);
  }
  __device__ static void qk(const KStep& st, const QOp& qo, v4f (&S)[2]) {
    S[0] = qk1<2>(st, qo.b[1], qk1<0>(st, qo.b[0], v4f{0, 0, 0, 0}));
    S[1] = qk1<3>(st, qo.b[1], qk1<1>(st, qo.b[0], v4f{0, 0, 0, 0}));
  }
  // Clears the value codes of slots past nvalid (of this lane's 8) and gives them
  // scale byte 127.
  __device__ static void mask_v(VStep& st, int nvalid) {
    const uint32_t k0 = slot_bytes_kept(nvalid, 0), k1 = slot_bytes_kept(nvalid, 4);
#pragma unroll
    for (int X = 0; X < 2; ++X) {
#pragma unroll
      for (int q = 0; q < kCPL; ++q) {
        st.vc[X][q].x &= k0;
        st.vc[X][q].y &= k1;
      }
      st.vs[X].x = (st.vs[X].x & k0) | (~k0 & 0x7F7F7F7Fu);
      st.vs[X].y = (st.vs[X].y & k1) | (~k1 & 0x7F7F7F7Fu);
    }
  }
  __device__ static void pv(const VStep& st, const v8h (&P)[1][2], v4f (&O)[kTiles], int lane_head) {
    const v8h z = v8h{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      const v8h PX[2] = {lane_head == X ? P[0][0] : z, lane_head == X ? P[0][1] : z};
      // the conversion reads only the exponent field of its float scale
      const uint32_t s2[2] = {st.vs[X].x, st.vs[X].y};
      float sc[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int k = t & 3;
        sc[t] = __uint_as_float(k == 3 ? s2[t >> 2] >> 1 : s2[t >> 2] << (23 - 8 * k));
      }
#pragma unroll
      for (int q = 0; q < kCPL; ++q) {
        const uint32_t c[2] = {st.vc[X][q].x, st.vc[X][q].y};
        uint32_t Xv[8];   // slot t: (channel 2cp, channel 2cp + 1) scaled by 2^(byte_t - 127)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          v2h h;
          switch (t & 3) {
            case 0: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 0); break;
            case 1: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 1); break;
            case 2: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 2); break;
            default: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[t >> 2], sc[t], 3); break;
          }
          Xv[t] = __builtin_bit_cast(uint32_t, h);
        }
        uint32_t ev[4], od[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ev[i] = __builtin_amdgcn_perm(Xv[2 * i + 1], Xv[2 * i], 0x05040100u);   // low halves: even channel
          od[i] = __builtin_amdgcn_perm(Xv[2 * i + 1], Xv[2 * i], 0x07060302u);   // high halves: odd channel
        }
        O[2 * q] = mma2(__builtin_bit_cast(v8h, make_uint4(ev[0], ev[1], ev[2], ev[3])), PX, O[2 * q]);
        O[2 * q + 1] = mma2(__builtin_bit_cast(v8h, make_uint4(od[0], od[1], od[2], od[3])), PX, O[2 * q + 1]);
      }
    }
  }
  __device__ static int channel(int tile, int j4, int v) { return 2 * (kCPL * (4 * j4 + v) + (tile >> 1)) + (tile & 1); }
};

// FP4 with the PV on the scaled FP4 x FP8 MFMA as well (UQ_FLAG_PV_SCALED; the
// pages' dequantization folded into the scaled matrix instruction, [review] §3.2
// and [commentary] footnote 2).  V's group scales run along head_dim while PV
// contracts over tokens, so they cannot be block scales of the FP4 operand:
// they are folded into the probabilities instead, which become the FP8 operand,
// P * 2^(E_t - M) rounded to E4M3 per 32-channel group and 32-token block with
// block scale 2^M, M = the block's largest V exponent - 8 (at least -127).
// One KV head per item; a step is 8 pages (128 tokens), the contraction length
// of one scaled MFMA, and its probabilities are taken against the step's own
// largest logit (so that the rounding does not depend on which wave visits
// which step), then merged into the running state with the step maximum.
//
// Operand layouts of the 16x16x128 scaled MFMA (contraction index k): an FP4
// operand lane (row, j) holds k = 32j .. 32j + 31; an FP8 operand lane (col, j)
// holds k = 16j .. 16j + 15 (bytes 0..15) and 64 + 16j .. 64 + 16j + 15 (bytes
// 16..31); the block scale of lane (., j) applies to k = 32j .. 32j + 31
// whichever lanes hold those elements.  Token of k: block J = k / 32 is pages
// 2J, 2J + 1 of the step; inside it k = 32J + 8i + 2u + e is slot 4i + u of
// page 2J + e.
//   PV, FP4 operand (V^T, rows = channels): lane (r, j) takes the 16-byte code
//     rows of channel pair 16g + r in pages 2j and 2j + 1; two bit-field merges
//     give the even and the odd channel's 32 codes in that k order.
//   PV, FP8 operand (P, columns = query rows): dword m of lane (r, j) holds
//     k = 64(m >> 2) + 16j + 4(m & 3) + v, v = 0..3, i.e. page
//     4(m >> 2) + 2(j >> 1) + (v & 1), slot 8(j & 1) + 2(m & 3) + (v >> 1).
//   QK: token row i of MFMA m is that token with j = i >> 2, v = i & 3, so that
//     lane (r, j) of the result holds exactly its FP8 dword m in S[m].
//   Block maxima: the lane sees half of each of its two blocks (8 slots of both
//     pages); lane l ^ 16 has the other half.  The lane's own block scale (block
//     j) is held as a fold exponent by lane (r, 2(j & 1)).
template <int D> struct Fp4SpvPol {
  static constexpr bool kSpv = true;
  static constexpr int kShareAlpha = 6;
  static constexpr int kOcc = 1;
  static constexpr int kBuf = 2;
  static constexpr int kNH = 1, kNP = 8, kTok = 32;
  static constexpr int kBlk = Fp4Block<D>::kBytes;
  static constexpr int kCode = Fp4Block<D>::kCodeBytes;
  static constexpr int kGroups = D / 32;
  static constexpr int kCPL = D / 32;
  static constexpr int kTiles = D / 16;
  struct KStep {
    uint4 kc[8];          // MFMA m: token row lane%16 (see above), group lane/16
    uint32_t ks[4];       // scale bytes: MFMA m uses byte (m & 3) >> 1 of ks[2(m >> 2) + (m & 1)]
  };
  struct VStep {
    uint4 xc[kGroups], yc[kGroups];   // code rows of channel pair 16g + lane%16, pages 2j, 2j + 1
    uint2 e[4][kGroups];              // scale bytes of group g, slots 8(j & 1) .. + 7 of the lane's
                                      // FP8 pages 2(j >> 1), + 1, + 4, + 5
  };
  struct QOp { v8i b; };
  // The page id of a lane-dependent index x < 8: selects between the
  // wave-uniform ids (taken through readfirstlane, so that the selects are not
  // turned into an indexed load from a stack copy of the array).
  __device__ static int pick8(const int (&ids)[8], int x) {
    int r = __builtin_amdgcn_readfirstlane(ids[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k) r = x == k ? __builtin_amdgcn_readfirstlane(ids[k]) : r;
    return r;
  }
  __device__ static const uint8_t* block(const uint8_t* pool, int pid, int64_t page_bytes, const PageGeo& g) {
    return pool + (int64_t)pid * page_bytes + (int64_t)fp4_block_pos(g.head0, pid, g.H, g.mask) * kBlk;
  }
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4, int) {
    qo.b = load_q_fp8<D>(qrow, valid, j4);
  }
  // K of token row r16 of MFMA m: page 4(m >> 2) + 2(r16 >> 3) + (r16 & 1), slot
  // 8((r16 >> 2) & 1) + 2(m & 3) + ((r16 >> 1) & 1).
  __device__ static void load_k(KStep& st, const uint8_t* pool, const int (&ids)[8], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const int pa = 2 * (r16 >> 3) + (r16 & 1);
    const uint8_t* kb[2] = {block(pool, pick8(ids, pa), page_bytes, g), block(pool, pick8(ids, pa + 4), page_bytes, g)};
    const int par = (r16 >> 1) & 1, half = (r16 >> 2) & 1;
    const int slot0 = 8 * half + par;
    if (j4 < kGroups) {
#pragma unroll
      for (int m = 0; m < 8; ++m) st.kc[m] = load16_stream(kb[m >> 2] + (slot0 + 2 * (m & 3)) * (D / 2) + 16 * j4);
      // scale bytes are stored [slot % 4][group][slot / 4]; slot 8 half + 2(m & 3)
      // + par has slot % 4 = 2(m & 1) + par and slot / 4 = 2 half + ((m & 3) >> 1)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        st.ks[2 * x] = load4_stream(kb[x] + kCode + 4 * (par * kGroups + j4)) >> (16 * half);
        st.ks[2 * x + 1] = load4_stream(kb[x] + kCode + 4 * ((2 + par) * kGroups + j4)) >> (16 * half);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) st.kc[m] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 4; ++x) st.ks[x] = 0x7F7F7F7Fu;
    }
  }
  __device__ static void load_v(VStep& st, const uint8_t* pool, const int (&ids)[8], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const uint8_t* xb = block(pool, pick8(ids, 2 * j4), page_bytes, g);
    const uint8_t* yb = block(pool, pick8(ids, 2 * j4 + 1), page_bytes, g);
#pragma unroll
    for (int gg = 0; gg < kGroups; ++gg) {
      const int p = 16 * gg + r16;                              // channel pair
      const int row = 16 * (p % kCPL) + p / kCPL;               // its 16-byte code row
      st.xc[gg] = load16_stream(xb + row * kPage);
      st.yc[gg] = load16_stream(yb + row * kPage);
    }
    const int pe = 2 * (j4 >> 1), w = 8 * (j4 & 1);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint8_t* eb = block(pool, pick8(ids, pe + (x & 1) + 4 * (x >> 1)), page_bytes, g) + kCode + w;
#pragma unroll
      for (int gg = 0; gg < kGroups; ++gg) st.e[x][gg] = load8_stream(eb + kPage * gg);
    }
  }
  template <int M> __device__ static v4f qk1(const KStep& st, const QOp& qo) {
    const v8i a = v8i{(int)st.kc[M].x, (int)st.kc[M].y, (int)st.kc[M].z, (int)st.kc[M].w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qo.b, v4f{0, 0, 0, 0}, 4 /*A fp4*/, 0 /*B fp8*/,
                                                           (M & 3) >> 1, (int)st.ks[2 * (M >> 2) + (M & 1)], 0, 127);
  }
  __device__ static void qk(const KStep& st, const QOp& qo, v4f (&S)[8]) {
    S[0] = qk1<0>(st, qo);
    S[1] = qk1<1>(st, qo);
    S[2] = qk1<2>(st, qo);
    S[3] = qk1<3>(st, qo);
    S[4] = qk1<4>(st, qo);
    S[5] = qk1<5>(st, qo);
    S[6] = qk1<6>(st, qo);
    S[7] = qk1<7>(st, qo);
  }
  // Largest bytes of two pairs of words, one per 16-bit half of the result
  // (packed u16 maxima: the high byte of a half decides the unsigned 16-bit
  // order, so the maxima of the words and of the words shifted left by 8 carry
  // the largest odd and even bytes).
  __device__ static uint32_t umax16(uint32_t x, uint32_t y) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, x), __builtin_bit_cast(us2, y)));
  }
  __device__ static uint32_t max_byte4(uint2 a, uint2 b) {
    const uint32_t t = umax16(umax16(umax16(a.x, a.y), umax16(b.x, b.y)),
                              umax16(umax16(a.x << 8, a.y << 8), umax16(b.x << 8, b.y << 8)));
    return max(t >> 24, (t >> 8) & 0xFFu);
  }
  // Step PV: Z[tile] = the FP8 operand (folded P) times the V codes.  pf[4m + v]
  // is the probability of S[m][v]'s token (0 past the item); nv[x]: valid slots
  // of the lane's FP8 page x (2(j >> 1), + 1, + 4, + 5) inside its 8-slot window.
  __device__ static void pv(VStep& st, const float (&pf)[32], const int (&nv)[4], v4f (&Z)[kTiles], int lane) {
    const int j4 = lane >> 4, r16 = lane & 15;
    // exponents of slots past the item do not enter the block maxima
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint32_t k0 = slot_bytes_kept(nv[x], 0), k1 = slot_bytes_kept(nv[x], 4);
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        st.e[x][g].x &= k0;
        st.e[x][g].y &= k1;
      }
    }
    // block maxima: half 0 (pages 2(j >> 1), + 1: block j >> 1) in the low 16
    // bits, half 1 (block 2 + (j >> 1)) in the high 16 bits; completed with lane
    // l ^ 16, which holds the blocks' other 8 slots
    uint32_t bm[kGroups], sc[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      uint32_t mm = max_byte4(st.e[0][g], st.e[1][g]) | (max_byte4(st.e[2][g], st.e[3][g]) << 16);
      mm = umax16(mm, (uint32_t)__shfl_xor((int)mm, 16));
      // block scale bytes M + 127 = max(largest byte - 8, 0), per half
      bm[g] = umax16(mm, 0x00080008u) - 0x00080008u;
    }
    // the lane's own block scale (block j): half j >> 1 of lane (r, 2(j & 1))
    const int src = 32 * (j4 & 1) + r16;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const uint32_t o = (uint32_t)__shfl((int)bm[g], src);
      sc[g] = (j4 >> 1) ? o >> 16 : o & 0xFFFFu;
    }
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const int bma = (int)(bm[g] & 0xFFFFu), bmb = (int)(bm[g] >> 16);
      uint32_t bw[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        // S[m][v]: FP8 page 2(m >> 2) + (v & 1) of the lane, window slot
        // 2(m & 3) + (v >> 1): byte 2(m & 1) + (v >> 1) of word (m & 3) >> 1
        const int bmx = (m >> 2) ? bmb : bma;
        const uint2 e0 = st.e[2 * (m >> 2)][g], e1 = st.e[2 * (m >> 2) + 1][g];
        const uint32_t w0 = ((m & 3) >> 1) ? e0.y : e0.x, w1 = ((m & 3) >> 1) ? e1.y : e1.x;
        const int sh0 = 16 * (m & 1), sh1 = sh0 + 8;
        const float f0 = __builtin_amdgcn_ldexpf(pf[4 * m + 0], (int)((w0 >> sh0) & 0xFFu) - bmx);
        const float f1 = __builtin_amdgcn_ldexpf(pf[4 * m + 1], (int)((w1 >> sh0) & 0xFFu) - bmx);
        const float f2 = __builtin_amdgcn_ldexpf(pf[4 * m + 2], (int)((w0 >> sh1) & 0xFFu) - bmx);
        const float f3 = __builtin_amdgcn_ldexpf(pf[4 * m + 3], (int)((w1 >> sh1) & 0xFFu) - bmx);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
        bw[m] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, lo, true);
      }
      const v8i b = v8i{(int)bw[0], (int)bw[1], (int)bw[2], (int)bw[3], (int)bw[4], (int)bw[5], (int)bw[6], (int)bw[7]};
      const uint32_t xc[4] = {st.xc[g].x, st.xc[g].y, st.xc[g].z, st.xc[g].w};
      const uint32_t yc[4] = {st.yc[g].x, st.yc[g].y, st.yc[g].z, st.yc[g].w};
      uint32_t ev[4], od[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ev[i] = (xc[i] & 0x0F0F0F0Fu) | ((yc[i] << 4) & 0xF0F0F0F0u);   // even channel: X, Y slot pairs
        od[i] = ((xc[i] >> 4) & 0x0F0F0F0Fu) | (yc[i] & 0xF0F0F0F0u);   // odd channel
      }
      const v8i ae = v8i{(int)ev[0], (int)ev[1], (int)ev[2], (int)ev[3], 0, 0, 0, 0};
      const v8i ao = v8i{(int)od[0], (int)od[1], (int)od[2], (int)od[3], 0, 0, 0, 0};
      Z[2 * g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ae, b, Z[2 * g], 4 /*A fp4*/, 0 /*B fp8*/, 0, 127,
                                                                  0, (int)sc[g]);
      Z[2 * g + 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ao, b, Z[2 * g + 1], 4, 0, 0, 127, 0,
                                                                      (int)sc[g]);
    }
  }
  // Tile 2g + par, row 4j + v: channel pair 16g + 4j + v, channel 2 * pair + par.
  __device__ static int channel(int tile, int j4, int v) { return 2 * (16 * (tile >> 1) + 4 * j4 + v) + (tile & 1); }
};

// FP8 baseline.  QK runs on f16 MFMAs after an exact E4M3 -> f16 conversion:
// the FP8 x FP8 MFMAs (16x16x128 scaled and 16x16x32) drop low-order bits of
// small products when large ones are present in the same instruction, which
// with unrotated outlier channels moves logits by ~1e-4 relative.
template <int D> struct Fp8Pol {
  static constexpr int kShareAlpha = 6;
  static constexpr int kOcc = 1;
  static constexpr int kBuf = 3;
  // one KV head per item; a step is 4 pages; lane (r, j) holds the 16 slots of page j
  static constexpr int kNH = 1, kNP = 4, kTok = 16;
  __device__ static int lane_page(int j4) { return j4; }
  __device__ static int lane_slot0(int) { return 0; }
  static constexpr int kBlk = kPage * D;
  static constexpr int kTiles = D / 16;
  static constexpr int kLanesK = D / 32;   // lane groups holding 32 channels of a row
  struct KStep { uint4 k[4][2]; };     // K bytes 32j..32j+31 of token slot 4m + (lane%16)%4
  struct VStep { uint4 vc[kTiles]; };  // V bytes of channel 16t + lane%16, slots 0..15
  // q as f16 B operands: MFMA kk pairs k-block j with channels 32j + 8kk..+7
  struct QOp { v8h b[4]; };
  __device__ static v8h cvt8(uint32_t w0, uint32_t w1) {
    const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4, int) {
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
  __device__ static void load_k(KStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const int pid = pick_id(ids, r16 >> 2);
    const uint8_t* pg = pool + (int64_t)pid * page_bytes;
    const uint32_t rot = fp8_rot(pid, g.units, g.umask), pb = (uint32_t)page_bytes, hb = (uint32_t)(g.head0 * kBlk);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int slot = 4 * m + (r16 & 3);
      if (j4 < kLanesK) {
        st.k[m][0] = load16_stream(pg + fp8_wrap(hb + slot * D + 32 * j4, rot, pb));
        st.k[m][1] = load16_stream(pg + fp8_wrap(hb + slot * D + 32 * j4 + 16, rot, pb));
      } else {
        st.k[m][0] = st.k[m][1] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ static void load_v(VStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const int pid = pick_id(ids, j4);
    const uint8_t* pg = pool + (int64_t)pid * page_bytes;
    const uint32_t rot = fp8_rot(pid, g.units, g.umask), pb = (uint32_t)page_bytes, hb = (uint32_t)(g.head0 * kBlk);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) st.vc[t] = load16_stream(pg + fp8_wrap(hb + (16 * t + r16) * kPage, rot, pb));
  }
  __device__ static void qk(const KStep& st, const QOp& qo, v4f (&S)[4]) {
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
  // Clears the value bytes of slots past nvalid.
  __device__ static void mask_v(VStep& st, int nvalid) {
    const uint32_t k0 = slot_bytes_kept(nvalid, 0), k1 = slot_bytes_kept(nvalid, 4),
                   k2 = slot_bytes_kept(nvalid, 8), k3 = slot_bytes_kept(nvalid, 12);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      st.vc[t].x &= k0; st.vc[t].y &= k1; st.vc[t].z &= k2; st.vc[t].w &= k3;
    }
  }
  __device__ static void pv(const VStep& st, const v8h (&P)[2][2], v4f (&O)[kTiles], int) {
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
          a[i] = __builtin_bit_cast(uint32_t, h);
        }
        O[t] = mma2(__builtin_bit_cast(v8h, make_uint4(a[0], a[1], a[2], a[3])), P[half], O[t]);
      }
    }
  }
  __device__ static int channel(int tile, int j4, int v) { return 16 * tile + 4 * j4 + v; }
};

// BF16 baseline: K, q and V enter bf16 MFMAs as stored (every bf16 value exact),
// P as bf16 hi + lo.
template <int D> struct Bf16Pol {
  static constexpr bool kPBf16 = true;  // the PV takes P as bf16 hi + lo
  static constexpr int kShareAlpha = 3;
  static constexpr int kOcc = 1;
  static constexpr int kBuf = 2;
  // one KV head per item; a step is 4 pages; lane (r, j) holds the 16 slots of page j
  static constexpr int kNH = 1, kNP = 4, kTok = 16;
  __device__ static int lane_page(int j4) { return j4; }
  __device__ static int lane_slot0(int) { return 0; }
  static constexpr int kBlk = kPage * D * 2;
  static constexpr int kTiles = D / 16;
  static constexpr int kK = D / 32;     // 16x16x32 MFMAs per token row
  // Page loads are ordinary here: with the wider rows of this format nontemporal
  // loads measured ~2% slower (the FP4 and FP8 policies gain 7-11% from them).
  struct KStep { uint4 k[4][kK]; };      // K bf16 channels 32kk + 8j..+7 of token slot 4m + (lane%16)%4
  struct VStep { uint4 v[kTiles][2]; };  // V bf16 of channel 16t + lane%16, slots 0..7 and 8..15
  // q as bf16 B operands: MFMA kk, lane (h, j) holds channels 32kk + 8j..+7 of head h
  struct QOp { v8bf b[kK]; };
  __device__ static void load_q(QOp& qo, const uint8_t* qrow, bool valid, int j4, int) {
#pragma unroll
    for (int kk = 0; kk < kK; ++kk)
      qo.b[kk] = __builtin_bit_cast(v8bf, valid ? load16(qrow + 2 * (32 * kk + 8 * j4)) : make_uint4(0, 0, 0, 0));
  }
  __device__ static void load_k(KStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const uint8_t* kb = pool + (int64_t)pick_id(ids, r16 >> 2) * page_bytes + (int64_t)g.head0 * kBlk;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int slot = 4 * m + (r16 & 3);
#pragma unroll
      for (int kk = 0; kk < kK; ++kk) st.k[m][kk] = load16(kb + 2 * (slot * D + 32 * kk + 8 * j4));
    }
  }
  __device__ static void load_v(VStep& st, const uint8_t* pool, const int (&ids)[4], int64_t page_bytes,
                                const PageGeo& g, int r16, int j4) {
    const uint8_t* vb = pool + (int64_t)pick_id(ids, j4) * page_bytes + (int64_t)g.head0 * kBlk;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      st.v[t][0] = load16(vb + 2 * ((16 * t + r16) * kPage));
      st.v[t][1] = load16(vb + 2 * ((16 * t + r16) * kPage + 8));
    }
  }
  __device__ static void qk(const KStep& st, const QOp& qo, v4f (&S)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v4f acc = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < kK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, st.k[m][kk]), qo.b[kk], acc, 0, 0, 0);
      S[m] = acc;
    }
  }
  // Clears the values of slots past nvalid.
  __device__ static void mask_v(VStep& st, int nvalid) {
    uint32_t k[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) k[i] = slot_halves_kept(nvalid, 2 * i);
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        st.v[t][half].x &= k[4 * half]; st.v[t][half].y &= k[4 * half + 1];
        st.v[t][half].z &= k[4 * half + 2]; st.v[t][half].w &= k[4 * half + 3];
      }
  }
  __device__ static void pv(const VStep& st, const v8bf (&P)[2][2], v4f (&O)[kTiles], int) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const v8bf a = __builtin_bit_cast(v8bf, st.v[t][half]);
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, P[half][0], O[t], 0, 0, 0);
        O[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, P[half][1], O[t], 0, 0, 0);
      }
    }
  }
  __device__ static int channel(int tile, int j4, int v) { return 16 * tile + 4 * j4 + v; }
};

// Policies with the scaled-MFMA PV declare kSpv; those whose PV takes P as
// bf16 hi + lo (instead of f16 hi + lo) declare kPBf16.
template <class P, class = void> struct SpvOf : std::false_type {};
template <class P> struct SpvOf<P, std::void_t<decltype(P::kSpv)>> : std::bool_constant<P::kSpv> {};
template <class P, class = void> struct PBf16Of : std::false_type {};
template <class P> struct PBf16Of<P, std::void_t<decltype(P::kPBf16)>> : std::bool_constant<P::kPBf16> {};

// ------------------------------------------------------------------ plan
// The work of a call is the list of steps (4 pages) of all (sequence b, KV head
// hk) items, items in the order b * Hkv + hk.  Every workgroup derives in LDS
// sbase[b] = first step of item (b, 0), each item of sequence b having
// steps(b) = ceil(pages(b) / NP) steps (NP = 4, or 2 for KV-head pairs), and
// sbase[B] = T, the total.  Workgroup w
// then takes steps [w T / grid, (w + 1) T / grid): equal shares whatever the
// mix of lengths, items cut at share boundaries being merged across workgroups.
// Inclusive sum over the 64 lanes: Hillis-Steele inside each 16-lane row
// (DPP row shifts, lanes past the row start adding 0), then the row totals
// broadcast into the later rows (row_bcast:15 into rows 1 and 3, row_bcast:31
// into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

// floor(n / d) for 0 <= n < 2^31, d >= 1 and a quotient below 2^20, from rd =
// the hardware reciprocal of d (1 ulp): the float estimate is then within 0.2
// of n / d, so its truncation is off by at most one, fixed in exact integer
// arithmetic (q * d <= n + d < 2^32).
__device__ __forceinline__ int div_q20(int n, int d, float rd) {
  uint32_t q = (uint32_t)((float)n * rd);
  const int r = (int)((uint32_t)n - q * (uint32_t)d);
  q += r >= d ? 1u : 0u;
  q -= r < 0 ? 1u : 0u;
  return (int)q;
}

// Sequence length as used: clamped to [0, max_pages * 16] so that a length
// beyond its page-table row can never index past the row.
__device__ __forceinline__ int clamp_len(int L, int max_pages) {
  return L < 0 ? 0 : (L > max_pages * kPage ? max_pages * kPage : L);
}
template <int NP> __device__ __forceinline__ int seq_steps(int L) { return ((L + kPage - 1) / kPage + NP - 1) / NP; }

// Run by all 64 * NW threads; red: 2 NW ints of scratch.  Steps are NP pages;
// each sequence has Hi items (KV heads, or KV-head pairs).  Returns, in every
// thread, bit 0 set when the sequences' step counts differ, bit 1 when one of
// them has none and bit 2 when a length lies outside [0, 16 max_pages] (it is
// used clamped to that range).
template <int NW, int NP>
__device__ int wg_plan(const int32_t* __restrict__ seq_lens, int B, int Hi, int max_pages, int32_t* sbase,
                       int32_t* lens, int32_t* red) {
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = B > 0 ? seq_steps<NP>(clamp_len(seq_lens[0], max_pages)) : 0;
  int32_t carry = 0;
  int bits = 0;
  for (int b0 = 0; b0 < B; b0 += NT) {
    const int b = b0 + tid;
    const int raw = b < B ? seq_lens[b] : 0;
    const int L = clamp_len(raw, max_pages);
    if (b < B) lens[b] = L;
    const int s = seq_steps<NP>(L);
    const int ns = b < B ? s * Hi : 0;
    const int incl = wave_incl_scan(ns);
    const int wbits = (__any(b < B && s != s0) ? 1 : 0) | (__any(b < B && s == 0) ? 2 : 0) |
                      (__any(raw != L) ? 4 : 0);
    if (lane == 63) {
      red[wave] = incl;
      red[NW + wave] = wbits;
    }
    __syncthreads();
    int woff = 0, chunk = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      woff += w < wave ? red[w] : 0;
      chunk += red[w];
      bits |= red[NW + w];
    }
    if (b < B) sbase[b] = carry + woff + incl - ns;
    carry += chunk;
    __syncthreads();                               // red is rewritten by the next chunk
  }
  if (tid == 0) sbase[B] = carry;
  __syncthreads();
  return bits;
}

// Cost-balanced share boundaries sb[0 .. grid] (run by all 64 * NW threads;
// one barrier): workgroup w takes steps [sb[w], sb[w + 1]).  Each item is
// charged its steps plus `alpha` > 0, and the cost line is cut into grid equal
// parts, so that a share spanning many short items (several rounds, each with
// its own set-up, prologue latency, drain and merge) gets fewer steps.  Item
// f = b Hi + hk costs alpha and then its steps, so cost c maps to step
// base[b] + hk steps(b) + clamp(c - start of f - alpha, 0, steps(b)).  The
// caller keeps alpha <= (T / grid) / 2 and gives every sequence a step, so
// consecutive cuts lie more than alpha apart in cost and no share is empty.
template <int NW, int NP>
__device__ void share_plan(const int32_t* base, const int32_t* lens, int B, int Hi, int T, int grid, int alpha,
                           int32_t* sb) {
  constexpr int NT = 64 * NW;
  const int64_t C = (int64_t)T + (int64_t)alpha * B * Hi;   // < 2^53
  for (int w = threadIdx.x; w <= grid; w += NT) {
    int g = T;
    if (w < grid) {
      // t = floor(w C / grid); w C < 2^53 is exact in float64, and a quotient
      // that is not an integer is at least 1/grid from one, so the floor of the
      // rounded quotient is exact
      const int64_t t = (int64_t)floor((double)((int64_t)w * C) / (double)grid);
      // the last sequence b with cbase(b) = base[b] + alpha Hi b <= t
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)base[mid] + (int64_t)alpha * Hi * mid <= t) lo = mid;
        else hi = mid - 1;
      }
      const int sq = seq_steps<NP>(lens[lo]), per = sq + alpha;
      const uint32_t r = (uint32_t)(t - ((int64_t)base[lo] + (int64_t)alpha * Hi * lo));   // < Hi per < 2^32
      int hk = (int)(r / (uint32_t)per);
      hk = hk < Hi - 1 ? hk : Hi - 1;
      int64_t o = (int64_t)r - (int64_t)hk * per - alpha;
      o = o < 0 ? 0 : (o > sq ? sq : o);
      g = base[lo] + hk * sq + (int)o;
    }
    sb[w] = g;
  }
  __syncthreads();
}

// Query rows into LDS: E4M3 bytes of the (FP4: rotated) rows; BF16 keeps the
// bf16 values.  Each row is handled by 16 consecutive threads, part p holding
// channels E*p .. E*p + E - 1 (E = D/16).  load() only issues the global loads,
// so that they go out ahead of the first key/value loads (the vector-memory
// counter retires in order); finish() rotates, rounds and stores.  The
// normalized WHT is the Sylvester butterfly: stages h < E inside the thread,
// stages h >= E between parts p and p ^ (h/E), taken in float64 where every sum
// of bf16/f32 inputs is exact, so the E4M3 rounding sees the exact rotated value.
template <int D, int IN, int FMT> struct QueryRows {
  static constexpr int E = D / 16;
  static constexpr int kBytes = E * (IN == UQ_IN_BF16 ? 2 : 4);   // 8, 16 or 32
  uint4 w[2];

  // Channels E*p .. E*p + E - 1 of query row qrow (zeros when !valid).
  __device__ void load(const void* q, int64_t qrow, bool valid, int p) {
    w[0] = w[1] = make_uint4(0, 0, 0, 0);
    if (valid) {
      const uint8_t* src = static_cast<const uint8_t*>(q) + (qrow * D + E * p) * (IN == UQ_IN_BF16 ? 2 : 4);
      if constexpr (kBytes == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        w[0] = make_uint4(v.x, v.y, 0, 0);
      } else {
        w[0] = load16(src);
        if constexpr (kBytes == 32) w[1] = load16(src + 16);
      }
    }
  }

  template <int M> __device__ static void cross(double (&x)[E], int p) {
    const double sgn = (p & M) ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = __builtin_fma(x[e], sgn, lane_xor16<M>(x[e], p));
  }

  // Converts and stores the part into the LDS row dst (the 16 threads of a row
  // must call it together); FP4 rotates by c_d H, or with RV by
  // R = c_d H diag(s) with rot's signs.
  template <bool RV>
  __device__ __forceinline__ void finish(uint8_t* dst_row, int p, const Rot& rot) const {
    if constexpr (FMT == UQ_KV_BF16) {
      uint8_t* dst = dst_row + 2 * E * p;
      if constexpr (kBytes == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0].x, w[0].y);
      else *reinterpret_cast<uint4*>(dst) = w[0];
    } else {
      const uint32_t u[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
      double x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (IN == UQ_IN_BF16) x[e] = bf16_bits_to_f64((u[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        else x[e] = (double)__uint_as_float(u[e]);
      }
      if constexpr (FMT == UQ_KV_FP4) {
        if (RV && has_signs(rot)) {
#pragma unroll
          for (int e = 0; e < E; ++e) x[e] = flip_sign(x[e], sign_mask(rot, E * p + e));
        }
#pragma unroll
        for (int h = 1; h < E; h <<= 1)
#pragma unroll
          for (int i = 0; i < E; i += 2 * h)
#pragma unroll
            for (int j = i; j < i + h; ++j) {
              const double a0 = x[j], a1 = x[j + h];
              x[j] = a0 + a1;
              x[j + h] = a0 - a1;
            }
        // partner thread t ^ m holds the other half (the row's 16 threads are a
        // 16-lane row of the wave)
        cross<1>(x, p);
        cross<2>(x, p);
        cross<4>(x, p);
        cross<8>(x, p);
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = __builtin_fma(x[e], wht_c<D>(), 0.0);   // + 0: an exact zero is +0
      }
      uint32_t b[E / 4];
#pragma unroll
      for (int i = 0; i < E / 4; ++i) b[i] = e4m3x4_f64(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
      uint8_t* dst = dst_row + E * p;
      if constexpr (E == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(b[0], b[1]);
      else *reinterpret_cast<uint32_t*>(dst) = b[0];
    }
  }
};

// Normalizes one merged output row held as channels lane + 64k and, for FP4,
// rotates it back through R^T = diag(s) c_d H (the normalized WHT with stage
// h = 64 inside the lane and the others across lanes, then the cache's signs),
// then stores it.
template <int D, bool UNROT, bool RV>
__device__ __forceinline__ void store_row(float (&o)[D / 64], float l, float* dst, int lane, const Rot& rot) {
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
    if (RV && has_signs(rot)) {                 // channel lane + 64 k: bit lane % 32 of word 2 k + lane / 32
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const uint32_t w = (lane & 32) ? rot.s[2 * k + 1] : rot.s[2 * k];
        o[k] = flip_sign(o[k], ((w >> (lane & 31)) & 1u) << 31);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) dst[lane + 64 * k] = o[k];
}

// Value held by lane ^ M within each 32-lane half of the wave (M = 1 .. 16):
// DPP quad permutations for 1 and 2, row shifts for 4, a row rotation for 8,
// a swizzle for 16 -- none goes through the LDS crossbar's address path.
template <int M> __device__ __forceinline__ float xor32(float v, int lane) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
  else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
  else if constexpr (M == 4) {
    const int up = __builtin_amdgcn_mov_dpp(x, 0x104, 0xF, 0xF, true);   // row_shl:4, lane i <- i + 4
    const int dn = __builtin_amdgcn_mov_dpp(x, 0x114, 0xF, 0xF, true);   // row_shr:4, lane i <- i - 4
    return __int_as_float((lane & 4) ? dn : up);
  } else if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true));   // row_ror:8
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x401F));    // and 31, xor 16
}

// As store_row for a row held by one 32-lane half of the wave, channel
// (lane % 32) + 32 c in o[c]: the butterfly stages 32 and 64 run inside the
// lane, stages 1 .. 16 across lanes of the half.
template <int D, bool UNROT, bool RV>
__device__ __forceinline__ void store_row32(float (&o)[D / 32], float l, float* dst, bool live, int lane,
                                            const Rot& rot) {
  constexpr int PC = D / 32;
  const float inv = l > 0.f ? 1.f / l : 0.f;      // l == 0 only for empty sequences
#pragma unroll
  for (int c = 0; c < PC; ++c) o[c] *= inv;
  if constexpr (UNROT) {
#pragma unroll
    for (int h = 1; h < PC; h <<= 1)
#pragma unroll
      for (int c = 0; c < PC; ++c)
        if (!(c & h)) {
          const float x0 = o[c], x1 = o[c + h];
          o[c] = x0 + x1;
          o[c + h] = x0 - x1;
        }
    auto stage = [&](auto mtag) {
      constexpr int M = decltype(mtag)::value;
#pragma unroll
      for (int c = 0; c < PC; ++c) {
        const float other = xor32<M>(o[c], lane);
        o[c] = (lane & M) ? other - o[c] : o[c] + other;
      }
    };
    stage(std::integral_constant<int, 16>{});
    stage(std::integral_constant<int, 8>{});
    stage(std::integral_constant<int, 4>{});
    stage(std::integral_constant<int, 2>{});
    stage(std::integral_constant<int, 1>{});
#pragma unroll
    for (int c = 0; c < PC; ++c) o[c] *= wht_cf<D>();
    if (RV && has_signs(rot)) {                 // channel (lane % 32) + 32 c: bit lane % 32 of word c
#pragma unroll
      for (int c = 0; c < PC; ++c) o[c] = flip_sign(o[c], ((rot.s[c] >> (lane & 31)) & 1u) << 31);
    }
  }
  if (live) {
#pragma unroll
    for (int c = 0; c < PC; ++c) dst[(lane & 31) + 32 * c] = o[c];
  }
}

// Quantizes and stores a row of the fused step's newest token.
template <bool RV, class Row>
__device__ __forceinline__ void write_new(Row& row, uint8_t* blk, int off, bool live, bool is_v, int p,
                                          bool constopt, const Rot& rot) {
  row.template quantize<RV>(p, constopt, rot, is_v);
  if (live) {
    if (is_v) row.store_v(blk, off, p);
    else row.store_k(blk, off, p);
  }
}

// ------------------------------------------------------------------ decode
struct KArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t page_bytes;
  int32_t max_pages;
  const void* q;             // caller's query [B][Hq][D], bf16 or f32
  int32_t B, Hq, Hkv, G;
  int32_t hmask;             // Hkv - 1 when Hkv is a power of two, else -1
  int32_t units, umask;      // FP8: page_bytes / 256, units - 1 when a power of two, else -1
  float scale_log2;          // sm_scale * log2(e)
  float* out;                // [B][Hq][D]
  float* ml;                 // [2 * grid][16][2] partial (m in log2 units, l) of cut items
  float* po;                 // [2 * grid][16][D] partial O of cut items
  int32_t* cnt;              // [B][Hkv] arrival counters, zero between calls
  uint32_t* err;             // UQ_FLAG_CHECK: error word (UQ_CHECK_* bits OR-ed in), else null
  int32_t num_pages;         // pages in each pool (checked page ids lie in [0, num_pages))
  int32_t R;                 // items per round of a workgroup
  const void* k_new;         // fused step (FP4): the newest token's K and V, [B][Hkv][D]
  const void* v_new;         // in the query's dtype; null: attention only
  int32_t constopt;          // fused step: constOpt group scales for the written token
  Rot rot;                   // FP4: the cache's rotation variant
  unsigned long long* clocks;  // instrumentation: [min start, max end] wall clock, or null
};

// Split partials cross workgroups that may sit on different compute dies,
// whose L2 caches are not coherent with each other.  Rather than ordinary
// accesses bracketed by device-scope fences (each of which writes back and
// invalidates the whole L2 of the die, stalling every wave on it), the partials
// are written and read with relaxed device-scope atomic accesses, which write
// through and re-fetch past the L2 by themselves.  The one ordering needed,
// that all partial stores of a workgroup are complete before its arrival is
// counted, comes from waiting on the vector-memory counter before the barrier.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// LDS carve-up (bytes) of one workgroup of NW waves working on rounds of up to R
// items, each with G query heads:
//   qs     [R][G][D]       query rows (E4M3 bytes; BF16: bf16)
//   so     [R][NW][16][D]  per-wave partial O of each item (float), 16 >= G
//                          rows per slot so that slot offsets are constants
//   sm, sl [R][NW][16]     per-wave partial m (log2 units) and l (float)
//   rec    [R][8]          item records (int)
//   misc   [32]            step counter, per-item flags, plan scratch (int)
//   base   [B + 1]         plan (int)
//   lens   [B]             sequence lengths as used (int)
//   sb     [kMaxGrid + 1]  share boundaries (int)
constexpr int kSR = 16;   // rows of a wave slot in LDS (the 16 MFMA columns; an item has G <= 16)
struct Lds {
  int qs, so, sm, sl, rec, misc, base, lens, sb, total;
  __host__ __device__ static int up16(int x) { return (x + 15) & ~15; }
  __host__ __device__ Lds(int R, int NW, int G, int D, int esz, int B) {
    qs = 0;
    so = up16(qs + R * G * D * esz);
    sm = up16(so + R * NW * kSR * D * 4);
    sl = up16(sm + R * NW * kSR * 4);
    rec = up16(sl + R * NW * kSR * 4);
    misc = up16(rec + R * 8 * 4);
    base = up16(misc + 32 * 4);
    lens = up16(base + (B + 1) * 4);
    sb = up16(lens + B * 4);
    total = up16(sb + (kMaxGrid + 1) * 4);
  }
};

// Item record fields.
enum { kRecB = 0, kRecPBegin, kRecNpg, kRecHk, kRecLRel, kRecNStep, kRecSlot, kRecNContrib };

// One persistent workgroup per compute unit, NW = 4 * kOcc waves (so two waves
// share a SIMD when kOcc = 2), each taking an equal share of the steps of the
// call (see wg_plan).  A share is walked in rounds of up to R segments (the part
// of one item inside the share): the steps of a round form one list from which
// the waves claim steps one at a time through an LDS counter.  Waves that share
// a SIMD therefore end within a step of each other whatever the issue
// arbitration between them, and the prefetch runs on across segment boundaries.
// A wave keeps one running softmax state and parks it in its LDS slot for the
// segment when its next step belongs to another segment; at the end of the
// round the slots of each segment are merged.  A segment that is a whole item
// writes its output rows; otherwise the workgroup writes a partial (slot 2w for
// the first segment of its share, 2w + 1 for the last) and the last of the
// item's workgroups to arrive (device-scope counter) merges the partials.
template <class Pol, int D, int IN, int FMT, bool UNROT, bool RV>
__global__ __launch_bounds__(256 * Pol::kOcc, 1) void decode_kernel(const KArgs a,
                                                                   const int32_t* __restrict__ page_table,
                                                                   const int32_t* __restrict__ seq_lens) {
  constexpr int NW = 4 * Pol::kOcc;
  constexpr int NT = 64 * NW;
  constexpr int ESZ = FMT == UQ_KV_BF16 ? 2 : 1;
  constexpr int N = Pol::kBuf;
  constexpr int PER = D / 64;
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int NP = Pol::kNP, TOK = Pol::kTok;
  const int G = a.G * Pol::kNH;      // query rows (MFMA columns) of an item
  const int Hi = a.Hkv / Pol::kNH;   // items per sequence
  const Lds lay(a.R, NW, G, D, ESZ, a.B);
  uint8_t* qs = smem + lay.qs;
  float* so = reinterpret_cast<float*>(smem + lay.so);
  float* smx = reinterpret_cast<float*>(smem + lay.sm);
  float* slx = reinterpret_cast<float*>(smem + lay.sl);
  int32_t* rec = reinterpret_cast<int32_t*>(smem + lay.rec);
  int32_t* misc = reinterpret_cast<int32_t*>(smem + lay.misc);
  int32_t* base = reinterpret_cast<int32_t*>(smem + lay.base);
  int32_t* lens = reinterpret_cast<int32_t*>(smem + lay.lens);
  int32_t* ctr = misc;            // step counter of the round
  int32_t* flags = misc + 1;      // [kMaxR] last-split flags
  int32_t* red = misc + 16;       // [2 * NW] plan scratch

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, j4 = lane >> 4;
  if (a.clocks != nullptr && tid == 0) atomicMin(&a.clocks[0], (unsigned long long)__builtin_amdgcn_s_memrealtime());
  if (tid == 0) *ctr = 0;                          // ordered before the first claim by the plan's barriers
  const int plan_bits = wg_plan<NW, NP>(seq_lens, a.B, Hi, a.max_pages, base, lens, red);
  const int T = base[a.B];                       // < 2^31: the host bounds the step count
  // shares go to the first min(gridDim.x, T) workgroups, so that none is empty
  // and the workgroups holding steps of an item are consecutive
  const int grid = T < (int)gridDim.x ? T : (int)gridDim.x, wg = blockIdx.x;
  // Sequences of unequal lengths (none empty) get cost-balanced shares from an
  // LDS table; otherwise share_begin(w) = floor(w T / grid) in closed form, from
  // T = sq * grid + sr (w * sr < 2^20).
  int alpha = Pol::kShareAlpha;
  if (grid > 0 && 2 * alpha > T / grid) alpha = (T / grid) / 2;
  if ((plan_bits & 3) != 1 || grid < 1) alpha = 0;
  // UQ_FLAG_CHECK: bits found by this wave, OR-ed into the error word at the end
  uint32_t chk = a.err != nullptr && blockIdx.x == 0 && wave == 0 && (plan_bits & 4) ? UQ_CHECK_BAD_LEN : 0u;
  int32_t* sb = reinterpret_cast<int32_t*>(smem + lay.sb);
  if (alpha > 0) {
    share_plan<NW, NP>(base, lens, a.B, Hi, T, grid, alpha, sb);
  } else {
    const int sq = grid > 0 ? T / grid : 0, sr = T - sq * grid;
    const float r_grid = __builtin_amdgcn_rcpf((float)grid);
    for (int w = tid; w <= grid; w += NT) sb[w] = w * sq + div_q20(w * sr, grid, r_grid);
    __syncthreads();
  }
  const float r_hi = __builtin_amdgcn_rcpf((float)Hi);
  const float grid_per_cost = (float)grid * __builtin_amdgcn_rcpf((float)T + (float)alpha * (float)(a.B * Hi));
  const float falpha = (float)alpha;
  auto share_begin = [&](int w) -> int { return sb[w]; };
  // the w whose share holds step g of item f: estimated from the cost of g
  // (g + alpha (f + 1)), then walked to the exact share
  auto owner = [&](int g, int f) -> int {
    int w = (int)(((float)g + falpha * (float)(f + 1)) * grid_per_cost);
    w = w < 0 ? 0 : (w >= grid ? grid - 1 : w);
    while (w > 0 && share_begin(w) > g) --w;
    while (w + 1 < grid && share_begin(w + 1) <= g) ++w;
    return w;
  };
  const int g_lo = wg < grid ? share_begin(wg) : 0, g_hi = wg < grid ? share_begin(wg + 1) : 0;

  for (int g_cur = g_lo; g_cur < g_hi;) {
    // ---- round set-up: segments k = 0 .. nR-1 are items f0 + k clipped to the
    // share.  Every wave derives them itself, segment k in its lane k, so no
    // barrier is needed before the claims; wave 0 also stores them in LDS for the
    // masked steps and the merge (read after the barriers below).
    int f0;
    {
      // b: the last index with sbase[b] <= g_cur (a non-empty sequence), found
      // 64 candidates at a time with a ballot
      int lo = 0, n = a.B;                       // candidates lo .. lo + n - 1
      while (n > 1) {
        const int stride = (n + 63) / 64;
        const int c = lo + lane * stride;
        const int cnt = __builtin_popcountll(__ballot(lane * stride < n && base[c] <= g_cur));
        lo += (cnt - 1) * stride;
        n = min(stride, n - (cnt - 1) * stride);
      }
      const int steps = seq_steps<NP>(lens[lo]);   // per item of sequence lo (> 0: base[lo] <= g_cur < base[lo + 1])
      f0 = lo * Hi + div_q20(g_cur - base[lo], steps, __builtin_amdgcn_rcpf((float)steps));
    }
    int sg_b = 0, sg_hk = 0, sg_pbeg = 0, sg_npg = 0, sg_lrel = 0, sg_nstep = 0, sg_slot = -1, sg_ncontrib = 1;
    int sg_end = 0;
    bool sg_ok = false, sg_new = false;
    {
      const int f = f0 + lane;
      if (lane < a.R && f < a.B * Hi) {
        const int b = div_q20(f, Hi, r_hi);
        const int hk = f - b * Hi;
        const int steps = seq_steps<NP>(lens[b]);
        const int start = base[b] + hk * steps, end = start + steps;
        sg_ok = lane == 0 || start < g_hi;
        const int s_lo = start > g_cur ? start : g_cur, s_hi = end < g_hi ? end : g_hi;
        const int L = lens[b];
        const int pages = (L + kPage - 1) / kPage;
        sg_b = b;
        sg_hk = hk;
        sg_pbeg = NP * (s_lo - start);
        sg_npg = max(min(pages - sg_pbeg, NP * (s_hi - s_lo)), 0);
        sg_lrel = L - sg_pbeg * kPage;
        sg_nstep = max(s_hi - s_lo, 0);
        const bool partial = s_lo > start || s_hi < end;
        sg_slot = partial ? 2 * wg + (g_lo >= start ? 0 : 1) : -1;
        sg_ncontrib = partial ? owner(end - 1, f) - owner(start, f) + 1 : 1;
        sg_end = end;
        sg_new = s_hi == end && L > 0;           // the item's last step, holding its newest token
      }
    }
    const int nR = __builtin_popcountll(__ballot(sg_ok));   // valid segments are lanes 0 .. nR-1
    if (lane >= nR) sg_nstep = 0, sg_new = false;
    const int sg_incl = wave_incl_scan(sg_nstep);
    const int sg_first = sg_incl - sg_nstep;                 // first step of segment `lane` in the round
    const int T = __builtin_amdgcn_readlane(sg_incl, nR - 1);
    if (wave == 0 && lane < nR) {
      int32_t* r = rec + 8 * lane;
      r[kRecB] = sg_b;
      r[kRecPBegin] = sg_pbeg;
      r[kRecNpg] = sg_npg;
      r[kRecHk] = sg_hk;
      r[kRecLRel] = sg_lrel;
      r[kRecNStep] = sg_nstep;
      r[kRecSlot] = sg_slot;
      r[kRecNContrib] = sg_ncontrib;
    }
    {
      const int e = __builtin_amdgcn_readlane(sg_end, nR - 1);
      g_cur = e < g_hi ? e : g_hi;               // next round starts after the last segment
    }
    for (int i = tid; i < nR * NW * kSR; i += NT) smx[i] = -INFINITY;   // parks come after the barrier below

    // query rows of the round, row r = k * G + h; the first pass's loads go out
    // ahead of the key/value prologue
    const int nrows = nR * G;
    auto qrow_of = [&](int r) -> int64_t {       // r < nrows; segment r / G's record from its lane
      const int k = r / G, h = r - k * G;
      return (int64_t)__shfl(sg_b, k) * a.Hq + (int64_t)__shfl(sg_hk, k) * G + h;
    };
    const int qr0 = tid >> 4, qp = tid & 15;
    QueryRows<D, IN, FMT> qrows;
    qrows.load(a.q, qr0 < nrows ? qrow_of(qr0) : 0, qr0 < nrows, qp);

    // ---- fused step: the newest token of each item whose last step is in this
    // round is written here, by wave k for segment k (rows: the item's kNH K
    // heads, then its V heads, D/8 lanes per row).  Only the wave that claims
    // that last step reads the page slot, and the claim comes after one of the
    // barriers below: the one before the main loop when the step's index in the
    // round is past the NW * (N + 1) indices taken in the prologue, else one
    // right after the write, before any claim.
    using NewRow = Fp4Row<D, IN, D / 8>;
    NewRow nrow;
    uint8_t* nblk = nullptr;
    int noff = 0;
    bool nwrite = false;               // this wave has a row to write (row lanes: nlive)
    int np = 0;                        // lane part of the lane's row
    bool nlive = false, nv = false;    // the lane's row exists / is a V row
    if constexpr (FMT == UQ_KV_FP4) {
      // segment k of a round is written by wave k: rounds hold at most NW
      // segments (launch_one)
      if (a.k_new != nullptr) {
        const uint64_t nm = __ballot(sg_new);
        if ((nm >> wave) & 1) {
          nwrite = true;
          int ln = lane;                   // opaque: the lane-dependent addresses are formed here, not
          asm volatile("" : "+v"(ln));     // kept in registers across rounds
          const int nr = ln / (D / 8);
          np = ln % (D / 8);
          nlive = nr < 2 * Pol::kNH;
          nv = nr >= Pol::kNH;
          const int b = __builtin_amdgcn_readlane(sg_b, wave), it = __builtin_amdgcn_readlane(sg_hk, wave);
          const int t = lens[b] - 1;
          int page = page_table[(int64_t)b * a.max_pages + (t >> 4)];
          if (a.err != nullptr && (uint32_t)page >= (uint32_t)a.num_pages) {   // checked: no write
            chk |= UQ_CHECK_BAD_PAGE;
            page = 0;
            nlive = false;
          }
          const int head = Pol::kNH * it + (nlive ? nr % Pol::kNH : 0);
          nrow.load(nv && nlive ? a.v_new : a.k_new, (int64_t)b * a.Hkv + head, np);
          nblk = const_cast<uint8_t*>(nv && nlive ? a.v_pool : a.k_pool) + (int64_t)page * a.page_bytes +
                 (int64_t)fp4_block_pos(head, page, a.Hkv, a.hmask) * NewRow::BLK;
          noff = t & 15;
        }
        if (__ballot(sg_new && sg_first + sg_nstep <= NW * (N + 1)) != 0) {
          if (nwrite) {
            write_new<RV>(nrow, nblk, noff, nlive, nv, np, a.constopt != 0, a.rot);
            nwrite = false;
          }
          __syncthreads();
        }
      }
    }

    // ---- step claims
    constexpr int kIds = NP < 4 ? 4 : NP;
    struct Claim {
      int meta;          // < 0: no step; else full << 28 | item << 20 | step
      int hk;
      int ids[kIds];     // page ids of the step's NP pages (page 0 of the pool when none)
    };
    // A claim takes the next step index from the LDS counter, then reads the
    // step's page ids.  The prologue takes all its indices first: LDS and
    // scalar-memory results share one completion counter, so an index taken
    // after a page-table read would wait for that read.
    auto take = [&]() {
      int g = 0;
      if (lane == 0) g = atomicAdd(ctr, 1);
      return __builtin_amdgcn_readlane(g, 0);
    };
    auto claim_at = [&](int g) {
      Claim c;
      if (g >= T) {
        c.meta = -1;
        c.hk = 0;
#pragma unroll
        for (int x = 0; x < kIds; ++x) c.ids[x] = 0;
        return c;
      }
      // segment k: the last one whose first step is <= g
      const int k = __builtin_popcountll(__ballot(lane >= 1 && lane < nR && sg_first <= g));
      const int s = g - __builtin_amdgcn_readlane(sg_first, k);
      const int b = __builtin_amdgcn_readlane(sg_b, k);
      const int p_begin = __builtin_amdgcn_readlane(sg_pbeg, k);
      const int npg = __builtin_amdgcn_readlane(sg_npg, k);
      const int lrel = __builtin_amdgcn_readlane(sg_lrel, k);
      c.hk = __builtin_amdgcn_readlane(sg_hk, k);
      // wave-uniform page-table reads: scalar loads, outside the in-order
      // vector-memory counter of the key/value loads
      const int32_t* pt = page_table + (int64_t)b * a.max_pages + p_begin;
#pragma unroll
      for (int x = 0; x < kIds; ++x) c.ids[x] = x < NP ? pt[min(NP * s + x, npg - 1)] : 0;
      if (a.err != nullptr) {                    // checked: an id outside the pool reads page 0
#pragma unroll
        for (int x = 0; x < kIds; ++x)
          if ((uint32_t)c.ids[x] >= (uint32_t)a.num_pages) {
            c.ids[x] = 0;
            chk |= UQ_CHECK_BAD_PAGE;
          }
      }
      const bool full = (NP * s + NP <= npg) && ((NP * s + NP) * kPage <= lrel);
      c.meta = (full ? 1 << 28 : 0) | (k << 20) | s;
      return c;
    };
    auto claim = [&]() { return claim_at(take()); };
    auto load_k = [&](typename Pol::KStep& st, const Claim& c) {
      Pol::load_k(st, a.k_pool, c.ids, a.page_bytes, PageGeo{c.hk * Pol::kNH, a.Hkv, a.hmask, a.units, a.umask},
                  r16, j4);
    };
    auto load_v = [&](typename Pol::VStep& st, const Claim& c) {
      Pol::load_v(st, a.v_pool, c.ids, a.page_bytes, PageGeo{c.hk * Pol::kNH, a.Hkv, a.hmask, a.units, a.umask},
                  r16, j4);
    };

    // ---- prologue: N K and N - 1 V buffers.  K is consumed by the QK at the
    // start of a step, so its buffer is refilled for step s + N right after; V is
    // used at the end of a step and its buffer is refilled for step s + N - 1 at
    // the start of the next.  Loads of claims past the end read page 0 of the
    // pool (always present) so that every path issues the same loads.
    typename Pol::KStep kst[N];
    typename Pol::VStep vst[N];
    int meta[N + 1];               // meta[j]: step j after the current one
    Claim cv, ck;                  // next V load (step + N - 1) and next K load (step + N)
    Claim c0[N];                   // all page-table reads go out before the first key/value load
    int g0[N + 1];
#pragma unroll
    for (int i = 0; i <= N; ++i) g0[i] = take();
#pragma unroll
    for (int i = 0; i < N; ++i) {
      c0[i] = claim_at(g0[i]);
      meta[i] = c0[i].meta;
    }
    ck = claim_at(g0[N]);
    meta[N] = ck.meta;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      load_k(kst[i], c0[i]);
      if (i < N - 1) load_v(vst[i], c0[i]);
    }
    cv = c0[N - 1];
    // The newest token's write, while the first steps' loads are in flight: those
    // steps do not hold its slot (when one of the round's first NW (N + 1) steps
    // is an item's last, the write went out before the claims, above); it is
    // ordered before the main loop's claims by the barrier below.
    if constexpr (FMT == UQ_KV_FP4) {
      if (nwrite) write_new<RV>(nrow, nblk, noff, nlive, nv, np, a.constopt != 0, a.rot);
    }

    if (qr0 < nrows) qrows.template finish<RV>(qs + qr0 * D * ESZ, qp, a.rot);
    for (int r = qr0 + NT / 16; r < nrows; r += NT / 16) {
      QueryRows<D, IN, FMT> more;
      more.load(a.q, qrow_of(r), true, qp);
      more.template finish<RV>(qs + r * D * ESZ, qp, a.rot);
    }
    __syncthreads();

    // ---- running state of the item the wave is on
    typename Pol::QOp qo;
    const int lane_head = r16 / a.G;   // which KV head of the item this lane's column belongs to
    float m_run = -INFINITY, l_run = 0.f;
    v4f O[Pol::kTiles];
    int acc_k = -1;

    auto park = [&]() {            // running state -> LDS slot (acc_k, wave)
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      if (r16 < G) {
        const int slot = (acc_k * NW + wave) * kSR + r16;
        float* o = so + slot * D;
#pragma unroll
        for (int tt = 0; tt < Pol::kTiles; ++tt)
#pragma unroll
          for (int v = 0; v < 4; ++v) o[Pol::channel(tt, j4, v)] = O[tt][v];
        if (j4 == 0) {
          smx[slot] = m_run * a.scale_log2;
          slx[slot] = l_tot;
        }
      }
    };
    auto begin_item = [&](int k) {
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int t = 0; t < Pol::kTiles; ++t) O[t] = v4f{0, 0, 0, 0};
      Pol::load_q(qo, qs + (k * G + r16) * D * ESZ, r16 < G, j4, lane_head);
      acc_k = k;
    };

    // Softmax and PV of step s of the current item given its logits S.  Slots
    // past the item (pages past its split, tokens past the sequence) get logit
    // -inf and value zero; the masking is applied on every step (all slots valid
    // on full ones), which costs a few ALU operations but keeps a single copy of
    // the step code and its register allocation.
    auto finish_step = [&](v4f (&S)[TOK / 4], typename Pol::VStep& st, int s, bool full) {
     if constexpr (SpvOf<Pol>::value) {
      // Scaled-MFMA PV: the step's probabilities against its own largest logit
      // of each row, its PV into fresh accumulators, then merged into the running
      // state (m_run = -inf before the first step: weight 0 for the empty state).
      // valid slots of the lane's FP8 pages 2(j >> 1), + 1, + 4, + 5 inside its
      // 8-slot window 8(j & 1) .. + 7
      int nv[4] = {8, 8, 8, 8};
      if (!full) {
        const int npg = rec[8 * acc_k + kRecNpg], lrel = rec[8 * acc_k + kRecLRel];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int px = NP * s + 2 * (j4 >> 1) + (x & 1) + 4 * (x >> 1);
          nv[x] = px < npg ? max(min(8, lrel - px * kPage - 8 * (j4 & 1)), 0) : 0;
        }
      }
      float t[TOK];
#pragma unroll
      for (int m = 0; m < TOK / 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          t[4 * m + v] = 2 * (m & 3) + (v >> 1) < nv[2 * (m >> 2) + (v & 1)] ? S[m][v] : -INFINITY;
      float mx = t[0];
#pragma unroll
      for (int i = 1; i < TOK; ++i) mx = fmaxf(mx, t[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float neg = -mx * a.scale_log2;
      float pf[TOK];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < TOK; ++i) {
        pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[i], a.scale_log2, neg));
        psum += pf[i];
      }
      v4f Z[Pol::kTiles];
#pragma unroll
      for (int tt = 0; tt < Pol::kTiles; ++tt) Z[tt] = v4f{0, 0, 0, 0};
      Pol::pv(st, pf, nv, Z, lane);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
      const float beta = __builtin_amdgcn_exp2f((mx - m_new) * a.scale_log2);
      l_run = __builtin_fmaf(l_run, alpha, psum * beta);
#pragma unroll
      for (int tt = 0; tt < Pol::kTiles; ++tt) O[tt] = O[tt] * alpha + Z[tt] * beta;
      m_run = m_new;
     } else {
      int nvalid = TOK;                            // valid ones among this lane's TOK slots
      if (!full) {
        const int npg = rec[8 * acc_k + kRecNpg], lrel = rec[8 * acc_k + kRecLRel];
        const int pj = NP * s + Pol::lane_page(j4);
        const int in_page = pj < npg ? min(kPage, lrel - pj * kPage) : 0;
        nvalid = min(max(in_page - Pol::lane_slot0(j4), 0), TOK);
      }
      float t[TOK];
#pragma unroll
      for (int m = 0; m < TOK / 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) t[4 * m + v] = 4 * m + v < nvalid ? S[m][v] : -INFINITY;
      // Conditional rescaling: exponents are taken against the running reference
      // m_run as long as every lane's probabilities sum to at most 2^8 (so each
      // p <= 2^8, well inside float16).  Otherwise (a logit above the reference by
      // more than 8 binades, the first step, or a NaN from -inf - -inf) the
      // reference is raised to the row maximum across the 4 lanes of the row, l
      // and O are rescaled and the probabilities recomputed.
      float neg_mc = -m_run * a.scale_log2;
      float pf[TOK];
#pragma unroll
      for (int i = 0; i < TOK; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[i], a.scale_log2, neg_mc));
      float psum = pf[0];
#pragma unroll
      for (int i = 1; i < TOK; ++i) psum += pf[i];
      if (__any(!(psum <= 256.f))) {
        float mx = t[0];
#pragma unroll
        for (int i = 1; i < TOK; ++i) mx = fmaxf(mx, t[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale_log2);
        l_run *= alpha;
#pragma unroll
        for (int tt = 0; tt < Pol::kTiles; ++tt) O[tt] *= alpha;
        m_run = m_new;
        neg_mc = -m_run * a.scale_log2;
#pragma unroll
        for (int i = 0; i < TOK; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[i], a.scale_log2, neg_mc));
        psum = pf[0];
#pragma unroll
        for (int i = 1; i < TOK; ++i) psum += pf[i];
      }
      l_run += psum;
      using POp = std::conditional_t<PBf16Of<Pol>::value, v8bf, v8h>;
      POp Pm[TOK / 8][2];
#pragma unroll
      for (int half = 0; half < TOK / 8; ++half) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (PBf16Of<Pol>::value) split_bf16x2(pf[8 * half + 2 * i], pf[8 * half + 2 * i + 1], hw[i], lw[i]);
          else split_f16x2(pf[8 * half + 2 * i], pf[8 * half + 2 * i + 1], hw[i], lw[i]);
        }
        Pm[half][0] = __builtin_bit_cast(POp, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        Pm[half][1] = __builtin_bit_cast(POp, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
      Pol::mask_v(st, nvalid);
      Pol::pv(st, Pm, O, lane_head);
     }
    };

    for (;;) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int mc = meta[0];
        if (mc < 0) goto steps_done;
        const int kc = (mc >> 20) & 0xFF, sc = mc & 0xFFFFF;
        if (kc != acc_k) {
          if (acc_k >= 0) park();
          begin_item(kc);
        }
        load_v(vst[(i + N - 1) % N], cv);        // V of step + N - 1
        v4f S[TOK / 4];
        Pol::qk(kst[i], qo, S);
        load_k(kst[i], ck);                      // K of step + N
        cv = ck;
#pragma unroll
        for (int j = 0; j < N; ++j) meta[j] = meta[j + 1];
        ck = claim();
        meta[N] = ck.meta;
        finish_step(S, vst[i], sc, (mc >> 28) & 1);
      }
    }
  steps_done:
    if (acc_k >= 0) park();
    __syncthreads();

    // ---- merge the wave slots of each segment: a wave takes two rows at a time,
    // lanes 0-31 the first and 32-63 the second, channels (lane % 32) + 32 c
    // (row pairs indexed by wave-uniform scalars; the rows differ per half)
    {
      constexpr int PC = D / 32;
      int ln = lane;                             // opaque: the lane-derived values are formed here,
      asm volatile("" : "+v"(ln));               // not held in registers from the kernel's start
      const int half = ln >> 5, l32 = ln & 31;
      for (int row0 = 2 * __builtin_amdgcn_readfirstlane(wave); row0 < nrows; row0 += 2 * NW) {
        const int row = row0 + half;
        const bool have = row < nrows;
        const int rr = have ? row : row0;
        const int k = rr / G, h = rr - k * G;
        const int32_t* r = rec + 8 * k;
        const int slot0 = k * NW * kSR + h;      // slot of wave w: slot0 + w * kSR
        // all slot reads first, then the weighted sum without branches; a slot of
        // a wave that took no step has m = -inf and stale l and O, masked out
        float ms[NW], ls[NW], os[NW][PC];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          ms[w] = smx[slot0 + w * kSR];
          ls[w] = slx[slot0 + w * kSR];
#pragma unroll
          for (int c = 0; c < PC; ++c) os[w][c] = so[(slot0 + w * kSR) * D + l32 + 32 * c];
        }
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) m = fmaxf(m, ms[w]);
        float o[PC], l = 0.f;
#pragma unroll
        for (int c = 0; c < PC; ++c) o[c] = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const bool live = ms[w] > -INFINITY;
          const float wt = live ? __builtin_amdgcn_exp2f(ms[w] - m) : 0.f;
          l = live ? fmaf(wt, ls[w], l) : l;
#pragma unroll
          for (int c = 0; c < PC; ++c) o[c] = live ? fmaf(wt, os[w][c], o[c]) : o[c];
        }
        const int nstep = r[kRecNStep], slot = r[kRecSlot];   // nstep == 0: empty sequence, written below
        const bool whole = have && nstep > 0 && slot < 0;
        if (have && nstep > 0 && slot >= 0) {
          const int64_t prow = (int64_t)slot * G + h;
#pragma unroll
          for (int c = 0; c < PC; ++c) st_dev(a.po + prow * D + l32 + 32 * c, o[c]);
          if (l32 == 0) {
            st_dev(a.ml + 2 * prow, m);
            st_dev(a.ml + 2 * prow + 1, l);
          }
        }
        if (__any(whole))                        // the whole wave runs the butterflies
          store_row32<D, UNROT, RV>(o, l, a.out + ((int64_t)r[kRecB] * a.Hq + (int64_t)r[kRecHk] * G + h) * D, whole,
                                ln, a.rot);
      }
    }

    bool any_partial = false;
#pragma unroll
    for (int k = 0; k < kMaxR; ++k) any_partial |= k < nR && rec[8 * k + kRecSlot] >= 0;
    if (any_partial) {
      // publish the partials; the last workgroup of an item to arrive merges them
      wait_vmem();
      __syncthreads();
      if (tid < nR) {
        const int32_t* r = rec + 8 * tid;
        int is_last = 0;
        if (r[kRecSlot] >= 0) {
          int32_t* c = a.cnt + (int64_t)r[kRecB] * Hi + r[kRecHk];
          const int old = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          is_last = old == r[kRecNContrib] - 1;
          if (is_last) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        flags[tid] = is_last;
      }
      __syncthreads();
      // Two rows per wave at a time, lanes 0-31 the first and 32-63 the second
      // (channels (lane % 32) + 32 c).  A row's contributors go 32 at a time, lane
      // i of the half holding contributor c0 + i's (m, l); their O rows are read
      // 16 contributors per batch, the first batch together with the (m, l)
      // reads, so that a merge of up to 16 contributors waits for one round trip
      // (each read goes past the L2 to the device level).
      constexpr int PC = D / 32;
      constexpr int BATCH = 16;
      const int half = lane >> 5, l32 = lane & 31;
      for (int row0 = 2 * __builtin_amdgcn_readfirstlane(wave); row0 < nrows; row0 += 2 * NW) {
        const int row = row0 + half;
        const int rr = row < nrows ? row : row0;
        const int k = rr / G, h = rr - k * G;
        const bool mine = row < nrows && flags[k] != 0;
        if (!__any(mine)) continue;
        const int32_t* r = rec + 8 * k;
        const int b = r[kRecB], hk = r[kRecHk];
        const int steps = seq_steps<NP>(lens[b]);
        const int start = base[b] + hk * steps;
        const int w0 = owner(start, b * Hi + hk), n = mine ? r[kRecNContrib] : 0;
        // partial of contributor w0 + i: slot 2w if the item begins its share, else 2w + 1
        auto prow_of = [&](int i) -> int64_t {
          const int w = w0 + i;
          return (int64_t)(2 * w + (share_begin(w) >= start ? 0 : 1)) * G + h;
        };
        const int nmax = max(n, __shfl_xor(n, 32));              // the wave's loop bound
        float m = -INFINITY, l = 0.f, o[PC];
#pragma unroll
        for (int c = 0; c < PC; ++c) o[c] = 0.f;
        for (int c0 = 0; c0 < nmax; c0 += 32) {
          const int nc = min(32, n - c0);                         // <= 0: no contributor left in this half
          float vm = -INFINITY, vl = 0.f;
          if (l32 < nc) {
            const float* v = a.ml + 2 * prow_of(c0 + l32);
            vm = ld_dev(v);
            vl = ld_dev(v + 1);
          }
          const int ncmax = min(32, nmax - c0);
          float buf[BATCH][PC];
          auto fetch = [&](int i0) {                              // contributors c0 + i0 ..: past nc, weight 0
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
              if (nc > 0) {
                const float* src = a.po + prow_of(c0 + min(i0 + j, nc - 1)) * D + l32;
#pragma unroll
                for (int c = 0; c < PC; ++c) buf[j][c] = ld_dev(src + 32 * c);
              } else {
#pragma unroll
                for (int c = 0; c < PC; ++c) buf[j][c] = 0.f;
              }
            }
          };
          fetch(0);
          float mc = vm;
#pragma unroll
          for (int x = 16; x >= 1; x >>= 1) mc = fmaxf(mc, __shfl_xor(mc, x));
          const float mn = fmaxf(m, mc);
          const float keep = m > -INFINITY ? __builtin_amdgcn_exp2f(m - mn) : 0.f;   // rescale of earlier chunks
          const float wt = vm > -INFINITY ? __builtin_amdgcn_exp2f(vm - mn) : 0.f;
          float lw = wt * vl;
#pragma unroll
          for (int x = 16; x >= 1; x >>= 1) lw += __shfl_xor(lw, x);
          l = l * keep + lw;
#pragma unroll
          for (int c = 0; c < PC; ++c) o[c] *= keep;
          m = mn;
          for (int i0 = 0; i0 < ncmax; i0 += BATCH) {
            if (i0 > 0) fetch(i0);
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
              // the weight of contributor c0 + i0 + j, from its lane of the half (0 past nc)
              const float ws = __shfl(wt, 32 * half + min(i0 + j, 31));
              const float wj = i0 + j < nc ? ws : 0.f;
#pragma unroll
              for (int c = 0; c < PC; ++c) o[c] += wj * buf[j][c];
            }
          }
        }
        store_row32<D, UNROT, RV>(o, l, a.out + ((int64_t)b * a.Hq + (int64_t)hk * G + h) * D, mine, lane, a.rot);
      }
    }
    if (tid == 0) *ctr = 0;                        // every claim of this round is done (barrier above)
    __syncthreads();                               // LDS is reused by the next round
  }

  if (chk != 0u && lane == 0) __hip_atomic_fetch_or(a.err, chk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // rows of empty sequences are zero
  for (int b = wg; b < a.B; b += gridDim.x) {
    if (lens[b] > 0) continue;                     // the plan's clamped lengths, still in LDS
    for (int i = tid; i < a.Hq * D; i += NT) a.out[(int64_t)b * a.Hq * D + i] = 0.f;
  }
  if (a.clocks != nullptr) {                       // after every wave of the workgroup has finished
    __syncthreads();
    if (tid == 0) atomicMax(&a.clocks[1], (unsigned long long)__builtin_amdgcn_s_memrealtime());
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compute units and LDS bytes per workgroup of the current device, cached.
struct DeviceLimits { int cus, lds; };
DeviceLimits device_limits() {
  static std::atomic<int> cache_cus[64], cache_lds[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int cus = cache_cus[dev].load(std::memory_order_relaxed), lds = cache_lds[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lds <= 0)
      lds = 64 * 1024;
    cache_lds[dev].store(lds, std::memory_order_relaxed);
    cache_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return {cus, lds};
}

template <int D, int IN, int FMT, bool UNROT, class Pol, bool RV = false>
hipError_t launch_one(const DecodeArgs& a, const KArgs& k0, hipStream_t s) {
  constexpr int NW = 4 * Pol::kOcc;
  constexpr int ESZ = FMT == UQ_KV_BF16 ? 2 : 1;
  const DeviceLimits dl = device_limits();
  const int G = a.Hq / a.Hkv * Pol::kNH;   // rows of an item
  const int grid = dl.cus < kMaxGrid ? dl.cus : kMaxGrid;
  // segments per round: as many as fit in LDS (the share of a workgroup usually
  // spans a few items)
  int R = kMaxR < NW ? kMaxR : NW;     // the fused step's write of segment k is done by wave k
  while (R > 1 && Lds(R, NW, G, D, ESZ, a.B).total > dl.lds) --R;
  const int lds = Lds(R, NW, G, D, ESZ, a.B).total;
  if (lds > dl.lds) return hipErrorInvalidConfiguration;
  auto kern = decode_kernel<Pol, D, IN, FMT, UNROT, RV>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  KArgs k = k0;
  k.R = R;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), (size_t)lds, s, k, a.page_table, a.seq_lens);
  return hipGetLastError();
}

template <class T> struct PolTag {
  using type = T;
};

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
  k.hmask = a.hmask;
  k.units = (int32_t)(a.page_bytes >> 8);
  k.umask = pow2_mask(k.units);
  k.G = a.Hq / a.Hkv;
  k.scale_log2 = a.sm_scale * 1.4426950408889634f;
  k.out = a.out;
  k.ml = reinterpret_cast<float*>(a.ws + L.ml);
  k.po = reinterpret_cast<float*>(a.ws + L.po);
  k.cnt = reinterpret_cast<int32_t*>(a.ws + L.cnt);
  k.err = a.check ? reinterpret_cast<uint32_t*>(a.ws + L.err) : nullptr;
  k.num_pages = a.num_pages;
  k.k_new = a.k_new;
  k.v_new = a.v_new;
  k.constopt = a.constopt ? 1 : 0;
  k.rot = a.rot;
  k.clocks = reinterpret_cast<unsigned long long*>(a.clocks);
  hipError_t e;
  if (a.ev_start != nullptr && (e = hipEventRecord(a.ev_start, s)) != hipSuccess) return e;
  const bool bf = a.q_dtype == UQ_IN_BF16;
  // FP4 caches with a rotation variant take their own instantiations, so the
  // plain path carries none of the variant code
  auto fp4 = [&](auto pol, auto rv) -> hipError_t {
    using P = typename decltype(pol)::type;
    constexpr bool RV = decltype(rv)::value;
    if (a.unrotate) return bf ? launch_one<D, UQ_IN_BF16, UQ_KV_FP4, true, P, RV>(a, k, s)
                              : launch_one<D, UQ_IN_F32, UQ_KV_FP4, true, P, RV>(a, k, s);
    return bf ? launch_one<D, UQ_IN_BF16, UQ_KV_FP4, false, P, RV>(a, k, s)
              : launch_one<D, UQ_IN_F32, UQ_KV_FP4, false, P, RV>(a, k, s);
  };
  const bool rv = a.rot.k_only != 0u || (a.rot.s[0] | a.rot.s[1] | a.rot.s[2] | a.rot.s[3]) != 0u;
  if (a.format == UQ_KV_FP4 && a.pv_scaled) {
    e = rv ? fp4(PolTag<Fp4SpvPol<D>>{}, std::true_type{}) : fp4(PolTag<Fp4SpvPol<D>>{}, std::false_type{});
  } else if (a.format == UQ_KV_FP4 && k.G <= 8 && a.Hkv % 2 == 0) {
    // KV-head pairs fill the 16 MFMA columns
    e = rv ? fp4(PolTag<Fp4PairPol<D>>{}, std::true_type{}) : fp4(PolTag<Fp4PairPol<D>>{}, std::false_type{});
  } else if (a.format == UQ_KV_FP4) {
    e = rv ? fp4(PolTag<Fp4Pol<D>>{}, std::true_type{}) : fp4(PolTag<Fp4Pol<D>>{}, std::false_type{});
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
  (void)Hq;
  const size_t G = 16;   // rows of an item, at most (query heads per KV head, or per KV-head pair)
  DecodeLayout L;
  size_t off = 0;
  L.err = off; off = align256(off + sizeof(uint32_t));
  L.cnt = off; off = align256(off + sizeof(int32_t) * (size_t)B * Hkv);
  L.ml = off; off = align256(off + sizeof(float) * 2 * (2 * (size_t)kMaxGrid) * G);
  L.po = off; off = align256(off + sizeof(float) * (2 * (size_t)kMaxGrid) * G * D);
  L.total = off;
  return L;
}


// ------------------------------------------------------------------ chunked prefill
// Causal attention of chunks of query tokens over the FP4 cache ([review] §1 and
// §5.4: a new turn's tokens read the resident prefix instead of re-prefilling it).
// A workgroup of 8 waves (two per SIMD) takes kPfRows query rows, rows
// r = t G + h for QT = kPfRows / G consecutive chunk tokens t of one sequence and
// the G query heads of one KV head, and walks the cache from position 0 to its
// last token's position in steps of 8 pages (128 keys), each two MFMA sub-steps
// of 4 pages (64 keys).  Per step:
//   - the values are converted once for the whole workgroup: wave x takes page
//     x of the step, each lane one channel pair of it (all 16 slots at d = 128),
//     turns it into float16 with the hardware FP4 converter and the slots' group
//     scales, and writes both channels transposed ([channel][token]) into one of
//     two LDS buffers (the next step's, while this step's is read);
//   - the keys are staged the same way, as the pages' bytes (PfK), and every
//     wave reads its operands from there in the FP4 decode's layout; then, for
//     its two 16-row column blocks and each sub-step, it runs the scaled-MFMA
//     QK, the online softmax with lazy rescaling, and the PV on f16 MFMAs with
//     P as hi + lo and V^T operands read from LDS (the next step's staging sits
//     between the two sub-steps);
//   - one barrier, after which the buffer just read may be written again.
// Logits past a row's own position get -inf (causal); steps that lie wholly
// before a wave's rows take no mask, and steps wholly past them no work.  Value
// slots past the sequence end convert to zero.  Rows are rotated back and stored
// like the decode's.
namespace {
constexpr int kPfWaves = 8;                               // two per SIMD
constexpr int kPfNB = 2;                                  // column blocks per wave
constexpr int kPfRows = 16 * kPfNB * kPfWaves;            // query rows of a workgroup
constexpr int kPfMaxSeqs = 4096;                          // plan in LDS
constexpr int kPfPages = 8;                               // pages per staged step
constexpr int kPfKeys = kPfPages * kPage;                 // keys per staged step
constexpr int kPfSubKeys = 4 * kPage;                     // keys per MFMA sub-step (Fp4Pol's step)
constexpr int kPfVRow = 2 * kPfKeys + 16;                 // bytes per channel row of a value buffer (pf_v_off)

struct PfArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t page_bytes;
  int32_t max_pages;
  const void* q;              // [Tq][Hq][D]
  const int32_t* cu_q;        // [B + 1] first q row of each sequence's chunk
  const int32_t* page_table;  // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  float* out;                 // [Tq][Hq][D]
  int32_t B, Hq, Hkv, G, QT;
  uint32_t g_mul;             // ceil(2^16 / G): (x g_mul) >> 16 = x / G for 0 <= x < 256, G <= 256
  int32_t hmask;              // Hkv - 1 when Hkv is a power of two, else -1
  float scale_log2;
  Rot rot;                    // the cache's rotation variant
  int32_t unrot;              // rotate the output back (V rotated)
};

template <int D>
struct PfLds {
  // The query rows and the value buffers are dead once the last step has ended;
  // the output stage then reuses their bytes.
  static constexpr int kQs = 0;                                   // [kPfRows][D] E4M3 query rows
  static constexpr int kVBuf = D * kPfVRow;                       // [D][kPfKeys] float16 (pf_v_off)
  static constexpr int kV = kQs + kPfRows * D;                    // two value buffers
  static constexpr int kKBuf = kPfPages * (Fp4Block<D>::kBytes + 16);   // a step's key blocks (PfK)
  static constexpr int kK = kV + 2 * kVBuf;                       // two key buffers
  static constexpr int kLoopEnd = kK + 2 * kKBuf;
  static constexpr int kStage = 0;                                // [kPfWaves][16][D] float rows
  static constexpr int kStageEnd = kPfWaves * 16 * D * 4;
  static constexpr int kL = kLoopEnd > kStageEnd ? kLoopEnd : kStageEnd;   // [kPfWaves][16] float l
  static constexpr int kStart = kL + kPfWaves * 16 * 4;           // [kPfMaxSeqs] first block of the i-th sequence
  static constexpr int kSeq = kStart + kPfMaxSeqs * 4;            // [kPfMaxSeqs] the i-th sequence of the order
  static constexpr int kMisc = kSeq + kPfMaxSeqs * 4;             // [2][kPfWaves] scan partials, octave mask
  static constexpr int kTotal = kMisc + 2 * kPfWaves * 4 + 4;
};

// The keys of a step are staged once per workgroup: the FP4 head block of each
// of its kPfPages pages verbatim, at a stride of kBlk + 16 bytes (which spreads
// the operand reads of a key row group's 16 lanes over all LDS banks).  Lane u
// copies kCodeLane code bytes of page u / 64 (the wave's page); lanes
// u < kScLanes also copy one scale dword, of page u % 8 (the other lanes load
// one too, and drop it, so that every lane issues the same loads).
template <int D> struct PfK {
  static constexpr int kBlk = Fp4Block<D>::kBytes;
  static constexpr int kCode = Fp4Block<D>::kCodeBytes;
  static constexpr int kStride = kBlk + 16;
  static constexpr int kCodeLane = kCode / 64;                 // 16 (d 128), 8 (d 64)
  static constexpr int kScWords = (kBlk - kCode) / 4;          // scale dwords of a page
  static constexpr int kScLanes = kPfPages * kScWords;
  uint32_t c[kCodeLane / 4];
  uint32_t s;
};

// kb: the head block of this lane's code page; kbs: that of page tid % 8.
template <int D>
__device__ __forceinline__ void pf_load_k(PfK<D>& r, const uint8_t* kb, const uint8_t* kbs, int tid) {
  using K = PfK<D>;
  const uint8_t* cp = kb + (tid & 63) * K::kCodeLane;
  if constexpr (K::kCodeLane == 16) {
    const uint4 v = load16_stream(cp);
    r.c[0] = v.x;
    r.c[1] = v.y;
    r.c[2] = v.z;
    r.c[3] = v.w;
  } else {
    const uint2 v = load8_stream(cp);
    r.c[0] = v.x;
    r.c[1] = v.y;
  }
  r.s = load4_stream(kbs + K::kCode + 4 * ((tid >> 3) % K::kScWords));
}

template <int D>
__device__ __forceinline__ void pf_store_k(const PfK<D>& r, uint8_t* kbuf, int x, int tid) {
  using K = PfK<D>;
  uint8_t* cp = kbuf + x * K::kStride + (tid & 63) * K::kCodeLane;
  if constexpr (K::kCodeLane == 16) *reinterpret_cast<uint4*>(cp) = make_uint4(r.c[0], r.c[1], r.c[2], r.c[3]);
  else *reinterpret_cast<uint2*>(cp) = make_uint2(r.c[0], r.c[1]);
  if (tid < K::kScLanes) *reinterpret_cast<uint32_t*>(kbuf + (tid & 7) * K::kStride + K::kCode + 4 * (tid >> 3)) = r.s;
}

// The QK operand of Fp4Pol (its load_k layout) read from a staged step.
template <int D>
__device__ __forceinline__ void pf_read_k(typename Fp4Pol<D>::KStep& st, const uint8_t* kbuf, int r16, int j4) {
  using K = PfK<D>;
  const uint8_t* kb = kbuf + (r16 >> 2) * K::kStride;
  if (j4 < D / 32) {
#pragma unroll
    for (int m = 0; m < 4; ++m) st.kc[m] = *reinterpret_cast<const uint4*>(kb + (4 * m + (r16 & 3)) * (D / 2) + 16 * j4);
    // scale bytes are stored [slot % 4][group][slot / 4]: one dword per lane
    st.ks = *reinterpret_cast<const uint32_t*>(kb + K::kCode + 4 * ((r16 & 3) * (D / 32) + j4));
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) st.kc[m] = make_uint4(0, 0, 0, 0);
    st.ks = 0x7F7F7F7Fu;
  }
}

// Byte offset, in a value buffer, of channel c's tokens 8 tb .. 8 tb + 7 (16 B).
// Rows of kPfVRow = 2 kPfKeys + 16 bytes: the padding puts 16 consecutive channels' chunk
// tb in 16 different bank groups, so the PV operand reads (16 lanes, 16
// consecutive channels) are conflict free with one base address per lane, and
// the conversion's stores (16 lanes, 8 consecutive channel pairs) meet at most
// two to a bank group.
__device__ __forceinline__ int pf_v_off(int c, int tb) { return c * kPfVRow + 16 * tb; }

// A step's values are converted by all the workgroup's lanes: lane u takes page
// x = u / 64 of the step (the wave's), channel pair p = (u % 64) / kParts of it
// (held by code row 16 q + r for p = (D/32) r + q, byte t = slot t) and the
// kSlots slots kSlots part .. of that row, with their scale bytes (those of p's
// group, byte t = slot t).
template <int D> struct PfV {
  static constexpr int kRows = D / 2;                          // code rows of a page
  static constexpr int kParts = 64 / kRows;                    // lanes per row: 1 (d 128), 2 (d 64)
  static constexpr int kSlots = kPage / kParts;                // slots per lane: 16, 8
  static constexpr int kW = kSlots / 4;
  uint32_t c[kW], s[kW];
};
// the code row that holds channel pair p
template <int D> __device__ __forceinline__ int pf_row(int p) { return 16 * (p % (D / 32)) + p / (D / 32); }

template <int D>
__device__ __forceinline__ void pf_load_v(PfV<D>& r, const uint8_t* vb, int p, int part) {
  using V = PfV<D>;
  const uint8_t* cb = vb + pf_row<D>(p) * kPage + V::kSlots * part;
  const uint8_t* sb = vb + Fp4Block<D>::kCodeBytes + kPage * (p / 16) + V::kSlots * part;
  if constexpr (V::kW == 4) {
    const uint4 c = load16_stream(cb), sc = load16_stream(sb);
    r.c[0] = c.x; r.c[1] = c.y; r.c[2] = c.z; r.c[3] = c.w;
    r.s[0] = sc.x; r.s[1] = sc.y; r.s[2] = sc.z; r.s[3] = sc.w;
  } else {
    const uint2 c = load8_stream(cb), sc = load8_stream(sb);
    r.c[0] = c.x; r.c[1] = c.y;
    r.s[0] = sc.x; r.s[1] = sc.y;
  }
}

// Channels 2p and 2p + 1 of the lane's slots as float16 (slots at or past nvalid
// give zero: their codes are cleared and their scale set to 2^0), stored as
// tokens 16 x + kSlots part .. of the value buffer.
template <int D>
__device__ __forceinline__ void pf_store_v(PfV<D> r, uint8_t* vbuf, int x, int p, int part, int nvalid) {
  using V = PfV<D>;
  constexpr int NS = V::kSlots;
  const int first = NS * part;
  if (nvalid < first + NS) {
#pragma unroll
    for (int w = 0; w < V::kW; ++w) {
      const uint32_t k = slot_bytes_kept(nvalid, first + 4 * w);
      r.c[w] &= k;
      r.s[w] = (r.s[w] & k) | (~k & 0x7F7F7F7Fu);
    }
  }
  uint32_t X[NS];   // slot first + t: (channel 2p, channel 2p + 1)
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    // the converter reads only the exponent field of its scale: byte k of a
    // scale word shifted into bits 23..30
    const int k = t & 3;
    const float sc = __uint_as_float(k == 3 ? r.s[t >> 2] >> 1 : r.s[t >> 2] << (23 - 8 * k));
    v2h h;
    switch (k) {
      case 0: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.c[t >> 2], sc, 0); break;
      case 1: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.c[t >> 2], sc, 1); break;
      case 2: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.c[t >> 2], sc, 2); break;
      default: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.c[t >> 2], sc, 3); break;
    }
    X[t] = __builtin_bit_cast(uint32_t, h);
  }
  uint32_t ev[NS / 2], od[NS / 2];
#pragma unroll
  for (int i = 0; i < NS / 2; ++i) {
    ev[i] = __builtin_amdgcn_perm(X[2 * i + 1], X[2 * i], 0x05040100u);   // low halves: channel 2p
    od[i] = __builtin_amdgcn_perm(X[2 * i + 1], X[2 * i], 0x07060302u);   // high halves: channel 2p + 1
  }
  // 8 slots (one 16-B chunk of tokens) per store
#pragma unroll
  for (int h = 0; h < NS / 8; ++h) {
    const int tb = 2 * x + (NS == 16 ? h : part);
    *reinterpret_cast<uint4*>(vbuf + pf_v_off(2 * p, tb)) = make_uint4(ev[4 * h], ev[4 * h + 1], ev[4 * h + 2], ev[4 * h + 3]);
    *reinterpret_cast<uint4*>(vbuf + pf_v_off(2 * p + 1, tb)) = make_uint4(od[4 * h], od[4 * h + 1], od[4 * h + 2], od[4 * h + 3]);
  }
}

template <int D, int IN>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_kernel(const PfArgs a) {
  using Pol = Fp4Pol<D>;
  using KStep = typename Pol::KStep;
  constexpr int NT = 64 * kPfWaves;
  constexpr int TOK = Pol::kTok;                               // 16 slots of one page per lane
  constexpr int kTiles = D / 16;
  using L = PfLds<D>;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* qs = smem + L::kQs;
  uint8_t* vbuf0 = smem + L::kV;
  uint8_t* vbuf1 = smem + L::kV + L::kVBuf;
  uint8_t* kbuf0 = smem + L::kK;
  uint8_t* kbuf1 = smem + L::kK + L::kKBuf;
  float* stage = reinterpret_cast<float*>(smem + L::kStage);
  float* stage_l = reinterpret_cast<float*>(smem + L::kL);
  int32_t* start = reinterpret_cast<int32_t*>(smem + L::kStart);
  int32_t* seq = reinterpret_cast<int32_t*>(smem + L::kSeq);
  int32_t* red = reinterpret_cast<int32_t*>(smem + L::kMisc);
  uint32_t* octaves = reinterpret_cast<uint32_t*>(smem + L::kMisc + 2 * kPfWaves * 4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform values stay scalar
  const int r16 = lane & 15, j4 = lane >> 4;
  const int hk = (int)(blockIdx.x % (unsigned)a.Hkv);

  // ---- plan.  The blocks (QT chunk tokens of one sequence) are handed out
  // longest first, so that the long ones do not start last: sequences by the
  // octave of their length, longest octave first, in index order within one; a
  // sequence's blocks from its last; the KV heads of a block adjacent.  Every
  // workgroup derives the same order: start[i] = first block of the i-th
  // sequence of it, seq[i] = that sequence.
  auto nblk_of = [&](int b) { return (a.cu_q[b + 1] - a.cu_q[b] + a.QT - 1) / a.QT; };
  auto octave_of = [&](int b) { return 31 - __builtin_clz((uint32_t)max(clamp_len(a.seq_lens[b], a.max_pages), 1)); };
  if (tid == 0) *octaves = 0u;
  __syncthreads();
  for (int b = tid; b < a.B; b += NT)
    if (nblk_of(b) > 0) atomicOr(octaves, 1u << octave_of(b));
  __syncthreads();
  uint32_t left = __builtin_amdgcn_readfirstlane(*octaves);
  int carry = 0, ncarry = 0;                                   // blocks, sequences so far
  while (left != 0u) {
    const int oct = 31 - __builtin_clz(left);
    left &= ~(1u << oct);
    for (int b0 = 0; b0 < a.B; b0 += NT) {
      const int b = b0 + tid;
      const int n = b < a.B && octave_of(b) == oct ? nblk_of(b) : 0;
      const int one = n > 0 ? 1 : 0;
      const int incl = wave_incl_scan(n), incl1 = wave_incl_scan(one);
      if (lane == 63) {
        red[wave] = incl;
        red[kPfWaves + wave] = incl1;
      }
      __syncthreads();
      int woff = 0, chunk = 0, woff1 = 0, chunk1 = 0;
#pragma unroll
      for (int w = 0; w < kPfWaves; ++w) {
        woff += w < wave ? red[w] : 0;
        chunk += red[w];
        woff1 += w < wave ? red[kPfWaves + w] : 0;
        chunk1 += red[kPfWaves + w];
      }
      if (one) {
        const int i = ncarry + woff1 + incl1 - 1;
        start[i] = carry + woff + incl - n;
        seq[i] = b;
      }
      carry += chunk;
      ncarry += chunk1;
      __syncthreads();
    }
  }
  const int item = (int)(blockIdx.x / (unsigned)a.Hkv);
  if (item >= carry) return;                                   // past the last block: idle
  int lo = 0, hi = ncarry - 1;                                 // the last i with start[i] <= item
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= item) lo = mid;
    else hi = mid - 1;
  }
  // the block's sequence and first chunk token: the same in every lane (scalar)
  const int b = __builtin_amdgcn_readfirstlane(seq[lo]);
  const int q0 = a.cu_q[b], qlen = a.cu_q[b + 1] - q0;
  const int t0 = (nblk_of(b) - 1 - (item - __builtin_amdgcn_readfirstlane(start[lo]))) * a.QT;  // first chunk token of the block
  const int nt = min(a.QT, qlen - t0);                          // its tokens (at least one)
  const int Ls = clamp_len(a.seq_lens[b], a.max_pages);
  const int pos0 = Ls - qlen + t0;                              // position of token t0
  const int nrows = nt * a.G;
  // row / G for a workgroup row (below kPfRows) by a multiply: no division
  // sequence whose reciprocal would stay live through the step loop
  auto div_g = [&](int r) { return (int)(__umul24((uint32_t)r, a.g_mul) >> 16); };
  const int npages = (Ls + kPage - 1) / kPage;
  // position of row r; padding rows (r >= nrows: zero queries, not stored) take
  // the last row's, so that positions never decrease with r
  auto row_pos = [&](int r) -> int {
    const int p = pos0 + div_g(min(r, nrows - 1));
    return p < 0 ? 0 : p;
  };
  const int steps = row_pos(nrows - 1) / kPfKeys + 1;

  // ---- query rows: rotate, round to E4M3, into LDS
  for (int r = tid >> 4; r < kPfRows; r += NT / 16) {
    const int p = tid & 15;
    QueryRows<D, IN, UQ_KV_FP4> qr;
    const bool valid = r < nrows;
    const int rg = valid ? div_g(r) : 0;
    const int64_t qrow = (int64_t)(q0 + t0 + rg) * a.Hq + (int64_t)hk * a.G + (valid ? r - rg * a.G : 0);
    qr.load(a.q, qrow, valid, p);
    qr.template finish<true>(qs + r * D, p, a.rot);
  }
  __syncthreads();

  typename Pol::QOp qo[kPfNB];
  int rpos[kPfNB];                                             // position of this lane's row in block c
  float m_run[kPfNB], l_run[kPfNB];
  v4f O[kPfNB][kTiles];
#pragma unroll
  for (int c = 0; c < kPfNB; ++c) {
    const int row = (wave * kPfNB + c) * 16 + r16;
    Pol::load_q(qo[c], qs + row * D, true, j4, 0);
    rpos[c] = row_pos(row);
    m_run[c] = -INFINITY;
    l_run[c] = 0.f;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) O[c][t] = v4f{0, 0, 0, 0};
  }
  // steps before s_free hold no key past any row of the wave; steps past s_last
  // hold none at or before them
  const int s_free = (row_pos(wave * kPfNB * 16) + 1) / kPfKeys;
  const int s_last = row_pos(wave * kPfNB * 16 + kPfNB * 16 - 1) / kPfKeys;

  const int32_t* pt = a.page_table + (int64_t)b * a.max_pages;
  // Page ids are read two steps ahead, and every load of the loop is issued
  // whether or not its step exists (indices clamped into the sequence's row of
  // the table, so the bytes read are the cache's own), in a fixed order: a wait
  // for one load then never waits for loads issued after it.  Lane l reads the
  // id of page l % 8 of a step; a lane copying page x's bytes takes its id from
  // lane x.
  auto page_ids = [&](int s) { return pt[max(min(kPfPages * s + (lane & 7), npages - 1), 0)]; };
  using VC = PfV<D>;
  const int vx = wave;                                         // the page whose keys and values this lane copies
  const int vp = (tid & 63) / VC::kParts, vpart = (tid & 63) % VC::kParts;
  auto head_block = [&](const uint8_t* pool, int pid) {
    return pool + (int64_t)pid * a.page_bytes + (int64_t)fp4_block_pos(hk, pid, a.Hkv, a.hmask) * Pol::kBlk;
  };
  auto v_valid = [&](int s) { return min(max(Ls - (kPfKeys * s + kPage * vx), 0), kPage); };
  // raw keys and values of the step whose page ids are in ids
  auto load_raw = [&](PfK<D>& kr, VC& vr, int ids) {
    const int pid = __builtin_amdgcn_readlane(ids, vx);
    pf_load_k<D>(kr, head_block(a.k_pool, pid), head_block(a.k_pool, ids), tid);
    pf_load_v<D>(vr, head_block(a.v_pool, pid), vp, vpart);
  };

  PfK<D> kr;
  VC vr;
  int ids;                                                     // page ids of step s + 2
  {
    load_raw(kr, vr, page_ids(0));
    const int id1 = page_ids(1);
    pf_store_k<D>(kr, kbuf0, vx, tid);
    pf_store_v<D>(vr, vbuf0, vx, vp, vpart, v_valid(0));
    load_raw(kr, vr, id1);
    ids = page_ids(2);
  }
  __syncthreads();

  // A staged step is two MFMA sub-steps of 4 pages (64 keys) each, the FP4
  // decode's step: the keys of sub-step `sub` are pages 4 sub .. 4 sub + 3 of
  // the staged ones, its values tokens 64 sub .. of the value buffer.
  v8h P[kPfNB][TOK / 8][2];
  // QK and online softmax of both column blocks, leaving P.  MASK: the step
  // reaches past some row of the wave.
  auto softmax_sub = [&](auto mask_t, int s, int sub, const uint8_t* kb) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_t)::value;
    const int key0 = kPfKeys * s + kPfSubKeys * sub + kPage * j4;   // first key of this lane's page
    KStep kc;
    pf_read_k<D>(kc, kb + 4 * sub * PfK<D>::kStride, r16, j4);
#pragma unroll
    for (int c = 0; c < kPfNB; ++c) {
      v4f S[TOK / 4];
      Pol::qk(kc, qo[c], S);
      float t[TOK];
#pragma unroll
      for (int m = 0; m < TOK / 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) t[4 * m + v] = S[m][v];
      if constexpr (MASK) {
        const int nvalid = min(max(rpos[c] - key0 + 1, 0), TOK);   // causal: keys <= the row's position
#pragma unroll
        for (int i = 0; i < TOK; ++i) t[i] = i < nvalid ? t[i] : -INFINITY;
      }
      float neg_mc = -m_run[c] * a.scale_log2;
      float pf[TOK];
#pragma unroll
      for (int i = 0; i < TOK; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[i], a.scale_log2, neg_mc));
      float psum = pf[0];
#pragma unroll
      for (int i = 1; i < TOK; ++i) psum += pf[i];
      if (__any(!(psum <= 256.f))) {
        float mx = t[0];
#pragma unroll
        for (int i = 1; i < TOK; ++i) mx = fmaxf(mx, t[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[c], mx);
        // a row whose every key so far is masked keeps m = -inf and takes no rescale
        const float alpha = m_new > -INFINITY ? __builtin_amdgcn_exp2f((m_run[c] - m_new) * a.scale_log2) : 1.f;
        const float keep = m_run[c] > -INFINITY ? alpha : 0.f;
        l_run[c] *= keep;
#pragma unroll
        for (int tt = 0; tt < kTiles; ++tt) O[c][tt] *= keep;
        m_run[c] = m_new;
        neg_mc = m_new > -INFINITY ? -m_new * a.scale_log2 : 0.f;
#pragma unroll
        for (int i = 0; i < TOK; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[i], a.scale_log2, neg_mc));
        psum = pf[0];
#pragma unroll
        for (int i = 1; i < TOK; ++i) psum += pf[i];
      }
      l_run[c] += psum;
#pragma unroll
      for (int half = 0; half < TOK / 8; ++half) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_f16x2(pf[8 * half + 2 * i], pf[8 * half + 2 * i + 1], hw[i], lw[i]);
        P[c][half][0] = __builtin_bit_cast(v8h, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        P[c][half][1] = __builtin_bit_cast(v8h, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
    }
  };
  // PV of both column blocks.  Output tiles in pairs: the 16 MFMAs of a pair
  // touch each of its four accumulators every fourth MFMA, so that no MFMA waits
  // for the result of the one before it.  V^T operands are read a pair ahead.
  auto pv_sub = [&](int sub, const uint8_t* vb) __attribute__((always_inline)) {
    auto rd = [&](int q, int h) {
      return *reinterpret_cast<const v8h*>(vb + pf_v_off(16 * q + r16, 8 * sub + 2 * j4 + h));
    };
    v8h va[2][2][2];                                           // [pair buffer][tile of the pair][half]
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int h = 0; h < 2; ++h) va[0][qq][h] = rd(qq, h);
#pragma unroll
    for (int qp = 0; qp < kTiles / 2; ++qp) {
      if (qp + 1 < kTiles / 2) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int h = 0; h < 2; ++h) va[(qp + 1) & 1][qq][h] = rd(2 * (qp + 1) + qq, h);
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int c = 0; c < kPfNB; ++c)
              O[c][2 * qp + qq] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[qp & 1][qq][half], P[c][half][hl],
                                                                        O[c][2 * qp + qq], 0, 0, 0);
    }
  };

  // One step s: the keys and values of step s in LDS buffers s & 1, the raw keys
  // and values of step s + 1 in kr, vr.
  auto step = [&](auto mask_t, auto odd_t, int s) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(odd_t)::value;                // s & 1, known where the step is placed
    const bool active = !decltype(mask_t)::value || s <= s_last;   // wave-uniform
    const uint8_t* kb = ODD ? kbuf1 : kbuf0;
    const uint8_t* vb = ODD ? vbuf1 : vbuf0;
    if (active) {
      softmax_sub(mask_t, s, 0, kb);
      pv_sub(0, vb);
    }
    // the next step's keys and values (past the last step: a clamped page; its
    // values cleared), between the sub-steps: after a PV, so that no
    // probabilities are live, and with a sub-step's work on each side for the
    // other wave of the SIMD to overlap (at the step's end it ran 3% slower)
    pf_store_k<D>(kr, ODD ? kbuf0 : kbuf1, vx, tid);
    pf_store_v<D>(vr, ODD ? vbuf0 : vbuf1, vx, vp, vpart, v_valid(s + 1));
    load_raw(kr, vr, ids);                                     // step s + 2
    ids = page_ids(s + 3);
    if (active) {
      softmax_sub(mask_t, s, 1, kb);
      pv_sub(1, vb);
    }
    __syncthreads();                                           // buffers s & 1 are free again
  };
  using Free = std::false_type;
  using Masked = std::true_type;
  using Even = std::false_type;
  using Odd = std::true_type;
  // The step loop is unrolled by two so that each step's LDS buffers are fixed
  // offsets.
  int s = 0;
  for (; s + 2 <= s_free && s + 2 <= steps; s += 2) {
    step(Free{}, Even{}, s);
    step(Free{}, Odd{}, s + 1);
  }
  if (s < s_free && s < steps) step(Free{}, Even{}, s++);
  if ((s & 1) && s < steps) step(Masked{}, Odd{}, s++);
  for (; s < steps; s += 2) {
    step(Masked{}, Even{}, s);
    if (s + 1 < steps) step(Masked{}, Odd{}, s + 1);
  }

  // ---- rows out: block by block through the wave's LDS stage (16 rows), two
  // rows at a time per wave (one per 32-lane half), normalized, rotated back.
  // Every wave has passed the last step's barrier: the stage's bytes are free.
  constexpr int PC = D / 32;
  float* st = stage + wave * 16 * D;
  float* stl = stage_l + wave * 16;
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int c = 0; c < kPfNB; ++c) {
    float l_tot = l_run[c] + __shfl_xor(l_run[c], 16);
    l_tot += __shfl_xor(l_tot, 32);
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v) st[r16 * D + 16 * tt + 4 * j4 + v] = O[c][tt][v];
    if (j4 == 0) stl[r16] = l_tot;
    __builtin_amdgcn_s_waitcnt(0xC07F);                         // lgkmcnt(0): the stage is written
    __builtin_amdgcn_wave_barrier();
    for (int rr = 0; rr < 16; rr += 2) {
      const int rloc = rr + half;
      const int row = (wave * kPfNB + c) * 16 + rloc;
      float o[PC];
#pragma unroll
      for (int k = 0; k < PC; ++k) o[k] = st[rloc * D + l32 + 32 * k];
      const float l = stl[rloc];
      const bool live = row < nrows;
      const int rg = div_g(row);
      const int64_t orow = live ? (int64_t)(q0 + t0 + rg) * a.Hq + (int64_t)hk * a.G + row - rg * a.G : 0;
      if (a.unrot) store_row32<D, true, true>(o, l, a.out + orow * D, live, lane, a.rot);
      else store_row32<D, false, true>(o, l, a.out + orow * D, live, lane, a.rot);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();                           // the stage is reused by the next block
  }
}
}  // namespace

hipError_t launch_prefill(const PrefillArgs& p, hipStream_t s) {
  PfArgs a;
  a.k_pool = p.k_pool;
  a.v_pool = p.v_pool;
  a.page_bytes = p.page_bytes;
  a.max_pages = p.max_pages;
  a.q = p.q;
  a.cu_q = p.cu_q;
  a.page_table = p.page_table;
  a.seq_lens = p.seq_lens;
  a.out = p.out;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.hmask = p.hmask;
  a.G = p.Hq / p.Hkv;
  a.QT = kPfRows / a.G;
  a.g_mul = (65536u + (uint32_t)a.G - 1u) / (uint32_t)a.G;
  a.scale_log2 = p.sm_scale * 1.4426950408889634f;
  a.rot = p.rot;
  a.unrot = p.rot.k_only ? 0 : 1;
  // blocks: at most ceil(Tq / QT) + B (each sequence ends at most one partial
  // block); one workgroup per block and KV head
  const int64_t nblk = ((int64_t)p.Tq + a.QT - 1) / a.QT + p.B;
  if (nblk * p.Hkv > INT32_MAX / 2) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(nblk * p.Hkv));
  auto go = [&](auto kern, size_t lds) -> hipError_t {
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * kPfWaves), lds, s, a);
    return hipGetLastError();
  };
  const bool bf = p.q_dtype == UQ_IN_BF16;
  if (p.D == 128)
    return bf ? go(prefill_kernel<128, UQ_IN_BF16>, PfLds<128>::kTotal) : go(prefill_kernel<128, UQ_IN_F32>, PfLds<128>::kTotal);
  return bf ? go(prefill_kernel<64, UQ_IN_BF16>, PfLds<64>::kTotal) : go(prefill_kernel<64, UQ_IN_F32>, PfLds<64>::kTotal);
}

int prefill_max_seqs() { return kPfMaxSeqs; }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.D == 128 ? launch_decode_d<128>(a, s) : launch_decode_d<64>(a, s);
}

}  // namespace uq
