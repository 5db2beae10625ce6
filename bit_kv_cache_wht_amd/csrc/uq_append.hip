// Cache write kernels: FP4 (rotate + quantize + pack), FP8 and BF16 baselines,
// and the query rotation to FP8.
//
// [review] = "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
//            (manon006.tistory.com/395)
// [commentary] = pheeree.github.io "kv-cache-4bit-serving-residency-collapse"
//
// FP4 work mapping: a row is one (token, KV head) vector of K or of V, spread
// over LPR consecutive lanes (see append_fp4_kernel); after the butterfly each
// lane owns the same channels of the rotated row, so group absmax, scale,
// rounding and packing need at most a max across the lanes of a group.
#include <algorithm>

#include "uq_device.h"
#include "uq_fp4_row.h"
#include "uq_internal.h"

namespace uq {

// FP4 write path ([review] §3.1; [commentary] footnote 2): WHT, group absmax,
// UE8M0 scale byte, E2M1 codes, two codes per byte, paged store (Fp4Row).
//
// LPR = D / 32 lanes per row (E = 32: one quantization group per lane) for large
// batches; LPR = D / 8 (E = 8, four lanes per group) when few rows are written,
// which cuts the float64 work each lane does on its own.
template <int D, int IN, int LPR, bool RV>
__global__ __launch_bounds__(256) void append_fp4_kernel(AppendArgs a) {
  using Row = Fp4Row<D, IN, LPR>;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int p = lane % LPR;
  const int64_t nrows = 2LL * a.T * a.H;
  const int64_t row0 = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * RPW;
  if (row0 >= nrows) return;                       // whole wave idle (no barriers used)
  const int64_t row = row0 + lane / LPR;
  const bool in_range = row < nrows;
  const int64_t r = in_range ? row : 0;            // idle lanes read row 0 (in bounds)
  const int64_t kv_rows = (int64_t)a.T * a.H;
  const bool is_v = r >= kv_rows;
  const int64_t tr = is_v ? r - kv_rows : r;       // token * H + head
  const int t = (int)(tr / a.H), h = (int)(tr - (int64_t)t * a.H);
  const int slot = a.slot_mapping[t];

  Row x;
  x.load(is_v ? a.v : a.k, tr, p);
  x.template quantize<RV>(p, a.constopt != 0, a.rot, is_v);
  if (!in_range || slot < 0) return;
  const int page = slot >> 4, off = slot & 15;
  uint8_t* blk = (is_v ? a.v_pool : a.k_pool) + (int64_t)page * a.page_bytes +
                 (int64_t)fp4_block_pos(h, page, a.H, a.hmask) * Row::BLK;
  if (!is_v) x.store_k(blk, off, p);
  else x.store_v(blk, off, p);
}

// Large writes: a persistent grid-stride loop over groups of RPW rows per wave,
// each wave fetching its next group's inputs (and slots) before working on the
// current one, so that the float64 work of one group hides the memory latency
// of the next.  A group is RPW consecutive tokens of one KV head of K or of V
// (group g: K|V head kvh = g / nblk, tokens RPW (g % nblk) ..), so that when
// the tokens fill a page's slots in order, the lanes of one store instruction
// write adjacent bytes of a page (V: one 16-byte slot row per channel pair; K:
// whole rows) and the stores merge into full lines.
template <int D, int IN, int LPR, bool RV>
__global__ __launch_bounds__(256) void append_fp4_stream_kernel(AppendArgs a) {
  using Row = Fp4Row<D, IN, LPR>;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int p = lane % LPR;
  const int nblk = (a.T + RPW - 1) / RPW;          // token blocks per K|V head
  const int groups = 2 * a.H * nblk;               // < 2^31: the host bounds 2 T H
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  int g = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (g >= groups) return;                         // whole wave idle (no barriers used)
  const double rblk = 1.0 / (double)nblk;
  struct In {
    Row x;
    int slot, tr, h;
    bool is_v, live;
  };
  auto fetch = [&](In& in, int grp) {
    // grp / nblk through a float64 reciprocal (grp < 2^31: the quotient is off
    // by at most one), then corrected
    int kvh = (int)((double)grp * rblk);
    kvh -= kvh * nblk > grp ? 1 : 0;
    kvh += (kvh + 1) * nblk <= grp ? 1 : 0;
    const int t = (grp - kvh * nblk) * RPW + lane / LPR;
    in.live = t < a.T;
    const int tt = in.live ? t : 0;                // idle lanes read token 0 (in bounds)
    in.is_v = kvh >= a.H;
    in.h = in.is_v ? kvh - a.H : kvh;
    in.tr = tt * a.H + in.h;                       // token * H + head
    in.slot = a.slot_mapping[tt];
    in.x.load(in.is_v ? a.v : a.k, in.tr, p);
  };
  auto work = [&](In& in) {
    in.x.template quantize<RV>(p, a.constopt != 0, a.rot, in.is_v);
    if (in.live && in.slot >= 0) {
      const int page = in.slot >> 4, off = in.slot & 15;
      uint8_t* blk = (in.is_v ? a.v_pool : a.k_pool) + (int64_t)page * a.page_bytes +
                     (int64_t)fp4_block_pos(in.h, page, a.H, a.hmask) * Row::BLK;
      if (!in.is_v) in.x.store_k(blk, off, p);
      else in.x.store_v(blk, off, p);
    }
  };
  // Two input buffers used in turn (no copy between iterations).  The next
  // group is fetched unconditionally (the last wave's fetch reads the final
  // group again and goes unused): a fetch on one path only would make the wait
  // for the current group's loads also wait for the prefetch.
  In b0, b1;
  fetch(b0, g);
  for (;;) {
    int gn = g + nwaves;
    fetch(b1, min(gn, groups - 1));
    work(b0);
    if (gn >= groups) break;
    g = gn;
    gn = g + nwaves;
    fetch(b0, min(gn, groups - 1));
    work(b1);
    if (gn >= groups) break;
    g = gn;
  }
}

// Baseline writes: one thread per 8 channels of a (token, head, K|V) row.
template <int D, int IN, int FMT>
__global__ __launch_bounds__(256) void append_plain_kernel(AppendArgs a) {
  constexpr int TPR = D / 8;                      // threads per row
  constexpr int ESZ = FMT == UQ_KV_FP8 ? 1 : 2;   // stored bytes per element
  constexpr int BLK = kPage * D * ESZ;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t kv_rows = (int64_t)a.T * a.H;
  const int64_t row = gid / TPR;
  if (row >= 2 * kv_rows) return;
  const int c0 = (int)(gid - row * TPR) * 8;
  const bool is_v = row >= kv_rows;
  const int64_t tr = is_v ? row - kv_rows : row;
  const int t = (int)(tr / a.H), h = (int)(tr - (int64_t)t * a.H);
  const int slot = a.slot_mapping[t];
  if (slot < 0) return;
  const int page = slot >> 4, off = slot & 15;
  const void* src = is_v ? a.v : a.k;
  float f[8];
  uint32_t bits[8];
  if constexpr (IN == UQ_IN_BF16) {
    const uint4 u = load16(static_cast<const uint16_t*>(src) + tr * D + c0);
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bits[2 * i] = d[i] & 0xFFFFu;
      bits[2 * i + 1] = d[i] >> 16;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(bits[i] << 16);
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + tr * D + c0);
    const float4 f0 = p[0], f1 = p[1];
    f[0] = f0.x; f[1] = f0.y; f[2] = f0.z; f[3] = f0.w; f[4] = f1.x; f[5] = f1.y; f[6] = f1.z; f[7] = f1.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) bits[i] = f32_to_bf16_bits(f[i]);
  }
  uint8_t* blk = (is_v ? a.v_pool : a.k_pool) + (int64_t)page * a.page_bytes + (int64_t)h * BLK;
  if constexpr (FMT == UQ_KV_FP8) {
    const uint32_t b0 = e4m3x4_f32(f[0], f[1], f[2], f[3]), b1 = e4m3x4_f32(f[4], f[5], f[6], f[7]);
    uint8_t* pg = (is_v ? a.v_pool : a.k_pool) + (int64_t)page * a.page_bytes;
    const uint32_t rot = fp8_rot(page, a.units, a.umask), pb = (uint32_t)a.page_bytes, hb = (uint32_t)(h * BLK);
    if (!is_v) {
      *reinterpret_cast<uint2*>(pg + fp8_wrap(hb + off * D + c0, rot, pb)) = make_uint2(b0, b1);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pg[fp8_wrap(hb + (c0 + i) * kPage + off, rot, pb)] = (uint8_t)((i < 4 ? b0 : b1) >> (8 * (i & 3)));
    }
  } else {
    uint16_t* blk16 = reinterpret_cast<uint16_t*>(blk);
    if (!is_v) {
      *reinterpret_cast<uint4*>(blk16 + off * D + c0) =
          make_uint4(bits[0] | bits[1] << 16, bits[2] | bits[3] << 16, bits[4] | bits[5] << 16, bits[6] | bits[7] << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) blk16[(c0 + i) * kPage + off] = (uint16_t)bits[i];
    }
  }
}

// Query rotation ([review] §3.2): q_fp8 = E4M3(c_d * H_d q) from float64.
// Same row mapping as the FP4 write path; ROT = false gives the unrotated
// E4M3 query of the FP8 baseline.
template <int D, int IN, bool ROT>
__global__ __launch_bounds__(256) void query_kernel(const void* q, uint8_t* out, int rows, Rot rot) {
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
  load_row32<IN>(q, r * D + 32 * p, x);
  if constexpr (ROT) {
    if (has_signs(rot)) {                          // R = c_d H diag(s): the signs first
#pragma unroll
      for (int e = 0; e < 32; ++e) x[e] = flip_sign(x[e], sign_mask(rot, 32 * p + e));
    }
    wht_row<D>(x, lane);
  }
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3x4_f64(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  if (!in_range) return;
  uint4* o = reinterpret_cast<uint4*>(out + r * D + 32 * p);
  o[0] = make_uint4(w[0], w[1], w[2], w[3]);
  o[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

#ifndef APPEND_LPR
#define APPEND_LPR(D) ((D) / 32)
#endif
#ifndef APPEND_BPC
#define APPEND_BPC 16
#endif
static int append_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

static unsigned grid_rows(int64_t rows, int rows_per_wave) {
  const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
  return (unsigned)((waves + 3) / 4);
}

template <int D, int IN, bool RV>
static void launch_fp4_rows(const AppendArgs& a, int64_t rows, hipStream_t s) {
  // D/8 lanes per row (8 channels each) while the rows fill less than about two
  // waves per SIMD at D/32 lanes per row; D/32 lanes per row beyond that
  constexpr int kFewRows = 256 * 4 * 2 * (64 / (D / 32));
  if (rows < kFewRows) {
    hipLaunchKernelGGL((append_fp4_kernel<D, IN, D / 8, RV>), dim3(grid_rows(rows, 64 / (D / 8))), dim3(256), 0, s,
                       a);
  } else {
    constexpr int LPR = APPEND_LPR(D);
    const unsigned blocks = (unsigned)std::min<int64_t>(grid_rows(rows, 64 / LPR), (int64_t)append_cus() * APPEND_BPC);
    hipLaunchKernelGGL((append_fp4_stream_kernel<D, IN, LPR, RV>), dim3(blocks), dim3(256), 0, s, a);
  }
}

template <bool RV>
static void launch_fp4_dispatch(const AppendArgs& a, int D, int in, int64_t rows, hipStream_t s) {
  if (D == 128 && in == UQ_IN_BF16) launch_fp4_rows<128, UQ_IN_BF16, RV>(a, rows, s);
  else if (D == 128) launch_fp4_rows<128, UQ_IN_F32, RV>(a, rows, s);
  else if (in == UQ_IN_BF16) launch_fp4_rows<64, UQ_IN_BF16, RV>(a, rows, s);
  else launch_fp4_rows<64, UQ_IN_F32, RV>(a, rows, s);
}

hipError_t launch_append_fp4(const AppendArgs& a, int D, int in, hipStream_t s) {
  const int64_t rows = 2LL * a.T * a.H;
  // caches with a rotation variant take their own instantiations, so the
  // plain path carries none of the variant code
  const bool rv = a.rot.k_only != 0u || (a.rot.s[0] | a.rot.s[1] | a.rot.s[2] | a.rot.s[3]) != 0u;
  if (rv) launch_fp4_dispatch<true>(a, D, in, rows, s);
  else launch_fp4_dispatch<false>(a, D, in, rows, s);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_plain(const AppendArgs& a, int D, int in, hipStream_t s) {
  const int64_t threads = 2LL * a.T * a.H * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (D == 128 && in == UQ_IN_BF16) hipLaunchKernelGGL((append_plain_kernel<128, UQ_IN_BF16, FMT>), grid, block, 0, s, a);
  else if (D == 128) hipLaunchKernelGGL((append_plain_kernel<128, UQ_IN_F32, FMT>), grid, block, 0, s, a);
  else if (in == UQ_IN_BF16) hipLaunchKernelGGL((append_plain_kernel<64, UQ_IN_BF16, FMT>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((append_plain_kernel<64, UQ_IN_F32, FMT>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendArgs& a, int D, int in, hipStream_t s) { return launch_plain<UQ_KV_FP8>(a, D, in, s); }
hipError_t launch_append_bf16(const AppendArgs& a, int D, int in, hipStream_t s) { return launch_plain<UQ_KV_BF16>(a, D, in, s); }

hipError_t launch_query(const void* q, int in, uint8_t* out, int rows, int D, bool rot, const Rot& signs,
                        hipStream_t s) {
  const dim3 grid(grid_rows(rows, 64 / (D / 32))), block(256);
#define UQ_Q(DD, II, RR) hipLaunchKernelGGL((query_kernel<DD, II, RR>), grid, block, 0, s, q, out, rows, signs)
  if (D == 128) {
    if (in == UQ_IN_BF16) { if (rot) UQ_Q(128, UQ_IN_BF16, true); else UQ_Q(128, UQ_IN_BF16, false); }
    else { if (rot) UQ_Q(128, UQ_IN_F32, true); else UQ_Q(128, UQ_IN_F32, false); }
  } else {
    if (in == UQ_IN_BF16) { if (rot) UQ_Q(64, UQ_IN_BF16, true); else UQ_Q(64, UQ_IN_BF16, false); }
    else { if (rot) UQ_Q(64, UQ_IN_F32, true); else UQ_Q(64, UQ_IN_F32, false); }
  }
#undef UQ_Q
  return hipGetLastError();
}

}  // namespace uq
