// Host-side declarations shared by the libuq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/uq.h"

namespace uq {

// A cache's rotation variant as the FP4 kernels take it (by value): k_only = V
// stored in its own basis; s = sign bits of R = c_d H_d diag(s), bit i % 32 of
// s[i / 32] set for s_i = -1 (all zero for the plain transform).
struct Rot {
  uint32_t k_only;
  uint32_t s[4];
};

struct AppendArgs {
  const void* k;              // [T][H][D] bf16 or f32
  const void* v;
  const int32_t* slot_mapping;
  uint8_t* k_pool;
  uint8_t* v_pool;
  int64_t page_bytes;         // bytes of one page of one pool
  int32_t T, H;
  int32_t hmask;              // H - 1 when H is a power of two, else -1 (FP4 block positions)
  int32_t units, umask;       // FP8: page_bytes / 256, and units - 1 when a power of two, else -1
  int32_t constopt;           // FP4: constOpt group scales (UQ_FLAG_SCALE_CONSTOPT)
  Rot rot;                    // FP4: the cache's rotation variant
};

// Launchers return the hipError_t of the launch.
hipError_t launch_append_fp4(const AppendArgs& a, int head_dim, int in_dtype, hipStream_t s);
hipError_t launch_append_fp8(const AppendArgs& a, int head_dim, int in_dtype, hipStream_t s);
hipError_t launch_append_bf16(const AppendArgs& a, int head_dim, int in_dtype, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_query(const void* q, int in_dtype, uint8_t* q_fp8, int rows, int head_dim,
                        bool rotate, const Rot& signs, hipStream_t s);


struct DecodeLayout {
  size_t err, cnt, ml, po, total;   // byte offsets into the workspace
};

constexpr int kMaxDecodeSeqs = 8192;   // per-workgroup plan lives in LDS

DecodeLayout decode_layout(int format, int num_seqs, int num_q_heads, int num_kv_heads, int head_dim);

struct DecodeArgs {
  int format;
  const void* q;             // caller's query (bf16 / f32)
  int q_dtype;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t page_bytes;
  const int32_t* page_table;
  int32_t max_pages;
  const int32_t* seq_lens;
  int32_t B, Hq, Hkv, D;
  int32_t hmask;             // Hkv - 1 when Hkv is a power of two, else -1
  float sm_scale;
  float* out;
  uint8_t* ws;
  DecodeLayout lay;
  bool check;                // UQ_FLAG_CHECK: validate page ids and lengths, report in the error word
  int32_t num_pages;         // pages in each pool (for the check)
  bool unrotate;             // FP4: rotate the output back (through R^T)
  bool pv_scaled;            // FP4: PV on the scaled FP4 x FP8 MFMA (UQ_FLAG_PV_SCALED)
  bool constopt;             // fused FP4 step: constOpt scales for the written token
  Rot rot;                   // FP4: the cache's rotation variant
  const void* k_new;         // fused FP4 step: newest token's K/V [B][Hkv][D] (q_dtype), or null
  const void* v_new;
  hipEvent_t ev_start, ev_stop;   // optional, recorded around the main kernel
  uint64_t* clocks;               // optional: wall-clock span of the main kernel (min start, max end)
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

struct PrefillArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  int64_t page_bytes;
  int32_t max_pages;
  const void* q;               // [Tq][Hq][D]
  int32_t q_dtype;
  const int32_t* cu_q;         // [B + 1]
  const int32_t* page_table;   // [B][max_pages]
  const int32_t* seq_lens;     // [B]
  float* out;                  // [Tq][Hq][D]
  int32_t B, Hq, Hkv, D, Tq;
  int32_t hmask;               // Hkv - 1 when Hkv is a power of two, else -1
  float sm_scale;
  Rot rot;                     // the cache's rotation variant
};

// H - 1 when H is a power of two, else -1 (the FP4 block-position and FP8
// rotation masks).
inline int32_t pow2_mask(int32_t H) { return H > 0 && (H & (H - 1)) == 0 ? H - 1 : -1; }
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
int prefill_max_seqs();

}  // namespace uq
