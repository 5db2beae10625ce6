// extern "C" entry points of libuq: argument validation (host only, before any
// HIP call) and kernel launches.  Declarations and semantics: include/uq.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "uq_internal.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
thread_local uint64_t* g_prof_clocks = nullptr;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return UQ_OK;
  g_last_hip_error = (int)e;
  return UQ_ERR_HIP;
}

bool dim_ok(int d) { return d == 64 || d == 128; }

// Cache descriptor checks shared by every entry point.
int check_cache(const uq_kv_cache* c, int want_format) {
  if (c == nullptr) return UQ_ERR_INVALID_ARG;
  if (c->format != want_format) return UQ_ERR_INVALID_ARG;
  if (c->page_size != UQ_PAGE_SIZE) return UQ_ERR_UNSUPPORTED;
  if (!dim_ok(c->head_dim)) return UQ_ERR_UNSUPPORTED;
  if (c->num_kv_heads < 1 || c->num_pages < 1) return UQ_ERR_INVALID_ARG;
  if (c->num_kv_heads > 65536) return UQ_ERR_UNSUPPORTED;   // page offsets are 32-bit
  if (c->k_pool == nullptr || c->v_pool == nullptr) return UQ_ERR_INVALID_ARG;
  // rotation variants: FP4 only; sign bits only with UQ_ROT_SIGNS and below head_dim
  if ((c->rotation & ~(UQ_ROT_K_ONLY | UQ_ROT_SIGNS)) != 0u) return UQ_ERR_INVALID_ARG;
  if (c->rotation != 0u && c->format != UQ_KV_FP4) return UQ_ERR_INVALID_ARG;
  for (int w = 0; w < 4; ++w) {
    const uint32_t allowed = (c->rotation & UQ_ROT_SIGNS) && 32 * w < c->head_dim ? ~0u : 0u;
    if ((c->rotation_signs[w] & ~allowed) != 0u) return UQ_ERR_INVALID_ARG;
  }
  return UQ_OK;
}

// The rotation variant of a validated cache as the kernels take it.
uq::Rot rot_of(const uq_kv_cache* c) {
  uq::Rot r;
  r.k_only = (c->rotation & UQ_ROT_K_ONLY) ? 1u : 0u;
  for (int w = 0; w < 4; ++w) r.s[w] = (c->rotation & UQ_ROT_SIGNS) ? c->rotation_signs[w] : 0u;
  return r;
}

// ---- scratch of the no-allocation decode (uq_decode_attention_noalloc)
// Its workspace is this static device array, one per GPU the library runs on.
// The layout is fixed whatever the call's shape: the arrival counters (zero
// when a call starts; every complete call leaves them zero) always occupy the
// first kNoallocCounterBytes, so a later call with another shape never finds a
// partial of an earlier call where it expects a counter.
constexpr int kNoallocMaxItems = 65536;                        // num_seqs * num_kv_heads, at most
constexpr size_t kNoallocCounterBytes = 4 * (size_t)kNoallocMaxItems;
constexpr size_t kNoallocScratchBytes = 17301504;              // counters + partials for head_dim 128

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

uq::DecodeLayout noalloc_layout(int head_dim) {
  const uq::DecodeLayout shaped = uq::decode_layout(UQ_KV_FP4, 1, 1, 1, head_dim);
  uq::DecodeLayout L;
  L.err = 0;                                                    // unused: no UQ_FLAG_CHECK here
  L.cnt = 0;
  L.ml = kNoallocCounterBytes;                                  // a multiple of 256
  L.po = L.ml + (shaped.po - shaped.ml);
  L.total = L.po + (shaped.total - shaped.po);
  return L;
}

__global__ void zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device address of `scratch` on the current device, taken once per device
// with hipGetSymbolAddress (on the host the array's name is only a stand-in for
// the symbol and must never be passed to a kernel).  The first call on a device
// also clears the counter region, with a fill kernel on the call's stream ahead
// of the call's own kernel.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return UQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (ptr == nullptr) return UQ_ERR_HIP;
    const int n = (int)(kNoallocCounterBytes / 4);
    hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(ptr), n);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return UQ_OK;
}

typedef hipError_t (*append_launcher)(const uq::AppendArgs&, int, int, hipStream_t);

int append_common(const uq_kv_cache* cache, int format, const void* k_new, const void* v_new, int32_t in_dtype,
                  const int32_t* slot_mapping, int32_t num_tokens, uint32_t flags, uq_stream_t stream,
                  append_launcher launch) {
  int st = check_cache(cache, format);
  if (st != UQ_OK) return st;
  const uint32_t allowed = format == UQ_KV_FP4 ? UQ_FLAG_SCALE_CONSTOPT : 0u;
  if ((flags & ~allowed) != 0u) return UQ_ERR_INVALID_ARG;
  if (in_dtype != UQ_IN_BF16 && in_dtype != UQ_IN_F32) return UQ_ERR_INVALID_ARG;
  if (num_tokens < 0) return UQ_ERR_INVALID_ARG;
  // the kernels index the 2 T H rows (K and V) in 32 bits
  if ((int64_t)2 * num_tokens * cache->num_kv_heads > INT32_MAX) return UQ_ERR_UNSUPPORTED;
  if (num_tokens == 0) return UQ_OK;
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr) return UQ_ERR_INVALID_ARG;
  uq::AppendArgs a;
  a.k = k_new;
  a.v = v_new;
  a.slot_mapping = slot_mapping;
  a.k_pool = static_cast<uint8_t*>(cache->k_pool);
  a.v_pool = static_cast<uint8_t*>(cache->v_pool);
  a.page_bytes = (int64_t)uq_page_bytes(cache);
  a.T = num_tokens;
  a.H = cache->num_kv_heads;
  a.hmask = uq::pow2_mask(cache->num_kv_heads);
  a.units = (int32_t)(a.page_bytes >> 8);
  a.umask = uq::pow2_mask(a.units);
  a.constopt = (flags & UQ_FLAG_SCALE_CONSTOPT) ? 1 : 0;
  a.rot = rot_of(cache);
  return hip_status(launch(a, cache->head_dim, in_dtype, reinterpret_cast<hipStream_t>(stream)));
}

// Decode entry points.  `noalloc`: the workspace is the library's static
// scratch array (fixed layout), set up after every argument check has passed.
int decode_common(const uq_kv_cache* cache, int format, const void* q, int32_t q_dtype, const int32_t* page_table,
                  int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                  float sm_scale, float* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                  uq_stream_t stream, const void* k_new = nullptr, const void* v_new = nullptr,
                  bool noalloc = false) {
  int st = check_cache(cache, format);
  if (st != UQ_OK) return st;
  // the constOpt bit selects the scale rule of the fused step's write; the
  // check reports into the workspace, which the no-allocation variant hides
  const uint32_t allowed = (noalloc ? 0u : UQ_FLAG_CHECK) |
                           (format != UQ_KV_FP4 ? 0u
                            : UQ_FLAG_OUT_ROTATED | UQ_FLAG_PV_SCALED |
                                  (k_new != nullptr ? UQ_FLAG_SCALE_CONSTOPT : 0u));
  if ((flags & ~allowed) != 0u) return UQ_ERR_INVALID_ARG;
  if (q_dtype != UQ_IN_BF16 && q_dtype != UQ_IN_F32) return UQ_ERR_INVALID_ARG;
  if (format == UQ_KV_BF16 && q_dtype != UQ_IN_BF16) return UQ_ERR_UNSUPPORTED;
  if (num_seqs < 0 || max_pages_per_seq < 1 || num_q_heads < 1) return UQ_ERR_INVALID_ARG;
  if (num_seqs > uq::kMaxDecodeSeqs) return UQ_ERR_UNSUPPORTED;
  // the step list (4 pages per step, all sequences and KV heads) is indexed in
  // 31 bits, and a step's index inside its item in 20 bits (an item has at most
  // ceil(max_pages_per_seq / 2) steps)
  if (max_pages_per_seq > (1 << 21) ||
      (int64_t)num_seqs * ((max_pages_per_seq + 3) / 4) * cache->num_kv_heads > INT32_MAX)
    return UQ_ERR_UNSUPPORTED;
  if (num_q_heads % cache->num_kv_heads != 0) return UQ_ERR_UNSUPPORTED;
  if (num_q_heads / cache->num_kv_heads > 16) return UQ_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.f) || sm_scale > 3.0e38f) return UQ_ERR_INVALID_ARG;   // NaN, <= 0, inf
  if (num_seqs == 0) return UQ_OK;
  if (q == nullptr || page_table == nullptr || seq_lens == nullptr || out == nullptr) return UQ_ERR_INVALID_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return UQ_ERR_INVALID_ARG;
  uq::DecodeLayout lay;
  if (noalloc) {
    if ((int64_t)num_seqs * cache->num_kv_heads > kNoallocMaxItems) return UQ_ERR_WORKSPACE;
    lay = noalloc_layout(cache->head_dim);
    if (lay.total > kNoallocScratchBytes) return UQ_ERR_WORKSPACE;
    const int sst = noalloc_scratch(reinterpret_cast<hipStream_t>(stream), &workspace);
    if (sst != UQ_OK) return sst;
  } else {
    const size_t need = uq_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_pages_per_seq);
    if (workspace == nullptr || workspace_bytes < need) return UQ_ERR_WORKSPACE;
    lay = uq::decode_layout(format, num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim);
  }
  uq::DecodeArgs a;
  a.format = format;
  a.q = q;
  a.q_dtype = q_dtype;
  a.k_pool = static_cast<const uint8_t*>(cache->k_pool);
  a.v_pool = static_cast<const uint8_t*>(cache->v_pool);
  a.page_bytes = (int64_t)uq_page_bytes(cache);
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.B = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = cache->num_kv_heads;
  a.D = cache->head_dim;
  a.hmask = uq::pow2_mask(cache->num_kv_heads);
  a.sm_scale = sm_scale;
  a.out = out;
  a.ws = static_cast<uint8_t*>(workspace);
  a.lay = lay;
  a.check = (flags & UQ_FLAG_CHECK) != 0u;
  a.num_pages = cache->num_pages;
  a.rot = rot_of(cache);
  a.unrotate = format == UQ_KV_FP4 && !(flags & UQ_FLAG_OUT_ROTATED) && a.rot.k_only == 0u;
  a.constopt = (flags & UQ_FLAG_SCALE_CONSTOPT) != 0u;
  a.pv_scaled = (flags & UQ_FLAG_PV_SCALED) != 0u;
  a.k_new = k_new;
  a.v_new = v_new;
  a.ev_start = g_prof_start;
  a.ev_stop = g_prof_stop;
  a.clocks = g_prof_clocks;
  g_prof_clocks = nullptr;
  g_prof_start = g_prof_stop = nullptr;
  return hip_status(uq::launch_decode(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

size_t uq_head_block_bytes(int32_t format, int32_t head_dim) {
  if (!dim_ok(head_dim)) return 0;
  switch (format) {
    case UQ_KV_FP4: return (size_t)UQ_PAGE_SIZE * head_dim / 2 + (size_t)UQ_PAGE_SIZE * head_dim / UQ_GROUP;
    case UQ_KV_FP8: return (size_t)UQ_PAGE_SIZE * head_dim;
    case UQ_KV_BF16: return (size_t)UQ_PAGE_SIZE * head_dim * 2;
    default: return 0;
  }
}

size_t uq_page_bytes(const uq_kv_cache* c) {
  if (c == nullptr || c->num_kv_heads < 1 || c->page_size != UQ_PAGE_SIZE) return 0;
  return (size_t)c->num_kv_heads * uq_head_block_bytes(c->format, c->head_dim);
}

int uq_quantize_append(const uq_kv_cache* cache, const void* k_new, const void* v_new, int32_t in_dtype,
                       const int32_t* slot_mapping, int32_t num_tokens, uint32_t flags, uq_stream_t stream) {
  return append_common(cache, UQ_KV_FP4, k_new, v_new, in_dtype, slot_mapping, num_tokens, flags, stream,
                       uq::launch_append_fp4);
}

int uq_append_fp8(const uq_kv_cache* cache, const void* k_new, const void* v_new, int32_t in_dtype,
                  const int32_t* slot_mapping, int32_t num_tokens, uint32_t flags, uq_stream_t stream) {
  return append_common(cache, UQ_KV_FP8, k_new, v_new, in_dtype, slot_mapping, num_tokens, flags, stream,
                       uq::launch_append_fp8);
}

int uq_append_bf16(const uq_kv_cache* cache, const void* k_new, const void* v_new, int32_t in_dtype,
                   const int32_t* slot_mapping, int32_t num_tokens, uint32_t flags, uq_stream_t stream) {
  return append_common(cache, UQ_KV_BF16, k_new, v_new, in_dtype, slot_mapping, num_tokens, flags, stream,
                       uq::launch_append_bf16);
}

int uq_rotate_quantize_query(const void* q, int32_t in_dtype, uint8_t* q_fp8, int32_t rows, int32_t head_dim,
                             uq_stream_t stream) {
  if (in_dtype != UQ_IN_BF16 && in_dtype != UQ_IN_F32) return UQ_ERR_INVALID_ARG;
  if (!dim_ok(head_dim)) return UQ_ERR_UNSUPPORTED;
  if (rows < 0) return UQ_ERR_INVALID_ARG;
  if (rows == 0) return UQ_OK;
  if (q == nullptr || q_fp8 == nullptr) return UQ_ERR_INVALID_ARG;
  return hip_status(uq::launch_query(q, in_dtype, q_fp8, rows, head_dim, true, uq::Rot{},
                                     reinterpret_cast<hipStream_t>(stream)));
}

int uq_rotate_quantize_query_cache(const uq_kv_cache* cache, const void* q, int32_t in_dtype, uint8_t* q_fp8,
                                   int32_t rows, uq_stream_t stream) {
  const int st = check_cache(cache, UQ_KV_FP4);
  if (st != UQ_OK) return st;
  if (in_dtype != UQ_IN_BF16 && in_dtype != UQ_IN_F32) return UQ_ERR_INVALID_ARG;
  if (rows < 0) return UQ_ERR_INVALID_ARG;
  if (rows == 0) return UQ_OK;
  if (q == nullptr || q_fp8 == nullptr) return UQ_ERR_INVALID_ARG;
  return hip_status(uq::launch_query(q, in_dtype, q_fp8, rows, cache->head_dim, true, rot_of(cache),
                                     reinterpret_cast<hipStream_t>(stream)));
}

size_t uq_decode_workspace_bytes(const uq_kv_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_pages_per_seq) {
  if (cache == nullptr || !dim_ok(cache->head_dim) || cache->num_kv_heads < 1) return 0;
  if (cache->format < UQ_KV_FP4 || cache->format > UQ_KV_BF16) return 0;
  if (num_seqs < 0 || num_q_heads < 1 || max_pages_per_seq < 1) return 0;
  return uq::decode_layout(cache->format, num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim).total;
}

int uq_decode_attention(const uq_kv_cache* cache, const void* q, int32_t q_dtype, const int32_t* page_table,
                        int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                        float sm_scale, float* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                        uq_stream_t stream) {
  return decode_common(cache, UQ_KV_FP4, q, q_dtype, page_table, max_pages_per_seq, seq_lens, num_seqs, num_q_heads,
                       sm_scale, out, workspace, workspace_bytes, flags, stream);
}

int uq_decode_attention_noalloc(const uq_kv_cache* cache, const void* q, int32_t q_dtype, const int32_t* page_table,
                                int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                int32_t num_q_heads, float sm_scale, float* out, uint32_t flags, uq_stream_t stream) {
  return decode_common(cache, UQ_KV_FP4, q, q_dtype, page_table, max_pages_per_seq, seq_lens, num_seqs, num_q_heads,
                       sm_scale, out, nullptr, 0, flags, stream, nullptr, nullptr, true);
}

int uq_append_decode_attention(const uq_kv_cache* cache, const void* k_new, const void* v_new, const void* q,
                               int32_t in_dtype, const int32_t* page_table, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, float sm_scale,
                               float* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                               uq_stream_t stream) {
  if (num_seqs > 0 && (k_new == nullptr || v_new == nullptr)) return UQ_ERR_INVALID_ARG;
  return decode_common(cache, UQ_KV_FP4, q, in_dtype, page_table, max_pages_per_seq, seq_lens, num_seqs, num_q_heads,
                       sm_scale, out, workspace, workspace_bytes, flags, stream, k_new, v_new);
}

int uq_decode_attention_fp8(const uq_kv_cache* cache, const void* q, int32_t q_dtype, const int32_t* page_table,
                            int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            float sm_scale, float* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                            uq_stream_t stream) {
  return decode_common(cache, UQ_KV_FP8, q, q_dtype, page_table, max_pages_per_seq, seq_lens, num_seqs, num_q_heads,
                       sm_scale, out, workspace, workspace_bytes, flags, stream);
}

int uq_decode_attention_bf16(const uq_kv_cache* cache, const void* q, int32_t q_dtype, const int32_t* page_table,
                             int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                             float sm_scale, float* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                             uq_stream_t stream) {
  return decode_common(cache, UQ_KV_BF16, q, q_dtype, page_table, max_pages_per_seq, seq_lens, num_seqs, num_q_heads,
                       sm_scale, out, workspace, workspace_bytes, flags, stream);
}

int uq_profile_next_decode(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return UQ_ERR_INVALID_ARG;
  g_prof_start = static_cast<hipEvent_t>(start_event);
  g_prof_stop = static_cast<hipEvent_t>(stop_event);
  return UQ_OK;
}

int uq_profile_next_decode_clock(uint64_t* clocks, int32_t* clock_khz) {
  if (clock_khz != nullptr) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return UQ_ERR_HIP;
    *clock_khz = khz;
  }
  g_prof_clocks = clocks;
  return UQ_OK;
}

int uq_prefill_attention(const uq_kv_cache* cache, const void* q, int32_t q_dtype, const int32_t* cu_seqlens_q,
                         int32_t total_q, const int32_t* page_table, int32_t max_pages_per_seq,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, float sm_scale, float* out,
                         uint32_t flags, uq_stream_t stream) {
  int st = check_cache(cache, UQ_KV_FP4);
  if (st != UQ_OK) return st;
  if (flags != 0u) return UQ_ERR_INVALID_ARG;
  if (q_dtype != UQ_IN_BF16 && q_dtype != UQ_IN_F32) return UQ_ERR_INVALID_ARG;
  if (num_seqs < 0 || total_q < 0 || max_pages_per_seq < 1 || num_q_heads < 1) return UQ_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads != 0 || num_q_heads / cache->num_kv_heads > 128) return UQ_ERR_UNSUPPORTED;
  if (num_seqs > uq::prefill_max_seqs() || max_pages_per_seq > (1 << 26)) return UQ_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.f) || !(sm_scale < INFINITY)) return UQ_ERR_INVALID_ARG;
  if (num_seqs == 0 || total_q == 0) return UQ_OK;
  if (q == nullptr || cu_seqlens_q == nullptr || page_table == nullptr || seq_lens == nullptr || out == nullptr)
    return UQ_ERR_INVALID_ARG;
  uq::PrefillArgs a;
  a.k_pool = static_cast<const uint8_t*>(cache->k_pool);
  a.v_pool = static_cast<const uint8_t*>(cache->v_pool);
  a.page_bytes = (int64_t)uq_page_bytes(cache);
  a.max_pages = max_pages_per_seq;
  a.q = q;
  a.q_dtype = q_dtype;
  a.cu_q = cu_seqlens_q;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.B = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = cache->num_kv_heads;
  a.D = cache->head_dim;
  a.hmask = uq::pow2_mask(cache->num_kv_heads);
  a.Tq = total_q;
  a.sm_scale = sm_scale;
  a.rot = rot_of(cache);
  return hip_status(uq::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

int uq_stream_read(const void* src, size_t bytes, uint32_t* sink, uq_stream_t stream) {
  if (bytes == 0) return UQ_OK;
  if (src == nullptr || sink == nullptr) return UQ_ERR_INVALID_ARG;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return UQ_ERR_INVALID_ARG;
  return hip_status(uq::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

const char* uq_status_string(int status) {
  switch (status) {
    case UQ_OK: return "ok";
    case UQ_ERR_INVALID_ARG: return "invalid argument";
    case UQ_ERR_UNSUPPORTED: return "unsupported shape or format";
    case UQ_ERR_WORKSPACE: return "workspace missing or too small";
    case UQ_ERR_HIP: return "HIP error (see uq_last_hip_error)";
    default: return "unknown status";
  }
}

int uq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
