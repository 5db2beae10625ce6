/*
 * uq.h -- C ABI of libuq: UltraQuant-style FP4 KV cache for AMD MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [review]     "[arXiv 2606.20474] UltraQuant: 컨텍스트가 긴 에이전트를 위한 4비트 KV 캐싱"
 *                (manon006.tistory.com/395)
 *   [commentary] "kv-cache-4bit-serving-residency-collapse" (pheeree.github.io, 2026-09-01),
 *                whose footnotes quote the paper in English
 *   [tq-guide]   "TurboQuant 완전 정리 - 이론 최적에 근접한 KV 캐시·벡터 검색 양자화와 vLLM 실측"
 *                (juhoplayground.github.io)
 *
 * The write path ([review] §3.1) rotates each new key and value head vector with
 * a normalized Walsh-Hadamard transform, takes the absolute maximum of every
 * 32-channel group, stores the group scale as a UE8M0 byte (scale = byte - 127)
 * and rounds each channel to the FP4 E2M1 grid; 32 codes (16 B) plus the scale
 * byte make 17 B per group, 4.25 bits per element ([commentary] footnote 2).
 * Dequantization is value = code * 2^(byte - 127) ([review] §3.2).  The decode
 * side rotates the query into the key basis, rounds it to FP8 E4M3 once, outside
 * the key loop ([review] §3.2, §4.2), and runs attention over the paged cache.
 * BF16 and FP8 E4M3 caches on the same paged layout are the baselines
 * ([review] §4.3).
 *
 * Conventions where the pages are silent:
 *   - the WHT is the Sylvester Hadamard matrix in natural order scaled by
 *     sqrt(1/head_dim), applied to K and to V; the attention output is rotated
 *     back, so `out` is in the original basis (K-only rotation and a random
 *     sign diagonal are variants of a cache: UQ_ROT_*);
 *   - the scale exponent E is the least integer with absmax <= 6 * 2^E, clamped
 *     to [-127, 127] (never clips); rounding is to nearest, ties to even code;
 *     the sign bit is the sign of the value; every rounding decision (scale,
 *     code, E4M3 query byte) is taken in float64 on the rotated value, which is
 *     the exact Hadamard sum S times c_d (the double nearest sqrt(1/d)), rounded
 *     once, plus +0;
 *   - exact-sum domain: the rotation sums in float64 butterflies, which are exact
 *     -- and the stored bytes therefore a function of the exact rotated values --
 *     for every row (head_dim input values) that are all integer multiples of
 *     2^u with sum |x_i| < 2^(u+53) for some integer u.  Every bf16 row whose
 *     nonzero magnitudes span at most 38 binades (2^38) and every f32 row
 *     spanning at most 22 is inside.  Outside it each rotated value can differ
 *     from the exact one by at most (log2(d) + 2) * 2^-53 * c_d * sum |x_i|, and
 *     the bytes are the rounding decisions of such a value;
 *   - FP8 is OCP E4M3 (bias 7, max 448), round to nearest even, saturating.
 *
 * Memory and ownership
 *   All pointers named *pool, k_new, v_new, q, q_fp8, out, slot_mapping,
 *   page_table, seq_lens and workspace are DEVICE pointers owned by the caller.
 *   The library allocates nothing and keeps no state between calls apart from
 *   the loaded code object and a thread-local error code; calls are reentrant.
 *   Every call enqueues its kernels on `stream` (NULL = the default stream) and
 *   returns without synchronizing.  Arguments are validated on the host before
 *   any launch; device-resident contents (page ids, slots, lengths) are trusted:
 *   an out-of-range value there is undefined behaviour, except that the decode
 *   entry points check page ids and lengths under UQ_FLAG_CHECK.
 *
 * Paged layout (part of the ABI).  A pool is [num_pages][uq_page_bytes]; a page
 * holds the num_kv_heads head-blocks back to back, nothing else (FP4: exactly
 * 17 bytes per 32 elements); token position t of a sequence lives in page
 * page_table[t / 16] at slot t % 16.  The pages fix 17 B per group and paging,
 * not the byte order inside a page; the order below serves the decode's
 * operand loads, and FP4 and FP8 pages rotate their contents with the page id
 * so that blocks start at different offsets from page to page (on MI355X
 * blocks that always start at the same offset can stream more slowly).
 *   FP4: the block of KV head h in page P is at block position (h + 2P) mod
 *        num_kv_heads (for an even head count, a pair's two blocks stay
 *        adjacent and the pairs rotate by one pair position per page);
 *   FP8: the page (blocks back to back, head h at position h) is rotated by
 *        256 bytes per page id: byte b of it is stored at byte
 *        (b + 256 * (P mod (page_bytes / 256))) mod page_bytes, so that pages
 *        start their blocks at different offsets modulo 16 KB (FP8 pages of 8
 *        heads are exactly 16 KB, and the FP8 decode streamed up to 1.5x more
 *        slowly without it);
 *   BF16: the block of KV head h is at position h.
 * Head-block layouts (d = head_dim, 16 slots):
 *   FP4  K: codes [16 slot][d/2 B] (byte j: channel 2j low nibble, 2j+1 high),
 *           then scales [slot % 4][d/32 group][slot / 4]       = 17*d/2 bytes
 *   FP4  V: codes [d/2 row][16 slot] (byte: channel 2c low nibble, 2c+1 high
 *           nibble of channel pair c, stored in row 16*(c % (d/32)) + c/(d/32)),
 *           then scales [d/32 group][16 slot]                  = 17*d/2 bytes
 *   FP8  K: [16 slot][d] E4M3 bytes;   FP8  V: [d][16 slot] E4M3 bytes
 *   BF16 K: [16 slot][d] bf16;         BF16 V: [d][16 slot] bf16
 * K is slot-major because the QK product contracts over channels; V is
 * channel-major because the PV product contracts over tokens.
 */
#ifndef UQ_H
#define UQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* uq_stream_t;   /* a hipStream_t; NULL = default stream */

enum uq_status {
  UQ_OK = 0,
  UQ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum, inconsistent sizes   */
  UQ_ERR_UNSUPPORTED = -2,   /* head_dim not 64/128, page_size not 16, H_q/H_kv not 1..16  */
  UQ_ERR_WORKSPACE = -3,     /* workspace null or smaller than uq_decode_workspace_bytes  */
  UQ_ERR_HIP = -4            /* a HIP call failed; uq_last_hip_error() has the hipError_t */
};

enum uq_kv_format { UQ_KV_FP4 = 0, UQ_KV_FP8 = 1, UQ_KV_BF16 = 2 };
enum uq_in_dtype { UQ_IN_BF16 = 0, UQ_IN_F32 = 1 };

#define UQ_PAGE_SIZE 16
#define UQ_GROUP 32
#define UQ_FLAG_OUT_ROTATED 1u   /* FP4 decode: leave `out` in the rotated (WHT) basis */
/* FP4 write (uq_quantize_append, the fused step): constOpt group scales
 * ([review] §3.3 "constant-optimized scaling", §6.2): E = the integer nearest
 * to log2(RN(0.156 * m)) (m = group absmax of the rotated row, rounding in the
 * log domain), clamped to [-127, 127], m = 0 giving -127; codes x / 2^E then
 * saturate at +-6.  Without it E is the least integer with m <= 6 * 2^E. */
#define UQ_FLAG_SCALE_CONSTOPT 2u
/* Decode entry points with a workspace (uq_decode_attention, _fp8, _bf16 and
 * uq_append_decode_attention): check the device-resident contents that are
 * otherwise trusted.  A sequence length outside [0, 16 * max_pages_per_seq]
 * ORs UQ_CHECK_BAD_LEN, a page id read outside [0, num_pages) ORs
 * UQ_CHECK_BAD_PAGE into the 32-bit error word at byte offset 0 of the
 * workspace.  The word is never cleared by the library: zero it before a call
 * to see that call's findings (it is read after the call, in stream order).
 * A bad length is used clamped to that range; a bad page id is replaced by
 * page 0 before any address is formed from it, and the fused step writes no
 * token into a page whose id is bad, so the call reads and writes only inside
 * the pools, the page table and its other arguments.  Rows of a sequence with
 * a bad length or page id are then meaningless.  Without the flag these
 * contents are trusted and an out-of-range value is undefined behaviour. */
#define UQ_FLAG_CHECK 4u
#define UQ_CHECK_BAD_LEN 1u
#define UQ_CHECK_BAD_PAGE 2u
/* FP4 decode (uq_decode_attention, its no-allocation variant and
 * uq_append_decode_attention): run PV on the scaled FP4 x FP8 matrix
 * instruction as well ([review] §3.2 "dequantization rule과 scaled-MFMA", §6.3;
 * [commentary] footnote 2).  V's group scales run along head_dim while PV sums
 * over tokens, so they are folded into the probabilities: each 128-token step
 * (positions 128 s .. 128 s + 127 of a sequence) takes its probabilities
 * against its own largest logit of each query row; per 32-channel group and
 * 32-token block, P * 2^(E_t - M) is rounded to FP8 E4M3 (M = the block's
 * largest V exponent minus 8, at least -127, as the block's UE8M0 scale) and
 * multiplied by V's FP4 codes; the steps are combined as in the online
 * softmax, with the unrounded sums of P.  The E4M3 rounding costs accuracy:
 * about 3.5e-3 relative L2 on 8K-token decode statistics (against ~1e-6 for
 * the default PV, f16 hi + lo probabilities times the exactly converted V);
 * an opt-in variant, not the default. */
#define UQ_FLAG_PV_SCALED 8u

/* Cache descriptor; read at call time, never retained. */
/* Rotation variants of an FP4 cache (uq_kv_cache.rotation; 0 = K and V rotated
 * by the normalized Walsh-Hadamard transform c_d H_d, the default).  Every call
 * on one cache must use the same variant: it fixes how the stored bytes encode
 * K and V.
 *
 * UQ_ROT_K_ONLY ([review] §3.1 table "Rotation": the rotation is applied to K;
 * [commentary] footnote 1: "asymmetric K/V treatment"): V is quantized in its
 * own basis (a zero channel stored as +0); K and the query are rotated as
 * usual, and the attention output needs no rotating back (UQ_FLAG_OUT_ROTATED
 * then changes nothing).
 *
 * UQ_ROT_SIGNS ([tq-guide] "알고리즘 원리", "랜덤 회전과 Beta 분포": a random sign
 * diagonal times the Hadamard matrix): the rotation is R = c_d H_d diag(s),
 * s_i = -1 where bit i % 32 of rotation_signs[i / 32] is set, else +1; K, V
 * and the query go through R and the output back through R^T = diag(s) c_d H_d.
 * The caller draws s, once per cache.  Bits at or above head_dim must be 0, and
 * all four words must be 0 without this bit.  uq_rotate_quantize_query always
 * applies the plain transform; uq_rotate_quantize_query_cache applies the
 * cache's. */
#define UQ_ROT_K_ONLY 1u
#define UQ_ROT_SIGNS 2u

typedef struct uq_kv_cache {
  int32_t format;        /* enum uq_kv_format                                   */
  int32_t num_pages;     /* pages in each pool                                  */
  int32_t page_size;     /* tokens per page; must be 16                          */
  int32_t num_kv_heads;  /* 1 .. 65536                                            */
  int32_t head_dim;      /* 64 or 128                                            */
  void* k_pool;          /* device, [num_pages][uq_page_bytes], 256-B aligned; see
                            "Paged layout" for the block positions in a page     */
  void* v_pool;          /* device, same shape                                    */
  uint32_t rotation;     /* UQ_ROT_* bits; FP4 only (0 for FP8 and BF16)           */
  uint32_t rotation_signs[4];   /* with UQ_ROT_SIGNS: the sign bits of s          */
} uq_kv_cache;

/* Bytes of one head-block (one KV head of one page): FP4 17*d/2, FP8 16*d,
 * BF16 32*d; 0 for an unknown format or head_dim.  Host only. */
size_t uq_head_block_bytes(int32_t format, int32_t head_dim);

/* Bytes of one page of one pool: num_kv_heads head-blocks (FP4: num_kv_heads *
 * 17 * d / 2; FP8: num_kv_heads * 16 * d; BF16: num_kv_heads * 32 * d).  0 if
 * the descriptor is invalid.  Host only. */
size_t uq_page_bytes(const uq_kv_cache* cache);

/*
 * FP4 write path ([review] §3.1; [commentary] footnote 2): for each token
 * t < num_tokens with slot = slot_mapping[t] >= 0, rotate k_new[t][h] and
 * v_new[t][h] (h < num_kv_heads) with the normalized WHT in float64, quantize
 * every 32-channel group to E2M1 codes plus a UE8M0 scale byte and store them at
 * page slot/16, slot slot%16 of k_pool / v_pool.  slot < 0 skips the token.
 *   k_new, v_new  device [num_tokens][num_kv_heads][head_dim], bf16 or f32
 *                 (in_dtype), contiguous
 *   slot_mapping  device int32 [num_tokens]
 *   flags         0 or UQ_FLAG_SCALE_CONSTOPT (else UQ_ERR_INVALID_ARG)
 * cache->format must be UQ_KV_FP4.  Two tokens mapped to the same slot in one
 * call race.  num_tokens == 0 is a no-op; 2 * num_tokens * num_kv_heads above
 * 2^31 - 1 is UQ_ERR_UNSUPPORTED (the same limit holds for uq_append_fp8 and
 * uq_append_bf16).
 */
int uq_quantize_append(const uq_kv_cache* cache, const void* k_new, const void* v_new,
                       int32_t in_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                       uint32_t flags, uq_stream_t stream);

/* FP8 baseline write ([review] §4.3 "hardware FP8 KV"): each value rounded to
 * OCP E4M3 (nearest even, saturating at 448), scale 1, no rotation.  Same
 * arguments as uq_quantize_append; cache->format must be UQ_KV_FP8. */
int uq_append_fp8(const uq_kv_cache* cache, const void* k_new, const void* v_new,
                  int32_t in_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                  uint32_t flags, uq_stream_t stream);

/* BF16 baseline write ([review] §4.3 "BF16"): plain copy (f32 input rounded to
 * nearest even bf16).  cache->format must be UQ_KV_BF16. */
int uq_append_bf16(const uq_kv_cache* cache, const void* k_new, const void* v_new,
                   int32_t in_dtype, const int32_t* slot_mapping, int32_t num_tokens,
                   uint32_t flags, uq_stream_t stream);

/*
 * Query rotation ([review] §3.2, §4.2): q_fp8[r][c] = E4M3(c_d * (H_d q[r])[c]),
 * rounded directly from the float64 rotated value.
 *   q      device [rows][head_dim], bf16 or f32 (in_dtype)
 *   q_fp8  device uint8 [rows][head_dim]
 * head_dim must be 64 or 128.
 */
int uq_rotate_quantize_query(const void* q, int32_t in_dtype, uint8_t* q_fp8, int32_t rows,
                             int32_t head_dim, uq_stream_t stream);

/* The query rotation of an FP4 cache, with the cache's rotation variant
 * ([review] §3.2; [tq-guide] "랜덤 회전과 Beta 분포" for UQ_ROT_SIGNS): q_fp8[r][c] =
 * E4M3((R q[r])[c]) with R = c_d H_d diag(s) for a UQ_ROT_SIGNS cache, c_d H_d
 * otherwise (a UQ_ROT_K_ONLY cache rotates its queries like its keys), so
 * that the bytes are the query operand the decode forms for this cache.
 *   cache  FP4 descriptor (head_dim, rotation, rotation_signs are read; the
 *          pools are not touched)
 *   q, in_dtype, q_fp8, rows  as uq_rotate_quantize_query
 */
int uq_rotate_quantize_query_cache(const uq_kv_cache* cache, const void* q, int32_t in_dtype, uint8_t* q_fp8,
                                   int32_t rows, uq_stream_t stream);

/* Workspace bytes needed by the decode entry points for this shape (an upper
 * bound valid for every seq_lens content).  0 if the arguments are invalid. */
size_t uq_decode_workspace_bytes(const uq_kv_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_pages_per_seq);

/*
 * FP4 decode attention ([review] §3.2, §4.2, §6.3): for each sequence b and
 * query head h, out[b][h] = sum_j p_j * V[j] with p = softmax_j(sm_scale *
 * qhat . K[j]) over tokens j < seq_lens[b], where qhat is the rotated E4M3
 * query and K, V are the dequantized rotated cache rows of KV head
 * h / (num_q_heads / num_kv_heads); the result is rotated back with the same
 * normalized WHT unless UQ_FLAG_OUT_ROTATED is set.
 *   q           device [num_seqs][num_q_heads][head_dim], bf16 or f32 (q_dtype)
 *   page_table  device int32 [num_seqs][max_pages_per_seq]; entries past
 *               ceil(seq_lens[b] / 16) are not read
 *   seq_lens    device int32 [num_seqs], each in [0, 16 * max_pages_per_seq]
 *               (values outside are clamped to that range)
 *   out         device float [num_seqs][num_q_heads][head_dim]; must not alias
 *               any input; a sequence of length 0 gives a zero row
 *   workspace   device, >= uq_decode_workspace_bytes(...) bytes, 256-B aligned,
 *               zero-filled before its first use; every call leaves it ready for
 *               the next one (no clearing needed).  Its first 4 bytes are the
 *               UQ_FLAG_CHECK error word.  Calls that overlap in time must not
 *               share a workspace.
 *   flags       UQ_FLAG_OUT_ROTATED and UQ_FLAG_PV_SCALED (FP4), UQ_FLAG_CHECK
 * num_q_heads must be a multiple of num_kv_heads with a ratio of 1..16,
 * num_seqs at most 8192, max_pages_per_seq at most 2^21 and
 * num_seqs * ceil(max_pages_per_seq / 4) * num_kv_heads below 2^31 (else
 * UQ_ERR_UNSUPPORTED), and sm_scale positive and finite.
 * Accuracy: codes and scales enter exactly; logits and the softmax are float32,
 * probabilities and dequantized values enter the PV product as float16, so V
 * groups must have E <= 13 (|v| <= 49152) to stay finite in float16 (with
 * UQ_FLAG_PV_SCALED the probabilities are FP8 instead, see there, and V's
 * codes and scales enter the product exactly).
 */
int uq_decode_attention(const uq_kv_cache* cache, const void* q, int32_t q_dtype,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                        float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                        uint32_t flags, uq_stream_t stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the FP4 decode
 * of uq_decode_attention without a workspace argument.  Its split partials and
 * arrival counters live in a static device array of the library, 17,301,504
 * bytes per GPU it runs on, held until the process ends; the call itself
 * allocates nothing.  The first call on a device finds the array's address
 * (hipGetSymbolAddress) and clears its counters with a fill kernel on `stream`.
 * Arguments and results as uq_decode_attention, except that UQ_FLAG_CHECK is
 * refused (UQ_ERR_INVALID_ARG: there is no workspace to hold its error word);
 * in addition num_seqs * num_kv_heads above 65,536 is UQ_ERR_WORKSPACE.  Every call on one GPU shares
 * the array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must not be issued; calls in stream order are safe.
 */
int uq_decode_attention_noalloc(const uq_kv_cache* cache, const void* q, int32_t q_dtype,
                                const int32_t* page_table, int32_t max_pages_per_seq,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                float sm_scale, float* out, uint32_t flags, uq_stream_t stream);

/*
 * One FP4 decode step in a single launch ([review] §3.1 write path followed by
 * the §3.2 decode): for every sequence b with L = seq_lens[b] > 0, writes the
 * step's newest token -- k_new[b][h] and v_new[b][h] for every KV head h -- at
 * position L - 1 (page page_table[b][(L-1)/16], slot (L-1) % 16) with exactly
 * the bytes uq_quantize_append would store there, then computes
 * uq_decode_attention over positions 0 .. L-1, the new token included.  The
 * result equals uq_quantize_append with slot_mapping[b] = that slot followed by
 * uq_decode_attention.
 *   k_new, v_new  device [num_seqs][num_kv_heads][head_dim], in_dtype
 *   q             device [num_seqs][num_q_heads][head_dim], in_dtype
 *   flags         UQ_FLAG_OUT_ROTATED and UQ_FLAG_PV_SCALED as for
 *                 uq_decode_attention, and UQ_FLAG_SCALE_CONSTOPT for the write
 *                 as for uq_quantize_append
 *   other arguments and limits as uq_decode_attention; cache->format must be
 *   UQ_KV_FP4.  Sequences of length 0 write nothing.  The written slot must not
 *   be shared with another sequence's range (it never is when page tables do
 *   not share pages).
 */
int uq_append_decode_attention(const uq_kv_cache* cache, const void* k_new, const void* v_new, const void* q,
                               int32_t in_dtype, const int32_t* page_table, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, float sm_scale,
                               float* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                               uq_stream_t stream);

/*
 * Chunked-prefill attention over an FP4 cache ([review] §1 and §5.4: the tokens
 * of a new turn attend to the resident prefix instead of re-prefilling it).
 * Sequence b's chunk -- q rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 -- holds
 * its last q_len = cu_seqlens_q[b+1] - cu_seqlens_q[b] positions, already
 * written to the cache; chunk token j, at position P = seq_lens[b] - q_len + j,
 * attends to positions 0 .. P (causal).  Each output row equals the
 * uq_decode_attention row of that query over a sequence of length P + 1: q is
 * rotated and rounded to E4M3, the output is rotated back.
 *   q             device [total_q][num_q_heads][head_dim], q_dtype (bf16 or f32)
 *   cu_seqlens_q  device int32 [num_seqs + 1], non-decreasing, cu[0] = 0,
 *                 cu[num_seqs] = total_q, each chunk no longer than its sequence
 *   page_table, max_pages_per_seq, seq_lens, sm_scale as uq_decode_attention
 *   out           device float32 [total_q][num_q_heads][head_dim]
 *   flags         must be 0
 * cache->format must be UQ_KV_FP4; num_q_heads a multiple of num_kv_heads with
 * at most 128 query heads per KV head; num_seqs <= 4096 (else
 * UQ_ERR_UNSUPPORTED).  No workspace.  total_q == 0 or num_seqs == 0 is a
 * no-op.  Device-resident contents that break the rules above are undefined
 * behaviour.
 */
int uq_prefill_attention(const uq_kv_cache* cache, const void* q, int32_t q_dtype,
                         const int32_t* cu_seqlens_q, int32_t total_q, const int32_t* page_table,
                         int32_t max_pages_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_q_heads, float sm_scale, float* out, uint32_t flags,
                         uq_stream_t stream);

/* FP8 baseline decode: same arguments; cache->format must be UQ_KV_FP8; the
 * query is rounded to E4M3 without rotation and `out` needs no unrotation
 * (flags: 0 or UQ_FLAG_CHECK).  E4M3 K, q and V convert exactly to float16 for
 * the matrix products; P enters as float16 hi + lo, as in the FP4 decode. */
int uq_decode_attention_fp8(const uq_kv_cache* cache, const void* q, int32_t q_dtype,
                            const int32_t* page_table, int32_t max_pages_per_seq,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                            float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                            uint32_t flags, uq_stream_t stream);

/* BF16 baseline decode: same arguments; cache->format must be UQ_KV_BF16 and
 * q_dtype must be UQ_IN_BF16 (flags: 0 or UQ_FLAG_CHECK).  K, q and V enter
 * bf16 matrix products as stored (every finite bf16 value exactly; products
 * summed in float32), P as bf16 hi + lo (16 significant bits). */
int uq_decode_attention_bf16(const uq_kv_cache* cache, const void* q, int32_t q_dtype,
                             const int32_t* page_table, int32_t max_pages_per_seq,
                             const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                             float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                             uint32_t flags, uq_stream_t stream);

/* Instrumentation: the next decode call on this thread (any format) records
 * `start` immediately before and `stop` immediately after its main split-K
 * attention kernel, on that call's stream, then forgets both.  The events are
 * caller-owned hipEvent_t handles (created with timing enabled); passing NULL
 * for both cancels a pending request.  Nothing is skipped or reordered. */
int uq_profile_next_decode(void* start_event, void* stop_event);

/* Instrumentation: the next decode call on this host thread (any decode entry
 * point) has its attention kernel record the device's constant wall clock
 * (s_memrealtime) as each workgroup starts and after it ends:
 * clocks[0] = min(clocks[0], earliest start), clocks[1] = max(clocks[1], latest
 * end), by device-scope atomics, in stream order with the kernel.  `clocks` is
 * caller-owned device memory holding two uint64_t, set to {UINT64_MAX, 0}
 * beforehand; clocks[1] - clocks[0] is the kernel's span in ticks.  If
 * clock_khz is not NULL it receives the clock's rate (kHz) for the current
 * device.  Passing clocks = NULL cancels a pending request.  Nothing is skipped
 * or reordered; the kernel adds two atomics per workgroup and one barrier. */
int uq_profile_next_decode_clock(uint64_t* clocks, int32_t* clock_khz);

/* Instrumentation: a plain streaming read of `bytes` bytes of device memory at
 * `src`, the reference rate for a kernel bound by HBM reads (each byte loaded
 * once, coalesced, with nontemporal loads; nothing written but one 32-bit
 * word).  The XOR of all the
 * buffer's little-endian 32-bit words is XORed into *sink (device memory,
 * caller-owned; zero it first to read the XOR itself).  `src` must be 16-byte
 * aligned and `bytes` a multiple of 16 (else UQ_ERR_INVALID_ARG); bytes == 0
 * launches nothing.  Asynchronous on `stream`. */
int uq_stream_read(const void* src, size_t bytes, uint32_t* sink, uq_stream_t stream);

/* Static description of a status code. */
const char* uq_status_string(int status);

/* hipError_t of the last UQ_ERR_HIP returned on this thread (0 if none). */
int uq_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* UQ_H */
