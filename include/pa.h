/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV append + PagedAttention forward.
 *
 * Operation (PagedAttention -- CUDA Design Document, section 4 "Schema -- The
 * Compatible Contract", and Design: WebGPU PagedAttention, section 3 "Op
 * contract"): causal grouped-query attention over packed variable-length
 * queries.  Query tokens of all in-flight requests are packed along one axis
 * and delimited by cumulative_sequence_length; request b owns tokens
 * [cum[b], cum[b+1]) and its j-th new token sits at position past_seqlens[b] + j.
 * K/V of every position live in a shared fp16 block pool
 * [num_blocks, block_size, kv_num_heads, head_size]; block_table[b][i] names the
 * physical block holding positions [i*block_size, (i+1)*block_size) of request b.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer unless it says "host".  The
 *     caller owns and allocates every buffer; the library allocates nothing per
 *     call, never synchronizes, and never reads device memory on the host.
 *   - fp16 tensors are IEEE binary16, row-major, and must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it, in order; results are ready when the stream reaches them.
 *   - Errors: a non-PA_OK status means nothing was enqueued.  pa_last_error()
 *     returns a thread-local message naming the offending argument and the
 *     value expected.  Device-resident values (lengths, table entries) cannot be
 *     checked on the host; out-of-range device values never cause an
 *     out-of-bounds access (they are clamped or the token is skipped) but give
 *     unspecified results.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1, /* malformed request (validation rules)      */
  PA_ERR_UNSUPPORTED = 2,      /* well formed, but not served by a kernel   */
  PA_ERR_DEVICE = 3            /* a HIP runtime call failed                 */
} pa_status;

/* Attributes (PagedAttention -- CUDA Design Document, section 4.5; Design:
 * WebGPU PagedAttention, section 3.1).  Host struct. */
typedef struct {
  int32_t num_heads;          /* query heads H, > 0                                    */
  int32_t kv_num_heads;       /* K/V heads Hkv, > 0, H % Hkv == 0; q head h reads
                                 kv head h / (H / Hkv)                                 */
  int32_t head_size;          /* D; multiple of 8; kernels serve 64, 128, 256          */
  int32_t block_size;         /* tokens per pool block; power of two >= 16             */
  float scale;                /* 0 -> 1/sqrt(head_size) (section 12.6); finite         */
  float softcap;              /* 0 -> off; > 0 -> s = softcap*tanh(s_scaled/softcap),
                                 applied before masking (section 8.5 note); finite     */
  int32_t local_window_size;  /* -1 -> off; W >= 1 admits the W positions ending at
                                 the query's own (section 4.5, section 9)              */
  int32_t do_rotary;          /* 0/1: rotate new K (pa_append_kv) and Q (pa_forward)
                                 at their absolute position                            */
  int32_t rotary_interleaved; /* 0: pairs (i, i + r/2); 1: pairs (2i, 2i+1)            */
  int32_t cache_dtype;        /* element type of both caches (section 8.2):
                                 PA_CACHE_FP16 (0), PA_CACHE_INT8 (1) or
                                 PA_CACHE_FP8_E4M3FN (2); see "Quantized caches"     */
  int32_t k_quant_type;       /* PA_QUANT_NONE (0), PA_QUANT_PER_TENSOR (1) or
                                 PA_QUANT_PER_CHANNEL (2) for the K cache            */
  int32_t v_quant_type;       /* the same for the V cache (chosen independently)    */
  const void *head_sink;      /* NULL, or DEVICE fp16 [num_heads], 2-byte aligned: the
                                 sink logit s_h of each head, which joins the softmax
                                 denominator only (section 6.1):
                                 p_i = e^(x_i - m) / (e^(s_h - m) + sum_j e^(x_j - m)),
                                 x the score after scale and softcap; finite or -inf */
  int32_t use_smooth_softmax; /* 0/1: with head_sink NULL, a sink of 0 for every head
                                 (an explicit head_sink takes precedence)           */
  const void *q_norm_weight;  /* NULL, or DEVICE fp16 [head_size], 16-byte aligned:
                                 QK-Norm weight of Q (section 7.1), shared by heads  */
  const void *k_norm_weight;  /* the same for the new K (pa_append_kv); both weights or
                                 neither; head_size 64, 128 or 256.  Each head row x
                                 becomes fp16(x * w / sqrt(mean(x^2) + eps)), sum of
                                 squares in fp32, before RoPE (section 7.2); cached K
                                 is stored normalized, and pa_forward stages the
                                 normalized Q in its workspace                       */
  float qk_norm_epsilon;      /* 0 -> 1e-6 (section 7.1 default); else finite, > 0    */
  int32_t kv_cache_layout;    /* PA_LAYOUT_SEPARATE (0) or PA_LAYOUT_LATENT (1); see
                                 "Latent attention"                                  */
  int32_t v_head_size;        /* 0 = head_size; else 1..head_size, LATENT only: the V
                                 channels of each row and of each output head         */
  int32_t rotary_offset;      /* first rotated channel of a head, a multiple of 8;
                                 RoPE covers [rotary_offset, rotary_offset +
                                 rotary_dim) (section 12.5); 0 = from channel 0       */
} pa_attn_params;

/* Latent attention (MLA; PagedAttention -- CUDA Design Document, section 12).
 * With kv_cache_layout = PA_LAYOUT_LATENT there is one cache: key_cache holds
 * [num_blocks, block_size, 1, head_size] rows (kv_num_heads = 1), V is the
 * leading v_head_size channels of each row (section 12.2), value and
 * value_cache are NULL, and pa_forward writes out as [token_count, num_heads *
 * v_head_size].  Absorbed DeepSeek-style rows are 576 channels (512 latent +
 * 64 rotary, rotary_offset 512) with v_head_size 512: the shape the kernel
 * serves (others: PA_ERR_UNSUPPORTED), for fp16 caches smaller than 4 GiB.
 * Rules (section 12.10): an explicit scale when v_head_size != head_size
 * (section 12.6), no head_sink / smooth softmax / QK-Norm, no V quantization,
 * and RoPE only past the V channels (rotary_offset >= v_head_size).  Every
 * token runs on the latent kernel. */
enum { PA_LAYOUT_SEPARATE = 0, PA_LAYOUT_LATENT = 1 };

/* Quantized caches (PagedAttention -- CUDA Design Document, section 8).
 * With cache_dtype != PA_CACHE_FP16 both caches hold one signed byte per
 * element, [num_blocks, block_size, kv_num_heads, head_size]: int8 two's
 * complement, or float8 e4m3fn (sign, 4 exponent bits of bias 7, 3 mantissa
 * bits, no infinities, 0x7f/0xff NaN).  The value of code c is c * s with
 * zero point 0 (section 8.3.1) and s the fp32 scale of its channel: one value
 * for the whole cache (PER_TENSOR, k_scale[0]) or one per (kv head, channel)
 * (PER_CHANNEL, k_scale[kvh * head_size + d], the [kv_num_heads, 1,
 * head_size] layout of section 8.3).  pa_append_kv stores
 * saturate(round-half-even(fp32(x) / s)) of the fp16 value x the fp16 cache
 * would hold (after rotary; one fp32 division): int8 saturates to
 * [-128, 127], e4m3fn to +-448 (section 8.4, write path).  pa_forward
 * dequantizes in the kernel (section 8.5, phase 3): a PER_TENSOR K scale is
 * folded into the score scale, a PER_CHANNEL one into Q (rounded to fp16), and
 * the V scale is applied to the output accumulator.  Decode rows read the
 * codes in the decode kernel; multi-token requests in the prefill kernels,
 * which turn each lane's codes into fp16 on their way into LDS.
 * Scales are positive finite values (they are device data and not checked).
 * Validation (section 8.7): a quantized cache_dtype
 * needs both quant types non-NONE, fp16 needs both NONE; a quant type other
 * than NONE needs its scale and NONE forbids it. */
enum { PA_CACHE_FP16 = 0, PA_CACHE_INT8 = 1, PA_CACHE_FP8_E4M3FN = 2 };
enum { PA_QUANT_NONE = 0, PA_QUANT_PER_TENSOR = 1, PA_QUANT_PER_CHANNEL = 2 };

/* The paged cache and the per-step request layout.  Host struct holding
 * device pointers. */
typedef struct {
  void *key_cache;                          /* [num_blocks, block_size, Hkv, D] of
                                               fp16, or of byte codes when quantized */
  void *value_cache;                        /* same shape; both mutated in place by
                                               pa_append_kv (cache outputs alias the
                                               inputs, section 4.4); NULL when LATENT */
  int64_t num_blocks;                       /* > 0; num_blocks * block_size < 2^32   */
  const int32_t *block_table;               /* int32 [batch_size, max_blocks_per_seq]
                                               row-major; entries past a request's
                                               length are never read.  -1 (or any
                                               value outside [0, num_blocks)) is an
                                               unmapped block (section 9.2 item 3,
                                               section 9.3.1): the derived append
                                               writes nothing there and the forward
                                               masks its positions out            */
  int32_t max_blocks_per_seq;               /* > 0; capacity = this * block_size     */
  const int32_t *cumulative_sequence_length;/* int32 [batch_size + 1], cum[0] = 0,
                                               non-decreasing, cum[batch] <= tokens  */
  const int32_t *past_seqlens;              /* int32 [batch_size], >= 0              */
  int32_t batch_size;                       /* > 0                                   */
  int32_t token_count;                      /* T >= 0; rows of query/key/value/out   */
  const int32_t *slot_mapping;              /* NULL, or int32 [token_count], 4-byte
                                               aligned: the write slot of each new
                                               token (pa_append_kv only; section 5) */
  const float *k_scale;                     /* fp32 scales of a quantized K cache:
                                               [1] (PER_TENSOR, 4-byte aligned) or
                                               [kv_num_heads, head_size]
                                               (PER_CHANNEL, 16-byte aligned); NULL
                                               when k_quant_type is NONE             */
  const float *v_scale;                     /* the same for the V cache              */
} pa_paged_kv;

/*
 * pa_append_kv -- scatter the new tokens' K/V into their pool slots
 * (PagedAttention -- CUDA Design Document, section 5.1 "derived write slot",
 * section 5.2 explicit slot_mapping; section 7.2 / 12.5 for rotary applied
 * to K before the write).
 *
 *   key, value : fp16 [token_count, kv_num_heads * head_size]
 *   cos_cache, sin_cache : fp16 [rotary_rows, rotary_dim / 2]; both non-NULL iff
 *                params->do_rotary; rotary_dim even, <= head_size;
 *                rotary_rows >= max_blocks_per_seq * block_size.
 *
 * Token t of request b (cum[b] <= t < cum[b+1], j = t - cum[b]) at position
 * p = past[b] + j is written to block block_table[b][p / block_size], offset
 * p % block_size, for every kv head.  With rotary the stored K is
 * fp16(fp32(x*cos - y*sin)) of its channel pair.  With params->k_norm_weight
 * the K row is first RMS-normed to fp16 (section 7.2: norm, then RoPE, then
 * write; a quantized cache stores the codes of the result).  Tokens t >= cum[batch_size]
 * write nothing; every other slot keeps its bytes.  Enqueue before
 * pa_forward on the same stream.
 *
 * With kv->slot_mapping (section 5.2) the write slot of token t is
 * s = slot_mapping[t], the flat index block * block_size + offset: the rows
 * go to block s / block_size, offset s % block_size, and s = -1 writes
 * nothing (the token's query still attends; prefix-cached and rejected
 * speculative tokens).  K is still rotated at the token's position
 * past[b] + j.  Values outside [-1, num_blocks * block_size) are undefined
 * by section 5.4; they write nothing here.  block_table, past and cum still
 * define what pa_forward reads.
 */
pa_status pa_append_kv(const pa_attn_params *params, const pa_paged_kv *kv,
                       const void *key, const void *value,
                       const void *cos_cache, const void *sin_cache,
                       int32_t rotary_rows, int32_t rotary_dim, void *stream);

/*
 * pa_forward_workspace_bytes -- device workspace pa_forward needs for these
 * static shapes and optional replay-wide bounds (host call, writes *bytes).
 *
 *   max_query_len_bound : 0 = unknown, else an upper bound on any request's
 *                         new-token count for every step it will serve
 *   max_kv_len_bound    : 0 = unknown, else an upper bound on any request's
 *                         past + new length
 * (PagedAttention -- CUDA Design Document, section 4.7: bounds only size
 * launches and workspace, never a mask; 0 falls back to token_count and to
 * max_blocks_per_seq * block_size; over-large bounds are clamped.)  With
 * QK-Norm the workspace also stages the normalized queries, token_count *
 * num_heads * head_size fp16 (section 7.3).
 */
pa_status pa_forward_workspace_bytes(const pa_attn_params *params, const pa_paged_kv *kv,
                                     int32_t max_query_len_bound, int32_t max_kv_len_bound,
                                     size_t *bytes);

/*
 * pa_forward -- attention output of every packed token
 * (PagedAttention -- CUDA Design Document, section 4; GroupQueryAttention CPU
 * Implementation Notes, "Flash Decoding" for the split-KV merge).
 *
 *   query     : fp16 [token_count, num_heads * head_size]
 *   cos_cache, sin_cache, rotary_rows, rotary_dim : as for pa_append_kv; Q is
 *               rotated at its position on load (never written back)
 *   workspace : device scratch of >= pa_forward_workspace_bytes() bytes for the
 *               same shapes and bounds (may be NULL when that is 0); contents
 *               on entry are irrelevant; not shared with a concurrent call
 *   out       : fp16 [token_count, num_heads * head_size]
 *
 * out[t, h*D:(h+1)*D] = sum_tau softmax_tau(cap(scale * q_t,h . k_tau)) v_tau over
 * positions tau of t's request with tau <= p_t and (W < 0 or tau > p_t - W), K/V
 * read from the pool (so pa_append_kv must run first).  Positions whose block
 * is unmapped (block_table entry -1) are masked out like positions outside the
 * window; a row left with no admitted key is written as 0.  Rows of tokens
 * t >= cum[batch_size] are written as 0.  A bound smaller than a real length
 * violates the contract: work is omitted, memory stays safe.
 */
pa_status pa_forward(const pa_attn_params *params, const pa_paged_kv *kv,
                     const void *query,
                     const void *cos_cache, const void *sin_cache,
                     int32_t rotary_rows, int32_t rotary_dim,
                     int32_t max_query_len_bound, int32_t max_kv_len_bound,
                     void *workspace, size_t workspace_bytes,
                     void *out, void *stream);

/*
 * pa_forward_noalloc -- pa_forward with the library's own workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, semantics and errors as pa_forward without the workspace
 * pair; the caller still owns query, out and the cache.  The workspace is a
 * file-scope device array of PA_NOALLOC_SCRATCH_BYTES (128 MiB) that every GPU
 * the library runs on holds until the process ends; the call allocates
 * nothing (no hipMalloc / hipFree, no stream or event creation: all launches
 * go on `stream`, one after another).  A plan that needs more than
 * PA_NOALLOC_SCRATCH_BYTES (pa_forward_workspace_bytes with the same shapes
 * and bounds) returns PA_ERR_UNSUPPORTED before any device call.  Nothing in
 * the array needs to start at zero (the plan kernel writes every value a
 * later kernel reads).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race.
 */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)
pa_status pa_forward_noalloc(const pa_attn_params *params, const pa_paged_kv *kv,
                             const void *query,
                             const void *cos_cache, const void *sin_cache,
                             int32_t rotary_rows, int32_t rotary_dim,
                             int32_t max_query_len_bound, int32_t max_kv_len_bound,
                             void *out, void *stream);

/* Thread-local text of the last error on this thread ("" if none). */
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PA_H_ */
