/*
 * pa_testing.h -- test and measurement entry points of libpa.so.  Not part of
 * the op's contract (include/pa.h): forced kernel routing for parity tests,
 * a plan description for logs, per-kernel timing and a streaming-read probe
 * for benchmarks.  Conventions (device pointers, errors, streams) are those
 * of pa.h.
 */
#ifndef PA_TESTING_H_
#define PA_TESTING_H_

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Forced routing.  All zeros is the automatic choice pa_forward makes.
 * Every forced choice computes the same function; only the summation order
 * (and so the rounding) may differ. */
typedef struct {
  int32_t path;           /* 0 = auto (token_count <= batch_size -> decode kernel only,
                             else decode + prefill kernels); 1 = decode kernel for every
                             token; 2 = decode kernel for q_len == 1 requests, prefill
                             kernel for the rest (SEPARATE caches only, else
                             PA_ERR_UNSUPPORTED)                                        */
  int32_t split_tokens;   /* 0 = auto; else the decode KV split length in tokens, a
                             multiple of 64                                             */
  int32_t prefill_pieces; /* 0 = auto; else 1..4 workgroups sharing one prefill tile's
                             key range, merged on the device                            */
  int32_t prefill_kernel; /* 0 = auto; 1 = 4-wave prefill kernel (32 query rows per
                             wave); 2 = 8-wave kernel (16 rows per wave), head_size 256
                             with each cache smaller than 4 GiB; 3 = 8-wave kernel of 32
                             rows per wave (tiles of 256 rows), head_size 256 with
                             each cache smaller than 4 GiB; else PA_ERR_UNSUPPORTED     */
} pa_routing;

/* pa_forward_workspace_bytes / pa_forward with a forced routing (non-NULL). */
pa_status pa_forward_workspace_bytes_routed(const pa_attn_params *params, const pa_paged_kv *kv,
                                            const pa_routing *routing,
                                            int32_t max_query_len_bound,
                                            int32_t max_kv_len_bound, size_t *bytes);
pa_status pa_forward_routed(const pa_attn_params *params, const pa_paged_kv *kv,
                            const pa_routing *routing, const void *query,
                            const void *cos_cache, const void *sin_cache,
                            int32_t rotary_rows, int32_t rotary_dim,
                            int32_t max_query_len_bound, int32_t max_kv_len_bound,
                            void *workspace, size_t workspace_bytes, void *out, void *stream);

/* Host call: writes into `buf` (host, `len` bytes) a one-line description of
 * the launches the forward would make (path, grids, split length) for these
 * shapes, routing (NULL = automatic) and bounds. */
pa_status pa_describe_plan(const pa_attn_params *params, const pa_paged_kv *kv,
                           const pa_routing *routing, int32_t max_query_len_bound,
                           int32_t max_kv_len_bound, char *buf, size_t len);

/*
 * Per-kernel timing on the launch stream.  While enabled, the library
 * launches every kernel with a start/stop event pair that the dispatch
 * itself timestamps, and pa_timing_read() sums their elapsed times per stage
 * (synchronizing on the recorded events).  Enabling creates the events
 * (2 * max_launches); it is not meant for graph capture.
 */
enum { PA_STAGE_APPEND = 0, PA_STAGE_DECODE = 1, PA_STAGE_MERGE = 2, PA_STAGE_PREFILL = 3,
       PA_STAGE_PLAN = 4, PA_STAGE_PREFILL_MERGE = 5, PA_STAGE_Q_NORM = 6, PA_NUM_STAGES = 7 };
pa_status pa_timing_enable(int32_t max_launches);
pa_status pa_timing_disable(void);
pa_status pa_timing_read(int32_t stage, double *total_ms, int32_t *launches);

/*
 * Streaming read of `bytes` bytes at `src` (a multiple of 16384, 16-byte
 * aligned): every byte is loaded once, 16 bytes per lane and four loads in
 * flight per lane, and nothing is written (`sink`, 4 device bytes, is only
 * written if the data XOR to a fixed constant, which keeps the loads).
 * Timed by the caller with events on `stream`: the practical HBM read
 * ceiling the decode kernel's bandwidth is set beside.
 */
pa_status pa_bench_stream_read(const void *src, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_TESTING_H_ */
