/*
 * libsplash_attn -- one rank's share of decode attention over a paged latent
 * KV head, the merge of partial results, and the KV-page repack, for AMD
 * Instinct MI355X (gfx950).
 *
 * Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of
 * Attention with Seamless Handoff for LLM Serving" (weekinpapers.com); the
 * thelatestinai page is that paper's summary with its appendix tables
 * (thelatestinai.com).
 *
 * The method (SPLASH, weekinpapers page, Abstract) rests on attention with few
 * or no KV heads: every query head of a request attends to one shared latent
 * KV row per token, so where a request's cache lives is independent of how the
 * attention weights are sharded.  A layout is then only a choice of share
 * (thelatestinai page, Appendix Table 2 and its caption):
 *   TP            a slice of the query heads, every request's whole history;
 *   CP            a contiguous token range of every request, the tokens
 *                 split evenly over the ranks, emitted as partial output +
 *                 log-sum-exp and merged afterwards;
 *   DP-attention  the whole histories of the requests a rank owns, the
 *   and DOP       requests dealt to the ranks in equal numbers.
 * One call of splash_decode_attn computes any of these shares: a head range,
 * a token range and the set of requests in the batch passed to the call.
 * splash_lse_merge combines partial results over disjoint token ranges (the
 * cross-rank attention merge of CP; the zot.news page on Decode Token
 * Parallelism calls it the cross-node attention merge).  splash_kv_repack moves
 * whole KV pages between two pools, the state that must move when a layout
 * hands off (Abstract: moved in the background, handed off at a batch
 * boundary).
 *
 * Conventions for every call
 *  - All tensor pointers are device memory owned by the caller.  The library
 *    keeps no pointer after a call returns.
 *  - Calls are asynchronous on `stream` (0 = the null stream).
 *  - Return value: SPLASH_OK, or a negative error code.  Bad host arguments are
 *    rejected before anything is launched.  splash_last_error() returns a
 *    thread-local message for the last nonzero status.
 *  - Errors that only the device can see (a block-table or repack index
 *    outside its pool) never fault: the kernel treats the entry as described
 *    per call and raises a bit in the library's device error word, read with
 *    splash_device_errors().
 */
#ifndef SPLASH_ATTN_H
#define SPLASH_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLASH_OK 0
#define SPLASH_EINVAL (-1)        /* bad host argument; nothing launched */
#define SPLASH_EUNSUPPORTED (-2)  /* d_qk, d_v or page_size outside the built set */
#define SPLASH_EHIP (-3)          /* a HIP call or launch failed */

/* Device error bits (splash_device_errors). */
#define SPLASH_DEVERR_BAD_PAGE 1      /* decode: block-table entry outside [0, num_pages) */
#define SPLASH_DEVERR_REPACK_PAIR 2   /* repack: a pair was rejected (see splash_kv_repack) */
#define SPLASH_DEVERR_PARTIAL_RANGE 4 /* reserved; no longer raised (split-KV partials carry a
                                         power-of-two scale per row and column group, so no value is
                                         clamped) */

/* Shape of a paged latent-KV decode batch. */
typedef struct splash_desc {
  int32_t num_reqs;          /* B: requests in the batch (rows of q, block_table, seq_lens) */
  int32_t num_heads;         /* H: query heads per request (q's head stride) */
  int32_t d_qk;              /* dims of a latent KV row and of a query: 576 (512 latent + 64 rope) or 80 */
  int32_t d_v;               /* V = the first d_v dims of the same row: 512 or 64 */
  int32_t page_size;         /* tokens per KV page: 16, 32, 64, 128 or 256 */
  int32_t max_pages_per_req; /* block_table row stride */
  int32_t num_pages;         /* pages in the pool (valid physical page ids are [0, num_pages)) */
  int32_t num_splits;        /* split-KV chunks per request (equal token ranges); 0 = library's choice
                                (env SPLASH_NUM_SPLITS overrides).  While num_reqs x chunks x head
                                groups is below the CU count, each of two or more chunks is
                                computed by several workgroups over equal sub-ranges, and the
                                merge combines them all; 1 always runs unsplit.  Tuning
                                overrides, read on the host at each call: SPLASH_CHUNK_WORKGROUPS
                                (workgroups per forced chunk, 1..64), SPLASH_PLAN_HEADER (tiles a
                                segment start counts as in the device plan, 0..64) and
                                SPLASH_WG_HEADS (query heads per workgroup: 16, 32, 64 or 128) */
  float scale;               /* softmax scale applied to q.k, e.g. 1/sqrt(192) */
  int32_t num_kv_heads;      /* G latent KV heads per token (0 or 1: one); num_heads must be a multiple */
} splash_desc;

/*
 * Decode attention of one share.  For each request b < num_reqs and each head
 * h in [head_lo, head_hi):
 *   g = h / (num_heads / G)   (query heads share KV heads in contiguous groups)
 *   lo = max(tok_lo, 0), hi = min(tok_hi, seq_lens[b])
 *   k_t = kv_pages[block_table[b][t / page_size]][t % page_size][g][0 .. d_qk)
 *   v_t = k_t[0 .. d_v)
 *   out[b][h - head_lo][:] = sum_t softmax_t(scale * q[b][h] . k_t) v_t   over t in [lo, hi)
 *   lse[b][h - head_lo]    = log(sum_t exp(scale * q[b][h] . k_t))       (natural log)
 * An empty range gives out = 0 and lse = -inf.
 *
 *   q            bf16 [num_reqs][num_heads][d_qk], rows contiguous
 *   kv_pages     bf16 [num_pages][page_size][G][d_qk] (G = num_kv_heads; the
 *                premise is attention whose query heads share one or a few
 *                KV heads, weekinpapers
 *                page, Abstract: G = 1 is the latent-KV case, G > 1 groups
 *                the query heads onto a few shared KV heads)
 *   block_table  int32 [num_reqs][max_pages_per_req]; only the entries that
 *                cover [lo, hi) are read.  An entry outside [0, num_pages) is
 *                read as page 0 and raises SPLASH_DEVERR_BAD_PAGE.
 *   seq_lens     int32 [num_reqs], tokens in each request's cache
 *   out          fp32 [num_reqs][head_hi - head_lo][d_v]
 *   lse          fp32 [num_reqs][head_hi - head_lo], or NULL
 * The work is split into KV chunks (split-KV) when the share is too small to
 * fill the GPU: the kernel cuts the batch's tiles (32 tokens each) into
 * equal ranges from the device's seq_lens, a request inside one range is
 * written directly, and a request cut by range boundaries leaves partials in
 * a library-owned workspace that a merge kernel on the same stream combines.
 * A partial output is kept in fp16 divided by a power of two per row and
 * 128- or 256-column group (so any finite value keeps fp16's relative
 * precision), its LSE in fp32.  Every KV head the share touches is served by
 * the same launch (one decode kernel, plus one merge kernel when split).
 * Workspace: one per (device, stream), allocated on first need and grown on
 * demand (growth synchronises that stream, then frees the old buffer), freed
 * by splash_release_workspace.  Calls on different streams therefore never
 * share partials.  Under stream capture a call may use its stream's
 * workspace but not grow it: it then returns SPLASH_EINVAL (make one eager
 * call of the same share on the capturing stream first).  A captured graph
 * keeps the workspace's address, so growing that stream's workspace later or
 * calling splash_release_workspace invalidates such graphs.
 * Errors: SPLASH_EINVAL for null pointers, non-positive sizes, head range
 * outside [0, num_heads) or empty, tok_hi < tok_lo, num_kv_heads < 0 or not
 * dividing num_heads; SPLASH_EUNSUPPORTED for
 * (d_qk, d_v) not in {(576, 512), (80, 64)} or an unsupported page_size.
 */
int splash_decode_attn(const splash_desc* desc, const void* q, const void* kv_pages,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int32_t head_lo, int32_t head_hi, int32_t tok_lo, int32_t tok_hi,
                       float* out, float* lse, hipStream_t stream);

/*
 * splash_decode_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and kernels as splash_decode_attn,
 * but the split-KV workspace is the library's static per-device scratch
 * array of SPLASH_NOALLOC_SCRATCH_BYTES (72 MiB), which each GPU the
 * library runs on holds until the process ends.  The call makes no
 * hipMalloc / hipFree and no other allocating call, and records no
 * profiling events.
 *  - A share whose split-KV workspace (splash_decode_plan's
 *    workspace_bytes) exceeds the scratch is rejected with SPLASH_EINVAL
 *    before anything is launched.
 *  - Every call on a GPU shares that GPU's scratch: calls that overlap on
 *    one GPU (on different streams, or from different threads, while an
 *    earlier call's kernels still run) race and give wrong results.  Calls
 *    in one stream's order are safe.  Nothing in the scratch needs clearing
 *    between calls (every value a merge reads is written by the same call).
 */
#define SPLASH_NOALLOC_SCRATCH_BYTES ((int64_t)72 << 20)
int splash_decode_attn_noalloc(const splash_desc* desc, const void* q, const void* kv_pages,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t head_lo,
                               int32_t head_hi, int32_t tok_lo, int32_t tok_hi, float* out, float* lse,
                               hipStream_t stream);

/*
 * Merge n_parts partial results over disjoint token sets, per row:
 *   M = max_p lses[p][r] over finite entries
 *   lse_out[r] = M + log(sum_p exp(lses[p][r] - M))
 *   out[r][:]  = sum_p exp(lses[p][r] - lse_out[r]) * partials[p][r][:]
 * Parts with lse = -inf count for nothing: whatever their partial rows hold
 * (NaN included) does not reach the result, though the whole partials buffer
 * may be read; a row with no live part gets out = 0, lse_out = -inf.
 *   partials fp32 [n_parts][rows][d_v], lses fp32 [n_parts][rows]
 *   out fp32 [rows][d_v], lse_out fp32 [rows] or NULL
 * Errors: SPLASH_EINVAL for null pointers, n_parts < 1, rows < 0, d_v < 1,
 * d_v not a multiple of 4, or partials / out not 16-byte aligned.
 */
int splash_lse_merge(const float* partials, const float* lses, int32_t n_parts, int32_t rows,
                     int32_t d_v, float* out, float* lse_out, hipStream_t stream);

/*
 * Copy whole pages: for every pair (s, d) = (src_table[r][j], dst_table[r][j]),
 *   dst_pages[d][0 .. page_bytes) = src_pages[s][0 .. page_bytes)
 * The pair (-1, -1) is padding.  A pair with exactly one negative entry, or
 * an index outside [0, src_num_pages) / [0, dst_num_pages), is rejected: it
 * is not copied, it is counted in *err_count (device int32, incremented
 * atomically; may be NULL) and it raises SPLASH_DEVERR_REPACK_PAIR.  Pages are
 * copied bit-exactly.  Source and destination pages must not overlap, and no
 * destination page may appear twice.
 *   src_table, dst_table  int32 [n_reqs][max_pages]
 * Errors: SPLASH_EINVAL for null pointers, n_reqs < 0, max_pages < 0,
 * page_bytes < 1, negative pool sizes.
 */
int splash_kv_repack(const void* src_pages, const int32_t* src_table, void* dst_pages,
                     const int32_t* dst_table, int32_t n_reqs, int32_t max_pages, int64_t page_bytes,
                     int32_t src_num_pages, int32_t dst_num_pages, int32_t* err_count,
                     hipStream_t stream);

/* Thread-local message of the last call that returned nonzero ("" if none). */
const char* splash_last_error(void);

/*
 * Synchronise the current device, return its device error word (an OR of
 * SPLASH_DEVERR_* bits raised since the last clear) in *flags, and clear it if
 * `clear` is nonzero.  Returns SPLASH_OK or SPLASH_EHIP.
 */
int splash_device_errors(int32_t* flags, int32_t clear);

/* Free every split-KV workspace of the current device (synchronises it).
 * Graphs captured with a split-KV call on this device become invalid. */
int splash_release_workspace(void);

/*
 * The launch plan splash_decode_attn would use for this share, without
 * launching anything (a pure host function): split-KV partials per request
 * (forced chunks times the workgroups computing each),
 * workgroups per (request, chunk) along the heads (over all KV heads the
 * share touches), and workspace bytes.
 * Returns the same validation status as splash_decode_attn.
 */
int splash_decode_plan(const splash_desc* desc, int32_t head_lo, int32_t head_hi, int32_t tok_lo,
                       int32_t tok_hi, int32_t* num_splits, int32_t* head_groups,
                       int64_t* workspace_bytes);

/*
 * Launch profiling.  Between splash_profile_start() and splash_profile_stop()
 * the library brackets each kernel it launches with two HIP events on the
 * launch stream; stop() synchronises the current device and returns the
 * summed durations per kernel kind.  For measurement only: it adds two event
 * records per launch and is not thread-safe across concurrent callers.
 */
typedef struct splash_profile {
  int32_t decode_launches;     /* decode-attention kernels (one per splash_decode_attn) */
  int32_t merge_launches;      /* split-KV merge kernels inside splash_decode_attn */
  int32_t repack_launches;     /* splash_kv_repack kernels */
  double decode_ms;            /* summed kernel durations, milliseconds */
  double merge_ms;
  double repack_ms;
  int32_t lse_merge_launches;  /* splash_lse_merge kernels */
  double lse_merge_ms;
} splash_profile;

int splash_profile_start(void);
int splash_profile_stop(splash_profile* out);

/*
 * Peaks of the current GPU as measured (roofline context for the kernels
 * above; no part of the attention path):
 *  - mfma_bf16_tflops: dense v_mfma_f32_32x32x16_bf16 rate with one wave per
 *    SIMD on every CU, best of three ~2 ms runs;
 *  - mfma_clock_ghz: the shader clock during that run (s_memtime cycles
 *    over the 100 MHz s_memrealtime clock, averaged over workgroups);
 *  - hbm_read_gbps: streaming read rate over the caller's device buffer
 *    `buf` of `bytes` (>= 1 MiB, 16-byte aligned; use >= 1 GiB so that the
 *    256 MiB Infinity Cache does not serve it), best of three.
 * Synchronises `stream`.  Returns SPLASH_OK, SPLASH_EINVAL (bad arguments)
 * or SPLASH_EHIP.  Results live in a small per-device array the library
 * owns; concurrent calls on one device race on it.
 */
typedef struct splash_peaks {
  double mfma_bf16_tflops;
  double mfma_clock_ghz;
  double hbm_read_gbps;
} splash_peaks;

int splash_measure_peaks(const void* buf, int64_t bytes, splash_peaks* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLASH_ATTN_H */
