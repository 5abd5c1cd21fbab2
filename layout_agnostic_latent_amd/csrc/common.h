// Internal declarations shared by the host layer (api.hip) and the kernel
// translation units of libsplash_attn.  Not part of the public C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splash {

// Device error bits (the SPLASH_DEVERR_* values of the public header).
constexpr int32_t kDevErrBadPage = 1;
constexpr int32_t kDevErrRepackPair = 2;
constexpr int32_t kDevErrPartialRange = 4;

// Arguments of one decode-attention launch (passed by value to the kernel).
struct DecodeArgs {
  const uint16_t* q;         // bf16 [B][H][d_qk]
  const uint16_t* kv;        // bf16 [num_pages][page_size][G][d_qk] (G = 1: [num_pages][page_size][d_qk])
  const int32_t* bt;         // int32 [B][max_pages]
  const int32_t* seq_lens;   // int32 [B]
  float* out;                // fp32 [B][Hs][d_v], the caller's output (partial_out = 0), or
                             // fp16 [splits][B][Hs][d_v] split-KV partials (partial_out = 1)
  float* lse;                // fp32 [splits][B][Hs], may be null when splits = 1
  int32_t* dev_err;          // library device error word
  int64_t q_req_stride;      // H * d_qk
  int64_t page_stride;       // page_size * kv_row
  int32_t kv_row;            // elements per token in the pool: G * d_qk
  int64_t out_split_stride;  // B * Hs * d_v
  int64_t lse_split_stride;  // B * Hs
  int32_t max_pages;
  int32_t num_pages;
  int32_t page_shift;        // log2(page_size)
  int32_t head_lo;
  int32_t n_heads;           // Hs = head_hi - head_lo
  // Shared KV heads: query head h reads KV head h / kv_group.  blockIdx.z is
  // (KV head kv_first + z / z_per_kv, head group z % z_per_kv of that KV
  // head's part of the share).
  int32_t kv_group;          // query heads per KV head (H / G)
  int32_t kv_first;          // first KV head the share touches
  int32_t z_per_kv;          // head groups per KV head
  int32_t tok_lo;
  int32_t tok_hi;
  int32_t fixed_splits;      // > 0: every request is cut into this many chunks
  int32_t chunk_tiles;       // fixed_splits == 0: 32-token tiles per chunk
  int32_t partial_out;       // 1: out/lse are split-KV partials (merged afterwards); out holds fp16
  // Work-list mode (plan_target > 0): the chunks are cut from the device's
  // seq_lens inside the kernel.  Every workgroup computes the plan (one
  // chunk length for the batch so that its total tiles fill about
  // plan_target workgroups, clamped to [plan_min_chunk, plan_max_chunk];
  // full chunks numbered first, then one remainder chunk per request) and
  // takes item blockIdx.x; partial slot s holds rows [s][head][d_v]
  // (out_split_stride = Hs * d_v).  Workgroup (0, 0, 0) writes, per
  // request, {first full-chunk slot, full chunks, remainder slot or -1, 0}
  // to req_info for the merge.
  int32_t num_reqs;
  int32_t plan_target;
  int32_t plan_min_chunk;
  int32_t plan_max_chunk;
  int4* req_info;
  float scale_log2;          // scale * log2(e)
};

// Kernel variants: (d_qk, d_v) with WH waves along the heads (32 heads each)
// and WV waves along the V columns; max_chunk_tiles bounds the 32-token
// tiles any one workgroup of the launch processes (it selects how the DMA
// addresses are kept).
struct DecodeVariant {
  int d_qk, d_v, wh, wv;
  int64_t max_chunk_tiles;
};

// Records `msg` as the thread's last error (splash_last_error) and returns
// `code`; for entry points defined outside api.hip.
int report_error(int code, const char* msg);

// Each launcher takes two optional events that, when non-null, record the
// start and end of the kernel itself (hipExtLaunchKernelGGL), for profiling.
hipError_t launch_decode(const DecodeVariant& v, dim3 grid, const DecodeArgs& a, hipStream_t stream,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

hipError_t launch_lse_merge(const float* partials, const float* lses, int32_t n_parts, int32_t rows,
                            int32_t d_v, float* out, float* lse_out, hipStream_t stream,
                            hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Work-list mode handles batches of up to this many requests.
constexpr int kPlanMaxReqs = 8192;

// Merge of the work-list partials: row (b, h) combines the parts listed in
// req_info[b] (rows = B * hs).
// Merge of split-KV partials (fp16 O, fp32 LSE) into the caller's fp32
// rows: uniform parts at p * rows + row, or the parts listed per request.
// d_v a multiple of 8, at most 512.
hipError_t launch_split_merge(const uint16_t* partials, const float* lses, int32_t n_parts, int32_t rows,
                              int32_t d_v, float* out, float* lse_out, hipStream_t stream,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_split_merge_segmented(const uint16_t* partials, const float* lses, const int4* req_info,
                                        int32_t rows, int32_t hs, int32_t d_v, float* out, float* lse_out,
                                        hipStream_t stream, hipEvent_t ev_start = nullptr,
                                        hipEvent_t ev_stop = nullptr);

hipError_t launch_lse_merge_segmented(const float* partials, const float* lses, const int4* req_info, int32_t rows,
                                      int32_t hs, int32_t d_v, float* out, float* lse_out, hipStream_t stream,
                                      hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

hipError_t launch_kv_repack(const void* src, const int32_t* src_table, void* dst, const int32_t* dst_table,
                            int64_t n_pairs, int64_t page_bytes, int32_t src_num_pages,
                            int32_t dst_num_pages, int32_t* err_count, int32_t* dev_err,
                            hipStream_t stream, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

constexpr int kTileTok = 32;  // tokens per LDS tile of the decode kernel

}  // namespace splash
