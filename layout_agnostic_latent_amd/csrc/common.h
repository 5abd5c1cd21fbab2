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
constexpr int32_t kDevErrPartialRange = 4;  // reserved: no longer raised

// Arguments of one decode-attention launch (passed by value to the kernel).
struct DecodeArgs {
  const uint16_t* q;         // bf16 [B][H][d_qk]
  const uint16_t* kv;        // bf16 [num_pages][page_size][G][d_qk] (G = 1: [num_pages][page_size][d_qk])
  const int32_t* bt;         // int32 [B][max_pages]
  const int32_t* seq_lens;   // int32 [B]
  float* out;                // the caller's output, fp32 [B][Hs][d_v]
  float* lse;                // the caller's LSE, fp32 [B][Hs], or null
  // Split-KV partials (when the share is split): row p of the partial
  // buffers is one head's partial result.  part_o holds, per column group
  // of partial_group_cols columns, O / 2^e in fp16 (e >= 0 keeps it inside
  // the fp16 range); part_l holds per row and group the record {LSE, 2^e}.
  // Grid mode: row (split * B + b) * Hs + h; stream mode: row slot * Hs + h.
  uint16_t* part_o;          // fp16 [rows][d_v]
  float* part_l;             // float2 [rows][d_v / partial_group_cols]
  int32_t* dev_err;          // library device error word
  int64_t q_req_stride;      // H * d_qk
  int64_t page_stride;       // page_size * kv_row
  int32_t kv_row;            // elements per token in the pool: G * d_qk
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
  int32_t num_reqs;          // B
  // Grid mode (plan_target == 0): workgroup (x, b) takes chunk x of request
  // b; every chunk is a partial when grid_partial, else the whole range goes
  // to the caller's output.
  int32_t fixed_splits;      // > 0: every request is cut into this many chunks
  int32_t fixed_sub;         // fixed_splits > 0: workgroups per chunk, over equal sub-ranges of it
  int32_t chunk_tiles;       // fixed_splits == 0: 32-token tiles per chunk
  int32_t grid_partial;
  // Stream mode (plan_target > 0): the batch's tiles cut into equal ranges
  // on the device (stream_plan_*), at most plan_target per head group;
  // req_info[b] is request b's merge record (stream_record: first and last
  // range, slot of the first segment, kind).
  int32_t plan_target;
  int32_t plan_min_chunk;
  int32_t plan_header;       // tiles a segment start is counted as
  int4* req_info;
  float scale_log2;          // scale * log2(e)
};

// Merge record of a request in stream mode, {x, y, z, w}: its tiles lie in
// ranges x .. y; its first part is in slot z, part k > 0 in slot x + k;
// w = kStreamParts (merge the parts), kStreamDirect (written by the decode
// kernel) or kStreamEmpty (no tile: O = 0, LSE = -inf).
constexpr int32_t kStreamParts = 0;
constexpr int32_t kStreamDirect = 1;
constexpr int32_t kStreamEmpty = 2;

// Kernel variants: (d_qk, d_v) with WH waves along the heads (32 heads each)
// and WV waves along the V columns; max_chunk_tiles bounds the 32-token
// tiles any one workgroup of the launch processes (it selects how the DMA
// addresses are kept).
struct DecodeVariant {
  int d_qk, d_v, wh, wv;
  int64_t max_chunk_tiles;
  int head_tile;  // heads per MFMA tile: 32 (32x32x16 kernel) or 16 (16x16x32 kernel, wh = 1, wv = 4)
};

// Records `msg` as the thread's last error (splash_last_error) and returns
// `code`; for entry points defined outside api.hip.
int report_error(int code, const char* msg);

// Each launcher takes two optional events that, when non-null, record the
// start and end of the kernel itself (hipExtLaunchKernelGGL), for profiling.
hipError_t launch_decode16(const DecodeVariant& v, dim3 grid, const DecodeArgs& a, hipStream_t stream,
                           hipEvent_t e0, hipEvent_t e1);
hipError_t launch_decode(const DecodeVariant& v, dim3 grid, const DecodeArgs& a, hipStream_t stream,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

hipError_t launch_lse_merge(const float* partials, const float* lses, int32_t n_parts, int32_t rows,
                            int32_t d_v, float* out, float* lse_out, hipStream_t stream,
                            hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Stream mode handles batches of up to this many requests.
constexpr int kPlanMaxReqs = 8192;

// Merge of split-KV partials (fp16 O divided by a power of two per row and
// column group of 2^sc_shift columns; `recs` [rows][groups] holds the
// part's {LSE, power of two} for each group) into the caller's fp32 rows
// (rows = B * hs).  Grid mode: n_parts uniform parts at p * rows + row.
// Stream mode (req_info): row (b, h) combines the parts of request b's
// record; rows the decode kernel wrote directly are left alone.  d_v a
// multiple of 8, at most 512.
hipError_t launch_split_merge(const uint16_t* partials, const float* recs, int32_t sc_shift, int32_t n_parts,
                              int32_t rows, int32_t d_v, float* out, float* lse_out, hipStream_t stream,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_split_merge_stream(const uint16_t* partials, const float* recs, int32_t sc_shift,
                                     const int4* req_info, int32_t rows, int32_t hs, int32_t d_v, float* out,
                                     float* lse_out, hipStream_t stream, hipEvent_t ev_start = nullptr,
                                     hipEvent_t ev_stop = nullptr);

// Columns per scale group of a decode variant's split-KV partials (its
// epilogue stores a row in passes of up to 8 blocks of 32 columns per wave).
constexpr int partial_group_cols(int d_v, int wv) { return (d_v / 32 / wv < 8 ? d_v / 32 / wv : 8) * 32; }

hipError_t launch_kv_repack(const void* src, const int32_t* src_table, void* dst, const int32_t* dst_table,
                            int64_t n_pairs, int64_t page_bytes, int32_t src_num_pages,
                            int32_t dst_num_pages, int32_t* err_count, int32_t* dev_err,
                            hipStream_t stream, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

constexpr int kTileTok = 32;  // tokens per LDS tile of the decode kernel

}  // namespace splash
