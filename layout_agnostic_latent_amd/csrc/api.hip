// Host side of libsplash_attn: argument validation, the launch plan
// (kernel variant, split-KV chunking), the split-KV workspace, the device
// error word and the exported C functions declared in include/splash_attn.h.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "splash_attn.h"
#include "common.h"

// Device error word: an OR of SPLASH_DEVERR_* bits.  Each device holds its
// own copy; its address is looked up per device.
__device__ int32_t g_splash_dev_err = 0;

namespace splash {
namespace {

constexpr int kMaxDevices = 64;
constexpr int kNumCUs = 256;  // MI355X: 256 compute units in 8 XCDs
constexpr int kMaxChunkTiles = 128;  // longest split-KV chunk (4,096 tokens)

// Message of the thread's last failing call (fixed size: reporting an error
// allocates nothing).
thread_local char t_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_last_error, sizeof(t_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(SPLASH_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Launch profiling: events bracketing each kernel while enabled.
enum LaunchKind { kDecode = 0, kMerge = 1, kRepack = 2, kLseMerge = 3 };
struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};
bool g_profiling = false;
std::vector<TimedLaunch> g_timed;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch(start_event, stop_event)`; while profiling, the events are
// attached to the kernel dispatch itself and kept for splash_profile_stop.
// Profiling is skipped for calls that must not allocate (the event pool and
// the launch list are host containers that may grow).
thread_local bool t_no_alloc = false;

template <typename F>
hipError_t timed(int kind, F&& launch) {
  if (!g_profiling || t_no_alloc) return launch(nullptr, nullptr);
  TimedLaunch t{kind, take_event(), take_event()};
  if (!t.start || !t.stop) return launch(nullptr, nullptr);
  hipError_t e = launch(t.start, t.stop);
  g_timed.push_back(t);
  return e;
}

// One split-KV workspace per (device, stream): calls on different streams
// never share one, so their decode and merge kernels cannot overwrite each
// other's partials.
struct Workspace {
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};
struct DeviceState {
  int32_t* dev_err = nullptr;  // address of g_splash_dev_err on this device
  std::vector<Workspace> ws;
};
std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

int current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (*dev < 0 || *dev >= kMaxDevices) return fail(SPLASH_EHIP, "device index %d out of range", *dev);
  return SPLASH_OK;
}

// Caller holds g_mu.
int device_error_word(int dev, int32_t** out) {
  DeviceState& st = g_dev[dev];
  if (!st.dev_err) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_splash_dev_err));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(g_splash_dev_err)");
    st.dev_err = (int32_t*)p;
  }
  *out = st.dev_err;
  return SPLASH_OK;
}

// Scratch memory of splash_decode_attn_noalloc: the split-KV workspace of
// callers that cannot allocate.  Each device holds its own copy for the life
// of the process; host code reaches it only through the per-device address
// from hipGetSymbolAddress (the array's name in host code is a host-side
// stand-in, not a device address).
constexpr size_t kScratchBytes = (size_t)72 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Caller holds g_mu.  Device address of `scratch` on `dev` (the current
// device), looked up once per device.
void* g_scratch[kMaxDevices] = {};
int scratch_address(int dev, void** out) {
  if (!g_scratch[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SPLASH_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SPLASH_OK;
}

// Caller holds g_mu.  The split-KV workspace of `stream` on `dev`, grown
// (never shrunk) to at least `bytes`.  Growing frees the old buffer after
// the stream's work on it is done, so it is refused while the stream is
// being captured into a graph (a captured kernel would keep the old
// address).
int ensure_workspace(int dev, hipStream_t stream, size_t bytes, void** out) {
  DeviceState& st = g_dev[dev];
  Workspace* w = nullptr;
  for (Workspace& x : st.ws)
    if (x.stream == stream) w = &x;
  if (!w) {
    st.ws.push_back(Workspace{stream, nullptr, 0});
    w = &st.ws.back();
  }
  if (w->bytes < bytes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return fail_hip(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(SPLASH_EINVAL,
                  "the split-KV workspace of this stream must grow to %zu bytes, which is not possible during "
                  "stream capture: make one eager call of the same share on this stream first, or use "
                  "splash_decode_attn_noalloc",
                  bytes);
    if (w->ptr) {
      e = hipStreamSynchronize(stream);  // kernels in flight may still use the old buffer
      if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
      e = hipFree(w->ptr);
      w->ptr = nullptr;
      w->bytes = 0;
      if (e != hipSuccess) return fail_hip(e, "hipFree(workspace)");
    }
    const size_t grown = bytes + bytes / 4;
    e = hipMalloc(&w->ptr, grown);
    if (e != hipSuccess) {
      w->ptr = nullptr;
      return fail_hip(e, "hipMalloc(split-KV workspace)");
    }
    w->bytes = grown;
  }
  *out = w->ptr;
  return SPLASH_OK;
}

int page_shift_of(int ps) {
  for (int s = 4; s <= 8; ++s)
    if (ps == (1 << s)) return s;
  return -1;
}

struct Plan {
  DecodeVariant variant;
  int head_groups;      // workgroups along the heads (KV heads touched x z_per_kv)
  int heads_per_group;  // head_tile * wh
  int kv_group;         // query heads per KV head
  int kv_first;         // first KV head the share touches
  int z_per_kv;         // head groups per KV head
  int grid_splits;      // split-KV chunks per request (grid mode: the blockIdx.x extent)
  int fixed_splits;     // > 0: every request cut into this many chunks
  int fixed_sub;        // ... each computed by this many workgroups (equal sub-ranges)
  int chunk_tiles;      // otherwise: 32-token tiles per chunk
  // Stream mode: the decode kernel cuts the batch's tiles into at most
  // `target` equal ranges per head group (the grid's x extent) from the real
  // lengths; each range leaves at most two partials.
  bool stream;
  int target;
  int header;           // tiles a segment start is counted as in the device plan
  int64_t workspace_bytes;
};

// The fixed cost of starting a segment (Q loads, pipeline fill and drain,
// the epilogue) in units of one tile of the variant's loop.  Measured on
// MI355X for 128-head groups by the decode time of the 64-request
// transition batch against the header: 0 / 3 / 5 / 8 / 12 / 16 tiles gave
// 242 / 237 / 236 / 232 / 226 / 230 us (best of five).  Narrower head
// groups have cheaper tiles, so the same start counts as more of them.
constexpr int kMinRangeTiles = 4;
int segment_header_tiles(int heads_per_group) {
  if (const char* env = getenv("SPLASH_PLAN_HEADER")) {
    const int v = atoi(env);
    if (v >= 0 && v <= 64) return v;
  }
  return heads_per_group >= 128 ? 12 : (heads_per_group >= 64 ? 20 : 32);
}

// Split-KV workspace layout (byte offsets; every part 256-byte aligned):
// `parts` partial rows of fp16 outputs, their {LSE, scale} records (one per
// column group), then (in stream mode) each request's merge record.
struct PartLayout {
  int64_t part_o, part_l, req_info, total;
};
int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }
PartLayout part_layout(int64_t parts, int64_t d_v, int64_t groups, int64_t records) {
  PartLayout w;
  w.part_o = 0;
  w.part_l = align256(w.part_o + parts * d_v * (int64_t)sizeof(uint16_t));
  w.req_info = align256(w.part_l + parts * groups * 8);
  w.total = align256(w.req_info + records * 16);
  return w;
}

// Latent KV heads of the pool (0 in the descriptor means one).
int kv_heads_of(const splash_desc* d) { return d->num_kv_heads > 0 ? d->num_kv_heads : 1; }

int validate_decode(const splash_desc* d, int32_t head_lo, int32_t head_hi, int32_t tok_lo, int32_t tok_hi) {
  if (!d) return fail(SPLASH_EINVAL, "desc is NULL");
  if (d->num_kv_heads < 0) return fail(SPLASH_EINVAL, "num_kv_heads = %d < 0", d->num_kv_heads);
  if (d->num_heads > 0 && d->num_heads % kv_heads_of(d))
    return fail(SPLASH_EINVAL, "num_heads = %d not a multiple of num_kv_heads = %d", d->num_heads, d->num_kv_heads);
  if (d->num_reqs < 0) return fail(SPLASH_EINVAL, "num_reqs = %d < 0", d->num_reqs);
  if (d->num_heads <= 0) return fail(SPLASH_EINVAL, "num_heads = %d <= 0", d->num_heads);
  if (d->max_pages_per_req <= 0) return fail(SPLASH_EINVAL, "max_pages_per_req = %d <= 0", d->max_pages_per_req);
  if (d->num_pages <= 0) return fail(SPLASH_EINVAL, "num_pages = %d <= 0", d->num_pages);
  if (d->num_splits < 0) return fail(SPLASH_EINVAL, "num_splits = %d < 0", d->num_splits);
  if (!(d->scale == d->scale) || d->scale == 1.0f / 0.0f || d->scale == -1.0f / 0.0f)
    return fail(SPLASH_EINVAL, "scale is not finite");
  if (head_lo < 0 || head_hi > d->num_heads || head_lo >= head_hi)
    return fail(SPLASH_EINVAL, "head range [%d, %d) not a non-empty subrange of [0, %d)", head_lo, head_hi,
                d->num_heads);
  if (tok_hi < tok_lo) return fail(SPLASH_EINVAL, "tok_hi = %d < tok_lo = %d", tok_hi, tok_lo);
  if (!((d->d_qk == 576 && d->d_v == 512) || (d->d_qk == 80 && d->d_v == 64)))
    return fail(SPLASH_EUNSUPPORTED, "(d_qk, d_v) = (%d, %d) not built; supported: (576, 512), (80, 64)", d->d_qk,
                d->d_v);
  if (page_shift_of(d->page_size) < 0)
    return fail(SPLASH_EUNSUPPORTED, "page_size = %d not in {16, 32, 64, 128, 256}", d->page_size);
  if ((int64_t)d->max_pages_per_req * d->page_size > (int64_t)1 << 30)
    return fail(SPLASH_EINVAL, "max_pages_per_req * page_size exceeds 2^30 tokens");
  return SPLASH_OK;
}

int make_plan(const splash_desc* d, int32_t head_lo, int32_t head_hi, int32_t tok_lo, int32_t tok_hi, Plan* p) {
  int rc = validate_decode(d, head_lo, head_hi, tok_lo, tok_hi);
  if (rc) return rc;
  const int hs = head_hi - head_lo;
  // KV heads the share touches, and the most query heads any one of them serves
  const int group = d->num_heads / kv_heads_of(d);
  const int kv_first = head_lo / group, kv_last = (head_hi - 1) / group;
  int slice = 0;
  for (int g = kv_first; g <= kv_last; ++g) {
    const int lo = head_lo > g * group ? head_lo : g * group;
    const int hi = head_hi < (g + 1) * group ? head_hi : (g + 1) * group;
    if (hi - lo > slice) slice = hi - lo;
  }
  const int wv_max = d->d_v / 32 >= 4 ? 4 : d->d_v / 32;
  // Heads per workgroup: 32 (4 waves split the V columns), 64 (2 head
  // groups x 2 column halves) or 128 (4 head groups).  SPLASH_WG_HEADS
  // overrides the choice (tuning).
  const bool latent = d->d_qk == 576 && d->d_v == 512;
  int wg_heads = slice <= 16 && latent ? 16 : (slice <= 32 ? 32 : (slice <= 64 ? 64 : 128));
  if (const char* env = getenv("SPLASH_WG_HEADS")) {
    const int v = atoi(env);
    if ((v == 16 && latent) || v == 32 || v == 64 || v == 128) wg_heads = v;
  }
  if (wg_heads == 16) {
    p->variant = {d->d_qk, d->d_v, 1, 4, 0, 16};
  } else if (wg_heads == 32) {
    p->variant = {d->d_qk, d->d_v, 1, wv_max, 0, 32};
  } else if (wg_heads == 64 && d->d_v / 32 >= 2 && d->d_qk == 576) {
    p->variant = {d->d_qk, d->d_v, 2, 2, 0, 32};
  } else {
    p->variant = {d->d_qk, d->d_v, 4, 1, 0, 32};
  }
  p->heads_per_group = p->variant.head_tile * p->variant.wh;
  p->kv_group = group;
  p->kv_first = kv_first;
  p->z_per_kv = (slice + p->heads_per_group - 1) / p->heads_per_group;
  p->head_groups = (kv_last - kv_first + 1) * p->z_per_kv;
  if (p->head_groups > 65535) return fail(SPLASH_EINVAL, "too many head groups (%d)", p->head_groups);

  // Longest token range any request can have in this share.
  const int64_t cap = (int64_t)d->max_pages_per_req * d->page_size;
  const int64_t lo = tok_lo > 0 ? tok_lo : 0;
  const int64_t hi = tok_hi < cap ? tok_hi : cap;
  const int64_t range = hi > lo ? hi - lo : 0;
  const int64_t max_tiles = range > 0 ? (hi + kTileTok - 1) / kTileTok - lo / kTileTok : 0;

  int forced = d->num_splits;
  if (forced == 0) {
    const char* env = getenv("SPLASH_NUM_SPLITS");
    if (env && *env) forced = atoi(env);
    if (forced < 0) forced = 0;
  }
  const int64_t base = (int64_t)d->num_reqs * p->head_groups;
  if (forced > 0) {
    // The caller's chunks; while two or more leave CUs idle (fewer
    // workgroups than CUs), each chunk is computed by several workgroups
    // over equal sub-ranges of its tiles, and the merge combines every
    // sub-range.  One chunk (num_splits = 1) always runs unsplit.
    int64_t sub = forced > 1 && base * forced > 0 ? kNumCUs / (base * forced) : 1;
    const char* env = forced > 1 ? getenv("SPLASH_CHUNK_WORKGROUPS") : nullptr;
    if (env) {
      const int v = atoi(env);
      if (v >= 1 && v <= 64) sub = v;
    }
    if (sub < 1) sub = 1;
    if (max_tiles > 0 && sub > (max_tiles + forced - 1) / forced) sub = (max_tiles + forced - 1) / forced;
    if (sub < 1) sub = 1;
    p->fixed_splits = forced;
    p->fixed_sub = (int)sub;
    p->chunk_tiles = 0;
    p->grid_splits = forced * sub <= 65535 ? (int)(forced * sub) : 65536;
  } else {
    // Aim for one round of about one workgroup per CU (each holds ~147 KiB
    // of LDS), with chunks of 4..128 tiles (128..4096 tokens): a chunk pays
    // a fixed cost (Q load, pipeline fill, the store of its partial output),
    // and every extra chunk adds a partial that the merge reads back.
    int64_t want = base > 0 ? (kNumCUs + base - 1) / base : 1;
    int64_t chunk = want > 0 ? (max_tiles + want - 1) / want : max_tiles;
    if (chunk < 4) chunk = 4;
    if (chunk > kMaxChunkTiles) chunk = kMaxChunkTiles;
    if (max_tiles == 0) chunk = 1;
    p->fixed_splits = 0;
    p->fixed_sub = 1;
    p->chunk_tiles = (int)chunk;
    p->grid_splits = max_tiles > 0 ? (int)((max_tiles + chunk - 1) / chunk) : 1;
  }
  if (p->grid_splits < 1) p->grid_splits = 1;
  if (p->grid_splits > 65535) return fail(SPLASH_EINVAL, "too many split-KV chunks (%d)", p->grid_splits);
  p->stream = false;
  p->target = 0;
  p->header = 0;
  // Longest run of tiles any one workgroup gets: forced splits cut each
  // request's tiles evenly, grid chunks are at most kMaxChunkTiles.
  p->variant.max_chunk_tiles = forced > 0 ? ((max_tiles + forced - 1) / forced + p->fixed_sub - 1) / p->fixed_sub
                                          : (max_tiles < kMaxChunkTiles ? max_tiles : kMaxChunkTiles);
  const int64_t rows = (int64_t)d->num_reqs * hs;
  const int64_t groups = d->d_v / partial_group_cols(d->d_v, p->variant.wv);
  if (p->grid_splits == 1) {
    p->workspace_bytes = 0;
  } else if (forced > 0 || d->num_reqs > kPlanMaxReqs) {
    p->workspace_bytes = part_layout((int64_t)p->grid_splits * rows, d->d_v, groups, 0).total;
  } else {
    // Requests may be shorter than the table's capacity (ragged batches):
    // the kernel cuts the batch's tiles (each request's run counted with a
    // header of `header` tiles for the cost of a segment start) into at
    // most `target` equal ranges per head group, of at least kMinRangeTiles
    // tiles, each leaving at most two partials; a range holds at most
    // ceil(B * (max_tiles + header) / target) + 1 tiles.  The device plan is
    // 32-bit, so longer batches take the grid plan.
    p->header = segment_header_tiles(p->heads_per_group);
    const int64_t tv_max = (int64_t)d->num_reqs * (max_tiles + p->header);
    p->target = (int)((kNumCUs + p->head_groups - 1) / p->head_groups);
    if (tv_max >= ((int64_t)1 << 31)) {
      p->workspace_bytes = part_layout((int64_t)p->grid_splits * rows, d->d_v, groups, 0).total;
      return SPLASH_OK;
    }
    p->stream = true;
    const int64_t per = (tv_max + p->target - 1) / p->target + 1;
    p->variant.max_chunk_tiles = per > kMinRangeTiles + 1 ? per : kMinRangeTiles + 1;
    p->workspace_bytes = part_layout(2 * (int64_t)p->target * hs, d->d_v, groups, d->num_reqs).total;
  }
  return SPLASH_OK;
}

}  // namespace

int report_error(int code, const char* msg) { return fail(code, "%s", msg); }

}  // namespace splash

using namespace splash;

extern "C" {

const char* splash_last_error(void) { return t_last_error; }

int splash_decode_plan(const splash_desc* desc, int32_t head_lo, int32_t head_hi, int32_t tok_lo, int32_t tok_hi,
                       int32_t* num_splits, int32_t* head_groups, int64_t* workspace_bytes) {
  Plan p;
  int rc = make_plan(desc, head_lo, head_hi, tok_lo, tok_hi, &p);
  if (rc) return rc;
  if (num_splits) *num_splits = p.grid_splits;
  if (head_groups) *head_groups = p.head_groups;
  if (workspace_bytes) *workspace_bytes = p.workspace_bytes;
  return SPLASH_OK;
}

}  // extern "C"

namespace splash {
namespace {

// Decode attention of the share's heads [head_lo, head_hi): one decode
// launch over every KV head the share touches (and one merge when split).
// `fixed_ws` (with `fixed_ws_bytes`) is a workspace to use instead of the
// stream's own, which is then never allocated or grown.
int decode_share(const splash_desc* desc, const void* q, const uint16_t* kv, const int32_t* block_table,
                 const int32_t* seq_lens, int32_t head_lo, int32_t head_hi, int32_t tok_lo, int32_t tok_hi,
                 float* out, float* lse, int dev, int32_t* dev_err, hipStream_t stream, void* fixed_ws = nullptr,
                 size_t fixed_ws_bytes = 0) {
  Plan p;
  int rc = make_plan(desc, head_lo, head_hi, tok_lo, tok_hi, &p);
  if (rc) return rc;
  const int hs = head_hi - head_lo;

  DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.kv = kv;
  a.kv_group = p.kv_group;
  a.kv_first = p.kv_first;
  a.z_per_kv = p.z_per_kv;
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.dev_err = dev_err;
  a.q_req_stride = (int64_t)desc->num_heads * desc->d_qk;
  a.kv_row = kv_heads_of(desc) * desc->d_qk;
  a.page_stride = (int64_t)desc->page_size * a.kv_row;
  a.max_pages = desc->max_pages_per_req;
  a.num_pages = desc->num_pages;
  a.page_shift = page_shift_of(desc->page_size);
  a.head_lo = head_lo;
  a.n_heads = hs;
  a.tok_lo = tok_lo;
  a.tok_hi = tok_hi;
  a.num_reqs = desc->num_reqs;
  a.fixed_splits = p.fixed_splits;
  a.fixed_sub = p.fixed_sub;
  a.chunk_tiles = p.chunk_tiles;
  a.scale_log2 = desc->scale * 1.4426950408889634f;
  a.out = out;
  a.lse = lse;

  const dim3 grid(p.stream ? p.target : p.grid_splits, p.stream ? 1 : desc->num_reqs, p.head_groups);
  if (p.grid_splits == 1) {
    hipError_t e = timed(kDecode, [&](hipEvent_t e0, hipEvent_t e1) {
      return launch_decode(p.variant, grid, a, stream, e0, e1);
    });
    if (e != hipSuccess) return fail_hip(e, "decode_attn launch");
    return SPLASH_OK;
  }
  // split-KV: partials in the workspace, then the merge writes the caller's rows
  void* ws;
  if (fixed_ws) {
    if ((size_t)p.workspace_bytes > fixed_ws_bytes)
      return fail(SPLASH_EINVAL, "this share needs %lld bytes of split-KV workspace, more than the %zu-byte scratch",
                  (long long)p.workspace_bytes, fixed_ws_bytes);
    ws = fixed_ws;
  } else if ((rc = ensure_workspace(dev, stream, (size_t)p.workspace_bytes, &ws))) {
    return rc;
  }
  const int64_t rows = (int64_t)desc->num_reqs * hs;
  const int gcols = partial_group_cols(desc->d_v, p.variant.wv);
  const int64_t groups = desc->d_v / gcols;
  const PartLayout w = p.stream ? part_layout(2 * (int64_t)p.target * hs, desc->d_v, groups, desc->num_reqs)
                                : part_layout((int64_t)p.grid_splits * rows, desc->d_v, groups, 0);
  const int sc_shift = __builtin_ctz((unsigned)gcols);
  char* base = (char*)ws;
  a.part_o = (uint16_t*)(base + w.part_o);
  a.part_l = (float*)(base + w.part_l);
  if (p.stream) {
    a.req_info = (int4*)(base + w.req_info);
    a.plan_target = p.target;
    a.plan_min_chunk = kMinRangeTiles;
    a.plan_header = p.header;
  } else {
    a.grid_partial = 1;
  }
  hipError_t e = timed(kDecode, [&](hipEvent_t e0, hipEvent_t e1) {
    return launch_decode(p.variant, grid, a, stream, e0, e1);
  });
  if (e != hipSuccess) return fail_hip(e, "decode_attn launch");
  e = timed(kMerge, [&](hipEvent_t e0, hipEvent_t e1) {
    return p.stream ? launch_split_merge_stream(a.part_o, a.part_l, sc_shift, a.req_info, (int32_t)rows, hs,
                                                desc->d_v, out, lse, stream, e0, e1)
                    : launch_split_merge(a.part_o, a.part_l, sc_shift, p.grid_splits, (int32_t)rows, desc->d_v,
                                         out, lse, stream, e0, e1);
  });
  if (e != hipSuccess) return fail_hip(e, "split-KV merge launch");
  return SPLASH_OK;
}

}  // namespace
}  // namespace splash

extern "C" {

int splash_decode_attn(const splash_desc* desc, const void* q, const void* kv_pages, const int32_t* block_table,
                       const int32_t* seq_lens, int32_t head_lo, int32_t head_hi, int32_t tok_lo, int32_t tok_hi,
                       float* out, float* lse, hipStream_t stream) {
  Plan p;
  int rc = make_plan(desc, head_lo, head_hi, tok_lo, tok_hi, &p);  // validates the descriptor and ranges
  if (rc) return rc;
  if (!q || !kv_pages || !block_table || !seq_lens || !out)
    return fail(SPLASH_EINVAL, "null tensor pointer (q, kv_pages, block_table, seq_lens and out are required)");
  if ((((uintptr_t)q) & 15) || (((uintptr_t)kv_pages) & 15) || (((uintptr_t)out) & 15))
    return fail(SPLASH_EINVAL, "q, kv_pages and out must be 16-byte aligned");
  if (desc->num_reqs == 0) return SPLASH_OK;
  int dev;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  int32_t* dev_err;
  if ((rc = device_error_word(dev, &dev_err))) return rc;
  return decode_share(desc, q, (const uint16_t*)kv_pages, block_table, seq_lens, head_lo, head_hi, tok_lo, tok_hi,
                      out, lse, dev, dev_err, stream);
}

int splash_decode_attn_noalloc(const splash_desc* desc, const void* q, const void* kv_pages,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t head_lo,
                               int32_t head_hi, int32_t tok_lo, int32_t tok_hi, float* out, float* lse,
                               hipStream_t stream) {
  Plan p;
  int rc = make_plan(desc, head_lo, head_hi, tok_lo, tok_hi, &p);
  if (rc) return rc;
  if (!q || !kv_pages || !block_table || !seq_lens || !out)
    return fail(SPLASH_EINVAL, "null tensor pointer (q, kv_pages, block_table, seq_lens and out are required)");
  if ((((uintptr_t)q) & 15) || (((uintptr_t)kv_pages) & 15) || (((uintptr_t)out) & 15))
    return fail(SPLASH_EINVAL, "q, kv_pages and out must be 16-byte aligned");
  if ((size_t)p.workspace_bytes > kScratchBytes)
    return fail(SPLASH_EINVAL, "this share needs %lld bytes of split-KV workspace, more than the %zu-byte scratch",
                (long long)p.workspace_bytes, kScratchBytes);
  if (desc->num_reqs == 0) return SPLASH_OK;
  int dev;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  int32_t* dev_err;
  if ((rc = device_error_word(dev, &dev_err))) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(dev, &ws))) return rc;
  t_no_alloc = true;
  rc = decode_share(desc, q, (const uint16_t*)kv_pages, block_table, seq_lens, head_lo, head_hi, tok_lo, tok_hi,
                    out, lse, dev, dev_err, stream, ws, kScratchBytes);
  t_no_alloc = false;
  return rc;
}

int splash_lse_merge(const float* partials, const float* lses, int32_t n_parts, int32_t rows, int32_t d_v,
                     float* out, float* lse_out, hipStream_t stream) {
  if (!partials || !lses || !out) return fail(SPLASH_EINVAL, "null tensor pointer (partials, lses, out)");
  if (n_parts < 1) return fail(SPLASH_EINVAL, "n_parts = %d < 1", n_parts);
  if (rows < 0) return fail(SPLASH_EINVAL, "rows = %d < 0", rows);
  if (d_v < 1 || (d_v & 3)) return fail(SPLASH_EINVAL, "d_v = %d must be a positive multiple of 4", d_v);
  if ((((uintptr_t)partials) & 15) || (((uintptr_t)out) & 15))
    return fail(SPLASH_EINVAL, "partials and out must be 16-byte aligned");
  hipError_t e;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    e = timed(kLseMerge, [&](hipEvent_t e0, hipEvent_t e1) {
      return launch_lse_merge(partials, lses, n_parts, rows, d_v, out, lse_out, stream, e0, e1);
    });
  }
  if (e != hipSuccess) return fail_hip(e, "lse_merge launch");
  return SPLASH_OK;
}

int splash_kv_repack(const void* src_pages, const int32_t* src_table, void* dst_pages, const int32_t* dst_table,
                     int32_t n_reqs, int32_t max_pages, int64_t page_bytes, int32_t src_num_pages,
                     int32_t dst_num_pages, int32_t* err_count, hipStream_t stream) {
  if (!src_pages || !src_table || !dst_pages || !dst_table)
    return fail(SPLASH_EINVAL, "null pointer (src_pages, src_table, dst_pages, dst_table)");
  if (n_reqs < 0 || max_pages < 0) return fail(SPLASH_EINVAL, "n_reqs = %d, max_pages = %d", n_reqs, max_pages);
  if (page_bytes < 1) return fail(SPLASH_EINVAL, "page_bytes = %lld < 1", (long long)page_bytes);
  if (src_num_pages < 0 || dst_num_pages < 0) return fail(SPLASH_EINVAL, "negative pool size");
  const int64_t n_pairs = (int64_t)n_reqs * max_pages;
  if (n_pairs > 0x7fffffff) return fail(SPLASH_EINVAL, "n_reqs * max_pages exceeds 2^31 - 1");
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  int32_t* dev_err;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((rc = device_error_word(dev, &dev_err))) return rc;
  hipError_t e = timed(kRepack, [&](hipEvent_t e0, hipEvent_t e1) {
    return launch_kv_repack(src_pages, src_table, dst_pages, dst_table, n_pairs, page_bytes, src_num_pages,
                            dst_num_pages, err_count, dev_err, stream, e0, e1);
  });
  if (e != hipSuccess) return fail_hip(e, "kv_repack launch");
  return SPLASH_OK;
}

int splash_device_errors(int32_t* flags, int32_t clear) {
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  int32_t* dev_err;
  if ((rc = device_error_word(dev, &dev_err))) return rc;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
  int32_t v = 0;
  e = hipMemcpy(&v, dev_err, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpy(device error word)");
  if (flags) *flags = v;
  if (clear) {
    const int32_t zero = 0;
    e = hipMemcpy(dev_err, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpy(clear device error word)");
  }
  return SPLASH_OK;
}

int splash_release_workspace(void) {
  int dev, rc;
  if ((rc = current_device(&dev))) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& st = g_dev[dev];
  if (st.ws.empty()) return SPLASH_OK;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");
  for (Workspace& w : st.ws) {
    if (w.ptr && e == hipSuccess) e = hipFree(w.ptr);
    w.ptr = nullptr;
  }
  st.ws.clear();
  if (e != hipSuccess) return fail_hip(e, "hipFree(workspace)");
  return SPLASH_OK;
}

int splash_profile_start(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_profiling = true;
  return SPLASH_OK;
}

int splash_profile_stop(splash_profile* out) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_profiling = false;
  splash_profile p;
  std::memset(&p, 0, sizeof(p));
  hipError_t e = hipDeviceSynchronize();
  int rc = SPLASH_OK;
  if (e != hipSuccess) rc = fail_hip(e, "hipDeviceSynchronize");
  for (const TimedLaunch& t : g_timed) {
    float ms = 0.0f;
    if (rc == SPLASH_OK && hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) ms = 0.0f;
    if (t.kind == kDecode) { p.decode_launches++; p.decode_ms += ms; }
    if (t.kind == kMerge) { p.merge_launches++; p.merge_ms += ms; }
    if (t.kind == kRepack) { p.repack_launches++; p.repack_ms += ms; }
    if (t.kind == kLseMerge) { p.lse_merge_launches++; p.lse_merge_ms += ms; }
    g_event_pool.push_back(t.start);
    g_event_pool.push_back(t.stop);
  }
  g_timed.clear();
  if (out) *out = p;
  return rc;
}

}  // extern "C"
