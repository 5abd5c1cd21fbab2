// Device helpers shared by the decode kernels: vector types, the LDS tile
// layout and its DMA, and the balanced split-KV plan.  Included by one
// translation unit per kernel family (everything here is internal to it).
#pragma once

#include <climits>

#include "common.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kPageLds = 4096;  // page ids of a chunk staged in LDS (16 KiB)
constexpr int kVPages = 4;      // VGPRs of page ids per lane: chunks of up to 256 pages
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p = exp2(s - m) stays <= 256

// LDS tile layout ("slabs"): the 16-byte chunk c of tile row r lives at
//   (c / 8) * SLAB_B + r * 128 + ((c % 8) ^ row_swizzle(r)) * 16,
// i.e. each group of 8 chunks (128 B) of all 32 rows forms a 4-KiB slab.
// One DMA instruction fills 8 rows x 128 B of one slab, so a lane's HBM
// offset within a tile depends only on the lane and on the parity of the
// instruction's row group.  The XOR makes the ds_read_b128 of 16 rows at one
// chunk, and the transposing reads of 4 rows x 4 chunks, hit distinct banks.
__device__ __forceinline__ uint32_t row_swizzle(uint32_t row) {
  return ((row >> 2) & 3u) | (((row >> 1) & 1u) << 2);
}

// One 16-byte-per-lane global -> LDS copy from a wave-uniform 64-bit base
// (SGPRs) plus a per-lane 32-bit offset; lane i's 16 bytes land at
// lds_addr + 16*i.  Issued from inline asm so that the compiler does not add
// a vmcnt(0) before every LDS read; completion is tracked by wait_vmcnt().
// Every KV byte is read once per call, so the load is non-temporal (nt):
// the stream does not displace reusable lines from the caches.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)),
               "v"(voff), "s"(sbase)
               : "memory");
}

// The same copy for instruction I of a wave's row group, `lds_addr` being
// that instruction's LDS destination: the 128-byte step between the
// instructions' global addresses is the immediate offset, which the
// hardware adds to the LDS address too, so m0 is lowered by it.
template <int I>
__device__ __forceinline__ void lds_dma16_imm(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3 nt" ::"{m0}"(lds_addr - 128 * I), "v"(voff),
               "s"(sbase), "n"(128 * I)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// max(x[l], x[l ^ 32]) for every lane l: lanes l and l^32 hold the two halves
// of one head's 32 scores.  v_permlane32_swap exchanges the two wave halves
// in the VALU, without an LDS round trip.
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}


// Balanced split-KV plan, computed by every workgroup from the device's
// seq_lens (the host knows only the block table's capacity, which for a
// ragged batch says little about the work).  Every request with work
// occupies a run of "virtual" tiles: a header of plan_header tiles (the
// fixed cost of starting a segment: Q loads, pipeline fill and drain, the
// epilogue, counted in tiles; no header when every request with work has
// the same length, whose equal ranges then fall on request boundaries)
// followed by its T_r real tiles, in request order.  The runs, TV tiles in
// all, are cut into ranges of L = ceil(TV / N)
// tiles, N = min(plan_target, ceil(TV / plan_min_chunk)); workgroup w takes
// [w L, (w + 1) L).  It walks the requests whose real tiles its range
// covers: a request inside one range is written directly to the caller's
// output; a request cut by a range boundary leaves one partial per range it
// touches, in slot w for the range's first segment and plan_target + w for
// its last (so a uniform batch's partials are contiguous, by range).
// Workgroup (0, 0, 0) writes each request's merge record (stream_record).
// All plan arithmetic is 32-bit: the host uses this plan only while every
// virtual tile count fits in 31 bits.
struct StreamPlan {
  int A, E;  // this workgroup's virtual tiles [A, E)
  int r;     // request whose run holds tile A (-1: nothing to do)
  int V;     // first virtual tile of request r's run
  int h;     // header tiles of every run
  int n0;    // real tiles of request r (> 0), so the segment walk need not load it again
};

struct StreamCut {
  int N, L;  // ranges and their length in virtual tiles
};
__device__ __forceinline__ StreamCut stream_cut(int TV, const DecodeArgs& a) {
  if (TV <= 0) return StreamCut{0, 1};
  const int n = (TV + a.plan_min_chunk - 1) / a.plan_min_chunk;
  const int N = n < a.plan_target ? n : a.plan_target;
  const int L = (TV + N - 1) / N;
  return StreamCut{(TV + L - 1) / L, L};
}
// Merge record of a request whose run is the virtual tiles [v0, v1).
__device__ __forceinline__ int4 stream_record(int v0, int v1, int header, StreamCut c, int slots) {
  if (v1 == v0) return make_int4(0, 0, 0, kStreamEmpty);
  const int wa = (v0 + header) / c.L, wb = (v1 - 1) / c.L;  // ranges of its first and last real tile
  if (wa == wb) return make_int4(wa, wb, 0, kStreamDirect);
  // range wa starts inside the run (header included): the request is its first segment
  return make_int4(wa, wb, wa * c.L >= v0 ? wa : slots + wa, kStreamParts);
}

// Tiles of request r's clipped range (scalar loads).
__device__ __forceinline__ int request_tiles(const DecodeArgs& a, int r) {
  const int lo = max(a.tok_lo, 0);
  const int cap = a.max_pages << a.page_shift;
  const int h = min(min(a.tok_hi, ((const int32_t __attribute__((address_space(4)))*)a.seq_lens)[r]), cap);
  return h > lo ? (h + kTileTok - 1) / kTileTok - lo / kTileTok : 0;
}

// The plan for batches of at most 64 requests, by every wave on its own:
// request r's run length in lane r, sums and prefixes as wave reductions
// (no LDS, no barrier).
__device__ StreamPlan stream_plan_wave(const DecodeArgs& a) {
  const int lane = threadIdx.x & 63;
  const int lo = max(a.tok_lo, 0);
  const int cap = a.max_pages << a.page_shift;
  int nt = 0;  // tiles of request `lane`
  if (lane < a.num_reqs) {
    const int hi = min(min(a.tok_hi, a.seq_lens[lane]), cap);
    nt = hi > lo ? (hi + kTileTok - 1) / kTileTok - lo / kTileTok : 0;
  }
  int tmax = nt, tmin = nt > 0 ? nt : INT_MAX;
  for (int d = 32; d >= 1; d >>= 1) {
    tmax = max(tmax, __shfl_xor(tmax, d, 64));
    tmin = min(tmin, __shfl_xor(tmin, d, 64));
  }
  const int header = tmin == tmax ? 0 : a.plan_header;
  const int nv = nt > 0 ? nt + header : 0;  // virtual tiles of request `lane`
  int incl = nv;
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  const int excl = incl - nv;
  const int TV = __shfl(incl, 63, 64);
  const StreamCut c = stream_cut(TV, a);
  if (blockIdx.x == 0 && blockIdx.z == 0 && threadIdx.x < 64 && lane < a.num_reqs)
    a.req_info[lane] = stream_record(excl, incl, header, c, a.plan_target);
  const int w = blockIdx.x;
  if (w >= c.N) return StreamPlan{0, 0, -1, 0, 0, 0};
  const int A = w * c.L, E = min(A + c.L, TV);  // the last range ends with the batch
  // the first run ending past A holds tile A (empty requests have no run)
  const unsigned long long bal = __ballot(lane < a.num_reqs && incl > A);
  const int r = __ffsll((long long)bal) - 1;
  return StreamPlan{A, E, r, __builtin_amdgcn_readlane(excl, r), header, __builtin_amdgcn_readlane(nt, r)};
}

// The same plan for batches of up to kPlanMaxReqs requests, by the
// workgroup: thread t sums the runs of requests [t * per, t * per + per), a
// wave scan and the waves' totals through LDS give every prefix.  `scratch`
// (LDS, >= 3 NT / 64 + 3 ints) is free again on return.
template <int NT>
__device__ StreamPlan stream_plan_block(const DecodeArgs& a, int32_t* scratch) {
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (a.num_reqs + NT - 1) / NT;
  // equal lengths?  (max and min over the requests with work)
  int tmax = 0, tmin = INT_MAX;
  for (int k = 0; k < per; ++k) {
    const int r = tid * per + k;
    if (r < a.num_reqs) {
      const int t = request_tiles(a, r);
      tmax = max(tmax, t);
      if (t > 0) tmin = min(tmin, t);
    }
  }
  for (int d = 32; d >= 1; d >>= 1) {
    tmax = max(tmax, __shfl_xor(tmax, d, 64));
    tmin = min(tmin, __shfl_xor(tmin, d, 64));
  }
  int* wsum = scratch;                // [NWV]
  int* found = scratch + NWV;         // {r, V, tiles of r}
  int* ext = scratch + NWV + 3;       // [NWV][2]: each wave's max and min
  if (lane == 0) {
    ext[2 * wave] = tmax;
    ext[2 * wave + 1] = tmin;
  }
  __syncthreads();
  for (int w = 0; w < NWV; ++w) {
    tmax = max(tmax, ext[2 * w]);
    tmin = min(tmin, ext[2 * w + 1]);
  }
  const int header = tmin == tmax ? 0 : a.plan_header;
  auto run = [&](int r) {
    const int t = request_tiles(a, r);
    return t > 0 ? t + header : 0;
  };
  int mine = 0;
  for (int k = 0; k < per; ++k) {
    const int r = tid * per + k;
    if (r < a.num_reqs) mine += run(r);
  }
  int incl = mine;
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  if (lane == 63) wsum[wave] = incl;
  if (tid == 0) found[0] = -1;
  __syncthreads();
  int before = 0, TV = 0;
  for (int w = 0; w < NWV; ++w) {
    if (w < wave) before += wsum[w];
    TV += wsum[w];
  }
  const StreamCut c = stream_cut(TV, a);
  const int w = blockIdx.x;
  const bool active = w < c.N;
  const int A = w * c.L, E = min(A + c.L, TV);  // the last range ends with the batch
  const bool writer = blockIdx.x == 0 && blockIdx.z == 0;
  int v = before + incl - mine;  // first virtual tile of this thread's first request
  for (int k = 0; k < per; ++k) {
    const int r = tid * per + k;
    if (r >= a.num_reqs) break;
    const int nv = run(r);
    if (writer) a.req_info[r] = stream_record(v, v + nv, header, c, a.plan_target);
    if (active && v <= A && A < v + nv) {  // exactly one run holds tile A
      found[0] = r;
      found[1] = v;
      found[2] = nv - header;
    }
    v += nv;
  }
  __syncthreads();
  const StreamPlan p{A, E, active ? found[0] : -1, found[1], header, found[2]};
  __syncthreads();
  return p;
}

}  // namespace
}  // namespace splash
