// Merge of partial attention results over disjoint token sets: the combine
// step of the CP layout (thelatestinai page, Appendix Table 2: each CP rank
// holds 1/T of every history) and of split-KV within one rank.  Per row:
//   M = max_p L_p,  L = M + log(sum_p exp(L_p - M)),  O = sum_p exp(L_p - L) O_p.
// HBM-bound: each partial value is read once, each output written once.
//
// Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of
// Attention with Seamless Handoff for LLM Serving" (weekinpapers.com); the
// thelatestinai page is that paper's summary with its appendix tables
// (thelatestinai.com).
#include "common.h"

namespace splash {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;
constexpr int kLdsParts = 2048;  // parts whose weights are kept in LDS (more are recomputed)
constexpr int kBatch = 8;        // partial rows a thread loads before combining them

// Parts of a row: either n_parts uniform parts at p * rows + row (the
// public merge and grid-mode split-KV), or the parts of the row's request
// in the decode kernel's stream plan.  at(row) resolves the row once; the
// result maps a part number to the partial row it lives in, and `skip`
// marks a row the decode kernel wrote itself.
struct UniformRow {
  int n;
  int64_t row, rows;
  bool skip;
  __device__ int64_t index(int p) const { return (int64_t)p * rows + row; }
};
struct UniformParts {
  int32_t n_parts, rows;
  __device__ UniformRow at(int64_t row) const { return {n_parts, row, rows, false}; }
};
struct StreamRow {
  int n, first_slot, first_range, hs, h;
  bool skip;
  __device__ int64_t index(int p) const { return (int64_t)(p == 0 ? first_slot : first_range + p) * hs + h; }
};
struct StreamParts {
  const int4* req_info;  // the decode kernel's merge record of each request
  int32_t hs;
  __device__ StreamRow at(int64_t row) const {
    const int r = (int)row;  // rows = B * hs < 2^31
    const int4 info = req_info[r / hs];
    const int n = info.w == kStreamParts ? info.y - info.x + 1 : 0;
    return {n, info.z, info.x, hs, r % hs, info.w == kStreamDirect};
  }
};

// Block-wide reductions over kMergeThreads threads through LDS.
__device__ float block_max(float v, float* red) {
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}
__device__ float block_sum(float v, float* red) {
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < kMergeThreads / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

// One workgroup per output row.  The row's LSEs are loaded by all threads at
// once (one round of loads) and reduced through LDS; the weights
// exp(L_p - L) stay in LDS.  The partial rows are then read by G groups of
// threads (G = threads / float4 columns), each group taking every G-th
// part, kBatch loads in flight per thread; the groups' sums meet in LDS.
template <typename Parts>
__global__ void __launch_bounds__(kMergeThreads) lse_merge_kernel(const float* __restrict__ P,
                                                                  const float* __restrict__ L, Parts parts,
                                                                  int32_t d_v, float* __restrict__ out,
                                                                  float* __restrict__ lse_out) {
  __shared__ float w_s[kLdsParts];
  __shared__ floatx4 acc_s[kMergeThreads];
  __shared__ float red[kMergeThreads / 64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const auto rp = parts.at(row);
  const int n = rp.n;
  const int c4n = d_v >> 2;
  floatx4* orow = (floatx4*)(out + (int64_t)row * d_v);

  float m = -INFINITY;
  for (int p = tid; p < n; p += kMergeThreads) {
    const float l = L[rp.index(p)];
    if (p < kLdsParts) w_s[p] = l;
    m = fmaxf(m, l);
  }
  const float M = block_max(m, red);
  if (M == -INFINITY) {  // no live part (NaN LSEs also end here: fmaxf ignores them)
    for (int c = tid; c < c4n; c += kMergeThreads) orow[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (lse_out && tid == 0) lse_out[row] = -INFINITY;
    return;
  }
  float sum = 0.0f;
  for (int p = tid; p < n; p += kMergeThreads) sum += __expf((p < kLdsParts ? w_s[p] : L[rp.index(p)]) - M);
  const float lse = M + __logf(block_sum(sum, red));
  for (int p = tid; p < n && p < kLdsParts; p += kMergeThreads) w_s[p] = __expf(w_s[p] - lse);  // -inf -> 0
  __syncthreads();

  const int G = c4n < kMergeThreads ? kMergeThreads / c4n : 1;  // part groups
  const int g = tid / (c4n < kMergeThreads ? c4n : kMergeThreads);
  for (int c0 = 0; c0 < c4n; c0 += kMergeThreads / G) {
    const int c = c0 + tid % (kMergeThreads / G);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (g < G && c < c4n) {
      for (int p0 = g * kBatch; p0 < n; p0 += G * kBatch) {
        floatx4 v[kBatch];
        float w[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int p = p0 + u;
          const int64_t pi = p < n ? rp.index(p) : 0;
          w[u] = p >= n ? 0.0f : (p < kLdsParts ? w_s[p] : __expf(L[pi] - lse));
          v[u] = w[u] != 0.0f ? ((const floatx4*)(P + pi * d_v))[c] : floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) acc += w[u] * v[u];
      }
    }
    if (G > 1) {
      acc_s[tid] = acc;
      __syncthreads();
      if (g == 0 && c < c4n) {
        for (int j = 1; j < G; ++j) acc += acc_s[tid + j * c4n];
        orow[c] = acc;
      }
      __syncthreads();
    } else if (c < c4n) {
      orow[c] = acc;
    }
  }
  if (lse_out && tid == 0) lse_out[row] = lse;
}

// Row-wave merge: one wave per output row, each lane 8 columns (d_v <= 512,
// a multiple of 8).  The LSEs and partial rows of up to kSplitBatch parts are
// loaded in one round (no address depends on a loaded value: a part with LSE
// -inf, whose row may never have been written, is read but given no weight
// by a select, so garbage in it cannot reach the sums), then combined, with
// an online rescale of the sums when a row has more parts.  No LDS and no
// barrier: the row's cost is one round trip to memory.  T is the partial
// element type: fp16 (split-KV partials) or fp32 (the caller's partials).
constexpr int kSplitBatch = 16;
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

// 8 consecutive partial values of one lane.
template <typename T>
struct Row8;
template <>
struct Row8<_Float16> {
  halfx8 v;
  __device__ void load(const _Float16* p) { v = *(const halfx8*)p; }
  __device__ void zero() { v = halfx8{}; }
  __device__ float get(int k) const { return (float)v[k]; }
};
template <>
struct Row8<float> {
  floatx4 a, b;
  __device__ void load(const float* p) {
    a = ((const floatx4*)p)[0];
    b = ((const floatx4*)p)[1];
  }
  __device__ void zero() { a = b = floatx4{0.f, 0.f, 0.f, 0.f}; }
  __device__ float get(int k) const { return k < 4 ? a[k] : b[k - 4]; }
};

// A part's LSE and the factor its stored values carry, for the columns of
// one lane: the caller's partials (one LSE per row, values as given), or
// the split-KV partials (per row and column group of 2^shift columns a
// record {LSE, power of two the group's values were divided by}).
struct PlainRecs {
  const float* L;
  __device__ float2 at(int64_t pi, int) const { return float2{L[pi], 1.0f}; }
};
struct GroupRecs {
  const float2* R;
  int32_t shift;
  __device__ float2 at(int64_t pi, int col) const {
    return R[(pi << (9 - shift)) + (col >> shift)];  // d_v = 512 columns: 2^(9 - shift) groups
  }
};
struct GroupRecsAny {  // any d_v (a multiple of 2^shift)
  const float2* R;
  int32_t shift, groups;
  __device__ float2 at(int64_t pi, int col) const { return R[pi * groups + (col >> shift)]; }
};
template <typename T, typename Parts, typename Recs>
__global__ void __launch_bounds__(256) split_merge_kernel(const T* __restrict__ P, Recs recs, Parts parts,
                                                          int32_t rows, int32_t d_v, float* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const auto rp = parts.at(row);
  if (rp.skip) return;
  const int n = rp.n;
  const int c = lane * 8;
  const bool active = c < d_v;
  const int cc = active ? c : 0;  // lanes past d_v read column 0's record
  float M = -INFINITY, S = 0.0f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < n; p0 += kSplitBatch) {
    float l[kSplitBatch], psc[kSplitBatch];
    Row8<T> v[kSplitBatch];
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u) {
      const bool live = p0 + u < n;
      const int64_t pi = live ? rp.index(p0 + u) : 0;
      const float2 rec = live ? recs.at(pi, cc) : float2{-INFINITY, 1.0f};
      l[u] = rec.x;
      psc[u] = rec.y;
      if (live && active) v[u].load(P + pi * d_v + c);
      else v[u].zero();
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u) mb = fmaxf(mb, l[u]);
    if (mb == -INFINITY) continue;  // no live part so far
    const float sc = __expf(M - mb);  // 0 while M is -inf
    S *= sc;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= sc;
#pragma unroll
    for (int u = 0; u < kSplitBatch; ++u) {
      if (l[u] != -INFINITY) {
        const float w = __expf(l[u] - mb);
        const float wv = w * psc[u];
        S += w;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += wv * v[u].get(k);
      }
    }
    M = mb;
  }
  floatx4* orow = (floatx4*)(out + row * d_v + c);
  if (M == -INFINITY) {  // every part empty
    if (active) {
      orow[0] = floatx4{0.f, 0.f, 0.f, 0.f};
      orow[1] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    if (lse_out && lane == 0) lse_out[row] = -INFINITY;
    return;
  }
  const float inv = 1.0f / S;
  if (active) {
    orow[0] = floatx4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    orow[1] = floatx4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (lse_out && lane == 0) lse_out[row] = M + __logf(S);
}

// The fp16 split-KV merge with the record layout of the decode kernel.
template <typename Parts>
hipError_t launch_fp16_merge(const uint16_t* partials, const float* recs, int32_t shift, Parts parts, int32_t rows,
                             int32_t d_v, float* out, float* lse_out, hipStream_t stream, hipEvent_t e0,
                             hipEvent_t e1) {
  if (d_v == 512)
    hipExtLaunchKernelGGL((split_merge_kernel<_Float16, Parts, GroupRecs>), dim3((rows + 3) / 4), dim3(256), 0,
                          stream, e0, e1, 0, (const _Float16*)partials, GroupRecs{(const float2*)recs, shift}, parts,
                          rows, d_v, out, lse_out);
  else
    hipExtLaunchKernelGGL((split_merge_kernel<_Float16, Parts, GroupRecsAny>), dim3((rows + 3) / 4), dim3(256), 0,
                          stream, e0, e1, 0, (const _Float16*)partials,
                          GroupRecsAny{(const float2*)recs, shift, d_v >> shift}, parts, rows, d_v, out, lse_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split_merge(const uint16_t* partials, const float* recs, int32_t sc_shift, int32_t n_parts,
                              int32_t rows, int32_t d_v, float* out, float* lse_out, hipStream_t stream,
                              hipEvent_t e0, hipEvent_t e1) {
  if (rows == 0) return hipSuccess;
  return launch_fp16_merge(partials, recs, sc_shift, UniformParts{n_parts, rows}, rows, d_v, out, lse_out, stream,
                           e0, e1);
}

hipError_t launch_split_merge_stream(const uint16_t* partials, const float* recs, int32_t sc_shift,
                                     const int4* req_info, int32_t rows, int32_t hs, int32_t d_v, float* out,
                                     float* lse_out, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  if (rows == 0) return hipSuccess;
  return launch_fp16_merge(partials, recs, sc_shift, StreamParts{req_info, hs}, rows, d_v, out, lse_out, stream, e0,
                           e1);
}

hipError_t launch_lse_merge(const float* partials, const float* lses, int32_t n_parts, int32_t rows,
                            int32_t d_v, float* out, float* lse_out, hipStream_t stream, hipEvent_t e0,
                            hipEvent_t e1) {
  if (rows == 0) return hipSuccess;
  if (d_v % 8 == 0 && d_v <= 512) {
    // one wave per row, every load of a row in one round
    hipExtLaunchKernelGGL((split_merge_kernel<float, UniformParts, PlainRecs>), dim3((rows + 3) / 4), dim3(256), 0,
                          stream, e0, e1, 0, partials, PlainRecs{lses}, UniformParts{n_parts, rows}, rows, d_v, out,
                          lse_out);
    return hipGetLastError();
  }
  hipExtLaunchKernelGGL(lse_merge_kernel<UniformParts>, dim3(rows), dim3(kMergeThreads), 0, stream, e0, e1, 0,
                        partials, lses, UniformParts{n_parts, rows}, d_v, out, lse_out);
  return hipGetLastError();
}

}  // namespace splash
