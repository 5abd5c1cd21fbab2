// Merge of partial attention results over disjoint token sets: the combine
// step of the CP layout (thelatestinai page, Appendix Table 2: each CP rank
// holds 1/T of every history) and of split-KV within one rank.  Per row:
//   M = max_p L_p,  L = M + log(sum_p exp(L_p - M)),  O = sum_p exp(L_p - L) O_p.
// HBM-bound: each partial value is read once, each output written once.
#include "common.h"

namespace splash {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 128;
constexpr int kBatch = 16;  // partial rows loaded before they are combined

// Parts of a row: either n_parts uniform parts at p * rows + row (the
// public merge and grid-mode split-KV), or the parts the decode kernel
// listed for the row's request (work-list split-KV).  at(row) resolves the
// row once; the result maps a part number to the partial row it lives in.
struct UniformRow {
  int n;
  int64_t row, rows;
  __device__ int64_t index(int p) const { return (int64_t)p * rows + row; }
};
struct UniformParts {
  int32_t n_parts, rows;
  __device__ UniformRow at(int64_t row) const { return {n_parts, row, rows}; }
};
struct ListedRow {
  int n, first, nfull, rem, hs, h;
  __device__ int64_t index(int p) const { return (int64_t)(p < nfull ? first + p : rem) * hs + h; }
};
struct ListedParts {
  const int4* req_info;  // {first full-chunk slot, full chunks, remainder slot or -1, 0}
  int32_t hs;
  __device__ ListedRow at(int64_t row) const {
    const int r = (int)row;  // rows = B * hs < 2^31
    const int4 info = req_info[r / hs];
    return {info.y + (info.z >= 0 ? 1 : 0), info.x, info.y, info.z, hs, r % hs};
  }
};

// One workgroup per row; each thread owns float4 columns.  The row's LSEs
// (a few floats) are read by every thread from L1/L2.
template <typename Parts>
__global__ void __launch_bounds__(kMergeThreads) lse_merge_kernel(const float* __restrict__ P,
                                                                  const float* __restrict__ L, Parts parts,
                                                                  int32_t d_v, float* __restrict__ out,
                                                                  float* __restrict__ lse_out) {
  const int64_t row = blockIdx.x;
  const auto rp = parts.at(row);
  const int n_parts = rp.n;
  const int c4n = d_v >> 2;
  floatx4* orow = (floatx4*)(out + row * d_v);
  if (n_parts <= kBatch) {
    // all LSEs in one round of loads, then all partial rows in one more
    int64_t pi[kBatch];
    float lp[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      pi[u] = u < n_parts ? rp.index(u) : 0;
      lp[u] = u < n_parts ? L[pi[u]] : -INFINITY;
    }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) M = fmaxf(M, lp[u]);
    if (M == -INFINITY) {  // no live part (NaN LSEs also end here: fmaxf ignores them)
      for (int c = threadIdx.x; c < c4n; c += kMergeThreads) orow[c] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (lse_out && threadIdx.x == 0) lse_out[row] = -INFINITY;
      return;
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) s += u < n_parts ? __expf(lp[u] - M) : 0.0f;
    const float lse = M + __logf(s);
    float w[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) w[u] = lp[u] != -INFINITY ? __expf(lp[u] - lse) : 0.0f;
    for (int c = threadIdx.x; c < c4n; c += kMergeThreads) {
      floatx4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        v[u] = w[u] != 0.0f ? ((const floatx4*)(P + pi[u] * d_v))[c] : floatx4{0.f, 0.f, 0.f, 0.f};
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kBatch; ++u) acc += w[u] * v[u];
      orow[c] = acc;
    }
    if (lse_out && threadIdx.x == 0) lse_out[row] = lse;
    return;
  }
  float M = -INFINITY;
  for (int p = 0; p < n_parts; ++p) M = fmaxf(M, L[rp.index(p)]);
  if (M == -INFINITY) {  // no live part (NaN LSEs also end here: fmaxf ignores them)
    for (int c = threadIdx.x; c < c4n; c += kMergeThreads) orow[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (lse_out && threadIdx.x == 0) lse_out[row] = -INFINITY;
    return;
  }
  float s = 0.0f;
  for (int p = 0; p < n_parts; ++p) s += __expf(L[rp.index(p)] - M);
  const float lse = M + __logf(s);
  for (int c = threadIdx.x; c < c4n; c += kMergeThreads) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    // kBatch parts' loads in flight at once; empty parts load nothing
    for (int p0 = 0; p0 < n_parts; p0 += kBatch) {
      floatx4 v[kBatch];
      float w[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int p = p0 + u;
        const int64_t pi = p < n_parts ? rp.index(p) : 0;
        const float lp = p < n_parts ? L[pi] : -INFINITY;
        w[u] = 0.0f;
        v[u] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (lp != -INFINITY) {
          w[u] = __expf(lp - lse);
          v[u] = ((const floatx4*)(P + pi * d_v))[c];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) acc += w[u] * v[u];
    }
    orow[c] = acc;
  }
  if (lse_out && threadIdx.x == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_lse_merge(const float* partials, const float* lses, int32_t n_parts, int32_t rows,
                            int32_t d_v, float* out, float* lse_out, hipStream_t stream, hipEvent_t e0,
                            hipEvent_t e1) {
  if (rows == 0) return hipSuccess;
  hipExtLaunchKernelGGL(lse_merge_kernel<UniformParts>, dim3(rows), dim3(kMergeThreads), 0, stream, e0, e1, 0,
                        partials, lses, UniformParts{n_parts, rows}, d_v, out, lse_out);
  return hipGetLastError();
}

hipError_t launch_lse_merge_segmented(const float* partials, const float* lses, const int4* req_info, int32_t rows,
                                      int32_t hs, int32_t d_v, float* out, float* lse_out, hipStream_t stream,
                                      hipEvent_t e0, hipEvent_t e1) {
  if (rows == 0) return hipSuccess;
  hipExtLaunchKernelGGL(lse_merge_kernel<ListedParts>, dim3(rows), dim3(kMergeThreads), 0, stream, e0, e1, 0,
                        partials, lses, ListedParts{req_info, hs}, d_v, out, lse_out);
  return hipGetLastError();
}

}  // namespace splash
