// KV-page repack: whole pages gathered through a source block table and
// scattered through a destination table.  This is the state that moves when
// SPLASH hands a request's cache to a new owner at a layout switch
// (weekinpapers page, Abstract: the state not already in place is moved in the
// background and handed off at a batch boundary).  A pure bandwidth copy;
// bit-exact by construction.
//
// Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of
// Attention with Seamless Handoff for LLM Serving" (weekinpapers.com); the
// thelatestinai page is that paper's summary with its appendix tables
// (thelatestinai.com).
#include "common.h"

namespace splash {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 512 threads x 9 loads of 16 bytes: a whole 73,728-byte page (64 tokens x
// 576 bf16) is in flight per workgroup before its stores.  With few pages
// to move (a 16-request handoff: 512 pages, two workgroups per CU) the copy
// is bound by bytes in flight per CU; 256 x 6 reached 4.0 TB/s there, this
// shape 5.8 TB/s (read + write).
constexpr int kRepackThreads = 512;
constexpr int kUnroll = 9;  // 16-byte loads in flight per thread before their stores

// One workgroup per (request, page) pair of the tables.
__global__ void __launch_bounds__(kRepackThreads) kv_repack_kernel(const uint8_t* __restrict__ src,
                                                                   const int32_t* __restrict__ st,
                                                                   uint8_t* __restrict__ dst,
                                                                   const int32_t* __restrict__ dt,
                                                                   int64_t page_bytes, int32_t ns, int32_t nd,
                                                                   int32_t* err_count, int32_t* dev_err) {
  const int64_t pair = blockIdx.x;
  const int32_t s = st[pair];
  const int32_t d = dt[pair];
  if (s < 0 && d < 0) return;  // padding
  if (s < 0 || d < 0 || s >= ns || d >= nd) {
    if (threadIdx.x == 0) {
      if (err_count) atomicAdd(err_count, 1);
      atomicOr(dev_err, kDevErrRepackPair);
    }
    return;
  }
  const uint8_t* sp = src + (int64_t)s * page_bytes;
  uint8_t* dp = dst + (int64_t)d * page_bytes;
  const bool vec = ((page_bytes & 15) == 0) && ((((uintptr_t)src) & 15) == 0) && ((((uintptr_t)dst) & 15) == 0);
  if (vec) {
    const u32x4* s4 = (const u32x4*)sp;
    u32x4* d4 = (u32x4*)dp;
    const int64_t n4 = page_bytes >> 4;
    for (int64_t base = 0; base < n4; base += (int64_t)kRepackThreads * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kRepackThreads + threadIdx.x;
        if (i < n4) v[u] = __builtin_nontemporal_load(s4 + i);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kRepackThreads + threadIdx.x;
        if (i < n4) __builtin_nontemporal_store(v[u], d4 + i);
      }
    }
  } else {
    for (int64_t i = threadIdx.x; i < page_bytes; i += kRepackThreads) dp[i] = sp[i];
  }
}

}  // namespace

hipError_t launch_kv_repack(const void* src, const int32_t* src_table, void* dst, const int32_t* dst_table,
                            int64_t n_pairs, int64_t page_bytes, int32_t src_num_pages,
                            int32_t dst_num_pages, int32_t* err_count, int32_t* dev_err,
                            hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  if (n_pairs == 0) return hipSuccess;
  hipExtLaunchKernelGGL(kv_repack_kernel, dim3((uint32_t)n_pairs), dim3(kRepackThreads), 0, stream, e0, e1, 0,
                        (const uint8_t*)src, src_table, (uint8_t*)dst, dst_table, page_bytes, src_num_pages,
                        dst_num_pages, err_count, dev_err);
  return hipGetLastError();
}

}  // namespace splash
