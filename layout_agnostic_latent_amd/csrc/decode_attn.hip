// Decode attention over a paged latent KV head, for one rank's share
// (a head range, a token range, the requests of the batch), on gfx950.
//
// The share shapes are those of the SPLASH layouts (thelatestinai page,
// Appendix Table 2): TP = head slice over whole histories, CP = token range of
// every history with partial output + LSE, DP-attention / DOP = whole owned
// requests.  Every query head of a request attends to the same latent row per
// token (weekinpapers page, Abstract: attention with few or no KV heads), and
// V is the first d_v dims of that row, so one LDS tile of KV rows feeds both
// contractions.
//
// Work decomposition.  A workgroup owns (request b, a chunk of 32-token tiles,
// a group of up to 32*WH heads).  Its WH*WV waves each hold 32 heads:
// wave (wh, wv) computes the scores of heads [32*wh, 32*wh+32) and the output
// columns of V block range wv.  With WV > 1 the score tile is computed
// redundantly by the WV waves of a head group (cheap at small head counts,
// where the kernel is bound by HBM, not by the matrix cores).
//
// Per 32-token tile:
//  * the KV rows (tile x d_qk bf16) land in an LDS ring slot through
//    global_load_lds_dwordx4 (no VGPR staging); each instruction moves 1 KiB
//    of whole 128-B lines, chunks permuted within a line by the row swizzle;
//  * S^T[tok][head] = K[tok][:] . Q^T on v_mfma_f32_32x32x16_bf16, K from LDS
//    with ds_read_b128, Q held in VGPRs for the whole chunk;
//  * online softmax in fp32 on exp2, one cross-half exchange per tile, with
//    the running max only moved when it grows by more than 2^8;
//  * O^T[v][head] += V^T[v][tok] . P^T[tok][head] on the same MFMA: P^T comes
//    straight from the S^T accumulator registers (bf16), V^T from LDS with
//    ds_read_b64_tr_b16 transposing loads.
// A chunk writes normalised O and LSE (to the caller's output, or to the
// split-KV workspace that splash_lse_merge then combines).
#include "common.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kLdsBytes = 160 * 1024;
constexpr int kMaxBuf = 4;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p = exp2(s - m) stays <= 256

// XOR applied to the 16-byte chunk index of tile row `row`.  It makes the
// ds_read_b128 of 16 consecutive rows at one chunk, and the transposing
// reads of 4 consecutive rows x 4 chunks, hit distinct LDS banks.
__device__ __forceinline__ uint32_t row_swizzle(uint32_t row) {
  return ((row >> 2) & 3u) | (((row >> 1) & 1u) << 2);
}

// One 16-byte-per-lane global -> LDS copy.  Lane i's 16 bytes land at
// lds_addr + 16*i.  Issued from inline asm so that the compiler does not add a
// vmcnt(0) before every LDS read; completion is tracked by wait_vmcnt().
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"{m0}"(lds_addr), "v"(src) : "memory");
}

// Same, with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit offset.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)),
               "v"(voff), "s"(sbase)
               : "memory");
}

// x *= alpha for an MFMA accumulator element.  Written against an AGPR
// operand so that the register allocator keeps the output accumulators in
// AGPRs (the multiply goes through one temporary VGPR).
__device__ __forceinline__ void scale_acc(float& x, float alpha) {
  float tmp;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(tmp)
               : "v"(alpha));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float wave_max_halves(float x) {
  // lanes l and l^32 hold the two halves of one head's 32 scores
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)p[e];
  return r;
}

template <int D_QK, int D_V, int WH, int WV>
struct Cfg {
  static constexpr int NW = WH * WV;
  static constexpr int NTHREADS = 64 * NW;
  static constexpr int NCH = D_QK / 8;               // 16-B chunks per KV row
  static constexpr int RC = (NCH + 7) / 8 * 8;       // LDS row stride in chunks
  static constexpr int ROWB = RC * 16;               // LDS bytes per tile row
  static constexpr int TILE_B = kTileTok * ROWB;     // LDS bytes per tile
  static constexpr int NBUF = (kLdsBytes / TILE_B) < kMaxBuf ? (kLdsBytes / TILE_B) : kMaxBuf;
  static constexpr int DMA_T = kTileTok * RC / 64;   // 1-KiB DMA instructions per tile
  static constexpr int DMA_W = DMA_T / NW;           // ... per wave
  static constexpr int KS = D_QK / 16;               // K-steps of the score MFMA
  static constexpr int VB = D_V / 32 / WV;           // 32-wide V blocks per wave
  static_assert(D_QK % 16 == 0 && D_V % (32 * WV) == 0 && D_V <= D_QK, "shape");
  static_assert(DMA_T % NW == 0, "DMA split");
  static_assert(NBUF >= 2, "LDS ring");
};

template <int D_QK, int D_V, int WH, int WV>
__global__ void __launch_bounds__(64 * WH * WV, 1) decode_attn_kernel(const DecodeArgs a) {
  using C = Cfg<D_QK, D_V, WH, WV>;
  __shared__ __attribute__((aligned(1024))) char smem[C::NBUF * C::TILE_B];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wh = wave % WH;
  const int wv = wave / WH;
  const int g = lane >> 5;   // k-group of the 32x32x16 operands
  const int n = lane & 31;   // head column (B / C operands), token row (A operand of QK)

  const int b = blockIdx.y;
  const int split = blockIdx.x;
  const int hs = (blockIdx.z * WH + wh) * 32 + n;  // head index within the share
  const bool head_ok = hs < a.n_heads;
  const int hs_safe = head_ok ? hs : 0;

  // Read-only tables through the constant address space: scalar loads, so
  // the vector-memory counter only ever counts the KV DMA.
  const int32_t __attribute__((address_space(4)))* bt_row =
      (const int32_t __attribute__((address_space(4)))*)(a.bt + (int64_t)b * a.max_pages);
  const int seq = ((const int32_t __attribute__((address_space(4)))*)a.seq_lens)[b];

  // ---- this workgroup's token range ----
  // tokens beyond the block table's capacity are never read
  const int lo = max(a.tok_lo, 0);
  const int hi = min(min(a.tok_hi, seq), a.max_pages << a.page_shift);
  int t_begin = 0, t_end = 0;  // absolute tile indices [t_begin, t_end)
  if (hi > lo) {
    const int tf = lo / kTileTok;
    const int nt = (hi + kTileTok - 1) / kTileTok - tf;
    const int chunk = a.fixed_splits > 0 ? (nt + a.fixed_splits - 1) / a.fixed_splits : a.chunk_tiles;
    t_begin = tf + split * chunk;
    t_end = min(t_begin + chunk, tf + nt);
  }
  const int mlo = max(lo, t_begin * kTileTok);
  const int mhi = min(hi, t_end * kTileTok);

  float* out_row = a.out + split * a.out_split_stride + ((int64_t)b * a.n_heads + hs_safe) * D_V;
  float* lse_ptr = a.lse ? a.lse + split * a.lse_split_stride + (int64_t)b * a.n_heads + hs_safe : nullptr;

  if (t_end <= t_begin) {  // empty chunk: O = 0, LSE = -inf
    if (head_ok) {
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int col = (wv * C::VB + vb) * 32 + rq * 8 + g * 4;
          *(floatx4*)(out_row + col) = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      if (lse_ptr && wv == 0 && g == 0) *lse_ptr = -INFINITY;
    }
    return;
  }
  const int ntiles = t_end - t_begin;

  // ---- Q for this wave's 32 heads: B operand of every score MFMA ----
  bf16x8 qf[C::KS];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_req_stride + (int64_t)(a.head_lo + hs_safe) * D_QK + 8 * g;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
    if (!head_ok) {
#pragma unroll
      for (int s = 0; s < C::KS; ++s) qf[s] = bf16x8{};
    }
  }

  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const int ps_mask = (1 << a.page_shift) - 1;
  const bool one_page_per_tile = a.page_shift >= 5;
  bool bad_page = false;  // reported once, after the last DMA has completed

  // Per-lane (row, chunk) of DMA instruction i of this wave, packed as
  // row | (byte offset of the chunk in the row) << 8.
  auto dma_rc = [&](int i) -> uint32_t {
    const int pos = (wave * C::DMA_W + i) * 64 + lane;
    const int row = pos / C::RC;
    int ch = (pos % C::RC) ^ (int)row_swizzle(row);
    if (ch >= C::NCH) ch = 0;  // row padding: any in-row chunk
    return (uint32_t)row | ((uint32_t)(ch * 16) << 8);
  };

  // Issue the DMA of absolute tile `t` into ring slot `slot`.  Rows outside
  // the chunk's [mlo, mhi) fetch a valid row of the same tile instead, so the
  // masked tokens see finite data (their probability is exactly 0).
  auto issue_tile = [&](int t, int slot) {
    const int tok0 = t * kTileTok;
    const int rlo = max(mlo - tok0, 0);
    const int rhi1 = min(mhi - tok0, kTileTok) - 1;
    const uint32_t lds_tile = smem_base + slot * C::TILE_B;
    int p0 = bt_row[tok0 >> a.page_shift];
    if ((unsigned)p0 >= (unsigned)a.num_pages) { bad_page = true; p0 = 0; }
    if (one_page_per_tile) {
      // all rows of the tile sit on one page: uniform base + per-lane offset
      const uint16_t* base = a.kv + (int64_t)p0 * a.page_stride + (int64_t)(tok0 & ps_mask) * D_QK;
#pragma unroll
      for (int i = 0; i < C::DMA_W; ++i) {
        const int row = min(max((int)(dma_rc(i) & 0xffu), rlo), rhi1);
        const uint32_t off = (uint32_t)row * (D_QK * 2) + (dma_rc(i) >> 8);
        lds_dma16_s(base, off, smem_base + slot * C::TILE_B + (wave * C::DMA_W + i) * 1024);
      }
    } else {
      // page_size 16: rows [0,16) and [16,32) may sit on two pages
      int p1 = p0;
      if (rhi1 >= 16) {
        p1 = bt_row[(tok0 + 16) >> a.page_shift];
        if ((unsigned)p1 >= (unsigned)a.num_pages) { bad_page = true; p1 = 0; }
      }
      const uint16_t* base0 = a.kv + (int64_t)p0 * a.page_stride;
      const uint16_t* base1 = a.kv + (int64_t)p1 * a.page_stride;
#pragma unroll
      for (int i = 0; i < C::DMA_W; ++i) {
        const int row = min(max((int)(dma_rc(i) & 0xffu), rlo), rhi1);
        const uint16_t* pg = row < 16 ? base0 : base1;
        const char* src = (const char*)(pg + (int64_t)((tok0 + row) & ps_mask) * D_QK) + (dma_rc(i) >> 8);
        lds_dma16(src, __builtin_amdgcn_readfirstlane(lds_tile + (wave * C::DMA_W + i) * 1024));
      }
    }
  };

  // ---- online-softmax state (per head = per lane column) ----
  floatx16 oacc[C::VB];
#pragma unroll
  for (int vb = 0; vb < C::VB; ++vb) oacc[vb] = floatx16{};
  float m_run = -INFINITY;  // running max in log2 units
  float l_run = 0.0f;       // this lane's half of the running sum of p (for the LSE)
  float lr_run = 0.0f;      // ... of p rounded to bf16, the weights PV uses (for normalising O)

  // Per-lane LDS byte offsets (within a ring slot) of the operand reads;
  // everything else is a compile-time immediate.
  //  K (A operand of QK), step s: row n, chunk (2s+g) ^ swz(n)
  //     = n*ROWB + 128*(s/4) + 16*((2*(s%4)) ^ z),  z = g ^ swz(n)
  uint32_t kofs[4];
  {
    const uint32_t z = (uint32_t)g ^ row_swizzle(n);
#pragma unroll
    for (int j = 0; j < 4; ++j) kofs[j] = n * C::ROWB + 16 * ((2u * j) ^ z);
  }
  //  V^T (A operand of PV) via ds_read_b64_tr_b16: lane (j, q) of each
  //  16-lane group reads row 16ks + 8h + 4g + j at column 32*vbg + 16*mh + 4q.
  //  With x = j>>1 and y_h = (2mh + (q>>1)) ^ (2h + g) the byte offset is
  //  (16ks+8h)*ROWB + 64*vbg  +  (4g+j)*ROWB + 16*y_h + 8*(q&1) + 64*(x ? (vbg odd ? -1 : 1) : 0).
  uint32_t vofs[2][2];  // [h][parity of vbg]
  {
    const int trj = (lane & 15) >> 2;
    const int trq = lane & 3;
    const int trmh = (lane >> 4) & 1;
    const int x = trj >> 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int y = (2 * trmh + (trq >> 1)) ^ (2 * h + g);
      const int basev = (4 * g + trj) * C::ROWB + 16 * y + 8 * (trq & 1) + 64 * wv * C::VB;
      vofs[h][0] = (uint32_t)(basev + (x ? 64 : 0));
      vofs[h][1] = (uint32_t)(basev - (x ? 64 : 0));
    }
  }
  const int vpar0 = (wv * C::VB) & 1;

#pragma unroll
  for (int i = 0; i < C::NBUF - 1; ++i)
    if (i < ntiles) issue_tile(t_begin + i, i);
  // Make the Q loads complete here, visibly to the compiler, so that it
  // places no vector-memory waits inside the tile loop (those would also
  // drain the KV prefetch, which the counter tracks too).
#pragma unroll
  for (int s = 0; s < C::KS; ++s) asm volatile("" ::"v"(qf[s]));

  for (int it = 0; it < ntiles; ++it) {
    // wait for this wave's DMA of tile `it`; younger tiles may stay in flight
    const int younger = min(ntiles - 1 - it, C::NBUF - 2);
    if (younger >= 2) wait_vmcnt<2 * C::DMA_W>();
    else if (younger == 1) wait_vmcnt<C::DMA_W>();
    else wait_vmcnt<0>();
    __syncthreads();  // every wave's DMA of tile `it` landed; slot of tile it-1 is free
    if (it + C::NBUF - 1 < ntiles) issue_tile(t_begin + it + C::NBUF - 1, (it + C::NBUF - 1) % C::NBUF);

    const int t = t_begin + it;
    const char* tile = smem + (it % C::NBUF) * C::TILE_B;

    // ---- S^T = K Q^T (32 tokens x 32 heads) ----
    floatx16 sacc = floatx16{};
    {
      constexpr int PF = C::KS < 4 ? C::KS : 4;  // K operands in flight
      bf16x8 kring[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) kring[s] = *(const bf16x8*)(tile + kofs[s & 3] + 128 * (s >> 2));
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const bf16x8 kf = kring[s % PF];
        if (s + PF < C::KS) kring[s % PF] = *(const bf16x8*)(tile + kofs[(s + PF) & 3] + 128 * ((s + PF) >> 2));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
      }
    }

    // ---- scores -> probabilities ----
    const int tok0 = t * kTileTok;
    const int rlo = max(mlo - tok0, 0);
    const int rhi = min(mhi - tok0, kTileTok);
    if ((rlo > 0) || (rhi < kTileTok)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < rlo || row >= rhi) sacc[r] = -INFINITY;
      }
    }
    float mloc = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, sacc[r]);
    mloc = wave_max_halves(mloc) * a.scale_log2;
    const bool need = mloc > m_run + kRescaleThreshold;
    if (__any(need)) {
      const float m_new = need ? mloc : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = oacc[vb][r];
          scale_acc(x, alpha);
          oacc[vb][r] = x;
        }
      m_run = m_new;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pf = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], a.scale_log2, -m_run));
      const __bf16 p = (__bf16)pf;
      pb[r >> 3][r & 7] = p;
      l_run += pf;
      lr_run += (float)p;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb) {
        const int par = (vpar0 ^ vb) & 1;
        const char* v0 = tile + vofs[0][par] + (16 * ks + 0) * C::ROWB + 64 * vb;
        const char* v1 = tile + vofs[1][par] + (16 * ks + 8) * C::ROWB + 64 * vb;
        const shortx4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)v0);
        const shortx4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)v1);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ks], oacc[vb], 0, 0, 0);
      }
    }
  }

  if (bad_page && lane == 0) atomicOr(a.dev_err, 1);

  // ---- epilogue: normalise and store ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float lr_tot = lr_run + __shfl_xor(lr_run, 32, 64);
  const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
  if (head_ok) {
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int col = (wv * C::VB + vb) * 32 + rq * 8 + g * 4;
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = oacc[vb][4 * rq + e] * inv;
        *(floatx4*)(out_row + col) = v;
      }
    if (lse_ptr && wv == 0 && g == 0)
      *lse_ptr = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int D_QK, int D_V, int WH, int WV>
hipError_t launch_variant(dim3 grid, const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_attn_kernel<D_QK, D_V, WH, WV>), grid, dim3(64 * WH * WV), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeVariant& v, dim3 grid, const DecodeArgs& a, hipStream_t stream) {
  if (v.d_qk == 576 && v.d_v == 512) {
    if (v.wh == 4 && v.wv == 1) return launch_variant<576, 512, 4, 1>(grid, a, stream);
    if (v.wh == 2 && v.wv == 2) return launch_variant<576, 512, 2, 2>(grid, a, stream);
    if (v.wh == 1 && v.wv == 4) return launch_variant<576, 512, 1, 4>(grid, a, stream);
  }
  if (v.d_qk == 80 && v.d_v == 64) {
    if (v.wh == 4 && v.wv == 1) return launch_variant<80, 64, 4, 1>(grid, a, stream);
    if (v.wh == 1 && v.wv == 2) return launch_variant<80, 64, 1, 2>(grid, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace splash
