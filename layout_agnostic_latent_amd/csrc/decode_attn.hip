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
#include <type_traits>

#include "common.h"

namespace splash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

constexpr int kPageLds = 4096;  // page ids of a chunk staged in LDS (16 KiB)
constexpr int kLdsBytes = 160 * 1024 - kPageLds * 4;
constexpr int kMaxBuf = 4;
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

// max(x[l], x[l ^ 32]) for every lane l: lanes l and l^32 hold the two halves
// of one head's 32 scores.  v_permlane32_swap exchanges the two wave halves
// in the VALU, without an LDS round trip.
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}


template <int D_QK, int D_V, int WH, int WV>
struct Cfg {
  static constexpr int NW = WH * WV;
  static constexpr int NTHREADS = 64 * NW;
  static constexpr int ROWG = D_QK * 2;              // bytes of a KV row in HBM
  static constexpr int NCH = D_QK / 8;               // 16-B chunks per KV row
  static constexpr int NSLAB = (NCH + 7) / 8;        // 128-B slabs per row (8 chunks each)
  static constexpr int SLAB_B = kTileTok * 128;      // LDS bytes of one slab of a tile
  static constexpr int TILE_B = NSLAB * SLAB_B;      // LDS bytes per tile
  static constexpr int NBUF = (kLdsBytes / TILE_B) < kMaxBuf ? (kLdsBytes / TILE_B) : kMaxBuf;
  static constexpr int DMA_T = NSLAB * (kTileTok / 8);  // 1-KiB DMA instructions per tile (8 rows x 128 B)
  static constexpr int DMA_W = DMA_T / NW;           // ... per wave
  static constexpr bool PADDED = (NCH % 8) != 0;     // rows padded to whole slabs
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
  __shared__ int32_t page_lds[kPageLds];  // this chunk's physical page ids

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

  // DMA instruction n of a tile fills slab n/4, rows 8*(n%4) .. +7: lane l
  // carries row 8*(n%4) + l/8 and chunk 8*(n/4) + ((l%8) ^ swizzle(row)).
  // With four waves, wave w issues the instructions of row group w.
  const int l8 = lane >> 3;
  auto dma_inst = [&](int i) { return C::NW == 4 ? 4 * i + wave : wave * C::DMA_W + i; };

  // The chunk's block-table entries [j0, j1) are staged in LDS once, so that
  // the tile loop issues no scalar-memory loads: an outstanding scalar load
  // would make every LDS-read wait in the loop a full drain of the counter
  // the two share.  Chunks with more pages than fit read the table through
  // the scalar cache instead.
  const int j0 = (t_begin * kTileTok) >> a.page_shift;
  const int j1 = (mhi - 1) >> a.page_shift;  // last page holding a token of the chunk
  const bool pt_lds = j1 - j0 < kPageLds;
  if (pt_lds) {
    const int32_t* src = a.bt + (int64_t)b * a.max_pages + j0;
    for (int j = threadIdx.x; j <= j1 - j0; j += C::NTHREADS) page_lds[j] = src[j];
    __syncthreads();
  }
  // Physical page of token `tok`.
  auto page_of = [&](int tok) -> int {
    int p = pt_lds ? __builtin_amdgcn_readfirstlane(page_lds[(tok >> a.page_shift) - j0]) : bt_row[tok >> a.page_shift];
    if ((unsigned)p >= (unsigned)a.num_pages) {
      bad_page = true;
      p = 0;
    }
    return p;
  };
  struct TilePages {
    int p0, p1;
  };
  auto pages_of = [&](int t) -> TilePages {
    const int tok0 = t * kTileTok;
    const int p0 = page_of(tok0);
    const int p1 = (!one_page_per_tile && min(mhi - tok0, kTileTok) > 16) ? page_of(tok0 + 16) : p0;
    return {p0, p1};
  };

  // DMA plan of absolute tile `t` (physical pages `pg`) into ring slot `slot`.
  // Rows outside the chunk's [mlo, mhi) fetch a valid row of the same tile
  // instead, so the masked tokens see finite data (their probability is
  // exactly 0).  An instruction's 8 rows never straddle two pages (pages hold
  // 16 or more rows and start at multiples of 16), even after clamping, so
  // every DMA takes a wave-uniform base address and a 32-bit per-lane offset.
  struct DmaPlan {
    const char* base0;  // + row * ROWG: rows on page p0
    const char* base1;  // + row * ROWG: rows 16..31 on page p1
    uint32_t lds;       // ring slot
    int rlo, rhi1;      // valid rows of the tile
  };
  auto dma_plan = [&](int t, int slot, TilePages pg) -> DmaPlan {
    const int tok0 = t * kTileTok;
    DmaPlan d;
    d.base0 = (const char*)(a.kv + (int64_t)pg.p0 * a.page_stride + (int64_t)(tok0 & ps_mask) * D_QK);
    d.base1 = (const char*)(a.kv + (int64_t)pg.p1 * a.page_stride) - 16 * C::ROWG;
    d.lds = smem_base + slot * C::TILE_B;
    d.rlo = max(mlo - tok0, 0);
    d.rhi1 = min(mhi - tok0, kTileTok) - 1;
    return d;
  };
  auto issue_one = [&](const DmaPlan& d, int i) {
    const int nn = dma_inst(i);
    const int R = 8 * (nn % 4);
    const int row = min(max(R + l8, d.rlo), d.rhi1);
    int chunk = 8 * (nn / 4) + ((lane & 7) ^ (int)row_swizzle(R + l8));
    if (C::PADDED && chunk >= C::NCH) chunk = 0;  // slab padding: any in-row chunk
    const char* base = (one_page_per_tile || min(max(R, d.rlo), d.rhi1) < 16) ? d.base0 : d.base1;
    lds_dma16_s(base, (uint32_t)(row * C::ROWG + chunk * 16), d.lds + nn * 1024);
  };

  // ---- online-softmax state (per head = per lane column) ----
  floatx16 oacc[C::VB];
#pragma unroll
  for (int vb = 0; vb < C::VB; ++vb) oacc[vb] = floatx16{};
  float m_run = -INFINITY;  // running max in log2 units
  float l_run = 0.0f;       // this lane's half of the running sum of p (for the LSE)
  float lr_run = 0.0f;      // ... of p rounded to bf16, the weights PV uses (normalises O)

  // Per-lane LDS byte offsets (within a ring slot) of the operand reads;
  // everything else is a compile-time immediate.
  //  K (A operand of QK), step s: row n, chunk 2s+g, i.e. slab s/4 and
  //  in-slab chunk 2*(s%4)+g:  (s/4)*SLAB_B + n*128 + 16*((2*(s%4)+g) ^ swz(n)).
  uint32_t kofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kofs[j] = n * 128 + 16 * ((2u * j + g) ^ row_swizzle(n));
  //  V^T (A operand of PV) via ds_read_b64_tr_b16: lane (j, q) of each
  //  16-lane group reads row r = 16ks + 8h + 4g + j at column 32*vbg + 16*mh + 4q,
  //  chunk c = 4*vbg + 2*mh + q/2, slab vbg/2.  With x = j>>1 and
  //  y_h = (2mh + (q>>1)) ^ (2h + g) the byte offset is
  //    (vbg/2)*SLAB_B + (16ks+8h)*128  +  (4g+j)*128 + 64*((vbg&1) ^ x) + 16*y_h + 8*(q&1).
  const int trj = (lane & 15) >> 2;
  const int trq = lane & 3;
  const int trmh = (lane >> 4) & 1;
  uint32_t vofs[2][2];  // [h][vbg & 1]
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int y = (2 * trmh + (trq >> 1)) ^ (2 * h + g);
      vofs[h][par] = (uint32_t)((4 * g + trj) * 128 + 64 * (par ^ (trj >> 1)) + 16 * y + 8 * (trq & 1));
    }
  auto vaddr = [&](int h, int ks, int vb) -> uint32_t {
    const int vbg = wv * C::VB + vb;
    return vofs[h][vbg & 1] + (uint32_t)((vbg >> 1) * C::SLAB_B + (16 * ks + 8 * h) * 128);
  };

  // One tile: scores, online softmax, output update.  With `with_dma`, the
  // DMA of a later tile (plan `dp`) is issued between the score MFMAs, so its
  // issue cost hides behind matrix work.
  auto compute_tile = [&](int it, auto with_dma, const DmaPlan& dp) {
    const int t = t_begin + it;
    const char* tile = smem + (it % C::NBUF) * C::TILE_B;

    // ---- S^T = K Q^T (32 tokens x 32 heads) ----
    // K operands are read PF steps ahead of the MFMA that consumes them; the
    // scheduling-group hints keep that interleave (one MFMA, one LDS read).
    floatx16 sacc = floatx16{};
    {
      constexpr int PF = C::KS < 4 ? C::KS : 4;  // K operands in flight
      bf16x8 kring[PF];
#pragma unroll
      for (int s = 0; s < PF; ++s) kring[s] = *(const bf16x8*)(tile + kofs[s & 3] + C::SLAB_B * (s >> 2));
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const bf16x8 kf = kring[s % PF];
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s + PF < C::KS) {
          kring[s % PF] = *(const bf16x8*)(tile + kofs[(s + PF) & 3] + C::SLAB_B * ((s + PF) >> 2));
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (decltype(with_dma)::value) {
#pragma unroll
          for (int i = 0; i < C::DMA_W; ++i)
            if ((i * C::KS) / C::DMA_W == s) issue_one(dp, i);
        }
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
    mloc = max_across_halves(mloc) * a.scale_log2;
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
    // Probabilities of the first 16 tokens (k-step 0 of PV), then the PV
    // MFMAs of k-step 0 interleaved with the second half of the softmax.
    bf16x8 pb[2];
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    auto probs = [&](int k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pf = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[8 * k + e], a.scale_log2, -m_run));
        pb[k][e] = (__bf16)pf;
        l_run += pf;
      }
      // sum of the rounded weights, two per v_dot2_f32_bf16
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pair = {pb[k][2 * e], pb[k][2 * e + 1]};
        lr_run = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lr_run, false);
      }
    };
    probs(0);

    // ---- O^T += V^T P^T ----
    // Two transposing LDS reads feed each MFMA; they run PV_PF MFMAs ahead.
    {
      constexpr int NM = 2 * C::VB;              // MFMAs per tile: (k-step, V block)
      constexpr int PV_PF = NM < 4 ? NM : 4;
      auto vread = [&](int i) -> bf16x8 {
        const int ks = i / C::VB, vb = i % C::VB;
        const char* v0 = tile + vaddr(0, ks, vb);
        const char* v1 = tile + vaddr(1, ks, vb);
        const shortx4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)v0);
        const shortx4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)v1);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vring[PV_PF];
#pragma unroll
      for (int i = 0; i < PV_PF; ++i) vring[i] = vread(i);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV_PF, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int ks = i / C::VB, vb = i % C::VB;
        if (i == C::VB) probs(1);  // its exps overlap the k-step 0 MFMAs still in flight
        const bf16x8 vf = vring[i % PV_PF];
        oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ks], oacc[vb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + PV_PF < NM) {
          vring[i % PV_PF] = vread(i + PV_PF);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    }
  };

#pragma unroll
  for (int i = 0; i < C::NBUF - 1; ++i)
    if (i < ntiles) {
      const DmaPlan d = dma_plan(t_begin + i, i, pages_of(t_begin + i));
#pragma unroll
      for (int k = 0; k < C::DMA_W; ++k) issue_one(d, k);
    }
  // Make the Q loads complete here, visibly to the compiler, so that it
  // places no vector-memory waits inside the tile loop (those would also
  // drain the KV prefetch, which the counter tracks too).
#pragma unroll
  for (int s = 0; s < C::KS; ++s) asm volatile("" ::"v"(qf[s]));

  // Main loop: after the barrier that frees its slot, the DMA of tile
  // it+NBUF-1 is issued between the score MFMAs of tile it, with its page
  // indices read one iteration ahead.  Two younger tiles stay in flight, so
  // the wait count is a constant.  The last NBUF-1 tiles issue no DMA.
  const std::integral_constant<bool, true> kDma;
  const std::integral_constant<bool, false> kNoDma;
  const int n_main = ntiles - (C::NBUF - 1);
  TilePages next = pages_of(t_begin + min(C::NBUF - 1, ntiles - 1));
  int it = 0;
  for (; it < n_main; ++it) {
    wait_vmcnt<(C::NBUF - 2) * C::DMA_W>();
    __syncthreads();  // every wave's DMA of tile `it` landed; slot of tile it-1 is free
    const int tn = t_begin + it + C::NBUF - 1;
    const DmaPlan dp = dma_plan(tn, (it + C::NBUF - 1) % C::NBUF, next);
    if (tn + 1 < t_end) next = pages_of(tn + 1);
    compute_tile(it, kDma, dp);
  }
  const DmaPlan none{nullptr, nullptr, 0u, 0, 0};
  for (; it < ntiles; ++it) {
    const int younger = ntiles - 1 - it;  // tiles still in flight behind this one
    if (younger >= 2) wait_vmcnt<2 * C::DMA_W>();
    else if (younger == 1) wait_vmcnt<C::DMA_W>();
    else wait_vmcnt<0>();
    __syncthreads();
    compute_tile(it, kNoDma, none);
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
hipError_t launch_variant(dim3 grid, const DecodeArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL((decode_attn_kernel<D_QK, D_V, WH, WV>), grid, dim3(64 * WH * WV), 0, stream, e0, e1, 0, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeVariant& v, dim3 grid, const DecodeArgs& a, hipStream_t stream, hipEvent_t e0,
                         hipEvent_t e1) {
  if (v.d_qk == 576 && v.d_v == 512) {
    if (v.wh == 4 && v.wv == 1) return launch_variant<576, 512, 4, 1>(grid, a, stream, e0, e1);
    if (v.wh == 2 && v.wv == 2) return launch_variant<576, 512, 2, 2>(grid, a, stream, e0, e1);
    if (v.wh == 1 && v.wv == 4) return launch_variant<576, 512, 1, 4>(grid, a, stream, e0, e1);
  }
  if (v.d_qk == 80 && v.d_v == 64) {
    if (v.wh == 4 && v.wv == 1) return launch_variant<80, 64, 4, 1>(grid, a, stream, e0, e1);
    if (v.wh == 1 && v.wv == 2) return launch_variant<80, 64, 1, 2>(grid, a, stream, e0, e1);
  }
  return hipErrorInvalidValue;
}

}  // namespace splash
