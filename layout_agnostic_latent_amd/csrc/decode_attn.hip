// Decode attention over a paged latent KV head, for one rank's share
// (a head range, a token range, the requests of the batch), on gfx950.
//
// The share shapes are those of the SPLASH layouts (thelatestinai page,
// Appendix Table 2): TP = head slice over whole histories, CP = token range of
// every history with partial output + LSE, DP-attention / DOP = whole owned
// requests.  Every query head of a request attends to the same latent row per
// token (weekinpapers page, Abstract: query heads sharing one or a few KV
// heads), and V is the first d_v dims of that row, so one LDS tile of KV rows
// feeds both contractions.
//
// Work decomposition.  A workgroup owns segments of (request b, a run of
// 32-token tiles, a group of up to 32*WH heads): one chunk of a grid, or the
// requests its range of the batch's tiles covers (the stream plan in
// decode_device.h).  Its WH*WV waves each hold 32 heads: wave (wh, wv)
// computes the scores of heads [32*wh, 32*wh+32) and the output columns of V
// block range wv.  With WV > 1 the WV waves of a head group split the score
// contraction's k-steps and sum their partial tiles through LDS.  Shares of
// at most 16 heads per KV head run the 16-head tile of decode_attn16.hip.
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
// The loop runs one tile behind on the output.  Iteration j scores tile j
// with the exponentials of tile j-1 between its MFMAs, then updates the
// output with tile j-1 while the VALU finds tile j's row max between the PV
// MFMAs: the softmax runs while the matrix cores work.
// A segment writes normalised O and LSE to the caller's output, or a scaled
// fp16 partial and its records to the split-KV workspace, which the merge
// kernel (lse_merge.hip) then combines on the same stream.
//
// Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of
// Attention with Seamless Handoff for LLM Serving" (weekinpapers.com); the
// thelatestinai page is that paper's summary with its appendix tables
// (thelatestinai.com).
#include <type_traits>

#include "decode_device.h"

namespace splash {
namespace {

constexpr int kLdsBytes = 160 * 1024 - kPageLds * 4;
constexpr int kMaxBuf = 4;
constexpr int kPlanStep = 22;  // PV MFMA after which the next tile's DMA plan is made (past the max slices)
constexpr int kTblLoadStep = 12;  // PV MFMA after which the table entry of that plan is read
// Tiles per segment the tile-address table holds (four waves x 4 bytes each:
// the 16 KiB page-id area of the four-wave, 32-head-per-wave variant).
constexpr int kTblTiles = 1024;

// x *= alpha for an MFMA accumulator element.  Written against an AGPR
// operand so that the register allocator keeps the output accumulators in
// AGPRs (the multiply goes through one temporary VGPR).
__device__ __forceinline__ void scale_acc(float& x, float alpha) {
  float tmp;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(x), "=&v"(tmp)
               : "v"(alpha));
}

// Score MFMAs with VGPR accumulators, issued from inline asm: the compiler
// gives every MFMA of a kernel that uses AGPRs the AGPR form, and the score
// tile would then have to share the AGPR file with the output accumulators
// (which fill it).  Accumulating back to back into the same registers needs
// no wait states.  The compiler takes an asm statement's output as written
// when the statement issues, while the matrix core writes it 8 passes later:
// a copy of the accumulator between two MFMAs of a chain (a live-range split
// of the register allocator) would read it in flight.  The accumulator is
// therefore pinned to fixed registers in every statement of the chain,
// v[2:17] (R = 0) or v[18:33] (R = 1), which leaves nothing to split.
// After the chain's last MFMA the VALU may read the result only 20 wait
// states later: with W the last statement carries them as s_nops; without,
// the caller issues at least 20 independent instructions first.
template <int R>
__device__ __forceinline__ void mfma_vgpr_first(floatx16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (R == 0) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "={v[2:17]}"(c) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "={v[18:33]}"(c) : "v"(a), "v"(b));
}
template <int R>
__device__ __forceinline__ void mfma_vgpr(floatx16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (R == 0) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+{v[2:17]}"(c) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+{v[18:33]}"(c) : "v"(a), "v"(b));
}
// The chain's result held in its registers up to this point (so that no
// copy of it is made while the matrix core may still be writing it).
template <int R>
__device__ __forceinline__ void chain_hold(floatx16& c) {
  if constexpr (R == 0) asm volatile("" : "+{v[2:17]}"(c));
  else asm volatile("" : "+{v[18:33]}"(c));
}
template <int R, bool W>
__device__ __forceinline__ void mfma_vgpr_last(floatx16& c, const bf16x8& a, const bf16x8& b) {
  if constexpr (!W) {
    mfma_vgpr<R>(c, a, b);
  } else if constexpr (R == 0) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+{v[2:17]}"(c)
                 : "v"(a), "v"(b));
  } else {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+{v[18:33]}"(c)
                 : "v"(a), "v"(b));
  }
}

template <int D_QK, int D_V, int WH, int WV>
struct Cfg {
  static constexpr int NW = WH * WV;
  static constexpr int NTHREADS = 64 * NW;
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
  static constexpr int NM = 2 * VB;                  // PV MFMAs per tile: (k-step, V block)
  static constexpr int KPF = KS < 4 ? KS : 4;        // K operands in flight (score MFMAs; <= KSW)
  static constexpr int VPF = NM < 4 ? NM : 4;        // V operands in flight (PV MFMAs)
  // DMA instructions of the next tile issued between the score MFMAs; the
  // rest go between the PV MFMAs.
  static constexpr int DMA_QK = DMA_W;
  static constexpr int PB = VB < 8 ? VB : 8;         // V blocks per epilogue pass
  static constexpr int PITCH = PB * 32 + 4;          // floats per staged output row (+16 B: banks)
  static constexpr int STAGE_B = NW * 32 * PITCH * 4;  // epilogue staging bytes
  // Split score contraction (the WV > 1 waves of a head group split V's
  // columns, so each would otherwise compute the same score tile): wave
  // (wh, wv) computes the scores over k-steps wv, wv + WV, ..., and the WV
  // partial tiles of a head group are summed through LDS.  The exchange
  // area takes the page-id area's place.
  static constexpr bool KSPLIT = WV > 1 && NW == 4 && KS % WV == 0;
  static constexpr int KSW = KSPLIT ? KS / WV : KS;  // k-steps of the score MFMAs per wave
  static constexpr int RING_B = NBUF * TILE_B;
  static constexpr int XCH_B = KSPLIT ? 4 * 16 * 64 * 4 : 0;  // four 32x32 fp32 partial tiles
  static constexpr int PAGE_LDS = KSPLIT ? 0 : kPageLds;     // page ids staged in LDS
  static constexpr int BODY_B = RING_B + XCH_B > STAGE_B ? RING_B + XCH_B : STAGE_B;
  static constexpr int SMEM_B = BODY_B + PAGE_LDS * 4;       // + the page-id area
  static_assert(SMEM_B <= 160 * 1024, "LDS");
  static_assert(D_QK % 16 == 0 && D_V % (32 * WV) == 0 && D_V <= D_QK, "shape");
  static_assert(DMA_T % NW == 0, "DMA split");
  static_assert(NBUF == 4, "LDS ring: two tiles computed, two in flight");
  static_assert(KS >= 2, "score chain");
  static_assert(VB % PB == 0, "epilogue passes");
};

// TBL: DMA addresses from a per-wave table of tile addresses built in the
// prologue (four waves, one row group each, no slab padding, chunks of at
// most kTblTiles tiles); otherwise from page ids looked up per tile.
template <int D_QK, int D_V, int WH, int WV, bool TBL>
__global__ void __launch_bounds__(64 * WH * WV, 1) decode_attn_kernel(const DecodeArgs a) {
  using C = Cfg<D_QK, D_V, WH, WV>;
  static_assert(!TBL || (C::NW == 4 && !C::PADDED && !C::KSPLIT && C::DMA_W <= 9 &&
                         C::BODY_B + 4 * kTblTiles * 4 <= C::SMEM_B && D_QK * 2 % 128 == 0),
                "tile-address table layout");
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM_B];
  // this chunk's physical page ids; with the split score contraction only
  // the plan's scratch, in the (then unused) exchange area
  int32_t* const page_lds = (int32_t*)(smem + (C::KSPLIT ? C::RING_B : C::BODY_B));

  // One segment: tiles [t_begin, t_end) of request b, its result written to
  // the caller's output (partial = false) or to partial row prow + head.
  // The arguments come in through `a`, a reference the segment loop below
  // hides from the optimiser, so that their loads are not hoisted out of the
  // loop and held in scalar registers across every segment.
  auto segment = [&](const DecodeArgs& a, const int b, const int t_begin, const int t_end, const int64_t prow,
                     const bool partial) {
  // Per-lane values are derived here from a thread index the optimiser
  // cannot see as loop invariant (held across segments they would take
  // registers from the tile loop).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wh = wave % WH;
  const int wv = wave / WH;
  const int g = lane >> 5;   // k-group of the 32x32x16 operands
  const int n = lane & 31;   // head column (B / C operands), token row (A operand of QK)
  // this workgroup's KV head and its query heads [k_lo, k_hi) within the share
  const int zk = blockIdx.z / a.z_per_kv;
  const int zz = blockIdx.z - zk * a.z_per_kv;
  const int kvh = a.kv_first + zk;
  const int k_lo = max(a.head_lo, kvh * a.kv_group) - a.head_lo;
  const int k_hi = min(a.head_lo + a.n_heads, (kvh + 1) * a.kv_group) - a.head_lo;
  const uint16_t* kv = a.kv + (int64_t)kvh * D_QK;
  const int head0 = k_lo + (zz * WH + wh) * 32;  // first head of this wave within the share
  const int hs = head0 + n;                      // this lane's head within the share
  const bool head_ok = hs < k_hi;
  const int hs_safe = head_ok ? hs : 0;
  const int lo = max(a.tok_lo, 0);
  // Read-only tables through the constant address space: scalar loads, so
  // the vector-memory counter only ever counts the KV DMA.
  const int32_t __attribute__((address_space(4)))* bt_row =
      (const int32_t __attribute__((address_space(4)))*)(a.bt + (int64_t)b * a.max_pages);
  const int seq = ((const int32_t __attribute__((address_space(4)))*)a.seq_lens)[b];
  // tokens beyond the block table's capacity are never read
  const int hi = min(min(a.tok_hi, seq), a.max_pages << a.page_shift);
  const int mlo = max(lo, t_begin * kTileTok);
  const int mhi = min(hi, t_end * kTileTok);

  float* out_row = a.out + ((int64_t)b * a.n_heads + hs_safe) * D_V;
  // the caller's LSE (a partial's LSE goes beside each of its group scales)
  float* lse_ptr = (!partial && a.lse) ? a.lse + (int64_t)b * a.n_heads + hs_safe : nullptr;
  constexpr int NG = D_V / partial_group_cols(D_V, WV);  // scale groups of a partial row
  constexpr int GW = NG / WV;                            // ... of them in this wave's V columns
  // partial row record of this lane's head: {LSE, 2^e} per column group
  float2* const prec = (float2*)a.part_l + (prow + hs_safe) * NG + wv * GW;

  if (t_end <= t_begin) {  // empty chunk: O = 0, LSE = -inf
    // A split-KV partial with LSE = -inf is never read by the merge, so only
    // the LSE is written there; the caller's own output gets the zeros.
    if (head_ok && !partial) {
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int col = (wv * C::VB + vb) * 32 + rq * 8 + g * 4;
          *(floatx4*)(out_row + col) = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (head_ok && lse_ptr && wv == 0 && g == 0) *lse_ptr = -INFINITY;
    if (head_ok && partial && g == 0) {
#pragma unroll
      for (int k = 0; k < GW; ++k) prec[k] = float2{-INFINITY, 1.0f};
    }
    return;
  }
  const int ntiles = t_end - t_begin;

  bf16x8 qf[C::KSW];  // Q of this wave's 32 heads, its k-steps (loaded in the prologue)
  // first k-step of this wave; its k-steps are ks0 + KST * s
  const int ks0 = C::KSPLIT ? wv : 0;
  constexpr int KST = C::KS / C::KSW;
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const int ps_mask = (1 << a.page_shift) - 1;
  const int row_b = a.kv_row * 2;  // bytes from one token's row to the next in the pool
  const bool one_page_per_tile = a.page_shift >= 5;
  bool bad_page = false;  // reported once, after the last DMA has completed

  // DMA instruction n of a tile fills slab n/4, rows 8*(n%4) .. +7: lane l
  // carries row 8*(n%4) + l/8 and chunk 8*(n/4) + ((l%8) ^ swizzle(row)).
  // With four waves, wave w issues the instructions of row group w.
  const int l8 = lane >> 3;
  auto dma_inst = [&](int i) { return C::NW == 4 ? 4 * i + wave : wave * C::DMA_W + i; };

  // Pages holding a token of [mlo, mhi): only their block-table entries are
  // read (a tile's rows below mlo fetch a row at or above it, see dma_plan).
  const int j0 = mlo >> a.page_shift;
  const int j1 = (mhi - 1) >> a.page_shift;
  // Where the tile loop finds the chunk's page ids (set up below, after the
  // first DMAs): 0 = the block table through the scalar cache, 1 = VGPRs
  // (page j0 + 64k + l in lane l of vpg[k]; read with v_readlane, no memory
  // access and no wait in the loop), 2 = LDS (chunks with more pages).
  const bool pt_vgpr = j1 - j0 < 64 * kVPages;
  const bool pt_lds = j1 - j0 < C::PAGE_LDS;
  int pt_mode = 0;
  int32_t vpg[kVPages];
  // Physical page of token `tok`.
  auto page_of = [&](int tok) -> int {
    const int idx = (tok >> a.page_shift) - j0;
    int p;
    if (pt_mode == 1) {
      // every register read with a constant index (a runtime index would put
      // vpg in scratch memory), the wave-uniform choice made on the scalars
      p = __builtin_amdgcn_readlane(vpg[0], idx & 63);
#pragma unroll
      for (int k = 1; k < kVPages; ++k) {
        const int q = __builtin_amdgcn_readlane(vpg[k], idx & 63);
        p = (idx >> 6) == k ? q : p;
      }
    } else {
      // kept a real branch: memory reads here must not be speculated into
      // the tile loop's common path, and their wait stays inside it (a wait
      // at the join would drain the LDS reads of every tile)
      asm volatile("" ::: "memory");
      p = pt_mode == 2 ? __builtin_amdgcn_readfirstlane(page_lds[idx]) : bt_row[tok >> a.page_shift];
      asm volatile("" ::"s"(p));
    }
    if ((unsigned)p >= (unsigned)a.num_pages) {
      bad_page = true;
      p = 0;
    }
    return p;
  };
  struct TilePages {
    int p0, p1;
  };
  // Pages of rows 0..15 and 16..31 of tile t.  Rows below mlo take a row at
  // or above it, so a half whose rows all lie below mlo is looked up at mlo
  // (the page of the first row it is clamped to): no entry before the range
  // is read.
  auto pages_of = [&](int t) -> TilePages {
    const int tok0 = t * kTileTok;
    const int p0 = page_of(max(tok0, mlo));
    const int p1 = (!one_page_per_tile && min(mhi - tok0, kTileTok) > 16) ? page_of(max(tok0 + 16, mlo)) : p0;
    return {p0, p1};
  };

  // DMA plan of absolute tile `t` (physical pages `pg`) into ring slot `slot`.
  // Rows outside the chunk's [mlo, mhi) fetch a valid row of the same tile
  // instead, so the masked tokens see finite data (their probability is
  // exactly 0).  An instruction's 8 rows never straddle two pages (pages hold
  // 16 or more rows and start at multiples of 16), even after clamping, so
  // every DMA takes a wave-uniform base address and a 32-bit per-lane offset.
  struct DmaPlan {
    const char* base0;  // + row * row_b: rows on page p0
    const char* base1;  // + row * row_b: rows 16..31 on page p1
    uint32_t lds;       // ring slot
    int rlo, rhi1;      // valid rows of the tile
    // four waves: wave w's instructions all carry rows 8w .. 8w+7 and differ
    // only by 128 B of chunk, so one lane offset and base serve them all
    const char* wbase;
    uint32_t voff;
  };
  auto dma_plan = [&](int t, int slot, TilePages pg) -> DmaPlan {
    const int tok0 = t * kTileTok;
    DmaPlan d;
    d.base0 = (const char*)(kv + (int64_t)pg.p0 * a.page_stride + (int64_t)(tok0 & ps_mask) * a.kv_row);
    d.base1 = (const char*)(kv + (int64_t)pg.p1 * a.page_stride) - 16 * row_b;
    d.lds = smem_base + slot * C::TILE_B;
    d.rlo = max(mlo - tok0, 0);
    d.rhi1 = min(mhi - tok0, kTileTok) - 1;
    if constexpr (C::NW == 4 && !C::PADDED) {
      const int R = 8 * wave;
      const int row = min(max(R + l8, d.rlo), d.rhi1);
      d.voff = (uint32_t)(row * row_b + 16 * ((lane & 7) ^ (int)row_swizzle(R + l8)));
      d.wbase = (one_page_per_tile || min(max(R, d.rlo), d.rhi1) < 16) ? d.base0 : d.base1;
    } else {
      d.voff = 0;
      d.wbase = nullptr;
    }
    return d;
  };
  auto issue_one = [&](const DmaPlan& d, int i) {
    if constexpr (TBL) {
      // one 64-bit base for the wave's nine instructions (immediate offsets);
      // instruction i fills slab i of the wave's rows, at d.lds + i * SLAB_B.
      // The slot address is re-read here so that each instruction's m0 is
      // computed in its own MFMA gap, not all in one.
      uint32_t l = __builtin_amdgcn_readfirstlane(d.lds);
      asm volatile("" : "+s"(l));
      switch (i) {
        case 0: lds_dma16_imm<0>(d.wbase, d.voff, l + 0 * C::SLAB_B); break;
        case 1: lds_dma16_imm<1>(d.wbase, d.voff, l + 1 * C::SLAB_B); break;
        case 2: lds_dma16_imm<2>(d.wbase, d.voff, l + 2 * C::SLAB_B); break;
        case 3: lds_dma16_imm<3>(d.wbase, d.voff, l + 3 * C::SLAB_B); break;
        case 4: lds_dma16_imm<4>(d.wbase, d.voff, l + 4 * C::SLAB_B); break;
        case 5: lds_dma16_imm<5>(d.wbase, d.voff, l + 5 * C::SLAB_B); break;
        case 6: lds_dma16_imm<6>(d.wbase, d.voff, l + 6 * C::SLAB_B); break;
        case 7: lds_dma16_imm<7>(d.wbase, d.voff, l + 7 * C::SLAB_B); break;
        default: lds_dma16_imm<8>(d.wbase, d.voff, l + 8 * C::SLAB_B); break;
      }
      return;
    }
    if constexpr (C::NW == 4 && !C::PADDED) {
      lds_dma16_s(d.wbase + 128 * i, d.voff, d.lds + (4 * i + wave) * 1024);
      return;
    }
    const int nn = dma_inst(i);
    const int R = 8 * (nn % 4);
    const int row = min(max(R + l8, d.rlo), d.rhi1);
    int chunk = 8 * (nn / 4) + ((lane & 7) ^ (int)row_swizzle(R + l8));
    if (C::PADDED && chunk >= C::NCH) chunk = 0;  // slab padding: any in-row chunk
    const char* base = (one_page_per_tile || min(max(R, d.rlo), d.rhi1) < 16) ? d.base0 : d.base1;
    lds_dma16_s(base, (uint32_t)(row * row_b + chunk * 16), d.lds + nn * 1024);
  };

  // Tile-address table (TBL): entry [w][i] locates the first row of wave w's
  // row group in tile i of the chunk, i.e. of token clamp(32 (t_begin + i) +
  // 8w, mlo, mhi - 1), as its byte offset from this KV head's base in units
  // of 128 B (rows, pages and the head offset are multiples of 128 B for
  // 576-wide rows; 32 bits cover pools of up to 512 GiB).  The group's other
  // rows are at most 7 rows further on the same page.  The lane offset is
  // the same for every interior tile; the first and last tiles clamp rows
  // outside [mlo, mhi) to the nearest valid row of the group.
  uint32_t* const tbl = (uint32_t*)(smem + C::BODY_B) + (TBL ? wave * kTblTiles : 0);
  const uint32_t chunk_off = 16u * ((uint32_t)(lane & 7) ^ row_swizzle(8 * wave + l8));
  const uint32_t voff_int = (uint32_t)(l8 * row_b) + chunk_off;
  // The plan of an interior tile, and the lane offset of an edge tile (the
  // first or the last of the segment; the main loop takes the two apart so
  // that each fits one MFMA gap).
  auto tbl_plan_interior = [&](uint32_t entry, int slot) -> DmaPlan {
    DmaPlan d{};
    d.wbase = (const char*)kv + ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(entry) << 7);
    d.lds = smem_base + slot * C::TILE_B + wave * 1024;
    d.voff = voff_int;
    return d;
  };
  auto tbl_edge_voff = [&](int i) -> uint32_t {
    const int tokg = (t_begin + i) * kTileTok + 8 * wave;
    const int tokw = min(max(tokg, mlo), mhi - 1);
    const int row = min(max(tokg + l8, mlo), mhi - 1);
    return (uint32_t)((row - tokw) * row_b) + chunk_off;
  };
  auto tbl_plan = [&](uint32_t entry, int i, int slot) -> DmaPlan {
    DmaPlan d = tbl_plan_interior(entry, slot);
    if (i == 0 || i == ntiles - 1) d.voff = tbl_edge_voff(i);
    return d;
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
  // split contraction: this wave's k-step s is ks0 + KST * s, at in-slab
  // chunk pair (ks0 + KST * s) % 4 of slab (ks0 + KST * s) / 4; with
  // KST = 2 or 4 the pair cycles through 4 / KST values
  constexpr int KPAIRS = C::KSPLIT ? 4 / KST : 1;
  uint32_t kofs_w[KPAIRS];
#pragma unroll
  for (int t = 0; t < KPAIRS; ++t)
    kofs_w[t] = n * 128 + 16 * ((2u * (uint32_t)(ks0 + KST * t) + g) ^ row_swizzle(n));
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

  // The tile loop is software-pipelined by one tile: iteration j computes the
  // scores of tile j with the exponentials of tile j-1 between its MFMAs,
  // then the output update of tile j-1 with tile j's row max between those
  // MFMAs, so that the softmax runs while the matrix cores work instead of
  // between the two contractions.

  // ---- S^T = K Q^T (32 tokens x 32 heads) of tile `it` ----
  // K operands are read PF steps ahead of the MFMA that consumes them.  With
  // `with_dma`, the DMA of a later tile (plan `dp`) is issued between the
  // MFMAs, so its issue cost hides behind matrix work.
  // With the split contraction the wave's partial tile (its k-steps) goes
  // through LDS and every wave returns the same full tile, summed in one
  // order.
  auto kaddr = [&](int s) -> uint32_t {  // LDS offset of this wave's k-step s within a tile
    if constexpr (C::KSPLIT) return kofs_w[s % KPAIRS] + C::SLAB_B * (s / KPAIRS);
    else return kofs[s & 3] + C::SLAB_B * (s >> 2);
  };
  // `reg` selects the chain's accumulator registers; without `waits` the
  // caller must issue 20 independent instructions before reading the scores.
  auto qk_tile = [&](int it, auto with_dma, bool do_dma, const DmaPlan& dp, auto&& hook, auto reg,
                     auto waits) -> floatx16 {
    constexpr int R = decltype(reg)::value;
    constexpr bool W = decltype(waits)::value || C::KSPLIT;  // the score exchange reads them at once
    const char* tile = smem + (it & (C::NBUF - 1)) * C::TILE_B;
    constexpr int PF = C::KPF < C::KSW ? C::KPF : C::KSW;
    floatx16 sacc;
    bf16x8 kring[PF];
#pragma unroll
    for (int s = 0; s < PF; ++s) kring[s] = *(const bf16x8*)(tile + kaddr(s));
#pragma unroll
    for (int s = 0; s < C::KSW; ++s) {
      const bf16x8 kf = kring[s % PF];
      if (s == 0) mfma_vgpr_first<R>(sacc, kf, qf[0]);
      else if (s == C::KSW - 1) mfma_vgpr_last<R, W>(sacc, kf, qf[s]);
      else mfma_vgpr<R>(sacc, kf, qf[s]);
      if (s + PF < C::KSW) kring[s % PF] = *(const bf16x8*)(tile + kaddr(s + PF));
      if constexpr (decltype(with_dma)::value) {
#pragma unroll
        for (int i = 0; i < C::DMA_QK; ++i)
          if ((i * C::KSW) / C::DMA_QK == s && do_dma) issue_one(dp, i);
      }
      hook(s);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (C::KSPLIT) {
      // partial tiles, lane-major: element 4q..4q+3 of lane l of wave w at
      // ((w * 4 + q) * 64 + l) * 16 bytes
      char* xch = smem + C::RING_B;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(floatx4*)(xch + ((wave * 4 + q) * 64 + lane) * 16) =
            floatx4{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
      __syncthreads();
      // the head group's waves are wh + WH * v, v < WV; summed in v order
      floatx4 part[WV][4];
#pragma unroll
      for (int v = 0; v < WV; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q) part[v][q] = *(const floatx4*)(xch + (((wh + WH * v) * 4 + q) * 64 + lane) * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        floatx4 t = part[0][q];
#pragma unroll
        for (int v = 1; v < WV; ++v) t = t + part[v][q];
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[4 * q + e] = t[e];
      }
    }
    return sacc;
  };

  // Tokens of tile `it` outside the chunk's range get score -inf.
  auto mask_tile = [&](floatx16& s, int it) {
    const int tok0 = (t_begin + it) * kTileTok;
    const int rlo = max(mlo - tok0, 0);
    const int rhi = min(mhi - tok0, kTileTok);
    if ((rlo > 0) || (rhi < kTileTok)) {
      // valid rows as a scalar bit mask; element r of this lane is row
      // 8*(r/4) + (r%4) + 4g, i.e. bit (8*(r/4) + (r%4)) of the mask >> 4g
      const uint32_t keep = (rhi >= 32 ? 0xffffffffu : ((1u << rhi) - 1u)) & ~((1u << rlo) - 1u);
      const uint32_t kg = keep >> (4 * g);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!((kg >> (8 * (r >> 2) + (r & 3))) & 1u)) s[r] = -INFINITY;
    }
  };

  // Row max of a score tile in log2 units (both halves of the head's column).
  auto tile_max = [&](const floatx16& s) -> float {
    float mloc = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mloc = fmaxf(mloc, s[r]);
    return max_across_halves(mloc) * a.scale_log2;
  };
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // ---- O^T += V^T P^T for tile `it` ----
  // Two transposing LDS reads feed each MFMA; they run PV_PF MFMAs ahead, and
  // the first PV_PF are issued by the caller (during the score MFMAs of the
  // next tile, so that their latency is hidden).  `step(i)` emits a slice of
  // other work (the next tile's row max) after MFMA i; the scheduling barrier
  // keeps each slice between its MFMAs, where the VALU runs while the matrix
  // core is busy.
  constexpr int NM = C::NM;
  constexpr int PV_PF = C::VPF;
  auto vread = [&](int it, int i) -> bf16x8 {
    const char* tile = smem + (it & (C::NBUF - 1)) * C::TILE_B;
    const int ks = i / C::VB, vb = i % C::VB;
    const char* v0 = tile + vaddr(0, ks, vb);
    const char* v1 = tile + vaddr(1, ks, vb);
    const shortx4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)v0);
    const shortx4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)v1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pv_tile = [&](int it, const bf16x8 (&p)[2], bf16x8 (&vring)[PV_PF], auto&& step) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int ks = i / C::VB, vb = i % C::VB;
      const bf16x8 vf = vring[i % PV_PF];
      oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[ks], oacc[vb], 0, 0, 0);
      if (i + PV_PF < NM) vring[i % PV_PF] = vread(it, i + PV_PF);
      step(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Hook for the score MFMAs of tile it+1: issue the first PV_PF operand
  // reads of tile `it` after the last PV_PF score MFMAs.
  auto vprefetch_hook = [&](int it, bf16x8 (&vring)[PV_PF]) {
    return [&, it](int sidx) {
      const int i = sidx - (C::KSW - PV_PF);
      if (i >= 0) vring[i] = vread(it, i);
    };
  };

  // Exponentials of a finished score tile, in 19 slices: a three-stage
  // pipeline over its 16 scores (exponent; exp2; the exact sum and the bf16
  // pair packing with the rounded sum).  The wave issues in order, so each
  // slice only uses values made one slice (at least one MFMA) earlier.
  // `pin` ties a value to its slice: pure arithmetic would otherwise be sunk
  // past the scheduling barriers to the end of the block.
  constexpr int kExpSlices = 19;
  auto pin = [](float& x) { asm volatile("" : "+v"(x)); };
  auto exp_slice = [&](int t, floatx16& sp, float m, uint32_t (&pw)[2][4], float& lsum, float& lrsum) {
    if (t < 16) {
      float x = __builtin_fmaf(sp[t], a.scale_log2, -m);
      pin(x);
      sp[t] = x;
    }
    if (t >= 1 && t <= 16) {
      float x = __builtin_amdgcn_exp2f(sp[t - 1]);
      pin(x);
      sp[t - 1] = x;
    }
    if (t >= 2 && t <= 17) {
      lsum += sp[t - 2];
      pin(lsum);
    }
    if (t >= 3 && t <= 17 && ((t - 2) & 1)) {  // pack p[e-1], p[e] (e = t-2 odd)
      const int e = t - 2;
      const bf16x2 pair = {(__bf16)sp[e - 1], (__bf16)sp[e]};
      uint32_t w = __builtin_bit_cast(uint32_t, pair);
      asm volatile("" : "+v"(w));
      pw[e >> 3][(e & 7) >> 1] = w;
    }
    if (t >= 4 && t <= 18 && ((t - 3) & 1)) {  // sum of the rounded pair packed one slice ago
      const int e = t - 3;
      lrsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e >> 3][(e & 7) >> 1]), ones, lrsum,
                                              false);
      pin(lrsum);
    }
  };
  auto pack_probs = [](const uint32_t (&pw)[2][4], bf16x8 (&p)[2]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const u32x4 w = {pw[k][0], pw[k][1], pw[k][2], pw[k][3]};
      p[k] = __builtin_bit_cast(bf16x8, w);
    }
  };
  // First score MFMA whose slack takes an exponential slice (the chain's
  // first steps carry the tile's first K reads and DMA instructions).
  constexpr int kExpStep0 = C::KSW >= kExpSlices + 2 ? 2 : 0;

  // Score phase of iteration j: the scores of tile j, with the exponentials
  // of tile j-1 (scores `sprev`, running max m_run) in the MFMAs' slack, so
  // that they run on the VALU while the matrix cores work.  Tile j-1's
  // weights are first consumed by its PV products, which come after these
  // score MFMAs.  Returns tile j's scores and tile j-1's packed weights; the
  // sums of tile j-1's weights are added to the running sums.
  // Main-loop iterations alternate the score chain between the two register
  // blocks (kAltChains): tile j's scores stay in their block while tile
  // j+1's chain accumulates in the other, and the chain's wait states are
  // left to the PV steps before the first slice that reads the scores.
  constexpr bool kAltChains = TBL && !C::KSPLIT && C::NM >= 16;
  constexpr int kSlice0 = kAltChains ? 6 : 0;
  // The main loop's exponentials spread over all 36 score MFMAs.  The wave
  // issues one instruction per 4-cycle slot and an MFMA occupies the matrix
  // core for 8, so the 7 slots after each MFMA are free for other work; a
  // gap with more delays the next MFMA.  A gap holds a K read and its wait
  // (2 slots), every fourth (steps 0, 4, .., 32) also a DMA (3 more).  An
  // exp2 takes 4 slots and one wait state before its result is read (5), and
  // one before it may read a value the VALU just wrote, so each goes alone
  // into an odd gap, its exponent one gap earlier:
  //   step 0:      exponent of element 0;
  //   step 4m+1:   exp2 of element 2m;   step 4m+3: exp2 of element 2m+1;
  //   step 4m+2:   sum of element 2m, exponents of elements 2m+1 and 2m+2,
  //                rounded sum of pair m-1;
  //   step 4m+4:   sum of element 2m+1, bf16 packing of pair m (m < 7);
  //   steps 32-35: the last sum, packing and rounded sum, then the running
  //   sums (each value is used at least one MFMA after it is made).
  constexpr bool kSpreadExp = kAltChains && C::KSW == 36 && C::DMA_QK == 9 && C::KPF == 4 && PV_PF == 4;
  auto exp_spread = [&](int st, floatx16& sp, float m, uint32_t (&pw)[2][4], float& lsum, float& lrsum) {
    auto expo = [&](int e) {
      float x = __builtin_fmaf(sp[e], a.scale_log2, -m);
      pin(x);
      sp[e] = x;
    };
    auto ex2 = [&](int e) {
      float x = __builtin_amdgcn_exp2f(sp[e]);
      pin(x);
      sp[e] = x;
    };
    auto add = [&](int e) {
      lsum += sp[e];
      pin(lsum);
    };
    auto pack = [&](int k) {
      const bf16x2 pair = {(__bf16)sp[2 * k], (__bf16)sp[2 * k + 1]};
      uint32_t w = __builtin_bit_cast(uint32_t, pair);
      asm volatile("" : "+v"(w));
      pw[k >> 2][k & 3] = w;
    };
    auto rsum = [&](int k) {
      lrsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[k >> 2][k & 3]), ones, lrsum, false);
      pin(lrsum);
    };
    if (st == 0) {
      expo(0);
    } else if (st <= 31) {
      const int mm = (st - 1) >> 2, r = (st - 1) & 3;
      if (r == 0) {
        ex2(2 * mm);
      } else if (r == 1) {
        add(2 * mm);
        expo(2 * mm + 1);
        if (mm < 7) expo(2 * mm + 2);
        if (mm >= 1) rsum(mm - 1);
      } else if (r == 2) {
        ex2(2 * mm + 1);
      } else {
        add(2 * mm + 1);
        pack(mm);
      }
    } else if (st == 32) {
      add(15);
    } else if (st == 33) {
      pack(7);
    } else if (st == 34) {
      rsum(7);
    }
  };
  auto qk_and_exp = [&](int it, auto with_dma, bool do_dma, const DmaPlan& dp, bf16x8 (&vring)[PV_PF],
                        floatx16& sprev, bf16x8 (&pcur)[2], auto reg, auto waits) -> floatx16 {
    constexpr bool spread = kSpreadExp && decltype(with_dma)::value;
    uint32_t pw[2][4];
    float lsum = 0.0f, lrsum = 0.0f;
    const float m = m_run;
    auto vpf = vprefetch_hook(it - 1, vring);
    floatx16 s = qk_tile(it, with_dma, do_dma, dp, [&](int sidx) {
      vpf(sidx);
      if constexpr (spread) {
        exp_spread(sidx, sprev, m, pw, lsum, lrsum);
        if (sidx == 35) {
          l_run += lsum;
          lr_run += lrsum;
        }
      } else {
        const int t = sidx - kExpStep0;
        if (t >= 0 && t < kExpSlices) exp_slice(t, sprev, m, pw, lsum, lrsum);
      }
      // the previous tile's scores keep the other block (no copy of them)
      if constexpr (kAltChains && decltype(with_dma)::value) chain_hold<1 - decltype(reg)::value>(sprev);
    }, reg, waits);
    if constexpr (!spread) {
#pragma unroll
      for (int t = C::KSW - kExpStep0; t < kExpSlices; ++t) exp_slice(t, sprev, m, pw, lsum, lrsum);
      l_run += lsum;
      lr_run += lrsum;
    }
    pack_probs(pw, pcur);
    return s;
  };

  // PV phase of iteration j: the output update of tile j-1 (weights `pcur`),
  // with tile j's row max and the new running max in slices between its
  // MFMAs; every slice only uses values made in earlier slices:
  //   slices 0-6: the row max (a max3 tree, then the other half's max),
  //   7-9:        scaled max and the new running max.
  // After the products, the output and the running sums are rescaled to the
  // new max if it moved (lazily: only when it grew by more than 2^8).
  // With the main loop's chains (no wait states of their own) the first
  // slice reading the scores comes after kSlice0 PV steps of at least four
  // instructions each.
  auto pv_and_max = [&](int it, floatx16& s, const bf16x8 (&pcur)[2], bf16x8 (&vring)[PV_PF], auto with_dma,
                        const DmaPlan& dp, auto&& extra, auto reg) {
    // tiles of the main loop (with_dma) lie strictly inside the chunk: only
    // the first and the last tile can hold rows outside [mlo, mhi)
    if constexpr (!decltype(with_dma)::value) mask_tile(s, it);
    float mx[4];
    float m_new = m_run;
    const float thr = m_run + kRescaleThreshold;
    bool need = false;
    auto max3 = [](float x, float y, float z) {
      float r;
      asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
      return r;
    };
    auto step = [&](int i) {
      extra(i);
      if constexpr (decltype(with_dma)::value && C::DMA_QK < C::DMA_W) {
        constexpr int ND = C::DMA_W - C::DMA_QK;
#pragma unroll
        for (int k = 0; k < ND; ++k)
          if ((k * C::NM) / ND == i) issue_one(dp, C::DMA_QK + k);
      }
      const int j = decltype(with_dma)::value ? i - kSlice0 : i;  // slice of this step
      if constexpr (kAltChains && decltype(with_dma)::value) {
        // the scores stay in the chain's registers: until the wait states
        // are covered (the PV steps before slice 0), and on into the next
        // tile's exponentials
        if (j >= 0) chain_hold<decltype(reg)::value>(s);
      }
      if (j == 0) {
        mx[0] = max3(s[0], s[1], s[2]);
        mx[1] = max3(s[3], s[4], s[5]);
      } else if (j == 1) {
        mx[2] = max3(s[6], s[7], s[8]);
        mx[3] = max3(s[9], s[10], s[11]);
      } else if (j == 2) {
        mx[0] = max3(mx[0], mx[1], s[15]);
        mx[1] = max3(s[12], s[13], s[14]);
      } else if (j == 3) {
        mx[0] = max3(mx[0], mx[2], mx[3]);
      } else if (j == 4) {
        mx[0] = max3(mx[0], mx[1], mx[1]);
      } else if (j == 5) {
        // both halves of the head's column: lane l and lane l ^ 32
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[0]), __float_as_uint(mx[0]), false, false);
        mx[1] = __uint_as_float(r[0]);
        mx[2] = __uint_as_float(r[1]);
        pin(mx[1]);
        pin(mx[2]);
      } else if (j == 6) {
        mx[0] = max3(mx[1], mx[2], mx[2]);
      } else if (j == 7) {
        mx[0] *= a.scale_log2;
        pin(mx[0]);
      } else if (j == 8) {
        need = mx[0] > thr;
      } else if (j == 9) {
        m_new = need ? mx[0] : m_run;
        pin(m_new);
      }
    };
    pv_tile(it - 1, pcur, vring, step);
    // slices beyond the MFMA count (variants with fewer V blocks)
    constexpr int kSteps = 10 + kSlice0 > kPlanStep + 3 ? 10 + kSlice0 : kPlanStep + 3;
#pragma unroll
    for (int i = C::NM; i < kSteps; ++i) step(i);
    const bool any_need = __any(need);
    if (any_need) {
      // the PV MFMAs above just wrote the accumulators: let them retire
      // before the VALU reads them
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
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
    }
    m_run = m_new;
  };

  const std::integral_constant<bool, true> kDma;
  const std::integral_constant<bool, false> kNoDma;
  const std::integral_constant<int, 0> kR0;
  const std::integral_constant<int, 1> kR1;
  const std::integral_constant<bool, true> kWaits;
  const std::integral_constant<bool, false> kNoWaits;

  // Prologue.  Order of issue: the chunk's page ids, Q, then the first two
  // tiles' DMA.  The Q loads touch 32 rows per instruction and so keep the
  // texture addresser busy for a while; the page-id loads, issued first,
  // land meanwhile, so the DMA needs no block-table fetch of its own.  Q and
  // tile 0 are waited for at iteration 0 (tile 1 stays in flight: it is
  // the youngest vector-memory work).

  // The chunk's block-table entries [j0, j1] are loaded once, so that the
  // tile loop issues no scalar-memory loads: an outstanding scalar load
  // would make every LDS-read wait in the loop a full drain of the counter
  // the two share.  Up to 64 * kVPages pages go to VGPRs, up to kPageLds to
  // LDS; longer chunks read the table through the scalar cache.
  const int32_t* bt_src = a.bt + (int64_t)b * a.max_pages + j0;
  // TBL: this wave's block-table entries, one per tile (lane i % 64 of
  // register i / 64), loaded before Q; the table is built once they land.
  constexpr int kTblRegs = TBL ? kTblTiles / 64 : 1;
  int32_t tpg[kTblRegs];
  if constexpr (TBL) {
    const int32_t* bt_b = a.bt + (int64_t)b * a.max_pages;
#pragma unroll
    for (int k = 0; k < kTblRegs; ++k) {
      tpg[k] = 0;
      if (k * 64 < ntiles) {
        const int i = min(k * 64 + lane, ntiles - 1);
        const int tokw = min(max((t_begin + i) * kTileTok + 8 * wave, mlo), mhi - 1);
        tpg[k] = bt_b[tokw >> a.page_shift];
      }
    }
  } else if (pt_vgpr) {
#pragma unroll
    for (int k = 0; k < kVPages; ++k) vpg[k] = j0 + 64 * k + lane <= j1 ? bt_src[64 * k + lane] : 0;
  } else if (pt_lds) {
    for (int j = threadIdx.x; j <= j1 - j0; j += C::NTHREADS) page_lds[j] = bt_src[j];
    __syncthreads();
    pt_mode = 2;
  }
  asm volatile("" ::: "memory");

  // ---- Q for this wave's 32 heads: B operand of every score MFMA ----
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_req_stride + (int64_t)(a.head_lo + hs_safe) * D_QK + 8 * g;
#pragma unroll
    for (int s = 0; s < C::KSW; ++s) qf[s] = *(const bf16x8*)(qp + 16 * (ks0 + KST * s));
    if (!head_ok) {
#pragma unroll
      for (int s = 0; s < C::KSW; ++s) qf[s] = bf16x8{};
    }
  }
  asm volatile("" ::: "memory");
  if constexpr (TBL) {
    // The table (the compiler waits for the entries, not for the younger Q
    // loads).  An entry outside the pool is read as page 0 and flagged.
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kTblRegs; ++k) {
      if (k * 64 < ntiles) {
        const int i = k * 64 + lane;
        const int tokw = min(max((t_begin + min(i, ntiles - 1)) * kTileTok + 8 * wave, mlo), mhi - 1);
        uint32_t pg = (uint32_t)tpg[k];
        if (i < ntiles && pg >= (uint32_t)a.num_pages) {
          bad = true;
          pg = 0;
        }
        const uint64_t off = (uint64_t)pg * (uint64_t)(a.page_stride * 2) + (uint64_t)((tokw & ps_mask) * row_b);
        if (i < ntiles) tbl[i] = (uint32_t)(off >> 7);
      }
    }
    if (__any(bad)) bad_page = true;
  } else if (pt_vgpr) {
    // the page ids are complete here (the compiler waits for them, not for
    // the younger Q loads), so the loop never waits on them
#pragma unroll
    for (int k = 0; k < kVPages; ++k) asm volatile("" ::"v"(vpg[k]));
    pt_mode = 1;
  }

  // Tiles 0 and 1 in flight (two ring slots stay free for the tiles being
  // computed).
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (i < ntiles) {
      const DmaPlan d = TBL ? tbl_plan(tbl[i], i, i) : dma_plan(t_begin + i, i, pages_of(t_begin + i));
#pragma unroll
      for (int k = 0; k < C::DMA_W; ++k) issue_one(d, k);
    }

  // Iteration 0: scores and row max of tile 0 (the output is still zero, so
  // the running max is simply set; its exponentials run during the next
  // scores).  Tile 2's DMA goes into its free slot.
  floatx16 sprev;  // masked scores of the previous tile, awaiting their exponentials
  DmaPlan dp;      // DMA of the tile two ahead of the one being scored
  {
    if (ntiles > 1) wait_vmcnt<C::DMA_W>();
    else wait_vmcnt<0>();
    __syncthreads();
    dp = TBL ? tbl_plan(tbl[min(2, ntiles - 1)], 2, 2 % C::NBUF)
             : dma_plan(t_begin + 2, 2 % C::NBUF, pages_of(t_begin + min(2, ntiles - 1)));
    // The compiler waits for each Q operand at its MFMA, counting only its
    // own loads: with tile 1's DMA younger than Q, the last of those waits
    // also drain tile 1.  Tile 2's DMA is therefore issued after the scores,
    // not between them (it would be drained too).
    floatx16 s = qk_tile(0, kNoDma, false, dp, [](int) {}, kR0, kWaits);
    if (2 < ntiles) {
#pragma unroll
      for (int k = 0; k < C::DMA_W; ++k) issue_one(dp, k);
    }
    mask_tile(s, 0);
    m_run = tile_max(s);
    sprev = s;
    if (3 < ntiles)
      dp = TBL ? tbl_plan(tbl[3], 3, 3 % C::NBUF) : dma_plan(t_begin + 3, 3 % C::NBUF, pages_of(t_begin + 3));
  }

  // Main loop, iteration j: wait for tile j and barrier (every wave is done
  // with tile j-2, whose slot takes tile j+2); scores of tile j with the DMA
  // of tile j+2 and the exponentials of tile j-1 interleaved; output update
  // of tile j-1 with tile j's row max, and, in the PV MFMAs' slack after the
  // max, the page lookups and DMA plan of tile j+3 (scalar work, off the path
  // into the next scores).
  // One younger tile (j+1) stays in flight across the wait.
  // With kAltChains consecutive iterations alternate the score chain's
  // registers (tile j's scores stay in place while tile j+1's accumulate)
  // and leave the chain's wait states to the PV steps before the first
  // slice.
  int it = 1;
  // One pipelined tile: the exponentials of `prev` under the tile's score
  // chain, then its PV steps; returns the tile's scores.
  auto iteration = [&](floatx16& prev, auto reg, auto waits) -> floatx16 {
    constexpr int R = decltype(reg)::value;
    if constexpr (kAltChains) chain_hold<1 - R>(prev);  // no home of its own between tiles
    wait_vmcnt<C::DMA_W>();
    __syncthreads();
    bf16x8 vring[PV_PF];
    bf16x8 pcur[2];
    floatx16 s = qk_and_exp(it, kDma, true, dp, vring, prev, pcur, reg, waits);
    DmaPlan dp_next = dp;
    const int tn = t_begin + it + 3;
    uint32_t entry = 0;  // table entry of tile it + 3 (TBL), read early, used at the plan step
    pv_and_max(it, s, pcur, vring, kDma, dp, [&](int i) {
      if constexpr (TBL) {
        // tile it + 3 >= 3 is the segment's first tile never, its last one at most once
        if (i == kTblLoadStep && tn < t_end) entry = tbl[it + 3];
        if (i == kPlanStep && tn < t_end) dp_next = tbl_plan_interior(entry, (it + 3) & (C::NBUF - 1));
        if (i == kPlanStep + 2 && tn == t_end - 1) dp_next.voff = tbl_edge_voff(it + 3);
      } else {
        if (i == kPlanStep && tn < t_end) dp_next = dma_plan(tn, (it + 3) & (C::NBUF - 1), pages_of(tn));
      }
    }, reg);
    if constexpr (kAltChains) chain_hold<R>(s);
    dp = dp_next;
    return s;
  };
  if constexpr (kAltChains) {
    // two scores variables, one per chain register block, so that neither
    // chain's result is copied to carry it into the next tile
    while (it + 2 < ntiles) {
      floatx16 s1 = iteration(sprev, kR1, kNoWaits);
      if (!(++it + 2 < ntiles)) {
        sprev = s1;
        break;
      }
      sprev = iteration(s1, kR0, kNoWaits);
      ++it;
    }
  } else {
    for (; it + 2 < ntiles; ++it) sprev = iteration(sprev, kR0, kWaits);
  }
  const DmaPlan none{nullptr, nullptr, 0u, 0, 0, nullptr, 0u};
  for (; it < ntiles; ++it) {
    if (it + 1 < ntiles) wait_vmcnt<C::DMA_W>();
    else wait_vmcnt<0>();
    __syncthreads();
    bf16x8 vring[PV_PF];
    bf16x8 pcur[2];
    floatx16 s = qk_and_exp(it, kNoDma, false, none, vring, sprev, pcur, kR0, kWaits);
    pv_and_max(it, s, pcur, vring, kNoDma, none, [](int) {}, kR0);
    sprev = s;
  }
  // Weights and output update of the last tile.
  {
    bf16x8 vring[PV_PF];
#pragma unroll
    for (int i = 0; i < PV_PF; ++i) vring[i] = vread(ntiles - 1, i);
    uint32_t pw[2][4];
    float lsum = 0.0f, lrsum = 0.0f;
#pragma unroll
    for (int t = 0; t < kExpSlices; ++t) exp_slice(t, sprev, m_run, pw, lsum, lrsum);
    l_run += lsum;
    lr_run += lrsum;
    bf16x8 plast[2];
    pack_probs(pw, plast);
    pv_tile(ntiles - 1, plast, vring, [](int) {});
  }
  // let the last PV MFMAs retire before the epilogue reads the accumulators
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
  if (bad_page && lane == 0) atomicOr(a.dev_err, kDevErrBadPage);

  // ---- epilogue: normalise and store ----
  // The accumulators hold, per lane, 16-byte pieces of 32 different output
  // rows; stored directly, every instruction would touch 32 rows.  Each wave
  // instead writes its rows into its own LDS region (the ring is free once
  // every wave is past its last PV) and stores them back as whole 1-KiB runs.
  // The stores are non-temporal: the rows go to memory now instead of sitting
  // dirty in L2 until the write-back at the kernel's end.
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float lr_tot = lr_run + __shfl_xor(lr_run, 32, 64);
  const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
  float pscale[GW];  // partial rows: 2^e of each of this wave's column groups
  __syncthreads();
  {
    float* stage = (float*)smem + wave * 32 * C::PITCH;
    float* out_base = a.out + ((int64_t)b * a.n_heads + head0) * D_V;
    constexpr int ROWF = C::PB * 32;  // staged floats per row and pass
    static_assert(ROWF == partial_group_cols(D_V, WV) && C::VB / C::PB == GW, "scale groups as the host lays them out");
#pragma unroll
    for (int pass = 0; pass < C::VB / C::PB; ++pass) {
      float pm = 0.0f;  // largest |value| this lane stages (partial rows)
#pragma unroll
      for (int vbl = 0; vbl < C::PB; ++vbl)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          floatx4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = oacc[pass * C::PB + vbl][4 * rq + e] * inv;
          if (partial) pm = fmaxf(fmaxf(pm, fmaxf(fabsf(v[0]), fabsf(v[1]))), fmaxf(fabsf(v[2]), fabsf(v[3])));
          *(floatx4*)(stage + n * C::PITCH + vbl * 32 + rq * 8 + 4 * g) = v;
        }
      const int col0 = (wv * C::VB + pass * C::PB) * 32;
      if (!partial) {
#pragma unroll
        for (int i = 0; i < 32 * ROWF / 256; ++i) {
          const int e = (i * 64 + lane) * 4;
          const int row = e / ROWF, col = e % ROWF;
          const floatx4 v = *(const floatx4*)(stage + row * C::PITCH + col);
          if (head0 + row < k_hi)
            __builtin_nontemporal_store(v, (floatx4*)(out_base + (int64_t)row * D_V + col0 + col));
        }
      } else {
        // Split-KV partial: the pass's ROWF columns of a row (one column
        // group) are stored in fp16 as O / 2^e, e >= 0 the smallest exponent
        // that brings the group's largest |O| below 2^15; 2^e goes to the
        // row's record for the merge.  The partial so keeps fp16's precision
        // relative to its largest value for any finite input.  The row's
        // 1 / 2^e sits in the staging row's padding.
        pm = fmaxf(pm, __shfl_xor(pm, 32, 64));  // the head's other half of the columns
        // e = max(0, exponent of pm - 15), read off the float's bits (pm =
        // m 2^(E - 126), m in [0.5, 1), E the biased exponent)
        const int sh = max(0, (int)((__float_as_uint(pm) >> 23) & 0xffu) - 141);
        pscale[pass] = __uint_as_float((uint32_t)(127 + sh) << 23);
        _Float16* hbase = (_Float16*)a.part_o + (prow + head0) * D_V;
        // rows of ordinary magnitude (every |O| < 2^15, e = 0: the common
        // case) are converted as they are; the scaled form (rare) is kept
        // as a loop, so that its code stays small
        if (__any(sh > 0)) {
          if (g == 0) stage[n * C::PITCH + ROWF] = __uint_as_float((uint32_t)(127 - sh) << 23);
#pragma unroll 1
          for (int i = 0; i < 32 * ROWF / 512; ++i) {
            const int e = (i * 64 + lane) * 8;
            const int row = e / ROWF, col = e % ROWF;
            const float isc = stage[row * C::PITCH + ROWF];
            const floatx4 v0 = *(const floatx4*)(stage + row * C::PITCH + col);
            const floatx4 v1 = *(const floatx4*)(stage + row * C::PITCH + col + 4);
            halfx8 h;
#pragma unroll
            for (int k = 0; k < 8; ++k) h[k] = (_Float16)((k < 4 ? v0[k] : v1[k - 4]) * isc);
            if (head0 + row < k_hi) __builtin_nontemporal_store(h, (halfx8*)(hbase + (int64_t)row * D_V + col0 + col));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32 * ROWF / 512; ++i) {
            const int e = (i * 64 + lane) * 8;
            const int row = e / ROWF, col = e % ROWF;
            const floatx4 v0 = *(const floatx4*)(stage + row * C::PITCH + col);
            const floatx4 v1 = *(const floatx4*)(stage + row * C::PITCH + col + 4);
            halfx8 h;
#pragma unroll
            for (int k = 0; k < 8; ++k) h[k] = (_Float16)(k < 4 ? v0[k] : v1[k - 4]);
            if (head0 + row < k_hi) __builtin_nontemporal_store(h, (halfx8*)(hbase + (int64_t)row * D_V + col0 + col));
          }
        }
      }
    }
  }
  const float lse_val = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  if (head_ok && lse_ptr && wv == 0 && g == 0) *lse_ptr = lse_val;
  if (head_ok && partial && g == 0) {
#pragma unroll
    for (int k = 0; k < GW; ++k) prec[k] = float2{lse_val, pscale[k]};
  }
  };  // segment

  // ---- the workgroup's segments ----
  // Grid mode: one chunk of request blockIdx.y.  Stream mode: the requests
  // the workgroup's range of the batch's tiles covers, in order.
  const bool stream = a.plan_target > 0;
  StreamPlan sp{0, 0, 0, 0, 0, 0};
  if (stream) {
    sp = a.num_reqs <= 64 ? stream_plan_wave(a) : stream_plan_block<C::NTHREADS>(a, page_lds);
    sp = StreamPlan{__builtin_amdgcn_readfirstlane(sp.A), __builtin_amdgcn_readfirstlane(sp.E),
                    __builtin_amdgcn_readfirstlane(sp.r), __builtin_amdgcn_readfirstlane(sp.V),
                    __builtin_amdgcn_readfirstlane(sp.h), __builtin_amdgcn_readfirstlane(sp.n0)};
    if (sp.r < 0) return;
  }
  const int lo = max(a.tok_lo, 0);
  int r = stream ? sp.r : blockIdx.y;
  int V = sp.V;  // stream mode: first virtual tile of request r's run
  for (int k = 0;; ++k) {
    int t_begin = 0, t_end = 0, b = r;
    int64_t prow = 0;
    bool partial = false;
    if (stream) {
      // next request with real tiles in [A, E) (empty requests have no run;
      // a range may end inside a run's header)
      int nt = k == 0 ? sp.n0 : 0;  // the first request's tiles come with the plan
      if (k > 0)
        while (V < sp.E && r < a.num_reqs && (nt = request_tiles(a, r)) == 0) ++r;
      const int R0 = V + sp.h;  // first real tile of the run
      if (V >= sp.E || r >= a.num_reqs || R0 >= sp.E) break;
      const int s0 = max(sp.A, R0), s1 = min(sp.E, R0 + nt);
      b = r;
      t_begin = lo / kTileTok + (s0 - R0);
      t_end = lo / kTileTok + (s1 - R0);
      partial = s0 != R0 || s1 != R0 + nt;
      prow = (int64_t)(k > 0 ? a.plan_target + blockIdx.x : blockIdx.x) * a.n_heads;  // first or last segment
      V = R0 + nt;
      ++r;
    } else {
      if (k > 0) break;
      const int seq = ((const int32_t __attribute__((address_space(4)))*)a.seq_lens)[b];
      const int hi = min(min(a.tok_hi, seq), a.max_pages << a.page_shift);
      if (hi > lo) {
        const int tf = lo / kTileTok;
        const int nt = (hi + kTileTok - 1) / kTileTok - tf;
        if (a.fixed_splits > 0) {
          // chunk blockIdx.x / fixed_sub of the request's fixed_splits equal
          // chunks, sub-range blockIdx.x % fixed_sub of that chunk
          const int chunk = (nt + a.fixed_splits - 1) / a.fixed_splits;
          const int c = blockIdx.x / a.fixed_sub, k = blockIdx.x - c * a.fixed_sub;
          const int cb = tf + c * chunk, ce = min(cb + chunk, tf + nt);
          const int sub = ce > cb ? (ce - cb + a.fixed_sub - 1) / a.fixed_sub : 0;
          t_begin = cb + k * sub;
          t_end = min(t_begin + sub, ce);
        } else {
          t_begin = tf + blockIdx.x * a.chunk_tiles;
          t_end = min(t_begin + a.chunk_tiles, tf + nt);
        }
      }
      partial = a.grid_partial != 0;
      prow = ((int64_t)blockIdx.x * a.num_reqs + b) * a.n_heads;
    }
    if (k > 0) __syncthreads();  // the previous segment's epilogue is done with LDS
    // the arguments as they lie in the kernel-argument segment (the launch's
    // only argument), read through a pointer the optimiser cannot follow
    typedef const DecodeArgs __attribute__((address_space(4)))* ArgPtr;
    ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    segment(*(const DecodeArgs*)ap, b, t_begin, t_end, prow, partial);
  }
}

template <int D_QK, int D_V, int WH, int WV, bool TBL = false>
hipError_t launch_variant(dim3 grid, const DecodeArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL((decode_attn_kernel<D_QK, D_V, WH, WV, TBL>), grid, dim3(64 * WH * WV), 0, stream, e0, e1, 0,
                        a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeVariant& v, dim3 grid, const DecodeArgs& a, hipStream_t stream, hipEvent_t e0,
                         hipEvent_t e1) {
  if (v.head_tile == 16) return launch_decode16(v, grid, a, stream, e0, e1);
  if (v.d_qk == 576 && v.d_v == 512) {
    if (v.wh == 4 && v.wv == 1) {
      // the table holds kTblTiles tiles and 32-bit offsets in 128-byte units
      if (v.max_chunk_tiles <= kTblTiles && (int64_t)a.num_pages * a.page_stride * 2 <= ((int64_t)1 << 39))
        return launch_variant<576, 512, 4, 1, true>(grid, a, stream, e0, e1);
      return launch_variant<576, 512, 4, 1>(grid, a, stream, e0, e1);
    }
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
