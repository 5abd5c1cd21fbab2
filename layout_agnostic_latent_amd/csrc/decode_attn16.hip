// Decode attention for shares of at most 16 query heads per KV head on
// gfx950: a TP rank's slice of the 128 heads over 8 ranks (thelatestinai
// page, Appendix Table 2: TP splits the heads), or every group of 16 query
// heads when G = 8 KV heads serve 128 (weekinpapers page, Abstract: query
// heads sharing a few KV heads).
//
// The score and output tiles are 16 heads wide, on v_mfma_f32_16x16x32_bf16
// (16 x 32 operands, 16 x 16 fp32 results), so no MFMA column is empty.  A
// workgroup of four waves owns (request, chunk of 32-token tiles, 16 heads)
// and shares one LDS ring of KV tiles (the layout and DMA of the wider
// kernel).  Per tile:
//  * scores S^T[tok][head] = K Q^T: wave w computes token half w % 2 over
//    k-half w / 2 (9 MFMAs of 32 dims each); the four 16 x 16 partials meet in
//    LDS, and every wave sums the two k-halves of both token halves in the
//    same order, so all four hold the same 32 x 16 score tile bit for bit;
//  * online softmax in fp32 on exp2 (the running max moved lazily), run by
//    every wave on its copy: 8 scores per lane;
//  * O^T[v][head] += V^T P^T over the wave's 128 V columns (8 MFMAs, k = the
//    tile's 32 tokens), V^T through ds_read_b64_tr_b16, P^T straight from the
//    packed weights in VGPRs.
// Q goes through a free ring slot (coalesced 1-KiB DMAs, then LDS reads), so
// that no vector-memory wait of the compiler's drains the KV prefetch.
//
// Pages cited: the weekinpapers page is "SPLASH: Switching Parallel Layouts of
// Attention with Seamless Handoff for LLM Serving" (weekinpapers.com); the
// thelatestinai page is that paper's summary with its appendix tables
// (thelatestinai.com).
#include "decode_device.h"

namespace splash {
namespace {

template <int D_QK, int D_V>
struct Cfg16 {
  static constexpr int NW = 4;                        // waves
  static constexpr int NTHREADS = 64 * NW;
  static constexpr int NSLAB = D_QK / 64;             // 128-B slabs per KV row
  static constexpr int SLAB_B = kTileTok * 128;       // LDS bytes of one slab of a tile
  static constexpr int TILE_B = NSLAB * SLAB_B;
  static constexpr int NBUF = 4;                      // ring slots: one computed, three in flight
  static constexpr int DMA_W = NSLAB * (kTileTok / 8) / NW;  // 1-KiB DMAs per wave per tile
  static constexpr int KS = D_QK / 32;                // k-steps of the score MFMA
  static constexpr int KSW = KS / 2;                  // ... per wave (one k-half)
  static constexpr int VB = D_V / 16 / NW;            // 16-column V blocks per wave
  static constexpr int COLS = D_V / NW;               // V columns per wave = one partial scale group
  static constexpr int KPF = 4;                       // K operands in flight
  static constexpr int VPF = 4;                       // V operands in flight
  static constexpr int RING_B = NBUF * TILE_B;
  static constexpr int XCH_B = 2 * NW * 64 * 16;      // two buffers of four 16 x 16 fp32 partials
  static constexpr int SMEM_B = RING_B + XCH_B;
  static constexpr int Q_B = 16 * D_QK * 2;           // 16 heads of Q, staged in ring slot 3
  static constexpr int Q_DMA = Q_B / 1024;            // 1-KiB DMAs of the Q block
  static_assert(D_QK % 64 == 0 && KS % 2 == 0, "whole slabs and two k-halves");
  static_assert(D_V % (16 * NW) == 0 && D_V <= D_QK, "V columns over the waves");
  static_assert(COLS == partial_group_cols(D_V, NW), "scale groups as the host lays them out");
  static_assert(NSLAB * (kTileTok / 8) % NW == 0, "DMA split");
  static_assert(Q_B % 1024 == 0 && Q_B <= TILE_B, "Q block in one ring slot");
  static_assert(SMEM_B <= 160 * 1024, "LDS");
  static_assert(KSW >= KPF && VB * 1 >= VPF, "prefetch depth");
};

template <int D_QK, int D_V>
__global__ void __launch_bounds__(256, 1) decode_attn16_kernel(const DecodeArgs a) {
  using C = Cfg16<D_QK, D_V>;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM_B];
  // the plan's scratch: the exchange area, unused until the first tile
  int32_t* const plan_lds = (int32_t*)(smem + C::RING_B);

  // One segment: tiles [t_begin, t_end) of request b, written to the
  // caller's output (partial = false) or to partial row prow + head.  The
  // arguments come through `a`, which the segment loop hides from the
  // optimiser (nothing is held in registers across segments).
  auto segment = [&](const DecodeArgs& a, const int b, const int t_begin, const int t_end, const int64_t prow,
                     const bool partial) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int th = wave & 1;   // token half of the score partial this wave computes
    const int kh = wave >> 1;  // its k-half
    const int g4 = lane >> 4;  // k group of the operands, row group of the results
    const int n = lane & 15;   // head column (B and C operands), token row (A operand of QK)
    const int zk = blockIdx.z / a.z_per_kv;
    const int zz = blockIdx.z - zk * a.z_per_kv;
    const int kvh = a.kv_first + zk;
    const int k_lo = max(a.head_lo, kvh * a.kv_group) - a.head_lo;
    const int k_hi = min(a.head_lo + a.n_heads, (kvh + 1) * a.kv_group) - a.head_lo;
    const uint16_t* kv = a.kv + (int64_t)kvh * D_QK;
    const int head0 = k_lo + zz * 16;  // first head of this workgroup within the share
    const int hs = head0 + n;          // this lane's head
    const bool head_ok = hs < k_hi;
    const int hs_safe = head_ok ? hs : 0;
    const int lo = max(a.tok_lo, 0);
    const int32_t __attribute__((address_space(4)))* bt_row =
        (const int32_t __attribute__((address_space(4)))*)(a.bt + (int64_t)b * a.max_pages);
    const int seq = ((const int32_t __attribute__((address_space(4)))*)a.seq_lens)[b];
    const int hi = min(min(a.tok_hi, seq), a.max_pages << a.page_shift);
    const int mlo = max(lo, t_begin * kTileTok);
    const int mhi = min(hi, t_end * kTileTok);
    const int col0 = wave * C::COLS;  // this wave's V columns [col0, col0 + COLS)

    float* out_row = a.out + ((int64_t)b * a.n_heads + hs_safe) * D_V + col0;
    float* lse_ptr = (!partial && a.lse) ? a.lse + (int64_t)b * a.n_heads + hs_safe : nullptr;
    constexpr int NG = D_V / C::COLS;
    float2* const prec = (float2*)a.part_l + (prow + hs_safe) * NG + wave;

    if (t_end <= t_begin) {  // empty chunk: O = 0, LSE = -inf
      if (head_ok && !partial) {
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb) *(floatx4*)(out_row + 16 * vb + 4 * g4) = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      if (head_ok && lse_ptr && wave == 0 && g4 == 0) *lse_ptr = -INFINITY;
      if (head_ok && partial && g4 == 0) *prec = float2{-INFINITY, 1.0f};
      return;
    }
    const int ntiles = t_end - t_begin;
    const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
    const int ps_mask = (1 << a.page_shift) - 1;
    const int row_b = a.kv_row * 2;
    const bool one_page_per_tile = a.page_shift >= 5;
    const int l8 = lane >> 3;
    bool bad_page = false;

    // The chunk's page ids: in VGPRs (page j0 + 64k + l in lane l of vpg[k])
    // when they fit, else read per tile through the scalar cache.
    const int j0 = mlo >> a.page_shift;
    const int j1 = (mhi - 1) >> a.page_shift;
    const bool pt_vgpr = j1 - j0 < 64 * kVPages;
    int32_t vpg[kVPages];
    auto page_of = [&](int tok) -> int {
      const int idx = (tok >> a.page_shift) - j0;
      int p;
      if (pt_vgpr) {
        p = __builtin_amdgcn_readlane(vpg[0], idx & 63);
#pragma unroll
        for (int k = 1; k < kVPages; ++k) {
          const int q = __builtin_amdgcn_readlane(vpg[k], idx & 63);
          p = (idx >> 6) == k ? q : p;
        }
      } else {
        asm volatile("" ::: "memory");
        p = bt_row[tok >> a.page_shift];
        asm volatile("" ::"s"(p));
      }
      if ((unsigned)p >= (unsigned)a.num_pages) {
        bad_page = true;
        p = 0;
      }
      return p;
    };
    // DMA of absolute tile t into ring slot `slot`: wave w carries rows
    // 8w .. 8w+7 of every slab (rows outside [mlo, mhi) fetch the nearest
    // valid row of the tile, so masked tokens see finite data).  Pages hold
    // 16 or more rows and start at multiples of 16, so the 8 rows of a wave
    // are on one page.
    auto issue_tile = [&](int t, int slot) {
      const int tok0 = t * kTileTok;
      const int rlo = max(mlo - tok0, 0);
      const int rhi1 = min(mhi - tok0, kTileTok) - 1;
      const int R = 8 * wave;
      const int rw = min(max(R, rlo), rhi1);  // the wave's first row, clamped
      const int tokw = tok0 + rw;
      const int p = page_of(tokw);
      const char* wbase = (const char*)(kv + (int64_t)p * a.page_stride + (int64_t)(tokw & ps_mask) * a.kv_row);
      const int row = min(max(R + l8, rlo), rhi1);
      const uint32_t voff = (uint32_t)((row - rw) * row_b + 16 * ((lane & 7) ^ (int)row_swizzle(R + l8)));
      const uint32_t lds = smem_base + slot * C::TILE_B + wave * 1024;
#pragma unroll
      for (int i = 0; i < C::DMA_W; ++i) lds_dma16_s(wbase + 128 * i, voff, lds + i * C::SLAB_B);
    };

    // ---- operand addressing within a ring slot ----
    //  K (A operand of QK), this wave's k-step s (absolute 9 kh + s): row
    //  16 th + n, chunk 4 (9 kh + s) + g4, i.e. slab (9 kh + s) / 2 and
    //  in-slab chunk 4 ((s + kh) & 1) + g4.
    const int krow = 16 * th + n;
    uint32_t kofs[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) kofs[par] = krow * 128 + 16 * ((4u * par + g4) ^ row_swizzle(krow));
    auto kaddr = [&](int s) -> uint32_t { return kofs[(s + kh) & 1] + ((9 * kh + s) >> 1) * C::SLAB_B; };
    //  V^T (A operand of PV): lane (j, q) of 16-lane group g4 reads row
    //  16 h + 4 g4 + j at columns col0 + 16 vb + 4q .. +3 (chunk 2 (vb & 3) +
    //  q / 2 of slab col0 / 64 + vb / 4), and receives after the transpose
    //  column n over those four rows: k-slots 8 g4 + 4h + (0..3) hold tokens
    //  16 h + 4 g4 + (0..3), as P^T's k-slots do below.
    const int trj = n >> 2, trq = lane & 3;
    uint32_t vofs[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 16 * h + 4 * g4 + trj;
        vofs[h][m] = (uint32_t)(r * 128 + 16 * (((2 * m + (trq >> 1)) & 7) ^ (int)row_swizzle(r)) + 8 * (trq & 1));
      }
    auto vread = [&](const char* tile, int vb) -> bf16x8 {
      const char* base = tile + (col0 / 64 + vb / 4) * C::SLAB_B;
      const shortx4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(base + vofs[0][vb & 3]));
      const shortx4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(base + vofs[1][vb & 3]));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // ---- prologue: page ids, Q and the first three tiles ----
    // Order of issue: the page-id loads, then Q's DMAs (latencies
    // overlapped); the compiler's wait for the page ids, at their first use
    // in the tiles' DMA plans, then also covers Q (it cannot count the DMAs).
    if (pt_vgpr) {
      const int32_t* bt_src = a.bt + (int64_t)b * a.max_pages + j0;
#pragma unroll
      for (int k = 0; k < kVPages; ++k) vpg[k] = j0 + 64 * k + lane <= j1 ? bt_src[64 * k + lane] : 0;
    }
    // Q of the 16 heads (contiguous rows) into slot 3: wave w issues DMAs
    // w, w + 4, ...; lanes past the share's last head reread its last row.
    {
      const int qdma = (C::Q_DMA - wave + 3) / 4;  // this wave's Q DMAs
      const char* qsrc = (const char*)(a.q + (int64_t)b * a.q_req_stride + (int64_t)(a.head_lo + head0) * D_QK);
      const int qbytes = (k_hi - head0 < 16 ? k_hi - head0 : 16) * D_QK * 2;
      for (int i = 0; i < qdma; ++i) {
        const int off = (wave + 4 * i) * 1024;
        const uint32_t voff = (uint32_t)min(off + 16 * lane, qbytes - 16);
        lds_dma16_s(qsrc, voff, smem_base + 3 * C::TILE_B + off);
      }
    }
    if (pt_vgpr) {
#pragma unroll
      for (int k = 0; k < kVPages; ++k) asm volatile("" ::"v"(vpg[k]));
    }
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (i < ntiles) issue_tile(t_begin + i, i);
    // Q landed (its DMAs are older than the tiles'), then read into registers
    if (ntiles >= 3) wait_vmcnt<3 * C::DMA_W>();
    else if (ntiles == 2) wait_vmcnt<2 * C::DMA_W>();
    else wait_vmcnt<C::DMA_W>();
    __syncthreads();
    bf16x8 qf[C::KSW];  // B operand: Q[head n][32 (9 kh + s) + 8 g4 .. +8]
    {
      const char* qrow = smem + 3 * C::TILE_B + n * (D_QK * 2) + 16 * g4;
#pragma unroll
      for (int s = 0; s < C::KSW; ++s) qf[s] = *(const bf16x8*)(qrow + 64 * (9 * kh + s));
      if (!head_ok) {
#pragma unroll
        for (int s = 0; s < C::KSW; ++s) qf[s] = bf16x8{};
      }
    }

    // ---- online-softmax state: per head (lane column), per lane's tokens ----
    floatx4 oacc[C::VB];
#pragma unroll
    for (int vb = 0; vb < C::VB; ++vb) oacc[vb] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max (log2 units), the same in every wave
    float l_run = 0.0f;       // this lane's share of the sum of p (for the LSE)
    float lr_run = 0.0f;      // ... of p rounded to bf16, the weights PV uses (normalises O)
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    for (int it = 0; it < ntiles; ++it) {
      // tile it landed for every wave; every wave is done with tile it - 1,
      // whose slot takes tile it + 3 (and, at it = 0, with the Q slot)
      if (it + 2 < ntiles) wait_vmcnt<2 * C::DMA_W>();
      else if (it + 1 < ntiles) wait_vmcnt<C::DMA_W>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (it + 3 < ntiles) issue_tile(t_begin + it + 3, (it + 3) & (C::NBUF - 1));
      const char* tile = smem + (it & (C::NBUF - 1)) * C::TILE_B;

      // scores: this wave's token half over its k-half
      floatx4 sp = {0.f, 0.f, 0.f, 0.f};
      bf16x8 kring[C::KPF];
#pragma unroll
      for (int s = 0; s < C::KPF; ++s) kring[s] = *(const bf16x8*)(tile + kaddr(s));
#pragma unroll
      for (int s = 0; s < C::KSW; ++s) {
        const bf16x8 kf = kring[s % C::KPF];
        if (s + C::KPF < C::KSW) kring[s % C::KPF] = *(const bf16x8*)(tile + kaddr(s + C::KPF));
        sp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sp, 0, 0, 0);
      }
      // the first V operands, independent of the exchange
      bf16x8 vring[C::VPF];
#pragma unroll
      for (int i = 0; i < C::VPF; ++i) vring[i] = vread(tile, i);
      // exchange: partial of wave w at ((buf * 4 + w) * 64 + lane) * 16
      char* xch = smem + C::RING_B + (it & 1) * (C::NW * 64 * 16);
      *(floatx4*)(xch + (wave * 64 + lane) * 16) = sp;
      __syncthreads();
      const floatx4 p0 = *(const floatx4*)(xch + (0 * 64 + lane) * 16);
      const floatx4 p1 = *(const floatx4*)(xch + (1 * 64 + lane) * 16);
      const floatx4 p2 = *(const floatx4*)(xch + (2 * 64 + lane) * 16);
      const floatx4 p3 = *(const floatx4*)(xch + (3 * 64 + lane) * 16);
      // s[e]: token 4 g4 + e (e < 4) or 16 + 4 g4 + e - 4, head n
      float s[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = p0[e] + p2[e];
        s[4 + e] = p1[e] + p3[e];
      }
      // tokens outside the chunk's range (first and last tile only)
      const int tok0 = (t_begin + it) * kTileTok;
      const int rlo = max(mlo - tok0, 0), rhi = min(mhi - tok0, kTileTok);
      if (rlo > 0 || rhi < kTileTok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = (e < 4 ? 0 : 16) + 4 * g4 + (e & 3);
          if (r < rlo || r >= rhi) s[e] = -INFINITY;
        }
      }
      // row max over the tile: the lane's 8, then the head's four lanes
      float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = max_across_halves(mx) * a.scale_log2;
      const bool need = mx > m_run + kRescaleThreshold;
      const float m_new = need ? mx : m_run;
      if (__any(need)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        lr_run *= alpha;
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb) oacc[vb] *= alpha;
      }
      m_run = m_new;
      // weights, their sums, and P^T packed as bf16 (k-slot 8 g4 + e)
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.scale_log2, -m_run));
        l_run += p[e];
      }
      uint32_t pw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2 pair = {(__bf16)p[2 * k], (__bf16)p[2 * k + 1]};
        pw[k] = __builtin_bit_cast(uint32_t, pair);
        lr_run = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lr_run, false);
      }
      const bf16x8 pt = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      // O^T += V^T P^T over the wave's columns
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb) {
        const bf16x8 vf = vring[vb % C::VPF];
        if (vb + C::VPF < C::VB) vring[vb % C::VPF] = vread(tile, vb + C::VPF);
        oacc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pt, oacc[vb], 0, 0, 0);
      }
    }
    if (bad_page && lane == 0) atomicOr(a.dev_err, kDevErrBadPage);

    // ---- epilogue ----
    // the head's sums over its four lanes (tokens 4 g4 + .. of each half)
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    float lr_tot = lr_run + __shfl_xor(lr_run, 16, 64);
    lr_tot += __shfl_xor(lr_tot, 32, 64);
    const float inv = lr_tot > 0.0f ? 1.0f / lr_tot : 0.0f;
    const float lse_val = l_tot > 0.0f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    // lane: head n, columns col0 + 16 vb + 4 g4 + (0..3).  Plain stores: each
    // instruction writes 32- or 64-byte pieces of 16 rows, which L2 merges
    // into whole lines (non-temporal stores sent them out as partial-line
    // writes: 2.4x the bytes, no faster)
    if (!partial) {
      if (head_ok) {
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb) *(floatx4*)(out_row + 16 * vb + 4 * g4) = oacc[vb] * inv;
      }
      if (head_ok && lse_ptr && wave == 0 && g4 == 0) *lse_ptr = lse_val;
    } else {
      // Split-KV partial: the wave's columns (one scale group) in fp16 as
      // O / 2^e, e >= 0 the smallest exponent that brings the group's
      // largest |O| below 2^15; {LSE, 2^e} to the row's record.
      float pm = 0.0f;
#pragma unroll
      for (int vb = 0; vb < C::VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) pm = fmaxf(pm, fabsf(oacc[vb][e] * inv));
      pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
      pm = max_across_halves(pm);
      const int sh = max(0, (int)((__float_as_uint(pm) >> 23) & 0xffu) - 141);
      const float isc = __uint_as_float((uint32_t)(127 - sh) << 23) * inv;
      if (head_ok) {
        _Float16* hrow = (_Float16*)a.part_o + (prow + hs) * D_V + col0;
#pragma unroll
        for (int vb = 0; vb < C::VB; ++vb) {
          typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
          halfx4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (_Float16)(oacc[vb][e] * isc);
          *(halfx4*)(hrow + 16 * vb + 4 * g4) = h;
        }
        if (g4 == 0) *prec = float2{lse_val, __uint_as_float((uint32_t)(127 + sh) << 23)};
      }
    }
  };  // segment

  // ---- the workgroup's segments (as in the wider kernel) ----
  const bool stream = a.plan_target > 0;
  StreamPlan sp{0, 0, 0, 0, 0, 0};
  if (stream) {
    sp = a.num_reqs <= 64 ? stream_plan_wave(a) : stream_plan_block<C::NTHREADS>(a, plan_lds);
    sp = StreamPlan{__builtin_amdgcn_readfirstlane(sp.A), __builtin_amdgcn_readfirstlane(sp.E),
                    __builtin_amdgcn_readfirstlane(sp.r), __builtin_amdgcn_readfirstlane(sp.V),
                    __builtin_amdgcn_readfirstlane(sp.h), __builtin_amdgcn_readfirstlane(sp.n0)};
    if (sp.r < 0) return;
  }
  const int lo = max(a.tok_lo, 0);
  int r = stream ? sp.r : blockIdx.y;
  int V = sp.V;
  for (int k = 0;; ++k) {
    int t_begin = 0, t_end = 0, b = r;
    int64_t prow = 0;
    bool partial = false;
    if (stream) {
      int nt = k == 0 ? sp.n0 : 0;  // the first request's tiles come with the plan
      if (k > 0)
        while (V < sp.E && r < a.num_reqs && (nt = request_tiles(a, r)) == 0) ++r;
      const int R0 = V + sp.h;
      if (V >= sp.E || r >= a.num_reqs || R0 >= sp.E) break;
      const int s0 = max(sp.A, R0), s1 = min(sp.E, R0 + nt);
      b = r;
      t_begin = lo / kTileTok + (s0 - R0);
      t_end = lo / kTileTok + (s1 - R0);
      partial = s0 != R0 || s1 != R0 + nt;
      prow = (int64_t)(k > 0 ? a.plan_target + blockIdx.x : blockIdx.x) * a.n_heads;
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
          const int chunk = (nt + a.fixed_splits - 1) / a.fixed_splits;
          const int c = blockIdx.x / a.fixed_sub, ks = blockIdx.x - c * a.fixed_sub;
          const int cb = tf + c * chunk, ce = min(cb + chunk, tf + nt);
          const int sub = ce > cb ? (ce - cb + a.fixed_sub - 1) / a.fixed_sub : 0;
          t_begin = cb + ks * sub;
          t_end = min(t_begin + sub, ce);
        } else {
          t_begin = tf + blockIdx.x * a.chunk_tiles;
          t_end = min(t_begin + a.chunk_tiles, tf + nt);
        }
      }
      partial = a.grid_partial != 0;
      prow = ((int64_t)blockIdx.x * a.num_reqs + b) * a.n_heads;
    }
    if (k > 0) __syncthreads();  // the previous segment is done with LDS
    typedef const DecodeArgs __attribute__((address_space(4)))* ArgPtr;
    ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    segment(*(const DecodeArgs*)ap, b, t_begin, t_end, prow, partial);
  }
}

}  // namespace

hipError_t launch_decode16(const DecodeVariant& v, dim3 grid, const DecodeArgs& a, hipStream_t stream,
                           hipEvent_t e0, hipEvent_t e1) {
  if (v.d_qk == 576 && v.d_v == 512) {
    hipExtLaunchKernelGGL((decode_attn16_kernel<576, 512>), grid, dim3(256), 0, stream, e0, e1, 0, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace splash
