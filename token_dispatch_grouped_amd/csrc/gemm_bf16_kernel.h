// Grouped expert GEMMs in bf16 on the gfx950 matrix cores ("grouped expert
// compute", Add MoE expert parallel training runtime, Major changes).
//
// One kernel template covers the six products of the SwiGLU expert FFN,
// forward and backward. For expert e it computes
//     C_e[m, n] = sum_k A_e(m, k) * B_e(n, k)
// where each operand is read either k-contiguous (row-major [rows, K]) or
// transposed (row-major [K, rows]):
//   gate/up fwd   H  = X W_gu^T      A = x_perm [R,d]  B = W_gu[e] [2F,d]   ragged M
//   down fwd      Y  = A W_down^T    A = a [R,F]       B = W_down[e] [d,F]  ragged M
//   down dgrad    dA = dY W_down     A = dy [R,d]      B^T = W_down[e]      ragged M
//   gate/up dgrad dX = dH W_gu       A = dh [R,2F]     B^T = W_gu[e]        ragged M
//   down wgrad    dW_down += dY^T a  A^T = dy, B^T = a                      ragged K
//   gate/up wgrad dW_gu  += dH^T X   A^T = dh, B^T = x_perm                 ragged K
// "Ragged" is the per-expert row count M_e = offsets[e+1] - offsets[e],
// which the host never reads: workgroups find their expert and tile from
// `offsets` on the device, so an expert with no rows gets no tile at all and
// any M_e (0 included) needs no padding.
//
// Tiling: a 512-thread workgroup (8 wavefronts, 2 x 4) computes a 256 x 256
// tile; each wavefront owns a 128 x 64 sub-tile of v_mfma_f32_32x32x16_bf16
// results held in fp32. k advances 64 at a time through a 2-slot LDS ring
// filled by the LDS DMA (global_load_lds_dwordx4; buffer_load_dwordx4 ... lds
// for the weight gradients' operands; tile data never passes through
// registers): the next stage is in flight while the current one is consumed. k-contiguous operands sit in 128-byte LDS rows with an XOR chunk
// swizzle; k-major operands are copied as they are and read through the
// transposing ds_read_b64_tr_b16.
//
// Scheduling: the ragged-M products run persistent, one workgroup per CU,
// each XCD walking a contiguous share of the tiles (groups of 4 row tiles x
// all column tiles) round-robin; the weight gradients run one workgroup per
// tile, experts heaviest first, runs of 8 tiles dealt to the XCDs in snake
// order.
//
// Epilogues: bf16 outputs are staged through LDS and written with 16-byte,
// fully coalesced stores (the MFMA is issued with its operands swapped so
// that each lane holds four consecutive output columns); the plain store
// stages one wavefront row at a time so that the next tile's first stage can
// land in the other ring slot meanwhile. The SwiGLU forward writes h and
// a = silu(gate) * up from the fp32 accumulators, and issues the next
// tile's first stage once h is out; the SwiGLU backward loads its h bands
// into LDS by DMA and rewrites them in place as dH, issuing the next tile's
// first stage during its last band. Weight gradients are read-modify-written
// in fp32, each element by exactly one workgroup (no atomics), one
// fragment's old values loading while the previous fragment is stored.
#pragma once

#include <algorithm>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

enum { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2, EPI_ACC_F32 = 3 };

struct GemmParams {
  const bf16_t *A;
  const bf16_t *B;
  void *C;                // bf16 output, or fp32 accumulator (EPI_ACC_F32)
  bf16_t *C2;             // EPI_SWIGLU_FWD: the activation a
  const bf16_t *H;        // EPI_SWIGLU_BWD: saved h
  const int32_t *offsets;
  const int32_t *order;   // ragged K: experts by descending row count
  int E;
  int M;                  // ragged K: rows of C
  int N;                  // columns of C (EPI_SWIGLU_FWD: F, the gate half)
  int K;                  // ragged M: reduction length
  int64_t lda, ldb, ldc;
  int64_t strideB;        // ragged M: per-expert stride of B
  int64_t strideC;        // ragged K: per-expert stride of C
  int F;
  int n_tiles, m_tiles;
  int total;              // logical workgroups
  // ragged K: columns [mix_cols, N) (128 of them) done by mix_mtiles edge
  // tiles of kEdgeBM x kEdgeBN per expert instead of half-empty BN columns
  int mix_cols, mix_mtiles;
};

MOE_DEVICE int swz(int row) { return (row ^ (row >> 3)) & 7; }


// 16 bytes per lane from global `g` into LDS at the wave-uniform byte address
// `lds_addr` + 16 * lane. Issued from asm so that the compiler adds no waits
// of its own; completion is awaited explicitly (s_waitcnt vmcnt) before the
// workgroup barrier that publishes a stage. The instruction has no register
// results, so nothing is left in flight in a register.
MOE_DEVICE void dma16(const void *g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}

// The same 16 bytes per lane through a buffer resource (base, num_records
// in bytes): lane offsets at or past num_records read zeros. Used for the
// k-major operands of the weight gradients, whose stage base moves on the
// scalar side while the lane offsets stay fixed.
typedef int rsrc_t __attribute__((ext_vector_type(4)));
MOE_DEVICE rsrc_t make_rsrc(const void *base, uint32_t num_records) {
  const uint64_t a = (uint64_t)base;
  rsrc_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int)num_records);
  r.w = 0x00020000;  // 32-bit data format, untyped access
  return r;
}
MOE_DEVICE void bdma16(rsrc_t rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

template <int N>
MOE_DEVICE void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

MOE_DEVICE void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Epilogue shared by the grouped GEMM kernels. With EPI_ACC_F32 the
// accumulators are in MFMA order (lane = column); otherwise in swapped order
// (lane = row, four consecutive columns per accumulator group) and LDS stages
// the tile. EPI_STORE stages one wavefront row (WM rows) at a time at byte
// offset HALF_OFF, so that the LDS below HALF_OFF can already receive the
// next tile's first stage; EPI_SWIGLU_FWD stages the whole tile (BM*BN*2
// bytes) and EPI_SWIGLU_BWD two band buffers (2*BM*BN bytes) from offset 0.
template <int BM, int BN, int WM, int WN, int EPI, int NT, int HALF_OFF, typename NextIssue>
MOE_DEVICE void epilogue(const GemmParams &p, f32x16_t (&acc)[WM / 32][WN / 32], u32x4_t *lds, int e, int m0,
                         int n_tile, int m_valid, int64_t crow0, int wm, int wn, NextIssue issue_next) {
  constexpr int WAVES_M = BM / WM;
  constexpr int WAVES_N = BN / WN;
  constexpr int FM = WM / 32, FN = WN / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  if constexpr (EPI == EPI_ACC_F32) {
    // acc[i][j][v] sits at tile row wm*WM + i*32 + 8*(v/4) + 4*lhi + (v%4),
    // tile column wn*WN + j*32 + l32. Fragment n = i*FN + j is finished as
    // a group of 16: its old values are loaded together (clamped addresses,
    // so no load waits on a branch) while fragment n-1 is written back, so
    // that one group's load latency overlaps the previous group's stores.
    float *C = (float *)p.C + (int64_t)e * p.strideC;
    constexpr int NGR = FM * FN;
    auto load_grp = [&](int n, float (&o)[16]) {
      const int i = n / FN, j = n % FN;
      const int c = n_tile * BN + wn * WN + j * 32 + l32;
      const int cc = c < p.N ? c : p.N - 1;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
        const int rr = r < m_valid ? r : m_valid - 1;
        o[v] = C[(int64_t)(m0 + rr) * p.ldc + cc];
      }
    };
    float cur[16], nxt[16];
    load_grp(0, cur);
#pragma unroll
    for (int n = 0; n < NGR; ++n) {
      if (n + 1 < NGR) load_grp(n + 1, nxt);
      const int i = n / FN, j = n % FN;
      const int c = n_tile * BN + wn * WN + j * 32 + l32;
      // the sums are formed before the conditional stores (the opaque copy
      // keeps the loads from being moved into the store branches, where each
      // would wait for every load in flight)
      float sum[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sum[v] = cur[v] + acc[i][j][v];
        asm volatile("" : "+v"(sum[v]));
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
        if (r < m_valid && c < p.N) C[(int64_t)(m0 + r) * p.ldc + c] = sum[v];
      }
      if (n + 1 < NGR) {
#pragma unroll
        for (int v = 0; v < 16; ++v) cur[v] = nxt[v];
      }
    }
    return;
  } else {  // the bf16 epilogues

  // Swapped layout: acc[i][j][4g + q] is tile row wm*WM + i*32 + l32 and
  // tile column wn*WN + j*32 + 8g + 4*lhi + q (q = 0..3 consecutive).
  // LDS staging: rows of sw bf16 (sw/8 chunks), chunk c of row r stored at
  // chunk c ^ (r & 15).
  bf16_t *stg = reinterpret_cast<bf16_t *>(lds);
  bf16_t *hstg = reinterpret_cast<bf16_t *>(reinterpret_cast<char *>(lds) + HALF_OFF);
  auto stg_off = [](int r, int col, int sw) -> int {  // element offset, col % 4 == 0
    const int c = col >> 3;
    return r * sw + ((c ^ (r & 15)) << 3) + (col & 7);
  };
  auto stg_put4 = [&](bf16_t *base, int r, int col, int sw, float x0, float x1, float x2, float x3) {
    uint2 v;
    v.x = pack_bf2(x0, x1);
    v.y = pack_bf2(x2, x3);
    *reinterpret_cast<uint2 *>(base + stg_off(r, col, sw)) = v;
  };
  // coalesced copy of a staged [WM][SW] row band (tile rows row0 ..) to
  // global memory; col_map gives the destination column of staged column c
  // (a multiple of 8), or -1. Thread t copies chunk t % CPR of rows
  // t / CPR + k * NT / CPR, reading SB chunks from LDS before storing them.
  auto flush = [&](auto sw_c, const bf16_t *base, int row0, bf16_t *dst, int64_t ld, auto col_map) {
    constexpr int SW = decltype(sw_c)::value;
    constexpr int CPR = SW / 8, RSTEP = NT / CPR, ITER = WM / RSTEP, SB = ITER < 4 ? ITER : 4;
    static_assert(NT % CPR == 0 && ITER * RSTEP == WM && ITER % SB == 0, "flush split");
    int t = tid;
    asm volatile("" : "+v"(t));  // addressing stays here, not above the main loop
    const int ch = t % CPR, r0 = t / CPR;
    const int gc = col_map(ch * 8);
    // the thread's rows are RSTEP apart: one row pointer, stepped
    bf16_t *rowp = dst + (crow0 + row0 + r0) * ld + (gc < 0 ? 0 : gc);
    const int64_t step = (int64_t)RSTEP * ld;
#pragma unroll
    for (int k0 = 0; k0 < ITER; k0 += SB) {
      u32x4_t v[SB];
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int r = r0 + (k0 + k) * RSTEP;
        v[k] = *reinterpret_cast<const u32x4_t *>(base + r * SW + ((ch ^ (r & 15)) << 3));
      }
#pragma unroll
      for (int k = 0; k < SB; ++k) {
        const int r = r0 + (k0 + k) * RSTEP;
        if (row0 + r < m_valid && gc >= 0) st16(rowp, v[k]);
        rowp += step;
      }
    }
  };

  if (EPI == EPI_STORE) {
    const int n0 = n_tile * BN;
#pragma unroll
    for (int h = 0; h < WAVES_M; ++h) {
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int r = i * 32 + l32;
              const int col = wn * WN + j * 32 + 8 * g + 4 * lhi;
              stg_put4(hstg, r, col, BN, acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                       acc[i][j][4 * g + 3]);
            }
      }
      __syncthreads();
      flush(std::integral_constant<int, BN>{}, hstg, h * WM, (bf16_t *)p.C, p.ldc,
            [&](int c) { return n0 + c < p.N ? n0 + c : -1; });
      __syncthreads();
    }
  } else if (EPI == EPI_SWIGLU_FWD) {
    // staged h tile from offset 0: gate columns [0, BN/2), up columns [BN/2, BN)
    const int g0 = n_tile * (BN / 2);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = wm * WM + i * 32 + l32;
          const int col = wn * (WN / 2) + j * 32 + 8 * g + 4 * lhi;
          const f32x16_t &ga = acc[i][j];
          const f32x16_t &ua = acc[i][j + FN / 2];
          stg_put4(stg, r, col, BN, ga[4 * g], ga[4 * g + 1], ga[4 * g + 2], ga[4 * g + 3]);
          stg_put4(stg, r, BN / 2 + col, BN, ua[4 * g], ua[4 * g + 1], ua[4 * g + 2], ua[4 * g + 3]);
        }
    __syncthreads();
    if (p.C) {  // NULL when h is not kept (the activations are recomputed later)
#pragma unroll
      for (int h = 0; h < WAVES_M; ++h)
        flush(std::integral_constant<int, BN>{}, stg + h * WM * BN, h * WM, (bf16_t *)p.C, p.ldc, [&](int c) {
          if (c < BN / 2) return g0 + c < p.N ? g0 + c : -1;
          const int g = g0 + c - BN / 2;
          return g < p.N ? p.F + g : -1;
        });
    }
    __syncthreads();
    // the h tile is out: the first half of its staging area takes the next
    // tile's first stage (ring slot 0), the second half the a tile
    issue_next();
    bf16_t *astg = stg + BM * (BN / 2);
    // staged a = silu(gate) * up tile, BN/2 columns
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = wm * WM + i * 32 + l32;
          const int col = wn * (WN / 2) + j * 32 + 8 * g + 4 * lhi;
          const f32x16_t &ga = acc[i][j];
          const f32x16_t &ua = acc[i][j + FN / 2];
          stg_put4(astg, r, col, BN / 2, silu_f(ga[4 * g]) * ua[4 * g], silu_f(ga[4 * g + 1]) * ua[4 * g + 1],
                   silu_f(ga[4 * g + 2]) * ua[4 * g + 2], silu_f(ga[4 * g + 3]) * ua[4 * g + 3]);
        }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < WAVES_M; ++h)
      flush(std::integral_constant<int, BN / 2>{}, astg + h * WM * (BN / 2), h * WM, p.C2, p.F,
            [&](int c) { return g0 + c < p.N ? g0 + c : -1; });
  } else {  // EPI_SWIGLU_BWD: dA -> dH = (dH_gate | dH_up) using the saved h
    // The tile is finished in bands through two LDS buffers. Band b is
    // accumulator row block i = b of every wavefront: tile rows
    // wm * WM + 32 b + (0..31) of both wavefront rows, so every wavefront
    // rewrites its own 32 x WN sub-block of each band. A buffer holds a band's
    // h_gate and h_up, each as eight wavefront sub-blocks [32][WN] with the
    // 16-byte chunks of a sub-block row swizzled by (row & 7).
    // The first wavefront row (the loaders) only loads: h by LDS DMA, each
    // loader fetching its own sub-block and the one below it, so its vmcnt
    // counts loads alone and its own arithmetic needs no other wavefront. The
    // second row (the storers) only stores. Between workgroup barriers:
    //   step 0        loaders: DMA bands 0 and 1, wait for band 0
    //   step 1        everyone: arithmetic of band 0
    //   step 2b       storers: store band b-1; loaders: wait for band b, its arithmetic
    //   step 2b+1     storers: arithmetic of band b; loaders: DMA band b+1 into
    //                 the buffer that band b-1 has just left
    // so that one row's arithmetic runs beside the other row's memory traffic.
    // Once band lb0 (the last one in buffer 0, ring slot 0) is read out, the
    // next tile's first stage is issued there. Rows past m_valid and columns
    // past N are clamped on load and never stored. Every valid h element a
    // workgroup reads lies in its own output tile and is read before the band
    // holding it is stored, so dH may overwrite h in place (p.C == p.H); a
    // clamped row may read an already rewritten row, for a result that is
    // dropped.
    constexpr int NBAND = FM;
    constexpr int SUB = 32 * WN;                  // elements of one wavefront's sub-block
    constexpr int HALF = WAVES_M * WAVES_N * SUB;  // elements of one staged half (= 32 WAVES_M x BN)
    constexpr int BUF = 2 * HALF * 2;             // bytes of one buffer (gate + up)
    constexpr int SCPR = WN / 8;                  // 16-byte chunks per sub-block row
    constexpr int RPQ = 1024 / (WN * 2);          // sub-block rows per DMA instruction
    constexpr int QPS = 32 / RPQ;                 // DMA instructions per sub-block and half
    constexpr int PER_BAND = WAVES_M * QPS * 2;   // DMA instructions per loader and band
    constexpr int BR = WAVES_M * 32;              // rows per band
    constexpr int CPR = BN / 8;
    constexpr int SCH = 2 * BR * CPR / (NT / 2);  // 16-byte chunks per storing thread
    constexpr int SB = 8;                         // chunks read from LDS before storing
    static_assert(SCPR == 8 && RPQ * QPS == 32, "sub-block rows are one 128-byte line");
    static_assert(WAVES_N * 64 == NT / 2 && WAVES_M == 2, "one wavefront row loads, the other stores");
    static_assert(2 * BUF <= 160 * 1024, "two band buffers must fit in LDS");
    static_assert(BUF == HALF_OFF, "band buffer 0 is ring slot 0");
    static_assert(HALF == BR * BN, "band shape");
    static_assert(SCH * (NT / 2) == 2 * BR * CPR && SCH % SB == 0 && (NT / 2) % CPR == 0, "store split");
    const int n0 = n_tile * BN;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wv < WAVES_N;
    const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
    // element offset of (sub-block row sr, logical chunk c) in sub-block sb
    auto sub_off = [](int sb, int sr, int c) { return sb * SUB + sr * WN + ((c ^ (sr & 7)) << 3); };
    // Each use takes an opaque copy of the lane index, so that no band's
    // addressing is computed early (above the main loop or for all bands at
    // once) and held in registers beside the accumulators.
    auto issue_band = [&](int b) {
      int lane_e = lane;
      asm volatile("" : "+v"(lane_e));
      const uint32_t base = lds0 + (uint32_t)((b & 1) * BUF);
#pragma unroll
      for (int h2 = 0; h2 < WAVES_M; ++h2) {
        const int sb = h2 * WAVES_N + wv;
#pragma unroll
        for (int q = 0; q < QPS; ++q) {
          const int sr = q * RPQ + lane_e / SCPR;
          const int ch = (lane_e % SCPR) ^ (sr & 7);
          int gcol = n0 + wv * WN + ch * 8;
          if (gcol > p.N - 8) gcol = p.N - 8;
          int rr = h2 * WM + b * 32 + sr;
          if (rr >= m_valid) rr = m_valid - 1;
          const bf16_t *src = p.H + (crow0 + rr) * p.ldc + gcol;
          const uint32_t off = (uint32_t)((sb * SUB + q * RPQ * WN) * 2);
          dma16(src, base + off);
          dma16(src + p.F, base + (uint32_t)(HALF * 2) + off);
        }
      }
    };
    // the wavefront's own sub-block of band b, h rewritten in place as dH
    auto arith = [&](int b) {
      int lane_e = lane;
      asm volatile("" : "+v"(lane_e));
      const int r = lane_e & 31, hi = lane_e >> 5;
      bf16_t *sg_tile = stg + (b & 1) * (2 * HALF);  // h_gate -> dH_gate
      bf16_t *su_tile = sg_tile + HALF;             // h_up   -> dH_up
      const int sb = wm * WAVES_N + wn;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i != b) continue;
        // the lane's FN*4 groups of four columns (group q = logical chunk q
        // of the sub-block row, half hi); the h of group q+1 is read from LDS
        // before group q is computed and written back, so that the read
        // latency overlaps the arithmetic
        constexpr int NG = FN * 4;
        auto goff = [&](int q) { return sub_off(sb, r, q) + 4 * hi; };
        uint2 hgn = *reinterpret_cast<const uint2 *>(sg_tile + goff(0));
        uint2 hun = *reinterpret_cast<const uint2 *>(su_tile + goff(0));
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const uint2 hg2 = hgn, hu2 = hun;
          if (q + 1 < NG) {
            hgn = *reinterpret_cast<const uint2 *>(sg_tile + goff(q + 1));
            hun = *reinterpret_cast<const uint2 *>(su_tile + goff(q + 1));
          }
          const int j = q >> 2, g = q & 3;
          const float hg[4] = {__uint_as_float(hg2.x << 16), __uint_as_float(hg2.x & 0xffff0000u),
                               __uint_as_float(hg2.y << 16), __uint_as_float(hg2.y & 0xffff0000u)};
          const float hu[4] = {__uint_as_float(hu2.x << 16), __uint_as_float(hu2.x & 0xffff0000u),
                               __uint_as_float(hu2.y << 16), __uint_as_float(hu2.y & 0xffff0000u)};
          float dg[4], du[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            // t = dA s, dH_up = t hg, dH_gate = t hu (1 + hg (1 - s)) = th + th u
            // with th = t hu and u = hg - hg s (s = sigmoid(hg))
            const float sgm = sigmoid_f(hg[v]);
            const float t = acc[i][j][4 * g + v] * sgm;
            const float th = t * hu[v];
            du[v] = t * hg[v];
            dg[v] = fmaf(th, fmaf(-hg[v], sgm, hg[v]), th);
          }
          uint2 og, ou;
          og.x = pack_bf2(dg[0], dg[1]);
          og.y = pack_bf2(dg[2], dg[3]);
          ou.x = pack_bf2(du[0], du[1]);
          ou.y = pack_bf2(du[2], du[3]);
          *reinterpret_cast<uint2 *>(sg_tile + goff(q)) = og;
          *reinterpret_cast<uint2 *>(su_tile + goff(q)) = ou;
        }
      }
    };
    // storers: band b from its buffer to dH, thread st taking chunk st % CPR
    // of rows st / CPR + k * (NT/2) / CPR, gate half first, SB chunks read
    // from LDS before they are stored
    auto store_band = [&](int b) {
      int st = tid - NT / 2;
      asm volatile("" : "+v"(st));
      const bf16_t *buf = stg + (b & 1) * (2 * HALF);
      const int ch = st % CPR;
      const bool col_ok = n0 + ch * 8 < p.N;
#pragma unroll
      for (int k0 = 0; k0 < SCH; k0 += SB) {
        u32x4_t v[SB];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const int c = st + (k0 + k) * (NT / 2);
          const int up = c >= BR * CPR;
          const int r = (c - up * BR * CPR) / CPR;
          const int off = up * HALF + sub_off((r >> 5) * WAVES_N + ch / SCPR, r & 31, ch % SCPR);
          v[k] = *reinterpret_cast<const u32x4_t *>(buf + off);
        }
#pragma unroll
        for (int k = 0; k < SB; ++k) {
          const int c = st + (k0 + k) * (NT / 2);
          const int up = c >= BR * CPR;
          const int r = (c - up * BR * CPR) / CPR;
          const int tr = (r >> 5) * WM + b * 32 + (r & 31);
          if (col_ok && tr < m_valid)
            st16((bf16_t *)p.C + (crow0 + tr) * p.ldc + (up ? p.F : 0) + n0 + ch * 8, v[k]);
        }
      }
    };
    // bands holding a valid row (band b does iff tile row 32 b is valid)
    const int nb = min(NBAND, (m_valid + 31) >> 5);
    const int lb0 = (nb - 1) & ~1;     // last band in buffer 0
    const int next_step = 2 * lb0 + 3;  // first step after its read-out (never, if past 2 nb)
    if (loader) {
      issue_band(0);
      if (nb > 1) {
        issue_band(1);
        wait_vm<PER_BAND>();
      } else {
        wait_vm<0>();
      }
    }
    __syncthreads();
    // unrolled, so that every band index below is a constant and the
    // accumulators stay in registers
#pragma unroll
    for (int s = 1; s <= 2 * NBAND; ++s) {
      if (s > 2 * nb) break;  // uniform
      if (s == next_step) issue_next();
      int band = -1;
      if (s & 1) {
        if (!loader || s == 1) band = s >> 1;
        else if ((s + 1) / 2 < nb) issue_band((s + 1) / 2);
      } else if (!loader) {
        store_band(s / 2 - 1);
      } else if (s / 2 < nb) {
        wait_vm<0>();  // a loader's only loads in flight are band s/2's
        band = s / 2;
      }
      if (band >= 0) arith(band);
      if (s < 2 * nb) __syncthreads();
    }
  }
  }  // the bf16 epilogues
}

constexpr int kGroupM = kGemmGroupM;  // row tiles per group in the ragged-M tile order
// k per LDS stage and ring slots: 64-deep stages make every k-contiguous tile
// row one 128-byte line; two slots of a 256x256 tile fill 128 KB of LDS (a
// 4-slot ring of 32-deep stages measured 5-10% slower on every product).
constexpr int kStageK = 64;
constexpr int kStages = 2;
// Edge tile of the weight gradients whose N is an odd multiple of 128 (F =
// 1408 = 5.5 x 256 for dW_down): the last 128 columns as 512 x 128 tiles
// (the area of a 256 x 256 tile; 4 x 2 wavefronts of 128 x 64; two 80 KB
// stages fill the 160 KB of LDS) instead of 256 x 256 tiles half past the
// edge, which cost a whole tile each: the down weight gradient 4% faster.
constexpr int kEdgeBM = 512, kEdgeBN = 128;

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane s supplies the address of 4 consecutive 16-bit elements of row s/4;
// lane j receives element j%4 of the rows loaded by lanes j/4 + 4q, q = 0..3.
// With row s/4 = k and columns 4*(s%4).. this hands every lane 4 consecutive
// k values of one column.
MOE_DEVICE i16x4_t lds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t *)(p));
}

// One operand's tile in an LDS stage of BK k values, filled by DMA.
//  KM = false: the source is k-contiguous (rows = m or n). The tile is
//    [ROWS][BK] bf16; chunk c of row r sits at c ^ kc_swz(r).
//  KM = true:  the source is k-major (rows = k, contiguous along m or n).
//    The tile is [64][ROWS] bf16; chunk c of row k sits at c ^ 4*(k % 4),
//    which keeps the transposing fragment reads free of bank conflicts.
// Every DMA instruction of a wave writes 1 KB of contiguous LDS.
// Chunk swizzle of a k-contiguous tile row with CPR 16-byte chunks (8 for
// 128-byte rows, 4 for 64-byte rows), conflict-free for the fragment reads.
template <int CPR>
MOE_DEVICE int kc_swz(int r) {
  return CPR == 8 ? swz(r) : ((r >> 2) & 3);
}

// BUF (k-major only): the DMA goes through a buffer resource whose base is
// the stage's first k row, each lane keeping a 32-bit offset, and k rows past
// kdim read zeros from the resource's range check instead of being clamped.
template <int ROWS, bool KM, int NW, int BK, bool BUF = false>
struct Operand {
  static constexpr int NT = NW * 64;
  static constexpr int BYTES = ROWS * BK * 2;
  static constexpr int NDMA = BYTES / (NT * 16);
  static_assert(NDMA * NT * 16 == BYTES, "tile/thread mismatch");
  static constexpr int ROWB = KM ? ROWS * 2 : BK * 2;  // bytes per LDS tile row
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per LDS row
  static constexpr int RPI = 1024 / ROWB;           // LDS rows per DMA instruction
  static_assert(!KM || CPR >= 16, "k-major tiles need at least 128 columns");
  static_assert(!BUF || KM, "buffer DMA is for k-major operands");

  const bf16_t *ptr[NDMA];  // KC: source at k = 0; KM: column base of the lane
  int krow[NDMA];           // KM: k row of the lane within a stage
  const char *kbase;        // BUF: column 0 of the tile at k = 0
  uint32_t voff[NDMA];      // BUF: byte offset of the lane's 16 bytes from a stage's base

  // base: first element of the tile's first row (KC) or of column 0 at k = 0
  // (KM); ld: row pitch; valid: rows (KC) or columns (KM) that exist;
  // row_map(r) (KC only) gives the source row of tile row r.
  template <typename RowMap>
  MOE_DEVICE void init(const bf16_t *base, int64_t ld, int valid, int wave, int lane, RowMap row_map) {
    kbase = reinterpret_cast<const char *>(base);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int r = (i * NW + wave) * RPI + lane / CPR;
      const int phys = lane % CPR;
      if (!KM) {
        const int c = phys ^ kc_swz<CPR>(r);
        ptr[i] = base + (int64_t)row_map(r) * ld + c * 8;
        krow[i] = 0;
      } else {
        const int c = phys ^ (4 * (r & 3));
        int col = c * 8;
        if (col >= valid) col = valid - 8;  // past-the-end columns feed masked outputs only
        ptr[i] = base + col;
        krow[i] = r;
        voff[i] = (uint32_t)(((int64_t)r * ld + col) * 2);  // r < BK: far below 2^32
      }
    }
  }
  // Issue the DMA of stage data at k0 into LDS byte address `dst` (+ wave's
  // 1 KB slices). KM sources clamp k rows to kdim-1; the tail is zeroed later.
  MOE_DEVICE void issue(int k0, int64_t ld, int kdim, uint32_t dst, int wave) const {
    if constexpr (BUF) {
      const int64_t rem = (int64_t)(kdim - k0) * ld * 2;  // bytes of valid rows from k0 on
      const rsrc_t rs = make_rsrc(kbase + (int64_t)k0 * ld * 2, rem > 0xffffffffLL ? 0xffffffffu : (uint32_t)rem);
#pragma unroll
      for (int i = 0; i < NDMA; ++i) bdma16(rs, voff[i], dst + (uint32_t)((i * NW + wave) * 1024));
      return;
    }
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const uint32_t d = dst + (uint32_t)((i * NW + wave) * 1024);
      if (!KM) {
        dma16(ptr[i] + k0, d);
      } else {
        int kk = k0 + krow[i];
        if (kk >= kdim) kk = kdim - 1;
        dma16(ptr[i] + (int64_t)kk * ld, d);
      }
    }
  }
  // 16-deep MFMA fragment of tile rows [rb, rb+32) (KC) or columns
  // [rb, rb+32) (KM) for step ks; `tile` points at the tile in LDS.
  MOE_DEVICE bf16x8_t frag(const char *tile, int rb, int ks, int lane) const {
    if (!KM) {
      const int r = rb + (lane & 31);
      const int c = ks * 2 + (lane >> 5);
      return __builtin_bit_cast(bf16x8_t,
                                *reinterpret_cast<const u32x4_t *>(tile + (r * CPR + (c ^ kc_swz<CPR>(r))) * 16));
    } else {
      const int b = lane & 15, g = lane >> 4;
      const int col = rb + 16 * (g & 1) + 4 * (b & 3);
      const int chunk = col >> 3, half = (col >> 2) & 1;
      const int k_lo = ks * 16 + 8 * (g >> 1) + (b >> 2);
      const int phys = chunk ^ (4 * (b >> 2));  // (k_lo + 4*rd) % 4 == b >> 2
      const char *a0 = tile + k_lo * ROWB + phys * 16 + half * 8;
      const i16x4_t lo = lds_read_tr16(a0);
      const i16x4_t hi = lds_read_tr16(a0 + 4 * ROWB);
      typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;
      const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }
};

// Operands of the ragged-M tile a persistent workgroup computes next.
struct NextTile {
  const bf16_t *Ab;
  const bf16_t *Bb;
  int n_tile, m_valid;
  bool valid;
};

// One output tile: operand set-up, the DMA-fed main loop and the epilogue.
// `pre`: stage 0 of this tile was issued by the previous tile. next_tile(nx)
// describes the workgroup's next tile (same K); the epilogues that free ring
// slot 0 early (plain store: before it starts; SwiGLU forward: once h is
// out; SwiGLU backward: during a last band held in buffer 1) ask for it
// there and issue its stage 0 into slot 0.
template <int BM, int BN, int WM, int WN, int NW, bool AKM, bool BKM, int EPI, bool RAGGED_K, int BK, int STAGES,
          typename NextFn>
MOE_DEVICE void gg_tile(const GemmParams &p, u32x4_t *lds, int e, int m0, int n_tile, int m_valid, int kdim,
                        int64_t crow0, const bf16_t *Ab, const bf16_t *Bb, bool pre, NextFn next_tile) {
  constexpr int NT = NW * 64;
  constexpr int WAVES_N = BN / WN;
  constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_M * WAVES_N == NW, "wavefront grid must cover the tile");
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(EPI != EPI_SWIGLU_FWD || (FN % 2) == 0, "gate/up pairs need an even fragment count");
  static_assert(RAGGED_K == (EPI == EPI_ACC_F32), "weight gradients are the ragged-K products");
  constexpr bool SWAP = EPI != EPI_ACC_F32;
  using OpA = Operand<BM, AKM, NW, BK, RAGGED_K>;
  using OpB = Operand<BN, BKM, NW, BK, RAGGED_K>;
  constexpr int STAGE_BYTES = OpA::BYTES + OpB::BYTES;
  constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  // staging: one wavefront row in ring slot 1 for EPI_STORE, the whole tile
  // for EPI_SWIGLU_FWD and EPI_SWIGLU_BWD (two band buffers)
  constexpr int STG_BYTES = EPI == EPI_STORE ? STAGE_BYTES + WM * BN * 2 : !SWAP ? 0 : BM * BN * 2;
  constexpr int LDS_BYTES = RING_BYTES > STG_BYTES ? RING_BYTES : STG_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one workgroup");
  // opaque copy: nothing derived from the thread index is hoisted out of a
  // persistent tile loop and held in registers across its tiles
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;

  const int n0 = n_tile * BN;

  auto init_ops = [&](OpA &oa, OpB &ob, const bf16_t *A_, const bf16_t *B_, int mv, int nt) {
    const int nb0 = nt * BN;
    oa.init(A_, p.lda, mv, wave, lane, [&](int r) { return r < mv ? r : mv - 1; });
    if (EPI == EPI_SWIGLU_FWD) {
      // B rows of the tile interleave gate and up rows per wavefront column
      ob.init(B_, p.ldb, p.N, wave, lane, [&](int r) {
        const int wcol = r / WN, q = r % WN;
        const int gi = nt * (BN / 2) + wcol * (WN / 2) + (q % (WN / 2));
        const int gc = gi < p.N ? gi : p.N - 1;  // past-the-end columns are masked on output
        return q < WN / 2 ? gc : p.F + gc;
      });
    } else if (!BKM) {
      ob.init(B_ + (int64_t)nb0 * p.ldb, p.ldb, p.N - nb0, wave, lane,
              [&](int r) { return r < p.N - nb0 ? r : p.N - nb0 - 1; });
    } else {
      ob.init(B_ + nb0, p.ldb, p.N - nb0, wave, lane, [&](int r) { return r; });
    }
  };
  OpA opa;
  OpB opb;
  init_ops(opa, opb, Ab, Bb, m_valid, n_tile);

  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int kt) {
    const uint32_t sb = lds0 + (uint32_t)((kt % STAGES) * STAGE_BYTES);
    const int k0 = kt * BK;
    opa.issue(k0, p.lda, kdim, sb, wave_u);
    opb.issue(k0, p.ldb, kdim, sb + OpA::BYTES, wave_u);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (kdim + BK - 1) / BK;
  constexpr int KS = BK / 16;
  bf16x8_t af[2][FM], bfr[2][FN];
  // ragged K: the last stage's rows past kdim are zeroed in the A fragments
  auto load_frags = [&](int stage, int ks, int set, bool tail) {
    const char *sa = reinterpret_cast<const char *>(lds) + (stage % STAGES) * STAGE_BYTES;
    const char *sb = sa + OpA::BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[set][i] = opa.frag(sa, wm * WM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[set][j] = opb.frag(sb, wn * WN + j * 32, ks, lane);
    if (RAGGED_K && tail) {
      const int kbase = stage * BK + ks * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (kbase + q >= kdim) af[set][i][q] = (__bf16)0.0f;
    }
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if (SWAP)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[set][j], af[set][i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[set][i], bfr[set][j], acc[i][j], 0, 0, 0);
      }
  };
  // Issue order inside each step: one MFMA, one LDS read, ... so that the
  // reads for the next step land while MFMAs run.
  constexpr int NREAD = FM * (AKM ? 2 : 1) + FN * (BKM ? 2 : 1);
  constexpr int NMFMA = FM * FN;
  auto interleave = [&]() {
    constexpr int PAIRS = NREAD < NMFMA ? NREAD : NMFMA;
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    if (NMFMA > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - PAIRS, 0);
    if (NREAD > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - PAIRS, 0);
  };

  // A ring of STAGES slots: stages kt+1 .. kt+STAGES-1 are in flight while
  // stage kt is consumed. The barrier of iteration kt sits before its last
  // step: every wave has then read all of stage kt (waited with lgkmcnt) and
  // stage kt+1 has landed, so stage kt+STAGES can be issued into the slot of
  // stage kt.
  constexpr int PER_STAGE = OpA::NDMA + OpB::NDMA;
  // wait until at most `younger` whole stages are still in flight
  auto wait_stages = [&](int younger) {
    if (STAGES > 3 && younger >= 3) wait_vm<3 * PER_STAGE>();
    else if (STAGES > 2 && younger == 2) wait_vm<2 * PER_STAGE>();
    else if (younger == 1) wait_vm<PER_STAGE>();
    else wait_vm<0>();
  };
#pragma unroll
  for (int st = 0; st < STAGES; ++st)
    if (st < nk && !(pre && st == 0)) issue(st);
  wait_stages(min(nk, STAGES) - 1);
  __builtin_amdgcn_s_barrier();
  load_frags(0, 0, 0, nk == 1);

  for (int kt = 0; kt < nk; ++kt) {
    const bool tail = kt == nk - 1;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      mfmas(ks & 1);
      load_frags(kt, ks + 1, (ks + 1) & 1, tail);
      interleave();
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_lds();
    // issued so far: stages up to min(kt+STAGES-1, nk-1); stage kt+1 needed
    wait_stages(min(STAGES - 2, nk - 2 - kt));
    __builtin_amdgcn_s_barrier();
    if (kt + STAGES < nk) issue(kt + STAGES);
    mfmas((KS - 1) & 1);
    // step 0 of stage kt+1 (on the last pass a harmless read of a stale slot,
    // kept unconditional so that it interleaves with the MFMAs above)
    load_frags(kt + 1, 0, 0, kt + 1 == nk - 1);
    interleave();
  }
  __syncthreads();  // every wave is done with the ring before it is reused
  // stage 0 of the next tile (same K) into ring slot 0: the plain store
  // epilogue stays clear of slot 0 throughout, the SwiGLU forward once its
  // h tile is out
  auto issue_next = [&]() {
    NextTile nx;
    next_tile(nx);  // decoded only here, so nothing of it is held through the main loop
    if (nx.valid) {
      OpA na;
      OpB nb;
      init_ops(na, nb, nx.Ab, nx.Bb, nx.m_valid, nx.n_tile);
      na.issue(0, p.lda, kdim, lds0, wave_u);
      nb.issue(0, p.ldb, kdim, lds0 + OpA::BYTES, wave_u);
    }
  };
  if (EPI == EPI_STORE) issue_next();
  epilogue<BM, BN, WM, WN, EPI, NT, STAGE_BYTES>(p, acc, lds, e, m0, n_tile, m_valid, crow0, wm, wn, issue_next);
}

// Grouped GEMM with DMA-fed LDS stages: 2 slots of 64-deep k, the next
// stage in flight while the current one is consumed. A and B are each either
// k-contiguous or k-major (transposed in the fragment reads). Ragged M
// (forward, dgrad) or ragged K (wgrad) over experts.
template <int BM, int BN, int WM, int WN, int NW, bool AKM, bool BKM, int EPI, bool RAGGED_K, int BK, int STAGES>
__global__ __launch_bounds__(NW * 64, 1) void gg_dma_kernel(GemmParams p) {
  constexpr int NT = NW * 64;
  constexpr int WAVES_N = BN / WN;
  constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_M * WAVES_N == NW, "wavefront grid must cover the tile");
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(EPI != EPI_SWIGLU_FWD || (FN % 2) == 0, "gate/up pairs need an even fragment count");
  static_assert(RAGGED_K == (EPI == EPI_ACC_F32), "weight gradients are the ragged-K products");
  constexpr bool SWAP = EPI != EPI_ACC_F32;
  using OpA = Operand<BM, AKM, NW, BK, RAGGED_K>;
  using OpB = Operand<BN, BKM, NW, BK, RAGGED_K>;
  constexpr int STAGE_BYTES = OpA::BYTES + OpB::BYTES;
  constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  // staging: one wavefront row in ring slot 1 for EPI_STORE, the whole tile
  // for EPI_SWIGLU_FWD and EPI_SWIGLU_BWD (two band buffers)
  constexpr int STG_BYTES = EPI == EPI_STORE ? STAGE_BYTES + WM * BN * 2 : !SWAP ? 0 : BM * BN * 2;
  constexpr int LDS_BYTES = RING_BYTES > STG_BYTES ? RING_BYTES : STG_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one workgroup");
  // the weight gradients also run edge tiles, whose ring takes all 160 KB
  __shared__ u32x4_t lds[(RAGGED_K ? 160 * 1024 : LDS_BYTES) / 16];
  if (!RAGGED_K) {
    // Persistent: the grid holds one workgroup per CU, 8-aligned, and XCD x
    // works through its contiguous share of the logical order (xcd_range)
    // round-robin over its nW workgroups, so the tiles in flight on an XCD
    // are consecutive ones. Logical order: groups of kGroupM row tiles,
    // column tile outer inside a group, so the workgroups resident on one
    // XCD share both operands; only the groups that hold real tiles count.
    MTileScan<BM> sc;
    sc.run(p.offsets, p.E);
    const int per = kGroupM * p.n_tiles;
    const int64_t L = min((sc.total + kGroupM - 1) / kGroupM * per, p.total);
    int lo, hi;
    xcd_range(blockIdx.x & 7, L, lo, hi);
    const int nW = gridDim.x >> 3;
    // logical workgroup -> expert, tile rows and column tile; false past the last tile
    auto decode = [&](int bid, int &e, int &m0, int64_t &crow0, int &n_tile, int &m_valid) {
      const int grp = bid / per, rem = bid - grp * per;
      n_tile = rem / kGroupM;
      const int mslot = grp * kGroupM + (rem - n_tile * kGroupM);
      int mt, row0, row1;
      if (!sc.find(mslot, e, mt, row0, row1)) return false;
      m0 = mt * BM;
      crow0 = (int64_t)row0 + m0;
      m_valid = min(BM, row1 - row0 - m0);
      return true;
    };
    bool pre = false;  // this tile's stage 0 is already in flight
    for (int bid = lo + (int)(blockIdx.x >> 3); bid < hi; bid += nW) {
      int e, m0, n_tile, m_valid;
      int64_t crow0;
      if (!decode(bid, e, m0, crow0, n_tile, m_valid)) {
        pre = false;
        continue;
      }
      // the next tile of this workgroup, asked for by the epilogues that
      // issue its first stage early; nvalid reports whether they did
      bool nvalid = false;
      auto next_tile = [&](NextTile &nx) {
        int ne, nm0;
        int64_t ncrow0;
        nx.valid = bid + nW < hi && decode(bid + nW, ne, nm0, ncrow0, nx.n_tile, nx.m_valid);
        nx.Ab = p.A + (nx.valid ? ncrow0 : 0) * p.lda;
        nx.Bb = p.B + (int64_t)(nx.valid ? ne : 0) * p.strideB;
        nvalid = nx.valid;
      };
      gg_tile<BM, BN, WM, WN, NW, AKM, BKM, EPI, RAGGED_K, BK, STAGES>(
          p, lds, e, m0, n_tile, m_valid, p.K, crow0, p.A + crow0 * p.lda, p.B + (int64_t)e * p.strideB, pre,
          next_tile);
      pre = nvalid;
      __syncthreads();  // the epilogue's LDS reads are done before the next tile's DMA
    }
  } else {
    int e, m0, n_tile, m_valid, kdim;
    int64_t crow0;
    const bf16_t *Ab;
    const bf16_t *Bb;
    // experts come heaviest first and the empty ones last, so the tiles of
    // the non-empty experts are the first ones of the logical order
    const int main_e = p.m_tiles * p.n_tiles;
    const int per_e = main_e + p.mix_mtiles;
    const int bid = xcd_snake_runs(blockIdx.x, min(nonempty_experts(p.offsets, p.E) * per_e, p.total));
    if (bid < 0) return;
    const int slot = bid / per_e;
    e = p.order ? p.order[slot] : slot;
    const int r = bid - slot * per_e;
    if constexpr (RAGGED_K) {
      if (r >= main_e) {  // an edge tile: rows [mm0, mm0 + 512) of columns [mix_cols, N)
        const int erow0 = p.offsets[e];
        const int ekdim = p.offsets[e + 1] - erow0;
        if (ekdim <= 0) return;  // empty expert: dW stays bit-identical
        const int mm0 = (r - main_e) * kEdgeBM;
        GemmParams q = p;  // the edge columns as a product of their own
        q.B = p.B + p.mix_cols;
        q.C = (float *)p.C + p.mix_cols;
        q.N = p.N - p.mix_cols;
        auto none = [&](NextTile &nx) { nx.valid = false; };
        gg_tile<kEdgeBM, kEdgeBN, WM, WN, NW, AKM, BKM, EPI, RAGGED_K, BK, STAGES>(
            q, lds, e, mm0, 0, min(kEdgeBM, p.M - mm0), ekdim, 0, p.A + (int64_t)erow0 * p.lda + mm0,
            q.B + (int64_t)erow0 * p.ldb, false, none);
        return;
      }
    }
    const int mt = r / p.n_tiles;
    n_tile = r - mt * p.n_tiles;
    const int row0 = p.offsets[e];
    kdim = p.offsets[e + 1] - row0;
    if (kdim <= 0) return;  // empty expert: dW stays bit-identical
    m0 = mt * BM;
    m_valid = min(BM, p.M - m0);
    crow0 = 0;
    Ab = p.A + (int64_t)row0 * p.lda + m0;      // k-major: column m0 at k = 0
    Bb = p.B + (int64_t)row0 * p.ldb;
    auto none = [&](NextTile &nx) { nx.valid = false; };
    gg_tile<BM, BN, WM, WN, NW, AKM, BKM, EPI, RAGGED_K, BK, STAGES>(p, lds, e, m0, n_tile, m_valid, kdim, crow0,
                                                                     Ab, Bb, false, none);
  }
}

// ---------------------------------------------------------------------------
// host side: the launch of one product
// ---------------------------------------------------------------------------
// Workgroups of a persistent launch on the current device: one per CU, a
// multiple of 8 so that every XCD holds the same number.
inline int persistent_grid() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 8;
    cached[dev] = n / 8 * 8;
  }
  return cached[dev];
}

template <int BM, int BN, int WM, int WN, bool AKM, bool BKM, int EPI, bool RAGGED_K>
hipError_t run_dma(GemmParams p, hipStream_t s) {
  if (p.total <= 0) return hipSuccess;
  constexpr int NW = (BM / WM) * (BN / WN);
  const int grid = RAGGED_K ? (p.total + 63) / 64 * 64 : std::min(persistent_grid(), (p.total + 7) / 8 * 8);
  gg_dma_kernel<BM, BN, WM, WN, NW, AKM, BKM, EPI, RAGGED_K, kStageK, kStages>
      <<<dim3((unsigned)grid), NW * 64, 0, s>>>(p);
  return hipGetLastError();
}

// The gate/up forward (SwiGLU epilogue) and the weight gradients are
// instantiated in gemm_bf16_ilp.hip, which is compiled with the max-ILP
// machine scheduler; every other product in gemm_bf16.hip with the default
// one (each choice the faster of the two for that kernel).
extern template hipError_t run_dma<kGemmBM, kGemmBN, kGemmBM / 2, kGemmBN / 4, false, false, EPI_SWIGLU_FWD, false>(
    GemmParams, hipStream_t);
extern template hipError_t run_dma<kGemmBM, kGemmBN, kGemmBM / 2, kGemmBN / 4, true, true, EPI_ACC_F32, true>(
    GemmParams, hipStream_t);

}  // namespace moe
