// Helpers shared by the grouped GEMM kernels (bf16 MFMA and fp32 paths).
#pragma once

#include "common.h"

namespace moe {

// Hardware hands workgroup b to XCD b % 8. XCD x owns the contiguous logical
// range [lo, hi) = [x*L/8, (x+1)*L/8) of the L logical workgroups that carry
// work, so that consecutive ones (which share operands) run on one XCD and
// every XCD gets the same amount of work even when the launch is sized for
// more.
MOE_DEVICE void xcd_range(int x, int64_t L, int &lo, int &hi) {
  lo = (int)(((int64_t)x * L) >> 3);
  hi = (int)(((int64_t)(x + 1) * L) >> 3);
}

// Balanced variant for work of uneven cost ordered heaviest first: runs of 8
// consecutive logical workgroups (tiles that share an operand slab) stay on
// one XCD, and the runs are dealt to the XCDs in snake order (0..7, 7..0,
// 0..7, ...) over the L logical workgroups that carry work, so that every
// XCD receives an even share of the heavy front of the order. Returns -1
// past the end; needs gridDim.x >= 64 * ceil(L/64).
MOE_DEVICE int xcd_snake_runs(int b, int L) {
  const int x = b & 7, j = b >> 3;
  const int rnd = j >> 3;
  const int run = rnd * 8 + ((rnd & 1) ? 7 - x : x);
  const int bid = run * 8 + (j & 7);
  return bid < L ? bid : -1;
}

// Number of experts with at least one row (E <= 256), wave-uniform.
MOE_DEVICE int nonempty_experts(const int32_t *__restrict__ offsets, int E) {
  const int lane = threadIdx.x & 63;
  int n = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    n += __popcll(__ballot(e < E && offsets[e + 1] > offsets[e]));
  }
  return __builtin_amdgcn_readfirstlane(n);
}

// Ragged-M tiles: BM-row tiles over all experts in expert order. Each lane
// counts the tiles of four experts (E <= 256) and a wavefront scan gives
// every lane the tiles before its experts and the total.
template <int BM>
struct MTileScan {
  int cnt[4];
  int first[5];  // offsets of the lane's four experts and the one after
  int exc, inc;
  int total;  // row tiles over all experts (wave-uniform)

  MOE_DEVICE void run(const int32_t *__restrict__ offsets, int E) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q <= 4; ++q) {
      const int e = lane * 4 + q;
      first[q] = e <= E ? offsets[e] : 0;
    }
    int sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane * 4 + q;
      const int c = e < E ? (first[q + 1] - first[q] + BM - 1) / BM : 0;
      cnt[q] = c;
      sum += c;
    }
    inc = wave_inclusive_scan(sum);
    exc = inc - sum;
    total = __builtin_amdgcn_readfirstlane(__shfl(inc, 63, 64));
  }
  // Expert, tile within it and the expert's row range [row0, row1) of the
  // mslot-th tile; false past the last.
  MOE_DEVICE bool find(int mslot, int &e_out, int &mt_out, int &row0_out, int &row1_out) const {
    const int lane = threadIdx.x & 63;
    const bool mine = mslot >= exc && mslot < inc;
    const uint64_t bal = __ballot(mine);
    if (bal == 0ull) return false;
    const int src = __ffsll((unsigned long long)bal) - 1;
    int e = 0, mt = 0, r0 = 0, r1 = 0;
    if (mine) {
      int r = mslot - exc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (r >= 0 && r < cnt[q]) {
          e = lane * 4 + q;
          mt = r;
          r0 = first[q];
          r1 = first[q + 1];
        }
        r -= cnt[q];
      }
    }
    e_out = __shfl(e, src, 64);
    mt_out = __shfl(mt, src, 64);
    row0_out = __shfl(r0, src, 64);
    row1_out = __shfl(r1, src, 64);
    return true;
  }
};

template <int BM>
MOE_DEVICE bool find_m_tile(const int32_t *__restrict__ offsets, int E, int mslot, int &e_out, int &mt_out) {
  MTileScan<BM> sc;
  sc.run(offsets, E);
  int r0, r1;
  return sc.find(mslot, e_out, mt_out, r0, r1);
}

}  // namespace moe
