// Helpers shared by the grouped GEMM kernels (bf16 MFMA and fp32 paths).
#pragma once

#include "common.h"

namespace moe {

// Spread logical workgroups so that consecutive ones (which share their A
// rows) run on the same XCD: hardware hands workgroup b to XCD b % 8.
MOE_DEVICE int xcd_remap(int bid, int grid) { return (bid & 7) * (grid >> 3) + (bid >> 3); }

// Balanced variant for work of uneven cost ordered heaviest first: runs of 8
// consecutive logical workgroups (tiles that share an operand slab) stay on
// one XCD, and successive runs go to successive XCDs, so every XCD receives
// its share of the heavy front of the order. The grid is a multiple of 64.
MOE_DEVICE int xcd_run_remap(int bid) {
  const int xcd = bid & 7, q = bid >> 3;
  return ((((q >> 3) << 3) + xcd) << 3) + (q & 7);
}

// Ragged-M tile lookup: the mslot-th BM-row tile over all experts in order.
// Each lane sums the tiles of four experts, a wavefront scan finds the owner.
// Returns false when mslot is past the last tile.
template <int BM>
MOE_DEVICE bool find_m_tile(const int32_t *__restrict__ offsets, int E, int mslot, int &e_out, int &mt_out) {
  const int lane = threadIdx.x & 63;
  int cnt[4];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane * 4 + q;
    int c = 0;
    if (e < E) c = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    cnt[q] = c;
    sum += c;
  }
  const int inc = wave_inclusive_scan(sum);
  const int exc = inc - sum;
  const bool mine = mslot >= exc && mslot < inc;
  const uint64_t bal = __ballot(mine);
  if (bal == 0ull) return false;
  const int src = __ffsll((unsigned long long)bal) - 1;
  int e = 0, mt = 0;
  if (mine) {
    int r = mslot - exc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (r >= 0 && r < cnt[q]) {
        e = lane * 4 + q;
        mt = r;
      }
      r -= cnt[q];
    }
  }
  e_out = __shfl(e, src, 64);
  mt_out = __shfl(mt, src, 64);
  return true;
}

}  // namespace moe
