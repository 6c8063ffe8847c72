// Split of one token's row of E per-expert values (logits, their gradients)
// over several lanes of a wavefront, shared by the routing and the
// auxiliary-loss kernels.
#pragma once

#include "common.h"

namespace moe {

// Lanes G that share one token's row of E per-expert values (logits, their
// gradients): the smallest power of two that leaves each lane at most eight
// values, at most eight lanes; and the most values V one lane then holds (8,
// or 16 / 32 for rows of more than 64).
constexpr int route_lanes(int E) { return E <= 8 ? 1 : E <= 16 ? 2 : E <= 32 ? 4 : 8; }
constexpr int route_lane_values(int E) { return E <= 64 ? 8 : E <= 128 ? 16 : 32; }
template <int G, int V>
struct RouteLane {
  static constexpr int kValues = V;
  // The row element that value i of lane g holds: with 16-byte rows
  // (E % 4 == 0) the chunks g, g + G, ... of four values, so that the G lanes
  // of a row read consecutive 16-byte chunks; else the values g, g + G, ...
  MOE_DEVICE static int elem(int i, int g, bool vec) { return vec ? 4 * (g + G * (i >> 2)) + (i & 3) : g + G * i; }
  // All of the lane's loads are issued before any is used: one round trip.
  template <typename P>
  MOE_DEVICE static void load(P *__restrict__ row, int E, int g, bool vec, float (&v)[kValues]) {
    if (vec) {
#pragma unroll
      for (int c = 0; c < kValues / 4; ++c) {
        const int e = 4 * (g + G * c);
        const float4 x = e < E ? *reinterpret_cast<const float4 *>(row + e) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[4 * c] = x.x;
        v[4 * c + 1] = x.y;
        v[4 * c + 2] = x.z;
        v[4 * c + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kValues; ++i) {
        const int e = g + G * i;
        v[i] = e < E ? row[e] : 0.f;
      }
    }
  }
};

}  // namespace moe
