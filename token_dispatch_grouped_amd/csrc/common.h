// Internal helpers shared by the HIP kernels of the MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define MOE_DEVICE __device__ __forceinline__

namespace moe {

// ---------------------------------------------------------------------------
// element types
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;  // bf16 storage (bit pattern)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

MOE_DEVICE float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (the gfx950 conversion instruction).
MOE_DEVICE bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// two fp32 -> packed bf16 pair (low half = a)
MOE_DEVICE uint32_t pack_bf2(float a, float b) {
  // one two-lane conversion (v_cvt_pk_bf16_f32 with both sources), each
  // element rounded to nearest even as f2bf does
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte chunk
  MOE_DEVICE static void unpack(const u32x4_t &v, float *o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
  }
  MOE_DEVICE static u32x4_t pack(const float *o) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(o[i]);
    return v;
  }
  MOE_DEVICE static float load(const float *p) { return *p; }
  MOE_DEVICE static void store(float *p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  MOE_DEVICE static void unpack(const u32x4_t &v, float *o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  MOE_DEVICE static u32x4_t pack(const float *o) {
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf2(o[2 * i], o[2 * i + 1]);
    return v;
  }
  MOE_DEVICE static float load(const bf16_t *p) { return bf2f(*p); }
  MOE_DEVICE static void store(bf16_t *p, float v) { *p = f2bf(v); }
};

MOE_DEVICE u32x4_t ld16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }
MOE_DEVICE void st16(void *p, const u32x4_t &v) { *reinterpret_cast<u32x4_t *>(p) = v; }

// Non-temporal 16-byte load: for data read once.
MOE_DEVICE u32x4_t ld16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

// Non-temporal 16-byte store: for streams written once and read much later.
MOE_DEVICE void st16_nt(void *p, const u32x4_t &v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}

// ---------------------------------------------------------------------------
// wave-level helpers (64-wide wavefronts)
// ---------------------------------------------------------------------------
constexpr int kWave = 64;

MOE_DEVICE float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

MOE_DEVICE int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// 1 / (1 + e^-z) with the hardware reciprocal (about 1 ulp); e^-z = inf gives 0.
MOE_DEVICE float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
MOE_DEVICE float silu_f(float z) { return z * sigmoid_f(z); }

}  // namespace moe
