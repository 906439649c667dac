// Internal helpers shared by the treeverify HIP sources (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treeverify.h"

#define TV_API extern "C" __attribute__((visibility("default")))

// A second build of the library (TV_PLAN_VARIANT=1) partitions and orders the work
// differently without changing any result: attention takes the ranked (sequence,
// chunk) order for every batch of two or more, pads its grid with idle workgroups and
// groups its merge rows the other way; expansion splits each logit row into chunks
// four times larger.  Tests demand bit-identical outputs from both builds, which an
// LDS race or an order-dependent reduction would break.
#ifndef TV_PLAN_VARIANT
#define TV_PLAN_VARIANT 0
#endif

namespace tv {

constexpr bool kPlanVariant = TV_PLAN_VARIANT != 0;
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Exclusive prefix sum over the lanes below of a small count 0 <= x < 2^BITS, and the
// wave's total, one ballot per bit: no lane exchanges data (a shuffle scan takes six
// dependent LDS-permute round trips).
template <int BITS>
__device__ __forceinline__ int wave_prefix_small(int x, int& total) {
  int pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const uint64_t m = __ballot((x >> b) & 1);
    pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    tot += __popcll(m) << b;
  }
  total = tot;
  return pre;
}

// a float64 moved across lanes by DPP (both halves with the same control; every lane
// in a row must be active for the patterns used here)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src);
  uint32_t hi = __shfl((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int wave_max_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = shfl_u64(v, lane_id() ^ o);
    v = w > v ? w : v;
  }
  return v;
}

// A dtype argument is one of the two the ABI names.  Its bits are read as an int: a C
// caller may pass any value, and an enum value outside the enumeration must not be
// used as one.
inline bool known_dtype(tv_dtype dt) {
  int v;
  __builtin_memcpy(&v, &dt, sizeof v);
  return v == TV_F32 || v == TV_BF16;
}

// Host-side launch check.
inline tv_status launch_status() {
  return hipGetLastError() == hipSuccess ? TV_OK : TV_ERR_HIP;
}

}  // namespace tv
