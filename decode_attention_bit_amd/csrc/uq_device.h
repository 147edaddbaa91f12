// Device helpers shared by the store and decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uq {

constexpr int kHeadDim = 256;   // the decode path's head dim (128 and 512 are templates too)
constexpr int kTile = 16;        // tokens per decode tile

// Slot format for head dim D (128, 256 or 512): D/2 bytes of K codes, D/2 of
// V codes, then D/32 K scale bytes and D/32 V scale bytes, 17 D / 16 bytes.
template <int D>
struct Fmt {
  static_assert(D == 128 || D == 256 || D == 512, "head dim");
  static constexpr int kSlot = D * 17 / 16;
  static constexpr int kKCode = 0, kVCode = D / 2, kKScale = D, kVScale = D + D / 32;
};

// The float64 nearest 1/sqrt(D): sqrt(2) = 0x1.6a09e667f3bcdp+0 correctly
// rounded, scaled by a power of two where D is an odd power of two.
template <int D>
constexpr double rot_scale() {
  return D == 256 ? 0.0625 : (D == 128 ? 0x1.6a09e667f3bcdp-4 : 0x1.6a09e667f3bcdp-5);
}

typedef int   v8i  __attribute__((ext_vector_type(8)));
typedef float v4f  __attribute__((ext_vector_type(4)));
typedef short v4s  __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bf16_to_f64(uint32_t h16) {
  return (double)__uint_as_float(h16 << 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// 2**k as a double for |k| <= 1022, built from its exponent field.
__device__ __forceinline__ double pow2(int k) {
  return __longlong_as_double((long long)(k + 1023) << 52);
}

// floor(log2(a)) of a normal, positive double, read from the exponent field.
__device__ __forceinline__ int floor_log2(double a) {
  return (int)((__double_as_longlong(a) >> 52) & 0x7FF) - 1023;
}

// The value lane (l xor m) holds, m a power of two below 64, without the LDS
// pipe: DPP quad permutes for m = 1, 2; DPP row shifts and a select for m = 4,
// 8 (a lane with bit m clear reads m lanes up, one with it set m lanes down,
// both inside the lane's row of 16); the gfx950 row / half swaps for m = 16,
// 32 (with both operands the same value, the first result holds the even
// row's (lower half's) value and the second the odd row's (upper half's)).
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t x, int m, int lane) {
  switch (m) {
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
    case 4: {
      const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x104, 0xF, 0xF, false);
      const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
      return (lane & 4) ? dn : up;
    }
    case 8: {
      const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x108, 0xF, 0xF, false);
      const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);
      return (lane & 8) ? dn : up;
    }
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
      return (lane & 16) ? r[0] : r[1];
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      return (lane & 32) ? r[0] : r[1];
    }
  }
}

__device__ __forceinline__ double xor_lane(double v, int m, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = xor_lane_u32((uint32_t)u, m, lane), hi = xor_lane_u32((uint32_t)(u >> 32), m, lane);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// x with its sign bit XORed with flip (0 or the sign bit): -x or x, exactly;
// IEEE subtraction o - x is by definition the sum (-x) + o, so a butterfly's
// upper output needs no separate subtraction.
__device__ __forceinline__ double negate_if(double x, uint32_t flip) {
  const uint64_t u = __double_as_longlong(x) ^ ((uint64_t)flip << 32);
  return __longlong_as_double(u);
}

// D-point Walsh-Hadamard butterfly (unnormalised), D = LPV E, over groups of
// LPV lanes (one vector per group): lane s of a group holds x[E s .. E s +
// E - 1] in v[0 .. E - 1], so index bits below log2(E) live inside a lane and
// the rest are lane bits 0 .. log2(LPV) - 1. Each stage maps (a, b) ->
// (a + b, a - b); the lane stages exchange through registers (xor_lane). In
// float64 the result is exact whenever every +-sum of the inputs fits 53
// bits, which holds for bf16 inputs whose non-zero magnitudes span at most
// 45 - log2(D) binades (37 at D = 256). Fewer lanes per vector trade lane
// exchanges for in-lane stages: better throughput with many vectors, longer
// chains with few. (Lane stages through the LDS pipe instead, one vector per
// wave, took 51 us for a store of 16384 x 4 vectors, and 60 us with register
// exchanges; the query prologue's latency fell from 2.81 to 2.68 us with them.)
template <int E, int LPV>
__device__ __forceinline__ void fwht_lanes(double v[E], int lane) {
#pragma unroll
  for (int m = 1; m < E; m <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (i & m) continue;
      const double a = v[i], b = v[i + m];
      v[i] = a + b;
      v[i + m] = a - b;
    }
  }
  static_assert(LPV == 16 || LPV == 32 || LPV == 64, "lanes per vector");
#pragma unroll
  for (int m = 1; m < LPV; m <<= 1) {
    const uint32_t flip = (lane & m) ? 0x80000000u : 0u;   // upper lane: o - v = (-v) + o
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = negate_if(v[i], flip) + xor_lane(v[i], m, lane);
  }
}

// UE8M0 block exponent: clamp(floor(log2 amax) - 2, -127, 127); -127 for an
// all-zero block (2 is the exponent of E2M1's largest magnitude, 6 = 1.5*2^2).
__device__ __forceinline__ int mx_block_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int e = floor_log2(amax) - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// float32 rounding of x to odd: the float32 next to x whose last bit is 1
// when x is not a float32 (exact otherwise). Rounding that to a format of at
// most 11 significand bits (E2M1, E4M3) then gives the same result as
// rounding x itself (Boldo and Melquiond, round-to-odd), and no threshold
// decision can flip: a value strictly between two float32 values never
// lands on one whose last bit is 0, which every rounding boundary of those
// formats is. Beyond float32's range the result is the largest finite
// float32 of x's sign.
__device__ __forceinline__ float to_f32_odd(double x) {
  const float f = (float)x;                        // nearest
  const double back = (double)f;
  uint32_t u = __float_as_uint(f);
  if (back != x && !(u & 1u)) u += fabs(back) < fabs(x) ? 1u : 0xFFFFFFFFu;   // the odd neighbour toward x
  return __uint_as_float(u);
}

// 4-bit E2M1 codes of two float32 values, a in bits 0-3 and b in bits 4-7:
// magnitude rounded to the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to
// the even code, saturating at 6, bit 3 the sign (also of a zero result).
// The gfx950 conversion at scale 1 follows exactly this rule (checked on
// every rounding boundary and tie, one float32 step either side, signed
// zeros, subnormals and values past 6).
__device__ __forceinline__ uint32_t e2m1_pair(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

typedef short v2s16 __attribute__((ext_vector_type(2)));
// E4M3 (fn) codes of two float32 values, a in bits 0-7, nearest even,
// saturating at 448: the gfx950 conversion rounds to nearest even and is
// exact below 464 but gives NaN above, so the inputs are clamped to
// [-448, 448] first.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.f, 448.f);
  b = __builtin_amdgcn_fmed3f(b, -448.f, 448.f);
  const v2s16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((v2s16){0, 0}, a, b, 1.0f, false);
  return (uint32_t)(uint16_t)r[0];
}

}  // namespace uq
