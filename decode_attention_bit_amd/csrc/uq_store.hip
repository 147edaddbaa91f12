// Store: rotate K by the D-point Hadamard, quantise K and V to FP4 E2M1 with
// one UE8M0 scale per 32 elements, and write 17 D / 16-byte cache slots
// (272 bytes at D = 256).
// (vLLM API docs, UltraQuantAttentionImpl: _ensure_on_device builds the pure
// Hadamard, orthonormal and symmetric; _store_kv rotates K and packs K+V into
// FP4/UE8M0 slots of kv_cache (num_blocks, block_size, Hk, slot_size).)
#include "uq_internal.h"

namespace uq {

// Four (token, KV head) pairs per wave, 16 lanes each: lane s of a pair
// owns elements E s .. E s + E - 1 (E = D / 16). K is rotated by the
// float64 butterfly (exact under the span condition of the rotation): its
// log2(E) low stages inside the lane, the four stages of the lane bits with
// DPP exchanges inside the lane's row of 16, so no stage goes through the
// LDS pipe. K is then scaled by its block's power of two in float64 and
// rounded to odd in float32; V is scaled in float32, which holds bf16 values
// and their power-of-two multiples exactly. Both are encoded by the E2M1
// conversion, so the codes are those of the exact scaled values. The amax of
// a 32-element block spans 32 / E lanes (one at D = 512); each lane writes
// E/2 contiguous code bytes of K and of V.
template <int D>
__global__ __launch_bounds__(256) void store16_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ cache, const int64_t* __restrict__ slot_mapping,
    int64_t n_pairs, int Hk, int64_t num_slots, int64_t ksn, int64_t ksh,
    int64_t vsn, int64_t vsh) {
  using F = Fmt<D>;
  constexpr int E = D / 16, LPB = E >= 32 ? 1 : 32 / E, NW = E / 8;   // NW: 32-bit code words per lane
  const int lane = threadIdx.x & 63, s = lane & 15;
  const int64_t pair = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  int64_t n = 0, slot = -1;
  int h = 0;
  if (pair < n_pairs) {
    n = pair / Hk;
    h = (int)(pair - n * Hk);
    slot = slot_mapping[n];
  }
  const bool write = slot >= 0 && slot < num_slots;

  // every lane runs the exchanges (zeros for a pair it does not write)
  double k[E];
  float v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    k[i] = 0.0;
    v[i] = 0.f;
  }
  if (write) {
    const uint16_t* kp = key + n * ksn + (int64_t)h * ksh + E * s;
    const uint16_t* vp = value + n * vsn + (int64_t)h * vsh + E * s;
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      const uint2 kr = *reinterpret_cast<const uint2*>(kp + 4 * c);
      const uint2 vr = *reinterpret_cast<const uint2*>(vp + 4 * c);
      k[4 * c] = bf16_to_f64(kr.x & 0xFFFF); k[4 * c + 1] = bf16_to_f64(kr.x >> 16);
      k[4 * c + 2] = bf16_to_f64(kr.y & 0xFFFF); k[4 * c + 3] = bf16_to_f64(kr.y >> 16);
      v[4 * c] = bf16_to_f32(vr.x & 0xFFFF); v[4 * c + 1] = bf16_to_f32(vr.x >> 16);
      v[4 * c + 2] = bf16_to_f32(vr.y & 0xFFFF); v[4 * c + 3] = bf16_to_f32(vr.y >> 16);
    }
  }
#pragma unroll
  for (int m = 1; m < E; m <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (i & m) continue;
      const double a = k[i], b = k[i + m];
      k[i] = a + b;
      k[i + m] = a - b;
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const uint32_t flip = (s & m) ? 0x80000000u : 0u;   // upper lane: o - v = (-v) + o
#pragma unroll
    for (int i = 0; i < E; ++i) k[i] = negate_if(k[i], flip) + xor_lane(k[i], m, lane);
  }
#pragma unroll
  for (int i = 0; i < E; ++i) {
    k[i] *= rot_scale<D>();            // 1/16 exact at D = 256; one rounding otherwise
    if (k[i] == 0.0) k[i] = 0.0;       // an exact zero carries no sign: +0
  }

  double ka = 0.0;
  float va = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    ka = fmax(ka, fabs(k[i]));
    va = fmaxf(va, fabsf(v[i]));
  }
#pragma unroll
  for (int m = 1; m < LPB; m <<= 1) {
    ka = fmax(ka, xor_lane(ka, m, lane));
    va = fmaxf(va, __uint_as_float(xor_lane_u32(__float_as_uint(va), m, lane)));
  }
  const int ke = mx_block_exponent(ka);
  const int ve = mx_block_exponent((double)va);
  const double kinv = pow2(-ke);
  const float vinv = (float)pow2(-ve);     // 2**-127 .. 2**127: a float32 value

  uint32_t kc[NW], vc[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kc[w] = 0;
    vc[w] = 0;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const int i = 8 * w + j;
      kc[w] |= e2m1_pair(to_f32_odd(k[i] * kinv), to_f32_odd(k[i + 1] * kinv)) << (4 * j);
      vc[w] |= e2m1_pair(v[i] * vinv, v[i + 1] * vinv) << (4 * j);
    }
  }
  if (!write) return;
  uint8_t* dst = cache + ((size_t)slot * Hk + h) * F::kSlot;
  if constexpr (NW == 1) {
    reinterpret_cast<uint32_t*>(dst + F::kKCode)[s] = kc[0];
    reinterpret_cast<uint32_t*>(dst + F::kVCode)[s] = vc[0];
  } else if constexpr (NW == 2) {
    reinterpret_cast<uint2*>(dst + F::kKCode)[s] = make_uint2(kc[0], kc[1]);
    reinterpret_cast<uint2*>(dst + F::kVCode)[s] = make_uint2(vc[0], vc[1]);
  } else {
    reinterpret_cast<uint4*>(dst + F::kKCode)[s] = make_uint4(kc[0], kc[1], kc[2], kc[3]);
    reinterpret_cast<uint4*>(dst + F::kVCode)[s] = make_uint4(vc[0], vc[1], vc[2], vc[3]);
  }
  if (s % LPB == 0) {
    dst[F::kKScale + (E * s) / 32] = (uint8_t)(ke + 127);
    dst[F::kVScale + (E * s) / 32] = (uint8_t)(ve + 127);
  }
}

__global__ void hadamard_kernel(int D, float* __restrict__ H, float v) {
  const int i = blockIdx.x, j = threadIdx.x;
  H[(size_t)i * D + j] = (__popc(i & j) & 1) ? -v : v;
}

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t pairs = a.N * a.Hk;
  const int64_t blocks = (pairs + 15) / 16;
#define UQ_STORE(DV)                                                                         \
  hipLaunchKernelGGL(store16_kernel<DV>, dim3((unsigned)blocks), dim3(256), 0, stream, a.key, a.value, \
                     a.cache, a.slot_mapping, pairs, a.Hk, a.num_blocks * (int64_t)a.block_size,   \
                     a.ksn, a.ksh, a.vsn, a.vsh)
  switch (a.D) {
    case 128: UQ_STORE(128); break;
    case 256: UQ_STORE(256); break;
    case 512: UQ_STORE(512); break;
    default: return hipErrorInvalidValue;
  }
#undef UQ_STORE
  return hipGetLastError();
}

hipError_t launch_hadamard(int D, float* H, hipStream_t stream) {
  hipLaunchKernelGGL(hadamard_kernel, dim3(D), dim3(D), 0, stream, D, H,
                     (float)(1.0 / sqrt((double)D)));
  return hipGetLastError();
}

}  // namespace uq
