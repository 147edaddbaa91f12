// Store: rotate K by the D-point Hadamard, quantise K and V to FP4 E2M1 with
// one UE8M0 scale per 32 elements, and write 17 D / 16-byte cache slots
// (272 bytes at D = 256).
// (vLLM API docs, UltraQuantAttentionImpl: _ensure_on_device builds the pure
// Hadamard, orthonormal and symmetric; _store_kv rotates K and packs K+V into
// FP4/UE8M0 slots of kv_cache (num_blocks, block_size, Hk, slot_size).)
#include "uq_internal.h"

namespace uq {

// One wave per (token, KV head): lane l owns elements E l .. E l + E - 1
// (E = D / 64), so a 32-element scale block is 32 / E consecutive lanes and
// the D/2 code bytes of a region are written as 64 contiguous stores of E/2
// bytes. K is rotated in float64, scaled by its power of two there and
// rounded to odd in float32; V is scaled in float32, which holds bf16 values
// and their power-of-two multiples exactly. Both are encoded by the E2M1
// conversion, so the codes are those of the exact scaled values.
template <int D>
__global__ __launch_bounds__(256) void store_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ cache, const int64_t* __restrict__ slot_mapping,
    int64_t n_pairs, int Hk, int64_t num_slots, int64_t ksn, int64_t ksh,
    int64_t vsn, int64_t vsh) {
  using F = Fmt<D>;
  constexpr int E = F::kPerLane, LPB = 32 / E;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= n_pairs) return;
  const int lane = threadIdx.x & 63;
  const int64_t n = pair / Hk;
  const int h = (int)(pair - n * Hk);
  const int64_t slot = slot_mapping[n];
  if (slot < 0 || slot >= num_slots) return;

  double k[E];
  float v[E];
  const uint16_t* kp = key + n * ksn + h * ksh + E * lane;
  const uint16_t* vp = value + n * vsn + h * vsh + E * lane;
  if constexpr (E == 2) {
    const uint32_t kr = *reinterpret_cast<const uint32_t*>(kp), vr = *reinterpret_cast<const uint32_t*>(vp);
    k[0] = bf16_to_f64(kr & 0xFFFF); k[1] = bf16_to_f64(kr >> 16);
    v[0] = bf16_to_f32(vr & 0xFFFF); v[1] = bf16_to_f32(vr >> 16);
  } else {
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

  fwht_wave<E>(k, lane);
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
    ka = fmax(ka, __shfl_xor(ka, m));
    va = fmaxf(va, __shfl_xor(va, m));
  }
  const int ke = mx_block_exponent(ka);
  const int ve = mx_block_exponent((double)va);
  const double kinv = pow2(-ke);
  const float vinv = (float)pow2(-ve);     // 2**-127 .. 2**127: a float32 value

  uint32_t kc = 0, vc = 0;
#pragma unroll
  for (int i = 0; i < E; i += 2) {
    kc |= e2m1_pair(to_f32_odd(k[i] * kinv), to_f32_odd(k[i + 1] * kinv)) << (4 * i);
    vc |= e2m1_pair(v[i] * vinv, v[i + 1] * vinv) << (4 * i);
  }
  uint8_t* dst = cache + ((size_t)slot * Hk + h) * F::kSlot;
  if constexpr (E == 2) {
    dst[F::kKCode + lane] = (uint8_t)kc;
    dst[F::kVCode + lane] = (uint8_t)vc;
  } else if constexpr (E == 4) {
    reinterpret_cast<uint16_t*>(dst + F::kKCode)[lane] = (uint16_t)kc;
    reinterpret_cast<uint16_t*>(dst + F::kVCode)[lane] = (uint16_t)vc;
  } else {
    reinterpret_cast<uint32_t*>(dst + F::kKCode)[lane] = kc;
    reinterpret_cast<uint32_t*>(dst + F::kVCode)[lane] = vc;
  }
  if (lane % LPB == 0) {
    dst[F::kKScale + lane / LPB] = (uint8_t)(ke + 127);
    dst[F::kVScale + lane / LPB] = (uint8_t)(ve + 127);
  }
}

__global__ void hadamard_kernel(int D, float* __restrict__ H, float v) {
  const int i = blockIdx.x, j = threadIdx.x;
  H[(size_t)i * D + j] = (__popc(i & j) & 1) ? -v : v;
}

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t pairs = a.N * a.Hk;
  const int64_t blocks = (pairs + 3) / 4;
#define UQ_STORE(DV)                                                                         \
  hipLaunchKernelGGL(store_kernel<DV>, dim3((unsigned)blocks), dim3(256), 0, stream, a.key, a.value, \
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
