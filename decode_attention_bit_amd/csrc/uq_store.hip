// Store: rotate K by the 256-point Hadamard, quantise K and V to FP4 E2M1 with
// one UE8M0 scale per 32 elements, and write 272-byte cache slots.
// (vLLM API docs, UltraQuantAttentionImpl: _ensure_on_device builds the pure
// Hadamard, orthonormal and symmetric; _store_kv rotates K and packs K+V into
// FP4/UE8M0 slots of kv_cache (num_blocks, block_size, Hk, slot_size).)
#include "uq_internal.h"

namespace uq {

// One wave per (token, KV head): lane l owns elements 4l .. 4l+3, so a 32-
// element scale block is 8 consecutive lanes and the 128 code bytes of a
// region are written as 64 contiguous 2-byte stores.
__global__ __launch_bounds__(256) void store_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ cache, const int64_t* __restrict__ slot_mapping,
    int64_t n_pairs, int Hk, int64_t num_slots, int64_t ksn, int64_t ksh,
    int64_t vsn, int64_t vsh) {
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= n_pairs) return;
  const int lane = threadIdx.x & 63;
  const int64_t n = pair / Hk;
  const int h = (int)(pair - n * Hk);
  const int64_t slot = slot_mapping[n];
  if (slot < 0 || slot >= num_slots) return;

  const uint2 kr = *reinterpret_cast<const uint2*>(key + n * ksn + h * ksh + 4 * lane);
  const uint2 vr = *reinterpret_cast<const uint2*>(value + n * vsn + h * vsh + 4 * lane);
  double k[4] = {bf16_to_f64(kr.x & 0xFFFF), bf16_to_f64(kr.x >> 16),
                 bf16_to_f64(kr.y & 0xFFFF), bf16_to_f64(kr.y >> 16)};
  double v[4] = {bf16_to_f64(vr.x & 0xFFFF), bf16_to_f64(vr.x >> 16),
                 bf16_to_f64(vr.y & 0xFFFF), bf16_to_f64(vr.y >> 16)};

  fwht256_wave(k, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    k[i] *= 0.0625;                    // 1/sqrt(256), exact
    if (k[i] == 0.0) k[i] = 0.0;       // an exact zero carries no sign: +0
  }

  double ka = fmax(fmax(fabs(k[0]), fabs(k[1])), fmax(fabs(k[2]), fabs(k[3])));
  double va = fmax(fmax(fabs(v[0]), fabs(v[1])), fmax(fabs(v[2]), fabs(v[3])));
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    ka = fmax(ka, __shfl_xor(ka, m));
    va = fmax(va, __shfl_xor(va, m));
  }
  const int ke = mx_block_exponent(ka);
  const int ve = mx_block_exponent(va);
  const double kinv = pow2(-ke), vinv = pow2(-ve);

  uint32_t kp = 0, vp = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kp |= e2m1_code(k[i], kinv) << (4 * i);
    vp |= e2m1_code(v[i], vinv) << (4 * i);
  }
  uint8_t* dst = cache + ((size_t)slot * Hk + h) * kSlotBytes;
  reinterpret_cast<uint16_t*>(dst + kKCodeOff)[lane] = (uint16_t)kp;
  reinterpret_cast<uint16_t*>(dst + kVCodeOff)[lane] = (uint16_t)vp;
  if ((lane & 7) == 0) {
    dst[kKScaleOff + (lane >> 3)] = (uint8_t)(ke + 127);
    dst[kVScaleOff + (lane >> 3)] = (uint8_t)(ve + 127);
  }
}

__global__ void hadamard_kernel(int D, float* __restrict__ H, float v) {
  const int i = blockIdx.x, j = threadIdx.x;
  H[(size_t)i * D + j] = (__popc(i & j) & 1) ? -v : v;
}

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t pairs = a.N * a.Hk;
  const int64_t blocks = (pairs + 3) / 4;
  hipLaunchKernelGGL(store_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.key,
                     a.value, a.cache, a.slot_mapping, pairs, a.Hk,
                     a.num_blocks * (int64_t)a.block_size, a.ksn, a.ksh, a.vsn, a.vsh);
  return hipGetLastError();
}

hipError_t launch_hadamard(int D, float* H, hipStream_t stream) {
  hipLaunchKernelGGL(hadamard_kernel, dim3(D), dim3(D), 0, stream, D, H,
                     (float)(1.0 / sqrt((double)D)));
  return hipGetLastError();
}

}  // namespace uq
