// Store: rotate K by the D-point Hadamard, quantise K and V to FP4 E2M1 with
// one UE8M0 scale per 32 elements, and write 17 D / 16-byte cache slots
// (272 bytes at D = 256).
// (vLLM API docs, UltraQuantAttentionImpl: _ensure_on_device builds the pure
// Hadamard, orthonormal and symmetric; _store_kv rotates K and packs K+V into
// FP4/UE8M0 slots of kv_cache (num_blocks, block_size, Hk, slot_size).)
#include "uq_internal.h"

namespace uq {

// LPS lanes per (token, KV head) pair, 64 / LPS pairs per wave: lane s of a
// pair owns elements E s .. E s + E - 1 (E = D / LPS). K is rotated by the
// float64 butterfly (exact under the span condition of the rotation): its
// log2(E) low stages inside the lane, the stages of the lane bits with
// register exchanges (DPP within rows of 16, the gfx950 row swaps for lane
// xor 16 and 32), so no stage goes through the LDS pipe. K is then scaled by
// its block's power of two in float64 and rounded to odd in float32; V is
// scaled in float32, which holds bf16 values and their power-of-two
// multiples exactly. Both are encoded by the E2M1 conversion, so the codes
// are those of the exact scaled values. The amax of a 32-element block spans
// 32 / E lanes; each lane writes E/2 contiguous code bytes of K and of V.
// LPS = 16 (long lane chains, four pairs per wave) for large stores, where
// throughput counts; LPS = 64 (one pair per wave, short chains spread over
// the chip) for the few tokens of a decode step, where latency does.
template <int D, int LPS>
__global__ __launch_bounds__(256) void store_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ cache, const int64_t* __restrict__ slot_mapping,
    int64_t n_pairs, int Hk, int64_t num_slots, int64_t ksn, int64_t ksh,
    int64_t vsn, int64_t vsh) {
  using F = Fmt<D>;
  static_assert(LPS == 16 || LPS == 32 || LPS == 64, "lanes per pair");
  constexpr int E = D / LPS, SPW = 64 / LPS;
  constexpr int LPB = E >= 32 ? 1 : 32 / E;         // lanes per 32-element block
  constexpr int NB = E / 2;                         // code bytes per lane and tensor
  constexpr int NW = NB >= 4 ? NB / 4 : 1;          // 32-bit code words per lane
  static_assert(E >= 2 && E <= 32, "elements per lane");
  const int lane = threadIdx.x & 63, s = lane % LPS;
  const int64_t pair = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * SPW + lane / LPS;
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
    if constexpr (E >= 4) {
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        const uint2 kr = *reinterpret_cast<const uint2*>(kp + 4 * c);
        const uint2 vr = *reinterpret_cast<const uint2*>(vp + 4 * c);
        k[4 * c] = bf16_to_f64(kr.x & 0xFFFF); k[4 * c + 1] = bf16_to_f64(kr.x >> 16);
        k[4 * c + 2] = bf16_to_f64(kr.y & 0xFFFF); k[4 * c + 3] = bf16_to_f64(kr.y >> 16);
        v[4 * c] = bf16_to_f32(vr.x & 0xFFFF); v[4 * c + 1] = bf16_to_f32(vr.x >> 16);
        v[4 * c + 2] = bf16_to_f32(vr.y & 0xFFFF); v[4 * c + 3] = bf16_to_f32(vr.y >> 16);
      }
    } else {
      const uint32_t kr = *reinterpret_cast<const uint32_t*>(kp);
      const uint32_t vr = *reinterpret_cast<const uint32_t*>(vp);
      k[0] = bf16_to_f64(kr & 0xFFFF); k[1] = bf16_to_f64(kr >> 16);
      v[0] = bf16_to_f32(vr & 0xFFFF); v[1] = bf16_to_f32(vr >> 16);
    }
  }
  fwht_lanes<E, LPS>(k, lane);
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

  // codes of elements 2j, 2j + 1 in byte j, low nibble first
  uint32_t kc[NW], vc[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kc[w] = 0;
    vc[w] = 0;
#pragma unroll
    for (int j = 0; j < (E < 8 ? E : 8); j += 2) {
      const int i = 8 * w + j;
      kc[w] |= e2m1_pair(to_f32_odd(k[i] * kinv), to_f32_odd(k[i + 1] * kinv)) << (4 * j);
      vc[w] |= e2m1_pair(v[i] * vinv, v[i + 1] * vinv) << (4 * j);
    }
  }
  if (!write) return;
  uint8_t* dst = cache + ((size_t)slot * Hk + h) * F::kSlot;
  if constexpr (NB == 1) {
    dst[F::kKCode + s] = (uint8_t)kc[0];
    dst[F::kVCode + s] = (uint8_t)vc[0];
  } else if constexpr (NB == 2) {
    reinterpret_cast<uint16_t*>(dst + F::kKCode)[s] = (uint16_t)kc[0];
    reinterpret_cast<uint16_t*>(dst + F::kVCode)[s] = (uint16_t)vc[0];
  } else if constexpr (NB == 4) {
    reinterpret_cast<uint32_t*>(dst + F::kKCode)[s] = kc[0];
    reinterpret_cast<uint32_t*>(dst + F::kVCode)[s] = vc[0];
  } else if constexpr (NB == 8) {
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

// Lanes per pair: 16, or more while that leaves fewer than about one wave
// per SIMD (1024 waves): a lane's chain grows with its share of the D
// elements, and a small grid leaves most of the chip idle. Measured at
// D = 256 (us):
//   tokens x 4 heads   32    256   512   1024  2048  4096
//   LPS 64            2.81  2.95  3.69  5.09  8.19  14.49
//   LPS 32            3.30  3.42  3.49  4.59  6.84  11.76
//   LPS 16            4.19  4.29  4.36  4.52  6.41  10.21
hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  const int64_t pairs = a.N * a.Hk;
  const int lps = pairs <= 1024 ? 64 : (pairs <= 2048 ? 32 : 16);
  const int64_t per_block = 4 * (64 / lps);
  const int64_t blocks = (pairs + per_block - 1) / per_block;
#define UQ_STORE_L(DV, L)                                                                           \
  hipLaunchKernelGGL((store_kernel<DV, L>), dim3((unsigned)blocks), dim3(256), 0, stream, a.key,     \
                     a.value, a.cache, a.slot_mapping, pairs, a.Hk,                                 \
                     a.num_blocks * (int64_t)a.block_size, a.ksn, a.ksh, a.vsn, a.vsh)
#define UQ_STORE(DV)                                   \
  do {                                                 \
    if (lps == 64) UQ_STORE_L(DV, 64);                 \
    else if (lps == 32) UQ_STORE_L(DV, 32);            \
    else UQ_STORE_L(DV, 16);                           \
  } while (0)
  switch (a.D) {
    case 128: UQ_STORE(128); break;
    case 256: UQ_STORE(256); break;
    case 512: UQ_STORE(512); break;
    default: return hipErrorInvalidValue;
  }
#undef UQ_STORE
#undef UQ_STORE_L
  return hipGetLastError();
}

hipError_t launch_hadamard(int D, float* H, hipStream_t stream) {
  hipLaunchKernelGGL(hadamard_kernel, dim3(D), dim3(D), 0, stream, D, H,
                     (float)(1.0 / sqrt((double)D)));
  return hipGetLastError();
}

}  // namespace uq
