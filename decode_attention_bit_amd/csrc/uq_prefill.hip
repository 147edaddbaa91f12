// Continuation prefill: a chunk of q_len new tokens attends to the sequence's
// cached prefix (FP4 in the paged cache) and to itself, causally.
// (vLLM API docs, ultraquant_attn, _ultraquant_continuation_prefill: the
// prefix is dequantised to the query dtype in the rotated basis, the chunk's
// K and the queries are rotated by the Hadamard and cast to the query dtype,
// and a dense causal attention over prefix + chunk aligns query i to absolute
// position cached_len + i.)
//
// Kernels:
//   prefill_vexp_kernel    the largest exponent of each 32-dim block of V,
//                          by parts of the keys;
//   prefill_gather_kernel  builds the operands: dequantised prefix K (and V
//                          for uq_dequant_kv), rotated queries and chunk
//                          keys (float64 butterfly, one rounding to bf16),
//                          the value tiles (fp16, scaled per block);
//   prefill_attn_kernel    flash attention over them on matrix cores
//                          (D = 128, 256), prefill_attn512_kernel at
//                          D = 512, prefill_attn16_kernel at D = 512 over
//                          token-major bf16 values (uq_prefill_attention).
#include "uq_internal.h"

namespace uq {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// bf16 bits of x (float64), nearest-even, in one rounding: x is first
// rounded to float32 by round-to-odd (truncate, then set the last bit if
// anything was cut off). Float32 keeps 16 significand bits more than bf16,
// so the second rounding gives the bf16 value nearest x (the double-rounding
// property of round-to-odd, Boldo and Melquiond 2008). Same exponent range,
// so overflow to infinity and subnormals come out as for x itself.
__device__ __forceinline__ uint32_t bf16_bits_rne(double x) {
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if (fabs((double)f) > fabs(x)) u -= 1;                     // magnitude one step down
  if ((double)__uint_as_float(u) != x) u |= 1;               // sticky bit
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// bf16 bits of the FP4 E2M1 code times 2**e (e = scale byte - 127), built
// from the fields: the value is 1 or 1.5 times a power of two, so it is
// exact, down to bf16's subnormals (2**-133 steps) and up to infinity.
__device__ __forceinline__ uint32_t e2m1_bf16_bits(uint32_t code, int e) {
  const uint32_t m = code & 7u;
  const uint32_t sign = (code & 8u) << 12;
  if (m == 0) return sign;
  const uint32_t half = (m >= 2u) ? (m & 1u) : 0u;          // mantissa 1.5
  const int E = (m < 2u ? -1 : (int)(m >> 1) - 1) + e;      // 0.5 = 1 * 2**-1
  const int biased = E + 127;
  if (biased >= 255) return sign | 0x7F80u;
  if (biased >= 1) return sign | ((uint32_t)biased << 7) | (half << 6);
  return sign | ((2u + half) << (E + 132));                 // value / 2**-133
}

// The FP4 E2M1 code's value times 2**e as float32 (exact while the result is
// a normal float32; ldexp rounds below that).
__device__ __forceinline__ float e2m1_scaled(uint32_t code, int e) {
  const uint32_t m = code & 7u;
  // magnitudes 0, 0.5 (m < 2: m / 2), then (2 + (m & 1)) * 2^(m/2 - 2): 1, 1.5, 2, 3, 4, 6
  const float mag = m < 2u ? 0.5f * (float)m : (float)(2u + (m & 1u)) * (float)(1u << ((m >> 1) - 1)) * 0.5f;
  const float x = __builtin_amdgcn_ldexpf(mag, e);
  return (code & 8u) ? -x : x;
}

// Chunk permutation of dim row `dim` in the tiled value layout. The P.V read
// of 16 consecutive dim rows (64 bytes apart), chunk g of each, then hits
// distinct banks both within each aligned group of 8 rows (128 bytes of
// banks) and across all 16 (256 bytes): the pairs (dim mod 2, swizzle) and
// (dim mod 4, swizzle) are distinct there.
__device__ __forceinline__ int vt_swizzle(int dim) { return ((dim >> 2) ^ (dim >> 1)) & 3; }

// Element offset of (key kk, dim) within one tile of the tiled value layout:
// key 16kb + 4g + i of a tile sits at slot s = i + 4kb of chunk g of its dim
// row (64 bytes per dim row, 32 keys).
__device__ __forceinline__ int vt_tile_offset(int kk, int dim) {
  const int g = (kk & 15) >> 2, s = (kk & 3) + ((kk >> 4) << 2);
  return dim * 32 + 8 * (g ^ vt_swizzle(dim)) + s;
}

// Largest exponent (floor(log2 |v|), or above) of each 32-dim block of the
// values of KV head blockIdx.y over part blockIdx.x of the keys (kVexpParts
// equal parts of 0 .. v_keys - 1): for a cached key the block's scale byte
// bounds it (the largest E2M1 magnitude is 6 = 1.5 * 2^2), for a chunk key
// the bf16 exponent fields of the block's values. -1000 where the part has
// no key. One workgroup per (part, KV head); the value tiles read the parts.
template <int D>
__global__ __launch_bounds__(256) void prefill_vexp_kernel(GatherArgs a) {
  using F = Fmt<D>;
  constexpr int NB = D / 32, PPK = D / 4;    // value blocks; 8-byte pieces per chunk key
  __shared__ int red[NB];
  const int part = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < NB) red[tid] = -1000;
  const int64_t per = (a.v_keys + kVexpParts - 1) / kVexpParts;
  const int64_t k0 = (int64_t)part * per, k1 = min(k0 + per, a.v_keys);
  int em[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) em[b] = -1000;
  // cached keys, one per thread: the block's scale bytes
  for (int64_t key = k0 + tid; key < min(k1, (int64_t)a.n_tok); key += 256) {
    const int phys = a.block_row[key >> a.log2_bs];
    if (phys < 0 || (int64_t)phys >= a.num_blocks) continue;     // read as zeros
    const uint8_t* sp = a.cache + ((((int64_t)phys << a.log2_bs) + (key & ((1 << a.log2_bs) - 1))) * a.Hk + h) *
                                      F::kSlot + F::kVScale;
    uint32_t w[NB / 4];
    if constexpr (NB == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(sp);
    } else if constexpr (NB == 8) {
      const uint2 x = *reinterpret_cast<const uint2*>(sp);
      w[0] = x.x;
      w[1] = x.y;
    } else {
      const uint4 x = *reinterpret_cast<const uint4*>(sp);
      w[0] = x.x;
      w[1] = x.y;
      w[2] = x.z;
      w[3] = x.w;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) em[b] = max(em[b], (int)((w[b >> 2] >> (8 * (b & 3))) & 0xFF) - 127 + 2);
  }
  // chunk keys: thread t takes 8-byte pieces t, t + 256, ... of the part's
  // rows (PPK pieces per key, so its 4 dims 4 (t % PPK) .. stay the same),
  // eight pieces in flight at a time
  const int64_t c0 = max(k0, (int64_t)a.n_tok);
  const int64_t n_pieces = max(k1 - c0, (int64_t)0) * PPK;
  int ec = -1000;
  for (int64_t base = 0; base < n_pieces; base += 8 * 256) {
    uint2 x[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t piece = base + 256 * u + tid;
      ok[u] = piece < n_pieces;
      x[u] = make_uint2(0, 0);
      if (ok[u])
        x[u] = *reinterpret_cast<const uint2*>(a.vsrc + (c0 + piece / PPK - a.n_tok) * a.vs_t +
                                               (int64_t)h * a.vs_h + 4 * (piece % PPK));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!ok[u]) continue;
      const uint32_t m = max(max((x[u].x >> 7) & 0xFF, (x[u].x >> 23) & 0xFF),
                             max((x[u].y >> 7) & 0xFF, (x[u].y >> 23) & 0xFF));
      ec = max(ec, (int)m - 127);
    }
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (em[b] > -1000) atomicMax(&red[b], em[b]);
  if (ec > -1000) atomicMax(&red[(4 * (tid % PPK)) / 32], ec);
  __syncthreads();
  if (tid < NB) a.vexp_part[((int64_t)h * kVexpParts + part) * NB + tid] = red[tid];
}

// fp16 bits of x (float32) rounded to nearest-even.
__device__ __forceinline__ uint32_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// One 32-key tile of the tiled values of KV head h, built by a whole
// workgroup (4 waves, 8 keys each) in LDS and written out as contiguous
// 16-byte stores, so that each dim row reaches memory whole. Lane l holds
// dims D/64 l .. D/64 l + D/64 - 1 of a key: from the cache for keys below
// n_tok (codes and scale byte of those dims), from vsrc for the chunk's keys
// up to v_keys, zero past them. Each value v of 32-dim block b is stored as
// fp16(v * 2^-shift_b), shift_b = (largest exponent of the block over all
// keys) - 14, so the block's largest magnitude lands below 2^15: exact for
// every value whose last significant bit is at least 2^(shift_b - 24), i.e.
// within about 2^38 (cached) or 2^31 (chunk) of the block's largest; smaller
// ones round to fp16's subnormals (absolute error at most 2^(shift_b - 25)).
template <int D>
__device__ __forceinline__ void value_tile(const GatherArgs& a, int h, int64_t j) {
  using F = Fmt<D>;
  constexpr int DL = D / 64;                 // dims per lane: 2, 4 or 8
  constexpr int NB = D / 32;
  __shared__ uint16_t img[32 * D];
  __shared__ int sh[NB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < NB) sh[tid] = -1000;
  __syncthreads();
  // the blocks' exponents over the kVexpParts parts are requested first,
  // then the lane's raw values of its 8 keys (codes and exponent of a cached
  // key, bf16 bits of a chunk key), so that both round trips overlap
  constexpr int NPT = kVexpParts * NB / 256;   // part entries per thread
  static_assert(NPT * 256 == kVexpParts * NB, "part entries");
  int pe[NPT];
  const int32_t* pp = a.vexp_part + (int64_t)h * kVexpParts * NB;
#pragma unroll
  for (int i = 0; i < NPT; ++i) pe[i] = pp[tid + 256 * i];
  uint32_t raw[8][DL / 2];
  int ek[8], kind[8];                        // kind: 0 zero, 1 cached, 2 chunk
#pragma unroll
  for (int kk0 = 0; kk0 < 8; ++kk0) {
    const int64_t key = 32 * j + 8 * wave + kk0;
    kind[kk0] = 0;
    ek[kk0] = 0;
#pragma unroll
    for (int i = 0; i < DL / 2; ++i) raw[kk0][i] = 0;
    if (key < a.n_tok) {
      const int phys = a.block_row[key >> a.log2_bs];
      if (phys >= 0 && (int64_t)phys < a.num_blocks) {
        const uint8_t* slot =
            a.cache + ((((int64_t)phys << a.log2_bs) + (key & ((1 << a.log2_bs) - 1))) * a.Hk + h) * F::kSlot;
        raw[kk0][0] = DL == 8   ? *reinterpret_cast<const uint32_t*>(slot + F::kVCode + 4 * lane)
                      : DL == 4 ? *reinterpret_cast<const uint16_t*>(slot + F::kVCode + 2 * lane)
                                : slot[F::kVCode + lane];
        ek[kk0] = (int)slot[F::kVScale + (DL * lane) / 32] - 127;
        kind[kk0] = 1;
      }
    } else if (key < a.v_keys) {
      const uint16_t* src = a.vsrc + (key - a.n_tok) * a.vs_t + (int64_t)h * a.vs_h + DL * lane;
      if constexpr (DL >= 4) {
#pragma unroll
        for (int c = 0; c < DL / 4; ++c) {
          const uint2 y = *reinterpret_cast<const uint2*>(src + 4 * c);
          raw[kk0][2 * c] = y.x;
          raw[kk0][2 * c + 1] = y.y;
        }
      } else {
        raw[kk0][0] = *reinterpret_cast<const uint32_t*>(src);
      }
      kind[kk0] = 2;
    }
  }
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (pe[i] > -1000) atomicMax(&sh[(tid + 256 * i) % NB], pe[i]);
  __syncthreads();
  if (j == 0 && tid < NB) a.vshift[h * NB + tid] = sh[tid] > -1000 ? sh[tid] - 14 : 0;
  const int shift = sh[(DL * lane) / 32] > -1000 ? sh[(DL * lane) / 32] - 14 : 0;
#pragma unroll
  for (int kk0 = 0; kk0 < 8; ++kk0) {
    const int kk = 8 * wave + kk0;
    float v[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      if (kind[kk0] == 1)        // code value times 2^(e - shift), see e2m1_scaled
        v[i] = e2m1_scaled((raw[kk0][0] >> (4 * i)) & 0xF, ek[kk0] - shift);
      else if (kind[kk0] == 2)
        v[i] = __builtin_amdgcn_ldexpf(__uint_as_float(((raw[kk0][i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << 16),
                                       -shift);
      else
        v[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < DL; ++i)
      img[vt_tile_offset(kk, DL * lane + i)] = (uint16_t)f16_bits(v[i]);
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(a.vt + ((int64_t)h * a.vt_tiles + j) * 32 * D);
  const uint4* srcl = reinterpret_cast<const uint4*>(img);
#pragma unroll
  for (int i = 0; i < 4 * D / 256; ++i) dst[256 * i + threadIdx.x] = srcl[256 * i + threadIdx.x];
}

// ---------------------------------------------------------------------------
// Gather. With tiled values (the continuation prefill) the first Hk * vt_tiles
// workgroups each build one value tile (value_tile). After them, waves with
// a role chosen by the wave's index (wave-uniform): first one wave per prefix
// slot (token, KV head) to dequantise, then up to three jobs over vectors of
// D bf16 (rotate or copy), four vectors per wave.
// Dequant: lanes 0-31 write K elements D/32 l .. D/32 l + D/32 - 1, lanes
// 32-63 the same V elements (token-major values only); each reads the code
// bytes and the one scale byte that cover them (D/32 <= 16 consecutive
// elements never straddle a 32-element block).
// Rotate: 16 lanes per vector; lane s of a vector holds x[D/16 s .. D/16 s +
// D/16 - 1] through the float64 butterfly (its low stages inside the lane,
// the four lane stages with register exchanges within the row of 16), then
// the float64 nearest 1/sqrt(D) and one rounding to bf16. (One vector per
// wave with the lane stages through the LDS pipe took 53 us for the gather
// of the 4096 + 2048-token prefill at D = 256.)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void prefill_gather_kernel(GatherArgs a) {
  using F = Fmt<D>;
  constexpr int EPL = D / 32;              // dequantised elements per lane
  constexpr int NCB = EPL / 2;             // code bytes per lane: 2, 4 or 8
  constexpr int E = D / 16;                // vector-job elements per lane: 8, 16 or 32
  int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  {
    if (a.vt) {                              // workgroup-uniform
      const int64_t n_vt = (int64_t)a.Hk * a.vt_tiles;
      if ((int64_t)blockIdx.x < n_vt) {
        value_tile<D>(a, (int)(blockIdx.x / a.vt_tiles), (int64_t)blockIdx.x % a.vt_tiles);
        return;
      }
      w -= 4 * n_vt;
    }
  }
  const int64_t n_slots = (int64_t)a.n_tok * a.Hk;
  if (w < n_slots) {
    const int64_t t = w / a.Hk;
    const int h = (int)(w - t * a.Hk);
    const int64_t entry = t >> a.log2_bs;
    const int phys = a.block_row[entry];
    const bool ok = phys >= 0 && (int64_t)phys < a.num_blocks;
    const bool is_v = lane >= 32;
    const int l = lane & 31;
    uint64_t codes = 0;
    int e = 0;
    if (ok) {
      const uint8_t* slot =
          a.cache + ((((int64_t)phys << a.log2_bs) + (t & ((1 << a.log2_bs) - 1))) * a.Hk + h) * F::kSlot;
      const uint8_t* src = slot + (is_v ? F::kVCode : F::kKCode) + NCB * l;
      if constexpr (NCB == 2)
        codes = *reinterpret_cast<const uint16_t*>(src);
      else if constexpr (NCB == 4)
        codes = *reinterpret_cast<const uint32_t*>(src);
      else
        codes = *reinterpret_cast<const uint64_t*>(src);
      e = (int)slot[(is_v ? F::kVScale : F::kKScale) + (EPL * l) / 32] - 127;
    }
    uint32_t o[NCB];
#pragma unroll
    for (int i = 0; i < NCB; ++i)
      o[i] = ok ? (e2m1_bf16_bits((uint32_t)(codes >> (8 * i)) & 0xF, e) |
                   (e2m1_bf16_bits((uint32_t)(codes >> (8 * i + 4)) & 0xF, e) << 16))
                : 0u;
    if (is_v && a.vt) return;                // the value tiles hold V
    uint16_t* dst = (is_v ? a.vout : a.kout) + t * a.os_t + (int64_t)h * a.os_h + EPL * l;
    if constexpr (NCB == 2) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
    } else {
#pragma unroll
      for (int i = 0; i < NCB / 4; ++i)
        *reinterpret_cast<uint4*>(dst + 8 * i) = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    }
    return;
  }
  w -= n_slots;
  const int s = lane & 15;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const VecJob& jb = a.job[j];
    const int64_t jw = (jb.n + 3) / 4;     // the job's waves
    if (w >= jw) {
      w -= jw;
      continue;
    }
    const int64_t vec = 4 * w + (lane >> 4);
    const bool valid = vec < jb.n;         // lanes of a missing vector run the exchanges on zeros
    const int64_t t = valid ? vec / jb.H : 0;
    const int h = valid ? (int)(vec - t * jb.H) : 0;
    // E bf16 per lane in 8-byte loads (the rows are only 8-byte aligned)
    const uint16_t* sp = jb.src + t * jb.ss_t + (int64_t)h * jb.ss_h + E * s;
    uint32_t r[E / 2];
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const uint2 x = valid ? *reinterpret_cast<const uint2*>(sp + 4 * i) : make_uint2(0, 0);
      r[2 * i] = x.x;
      r[2 * i + 1] = x.y;
    }
    if (jb.rotate) {
      double v[E];
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = bf16_to_f64((r[i >> 1] >> (16 * (i & 1))) & 0xFFFF);
      fwht_lanes<E, 16>(v, lane);
#pragma unroll
      for (int i = 0; i < E / 2; ++i)
        r[i] = bf16_bits_rne(v[2 * i] * rot_scale<D>()) | (bf16_bits_rne(v[2 * i + 1] * rot_scale<D>()) << 16);
    }
    if (!valid) return;
    uint16_t* dp = jb.dst + t * jb.ds_t + (int64_t)h * jb.ds_h + E * s;
#pragma unroll
    for (int i = 0; i < E / 4; ++i) *reinterpret_cast<uint2*>(dp + 4 * i) = make_uint2(r[2 * i], r[2 * i + 1]);
    return;
  }
}

// ---------------------------------------------------------------------------
// Attention. Workgroup = (block of query positions, KV head); its 128 columns
// are (position, query head) pairs of that KV head, column c -> position
// p0 + c / QG, head hk * QG + c % QG, so the QG heads sharing a KV head share
// every K/V tile. Wave w owns columns 16 CB w .. 16 CB w + 16 CB - 1 as CB
// 16-column blocks (CB = 1: eight waves, two per SIMD). Keys stream in tiles
// of 32 through a kStages-deep LDS ring filled by direct-to-LDS buffer loads
// (each wave moves its share of the 32 rows of K and of V, 1 KB per load);
// the rows are 2 D bytes with their 16-byte chunks permuted (chunk c of row r
// stored at c ^ f(r)) so that the reads below hit distinct banks: f(r) =
// r & 15 for K, ((r >> 2) & 3) << 2 for token-major V (tiled values: by dim,
// see vt_swizzle).
//
// V_MFMA_F32_16X16X32_BF16, lane l: row/col l%16, k-slots (l/16, 0..7);
// result lane l: col l%16, rows 4*(l/16) + i. Which k a slot stands for is
// free as long as both operands agree:
//   S^T (keys x cols) = K Q^T: A = K rows, slot (g, i) = d 32j + 8g + i for
//     step j (16 contiguous bytes of a K row), B = the same d of the query
//     (held in registers). The result leaves lane (col, g) with keys
//     16kb + 4g + i of its column.
//   O (cols x dims) += P V: slot (g, s) = key 4g + s (s < 4) or
//     16 + 4g + s - 4, exactly the keys lane (col, g) holds, so P as the A
//     operand needs no data movement. B = V: lane (r, g) reads the dword
//     holding dims 32b + 2r, 2r + 1 of those 8 keys and feeds two MFMAs, one
//     for the even dims (col r -> dim 32b + 2r) and one for the odd ones.
//     Rows of O are query columns, so a rescale is diag(f) O (see below).
// Online softmax in the log2 domain with a reference maximum that is only
// raised when a tile exceeds it by more than 8 (weights stay <= 2^8). With
// tiled values the weights enter P.V as fp16 against the fp16 value tiles
// (V_MFMA_F32_16X16X32_F16, same lane layouts); with token-major values each
// weight enters as a high and a low bf16 part (two MFMAs). The denominator
// sums exactly the weights the product uses.
// ---------------------------------------------------------------------------
// Matrix-core and buffer builtins behind plain functions: the attention
// kernel is a template over the head dim, and a builtin call whose operands
// depend on a template parameter keeps the host pass from emitting the
// kernel's launch stub.
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f32x4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int nrec) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, nrec, 0x00020000);
}
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint4* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}

constexpr int kKeyTile = 32;
constexpr int kColsPerWg = 128;
constexpr int kStages = 4;


// s_waitcnt on vector memory only (gfx9 encoding; expcnt and lgkmcnt left free)
#define UQP_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 0xF) | (((n) >> 4) << 14)) | (0x7 << 4) | (0xF << 8))

// Wait until at most min(K, ahead) tiles are still in flight (the waitcnt
// immediate must be a constant).
template <int K, int PER_TILE>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if constexpr (K == 0) {
    UQP_WAIT_VMCNT(0);
  } else {
    if (ahead >= K) {
      UQP_WAIT_VMCNT(K * PER_TILE);
    } else {
      wait_tiles<K - 1, PER_TILE>(ahead);
    }
  }
}

__device__ __forceinline__ float rowgroup_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// VT: values in the tiled layout the gather writes (one 16 KB block per tile
// and head, dim-major), so that a lane's 8 keys of one dim are one 16-byte
// read and O's columns are dims directly; otherwise values are token-major
// like the keys and each read dword feeds an even-dim and an odd-dim MFMA.
#ifndef UQ_PREFILL_CB
#define UQ_PREFILL_CB 1
#endif
constexpr int CB = UQ_PREFILL_CB;           // 16-column blocks per wave: 1 or 2

// DV: head dim, 256 or 128 (rows of 2 DV bytes, NCH chunks of 16 bytes; one
// 1 KB load moves RPL rows).
template <bool VT, int DV>
__global__ __launch_bounds__(64 * (8 / CB)) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, int64_t qs_t, int64_t qs_h, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kvs_t, int64_t kvs_h, uint16_t* __restrict__ out,
    int64_t os_t, int64_t os_h, int q_len, int cached_len, int QG, int ppw, float scale_log2,
    int64_t vt_tiles, const int32_t* __restrict__ vshift) {
  static_assert(DV == 128 || DV == 256, "head dim");
  constexpr int kRowBytes = 2 * DV, NCH = kRowBytes / 16, RPL = 64 / NCH;
  constexpr int kTileU4 = kKeyTile * kRowBytes / 16;      // 16-byte chunks per tile
  constexpr int NJ = DV / 32, NACC = DV / 16;              // query registers, accumulators
  // one array per stage and operand, so that the compiler can tell the slot
  // being read from the slots being filled
  __shared__ uint4 kr0[kTileU4], kr1[kTileU4], kr2[kTileU4], kr3[kTileU4];
  __shared__ uint4 vr0[kTileU4], vr1[kTileU4], vr2[kTileU4], vr3[kTileU4];

  // CB column blocks of 16 per wave, 128 / (16 CB) waves; each wave moves
  // ROWS of the 32 rows of every K and V tile, NDMA loads of 1 KB each
  constexpr int WAVES = 8 / CB, ROWS = kKeyTile / WAVES, NDMA = ROWS / RPL;
  static_assert(NDMA * RPL == ROWS && NDMA * WAVES * 1024 == kKeyTile * kRowBytes, "tile loads");
  const int n_ptiles = (q_len + ppw - 1) / ppw;
  const int p0 = (n_ptiles - 1 - (int)blockIdx.x) * ppw;    // latest positions (most keys) first
  const int hk = blockIdx.y;
  const int p_end = min(p0 + ppw, q_len);
  const int kend = cached_len + p_end;                      // keys the last position sees
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;

  int klim[CB], cpos[CB], chead[CB];
  bool cval[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int c = 16 * CB * wave + 16 * cb + r16;
    cpos[cb] = p0 + c / QG;
    chead[cb] = hk * QG + c % QG;
    cval[cb] = c < ppw * QG && cpos[cb] < q_len;
    klim[cb] = cached_len + cpos[cb] + 1;
  }
  // the query first, so that waiting for it never waits for a tile; the
  // addresses stay inside the tensor even for columns past the chunk
  v8bf qb[CB][NJ];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int pos = cval[cb] ? cpos[cb] : 0;
    const int head = cval[cb] ? chead[cb] : 0;
    const uint16_t* qp = q + (int64_t)pos * qs_t + (int64_t)head * qs_h + 8 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (cval[cb]) x = ld16(qp + 32 * j);
      qb[cb][j] = __builtin_bit_cast(v8bf, x);
    }
  }

  // Load i of this wave moves rows ROWS*w + RPL i + l/NCH of the tile, LDS chunk l%NCH.
  const uint32_t row_bytes = (uint32_t)(kvs_t * 2);
  uint32_t koff[NDMA], voff[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = ROWS * wave + RPL * i + lane / NCH, c = lane % NCH;
    koff[i] = r * row_bytes + 16 * (c ^ (r & 15));
    voff[i] = VT ? 1024 * (NDMA * wave + i) + 16 * lane : r * row_bytes + 16 * (c ^ (((r >> 2) & 3) << 2));
  }
  const int n_kt = (kend + kKeyTile - 1) / kKeyTile;
  auto issue = [&](uint4* ks, uint4* vs, int t) {
    const int key0 = t * kKeyTile;
    const int nv = min(kKeyTile, kend - key0);
    // the descriptors end at the last key the workgroup needs: rows past it land as zeros
    const int nrec = (nv - 1) * (int)row_bytes + kRowBytes;
    const int64_t base = (int64_t)key0 * kvs_t + (int64_t)hk * kvs_h;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc((void*)(k + base), nrec);
    const __amdgpu_buffer_rsrc_t rv =
        VT ? buffer_rsrc((void*)(v + ((int64_t)hk * vt_tiles + t) * (kKeyTile * DV)), kKeyTile * kRowBytes)
           : buffer_rsrc((void*)(v + base), nrec);
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      load_lds16(rk, ks + 64 * (NDMA * wave + i), koff[i]);
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      load_lds16(rv, vs + 64 * (NDMA * wave + i), voff[i]);
  };

  v4f acc[CB][NACC];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[cb][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  v4f lsum[CB];                                            // row sums of the weights
  float m_ref[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    lsum[cb] = (v4f){0.f, 0.f, 0.f, 0.f};
    m_ref[cb] = -INFINITY;
  }
  const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const v8h ones16 = __builtin_bit_cast(v8h, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));

  // Scores of one tile, S^T = K Q^T (K operands read four steps ahead).
  struct Scores {
    v4f s[2][CB];
  };
  auto scores = [&](const uint4* ks) {
    const uint8_t* kb_ = reinterpret_cast<const uint8_t*>(ks);
    Scores r;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) r.s[kb][cb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < DV / 128; ++h) {
      v8bf ka[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ka[kb][j] = __builtin_bit_cast(
              v8bf, ld16(kb_ + (16 * kb + r16) * kRowBytes + 16 * ((4 * (4 * h + j) + g) ^ r16)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            r.s[kb][cb] = mfma_bf16(ka[kb][j], qb[cb][4 * h + j], r.s[kb][cb]);
    }
    return r;
  };

  // Softmax and P.V of tile t from its scores.
  auto weigh = [&](const Scores& sc, const uint4* vs, int t) {
    const uint8_t* vb_ = reinterpret_cast<const uint8_t*>(vs);
    const auto& s = sc.s;
    // raw scores; only tiles that reach past the first position's last
    // visible key need the causal mask (a workgroup-uniform test)
    const int key0 = t * kKeyTile;
    float sv[CB][8], mt[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[cb][4 * kb + i] = s[kb][cb][i];
    if (key0 + kKeyTile > cached_len + p0 + 1) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + 16 * kb + 4 * g + i >= klim[cb]) sv[cb][4 * kb + i] = -INFINITY;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float x = sv[cb][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) x = fmaxf(x, sv[cb][i]);
      mt[cb] = rowgroup_max(x) * scale_log2;                  // scale > 0: max commutes
      if (t == 0) m_ref[cb] = mt[cb];
    }
    bool raise = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) raise = raise || mt[cb] > m_ref[cb] + 8.0f;
    if (__any(raise)) {
      // Rare: raise the reference and rescale row r of O by f_r, as the
      // product diag(f) O on float32 MFMAs, so that the accumulators are
      // only ever touched by MFMAs. V_MFMA_F32_16X16X4_F32 takes A[r][k]
      // from lane (r, k) and B[k][c] from lane (c, k); register i of an
      // accumulator, used as B, is O[4k + i][c], so A_i[r][k] = f_r when
      // r = 4k + i (this lane's own column factor) and 0 otherwise.
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float m_new = fmaxf(m_ref[cb], mt[cb]);
        const float f = m_new > m_ref[cb] ? exp2f(m_ref[cb] - m_new) : 1.f;
        float fsel[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fsel[i] = r16 == 4 * g + i ? f : 0.f;
#pragma unroll
        for (int j = 0; j < NACC + 1; ++j) {
          v4f& a = j < NACC ? acc[cb][j] : lsum[cb];
          v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < 4; ++i) d = mfma_f32x4(fsel[i], a[i], d);
          a = d;
        }
        m_ref[cb] = m_new;
      }
    }
    // weights p = 2^(s * scale_log2 - m_ref). Their row sums come from MFMAs
    // against ones, so they are the sums of exactly the weights the product
    // uses and land in O's row layout.
    if constexpr (VT) {
      // fp16 weights (11 significant bits, relative error at most 2^-11, so
      // at most 2^-11 |v - o| in the output) against the fp16 value tiles,
      // one MFMA per product
      v8h ph[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        uint32_t pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[cb][2 * i], scale_log2, -m_ref[cb]));
          const float pc = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[cb][2 * i + 1], scale_log2, -m_ref[cb]));
          pw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){pa, pc}, v2h));
        }
        ph[cb] = __builtin_bit_cast(v8h, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        lsum[cb] = mfma_f16(ph[cb], ones16, lsum[cb]);
      }
#pragma unroll
      for (int n = 0; n < NACC; ++n) {
        const int dim = 16 * n + r16;
        const v8h vh = __builtin_bit_cast(v8h, ld16(vb_ + dim * 64 + 16 * (g ^ vt_swizzle(dim))));
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb][n] = mfma_f16(ph[cb], vh, acc[cb][n]);
      }
      return;
    }
    // token-major bf16 values: each weight as two bf16 parts, hi = bf16(p)
    // and lo = bf16(p - hi) (p - hi is exact in float32), so a weight enters
    // the product with 16 significant bits (a single bf16 weight put up to
    // 2^-8 |v - o| into the output where a few keys dominate)
    v8bf pb[CB], pl[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      uint32_t pw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[cb][2 * i], scale_log2, -m_ref[cb]));
        const float pc = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[cb][2 * i + 1], scale_log2, -m_ref[cb]));
        pw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){pa, pc}, v2bf));
        const float ha = __uint_as_float(pw[i] << 16), hc = __uint_as_float(pw[i] & 0xFFFF0000u);
        lw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){pa - ha, pc - hc}, v2bf));
      }
      pb[cb] = __builtin_bit_cast(v8bf, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      pl[cb] = __builtin_bit_cast(v8bf, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      lsum[cb] = mfma_bf16(pb[cb], ones, lsum[cb]);
      lsum[cb] = mfma_bf16(pl[cb], ones, lsum[cb]);
    }
#pragma unroll
    for (int b = 0; b < NJ; ++b) {
      uint32_t w[8];
#pragma unroll
      for (int s_ = 0; s_ < 8; ++s_) {
        const int key = s_ < 4 ? 4 * g + s_ : 16 + 4 * g + (s_ - 4);
        const int chunk = (4 * b + (r16 >> 2)) ^ (((key >> 2) & 3) << 2);
        w[s_] = *reinterpret_cast<const uint32_t*>(vb_ + key * kRowBytes + 16 * chunk + 4 * (r16 & 3));
      }
      const uint4 ev = make_uint4(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                                  __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                                  __builtin_amdgcn_perm(w[5], w[4], 0x05040100u),
                                  __builtin_amdgcn_perm(w[7], w[6], 0x05040100u));
      const uint4 od = make_uint4(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                                  __builtin_amdgcn_perm(w[3], w[2], 0x07060302u),
                                  __builtin_amdgcn_perm(w[5], w[4], 0x07060302u),
                                  __builtin_amdgcn_perm(w[7], w[6], 0x07060302u));
      const v8bf ae = __builtin_bit_cast(v8bf, ev), ao = __builtin_bit_cast(v8bf, od);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        acc[cb][2 * b] = mfma_bf16(pb[cb], ae, acc[cb][2 * b]);
        acc[cb][2 * b] = mfma_bf16(pl[cb], ae, acc[cb][2 * b]);
        acc[cb][2 * b + 1] = mfma_bf16(pb[cb], ao, acc[cb][2 * b + 1]);
        acc[cb][2 * b + 1] = mfma_bf16(pl[cb], ao, acc[cb][2 * b + 1]);
      }
    }
  };

  // Software pipeline, one tile deep: step t makes tile t+1 visible to the
  // whole workgroup (the barrier also ends every wave's use of tile t-1),
  // refills tile t-1's stage with tile t+3, issues tile t+1's score MFMAs and
  // only then works through tile t's softmax and P.V, so the matrix cores
  // have work while the softmax runs. Past the last tile the extra scores
  // are computed from a stale stage and dropped.
  issue(kr0, vr0, 0);
  if (1 < n_kt) issue(kr1, vr1, 1);
  if (2 < n_kt) issue(kr2, vr2, 2);
  wait_tiles<kStages - 2, 2 * NDMA>(n_kt - 1);
  __syncthreads();
  Scores cur = scores(kr0);
#define UQP_STEP(KC, VC, KN, KF, VF)                                 \
  {                                                                  \
    wait_tiles<kStages - 3, 2 * NDMA>(n_kt - 2 - t);                 \
    __syncthreads();                                                 \
    if (t + kStages - 1 < n_kt) issue(KF, VF, t + kStages - 1);      \
    const Scores nxt = scores(KN);                                   \
    weigh(cur, VC, t);                                               \
    cur = nxt;                                                       \
    if (++t >= n_kt) break;                                          \
  }
  for (int t = 0;;) {
    UQP_STEP(kr0, vr0, kr1, kr3, vr3)
    UQP_STEP(kr1, vr1, kr2, kr0, vr0)
    UQP_STEP(kr2, vr2, kr3, kr1, vr1)
    UQP_STEP(kr3, vr3, kr0, kr2, vr2)
  }
#undef UQP_STEP

  // Epilogue: lane (r, g) holds, for column 4g + i, O at dims 16n + r (VT,
  // in units of 2^vshift of the dims' 32-block) or at dims 32b + 2r, 2r + 1
  // (even / odd accumulators), and that column's weight sum.
  int vsh[VT ? DV / 32 : 1];
#pragma unroll
  for (int b = 0; b < (VT ? DV / 32 : 1); ++b) vsh[b] = VT ? vshift[hk * (DV / 32) + b] : 0;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cl = 4 * g + i;                                   // column within the block
      const float inv = 1.f / lsum[cb][i];
      const int c = 16 * CB * wave + 16 * cb + cl;
      const int pos = p0 + c / QG;
      if (!(c < ppw * QG && pos < q_len)) continue;
      uint16_t* op = out + (int64_t)pos * os_t + (int64_t)(hk * QG + c % QG) * os_h;
      if constexpr (VT) {
#pragma unroll
        for (int n = 0; n < NACC; ++n)
          op[16 * n + r16] =
              __builtin_bit_cast(uint16_t, (__bf16)__builtin_amdgcn_ldexpf(acc[cb][n][i] * inv, vsh[n / 2]));
      } else {
#pragma unroll
        for (int b = 0; b < NJ; ++b)
          *reinterpret_cast<uint32_t*>(op + 32 * b + 2 * r16) = __builtin_bit_cast(
              uint32_t, __builtin_convertvector((v2f){acc[cb][2 * b][i] * inv, acc[cb][2 * b + 1][i] * inv}, v2bf));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Head dim 512: rows of 1 KB, so keys stream in tiles of 16 (four stages of
// K and V still fit in 128 KB of LDS) and values stay token-major. Four
// waves of 16 columns each (64 columns of one KV head; a wave's 128
// accumulator and 64 query registers need the register file of a SIMD to
// itself) and the same pipeline as above; what changes with the tile:
//   S^T (16 keys x 16 cols) = K Q^T takes D/32 MFMAs; lane (col, g) is left
//     with keys 4g + i of its column.
//   O += P V: a 16-key tile fills only half of the 32 k-slots, so the high
//     and low bf16 parts of each weight share one MFMA: slot (g, s) stands
//     for key 4g + (s & 3), the high part for s < 4 and the low one for
//     s >= 4, and B repeats that key's value in both halves. Lane (r, g)
//     reads 8 bytes (dims 64b + 4r .. 64b + 4r + 3) of each of its 4 keys;
//     byte permutes sort them by dim mod 4 into four B operands, one per
//     accumulator 4b + (dim mod 4).
// Chunk c of LDS row r holds chunk c ^ f(r) of the key's row: f(r) = r & 15
// for K (the 16 rows of a score read hit distinct banks), ((r >> 2) & 3) << 3
// for V (the four key groups of a value read sit 128 bytes apart).
// ---------------------------------------------------------------------------
constexpr int kColsPerWg16 = 64;

template <int DV>
__global__ __launch_bounds__(256) void prefill_attn16_kernel(
    const uint16_t* __restrict__ q, int64_t qs_t, int64_t qs_h, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kvs_t, int64_t kvs_h, uint16_t* __restrict__ out,
    int64_t os_t, int64_t os_h, int q_len, int cached_len, int QG, int ppw, float scale_log2) {
  constexpr int KT = 16, kRowBytes = 2 * DV, NCH = kRowBytes / 16;
  static_assert(NCH == 64, "one 1 KB load per row");
  constexpr int kTileU4 = KT * NCH;
  constexpr int NJ = DV / 32, NB = DV / 64, NACC = DV / 16;
  constexpr int WAVES = kColsPerWg16 / 16, ROWS = KT / WAVES;   // rows of K and of V each wave moves
  __shared__ uint4 kr0[kTileU4], kr1[kTileU4], kr2[kTileU4], kr3[kTileU4];
  __shared__ uint4 vr0[kTileU4], vr1[kTileU4], vr2[kTileU4], vr3[kTileU4];

  const int n_ptiles = (q_len + ppw - 1) / ppw;
  const int p0 = (n_ptiles - 1 - (int)blockIdx.x) * ppw;
  const int hk = blockIdx.y;
  const int p_end = min(p0 + ppw, q_len);
  const int kend = cached_len + p_end;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;

  const int c0 = 16 * wave + r16;
  const int cpos = p0 + c0 / QG;
  const bool cval = c0 < ppw * QG && cpos < q_len;
  const int klim = cached_len + cpos + 1;
  v8bf qb[NJ];
  {
    const uint16_t* qp = q + (int64_t)(cval ? cpos : 0) * qs_t + (int64_t)(cval ? hk * QG + c0 % QG : 0) * qs_h + 8 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (cval) x = ld16(qp + 32 * j);
      qb[j] = __builtin_bit_cast(v8bf, x);
    }
  }

  const uint32_t row_bytes = (uint32_t)(kvs_t * 2);
  uint32_t koff[ROWS], voff[ROWS];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    const int r = ROWS * wave + i;
    koff[i] = r * row_bytes + 16 * (lane ^ (r & 15));
    voff[i] = r * row_bytes + 16 * (lane ^ (((r >> 2) & 3) << 3));
  }
  const int n_kt = (kend + KT - 1) / KT;
  auto issue = [&](uint4* ks, uint4* vs, int t) {
    const int key0 = t * KT;
    const int nv = min(KT, kend - key0);
    const int nrec = (nv - 1) * (int)row_bytes + kRowBytes;
    const int64_t base = (int64_t)key0 * kvs_t + (int64_t)hk * kvs_h;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc((void*)(k + base), nrec);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc((void*)(v + base), nrec);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) load_lds16(rk, ks + 64 * (ROWS * wave + i), koff[i]);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) load_lds16(rv, vs + 64 * (ROWS * wave + i), voff[i]);
  };

  v4f acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
  v4f lsum = {0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;
  const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

  auto scores = [&](const uint4* ks) {
    const uint8_t* kb_ = reinterpret_cast<const uint8_t*>(ks);
    // two independent accumulation chains, added at the end
    v4f s[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int h = 0; h < NJ / 4; ++h) {
      v8bf ka[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ka[j] = __builtin_bit_cast(v8bf, ld16(kb_ + r16 * kRowBytes + 16 * ((4 * (4 * h + j) + g) ^ r16)));
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j & 1] = mfma_bf16(ka[j], qb[4 * h + j], s[j & 1]);
    }
    return s[0] + s[1];
  };

  auto weigh = [&](const v4f& s, const uint4* vs, int t) {
    const uint8_t* vb_ = reinterpret_cast<const uint8_t*>(vs);
    const int key0 = t * KT;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = s[i];
    if (key0 + KT > cached_len + p0 + 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + 4 * g + i >= klim) sv[i] = -INFINITY;
    }
    const float mt = rowgroup_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]))) * scale_log2;
    if (t == 0) m_ref = mt;
    if (__any(mt > m_ref + 8.0f)) {
      // raise the reference, O <- diag(f) O on float32 MFMAs (as above)
      const float m_new = fmaxf(m_ref, mt);
      const float f = m_new > m_ref ? exp2f(m_ref - m_new) : 1.f;
      float fsel[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fsel[i] = r16 == 4 * g + i ? f : 0.f;
#pragma unroll
      for (int j = 0; j < NACC + 1; ++j) {
        v4f& a = j < NACC ? acc[j] : lsum;
        v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) d = mfma_f32x4(fsel[i], a[i], d);
        a = d;
      }
      m_ref = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], scale_log2, -m_ref));
    const uint32_t h01 = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){p[0], p[1]}, v2bf));
    const uint32_t h23 = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){p[2], p[3]}, v2bf));
    const uint32_t l01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(
        (v2f){p[0] - __uint_as_float(h01 << 16), p[1] - __uint_as_float(h01 & 0xFFFF0000u)}, v2bf));
    const uint32_t l23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(
        (v2f){p[2] - __uint_as_float(h23 << 16), p[3] - __uint_as_float(h23 & 0xFFFF0000u)}, v2bf));
    const v8bf pb = __builtin_bit_cast(v8bf, make_uint4(h01, h23, l01, l23));
    lsum = mfma_bf16(pb, ones, lsum);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint2 w[4];
#pragma unroll
      for (int s_ = 0; s_ < 4; ++s_)
        w[s_] = *reinterpret_cast<const uint2*>(vb_ + (4 * g + s_) * kRowBytes + 128 * (b ^ g) + 8 * r16);
      const uint32_t x0 = __builtin_amdgcn_perm(w[1].x, w[0].x, 0x05040100u);
      const uint32_t y0 = __builtin_amdgcn_perm(w[3].x, w[2].x, 0x05040100u);
      const uint32_t x1 = __builtin_amdgcn_perm(w[1].x, w[0].x, 0x07060302u);
      const uint32_t y1 = __builtin_amdgcn_perm(w[3].x, w[2].x, 0x07060302u);
      const uint32_t x2 = __builtin_amdgcn_perm(w[1].y, w[0].y, 0x05040100u);
      const uint32_t y2 = __builtin_amdgcn_perm(w[3].y, w[2].y, 0x05040100u);
      const uint32_t x3 = __builtin_amdgcn_perm(w[1].y, w[0].y, 0x07060302u);
      const uint32_t y3 = __builtin_amdgcn_perm(w[3].y, w[2].y, 0x07060302u);
      acc[4 * b] = mfma_bf16(pb, __builtin_bit_cast(v8bf, make_uint4(x0, y0, x0, y0)), acc[4 * b]);
      acc[4 * b + 1] = mfma_bf16(pb, __builtin_bit_cast(v8bf, make_uint4(x1, y1, x1, y1)), acc[4 * b + 1]);
      acc[4 * b + 2] = mfma_bf16(pb, __builtin_bit_cast(v8bf, make_uint4(x2, y2, x2, y2)), acc[4 * b + 2]);
      acc[4 * b + 3] = mfma_bf16(pb, __builtin_bit_cast(v8bf, make_uint4(x3, y3, x3, y3)), acc[4 * b + 3]);
    }
  };

  issue(kr0, vr0, 0);
  if (1 < n_kt) issue(kr1, vr1, 1);
  if (2 < n_kt) issue(kr2, vr2, 2);
  wait_tiles<kStages - 2, 2 * ROWS>(n_kt - 1);
  __syncthreads();
  v4f cur = scores(kr0);
#define UQP_STEP16(KC, VC, KN, KF, VF)                               \
  {                                                                  \
    wait_tiles<kStages - 3, 2 * ROWS>(n_kt - 2 - t);                 \
    __syncthreads();                                                 \
    if (t + kStages - 1 < n_kt) issue(KF, VF, t + kStages - 1);      \
    const v4f nxt = scores(KN);                                      \
    weigh(cur, VC, t);                                               \
    cur = nxt;                                                       \
    if (++t >= n_kt) break;                                          \
  }
  for (int t = 0;;) {
    UQP_STEP16(kr0, vr0, kr1, kr3, vr3)
    UQP_STEP16(kr1, vr1, kr2, kr0, vr0)
    UQP_STEP16(kr2, vr2, kr3, kr1, vr1)
    UQP_STEP16(kr3, vr3, kr0, kr2, vr2)
  }
#undef UQP_STEP16

  // lane (r, g) holds, for column 4g + i, O at dims 64b + 4r + m in
  // accumulator 4b + m, and that column's weight sum
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 16 * wave + 4 * g + i;
    const float inv = 1.f / lsum[i];
    const int pos = p0 + c / QG;
    if (!(c < ppw * QG && pos < q_len)) continue;
    uint16_t* op = out + (int64_t)pos * os_t + (int64_t)(hk * QG + c % QG) * os_h + 4 * r16;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      *reinterpret_cast<uint2*>(op + 64 * b) = make_uint2(
          __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){acc[4 * b][i] * inv, acc[4 * b + 1][i] * inv}, v2bf)),
          __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){acc[4 * b + 2][i] * inv, acc[4 * b + 3][i] * inv}, v2bf)));
  }
}

// ---------------------------------------------------------------------------
// Head dim 512 over the continuation prefill's fp16 value tiles (32 keys,
// the tiled layout of the smaller head dims: dim rows of 64 bytes), with two
// waves per 16-column block: wave w owns columns 16 (w & 3) .. + 15 and dims
// 256 (w >> 2) .. + 255 of O. Each wave computes the scores of its columns
// over its half of the dims (16 MFMAs per tile); the two halves meet in LDS,
// double-buffered by tile parity so that the one barrier per tile orders
// them, and both waves then run the same softmax on the same full scores
// (a + b = b + a in float32), so their weights, sums and re-bases agree.
// A 32-key tile fills the k-slots of a 16x16x32 fp16 MFMA, so P.V takes one
// MFMA per 16 dims. K and V stream through separate two-stage rings (32 KB
// per stage): step t reads K of tile t + 1 for the scores and V of tile t
// for P.V, and refills the stages that tiles t (K) and t - 1 (V) left.
// Half the accumulators and query registers of prefill_attn16_kernel per
// wave: two waves share a SIMD.
// ---------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(512) void prefill_attn512_kernel(
    const uint16_t* __restrict__ q, int64_t qs_t, int64_t qs_h, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kvs_t, int64_t kvs_h, uint16_t* __restrict__ out,
    int64_t os_t, int64_t os_h, int q_len, int cached_len, int QG, int ppw, float scale_log2,
    int64_t vt_tiles, const int32_t* __restrict__ vshift) {
  constexpr int KT = kKeyTile, kRowBytes = 2 * DV, NCH = kRowBytes / 16;
  static_assert(NCH == 64, "one 1 KB load per row");
  constexpr int kTileU4 = KT * NCH;                // 32 KB per stage and operand
  constexpr int HD = DV / 2;                       // dims per wave
  constexpr int NJ = HD / 32, NACC = HD / 16;      // query registers, accumulators
  constexpr int WAVES = 8, ROWS = KT / WAVES;      // 1 KB rows of K and of V each wave moves
  __shared__ uint4 kr0[kTileU4], kr1[kTileU4], vr0[kTileU4], vr1[kTileU4];
  __shared__ v4f xs[2][2][WAVES][64];              // partial scores, by tile parity and key half

  const int n_ptiles = (q_len + ppw - 1) / ppw;
  const int p0 = (n_ptiles - 1 - (int)blockIdx.x) * ppw;
  const int hk = blockIdx.y;
  const int p_end = min(p0 + ppw, q_len);
  const int kend = cached_len + p_end;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cb = wave & 3, hf = wave >> 2;
  const int r16 = lane & 15, g = lane >> 4;

  const int c0 = 16 * cb + r16;
  const int cpos = p0 + c0 / QG;
  const bool cval = c0 < ppw * QG && cpos < q_len;
  const int klim = cached_len + cpos + 1;
  v8bf qb[NJ];
  {
    const uint16_t* qp = q + (int64_t)(cval ? cpos : 0) * qs_t + (int64_t)(cval ? hk * QG + c0 % QG : 0) * qs_h +
                         HD * hf + 8 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (cval) x = ld16(qp + 32 * j);
      qb[j] = __builtin_bit_cast(v8bf, x);
    }
  }

  const uint32_t row_bytes = (uint32_t)(kvs_t * 2);
  uint32_t koff[ROWS];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    const int r = ROWS * wave + i;
    koff[i] = r * row_bytes + 16 * (lane ^ (r & 15));
  }
  const int n_kt = (kend + KT - 1) / KT;
  auto issue_k = [&](uint4* ks, int t) {
    const int key0 = t * KT;
    const int nv = min(KT, kend - key0);
    // the descriptor ends at the last key the workgroup needs: rows past it land as zeros
    const int nrec = (nv - 1) * (int)row_bytes + kRowBytes;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc((void*)(k + (int64_t)key0 * kvs_t + (int64_t)hk * kvs_h), nrec);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) load_lds16(rk, ks + 64 * (ROWS * wave + i), koff[i]);
  };
  auto issue_v = [&](uint4* vs, int t) {          // the 32 KB tile is contiguous
    const __amdgpu_buffer_rsrc_t rv =
        buffer_rsrc((void*)(v + ((int64_t)hk * vt_tiles + t) * (KT * DV)), KT * kRowBytes);
#pragma unroll
    for (int i = 0; i < ROWS; ++i) load_lds16(rv, vs + 64 * (ROWS * wave + i), 1024 * (ROWS * wave + i) + 16 * lane);
  };

  v4f acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
  v4f lsum = {0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;
  const v8h ones16 = __builtin_bit_cast(v8h, make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));

  // S^T over this wave's dims (32-dim steps 8 hf .. 8 hf + 7) for the key
  // halves kb = 0, 1 of the tile: lane (col, g) gets keys 16 kb + 4 g + i
  auto pscores = [&](const uint4* ks, v4f (&s)[2]) {
    const uint8_t* kb_ = reinterpret_cast<const uint8_t*>(ks);
    s[0] = (v4f){0.f, 0.f, 0.f, 0.f};
    s[1] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < NJ / 4; ++h) {
      v8bf ka[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ka[kb][j] = __builtin_bit_cast(
              v8bf, ld16(kb_ + (16 * kb + r16) * kRowBytes + 16 * ((4 * (NJ * hf + 4 * h + j) + g) ^ r16)));
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_bf16(ka[kb][j], qb[4 * h + j], s[kb]);
    }
  };

  auto weigh = [&](const v4f (&s)[2], const uint4* vs, int t) {
    const uint8_t* vb_ = reinterpret_cast<const uint8_t*>(vs);
    const int key0 = t * KT;
    float sv[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * kb + i] = s[kb][i];
    if (key0 + KT > cached_len + p0 + 1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + 16 * kb + 4 * g + i >= klim) sv[4 * kb + i] = -INFINITY;
    }
    float x = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) x = fmaxf(x, sv[i]);
    const float mt = rowgroup_max(x) * scale_log2;
    if (t == 0) m_ref = mt;
    if (__any(mt > m_ref + 8.0f)) {
      // raise the reference, O <- diag(f) O on float32 MFMAs (as above)
      const float m_new = fmaxf(m_ref, mt);
      const float f = m_new > m_ref ? exp2f(m_ref - m_new) : 1.f;
      float fsel[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fsel[i] = r16 == 4 * g + i ? f : 0.f;
#pragma unroll
      for (int j = 0; j < NACC + 1; ++j) {
        v4f& a = j < NACC ? acc[j] : lsum;
        v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) d = mfma_f32x4(fsel[i], a[i], d);
        a = d;
      }
      m_ref = m_new;
    }
    // k-slot 8 g + s of the MFMAs stands for key 16 (s >> 2) + 4 g + (s & 3):
    // the weights in sv order, and chunk g of a dim row in the tiled layout
    uint32_t pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], scale_log2, -m_ref));
      const float pc = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], scale_log2, -m_ref));
      pw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){pa, pc}, v2h));
    }
    const v8h ph = __builtin_bit_cast(v8h, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    lsum = mfma_f16(ph, ones16, lsum);
#pragma unroll
    for (int n = 0; n < NACC; ++n) {
      const int dim = HD * hf + 16 * n + r16;
      const v8h vh = __builtin_bit_cast(v8h, ld16(vb_ + dim * 64 + 16 * (g ^ vt_swizzle(dim))));
      acc[n] = mfma_f16(ph, vh, acc[n]);
    }
  };

  // Step t: the barrier makes K of tile t + 1 and V of tile t visible (both
  // requested in step t - 1) and orders both halves' partial scores of tile
  // t (written in step t - 1) before they are read here; it also ends every
  // wave's use of K of tile t and V of tile t - 1, whose stages are refilled.
  // Past the last tile the extra scores come from a stale stage and are dropped.
  issue_k(kr0, 0);
  if (1 < n_kt) issue_k(kr1, 1);
  issue_v(vr0, 0);
  UQP_WAIT_VMCNT(ROWS);                            // K of tile 0 (V of tile 0 may still fly)
  __syncthreads();
  v4f mine[2];
  pscores(kr0, mine);
  xs[0][0][wave][lane] = mine[0];
  xs[0][1][wave][lane] = mine[1];
#define UQP_STEP512(KN, KF, VC, VF)                                  \
  {                                                                  \
    UQP_WAIT_VMCNT(0);                                               \
    __syncthreads();                                                 \
    if (t + 2 < n_kt) issue_k(KF, t + 2);                            \
    if (t + 1 < n_kt) issue_v(VF, t + 1);                            \
    v4f full[2];                                                     \
    full[0] = mine[0] + xs[t & 1][0][wave ^ 4][lane];                \
    full[1] = mine[1] + xs[t & 1][1][wave ^ 4][lane];                \
    pscores(KN, mine);                                               \
    xs[(t + 1) & 1][0][wave][lane] = mine[0];                        \
    xs[(t + 1) & 1][1][wave][lane] = mine[1];                        \
    weigh(full, VC, t);                                              \
    if (++t >= n_kt) break;                                          \
  }
  for (int t = 0;;) {
    UQP_STEP512(kr1, kr0, vr0, vr1)
    UQP_STEP512(kr0, kr1, vr1, vr0)
  }
#undef UQP_STEP512

  // lane (r, g) holds, for column 4g + i, O at dim HD hf + 16n + r in
  // accumulator n (in units of 2^vshift of the dim's 32-block), and that
  // column's weight sum
  int vsh[HD / 32];
#pragma unroll
  for (int b = 0; b < HD / 32; ++b) vsh[b] = vshift[hk * (DV / 32) + (HD / 32) * hf + b];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 16 * cb + 4 * g + i;
    const float inv = 1.f / lsum[i];
    const int pos = p0 + c / QG;
    if (!(c < ppw * QG && pos < q_len)) continue;
    uint16_t* op = out + (int64_t)pos * os_t + (int64_t)(hk * QG + c % QG) * os_h + HD * hf + r16;
#pragma unroll
    for (int n = 0; n < NACC; ++n)
      op[16 * n] = __builtin_bit_cast(uint16_t, (__bf16)__builtin_amdgcn_ldexpf(acc[n][i] * inv, vsh[n / 2]));
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  const int64_t tile_waves = a.vt ? 4 * (int64_t)a.Hk * a.vt_tiles : 0;
  const int64_t waves = tile_waves + (int64_t)a.n_tok * a.Hk + (a.job[0].n + 3) / 4 + (a.job[1].n + 3) / 4 +
                        (a.job[2].n + 3) / 4;
  if (waves == 0) return hipSuccess;
  if (a.vt) {                                 // the value tiles' exponent shifts first
    const dim3 vgrid(kVexpParts, (unsigned)a.Hk);
    if (a.D == kHeadDim)
      hipLaunchKernelGGL(prefill_vexp_kernel<256>, vgrid, dim3(256), 0, stream, a);
    else if (a.D == kHeadDim / 2)
      hipLaunchKernelGGL(prefill_vexp_kernel<128>, vgrid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(prefill_vexp_kernel<512>, vgrid, dim3(256), 0, stream, a);
  }
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  switch (a.D) {
    case 128: hipLaunchKernelGGL(prefill_gather_kernel<128>, grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL(prefill_gather_kernel<256>, grid, block, 0, stream, a); break;
    case 512: hipLaunchKernelGGL(prefill_gather_kernel<512>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int prefill_positions_per_wg(int QG, int D) {
  const int cols = D > kHeadDim ? kColsPerWg16 : kColsPerWg;
  return QG <= cols ? cols / QG : 0;
}

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t stream) {
  if (a.q_len == 0) return hipSuccess;
  if (a.D != kHeadDim && a.D != kHeadDim / 2 && a.D != 2 * kHeadDim) return hipErrorInvalidValue;
  const int ppw = prefill_positions_per_wg(a.QG, a.D);
  const int n_ptiles = (a.q_len + ppw - 1) / ppw;
  if (a.D == 2 * kHeadDim) {
    const dim3 grid16((unsigned)n_ptiles, (unsigned)a.Hk), block16(64 * (kColsPerWg16 / 16));
    const float sl2_16 = a.scale * 1.4426950408889634f;
    if (a.vt_tiles > 0) {
      if (!a.vshift) return hipErrorInvalidValue;
      hipLaunchKernelGGL((prefill_attn512_kernel<512>), grid16, dim3(512), 0, stream, a.q, a.qs_t, a.qs_h,
                         a.k, a.v, a.kvs_t, a.kvs_h, a.out, a.os_t, a.os_h, a.q_len, a.cached_len, a.QG, ppw,
                         sl2_16, (int64_t)a.vt_tiles, a.vshift);
    } else {
      hipLaunchKernelGGL((prefill_attn16_kernel<512>), grid16, block16, 0, stream, a.q, a.qs_t, a.qs_h, a.k,
                         a.v, a.kvs_t, a.kvs_h, a.out, a.os_t, a.os_h, a.q_len, a.cached_len, a.QG, ppw, sl2_16);
    }
    return hipGetLastError();
  }
  const dim3 grid((unsigned)n_ptiles, (unsigned)a.Hk), block(64 * (8 / CB));
  const float sl2 = a.scale * 1.4426950408889634f;
#define UQP_LAUNCH(VTV, DVV, TILES)                                                                      \
  hipLaunchKernelGGL((prefill_attn_kernel<VTV, DVV>), grid, block, 0, stream, a.q, a.qs_t, a.qs_h, a.k, \
                     a.v, a.kvs_t, a.kvs_h, a.out, a.os_t, a.os_h, a.q_len, a.cached_len, a.QG, ppw, sl2, \
                     (int64_t)(TILES), a.vshift)
  if (a.vt_tiles > 0) {
    if (!a.vshift) return hipErrorInvalidValue;
    if (a.D == kHeadDim) UQP_LAUNCH(true, 256, a.vt_tiles); else UQP_LAUNCH(true, 128, a.vt_tiles);
  } else {
    if (a.D == kHeadDim) UQP_LAUNCH(false, 256, 0); else UQP_LAUNCH(false, 128, 0);
  }
#undef UQP_LAUNCH
  return hipGetLastError();
}

}  // namespace uq
