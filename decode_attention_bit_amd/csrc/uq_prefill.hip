// Continuation prefill: a chunk of q_len new tokens attends to the sequence's
// cached prefix (FP4 in the paged cache) and to itself, causally.
// (vLLM API docs, ultraquant_attn, _ultraquant_continuation_prefill: the
// prefix is dequantised to the query dtype in the rotated basis, the chunk's
// K and the queries are rotated by the Hadamard and cast to the query dtype,
// and a dense causal attention over prefix + chunk aligns query i to absolute
// position cached_len + i.)
//
// Two kernels:
//   prefill_gather_kernel  builds the bf16 operands: dequantised prefix K/V,
//                          rotated queries and chunk keys (float64 butterfly,
//                          one rounding to bf16), copied chunk values;
//   prefill_attn_kernel    flash attention over them on bf16 matrix cores.
#include "uq_internal.h"

namespace uq {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
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

// ---------------------------------------------------------------------------
// Gather: one wave per unit of work, the role chosen by the wave's index
// (wave-uniform): first the prefix slots (token, KV head) to dequantise, then
// up to three jobs over vectors of 256 bf16 (rotate or copy).
// Dequant: lanes 0-31 write K elements 8l .. 8l+7, lanes 32-63 the same V
// elements; each reads the 4 code bytes and the scale byte that cover them.
// Rotate: lane l holds x[4l .. 4l+3] through the float64 butterfly.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_gather_kernel(GatherArgs a) {
  int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t n_slots = (int64_t)a.n_tok * a.Hk;
  if (w < n_slots) {
    const int64_t t = w / a.Hk;
    const int h = (int)(w - t * a.Hk);
    const int64_t entry = t >> a.log2_bs;
    const int phys = a.block_row[entry];
    const bool ok = phys >= 0 && (int64_t)phys < a.num_blocks;
    const bool is_v = lane >= 32;
    const int l = lane & 31;
    uint32_t codes = 0;
    int e = 0;
    if (ok) {
      const uint8_t* slot =
          a.cache + ((((int64_t)phys << a.log2_bs) + (t & ((1 << a.log2_bs) - 1))) * a.Hk + h) * kSlotBytes;
      codes = *reinterpret_cast<const uint32_t*>(slot + (is_v ? kVCodeOff : kKCodeOff) + 4 * l);
      e = (int)slot[(is_v ? kVScaleOff : kKScaleOff) + (l >> 2)] - 127;
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = ok ? (e2m1_bf16_bits((codes >> (8 * i)) & 0xF, e) |
                   (e2m1_bf16_bits((codes >> (8 * i + 4)) & 0xF, e) << 16))
                : 0u;
    uint16_t* dst = (is_v ? a.vout : a.kout) + t * a.os_t + (int64_t)h * a.os_h + 8 * l;
    *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    return;
  }
  w -= n_slots;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const VecJob& jb = a.job[j];
    if (w >= jb.n) {
      w -= jb.n;
      continue;
    }
    const int64_t t = w / jb.H;
    const int h = (int)(w - t * jb.H);
    const uint2 r = *reinterpret_cast<const uint2*>(jb.src + t * jb.ss_t + (int64_t)h * jb.ss_h + 4 * lane);
    uint2 res = r;
    if (jb.rotate) {
      double v[4] = {bf16_to_f64(r.x & 0xFFFF), bf16_to_f64(r.x >> 16), bf16_to_f64(r.y & 0xFFFF),
                     bf16_to_f64(r.y >> 16)};
      fwht256_wave(v, lane);
      res.x = bf16_bits_rne(v[0] * 0.0625) | (bf16_bits_rne(v[1] * 0.0625) << 16);
      res.y = bf16_bits_rne(v[2] * 0.0625) | (bf16_bits_rne(v[3] * 0.0625) << 16);
    }
    *reinterpret_cast<uint2*>(jb.dst + t * jb.ds_t + (int64_t)h * jb.ds_h + 4 * lane) = res;
    return;
  }
}

// ---------------------------------------------------------------------------
// Attention. Workgroup = (block of query positions, KV head); its 128 columns
// are (position, query head) pairs of that KV head, column c -> position
// p0 + c / QG, head hk * QG + c % QG, so the QG heads sharing a KV head share
// every K/V tile. Wave w owns columns 32w .. 32w+31 as two 16-column blocks.
// Keys stream in tiles of 32 through a double-buffered LDS copy (rows padded
// to 528 bytes so that the reads below hit distinct banks).
//
// V_MFMA_F32_16X16X32_BF16, lane l: row/col l%16, k-slots (l/16, 0..7);
// result lane l: col l%16, rows 4*(l/16) + i. Which k a slot stands for is
// free as long as both operands agree:
//   S^T (keys x cols) = K Q^T: A = K rows, slot (g, i) = d 32j + 8g + i for
//     step j (16 contiguous bytes of a K row), B = the same d of the query
//     (held in registers). The result leaves lane (col, g) with keys
//     16kb + 4g + i of its column.
//   O^T (dims x cols) += V^T P^T: slot (g, s) = key 4g + s (s < 4) or
//     16 + 4g + s - 4, exactly the keys lane (col, g) holds, so P^T needs no
//     data movement. A = V^T: lane (r, g) reads the dword holding dims
//     32b + 2r, 2r + 1 of those 8 keys and feeds two MFMAs, one for the even
//     dims (row r -> dim 32b + 2r) and one for the odd ones.
// Online softmax in the log2 domain with a reference maximum that is only
// raised when a tile exceeds it by more than 8 (weights stay <= 2^8 in bf16);
// the denominator sums the same bf16 weights the product uses.
// ---------------------------------------------------------------------------
constexpr int kKeyTile = 32;
constexpr int kRowBytes = 2 * kHeadDim + 16;
constexpr int kColsPerWg = 128;

__device__ __forceinline__ float rowgroup_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__global__ __launch_bounds__(256) void prefill_attn_kernel(
    const uint16_t* __restrict__ q, int64_t qs_t, int64_t qs_h, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kvs_t, int64_t kvs_h, uint16_t* __restrict__ out,
    int64_t os_t, int64_t os_h, int q_len, int cached_len, int QG, int ppw, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kKeyTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][kKeyTile * kRowBytes];

  const int n_ptiles = (q_len + ppw - 1) / ppw;
  const int p0 = (n_ptiles - 1 - (int)blockIdx.x) * ppw;    // latest positions (most keys) first
  const int hk = blockIdx.y;
  const int p_end = min(p0 + ppw, q_len);
  const int kend = cached_len + p_end;                      // keys the last position sees
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;

  int klim[2], cpos[2], chead[2];
  bool cval[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c = 32 * wave + 16 * cb + r16;
    cpos[cb] = p0 + c / QG;
    chead[cb] = hk * QG + c % QG;
    cval[cb] = c < ppw * QG && cpos[cb] < q_len;
    klim[cb] = cached_len + cpos[cb] + 1;
  }
  // addresses stay inside the tensors even for columns past the chunk
  v8bf qb[2][8];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int pos = cval[cb] ? cpos[cb] : 0;
    const int head = cval[cb] ? chead[cb] : 0;
    const uint16_t* qp = q + (int64_t)pos * qs_t + (int64_t)head * qs_h + 8 * g;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (cval[cb]) x = ld16(qp + 32 * j);
      qb[cb][j] = __builtin_bit_cast(v8bf, x);
    }
  }

  // tile t: 32 keys x 512 bytes of K and of V, 8 chunks of 16 bytes per thread
  uint4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int ci = tid + 256 * rr;
      const int key = t * kKeyTile + (ci >> 5);
      const int64_t off = (int64_t)min(key, kend - 1) * kvs_t + (int64_t)hk * kvs_h + 8 * (ci & 31);
      kreg[rr] = make_uint4(0, 0, 0, 0);
      vreg[rr] = make_uint4(0, 0, 0, 0);
      if (key < kend) {
        kreg[rr] = ld16(k + off);
        vreg[rr] = ld16(v + off);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int ci = tid + 256 * rr;
      const int off = (ci >> 5) * kRowBytes + 16 * (ci & 31);
      *reinterpret_cast<uint4*>(kbuf[buf] + off) = kreg[rr];
      *reinterpret_cast<uint4*>(vbuf[buf] + off) = vreg[rr];
    }
  };

  v4f acc[2][16];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[cb][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.f, 0.f};

  const int n_kt = (kend + kKeyTile - 1) / kKeyTile;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < n_kt; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_kt) load_tile(t + 1);
    const uint8_t* kb_ = kbuf[buf];
    const uint8_t* vb_ = vbuf[buf];

    v4f s[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) s[kb][cb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v8bf a = __builtin_bit_cast(v8bf, ld16(kb_ + (16 * kb + r16) * kRowBytes + 64 * j + 16 * g));
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          s[kb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[cb][j], s[kb][cb], 0, 0, 0);
      }
    }

    const int key0 = t * kKeyTile;
    float sv[2][8], mt[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * kb + 4 * g + i;
          sv[cb][4 * kb + i] = key < klim[cb] ? s[kb][cb][i] * scale_log2 : -INFINITY;
        }
      float x = sv[cb][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) x = fmaxf(x, sv[cb][i]);
      mt[cb] = rowgroup_max(x);
      if (t == 0) m_ref[cb] = mt[cb];
    }
    if (__any(mt[0] > m_ref[0] + 8.0f || mt[1] > m_ref[1] + 8.0f)) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const float m_new = fmaxf(m_ref[cb], mt[cb]);
        const float f = m_new > m_ref[cb] ? exp2f(m_ref[cb] - m_new) : 1.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[cb][j] *= f;
        l_part[cb] *= f;
        m_ref[cb] = m_new;
      }
    }
    v8bf pb[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      uint32_t pw[4];
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0_ = __builtin_amdgcn_exp2f(sv[cb][2 * i] - m_ref[cb]);
        const float p1_ = __builtin_amdgcn_exp2f(sv[cb][2 * i + 1] - m_ref[cb]);
        pw[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){p0_, p1_}, v2bf));
        lsum += __uint_as_float(pw[i] << 16) + __uint_as_float(pw[i] & 0xFFFF0000u);
      }
      l_part[cb] += lsum;
      pb[cb] = __builtin_bit_cast(v8bf, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    }

#pragma unroll
    for (int b = 0; b < 8; ++b) {
      uint32_t w[8];
#pragma unroll
      for (int s_ = 0; s_ < 8; ++s_) {
        const int key = s_ < 4 ? 4 * g + s_ : 16 + 4 * g + (s_ - 4);
        w[s_] = *reinterpret_cast<const uint32_t*>(vb_ + key * kRowBytes + 64 * b + 4 * r16);
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
      for (int cb = 0; cb < 2; ++cb) {
        acc[cb][2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, pb[cb], acc[cb][2 * b], 0, 0, 0);
        acc[cb][2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, pb[cb], acc[cb][2 * b + 1], 0, 0, 0);
      }
    }

    if (t + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float l1 = l_part[cb] + __shfl_xor(l_part[cb], 16);
    const float l_tot = l1 + __shfl_xor(l1, 32);
    if (!cval[cb]) continue;
    const float inv = 1.f / l_tot;
    uint16_t* op = out + (int64_t)cpos[cb] * os_t + (int64_t)chead[cb] * os_h + 8 * g;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const v4f e = acc[cb][2 * b], o = acc[cb][2 * b + 1];
      uint32_t r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){e[i] * inv, o[i] * inv}, v2bf));
      *reinterpret_cast<uint4*>(op + 32 * b) = make_uint4(r[0], r[1], r[2], r[3]);
    }
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.n_tok * a.Hk + a.job[0].n + a.job[1].n + a.job[2].n;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_gather_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

int prefill_positions_per_wg(int QG) { return QG <= kColsPerWg ? kColsPerWg / QG : 0; }

hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t stream) {
  if (a.q_len == 0) return hipSuccess;
  const int ppw = prefill_positions_per_wg(a.QG);
  const int n_ptiles = (a.q_len + ppw - 1) / ppw;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((unsigned)n_ptiles, (unsigned)a.Hk), dim3(256), 0, stream,
                     a.q, a.qs_t, a.qs_h, a.k, a.v, a.kvs_t, a.kvs_h, a.out, a.os_t, a.os_h, a.q_len,
                     a.cached_len, a.QG, ppw, a.scale * 1.4426950408889634f);
  return hipGetLastError();
}

}  // namespace uq
