// Decode: query prologue (Hadamard rotation + E4M3 haircut), split-KV stage 1
// over the paged 4-bit cache, and the stage-2 log-sum-exp merge.
// (vLLM API docs, flydsl_ultraquant_decode: scaled FP4 x E4M3 QK on matrix
// cores, native V conversion, grid over (sequence, KV head, partition) with
// per-partition partial output, max and sum, then _reduce_partitions over a
// (B, Hq, D/64) grid; triton_turboquant_decode_v2: stage 1 over
// (B, Hk, NUM_KV_SPLITS) covering every query head of a KV head, stage 2
// merge.)
#include "uq_internal.h"

namespace uq {

namespace {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ld8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

// ---------------------------------------------------------------------------
// Query prologue: q8 = E4M3(q H), one wave per (sequence, query head).
// The rotation runs in float64 and is exact, so the E4M3 rounding decision is
// taken on the exact product.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void qprologue_kernel(const uint16_t* __restrict__ query,
                                                        uint8_t* __restrict__ q8, int B, int Hq,
                                                        int64_t qsb, int64_t qsh) {
  const int64_t vec = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (vec >= (int64_t)B * Hq) return;
  const int lane = threadIdx.x & 63;
  const int64_t b = vec / Hq;
  const int64_t hq = vec - b * Hq;
  const uint2 r = *reinterpret_cast<const uint2*>(query + b * qsb + hq * qsh + 4 * lane);
  double v[4] = {bf16_to_f64(r.x & 0xFFFF), bf16_to_f64(r.x >> 16), bf16_to_f64(r.y & 0xFFFF),
                 bf16_to_f64(r.y >> 16)};
  fwht256_wave(v, lane);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) w |= e4m3_code(v[i] * 0.0625) << (8 * i);
  reinterpret_cast<uint32_t*>(q8 + vec * kHeadDim)[lane] = w;
}

// ---------------------------------------------------------------------------
// Stage 1. Workgroup = (sequence b, split s, sub-range, group of KV heads),
// one wave per KV head so that the adjacent 272-byte slots of one token are
// read by one CU. A wave walks its token range in 16-token tiles:
//   scores^T (16 tokens x 16 q-heads) = K (FP4, UE8M0 scales) x q8 (E4M3) on
//     two V_MFMA_SCALE_F32_16X16X128_F8F6F4 (d = 0..127, 128..255);
//   online softmax in the log2 domain; the running max is only raised when a
//     tile exceeds it by more than 8 (p stays <= 256, exact softmax);
//   O^T (256 d x 16 q-heads) += V^T (bf16, converted with its scale) x P^T
//     (bf16) on 16 V_MFMA_F32_16X16X16_BF16.
// Lane layouts (gfx950):
//   scaled MFMA A (FP4, 4 VGPRs): lane l -> row l%16, k = 32*(l/16) + j for
//     nibble j; its scale byte covers those 32 k.
//   scaled MFMA B (FP8, 8 VGPRs): lane l -> col l%16, byte j -> k = 16*(l/16)+j
//     for j < 16 and 64 + 16*(l/16) + (j-16) above.
//   16x16x16 bf16 A/B: lane l -> row/col l%16, k = 4*(l/16) + i.
//   Result: lane l -> col l%16, rows 4*(l/16) + i.
// So the score tile leaves lane (g = l%16, grp = l/16) holding tokens
// 4*grp .. 4*grp+3 of q-head g, which is exactly the P^T operand of the
// P.V product, and the O^T accumulator of lane l holds q-head l%16,
// d = 64*grp + 16*i + j (i = element, j = MFMA index).
// ---------------------------------------------------------------------------
struct Tile {
  uint4 ka, kb;      // K codes: bytes [16*grp, +16) and [64 + 16*grp, +16) of token l%16
  uint2 ks;          // K scale bytes of token l%16
  uint2 vd[4];       // V codes: bytes [8*(l%16), +8) of tokens 4*grp + i
  uint32_t vs[4];    // the V-scale dword holding block (l%16)/2 of tokens 4*grp + i
  int nvalid;        // tokens of the tile that are inside the sequence
};

__device__ __forceinline__ void load_tile(Tile& T, const uint8_t* __restrict__ cache,
                                          const int32_t* __restrict__ bt, int t, int L,
                                          int log2_bs, int64_t num_blocks, size_t row, int h,
                                          int n16, int grp) {
  const int tok0 = t * kTile;
  const int phys = bt[tok0 >> log2_bs];
  const bool ok = phys >= 0 && (int64_t)phys < num_blocks;
  const int nvalid = ok ? min(kTile, L - tok0) : 0;
  T.nvalid = nvalid;
  const uint8_t* base = cache +
                        ((((size_t)(ok ? phys : 0)) << log2_bs) + (tok0 & ((1 << log2_bs) - 1))) * row +
                        (size_t)h * kSlotBytes;
  if (n16 < nvalid) {
    const uint8_t* kp = base + n16 * row;
    T.ka = ld16(kp + kKCodeOff + 16 * grp);
    T.kb = ld16(kp + kKCodeOff + 64 + 16 * grp);
    T.ks = ld8(kp + kKScaleOff);
  } else {
    T.ka = make_uint4(0, 0, 0, 0);
    T.kb = make_uint4(0, 0, 0, 0);
    T.ks = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tk = 4 * grp + i;
    if (tk < nvalid) {
      const uint8_t* vp = base + tk * row;
      T.vd[i] = ld8(vp + kVCodeOff + 8 * n16);
      T.vs[i] = ld4(vp + kVScaleOff + 4 * (n16 >> 3));
    } else {
      T.vd[i] = make_uint2(0, 0);
      T.vs[i] = 0x7F7F7F7Fu;
    }
  }
}

// Byte M of each token's 8 V-code bytes holds d = 16*(l%16) + 2M (low nibble)
// and 2M + 1 (high nibble). Convert them for the lane's 4 tokens, regroup the
// bf16 halves by d, and accumulate two MFMAs (d even / odd).
template <int M>
__device__ __forceinline__ void pv_step(const Tile& T, const float vscale[4], const v4s& pb,
                                        v4f acc[16]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = (M < 4) ? T.vd[i].x : T.vd[i].y;
    w[i] = __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, vscale[i], M & 3));
  }
  const uint32_t e0 = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
  const uint32_t e1 = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
  const uint32_t o0 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
  const uint32_t o1 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
  const v4s ae = __builtin_bit_cast(v4s, make_uint2(e0, e1));
  const v4s ao = __builtin_bit_cast(v4s, make_uint2(o0, o1));
  acc[2 * M] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ae, pb, acc[2 * M], 0, 0, 0);
  acc[2 * M + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ao, pb, acc[2 * M + 1], 0, 0, 0);
}

template <int QG>
__device__ __forceinline__ void compute_tile(const Tile& T, const v8i& qb0, const v8i& qb1,
                                             float scale_log2, int n16, int grp, v4f acc[16],
                                             float& m_ref, float& l_part) {
  // ---- scores
  const int sc1 = (int)((T.ks.x >> (8 * grp)) & 0xFF);
  const int sc2 = (int)((T.ks.y >> (8 * grp)) & 0xFF);
  const v8i a1 = {(int)T.ka.x, (int)T.ka.y, (int)T.ka.z, (int)T.ka.w, 0, 0, 0, 0};
  const v8i a2 = {(int)T.kb.x, (int)T.kb.y, (int)T.kb.z, (int)T.kb.w, 0, 0, 0, 0};
  v4f sc = {0.f, 0.f, 0.f, 0.f};
  sc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, qb0, sc, 4, 0, 0, sc1, 0, 127);
  sc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a2, qb1, sc, 4, 0, 0, sc2, 0, 127);
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = (4 * grp + i < T.nvalid) ? sc[i] * scale_log2 : -INFINITY;

  // ---- online softmax (log2 domain), lazily re-based
  float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const bool need = mt > m_ref + 8.0f;
  if (__any(need)) {
    const float mn = need ? mt : m_ref;
    const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f(m_ref - mn);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] *= alpha;
    l_part *= alpha;
    m_ref = mn;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = (sv[i] == -INFINITY) ? 0.f : exp2f(sv[i] - m_ref);
  const uint32_t p01 = pack_bf16(p[0], p[1]);
  const uint32_t p23 = pack_bf16(p[2], p[3]);
  l_part += (bf16_to_f32(p01 & 0xFFFF) + bf16_to_f32(p01 >> 16)) +
            (bf16_to_f32(p23 & 0xFFFF) + bf16_to_f32(p23 >> 16));
  const v4s pb = __builtin_bit_cast(v4s, make_uint2(p01, p23));

  // ---- P.V: V codes -> bf16 with their block scale, then 16 MFMAs
  float vscale[4];
  const int vsh = 8 * ((n16 >> 1) & 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) vscale[i] = __uint_as_float(((T.vs[i] >> vsh) & 0xFFu) << 23);
  pv_step<0>(T, vscale, pb, acc);
  pv_step<1>(T, vscale, pb, acc);
  pv_step<2>(T, vscale, pb, acc);
  pv_step<3>(T, vscale, pb, acc);
  pv_step<4>(T, vscale, pb, acc);
  pv_step<5>(T, vscale, pb, acc);
  pv_step<6>(T, vscale, pb, acc);
  pv_step<7>(T, vscale, pb, acc);
}

template <int QG>
__global__ __launch_bounds__(512) void stage1_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    float scale_log2, int Hq, int Hk, int hpw, int hgroups, int S, int nsub, int log2_bs,
    int max_blocks, int64_t num_blocks, uint16_t* __restrict__ part_o,
    float* __restrict__ part_m, float* __restrict__ part_l) {
  int x = blockIdx.x;
  const int hg = x % hgroups;
  x /= hgroups;
  const int sub = x % nsub;
  x /= nsub;
  const int s = x % S;
  const int b = x / S;
  const int lane = threadIdx.x & 63;
  const int h = hg * hpw + (threadIdx.x >> 6);
  const int P = S * nsub, part = s * nsub + sub;

  int L = seq_lens[b];
  const int Lmax = max_blocks << log2_bs;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int n_tiles = (L + kTile - 1) / kTile;
  const int per_split = (n_tiles + S - 1) / S;
  const int t_begin = s * per_split;
  const int t_end = min(t_begin + per_split, n_tiles);
  const int span = max(t_end - t_begin, 0);
  const int per_sub = (span + nsub - 1) / nsub;
  const int u0 = t_begin + sub * per_sub;
  const int u1 = min(u0 + per_sub, t_end);

  const int n16 = lane & 15, grp = lane >> 4;
  const bool qlane = n16 < QG;
  const int hq = h * QG + (qlane ? n16 : 0);
  const size_t stat = ((size_t)b * Hq + hq) * P + part;

  if (u0 >= u1) {
    if (qlane && grp == 0) {
      part_m[stat] = -INFINITY;
      part_l[stat] = 0.f;
    }
    return;
  }

  v8i qb0 = {0, 0, 0, 0, 0, 0, 0, 0}, qb1 = {0, 0, 0, 0, 0, 0, 0, 0};
  if (qlane) {
    const uint8_t* qp = q8 + ((size_t)b * Hq + hq) * kHeadDim;
    const uint4 x0 = ld16(qp + 16 * grp), x1 = ld16(qp + 64 + 16 * grp);
    const uint4 x2 = ld16(qp + 128 + 16 * grp), x3 = ld16(qp + 192 + 16 * grp);
    qb0 = (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    qb1 = (v8i){(int)x2.x, (int)x2.y, (int)x2.z, (int)x2.w, (int)x3.x, (int)x3.y, (int)x3.z, (int)x3.w};
  }

  const size_t row = (size_t)Hk * kSlotBytes;
  const int32_t* bt = block_table + (size_t)b * max_blocks;
  v4f acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.f;

  Tile cur, nxt;
  load_tile(cur, cache, bt, u0, L, log2_bs, num_blocks, row, h, n16, grp);
  for (int t = u0; t < u1; ++t) {
    if (t + 1 < u1) load_tile(nxt, cache, bt, t + 1, L, log2_bs, num_blocks, row, h, n16, grp);
    compute_tile<QG>(cur, qb0, qb1, scale_log2, n16, grp, acc, m_ref, l_part);
    cur = nxt;
  }

  const float l1 = l_part + __shfl_xor(l_part, 16);
  const float l_tot = l1 + __shfl_xor(l1, 32);
  if (!qlane) return;
  if (grp == 0) {
    part_m[stat] = m_ref;
    part_l[stat] = l_tot;
  }
  if (l_tot > 0.f) {
    const float inv = 1.f / l_tot;
    uint16_t* op = part_o + stat * kHeadDim + 64 * grp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 lo, hi;
      lo.x = pack_bf16(acc[0][i] * inv, acc[1][i] * inv);
      lo.y = pack_bf16(acc[2][i] * inv, acc[3][i] * inv);
      lo.z = pack_bf16(acc[4][i] * inv, acc[5][i] * inv);
      lo.w = pack_bf16(acc[6][i] * inv, acc[7][i] * inv);
      hi.x = pack_bf16(acc[8][i] * inv, acc[9][i] * inv);
      hi.y = pack_bf16(acc[10][i] * inv, acc[11][i] * inv);
      hi.z = pack_bf16(acc[12][i] * inv, acc[13][i] * inv);
      hi.w = pack_bf16(acc[14][i] * inv, acc[15][i] * inv);
      reinterpret_cast<uint4*>(op + 16 * i)[0] = lo;
      reinterpret_cast<uint4*>(op + 16 * i)[1] = hi;
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 2: out = sum_p w_p O_p / sum_p w_p with w_p = l_p 2^(m_p - max m),
// over the partials with l_p > 0. Grid (B*Hq, D/64); the merge is per
// column, so the chunking does not change any result bit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void stage2_kernel(const uint16_t* __restrict__ part_o,
                                                    const float* __restrict__ part_m,
                                                    const float* __restrict__ part_l,
                                                    uint16_t* __restrict__ out, int P) {
  const size_t bh = blockIdx.x;
  const int d = blockIdx.y * 64 + threadIdx.x;
  const float* pm = part_m + bh * P;
  const float* pl = part_l + bh * P;
  float M = -INFINITY;
  for (int p = 0; p < P; ++p)
    if (pl[p] > 0.f) M = fmaxf(M, pm[p]);
  float num = 0.f, den = 0.f;
  for (int p = 0; p < P; ++p) {
    const float l = pl[p];
    if (l > 0.f) {
      const float w = l * exp2f(pm[p] - M);
      den += w;
      num += w * bf16_to_f32(part_o[(bh * P + p) * kHeadDim + d]);
    }
  }
  const float o = den > 0.f ? num / den : 0.f;
  const uint32_t w = pack_bf16(o, 0.f);
  out[bh * kHeadDim + d] = (uint16_t)(w & 0xFFFF);
}

int largest_divisor_upto(int n, int cap) {
  for (int d = cap < n ? cap : n; d > 1; --d)
    if (n % d == 0) return d;
  return 1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

DecodePlan plan_decode(int B, int Hq, int Hk, int num_kv_splits) {
  DecodePlan p{};
  p.B = B;
  p.Hq = Hq;
  p.Hk = Hk;
  p.QG = Hq / Hk;
  p.splits = num_kv_splits;
  // Enough waves to cover latency: aim for >= 4096 (16 per CU) by cutting each
  // split into contiguous sub-ranges handled by separate waves.
  const long units = (long)B * Hk * num_kv_splits;
  long nsub = (4096 + units - 1) / units;
  if (nsub < 1) nsub = 1;
  if (nsub > 8) nsub = 8;
  p.nsub = (int)nsub;
  p.parts = num_kv_splits * p.nsub;
  const size_t rows = (size_t)B * Hq;
  size_t off = 0;
  p.q8_off = off;
  off = align256(off + rows * kHeadDim);
  p.o_off = off;
  off = align256(off + rows * p.parts * kHeadDim * sizeof(uint16_t));
  p.m_off = off;
  off = align256(off + rows * p.parts * sizeof(float));
  p.l_off = off;
  off = align256(off + rows * p.parts * sizeof(float));
  p.total = off;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, int stage_mask,
                         hipStream_t stream) {
  uint8_t* q8 = a.workspace + p.q8_off;
  uint16_t* part_o = reinterpret_cast<uint16_t*>(a.workspace + p.o_off);
  float* part_m = reinterpret_cast<float*>(a.workspace + p.m_off);
  float* part_l = reinterpret_cast<float*>(a.workspace + p.l_off);
  const int64_t vecs = (int64_t)p.B * p.Hq;

  hipError_t e = hipSuccess;
  if (stage_mask & 1) {
    hipLaunchKernelGGL(qprologue_kernel, dim3((unsigned)((vecs + 3) / 4)), dim3(256), 0, stream,
                       a.query, q8, p.B, p.Hq, a.qsb, a.qsh);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  const int hpw = largest_divisor_upto(p.Hk, 8);
  const int hgroups = p.Hk / hpw;
  int log2_bs = 0;
  while ((1 << log2_bs) < a.block_size) ++log2_bs;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const dim3 grid1((unsigned)((int64_t)p.B * p.splits * p.nsub * hgroups));
  const dim3 block1(64 * hpw);
#define UQ_STAGE1(QGV)                                                                        \
  hipLaunchKernelGGL(stage1_kernel<QGV>, grid1, block1, 0, stream, q8, a.cache, a.block_table, \
                     a.seq_lens, scale_log2, p.Hq, p.Hk, hpw, hgroups, p.splits, p.nsub,     \
                     log2_bs, a.max_blocks_per_seq, a.num_blocks, part_o, part_m, part_l)
  if (stage_mask & 2) {
    switch (p.QG) {
      case 6: UQ_STAGE1(6); break;
      case 8: UQ_STAGE1(8); break;
      case 16: UQ_STAGE1(16); break;
      default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#undef UQ_STAGE1
  if (stage_mask & 4) {
    hipLaunchKernelGGL(stage2_kernel, dim3((unsigned)vecs, kHeadDim / 64), dim3(64), 0, stream,
                       part_o, part_m, part_l, a.out, p.parts);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace uq
