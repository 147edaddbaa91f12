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
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// two floats to fp16, round to nearest even
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2h));
}

// ---------------------------------------------------------------------------
// Query prologue: q8 = E4M3(q H), LPR lanes per (sequence, query head) row,
// 64 / LPR rows per wave, for head dims 128, 256 and 512. LPR = 64 (short
// lane chains) for the rows of a small batch, where latency counts; 16
// (more in-lane butterfly stages, fewer lane exchanges) for large batches,
// where throughput does.
// The rotation runs in float64 and is exact, so the E4M3 rounding decision is
// taken on the exact product (scaled by the float64 1/sqrt(D)).
// ---------------------------------------------------------------------------
template <int D, int LPR>
__global__ __launch_bounds__(256) void qprologue_kernel(const uint16_t* __restrict__ query,
                                                        uint8_t* __restrict__ q8, int B, int Hq,
                                                        int64_t qsb, int64_t qsh) {
  constexpr int E = D / LPR;                   // elements per lane
  static_assert(E >= 2 && E <= 32, "elements per lane");
  const int lane = threadIdx.x & 63, s = lane % LPR;
  const int64_t vec = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;
  const bool valid = vec < (int64_t)B * Hq;
  if (LPR == 64 && !valid) return;             // a whole wave; else every lane runs the exchanges
  const int64_t b = vec / Hq;
  const int64_t hq = vec - b * Hq;
  const uint16_t* qp = query + b * qsb + hq * qsh + E * s;
  double v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = 0.0;
  if (valid) {
    if constexpr (E == 2) {
      const uint32_t r = *reinterpret_cast<const uint32_t*>(qp);
      v[0] = bf16_to_f64(r & 0xFFFF);
      v[1] = bf16_to_f64(r >> 16);
    } else {
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        const uint2 r = *reinterpret_cast<const uint2*>(qp + 4 * c);
        v[4 * c] = bf16_to_f64(r.x & 0xFFFF);
        v[4 * c + 1] = bf16_to_f64(r.x >> 16);
        v[4 * c + 2] = bf16_to_f64(r.y & 0xFFFF);
        v[4 * c + 3] = bf16_to_f64(r.y >> 16);
      }
    }
  }
  fwht_lanes<E, LPR>(v, lane);
  // codes of the float64 products, through float32 rounded to odd
  uint32_t w[(E + 3) / 4] = {};
#pragma unroll
  for (int i = 0; i < E; i += 2)
    w[i / 4] |= e4m3_pair(to_f32_odd(v[i] * rot_scale<D>()), to_f32_odd(v[i + 1] * rot_scale<D>()))
                << (8 * (i % 4));
  if (!valid) return;
  uint8_t* dst = q8 + vec * D + E * s;
  if constexpr (E == 2) {
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[0];
  } else if constexpr (E == 4) {
    *reinterpret_cast<uint32_t*>(dst) = w[0];
  } else if constexpr (E == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int k = 0; k < E / 16; ++k)
      reinterpret_cast<uint4*>(dst)[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
  }
}

// ---------------------------------------------------------------------------
// Stage 1. Workgroup = (sequence b, split s, sub-range, group of KV heads),
// one wave per KV head so that the adjacent 272-byte slots of one token are
// read by one CU. A wave walks its token range in 16-token tiles:
//   scores^T (16 tokens x 16 q-heads) = K (FP4, UE8M0 scales) x q8 (E4M3) on
//     two V_MFMA_SCALE_F32_16X16X128_F8F6F4 (d = 0..127, 128..255);
//   online softmax in the log2 domain; the reference maximum is only raised
//     when a tile exceeds it by more than 8 (p stays <= 256, exact softmax);
//   O^T (256 d x 16 q-heads) += V^T (bf16, converted with its scale) x P^T
//     (bf16 high and low parts of each weight) on 16 V_MFMA_F32_16X16X32_BF16.
// Lane layouts (gfx950):
//   scaled MFMA A (FP4, 4 VGPRs): lane l -> row l%16, k = 32*(l/16) + j for
//     nibble j; its scale byte covers those 32 k.
//   scaled MFMA B (FP8, 8 VGPRs): lane l -> col l%16, byte j -> k = 16*(l/16)+j
//     for j < 16 and 64 + 16*(l/16) + (j-16) above.
//   16x16x32 bf16 A/B: lane l -> row/col l%16, eight k slots.
//   Result: lane l -> col l%16, rows 4*(l/16) + i.
// So the score tile leaves lane (g = l%16, grp = l/16) holding tokens
// 4*grp .. 4*grp+3 of q-head g, which is the P^T operand of the value
// product as it stands (B: col = q-head, k slots = those four tokens, high
// parts, then the same four tokens, low parts); the V^T operand (A) of lane
// l holds dims (D/16)*(l%16) + j of the same four tokens, twice. The
// accumulator O[j] of lane l then holds q-head l%16 at dims
// (D/16)*(4*(l/16) + i) + j: every value a lane accumulates belongs to its
// own head, whose softmax statistics the lane also holds.
// ---------------------------------------------------------------------------
template <int D>
struct Tile {
  uint4 kc[D / 128];           // K codes of token l%16: bytes [64m + 16*grp, +16), m < D/128
  uint32_t ks[D / 128];        // K scale bytes 4m .. 4m+3 of token l%16
  uint32_t vd[4][D / 128];     // V codes: bytes [(D/32)*(l%16), +D/32) of tokens 4*grp + i
  uint32_t vs[4];              // the V-scale dword holding block D*(l%16)/512 of tokens 4*grp + i
  int nvalid;                  // tokens of the tile that are inside the sequence
};

typedef __attribute__((address_space(3))) void lds_void;

// A wave streams the 16-token tiles of its own KV head through a private
// LDS ring: a tile is 16 slots (token stride `row` in the cache), moved by
// direct-to-LDS buffer loads of kDma bytes per lane. At D = 256 a 272-byte
// slot is 17 chunks of 16 bytes and a tile five loads (the last on 16
// lanes); at D = 512, 34 chunks and nine loads. At D = 128 a slot is 136
// bytes, only 8-byte aligned in the cache, so it moves as 34 dwords into an
// LDS token stride of 144 bytes (36 dwords, the last two filler), which
// keeps every LDS operand read 16-byte aligned.
template <int D>
struct Stage {
  static constexpr int kDma = D == 128 ? 4 : 16;
  static constexpr int kValid = Fmt<D>::kSlot / kDma;        // 34, 17, 34
  static constexpr int kPer = D == 128 ? 36 : kValid;        // per token in LDS
  static constexpr int kTokStride = kPer * kDma;             // 144, 272, 544
  static constexpr int kTileChunks = kTile * kPer;
  static constexpr int kLoads = (kTileChunks + 63) / 64;     // 9, 5, 9
  static constexpr int kTileU4 = kTile * kTokStride / 16;    // uint4 per tile in LDS
};

// The caller passes the tile's physical block (see stage1_kernel).
// One plain function per head dim, with literal constants (a function
// template holding these builtins is not viable in the host pass, and
// constants passed as arguments cost the loads' alias information, after
// which the compiler drains the ring before every LDS read).
#define UQ_DEFINE_ISSUE(NAME, SLOT, LOADS, CHUNKS, DMA)                                                \
  __device__ __forceinline__ int NAME(uint4* dst, const uint8_t* __restrict__ cache, int phys, int t,  \
                                      int L, int log2_bs, int64_t num_blocks, uint32_t row, int h,     \
                                      int lane, const uint32_t goff[LOADS]) {                          \
    const int tok0 = t * kTile;                                                                        \
    const bool ok = phys >= 0 && (int64_t)phys < num_blocks;                                           \
    const int nvalid = ok ? min(kTile, L - tok0) : 0;                                                  \
    const size_t tile_off =                                                                            \
        ((((size_t)(ok ? phys : 0)) << log2_bs) + (size_t)(tok0 & ((1 << log2_bs) - 1))) * row +       \
        (size_t)h * (SLOT);                                                                            \
    /* the descriptor ends at the last valid token: chunks past it land as zeros */                  \
    const int nrec = nvalid > 0 ? (nvalid - 1) * (int)row + (SLOT) : 0;                                \
    const __amdgpu_buffer_rsrc_t rs =                                                                  \
        __builtin_amdgcn_make_buffer_rsrc((void*)(cache + tile_off), (short)0, nrec, 0x00020000);      \
    _Pragma("unroll") for (int k = 0; k < (LOADS) - 1; ++k)                                            \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (64 * (DMA) / 16) * k), DMA,      \
                                               goff[k], 0, 0, 0);                                      \
    if (lane < (CHUNKS) - 64 * ((LOADS) - 1))                                                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (64 * (DMA) / 16) * ((LOADS) - 1)), \
                                               DMA, goff[(LOADS) - 1], 0, 0, 0);                       \
    return nvalid;                                                                                     \
  }
UQ_DEFINE_ISSUE(issue_tile_d128, 136, 9, 576, 4)
UQ_DEFINE_ISSUE(issue_tile_d256, 272, 5, 272, 16)
UQ_DEFINE_ISSUE(issue_tile_d512, 544, 9, 544, 16)
#undef UQ_DEFINE_ISSUE

// s_waitcnt on vector memory only (gfx9 encoding; expcnt and lgkmcnt left free)
#define UQ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 0xF) | (((n) >> 4) << 14)) | (0x7 << 4) | (0xF << 8))

// Wait until at most min(K, ahead) tiles (PER loads each) are still in
// flight: the waitcnt immediate must be a constant, so pick it by cases.
template <int K, int PER>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  if constexpr (K == 0) {
    UQ_WAIT_VMCNT(0);
  } else {
    if (ahead >= K) {
      UQ_WAIT_VMCNT(K * PER);
    } else {
      wait_tiles_ahead<K - 1, PER>(ahead);
    }
  }
}

// Operands of one staged tile (LDS token stride Stage<D>::kTokStride).
template <int D>
__device__ __forceinline__ void read_tile(Tile<D>& T, const uint4* __restrict__ src, int n16, int grp,
                                          int nvalid) {
  using F = Fmt<D>;
  constexpr int C = D / 128;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(src);
  const uint8_t* kp = base + n16 * Stage<D>::kTokStride;
#pragma unroll
  for (int m = 0; m < C; ++m) T.kc[m] = *reinterpret_cast<const uint4*>(kp + F::kKCode + 64 * m + 16 * grp);
  if constexpr (C == 1) {
    T.ks[0] = *reinterpret_cast<const uint32_t*>(kp + F::kKScale);
  } else if constexpr (C == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(kp + F::kKScale);
    T.ks[0] = x.x;
    T.ks[1] = x.y;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(kp + F::kKScale);
    T.ks[0] = x.x; T.ks[1] = x.y; T.ks[2] = x.z; T.ks[3] = x.w;
  }
  // V-scale dword of lane row n16: block D*n16/512, i.e. byte n16 >> (9 - log2 D)
  constexpr int vsh = D == 128 ? 4 : (D == 256 ? 3 : 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint8_t* vp = base + (4 * grp + i) * Stage<D>::kTokStride;
    // (read through the pointer, field by field: this form keeps the loads'
    // alias information, without which the ring is drained before the read)
    if constexpr (C == 1) {
      T.vd[i][0] = *reinterpret_cast<const uint32_t*>(vp + F::kVCode + 4 * n16);
    } else if constexpr (C == 2) {
      T.vd[i][0] = reinterpret_cast<const uint2*>(vp + F::kVCode + 8 * n16)->x;
      T.vd[i][1] = reinterpret_cast<const uint2*>(vp + F::kVCode + 8 * n16)->y;
    } else {
      T.vd[i][0] = reinterpret_cast<const uint4*>(vp + F::kVCode + 16 * n16)->x;
      T.vd[i][1] = reinterpret_cast<const uint4*>(vp + F::kVCode + 16 * n16)->y;
      T.vd[i][2] = reinterpret_cast<const uint4*>(vp + F::kVCode + 16 * n16)->z;
      T.vd[i][3] = reinterpret_cast<const uint4*>(vp + F::kVCode + 16 * n16)->w;
    }
    T.vs[i] = *reinterpret_cast<const uint32_t*>(vp + F::kVScale + 4 * (n16 >> vsh));
  }
  T.nvalid = nvalid;
}

// Byte M of each token's D/32 V-code bytes holds dims (D/16)*(l%16) + 2M
// (low nibble) and 2M + 1 (high nibble). Convert them for the lane's 4
// tokens, regroup the bf16 halves by dim, and accumulate two MFMAs (dim even
// / odd) into O^T: the values are the A operand (row = dim), the weights the
// B operand (column = query head), so each lane's accumulators belong to one
// query head. Each MFMA runs over k = 32: the lane's 4 tokens twice, against
// the high and the low bf16 parts of their weights (pb), so a weight enters
// the product with 16 significant bits, not 8.
template <int D, int M>
__device__ __forceinline__ void pv_step(const Tile<D>& T, const float vscale[4], const v8bf& pb,
                                        v4f acc[D / 16]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t src = T.vd[i][M >> 2];
    w[i] = __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, vscale[i], M & 3));
  }
  const uint32_t e0 = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
  const uint32_t e1 = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
  const uint32_t o0 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
  const uint32_t o1 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
  const v8bf ae = __builtin_bit_cast(v8bf, make_uint4(e0, e1, e0, e1));
  const v8bf ao = __builtin_bit_cast(v8bf, make_uint4(o0, o1, o0, o1));
  acc[2 * M] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, pb, acc[2 * M], 0, 0, 0);
  acc[2 * M + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, pb, acc[2 * M + 1], 0, 0, 0);
}

// Maximum over the four 16-lane row groups (lanes l, l^16, l^32, l^48), with
// the in-register row swaps of gfx950 instead of LDS permutes.
__device__ __forceinline__ float rowgroup_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Scores of one tile in the log2 domain (lane: q-head l%16, tokens 4*grp+i),
// -inf from token `lc` of the tile on (the end of the lane's query row) and
// past the tile's valid tokens, and for the tile's first `first` tokens
// (those before a sliding window), all only when `edge`; mt = the tile
// maximum for the lane's head.
template <int D>
__device__ __forceinline__ void qk_tile(const Tile<D>& T, const v8i qb[D / 128], float scale_log2,
                                        int grp, int first, bool edge, int lc, float sv[4], float& mt) {
  v4f sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D / 128; ++m) {
    const int scm = (int)((T.ks[m] >> (8 * grp)) & 0xFF);
    const v8i a = {(int)T.kc[m].x, (int)T.kc[m].y, (int)T.kc[m].z, (int)T.kc[m].w, 0, 0, 0, 0};
    sc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qb[m], sc, 4, 0, 0, scm, 0, 127);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = sc[i] * scale_log2;
  // edge (wave-uniform): the tile holds the end of some column's row or the
  // start of the window; lc: the lane's column's length from the tile's start
  if (edge) {
    const int lim = min(T.nvalid, lc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * grp + i >= lim || 4 * grp + i < first) sv[i] = -INFINITY;
  }
  mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mt = rowgroup_max(mt);
}

// Softmax weights p = 2^(s - m_ref) (<= 2^8 by the re-basing rule), then
// O^T += V^T P^T. Touches the accumulators only through MFMAs.
template <int D>
__device__ __forceinline__ void pv_tile(const Tile<D>& T, const float sv[4], float m_ref, int n16,
                                        v4f acc[D / 16], float& l_part) {
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref);
  // Each weight as the sum of two bf16 values: hi = bf16(p) and
  // lo = bf16(p - hi) (p - hi is exact in float32), within 2^-16 p of p. A
  // single bf16 weight (relative error up to 2^-8) put up to 2^-8 |v - o|
  // into the output where a few tokens dominate.
  const uint32_t h01 = pack_bf16(p[0], p[1]);
  const uint32_t h23 = pack_bf16(p[2], p[3]);
  const float q0 = __uint_as_float(h01 << 16), q1 = __uint_as_float(h01 & 0xFFFF0000u);
  const float q2 = __uint_as_float(h23 << 16), q3 = __uint_as_float(h23 & 0xFFFF0000u);
  const uint32_t l01 = pack_bf16(p[0] - q0, p[1] - q1);
  const uint32_t l23 = pack_bf16(p[2] - q2, p[3] - q3);
  // the denominator sums the weights the product uses (hi + lo), so a
  // dominant token passes through with weight exactly 1
  l_part += ((q0 + __uint_as_float(l01 << 16)) + (q1 + __uint_as_float(l01 & 0xFFFF0000u))) +
            ((q2 + __uint_as_float(l23 << 16)) + (q3 + __uint_as_float(l23 & 0xFFFF0000u)));
  const v8bf pb = __builtin_bit_cast(v8bf, make_uint4(h01, h23, l01, l23));
  float vscale[4];
  const int vsh = 8 * (((D * n16) / 512) & 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) vscale[i] = __uint_as_float(((T.vs[i] >> vsh) & 0xFFu) << 23);
  pv_step<D, 0>(T, vscale, pb, acc);
  pv_step<D, 1>(T, vscale, pb, acc);
  pv_step<D, 2>(T, vscale, pb, acc);
  pv_step<D, 3>(T, vscale, pb, acc);
  if constexpr (D >= 256) {
    pv_step<D, 4>(T, vscale, pb, acc);
    pv_step<D, 5>(T, vscale, pb, acc);
    pv_step<D, 6>(T, vscale, pb, acc);
    pv_step<D, 7>(T, vscale, pb, acc);
  }
  if constexpr (D >= 512) {
    pv_step<D, 8>(T, vscale, pb, acc);
    pv_step<D, 9>(T, vscale, pb, acc);
    pv_step<D, 10>(T, vscale, pb, acc);
    pv_step<D, 11>(T, vscale, pb, acc);
    pv_step<D, 12>(T, vscale, pb, acc);
    pv_step<D, 13>(T, vscale, pb, acc);
    pv_step<D, 14>(T, vscale, pb, acc);
    pv_step<D, 15>(T, vscale, pb, acc);
  }
}

// In-kernel query prologue at head dim 256: q8 = E4M3(q H) for the wave's
// QG query rows, computed while the first tiles are in flight. The 256-point
// Hadamard is the Kronecker square of the 16-point one (H256[16a+b][16a'+b']
// = H16[a][a'] H16[b][b'], popcounts add), so per row, with Q[a][b] =
// q[16a + b], Y = H16 Q H16 is two 16 x 16 x 16 products. Every product is q
// times +-1 and every partial sum a +-subset sum of the row, so float64 keeps
// them exact (the same exactness condition as the butterfly) and the E4M3
// rounding sees the exact y = Y / 16.
// V_MFMA_F64_16X16X4F64 reads A[m][k] from lane (m, k) and B[k][n] from lane
// (n, k), and returns row g + 4i of D in register i of lane (n, g) (measured;
// the 16-bit MFMAs return row 4g + i there).
//   Z = Q H16: MFMA kb takes, in lane (c, g), A = q[16c + 4g + kb] (row c,
//     k slot g -> b = 4g + kb) and B = H16[4g + kb][c]; Z[g + 4i][c] lands in
//     register i of lane (c, g).
//   Y = H16 Z: MFMA kb takes A = H16[c][4g + kb] and, as B, register kb of
//     the lane's own Z, i.e. Z[g + 4kb][c]: k slot g of MFMA kb stands for
//     a = g + 4kb while A carries column 4g + kb, its 2-bit halves swapped.
//     Since H16[m][swap(a)] = H16[swap(m)][a], the product is Y with its row
//     index swapped the same way, and the f64 layout swaps it back:
//     Y[4g + i][c] = y[16 (4g + i) + c] lands in register i of lane (c, g).
// The codes go through the wave's free LDS slot (QG rows of 256 bytes) into
// the scaled MFMA's B layout (lane (head c, g): bytes 16g .. 16g + 15 and
// 64 + 16g .. 64 + 16g + 15 of each 128-byte half of row c).
typedef double v4d __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4d mfma_f64(double a, double b, v4d c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <int QG>
__device__ __forceinline__ void load_query_rows(const uint16_t* __restrict__ query, int64_t qsb, int64_t qsh,
                                                int b, int h, int lane, uint2 qraw[QG]) {
  const int n16 = lane & 15, grp = lane >> 4;
  const uint16_t* qp = query + (int64_t)b * qsb + (int64_t)h * QG * qsh + 16 * n16 + 4 * grp;
#pragma unroll
  for (int r = 0; r < QG; ++r) qraw[r] = *reinterpret_cast<const uint2*>(qp + (int64_t)r * qsh);
}

template <int QG>
__device__ __forceinline__ void rotate_queries_d256(const uint2 qraw[QG], int lane, uint8_t* __restrict__ rows,
                                                    v8i qb[2]) {
  const int n16 = lane & 15, grp = lane >> 4;
  double hs[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) hs[kb] = (__popc((4 * grp + kb) & n16) & 1) ? -1.0 : 1.0;
#pragma unroll
  for (int r = 0; r < QG; ++r) {
    const double q[4] = {bf16_to_f64(qraw[r].x & 0xFFFF), bf16_to_f64(qraw[r].x >> 16),
                         bf16_to_f64(qraw[r].y & 0xFFFF), bf16_to_f64(qraw[r].y >> 16)};
    v4d z = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) z = mfma_f64(q[kb], hs[kb], z);
    v4d y = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) y = mfma_f64(hs[kb], z[kb], y);
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const uint32_t c = e4m3_pair(to_f32_odd(y[i] * 0.0625), to_f32_odd(y[i + 1] * 0.0625));
      rows[r * 256 + 16 * (4 * grp + i) + n16] = (uint8_t)c;
      rows[r * 256 + 16 * (4 * grp + i + 1) + n16] = (uint8_t)(c >> 8);
    }
  }
  // the wave's own LDS writes are seen by its later reads in program order
  if (n16 < QG) {
    const uint8_t* rp = rows + n16 * 256;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(rp + 128 * m + 16 * grp);
      const uint4 x1 = *reinterpret_cast<const uint4*>(rp + 128 * m + 64 + 16 * grp);
      qb[m] = (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
  }
}

// MODE 0: query codes from the workspace; 1: the query prologue inside
// (head dim 256); 2: multi-query rows paired as described below (QG <= 8).
template <int D, int QG, int HPW, int NSLOT, int MODE>
__global__ __launch_bounds__(64 * HPW) void stage1_kernel(
    const uint8_t* __restrict__ q8, const uint16_t* __restrict__ query, int64_t qsb, int64_t qsh,
    const uint8_t* __restrict__ cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ query_row, int n_rows,
    const int32_t* __restrict__ seq_lens,
    float scale_log2, int Hq, int Hk, int hgroups, int cs, int spw, int nsub, int P,
    int log2_bs, int max_blocks, int64_t num_blocks, int window, int n_qrows,
    uint16_t* __restrict__ part_o, float* __restrict__ part_m, float* __restrict__ part_l,
    int* __restrict__ part_e) {
  constexpr bool FUSEQ = MODE == 1, PAIR = MODE == 2;
  static_assert(!PAIR || QG <= 8, "paired rows need half the MFMA columns free");
  static_assert(NSLOT >= 2 && NSLOT <= 8, "ring depth");
  using S = Stage<D>;
  static_assert(NSLOT * HPW * S::kTileU4 * 16 <= 160 * 1024, "ring exceeds the LDS of a CU");
  constexpr int C = D / 128;               // scaled MFMAs per score tile
  constexpr int NA = D / 16;               // O^T accumulators
  // NSLOT-slot ring per wave; distinct arrays so that the compiler can tell
  // the slot being read from the slots being filled
#define UQ_RING_DECL(K) __shared__ uint4 ring##K[NSLOT > K ? HPW : 1][NSLOT > K ? S::kTileU4 : 1];
  UQ_RING_DECL(0) UQ_RING_DECL(1) UQ_RING_DECL(2) UQ_RING_DECL(3)
  UQ_RING_DECL(4) UQ_RING_DECL(5) UQ_RING_DECL(6) UQ_RING_DECL(7)
#undef UQ_RING_DECL

  // Workgroups are dealt to the 8 XCDs round-robin by index. The grid is
  // ordered partial-major (every (sequence, head group) of partial 0 first),
  // and within each band of n1 = B * hgroups workgroups the items rotate by
  // the partial index, so the partials of one sequence land on different
  // XCDs: the late, often empty, partials of short sequences are then spread
  // over the chip instead of all sitting on the same XCD.
  // With paired rows the even rows' workgroups come first and the odd rows'
  // (which exit when their row pairs) after them, each half in that order,
  // so the streaming workgroups are dispatched first and spread over the CUs.
  int rows = (int)(gridDim.x / (unsigned)(P * hgroups)), x = (int)blockIdx.x, r0 = 0, rstep = 1;
  if constexpr (PAIR) {
    const int n_even = (rows + 1) / 2, first_odd = n_even * P * hgroups;
    rstep = 2;
    if (x < first_odd) {
      rows = n_even;
    } else {
      x -= first_odd;
      rows -= n_even;
      r0 = 1;
    }
  }
  const int n1 = rows * hgroups;
  const int part = x / n1;                          // partial index within (b, head)
  int j = x - part * n1 + part % n1;
  j = j >= n1 ? j - n1 : j;
  const int hg = j % hgroups;
  const int b = r0 + rstep * (j / hgroups);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = hg * HPW + wave;

  // Split s covers tiles [s*cs, (s+1)*cs) counted from the first tile the
  // query attends to (tile 0, or the tile of a sliding window's first token);
  // cs comes from the table capacity (or the window), so every split is the
  // same size. A partial covers either spw consecutive splits or one of nsub
  // equal pieces of one split.
  const int g_rel = (part / nsub) * spw * cs;
  const int sub_len = (spw * cs + nsub - 1) / nsub;
  const int u_rel = g_rel + (part % nsub) * sub_len;
  const int n16 = lane & 15, grp = lane >> 4;
  static_assert(!FUSEQ || D == 256, "the in-kernel query prologue is built for head dim 256");
  // Query row b reads block-table row query_row[b] (its own row when there
  // is no mapping); a row outside the table reads as an empty sequence.
  const int trow = query_row ? query_row[b] : b;
  const bool row_ok = trow >= 0 && trow < n_rows;
  // Paired rows (QG <= 8, no window): query rows 2r and 2r + 1 that read the
  // same table row share the wave of row 2r, row 2r + 1 in MFMA columns
  // QG .. 2 QG - 1, so their common tiles are read once; the wave of row
  // 2r + 1 then has nothing to do. The split boundaries come from the table
  // capacity, the same for both rows; each column masks past its own length.
  bool paired = false;
  if constexpr (PAIR) {
    if (row_ok && (b ^ 1) < n_qrows && query_row[b ^ 1] == trow) {
      if (b & 1) return;
      paired = true;
    }
  }
  const int QC = paired ? 2 * QG : QG;               // query columns in use
  const bool qlane = n16 < QC;
  const int crow = (PAIR && n16 >= QG && paired) ? b + 1 : b;   // the column's query row
  const int hq = h * QG + (qlane ? (PAIR ? n16 % QG : n16) : 0);
  v8i qb[C];
#pragma unroll
  for (int m = 0; m < C; ++m) qb[m] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
  // the query rows (FUSEQ: bf16, rotated below) or their codes, requested
  // first so that they are not queued behind the tiles
  uint2 qraw[FUSEQ ? QG : 1];
  if constexpr (FUSEQ) {
    load_query_rows<QG>(query, qsb, qsh, b, h, lane, qraw);
  } else if (qlane) {
    const uint8_t* qp = q8 + ((size_t)crow * Hq + hq) * D;
#pragma unroll
    for (int m = 0; m < C; ++m) {
      const uint4 x0 = ld16(qp + 128 * m + 16 * grp), x1 = ld16(qp + 128 * m + 64 + 16 * grp);
      qb[m] = (v8i){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
  }
  const int32_t* bt = block_table + (size_t)(row_ok ? trow : 0) * max_blocks;
  // The wave's first table entry does not depend on the length unless a
  // sliding window moves the range, so its entries are requested together
  // with seq_lens: one round trip before the first tile is issued, not two.
  int e0 = (u_rel * kTile) >> log2_bs;
  int btv = (row_ok && e0 + lane < max_blocks) ? bt[e0 + lane] : 0;
  // entries e0 .. e0 + 7 also as scalars, which arrive with seq_lens: the
  // tiles that fill the ring at the start are issued from them, without
  // waiting for the vector load of btv
  int s_ent[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) s_ent[k] = bt[min(e0 + k, max_blocks - 1)];
  const int Lcap = max_blocks << log2_bs;
  int L = row_ok ? seq_lens[b] : 0;
  L = L < 0 ? 0 : (L > Lcap ? Lcap : L);
  // the column's own length (paired rows: each row's), L the longest; from
  // tile t_edge on a tile may hold the end of the shorter row
  int Lc = L, t_edge = 0x7FFFFFFF;
  if (PAIR && paired) {
    int L2 = seq_lens[b + 1];
    L2 = L2 < 0 ? 0 : (L2 > Lcap ? Lcap : L2);
    if (n16 >= QG) Lc = L2;
    t_edge = (L < L2 ? L : L2) / kTile;
    L = L > L2 ? L : L2;
  }
  // A sliding window of W tokens starts at token lo = L - W: the splits count
  // from lo's tile, and the tokens of that tile before lo are masked.
  const int lo = (window > 0 && L > window) ? L - window : 0;
  const int base = lo / kTile;
  const int u0 = base + u_rel;
  const int n_tiles = (L + kTile - 1) / kTile;
  const int u1 = min(min(u0 + sub_len, base + g_rel + spw * cs), n_tiles);
  if (base > 0) {
    e0 = (u0 * kTile) >> log2_bs;
    btv = (row_ok && e0 + lane < max_blocks) ? bt[e0 + lane] : 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s_ent[k] = bt[min(e0 + k, max_blocks - 1)];
  }
  const size_t stat = ((size_t)crow * Hq + hq) * P + part;

  if (u0 >= u1) {
    if (qlane && grp == 0) {
      part_m[stat] = -INFINITY;
      part_l[stat] = 0.f;
    }
    return;
  }

  const uint32_t row = (uint32_t)Hk * Fmt<D>::kSlot;
  uint32_t goff[S::kLoads];   // load k, lane -> chunk c: token c / kPer, piece c % kPer (filler: piece 0)
#pragma unroll
  for (int k = 0; k < S::kLoads; ++k) {
    const int c = min(64 * k + lane, S::kTileChunks - 1);
    const int piece = c % S::kPer;
    goff[k] = (c / S::kPer) * row + (piece < S::kValid ? piece : 0) * S::kDma;
  }
  static_assert(Fmt<D>::kSlot == (D == 128 ? 136 : D == 256 ? 272 : 544) &&
                    S::kLoads == (D == 256 ? 5 : 9) && S::kTileChunks == (D == 128 ? 576 : D == 256 ? 272 : 544) &&
                    S::kDma == (D == 128 ? 4 : 16),
                "the issue_tile_d* constants follow Stage<D>");
  // Physical block of tile TT: entries e0 .. e0 + 63 sit one per lane in
  // `btv`, loaded once; an entry past them (ranges of more than 64 blocks) is
  // read from memory when its tile is issued. The first fill of the ring
  // takes entries e0 .. e0 + 7 from the scalars (at most 7 tiles, at most one
  // entry each).
#define UQ_PHYS_B(TT)                                                                                  \
  ((((TT) * kTile) >> log2_bs) - e0 < 64                                                               \
       ? __builtin_amdgcn_readlane(btv, (((TT) * kTile) >> log2_bs) - e0)                              \
       : __builtin_amdgcn_readfirstlane(bt[((TT) * kTile) >> log2_bs]))
#define UQ_PHYS_S(TT) s_ent[((((TT) * kTile) >> log2_bs) - e0) & 7]
#define issue_at(SLOT, TT, PH)                                                                          \
  (D == 128 ? issue_tile_d128(SLOT, cache, PH, TT, L, log2_bs, num_blocks, row, h, lane, goff)         \
   : D == 256 ? issue_tile_d256(SLOT, cache, PH, TT, L, log2_bs, num_blocks, row, h, lane, goff)       \
              : issue_tile_d512(SLOT, cache, PH, TT, L, log2_bs, num_blocks, row, h, lane, goff))
#define issue(SLOT, TT) issue_at(SLOT, TT, UQ_PHYS_B(TT))

  // Softmax reference: the first tile's maximum. The weights 2^(s - m_ref)
  // are exact for any reference; keeping them <= 2^8 bounds their range. A
  // tile that exceeds the reference by more than that ends the tile loop:
  // outside it, each lane scales its accumulators and weight sum (all of its
  // own head) to the raised reference, and the loop resumes at that tile.
  // Inside the loop the accumulators are only touched by MFMAs, so they stay
  // in the accumulator registers and the rare rescale stays out of the loop
  // body.
  v4f acc[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_part = 0.f;
  int t0 = u0;
  // valid-token count of the tile in each slot, known when it is issued
  int nv_ring0 = 0, nv_ring1 = 0, nv_ring2 = 0, nv_ring3 = 0;
  int nv_ring4 = 0, nv_ring5 = 0, nv_ring6 = 0, nv_ring7 = 0;
#define UQ_PRE(K, PHYS) \
  if constexpr (NSLOT > K + 1) { if (t0 + K < u1) nv_ring##K = issue_at(ring##K[wave], t0 + K, PHYS(t0 + K)); }
  nv_ring0 = issue_at(ring0[wave], t0, UQ_PHYS_S(t0));
  UQ_PRE(1, UQ_PHYS_S) UQ_PRE(2, UQ_PHYS_S) UQ_PRE(3, UQ_PHYS_S) UQ_PRE(4, UQ_PHYS_S) UQ_PRE(5, UQ_PHYS_S)
  UQ_PRE(6, UQ_PHYS_S)
  if constexpr (FUSEQ) {
    // The ring's last slot is not filled before the first step: it holds the
    // code rows of the transpose, read back (and waited for) before that
    // step issues a tile into it.
#define UQ_SLOT_PTR(K) (NSLOT > K ? &ring##K[NSLOT > K ? wave : 0][0] : &ring0[0][0])
    uint4* const last = NSLOT == 2 ? UQ_SLOT_PTR(1) : NSLOT == 3 ? UQ_SLOT_PTR(2) : NSLOT == 4 ? UQ_SLOT_PTR(3)
                      : NSLOT == 5 ? UQ_SLOT_PTR(4) : NSLOT == 6 ? UQ_SLOT_PTR(5) : NSLOT == 7 ? UQ_SLOT_PTR(6)
                                                                                    : UQ_SLOT_PTR(7);
#undef UQ_SLOT_PTR
    static_assert(QG * 256 <= S::kTileU4 * 16, "a ring slot holds the code rows");
    rotate_queries_d256<QG>(qraw, lane, reinterpret_cast<uint8_t*>(last), qb);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the code rows are read before the slot refills
  }
  bool filled = true;
  for (;;) {
    Tile<D> T;
    float sv[4], mt;
    bool rebased = false;
    int t_stop = 0;
    if (!filled) {              // after a re-base the ring is refilled at t0
      nv_ring0 = issue(ring0[wave], t0);
      UQ_PRE(1, UQ_PHYS_B) UQ_PRE(2, UQ_PHYS_B) UQ_PRE(3, UQ_PHYS_B) UQ_PRE(4, UQ_PHYS_B) UQ_PRE(5, UQ_PHYS_B)
      UQ_PRE(6, UQ_PHYS_B)
    }
    filled = false;
    // Step t: tiles t .. t + NSLOT - 2 are in flight. Wait for tile t (the
    // later ones may stay pending), read it, start tile t + NSLOT - 1 into the
    // slot tile t - 1 used (already consumed), then compute tile t.
#define UQ_STEP(CUR, NXT)                                                        \
    {                                                                            \
      wait_tiles_ahead<NSLOT - 2, S::kLoads>(u1 - 1 - t);                        \
      read_tile<D>(T, CUR[wave], n16, grp, nv_##CUR);                            \
      if (t + NSLOT - 1 < u1) nv_##NXT = issue(NXT[wave], t + NSLOT - 1);        \
      qk_tile<D>(T, qb, scale_log2, grp, lo - t * kTile,                        \
                 T.nvalid < kTile || lo > t * kTile || (PAIR && t >= t_edge),          \
                 PAIR ? Lc - t * kTile : kTile, sv, mt);                          \
      if (t == u0) m_ref = (!PAIR || mt > -INFINITY) ? mt : 0.f;                 \
      if (__any(mt > m_ref + 8.0f)) { rebased = true; t_stop = t; break; }       \
      if (T.nvalid > 0) pv_tile<D>(T, sv, m_ref, n16, acc, l_part);              \
      if (++t >= u1) break;                                                      \
    }
    if constexpr (NSLOT == 2) {
      for (int t = t0;;) {
        UQ_STEP(ring0, ring1) UQ_STEP(ring1, ring0)
      }
    } else if constexpr (NSLOT == 3) {
      for (int t = t0;;) {
        UQ_STEP(ring0, ring2) UQ_STEP(ring1, ring0) UQ_STEP(ring2, ring1)
      }
    } else if constexpr (NSLOT == 4) {
      for (int t = t0;;) {
        UQ_STEP(ring0, ring3) UQ_STEP(ring1, ring0) UQ_STEP(ring2, ring1) UQ_STEP(ring3, ring2)
      }
    } else if constexpr (NSLOT == 5) {
      for (int t = t0;;) {
        UQ_STEP(ring0, ring4) UQ_STEP(ring1, ring0) UQ_STEP(ring2, ring1) UQ_STEP(ring3, ring2)
        UQ_STEP(ring4, ring3)
      }
    } else if constexpr (NSLOT == 6) {
      for (int t = t0;;) {
        UQ_STEP(ring0, ring5) UQ_STEP(ring1, ring0) UQ_STEP(ring2, ring1) UQ_STEP(ring3, ring2)
        UQ_STEP(ring4, ring3) UQ_STEP(ring5, ring4)
      }
    } else if constexpr (NSLOT == 7) {
      for (int t = t0;;) {
        UQ_STEP(ring0, ring6) UQ_STEP(ring1, ring0) UQ_STEP(ring2, ring1) UQ_STEP(ring3, ring2)
        UQ_STEP(ring4, ring3) UQ_STEP(ring5, ring4) UQ_STEP(ring6, ring5)
      }
    } else {
      for (int t = t0;;) {
        UQ_STEP(ring0, ring7) UQ_STEP(ring1, ring0) UQ_STEP(ring2, ring1) UQ_STEP(ring3, ring2)
        UQ_STEP(ring4, ring3) UQ_STEP(ring5, ring4) UQ_STEP(ring6, ring5) UQ_STEP(ring7, ring6)
      }
    }
#undef UQ_STEP
    if (!rebased) break;
    // Raise the reference to cover tile t_stop (never below the old one, so
    // the factor is <= 1) and rescale the lane's sums in place. Drain the
    // ring; the loop resumes at t_stop, which is then within 2^8 of the
    // reference.
    const float m_new = fmaxf(m_ref, mt);
    const float f = m_new > m_ref ? exp2f(m_ref - m_new) : 1.f;
#pragma unroll
    for (int j = 0; j < NA; ++j) acc[j] *= f;
    l_part *= f;
    m_ref = m_new;
    UQ_WAIT_VMCNT(0);
    t0 = t_stop;
  }
#undef UQ_PRE
#undef issue
#undef issue_at
#undef UQ_PHYS_S
#undef UQ_PHYS_B

  // Lane (head l%16, any grp) holds that head's weight sum after the reduction.
  const float l1 = l_part + __shfl_xor(l_part, 16);
  const float l_tot = l1 + __shfl_xor(l1, 32);
  // a non-empty range has l >= 1 (its largest weight is exactly 1); a
  // paired row may have no token in it (l = 0: an empty partial)
  const float inv = (!PAIR || l_tot > 0.f) ? 1.f / l_tot : 0.f;
  // The partial O / l of each query head is stored as an fp16 row times
  // 2^ex, with ex chosen from the row's largest magnitude so that it lands in
  // [2^14, 2^15): the rounding error is at most 2^-11 of the row maximum. The
  // row leaves as one contiguous store: the lanes first place their dims in
  // the wave's own ring, free now that every tile it issued has been
  // consumed (row stride 2 D + 16 bytes, RPS rows per slot), then each row is
  // read back across the wave. Lane (head l%16, grp) holds dims
  // (D/16)*(4*grp + i) + j of its head, so the head's maximum is one
  // reduction over the four row groups.
  constexpr int RS = D * 2 + 16;
  constexpr int RPS = S::kTileU4 * 16 / RS;
  static_assert(((PAIR ? 2 * QG : QG) + RPS - 1) / RPS <= NSLOT, "the ring cannot stage the partial rows");
#define UQ_OWN_PTR(K) (NSLOT > K ? &ring##K[NSLOT > K ? wave : 0][0] : &ring0[0][0])
  uint4* const own[8] = {UQ_OWN_PTR(0), UQ_OWN_PTR(1), UQ_OWN_PTR(2), UQ_OWN_PTR(3),
                         UQ_OWN_PTR(4), UQ_OWN_PTR(5), UQ_OWN_PTR(6), UQ_OWN_PTR(7)};
#undef UQ_OWN_PTR
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < NA; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(acc[j][i]));
  amax = rowgroup_max(amax * inv);
  const int ex = amax > 0.f ? (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 14 : 0;
  if (qlane && grp == 0) {
    part_m[stat] = (!PAIR || l_tot > 0.f) ? m_ref : -INFINITY;
    part_l[stat] = l_tot;
    part_e[stat] = ex;
  }
  if (qlane) {
    uint8_t* rowp = reinterpret_cast<uint8_t*>(own[n16 / RPS]) + (n16 % RPS) * RS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < NA; j += 8) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          w[k] = pack_f16(__builtin_amdgcn_ldexpf(acc[j + 2 * k][i] * inv, -ex),
                          __builtin_amdgcn_ldexpf(acc[j + 2 * k + 1][i] * inv, -ex));
        *reinterpret_cast<uint4*>(rowp + 2 * (NA * (4 * grp + i) + j)) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < (PAIR ? 2 * QG : QG); ++r) {
    if (PAIR && r >= QC) break;
    const size_t prow = ((size_t)(r < QG ? b : b + 1) * Hq + (size_t)h * QG + r % QG) * P + part;
    const uint8_t* rowp = reinterpret_cast<const uint8_t*>(own[r / RPS]) + (r % RPS) * RS;
    uint8_t* dst = reinterpret_cast<uint8_t*>(part_o + prow * D);
    if constexpr (D == 128) {
      *reinterpret_cast<uint32_t*>(dst + 4 * lane) = *reinterpret_cast<const uint32_t*>(rowp + 4 * lane);
    } else if constexpr (D == 256) {
      *reinterpret_cast<uint2*>(dst + 8 * lane) = *reinterpret_cast<const uint2*>(rowp + 8 * lane);
    } else {
      *reinterpret_cast<uint4*>(dst + 16 * lane) = *reinterpret_cast<const uint4*>(rowp + 16 * lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 2: out = sum_p w_p O_p / sum_p w_p with w_p = l_p 2^(m_p - max m),
// over the partials with l_p > 0, in one pass with a running maximum (the sums
// are rescaled when it rises); O_p is the stored fp16 row times 2^ex_p. One
// wave per (sequence, query head) row; lane l owns columns E l .. E l + E - 1
// (E = D / 64), so a partial row is one coalesced read, and eight partial rows
// are in flight per lane. The statistics are uniform across the wave: the
// rows of empty partials (never written) are neither read nor used.
// ---------------------------------------------------------------------------
// With many partials per row (G = 2 or 4), G waves of the workgroup share a
// row: wave g merges partials [g P / G, (g + 1) P / G) and the first wave
// folds the others' (max, denominator, sums) in from LDS.
template <int D, int G>
__global__ __launch_bounds__(256) void stage2_kernel(const uint16_t* __restrict__ part_o,
                                                     const float* __restrict__ part_m,
                                                     const float* __restrict__ part_l,
                                                     const int* __restrict__ part_e,
                                                     const float* __restrict__ sinks, int Hq,
                                                     uint16_t* __restrict__ out, int rows, int P) {
  static_assert(G == 1 || G == 2 || G == 4, "waves per row");
  constexpr int E = D / 64;                  // columns per lane: E l .. E l + E - 1
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (4 / G) + wave / G;
  const int g = wave % G;
  if (G == 1 && row >= rows) return;
  const bool valid = row < rows;
  const int lane = threadIdx.x & 63;
  const size_t rowc = valid ? (size_t)row : 0;
  const float* pm = part_m + rowc * P;
  const float* pl = part_l + rowc * P;
  const int* pe = part_e + rowc * P;
  const uint16_t* po = part_o + rowc * P * D + E * lane;
  const int pb = valid ? (int)(((long)g * P) / G) : 0;
  const int pend = valid ? (int)(((long)(g + 1) * P) / G) : 0;
  float M = -INFINITY, den = 0.f;
  if (sinks && g == 0 && valid) {   // the sink: a partial of weight 1 at its logit, with no value
    M = sinks[row % Hq] * 1.4426950408889634f;
    den = 1.f;
  }
  float a[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = 0.f;
  for (int p0 = pb; p0 < pend; p0 += 8) {
    uint32_t h[8][E / 2];
    float m[8], l[8];
    int ex[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = min(p0 + u, pend - 1);
      m[u] = pm[p];
      l[u] = p0 + u < pend ? pl[p] : 0.f;
      ex[u] = pe[p];
    }
    // only the rows of non-empty partials are read (an empty one was never written)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t* src = po + (size_t)min(p0 + u, pend - 1) * D;
      if (l[u] > 0.f) {
        if constexpr (E == 2) {
          h[u][0] = *reinterpret_cast<const uint32_t*>(src);
        } else if constexpr (E == 4) {
          const uint2 x = *reinterpret_cast<const uint2*>(src);
          h[u][0] = x.x; h[u][1] = x.y;
        } else {
          const uint4 x = *reinterpret_cast<const uint4*>(src);
          h[u][0] = x.x; h[u][1] = x.y; h[u][2] = x.z; h[u][3] = x.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E / 2; ++e) h[u][e] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (l[u] > 0.f) {
        const float Mn = fmaxf(M, m[u]);
        const float c = exp2f(M - Mn);            // 0 for the first partial, <= 1 after
        const float w = l[u] * exp2f(m[u] - Mn);
        den = den * c + w;
#pragma unroll
        for (int e = 0; e < E / 2; ++e) {
          const v2h x = __builtin_bit_cast(v2h, h[u][e]);
          a[2 * e] = a[2 * e] * c + w * __builtin_amdgcn_ldexpf((float)x[0], ex[u]);
          a[2 * e + 1] = a[2 * e + 1] * c + w * __builtin_amdgcn_ldexpf((float)x[1], ex[u]);
        }
        M = Mn;
      }
    }
  }
  if constexpr (G > 1) {
    __shared__ float xs[4][64][E + 2];
    if (g > 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) xs[wave][lane][e] = a[e];
      xs[wave][lane][E] = M;
      xs[wave][lane][E + 1] = den;
    }
    __syncthreads();
    if (g > 0 || !valid) return;
#pragma unroll
    for (int k = 1; k < G; ++k) {
      const float m2 = xs[wave + k][lane][E], d2 = xs[wave + k][lane][E + 1];
      if (d2 > 0.f) {
        const float Mn = fmaxf(M, m2);
        const float c1 = exp2f(M - Mn), c2 = exp2f(m2 - Mn);
        den = den * c1 + d2 * c2;
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] = a[e] * c1 + xs[wave + k][lane][e] * c2;
        M = Mn;
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint32_t r[E / 2];
#pragma unroll
  for (int e = 0; e < E / 2; ++e) r[e] = pack_bf16(a[2 * e] * inv, a[2 * e + 1] * inv);
  uint16_t* dst = out + (size_t)row * D + E * lane;
  if constexpr (E == 2) {
    *reinterpret_cast<uint32_t*>(dst) = r[0];
  } else if constexpr (E == 4) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(r[0], r[1]);
  } else {
    *reinterpret_cast<uint4*>(dst) = make_uint4(r[0], r[1], r[2], r[3]);
  }
}

// KV heads per stage-1 workgroup, one wave each: 4, 2 or 1, the largest
// that divides Hk (an odd count such as 3 takes one head per workgroup).
// At Hk = 8 four heads per workgroup measured 265 us on the ragged workload
// against 277 us for two.
int heads_per_workgroup(int hk) {
  for (int d = 4; d > 1; d /= 2)
    if (hk % d == 0) return d;
  return 1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Ring depth: three slots (two tiles in flight while one is computed)
// measured faster than four on every workload (decode 36.5-36.8 against
// 37.1-37.5 us per step; mixed, ragged and head dims 128, 512 too), five and
// eight slower.
#ifndef UQ_RING_SLOTS
#define UQ_RING_SLOTS 3
#endif
#ifndef UQ_TARGET_WAVES
#define UQ_TARGET_WAVES 1024
#endif
#ifndef UQ_TILES_PER_WAVE_MAX
#define UQ_TILES_PER_WAVE_MAX 64
#endif
// Ring depth per wave: as deep as the LDS of one CU allows for the
// workgroup's HPW waves (4352 bytes per slot), capped at UQ_RING_SLOTS.
template <int D>
constexpr int ring_slots(int hpw) {
  return (160 * 1024) / (hpw * Stage<D>::kTileU4 * 16) < UQ_RING_SLOTS
             ? (160 * 1024) / (hpw * Stage<D>::kTileU4 * 16)
             : UQ_RING_SLOTS;
}
constexpr long kTilesPerWaveMin = 4;
// At D = 128 a tile carries half the bytes for much the same serial work per
// wave (scores, softmax, the value MFMAs), so twice the waves stream it
// faster; at D = 256 and 512 more waves only add partials (measured).
static int target_waves(int D) { return D == 128 ? 2 * UQ_TARGET_WAVES : UQ_TARGET_WAVES; }

DecodePlan plan_decode(bool paired, int B, int Hq, int Hk, int num_kv_splits, int max_blocks_per_seq,
                       int block_size, int D) {
  DecodePlan p{};
  p.D = D;
  p.B = B;
  p.Hq = Hq;
  p.Hk = Hk;
  p.QG = Hq / Hk;
  p.splits = num_kv_splits;
  // Splits are sized from the table capacity, not from each sequence's
  // length: every split then holds the same number of tiles, a short
  // sequence simply has fewer non-empty ones, and waves carry equal work
  // whatever the length mix.
  const long max_tiles = ((long)max_blocks_per_seq * block_size + kTile - 1) / kTile;
  p.cs = (int)((max_tiles + num_kv_splits - 1) / num_kv_splits);
  // Partition policy: a wave has a fixed cost (its query, its partial write,
  // the ring fill), so it should stream as many tiles as the machine can
  // afford while the grid still offers about target_waves(D) waves when every
  // sequence is full. A partial is then a union of spw consecutive splits, or
  // one of nsub pieces of a split that is too long for one wave.
  // With paired query rows (multi-query rows of one sequence sharing a
  // wave) about half the rows' waves stream, so the budget counts pairs.
  const long rows_eff = paired ? ((long)B + 1) / 2 : (long)B;
  long budget = rows_eff * Hk * max_tiles / target_waves(D);
  budget = budget < kTilesPerWaveMin ? kTilesPerWaveMin
                                     : (budget > UQ_TILES_PER_WAVE_MAX ? UQ_TILES_PER_WAVE_MAX : budget);
  int spw = 1, nsub = 1;
  while (2 * spw <= num_kv_splits && 2L * spw * p.cs <= budget) spw *= 2;
  while (nsub < 8 && p.cs > 2L * nsub * budget) nsub *= 2;
  p.spw = spw;
  p.nsub = nsub;
  p.parts = ((num_kv_splits + spw - 1) / spw) * nsub;
  const size_t rows = (size_t)B * Hq;
  size_t off = 0;
  p.q8_off = off;
  off = align256(off + rows * D);
  p.o_off = off;
  off = align256(off + rows * p.parts * D * sizeof(uint16_t));
  p.m_off = off;
  off = align256(off + rows * p.parts * sizeof(float));
  p.l_off = off;
  off = align256(off + rows * p.parts * sizeof(float));
  p.e_off = off;
  off = align256(off + rows * p.parts * sizeof(int));
  p.total = off;
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, int stage_mask,
                         hipStream_t stream) {
  uint8_t* q8 = a.workspace + p.q8_off;
  uint16_t* part_o = reinterpret_cast<uint16_t*>(a.workspace + p.o_off);
  float* part_m = reinterpret_cast<float*>(a.workspace + p.m_off);
  float* part_l = reinterpret_cast<float*>(a.workspace + p.l_off);
  int* part_e = reinterpret_cast<int*>(a.workspace + p.e_off);
  const int64_t vecs = (int64_t)p.B * p.Hq;

  if (p.D != 128 && p.D != 256 && p.D != 512) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if (stage_mask & 1) {
    // lanes per row: 16 from 4096 rows on (the mixed serving step's 8192
    // rows: 6.00 -> 5.25 us), else 64 (3072 rows: 3.32 us against 3.63 with
    // 16; 1024 rows: 2.35 us)
    const int lpr = vecs <= 4096 ? 64 : 16;
    const int64_t per_block = 4 * (64 / lpr);
    const dim3 g((unsigned)((vecs + per_block - 1) / per_block));
#define UQ_QPRO(DV)                                                                                     \
    do {                                                                                                \
      if (lpr == 64)                                                                                    \
        hipLaunchKernelGGL((qprologue_kernel<DV, 64>), g, dim3(256), 0, stream, a.query, q8, p.B, p.Hq, \
                           a.qsb, a.qsh);                                                               \
      else                                                                                              \
        hipLaunchKernelGGL((qprologue_kernel<DV, 16>), g, dim3(256), 0, stream, a.query, q8, p.B, p.Hq, \
                           a.qsb, a.qsh);                                                               \
    } while (0)
    if (p.D == 128) UQ_QPRO(128);
    else if (p.D == 256) UQ_QPRO(256);
    else UQ_QPRO(512);
#undef UQ_QPRO
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // KV heads per workgroup (one wave each). Reading several heads of a token
  // row on one CU shares the cache lines their slots straddle.
  const int hpw = heads_per_workgroup(p.Hk);
  const int hgroups = p.Hk / hpw;
  int log2_bs = 0;
  while ((1 << log2_bs) < a.block_size) ++log2_bs;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  // With a sliding window the splits cut the tiles a window can touch (its
  // first token may sit mid-tile), not the whole table: the same partition
  // shape, so the same partial count and workspace, over fewer tiles.
  int cs = p.cs;
  if (a.window > 0) {
    const long max_tiles = ((long)a.max_blocks_per_seq * a.block_size + kTile - 1) / kTile;
    const long wt = ((long)a.window + kTile - 1) / kTile + 1;
    const long cmax = wt < max_tiles ? wt : max_tiles;
    cs = (int)((cmax + p.splits - 1) / p.splits);
  }
  const int64_t n_wg = (int64_t)p.B * p.parts * hgroups;
  const dim3 grid1((unsigned)n_wg);
  const dim3 block1(64 * hpw);
  // Stage 1 reads the query codes from the workspace, or (the two-launch
  // form, head dim 256) computes them itself.
  const bool fuse_q = p.D == 256 && (stage_mask & 8);
  // Multi-query rows of one sequence share reads in pairs (see stage1_kernel)
  // when the group leaves half the MFMA columns free and no window moves the
  // rows' ranges apart.
  const bool pair_rows = a.query_row != nullptr && a.window == 0 && p.QG <= 8 && !fuse_q;
  // At head dim 256 a grid of two waves per SIMD or more (counting only the
  // waves that stream: with paired rows half the grid exits at once) streams
  // through a two-slot ring (one tile in flight while one is computed):
  // mixed 246.7 against 251.6 us, ragged 252.8 against 260.8, long (2048
  // waves) 208 against 216 us for stage 1, with three slots; a grid of one
  // wave per SIMD keeps three (decode 36.0 against 39.9 us with two; two
  // query rows per sequence 40.7 against 44.0).
  const int64_t streaming_waves = pair_rows ? n_wg * hpw / 2 : n_wg * hpw;
  const bool two_slots = p.D == 256 && streaming_waves >= 2 * 1024;
#define UQ_STAGE1S(DV, QGV, HPWV, NS, MD)                                                         \
  hipLaunchKernelGGL((stage1_kernel<DV, QGV, HPWV, NS, MD>), grid1, block1, 0, stream, q8, a.query,  \
                     a.qsb, a.qsh, a.cache, a.block_table, a.query_row, a.n_rows, a.seq_lens,     \
                     scale_log2, p.Hq, p.Hk, hgroups,                                             \
                     cs, p.spw, p.nsub, p.parts, log2_bs, a.max_blocks_per_seq,                   \
                     a.num_blocks, a.window, p.B, part_o, part_m, part_l, part_e)
#define UQ_STAGE1F(DV, QGV, HPWV, NS)                                 \
  do {                                                                \
    if constexpr (QGV <= 8) {                                         \
      if (pair_rows) { UQ_STAGE1S(DV, QGV, HPWV, NS, 2); break; }     \
    }                                                                 \
    if constexpr (DV == 256) {                                        \
      if (fuse_q) UQ_STAGE1S(DV, QGV, HPWV, NS, 1);                   \
      else UQ_STAGE1S(DV, QGV, HPWV, NS, 0);                          \
    } else {                                                          \
      UQ_STAGE1S(DV, QGV, HPWV, NS, 0);                               \
    }                                                                 \
  } while (0)
#define UQ_STAGE1(DV, QGV, HPWV)                                      \
  do {                                                                \
    if (DV == 256 && two_slots) UQ_STAGE1F(DV, QGV, HPWV, 2);         \
    else UQ_STAGE1F(DV, QGV, HPWV, ring_slots<DV>(HPWV));             \
  } while (0)
#define UQ_STAGE1_HPW(DV, QGV)                  \
  do {                                          \
    switch (hpw) {                              \
      case 1: UQ_STAGE1(DV, QGV, 1); break;     \
      case 2: UQ_STAGE1(DV, QGV, 2); break;     \
      default: UQ_STAGE1(DV, QGV, 4); break;    \
    }                                           \
  } while (0)
#define UQ_STAGE1_QG(DV)                        \
  do {                                          \
    switch (p.QG) {                             \
      case 6: UQ_STAGE1_HPW(DV, 6); break;      \
      case 8: UQ_STAGE1_HPW(DV, 8); break;      \
      default: UQ_STAGE1_HPW(DV, 16); break;    \
    }                                           \
  } while (0)
  if (stage_mask & 2) {
    if (hpw != 1 && hpw != 2 && hpw != 4) return hipErrorInvalidValue;
    if (p.QG != 6 && p.QG != 8 && p.QG != 16) return hipErrorInvalidValue;
    if (p.D == 128) UQ_STAGE1_QG(128);
    else if (p.D == 256) UQ_STAGE1_QG(256);
    else UQ_STAGE1_QG(512);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
#undef UQ_STAGE1_QG
#undef UQ_STAGE1_HPW
#undef UQ_STAGE1
#undef UQ_STAGE1F
#undef UQ_STAGE1S
  if (stage_mask & 4) {
    // waves per row: one up to 16 partials, then two, then four
    const int gw = p.parts > 32 ? 4 : (p.parts > 16 ? 2 : 1);
    const dim3 g((unsigned)((vecs * gw + 3) / 4));
#define UQ_STAGE2(DV, GV) hipLaunchKernelGGL((stage2_kernel<DV, GV>), g, dim3(256), 0, stream, part_o, \
                                             part_m, part_l, part_e, a.sinks, p.Hq, a.out, (int)vecs, p.parts)
#define UQ_STAGE2_G(DV) do { if (gw == 1) UQ_STAGE2(DV, 1); else if (gw == 2) UQ_STAGE2(DV, 2); \
                             else UQ_STAGE2(DV, 4); } while (0)
    if (p.D == 128) UQ_STAGE2_G(128);
    else if (p.D == 256) UQ_STAGE2_G(256);
    else UQ_STAGE2_G(512);
#undef UQ_STAGE2_G
#undef UQ_STAGE2
    e = hipGetLastError();
  }
  return e;
}

}  // namespace uq
