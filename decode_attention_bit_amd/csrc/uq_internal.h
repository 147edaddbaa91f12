// Launch interfaces between the C-ABI layer (uq_api.hip) and the kernels.
#pragma once

#include "uq_device.h"

namespace uq {

struct StoreArgs {
  int D;                      // head dim: 128, 256 or 512
  const uint16_t* key;
  const uint16_t* value;
  uint8_t* cache;
  const int64_t* slot_mapping;
  int64_t N;
  int Hk;
  int64_t num_blocks;
  int block_size;
  int64_t ksn, ksh, vsn, vsh;
};

// Partial results of split-KV stage 1, carved out of the caller's workspace.
struct DecodePlan {
  int D;               // head dim: 128, 256 or 512
  int B, Hq, Hk, QG;
  int splits;          // num_kv_splits
  int cs;              // tiles per split: ceil(ceil(max_blocks * block_size / 16) / splits)
  int spw;             // consecutive splits covered by one partial (nsub == 1)
  int nsub;            // pieces one split is cut into (spw == 1)
  int parts;           // partials per (sequence, query head): ceil(splits / spw) * nsub
  size_t q8_off, o_off, m_off, l_off, e_off, total;   // byte offsets inside the workspace
};

struct DecodeArgs {
  const uint16_t* query;
  const uint8_t* cache;
  const int32_t* block_table;
  const int32_t* query_row;   // (B,) block-table row of each query, or null: row b
  int n_rows;                 // rows in block_table
  const int32_t* seq_lens;
  const float* sinks;         // (Hq,) sink logits, or null
  int window;                 // sliding window in tokens, 0: none
  float scale;
  uint16_t* out;
  int64_t num_blocks;
  int block_size;
  int max_blocks_per_seq;
  int64_t qsb, qsh;
  uint8_t* workspace;
};

// Continuation prefill operands. A job maps n = N * H vectors of D bf16
// (vector w -> row t = w / H, head h = w % H) from src to dst, rotated
// (dst = bf16(src H)) or copied.
struct VecJob {
  const uint16_t* src;
  int64_t ss_t, ss_h;
  uint16_t* dst;
  int64_t ds_t, ds_h;
  int64_t n;
  int H;
  int rotate;
};

// Tiled value layout of the continuation prefill (vt != null): per KV head,
// tiles of 32 keys, each D dim rows of 64 bytes; row d of tile j holds the
// 32 keys in the order the attention's P operand uses, its 16-byte chunks
// permuted by chunk ^ (((d >> 2) ^ (d >> 1)) & 3).
struct GatherArgs {
  int D;                     // head dim: 128, 256 or 512
  // dequantise tokens 0 .. n_tok-1 of a sequence (block_row[t / block_size])
  const uint8_t* cache;
  const int32_t* block_row;
  int n_tok;
  int Hk;
  int64_t num_blocks;
  int log2_bs;
  uint16_t* kout;
  uint16_t* vout;
  int64_t os_t, os_h;
  // Tiled values (vt != null): one workgroup per (KV head, 32-key tile)
  // builds the whole tile: keys below n_tok dequantised from the cache
  // (their V is then not written to vout), keys n_tok .. v_keys - 1 copied
  // from vsrc row key - n_tok, the rest of the last tile zero. The tiles hold
  // fp16 values times 2^-vshift[h][d / 32]: a first kernel writes, per
  // (KV head, part of the keys), the largest exponent of each 32-dim block
  // (vexp_part, Hk x kVexpParts x D / 32), and the tile workgroups take the
  // shift from it (the ones of tile 0 also store it in vshift, Hk x D / 32).
  uint16_t* vt;
  int64_t vt_tiles;          // tiles per KV head
  const uint16_t* vsrc;
  int64_t vs_t, vs_h;
  int64_t v_keys;
  int32_t* vexp_part;
  int32_t* vshift;
  VecJob job[3];
};

// Parts of the keys the value-exponent kernel splits each KV head into.
constexpr int kVexpParts = 256;

struct PrefillAttnArgs {
  const uint16_t* q;         // (q_len, Hq, D) rotated queries, bf16
  const uint16_t* k;         // (cached_len + q_len, Hk, D) rotated keys, bf16
  const uint16_t* v;         // same shape, values
  uint16_t* out;             // (q_len, Hq, D)
  int64_t qs_t, qs_h, kvs_t, kvs_h, os_t, os_h;
  int q_len, cached_len, Hk, QG;
  float scale;
  int64_t vt_tiles;          // > 0: v is in the tiled value layout with this many tiles per head
  int D;                     // head dim: 128, 256 or 512
  const int32_t* vshift;     // vt_tiles > 0: the tiles hold v * 2^-vshift[h][d / 32] in fp16
};

// Streaming-read probe over the blocks a decode reads.
struct StreamArgs {
  const uint8_t* cache;
  const int32_t* block_table;   // (B, max_blocks)
  const int32_t* seq_lens;      // (B,)
  int B, max_blocks, block_size, Hk, slot_bytes;
  int64_t num_blocks;
  uint32_t* sink;               // sink_words words, overwritten
  int sink_words;
};

DecodePlan plan_decode(bool paired, int B, int Hq, int Hk, int num_kv_splits, int max_blocks_per_seq,
                       int block_size, int D);

hipError_t launch_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_hadamard(int D, float* H, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);
hipError_t launch_prefill_attn(const PrefillAttnArgs& a, hipStream_t stream);
int prefill_positions_per_wg(int QG, int D);
hipError_t launch_stream_blocks(const StreamArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, int stage_mask, hipStream_t stream);

}  // namespace uq
