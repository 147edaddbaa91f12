// Launch interfaces between the C-ABI layer (uq_api.hip) and the kernels.
#pragma once

#include "uq_device.h"

namespace uq {

struct StoreArgs {
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
  int B, Hq, Hk, QG;
  int splits;          // num_kv_splits
  int cs;              // tiles per split: ceil(ceil(max_blocks * block_size / 16) / splits)
  int spw;             // consecutive splits covered by one partial (nsub == 1)
  int nsub;            // pieces one split is cut into (spw == 1)
  int parts;           // partials per (sequence, query head): ceil(splits / spw) * nsub
  size_t q8_off, o_off, m_off, l_off, total;   // byte offsets inside the workspace
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

DecodePlan plan_decode(int B, int Hq, int Hk, int num_kv_splits, int max_blocks_per_seq,
                       int block_size);

hipError_t launch_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_hadamard(int D, float* H, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, int stage_mask, hipStream_t stream);

}  // namespace uq
