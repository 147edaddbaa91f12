// Streaming-read probe: reads exactly the cache bytes a decode of the given
// sequences reads (every physical block a sequence's tokens live in, all KV
// heads, up to its last token), in block-table order, and nothing else. It
// does no arithmetic beyond an XOR of what it loads, so its rate is the
// ceiling a decode that streams the same blocks could reach on this GPU.
// The result words only keep the loads alive.
#include "uq_internal.h"

namespace uq {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte loads per lane in flight per round: 17 KB per wave, one round per
// physical block of the head-dim-256, four-KV-head, 16-token layout (17,408
// bytes); measured the fastest plain read of that layout (25.4 us for the
// 142.6 MB of 8192 shuffled blocks, against 27.7 with rounds of 16 loads)
constexpr int kProbeLoads = 17;

// One wave per range of (sequence, logical block) items of the (B, max_blocks)
// grid; an item past its sequence's last block is skipped. An item's bytes
// (tokens of the block up to the sequence's end, times Hk slots) are
// contiguous and read through one buffer descriptor that ends there, so the
// rounds' trailing loads past it return zeros without touching memory.
__global__ __launch_bounds__(256) void stream_blocks_kernel(
    const uint8_t* __restrict__ cache, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int B, int max_blocks, int log2_bs, int64_t num_blocks,
    uint32_t token_bytes, int items_per_wave, uint32_t* __restrict__ sink, int sink_words) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int64_t n_items = (int64_t)B * max_blocks;
  const int64_t i0 = (int64_t)wave * items_per_wave;
  const int64_t i1 = min(i0 + items_per_wave, n_items);
  const int bs = 1 << log2_bs;
  uint32_t x = 0;
  for (int64_t it = i0; it < i1; ++it) {
    const int b = (int)(it / max_blocks);
    const int j = (int)(it - (int64_t)b * max_blocks);
    int L = seq_lens[b];
    L = L < 0 ? 0 : min(L, max_blocks << log2_bs);
    const int ntok = min(bs, L - (j << log2_bs));
    if (ntok <= 0) continue;
    const int phys = block_table[it];
    if (phys < 0 || (int64_t)phys >= num_blocks) continue;
    const uint32_t bytes = (uint32_t)ntok * token_bytes;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cache + ((size_t)phys << log2_bs) * token_bytes), (short)0, (int)bytes, 0x00020000);
    for (uint32_t r = 0; r < bytes; r += 1024u * kProbeLoads) {
      uint4 v[kProbeLoads];
#pragma unroll
      for (int k = 0; k < kProbeLoads; ++k)
        v[k] = r + 1024u * k < bytes   // wave-uniform: no load issued past the item
                   ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rs, r + 1024u * k + 16u * lane, 0, 0))
                   : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int k = 0; k < kProbeLoads; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
  }
  sink[(wave * 64 + lane) % sink_words] = x;
}

}  // namespace

hipError_t launch_stream_blocks(const StreamArgs& a, hipStream_t stream) {
  int log2_bs = 0;
  while ((1 << log2_bs) < a.block_size) ++log2_bs;
  const int64_t n_items = (int64_t)a.B * a.max_blocks;
  // about 2048 waves (two per SIMD), each over an equal share of the items
  const int64_t per = (n_items + 2047) / 2048;
  const int64_t waves = (n_items + per - 1) / per;
  const dim3 grid((unsigned)((waves + 3) / 4));
  hipLaunchKernelGGL(stream_blocks_kernel, grid, dim3(256), 0, stream, a.cache, a.block_table,
                     a.seq_lens, a.B, a.max_blocks, log2_bs, a.num_blocks,
                     (uint32_t)a.Hk * (uint32_t)a.slot_bytes, (int)per, a.sink, a.sink_words);
  return hipGetLastError();
}

}  // namespace uq
