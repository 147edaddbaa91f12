// C ABI of libuq: host-side argument checks, then kernel launches. Every
// check runs before the first HIP call, so a rejected call touches no device
// state and can be exercised without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/uq.h"
#include "uq_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return UQ_OK;
}

bool pow2_in(long v, long lo, long hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(UQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int uq_build_hadamard(int D, float* H, void* stream) {
  if (!H) return fail(UQ_EINVAL, "uq_build_hadamard: H is null");
  if (!pow2_in(D, 1, 512)) return fail(UQ_EINVAL, "uq_build_hadamard: D=%d is not a power of two in [1, 512]", D);
  return hip_status(uq::launch_hadamard(D, H, (hipStream_t)stream), "uq_build_hadamard launch");
}

int uq_store(const uint16_t* key, const uint16_t* value, uint8_t* kv_cache,
             const int64_t* slot_mapping, int64_t N, int Hk, int D, int64_t num_blocks,
             int block_size, int slot_size, int64_t key_stride_n, int64_t key_stride_h,
             int64_t val_stride_n, int64_t val_stride_h, void* stream) {
  if (N < 0) return fail(UQ_EINVAL, "uq_store: N=%lld < 0", (long long)N);
  if (Hk < 1) return fail(UQ_EINVAL, "uq_store: Hk=%d < 1", Hk);
  if (num_blocks < 1) return fail(UQ_EINVAL, "uq_store: num_blocks=%lld < 1", (long long)num_blocks);
  if (D != 128 && D != 256 && D != 512)
    return fail(UQ_EUNSUPPORTED, "uq_store: head_dim %d unsupported (128, 256, 512)", D);
  if (slot_size != D * 17 / 16)
    return fail(UQ_EUNSUPPORTED, "uq_store: slot_size %d unsupported (17 * head_dim / 16 = %d)", slot_size, D * 17 / 16);
  if (!pow2_in(block_size, 16, 256))
    return fail(UQ_EUNSUPPORTED, "uq_store: block_size %d unsupported (16, 32, 64, 128, 256)", block_size);
  if (N == 0) return ok();
  if (!key || !value || !kv_cache || !slot_mapping) return fail(UQ_EINVAL, "uq_store: null pointer argument");
  if (key_stride_n < 0 || key_stride_h < 0 || val_stride_n < 0 || val_stride_h < 0 ||
      key_stride_n % 4 || key_stride_h % 4 || val_stride_n % 4 || val_stride_h % 4)
    return fail(UQ_EINVAL, "uq_store: strides must be non-negative multiples of 4 elements");
  if (!aligned(key, 8) || !aligned(value, 8) || !aligned(kv_cache, 16) || !aligned(slot_mapping, 8))
    return fail(UQ_EINVAL, "uq_store: misaligned pointer (key/value 8 B, kv_cache 16 B, slot_mapping 8 B)");
  if ((N * Hk + 3) / 4 > 0x7FFFFFFFLL) return fail(UQ_EUNSUPPORTED, "uq_store: N*Hk too large for one launch");
  uq::StoreArgs a{D, key, value, kv_cache, slot_mapping, N, Hk, num_blocks, block_size,
                  key_stride_n, key_stride_h, val_stride_n, val_stride_h};
  return hip_status(uq::launch_store(a, (hipStream_t)stream), "uq_store launch");
}

size_t uq_decode_workspace_bytes(int B, int Hq, int Hk, int D, int num_kv_splits,
                                 int max_blocks_per_seq, int block_size) {
  if (B < 1 || Hk < 1 || Hq < Hk || Hq % Hk || (D != 128 && D != 256 && D != 512) || num_kv_splits < 1 ||
      num_kv_splits > UQ_MAX_SPLITS || max_blocks_per_seq < 1 || !pow2_in(block_size, 16, 256) ||
      (long long)max_blocks_per_seq * block_size > 0x7FFFFFFFLL)
    return 0;
  // enough for either plan: multi-query rows that may pair cut finer partials
  const size_t t0 = uq::plan_decode(false, B, Hq, Hk, num_kv_splits, max_blocks_per_seq, block_size, D).total;
  const size_t t1 =
      Hq / Hk <= 8 ? uq::plan_decode(true, B, Hq, Hk, num_kv_splits, max_blocks_per_seq, block_size, D).total : 0;
  return t0 > t1 ? t0 : t1;
}

// Device scratch of uq_decode_no_alloc: the decode's workspace (query codes,
// partial rows and their statistics) for callers that cannot allocate. One
// copy per device, held from the library's load on that device until the
// process ends. Host code never uses the array's name as an address: each
// device's copy is at the address hipGetSymbolAddress gives with that device
// current, taken once per device and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[UQ_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The scratch address on the device of `stream` (which must be the current
// device: the symbol's address is per device).
int scratch_address(void* stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(UQ_EHIP, "uq_decode_no_alloc: hipGetDevice: %s", hipGetErrorString(e));
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice((hipStream_t)stream, &dev);
    if (e != hipSuccess) return fail(UQ_EHIP, "uq_decode_no_alloc: hipStreamGetDevice: %s", hipGetErrorString(e));
  }
  if (dev != cur)
    return fail(UQ_EINVAL, "uq_decode_no_alloc: the stream belongs to device %d, not the current device %d", dev, cur);
  if (dev < 0 || dev >= kMaxDevices) return fail(UQ_EUNSUPPORTED, "uq_decode_no_alloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(UQ_EHIP, "uq_decode_no_alloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ok();
}

}  // namespace

// use_scratch: the workspace is the device scratch (uq_decode_no_alloc);
// workspace and workspace_bytes are then ignored.
static int decode_impl(int stage_mask, const uint16_t* query, const uint8_t* kv_cache,
                       const int32_t* block_table, int n_table_rows, const int32_t* query_row,
                       const int32_t* seq_lens, float scale, int num_kv_splits,
                       const float* sinks, int sliding_window, uint16_t* out,
                       int B, int Hq, int Hk, int D, int64_t num_blocks, int block_size,
                       int max_blocks_per_seq, int64_t q_stride_b, int64_t q_stride_h,
                       void* workspace, size_t workspace_bytes, void* stream,
                       bool use_scratch = false) {
  if (stage_mask <= 0 || (stage_mask & ~15) || stage_mask == UQ_STAGE_FUSED_QUERY)
    return fail(UQ_EINVAL, "uq_decode: stage_mask %d is not a non-empty subset of 1|2|4 (| 8)", stage_mask);
  if ((stage_mask & UQ_STAGE_FUSED_QUERY) && !(stage_mask & UQ_STAGE_SPLIT))
    return fail(UQ_EINVAL, "uq_decode: UQ_STAGE_FUSED_QUERY needs UQ_STAGE_SPLIT");
  if (B < 1 || Hq < 1 || Hk < 1) return fail(UQ_EINVAL, "uq_decode: B=%d Hq=%d Hk=%d must be >= 1", B, Hq, Hk);
  if (num_blocks < 1 || max_blocks_per_seq < 1 || n_table_rows < 1)
    return fail(UQ_EINVAL, "uq_decode: num_blocks, max_blocks_per_seq and the table rows must be >= 1");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(UQ_EINVAL, "uq_decode: scale must be finite and > 0");
  if (sliding_window < 0) return fail(UQ_EINVAL, "uq_decode: sliding_window %d < 0", sliding_window);
  if (D != 128 && D != 256 && D != 512)
    return fail(UQ_EUNSUPPORTED, "uq_decode: head_dim %d unsupported (128, 256, 512)", D);
  if ((stage_mask & UQ_STAGE_FUSED_QUERY) && D != 256)
    return fail(UQ_EUNSUPPORTED, "uq_decode: the query prologue inside stage 1 is built for head dim 256, not %d", D);
  if (Hq % Hk) return fail(UQ_EUNSUPPORTED, "uq_decode: Hq=%d is not a multiple of Hk=%d", Hq, Hk);
  const int qg = Hq / Hk;
  if (qg != 6 && qg != 8 && qg != 16)
    return fail(UQ_EUNSUPPORTED, "uq_decode: GQA group %d unsupported (6, 8, 16)", qg);
  if (!pow2_in(block_size, 16, 256))
    return fail(UQ_EUNSUPPORTED, "uq_decode: block_size %d unsupported (16, 32, 64, 128, 256)", block_size);
  if (num_kv_splits < 1 || num_kv_splits > UQ_MAX_SPLITS)
    return fail(UQ_EUNSUPPORTED, "uq_decode: num_kv_splits %d outside [1, %d]", num_kv_splits, UQ_MAX_SPLITS);
  if ((long long)max_blocks_per_seq * block_size > 0x7FFFFFFFLL)
    return fail(UQ_EUNSUPPORTED, "uq_decode: max_blocks_per_seq * block_size exceeds 2^31");
  if (!query || !kv_cache || !block_table || !seq_lens || !out || (!workspace && !use_scratch))
    return fail(UQ_EINVAL, "uq_decode: null pointer argument");
  if (q_stride_b < 0 || q_stride_h < 0 || q_stride_b % 4 || q_stride_h % 4)
    return fail(UQ_EINVAL, "uq_decode: query strides must be non-negative multiples of 4 elements");
  if (!aligned(query, 8) || !aligned(kv_cache, 16) || !aligned(out, 16) || (!use_scratch && !aligned(workspace, 256)) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(query_row, 4) ||
      !aligned(sinks, 4))
    return fail(UQ_EINVAL, "uq_decode: misaligned pointer (query 8 B, kv_cache/out 16 B, workspace 256 B)");
  // query rows of one sequence may share stage-1 waves in pairs (QG <= 8, no
  // window); the plan then counts pairs
  const bool paired = query_row != nullptr && sliding_window == 0 && qg <= 8;
  const uq::DecodePlan plan =
      uq::plan_decode(paired, B, Hq, Hk, num_kv_splits, max_blocks_per_seq, block_size, D);
  if (use_scratch && plan.total > (size_t)UQ_NO_ALLOC_SCRATCH_BYTES)
    return fail(UQ_EWORKSPACE, "uq_decode_no_alloc: this shape needs %zu bytes of scratch, above the %zu-byte "
                "static buffer; use uq_decode with a workspace", plan.total, (size_t)UQ_NO_ALLOC_SCRATCH_BYTES);
  if (!use_scratch && workspace_bytes < plan.total)
    return fail(UQ_EWORKSPACE, "uq_decode: workspace %zu bytes < required %zu", workspace_bytes, plan.total);
  if ((long long)B * plan.parts * Hk > 0x7FFFFFFFLL || (long long)B * Hq > 0x7FFFFFFFLL)
    return fail(UQ_EUNSUPPORTED, "uq_decode: grid too large");
  if (use_scratch) {                       // every argument checked: now the first HIP call
    const int rc = scratch_address(stream, &workspace);
    if (rc != UQ_OK) return rc;
  }
  uq::DecodeArgs a{query, kv_cache, block_table, query_row, n_table_rows, seq_lens, sinks,
                   sliding_window, scale, out,
                   num_blocks, block_size,
                   max_blocks_per_seq, q_stride_b, q_stride_h,
                   reinterpret_cast<uint8_t*>(workspace)};
  return hip_status(uq::launch_decode(a, plan, stage_mask, (hipStream_t)stream),
                    "uq_decode launch");
}

int uq_decode_stages(int stage_mask, const uint16_t* query, const uint8_t* kv_cache,
                     const int32_t* block_table, const int32_t* seq_lens, float scale,
                     int num_kv_splits, uint16_t* out, int B, int Hq, int Hk, int D,
                     int64_t num_blocks, int block_size, int max_blocks_per_seq,
                     int64_t q_stride_b, int64_t q_stride_h, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return decode_impl(stage_mask, query, kv_cache, block_table, B, nullptr, seq_lens, scale,
                     num_kv_splits, nullptr, 0, out, B, Hq, Hk, D, num_blocks, block_size,
                     max_blocks_per_seq, q_stride_b, q_stride_h, workspace, workspace_bytes,
                     stream);
}

int uq_decode_partials(int B, int Hq, int Hk, int D, int num_kv_splits, int max_blocks_per_seq,
                       int block_size) {
  if (uq_decode_workspace_bytes(B, Hq, Hk, D, num_kv_splits, max_blocks_per_seq, block_size) == 0) return 0;
  return uq::plan_decode(false, B, Hq, Hk, num_kv_splits, max_blocks_per_seq, block_size, D).parts;
}

int uq_stream_blocks(const uint8_t* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                     int B, int Hk, int D, int64_t num_blocks, int block_size, int max_blocks_per_seq,
                     uint32_t* sink, int sink_words, void* stream) {
  if (B < 1 || Hk < 1 || num_blocks < 1 || max_blocks_per_seq < 1 || sink_words < 1)
    return fail(UQ_EINVAL, "uq_stream_blocks: B=%d Hk=%d num_blocks=%lld max_blocks=%d sink_words=%d", B, Hk,
                (long long)num_blocks, max_blocks_per_seq, sink_words);
  if (D != 128 && D != 256 && D != 512)
    return fail(UQ_EUNSUPPORTED, "uq_stream_blocks: head_dim %d unsupported (128, 256, 512)", D);
  if (!pow2_in(block_size, 16, 256))
    return fail(UQ_EUNSUPPORTED, "uq_stream_blocks: block_size %d unsupported (16, 32, 64, 128, 256)", block_size);
  if ((long long)block_size * Hk * (D * 17 / 16) > 0x7FFFFFFFLL || (long long)B * max_blocks_per_seq > 0x7FFFFFFFLL)
    return fail(UQ_EUNSUPPORTED, "uq_stream_blocks: shape too large");
  if (!kv_cache || !block_table || !seq_lens || !sink) return fail(UQ_EINVAL, "uq_stream_blocks: null pointer argument");
  if (!aligned(kv_cache, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(sink, 4))
    return fail(UQ_EINVAL, "uq_stream_blocks: misaligned pointer (kv_cache 16 B)");
  uq::StreamArgs a{kv_cache, block_table, seq_lens, B, max_blocks_per_seq, block_size, Hk, D * 17 / 16,
                   num_blocks, sink, sink_words};
  return hip_status(uq::launch_stream_blocks(a, (hipStream_t)stream), "uq_stream_blocks launch");
}

int uq_decode_ex(const uint16_t* query, const uint8_t* kv_cache, const int32_t* block_table,
                 int n_table_rows, const int32_t* query_row, const int32_t* seq_lens, float scale,
                 int num_kv_splits, const float* sinks, int sliding_window, uint16_t* out, int B,
                 int Hq, int Hk, int D, int64_t num_blocks, int block_size,
                 int max_blocks_per_seq, int64_t q_stride_b, int64_t q_stride_h, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (!query_row && n_table_rows != B)
    return fail(UQ_EINVAL, "uq_decode_ex: without query_row the table needs B=%d rows, not %d", B,
                n_table_rows);
  return decode_impl(UQ_STAGE_PROLOGUE | UQ_STAGE_SPLIT | UQ_STAGE_MERGE, query, kv_cache,
                     block_table, n_table_rows, query_row, seq_lens, scale, num_kv_splits, sinks,
                     sliding_window, out, B, Hq, Hk, D, num_blocks, block_size,
                     max_blocks_per_seq, q_stride_b, q_stride_h, workspace, workspace_bytes,
                     stream);
}

int uq_decode(const uint16_t* query, const uint8_t* kv_cache, const int32_t* block_table,
              const int32_t* seq_lens, float scale, int num_kv_splits, uint16_t* out, int B,
              int Hq, int Hk, int D, int64_t num_blocks, int block_size, int max_blocks_per_seq,
              int64_t q_stride_b, int64_t q_stride_h, void* workspace, size_t workspace_bytes,
              void* stream) {
  return uq_decode_stages(UQ_STAGE_PROLOGUE | UQ_STAGE_SPLIT | UQ_STAGE_MERGE, query, kv_cache,
                          block_table, seq_lens, scale, num_kv_splits, out, B, Hq, Hk, D,
                          num_blocks, block_size, max_blocks_per_seq, q_stride_b, q_stride_h,
                          workspace, workspace_bytes, stream);
}

int uq_decode_no_alloc(const uint16_t* query, const uint8_t* kv_cache, const int32_t* block_table,
                       const int32_t* seq_lens, float scale, int num_kv_splits, uint16_t* out, int B,
                       int Hq, int Hk, int D, int64_t num_blocks, int block_size, int max_blocks_per_seq,
                       int64_t q_stride_b, int64_t q_stride_h, void* stream) {
  return decode_impl(UQ_STAGE_PROLOGUE | UQ_STAGE_SPLIT | UQ_STAGE_MERGE, query, kv_cache, block_table, B,
                     nullptr, seq_lens, scale, num_kv_splits, nullptr, 0, out, B, Hq, Hk, D, num_blocks,
                     block_size, max_blocks_per_seq, q_stride_b, q_stride_h, nullptr, 0, stream, true);
}

int uq_rotate(const uint16_t* x, uint16_t* out, int64_t N, int H, int D, int64_t x_stride_n,
              int64_t x_stride_h, int64_t out_stride_n, int64_t out_stride_h, void* stream) {
  if (N < 0 || H < 1) return fail(UQ_EINVAL, "uq_rotate: N=%lld H=%d", (long long)N, H);
  if (D != 128 && D != 256 && D != 512)
    return fail(UQ_EUNSUPPORTED, "uq_rotate: head_dim %d unsupported (128, 256, 512)", D);
  if (N == 0) return ok();
  if (!x || !out) return fail(UQ_EINVAL, "uq_rotate: null pointer argument");
  if (x_stride_n < 0 || x_stride_h < 0 || out_stride_n < 0 || out_stride_h < 0 || x_stride_n % 4 ||
      x_stride_h % 4 || out_stride_n % 4 || out_stride_h % 4)
    return fail(UQ_EINVAL, "uq_rotate: strides must be non-negative multiples of 4 elements");
  if (!aligned(x, 8) || !aligned(out, 8)) return fail(UQ_EINVAL, "uq_rotate: x and out must be 8-byte aligned");
  if ((N * H + 3) / 4 > 0x7FFFFFFFLL) return fail(UQ_EUNSUPPORTED, "uq_rotate: N*H too large for one launch");
  uq::GatherArgs a{};
  a.D = D;
  a.job[0] = uq::VecJob{x, x_stride_n, x_stride_h, out, out_stride_n, out_stride_h, N * H, H, 1};
  return hip_status(uq::launch_gather(a, (hipStream_t)stream), "uq_rotate launch");
}

int uq_dequant_kv(const uint8_t* kv_cache, const int32_t* block_row, int n_tokens, uint16_t* k_out,
                  uint16_t* v_out, int Hk, int D, int64_t num_blocks, int block_size,
                  int64_t out_stride_t, int64_t out_stride_h, void* stream) {
  if (n_tokens < 0 || Hk < 1 || num_blocks < 1)
    return fail(UQ_EINVAL, "uq_dequant_kv: n_tokens=%d Hk=%d num_blocks=%lld", n_tokens, Hk, (long long)num_blocks);
  if (D != 128 && D != 256 && D != 512)
    return fail(UQ_EUNSUPPORTED, "uq_dequant_kv: head_dim %d unsupported (128, 256, 512)", D);
  if (!pow2_in(block_size, 16, 256))
    return fail(UQ_EUNSUPPORTED, "uq_dequant_kv: block_size %d unsupported (16, 32, 64, 128, 256)", block_size);
  if (n_tokens == 0) return ok();
  if (!kv_cache || !block_row || !k_out || !v_out) return fail(UQ_EINVAL, "uq_dequant_kv: null pointer argument");
  if (out_stride_t < 0 || out_stride_h < 0 || out_stride_t % 8 || out_stride_h % 8)
    return fail(UQ_EINVAL, "uq_dequant_kv: output strides must be non-negative multiples of 8 elements");
  if (!aligned(kv_cache, 16) || !aligned(block_row, 4) || !aligned(k_out, 16) || !aligned(v_out, 16))
    return fail(UQ_EINVAL, "uq_dequant_kv: misaligned pointer (kv_cache, k_out, v_out 16 B; block_row 4 B)");
  if (((long long)n_tokens * Hk + 3) / 4 > 0x7FFFFFFFLL)
    return fail(UQ_EUNSUPPORTED, "uq_dequant_kv: n_tokens*Hk too large for one launch");
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  uq::GatherArgs a{};
  a.D = D;
  a.cache = kv_cache;
  a.block_row = block_row;
  a.n_tok = n_tokens;
  a.Hk = Hk;
  a.num_blocks = num_blocks;
  a.log2_bs = log2_bs;
  a.kout = k_out;
  a.vout = v_out;
  a.os_t = out_stride_t;
  a.os_h = out_stride_h;
  return hip_status(uq::launch_gather(a, (hipStream_t)stream), "uq_dequant_kv launch");
}

static int check_attention_shape(const char* who, int q_len, int seq_len, int Hq, int Hk, int D, float scale) {
  if (q_len < 0 || seq_len < q_len || Hq < 1 || Hk < 1)
    return fail(UQ_EINVAL, "%s: q_len=%d seq_len=%d Hq=%d Hk=%d", who, q_len, seq_len, Hq, Hk);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(UQ_EINVAL, "%s: scale must be finite and > 0", who);
  if (D != UQ_HEAD_DIM && D != UQ_HEAD_DIM / 2 && D != 2 * UQ_HEAD_DIM)
    return fail(UQ_EUNSUPPORTED, "%s: head_dim %d unsupported (128, 256, 512)", who, D);
  if (Hq % Hk) return fail(UQ_EUNSUPPORTED, "%s: Hq=%d is not a multiple of Hk=%d", who, Hq, Hk);
  if (uq::prefill_positions_per_wg(Hq / Hk, D) < 1)
    return fail(UQ_EUNSUPPORTED, "%s: GQA group %d above %d", who, Hq / Hk, D > UQ_HEAD_DIM ? 64 : 128);
  if (Hk > 65535) return fail(UQ_EUNSUPPORTED, "%s: Hk=%d above 65535", who, Hk);
  return ok();
}

int uq_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                         int q_len, int seq_len, int Hq, int Hk, int D, float scale,
                         int64_t q_stride_t, int64_t q_stride_h, int64_t kv_stride_t,
                         int64_t kv_stride_h, int64_t out_stride_t, int64_t out_stride_h,
                         void* stream) {
  const int rc = check_attention_shape("uq_prefill_attention", q_len, seq_len, Hq, Hk, D, scale);
  if (rc != UQ_OK) return rc;
  if (q_len == 0) return ok();
  if (!q || !k || !v || !out) return fail(UQ_EINVAL, "uq_prefill_attention: null pointer argument");
  if (q_stride_t < 0 || q_stride_h < 0 || kv_stride_t < 0 || kv_stride_h < 0 || out_stride_t < 0 ||
      out_stride_h < 0 || q_stride_t % 8 || q_stride_h % 8 || kv_stride_t % 8 || kv_stride_h % 8 ||
      out_stride_t % 8 || out_stride_h % 8)
    return fail(UQ_EINVAL, "uq_prefill_attention: strides must be non-negative multiples of 8 elements");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(UQ_EINVAL, "uq_prefill_attention: q, k, v and out must be 16-byte aligned");
  // key rows are staged 32 at a time through one buffer descriptor each
  if (kv_stride_t < D || kv_stride_t >= (1LL << 25))
    return fail(UQ_EUNSUPPORTED, "uq_prefill_attention: kv_stride_t %lld outside [D, 2^25)", (long long)kv_stride_t);
  uq::PrefillAttnArgs a{q, k, v, out, q_stride_t, q_stride_h, kv_stride_t, kv_stride_h,
                        out_stride_t, out_stride_h, q_len, seq_len - q_len, Hk, Hq / Hk, scale, 0, D, nullptr};
  return hip_status(uq::launch_prefill_attn(a, (hipStream_t)stream), "uq_prefill_attention launch");
}

// Workspace of uq_continuation_prefill: rotated queries, keys of prefix +
// chunk (token-major), the values in the tiled layout of the attention
// kernels (per KV head, ceil(seq_len / 32) tiles of 64 D bytes, fp16 scaled
// per 32-dim block), then the blocks' exponent parts and shifts (int32);
// each section 256-byte aligned.
struct PrefillLayout {
  size_t q_off, k_off, v_off, e_off, s_off, total;
  long long vt_tiles;
};

static PrefillLayout prefill_layout(long long q_len, long long seq_len, int Hq, int Hk, int D) {
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  PrefillLayout l{};
  l.vt_tiles = (seq_len + 31) / 32;
  l.q_off = 0;
  l.k_off = a256((size_t)q_len * Hq * D * 2);
  l.v_off = l.k_off + a256((size_t)seq_len * Hk * D * 2);
  l.e_off = l.v_off + a256((size_t)Hk * l.vt_tiles * 32 * D * 2);
  l.s_off = l.e_off + a256((size_t)Hk * uq::kVexpParts * (D / 32) * 4);
  l.total = l.s_off + (size_t)Hk * (D / 32) * 4;
  return l;
}

size_t uq_continuation_prefill_workspace_bytes(int q_len, int max_seq_len, int Hq, int Hk, int D) {
  if (q_len < 0 || max_seq_len < q_len || Hq < 1 || Hk < 1 || Hq % Hk ||
      (D != UQ_HEAD_DIM && D != UQ_HEAD_DIM / 2 && D != 2 * UQ_HEAD_DIM) ||
      uq::prefill_positions_per_wg(Hq / Hk, D) < 1)
    return 0;
  const size_t t = prefill_layout(q_len, max_seq_len, Hq, Hk, D).total;
  return t > 0 ? t : 256;
}

int uq_continuation_prefill_stages(int stage_mask, const uint16_t* query, const uint16_t* key,
                                   const uint16_t* value, const uint8_t* kv_cache,
                                   const int32_t* block_row, int cached_len, float scale,
                                   uint16_t* out, int q_len, int Hq, int Hk, int D,
                                   int64_t num_blocks, int block_size, int64_t q_stride_t,
                                   int64_t q_stride_h, int64_t key_stride_t, int64_t key_stride_h,
                                   int64_t val_stride_t, int64_t val_stride_h, int64_t out_stride_t,
                                   int64_t out_stride_h, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  const char* who = "uq_continuation_prefill";
  if (stage_mask <= 0 || (stage_mask & ~3))
    return fail(UQ_EINVAL, "%s: stage_mask %d is not a non-empty subset of 1|2", who, stage_mask);
  if (cached_len < 0 || (long long)cached_len + q_len > 0x7FFFFFFFLL)
    return fail(UQ_EINVAL, "%s: cached_len=%d", who, cached_len);
  const int seq_len = cached_len + q_len;
  int rc = check_attention_shape(who, q_len, seq_len, Hq, Hk, D, scale);
  if (rc != UQ_OK) return rc;
  if (num_blocks < 1) return fail(UQ_EINVAL, "%s: num_blocks=%lld < 1", who, (long long)num_blocks);
  if (!pow2_in(block_size, 16, 256))
    return fail(UQ_EUNSUPPORTED, "%s: block_size %d unsupported (16, 32, 64, 128, 256)", who, block_size);
  if (q_len == 0) return ok();
  if (!query || !key || !value || !kv_cache || !out || !workspace || (cached_len > 0 && !block_row))
    return fail(UQ_EINVAL, "%s: null pointer argument", who);
  if (q_stride_t < 0 || q_stride_h < 0 || key_stride_t < 0 || key_stride_h < 0 || val_stride_t < 0 ||
      val_stride_h < 0 || q_stride_t % 4 || q_stride_h % 4 || key_stride_t % 4 || key_stride_h % 4 ||
      val_stride_t % 4 || val_stride_h % 4)
    return fail(UQ_EINVAL, "%s: input strides must be non-negative multiples of 4 elements", who);
  if (out_stride_t < 0 || out_stride_h < 0 || out_stride_t % 8 || out_stride_h % 8)
    return fail(UQ_EINVAL, "%s: output strides must be non-negative multiples of 8 elements", who);
  if (!aligned(query, 8) || !aligned(key, 8) || !aligned(value, 8) || !aligned(kv_cache, 16) ||
      !aligned(block_row, 4) || !aligned(out, 16) || !aligned(workspace, 256))
    return fail(UQ_EINVAL, "%s: misaligned pointer (query/key/value 8 B, kv_cache/out 16 B, workspace 256 B)", who);
  const PrefillLayout lay = prefill_layout(q_len, seq_len, Hq, Hk, D);
  if (workspace_bytes < lay.total)
    return fail(UQ_EWORKSPACE, "%s: workspace %zu bytes < required %zu", who, workspace_bytes, lay.total);
  const long long waves = (long long)(seq_len + 32) * Hk * 3 + (long long)q_len * Hq;
  if ((waves + 3) / 4 > 0x7FFFFFFFLL) return fail(UQ_EUNSUPPORTED, "%s: too large for one launch", who);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  uint16_t* qr = reinterpret_cast<uint16_t*>(ws + lay.q_off);
  uint16_t* kf = reinterpret_cast<uint16_t*>(ws + lay.k_off);
  uint16_t* vf = reinterpret_cast<uint16_t*>(ws + lay.v_off);
  const int64_t row = (int64_t)Hk * D;                   // token stride of the key/value buffers
  int log2_bs = 0;
  while ((1 << log2_bs) < block_size) ++log2_bs;
  uq::GatherArgs g{};
  g.D = D;
  g.cache = kv_cache;
  g.block_row = block_row;
  g.n_tok = cached_len;
  g.Hk = Hk;
  g.num_blocks = num_blocks;
  g.log2_bs = log2_bs;
  g.kout = kf;
  g.vout = nullptr;                         // the value tiles hold V
  g.os_t = row;
  g.os_h = D;
  g.vt = vf;
  g.vt_tiles = lay.vt_tiles;
  g.vsrc = value;
  g.vs_t = val_stride_t;
  g.vs_h = val_stride_h;
  g.v_keys = seq_len;
  g.vexp_part = reinterpret_cast<int32_t*>(ws + lay.e_off);
  g.vshift = reinterpret_cast<int32_t*>(ws + lay.s_off);
  g.job[0] = uq::VecJob{query, q_stride_t, q_stride_h, qr, (int64_t)Hq * D, D,
                        (int64_t)q_len * Hq, Hq, 1};
  g.job[1] = uq::VecJob{key, key_stride_t, key_stride_h, kf + (int64_t)cached_len * row, row, D,
                        (int64_t)q_len * Hk, Hk, 1};
  if (stage_mask & UQ_PREFILL_GATHER) {
    hipError_t e = uq::launch_gather(g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "uq_continuation_prefill gather launch");
  }
  if (!(stage_mask & UQ_PREFILL_ATTEND)) return ok();
  uq::PrefillAttnArgs a{qr, kf, vf, out, (int64_t)Hq * D, D, row, D,
                        out_stride_t, out_stride_h, q_len, cached_len, Hk, Hq / Hk, scale, lay.vt_tiles, D,
                        g.vshift};
  return hip_status(uq::launch_prefill_attn(a, (hipStream_t)stream), "uq_continuation_prefill attention launch");
}

int uq_continuation_prefill(const uint16_t* query, const uint16_t* key, const uint16_t* value,
                            const uint8_t* kv_cache, const int32_t* block_row, int cached_len,
                            float scale, uint16_t* out, int q_len, int Hq, int Hk, int D,
                            int64_t num_blocks, int block_size, int64_t q_stride_t,
                            int64_t q_stride_h, int64_t key_stride_t, int64_t key_stride_h,
                            int64_t val_stride_t, int64_t val_stride_h, int64_t out_stride_t,
                            int64_t out_stride_h, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return uq_continuation_prefill_stages(UQ_PREFILL_GATHER | UQ_PREFILL_ATTEND, query, key, value,
                                        kv_cache, block_row, cached_len, scale, out, q_len, Hq, Hk,
                                        D, num_blocks, block_size, q_stride_t, q_stride_h,
                                        key_stride_t, key_stride_h, val_stride_t, val_stride_h,
                                        out_stride_t, out_stride_h, workspace, workspace_bytes, stream);
}

const char* uq_last_error(void) { return g_err.c_str(); }

}  // extern "C"
