/*
 * uq.h - C ABI of libuq: UltraQuant-style 4-bit paged-KV decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * Method (vLLM API docs, "vllm/v1/attention/backends/ultraquant_attn",
 * UltraQuantAttentionImpl, and "vllm/v1/attention/ops/flydsl_ultraquant_decode"):
 * keys are rotated by the orthonormal, symmetric 256-point Hadamard matrix and
 * stored, with the values, as FP4 E2M1 codes with one UE8M0 power-of-two scale
 * per 32 elements in a block-table-indexed (paged) cache. Decode rotates the
 * query by the same matrix, rounds it to FP8 E4M3 (the "haircut"), and runs
 * split-KV attention: stage 1 writes a partial output, running max and sum of
 * exponentials per split; stage 2 merges the splits by log-sum-exp.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device memory on the current HIP device;
 *     the caller owns every buffer. The library allocates nothing, keeps no
 *     device state between calls and never synchronises the stream.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Results are visible once the stream has been synchronised.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Return value: UQ_OK (0) or a negative UQ_E* code. All argument checks
 *     run on the host before any HIP call, so a rejected call enqueues
 *     nothing; uq_last_error() returns a message for the calling thread.
 *
 * Cache slot (one token, one KV head) of head dim D, 17*D/16 bytes (272 for
 * D = 256, 136 for 128, 544 for 512):
 *   [0, D/2)          K codes: byte i holds element 2i in bits 0-3, 2i+1 in
 *                     bits 4-7; K is in the rotated basis
 *   [D/2, D)          V codes, same packing, not rotated
 *   [D, D + D/32)     K scale bytes, one per 32 consecutive elements
 *                     (UE8M0: 2**(b-127))
 *   [D + D/32, 17D/16) V scale bytes
 *   A 4-bit code is sign (bit 3) plus E2M1 magnitude {0,.5,1,1.5,2,3,4,6}.
 *   The scale byte of a block with maximum magnitude a is
 *   clamp(floor(log2 a) - 2, -127, 127) + 127 (0 for an all-zero block), the
 *   OCP MX shared-exponent rule; codes are rounded to nearest, ties to even,
 *   saturating at 6.
 * The cache is (num_blocks, block_size, Hk, 17*D/16) bytes, contiguous: slot s
 * of KV head h starts at byte (s * Hk + h) * 17*D/16.
 * The rotation of head dim D is the Sylvester Hadamard matrix with entries
 * (-1)**popcount(i & j) times one float64 scale, the nearest double to
 * 1/sqrt(D) (exactly 1/16 for D = 256).
 * Every call takes D in {128, 256, 512}.
 */
#ifndef UQ_H
#define UQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UQ_OK            0
#define UQ_EINVAL       -1   /* null pointer, non-positive size, bad stride */
#define UQ_EUNSUPPORTED -2   /* a shape or option the kernels do not cover  */
#define UQ_EWORKSPACE   -3   /* workspace smaller than uq_decode_workspace_bytes() */
#define UQ_EHIP         -4   /* a HIP launch failed                          */

#define UQ_HEAD_DIM   256                       /* the default head dim */
#define UQ_SLOT_BYTES 272                       /* its slot: 17 * 256 / 16 */
#define UQ_SLOT_BYTES_FOR(D) ((D) * 17 / 16)
#define UQ_MAX_SPLITS 512

/*
 * Build the normalised Sylvester Hadamard matrix
 * H[i][j] = (-1)**popcount(i & j) / sqrt(D) as D x D float32, row-major.
 * Follows _ensure_on_device on the UltraQuantAttentionImpl page: one matrix
 * serves as both Pi and PiT because it is orthonormal and symmetric.
 *   D: power of two, 1 <= D <= 512 (512: the rotation of the head-dim-512
 *      cache; entries are the float32 nearest the float64 1/sqrt(D)).
 *   H: (device) D*D floats, written.
 * Errors: UQ_EINVAL for a null H or D not a power of two in range.
 */
int uq_build_hadamard(int D, float* H, void* stream);

/*
 * Store N tokens: rotate each key vector by H (exactly, in float64), quantise
 * keys and values to FP4 E2M1 + UE8M0 per 32 elements, and write slot
 * slot_mapping[n] of every KV head. Follows _store_kv on the
 * UltraQuantAttentionImpl page (key, value (N, Hk, D); kv_cache
 * (num_blocks, block_size, Hk, slot_size); slot_mapping).
 *   key, value:   (device) bf16, element (n, h, d) at n*stride_n + h*stride_h + d
 *                 (strides in elements; d is contiguous).
 *   kv_cache:     (device) uint8, (num_blocks, block_size, Hk, 17*D/16),
 *                 in/out; only the written slots change.
 *   slot_mapping: (device) int64, (N,). A slot outside
 *                 [0, num_blocks * block_size) - for instance -1 for padding -
 *                 is skipped.
 *   D in {128, 256, 512}, slot_size 17*D/16, block_size a power of two in
 *   [16, 256]. N == 0 is a no-op.
 * Exactness: the rotation is exact when the non-zero magnitudes of a key
 * vector span at most 45 - log2(D) binades (37 for D = 256) (always true for bf16 data of ordinary
 * range); the cache bytes are then a function of the inputs alone.
 * Errors: UQ_EINVAL, UQ_EUNSUPPORTED, UQ_EHIP.
 */
int uq_store(const uint16_t* key, const uint16_t* value, uint8_t* kv_cache,
             const int64_t* slot_mapping, int64_t N, int Hk, int D,
             int64_t num_blocks, int block_size, int slot_size,
             int64_t key_stride_n, int64_t key_stride_h,
             int64_t val_stride_n, int64_t val_stride_h, void* stream);

/*
 * Bytes of device workspace uq_decode needs for this shape (0 on invalid
 * arguments). The analogue of the pooled segm_out / segm_max / segm_sum and
 * q_fp8 buffers of _SegmBufPool on the flydsl_ultraquant_decode page: query
 * E4M3 codes, one fp16 partial output row (with a power-of-two row scale)
 * and three 4-byte statistics (max, sum, scale exponent) per (sequence,
 * query head, partial). The count of partials depends on the
 * split count and on the block-table capacity max_blocks_per_seq *
 * block_size, never on the sequence lengths, so one workspace serves every
 * step of a fixed-shape batch. The size covers uq_decode_ex too, whose
 * multi-query rows may cut finer partials (at a GQA group of 8 or less).
 */
size_t uq_decode_workspace_bytes(int B, int Hq, int Hk, int D, int num_kv_splits,
                                 int max_blocks_per_seq, int block_size);

/*
 * Number of partial results stage 1 writes per (sequence, query head) for
 * this shape (0 on invalid arguments): one per run of whole splits, or per
 * piece of a split, as uq_decode cuts them. The workspace holds that many
 * rows per (sequence, query head).
 */
int uq_decode_partials(int B, int Hq, int Hk, int D, int num_kv_splits, int max_blocks_per_seq,
                       int block_size);

/*
 * Decode one query token per sequence against the paged 4-bit cache and
 * write out = softmax(scale * q8 . K^T) V per query head, where
 * q8 = E4M3(q H) and query head hq reads KV head hq / (Hq / Hk). Follows
 * flydsl_ultraquant_decode_attention on the flydsl_ultraquant_decode page
 * (query, kv_cache, block_table, seq_lens, scale, max_num_kv_splits ->
 * output (B, Hq, D) in the query dtype) and the split-KV stage 1 / stage 2
 * structure of triton_turboquant_decode_attention_v2. Enqueues three kernels
 * (query prologue, split-KV stage 1, log-sum-exp merge) on `stream`; no host
 * synchronisation and no allocation, so it can be captured in a HIP graph.
 * (The page rotates the query inside its decode kernel; that two-launch form
 * is uq_decode_stages(UQ_STAGE_SPLIT | UQ_STAGE_FUSED_QUERY | UQ_STAGE_MERGE)
 * at D = 256, bit for bit the same output.)
 *   query:       (device) bf16, element (b, hq, d) at b*q_stride_b + hq*q_stride_h + d.
 *   kv_cache:    (device) uint8 (num_blocks, block_size, Hk, 17*D/16), read only.
 *   block_table: (device) int32 (B, max_blocks_per_seq): logical block j of
 *                sequence b lives in physical block block_table[b][j].
 *   seq_lens:    (device) int32 (B,): tokens of each sequence, the current one
 *                included. Values are clamped to [0, max_blocks_per_seq*block_size];
 *                a sequence of length 0 yields zeros. Physical block ids outside
 *                [0, num_blocks) are read as empty blocks.
 *   scale:       softmax scale applied to q8 . k (finite, > 0).
 *   num_kv_splits: number of key ranges, 1..512. Split s covers the 16-token
 *                tiles [s*c, (s+1)*c) of every sequence, with
 *                c = ceil(ceil(max_blocks_per_seq*block_size / 16) / num_kv_splits),
 *                so splits past a sequence's end are empty. Stage 1 writes
 *                one partial per run of whole splits (or per piece of a
 *                split); the result does not depend on the count beyond
 *                rounding.
 *   out:         (device) bf16 (B, Hq, D) contiguous, written.
 *   workspace:   (device) at least uq_decode_workspace_bytes(B, Hq, Hk, D,
 *                num_kv_splits, max_blocks_per_seq, block_size) bytes, 256-byte aligned; contents need no
 *                initialisation and are overwritten.
 *   D in {128, 256, 512}; Hq % Hk == 0 with Hq / Hk in {6, 8, 16}; block_size
 *   a power of two in [16, 256].
 * Errors: UQ_EINVAL, UQ_EUNSUPPORTED, UQ_EWORKSPACE, UQ_EHIP.
 */
int uq_decode(const uint16_t* query, const uint8_t* kv_cache,
              const int32_t* block_table, const int32_t* seq_lens, float scale,
              int num_kv_splits, uint16_t* out, int B, int Hq, int Hk, int D,
              int64_t num_blocks, int block_size, int max_blocks_per_seq,
              int64_t q_stride_b, int64_t q_stride_h, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * uq_decode for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * the same output bit for bit, with the workspace taken from a device array
 * inside the library instead of the caller's memory. The array,
 * UQ_NO_ALLOC_SCRATCH_BYTES (64 MiB) per device, is held from the library's
 * load on a device until the process ends; its address is looked up once per
 * device (hipGetSymbolAddress) on the first call there. The call allocates
 * nothing and does not synchronise.
 *   Arguments as for uq_decode, without workspace and workspace_bytes.
 *   `stream` must belong to the current device (NULL: the current device's
 *   null stream).
 * Every call on a device shares that device's array: calls whose work may
 * overlap on one device (several streams, or several threads) race and must
 * be serialised by the caller. The array needs no initialisation: every byte
 * a call reads was written by that call.
 * Errors: as uq_decode; UQ_EWORKSPACE when the shape needs more than
 * UQ_NO_ALLOC_SCRATCH_BYTES (checked on the host before any HIP call, like
 * every argument; uq_decode_workspace_bytes gives the need), UQ_EINVAL for a
 * stream of another device.
 */
#define UQ_NO_ALLOC_SCRATCH_BYTES (64 << 20)
int uq_decode_no_alloc(const uint16_t* query, const uint8_t* kv_cache,
                       const int32_t* block_table, const int32_t* seq_lens, float scale,
                       int num_kv_splits, uint16_t* out, int B, int Hq, int Hk, int D,
                       int64_t num_blocks, int block_size, int max_blocks_per_seq,
                       int64_t q_stride_b, int64_t q_stride_h, void* stream);

/*
 * uq_decode with three options; uq_decode is this call with none of them.
 *
 * Multi-query rows (query_row). Several query rows may read the same
 * sequence, each with its own length. This is how the ultraquant_attn page
 * decodes a short continuation chunk (_prefill_attention, continuation
 * branch): query i of a chunk whose sequence holds cached_len tokens gets
 * the length cached_len + i + 1 and the sequence's block-table row, repeated
 * for every query of the chunk. Here the rows are not repeated: query row b
 * reads block-table row query_row[b]. Query rows 2r and 2r + 1 that read
 * the same table row (at a GQA group of 8 or less, without a window) are
 * decoded together, each tile of their common prefix read once; put the
 * queries of one sequence next to each other to benefit.
 *   query_row:    (device) int32 (B,), or NULL for query_row[b] = b (then
 *                 n_table_rows must be B). A value outside
 *                 [0, n_table_rows) makes that query's output zeros.
 *   block_table:  (device) int32 (n_table_rows, max_blocks_per_seq).
 *   seq_lens:     (device) int32 (B,): the length each query row attends to.
 *
 * Attention sinks (sinks). The ultraquant_attn page passes per-head sinks
 * to its unified kernel. Here a sink is one more logit per query head in
 * the softmax normaliser, with no value behind it, in the units of
 * scale * q8 . k: out = sum_t e^(x_t) v_t / (e^(s) + sum_t e^(x_t)).
 *   sinks:        (device) float32 (Hq,), or NULL; finite or -inf.
 *
 * Sliding window (sliding_window). The page's dense path passes a window W
 * as (W - 1, 0): a query sees itself and the W - 1 keys before it, so each
 * query row attends to the last min(W, seq_len) tokens. 0 means no window.
 *
 * Every other argument is as for uq_decode, with B the number of query rows
 * (query, out and the workspace are sized per query row).
 * Errors: as uq_decode; UQ_EINVAL also for n_table_rows < 1 (or != B
 * without query_row), sliding_window < 0, or a misaligned query_row / sinks.
 */
int uq_decode_ex(const uint16_t* query, const uint8_t* kv_cache,
                 const int32_t* block_table, int n_table_rows, const int32_t* query_row,
                 const int32_t* seq_lens, float scale, int num_kv_splits,
                 const float* sinks, int sliding_window, uint16_t* out,
                 int B, int Hq, int Hk, int D, int64_t num_blocks, int block_size,
                 int max_blocks_per_seq, int64_t q_stride_b, int64_t q_stride_h,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Same as uq_decode, restricted to the stages named in stage_mask:
 * UQ_STAGE_PROLOGUE (query rotation + E4M3 into the workspace: its first
 * B*Hq*D bytes then hold the E4M3 codes of q H, row b*Hq + hq),
 * UQ_STAGE_SPLIT (stage 1, reads the prologue's output) and UQ_STAGE_MERGE
 * (stage 2, reads stage 1's output). Running the three masks in that order on
 * one stream, with the same arguments and workspace, is exactly uq_decode;
 * it exists so a caller can time or capture each kernel on its own.
 * UQ_STAGE_FUSED_QUERY, with UQ_STAGE_SPLIT, makes stage 1 compute the query
 * codes itself (D = 256 only: the in-kernel Walsh-Hadamard rotation of the
 * flydsl_ultraquant_decode page, here a 16 x 16 Kronecker product on float64
 * matrix cores, exact, then E4M3); UQ_STAGE_SPLIT | UQ_STAGE_FUSED_QUERY |
 * UQ_STAGE_MERGE is then a two-launch decode, bit for bit uq_decode's output.
 * Every partial's workgroup repeats its rows' rotation, which measured slower
 * than the separate prologue launch on every workload, so uq_decode keeps
 * three launches.
 * Errors: as uq_decode, plus UQ_EINVAL for an empty or unknown mask (or
 * UQ_STAGE_FUSED_QUERY without UQ_STAGE_SPLIT) and UQ_EUNSUPPORTED for
 * UQ_STAGE_FUSED_QUERY at D != 256.
 */
#define UQ_STAGE_PROLOGUE 1
#define UQ_STAGE_SPLIT    2
#define UQ_STAGE_MERGE    4
#define UQ_STAGE_FUSED_QUERY 8
int uq_decode_stages(int stage_mask, const uint16_t* query, const uint8_t* kv_cache,
                     const int32_t* block_table, const int32_t* seq_lens, float scale,
                     int num_kv_splits, uint16_t* out, int B, int Hq, int Hk, int D,
                     int64_t num_blocks, int block_size, int max_blocks_per_seq,
                     int64_t q_stride_b, int64_t q_stride_h, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Continuation prefill (ultraquant_attn page, _prefill_attention continuation
 * branch for chunks above the decode threshold, and
 * _ultraquant_continuation_prefill): a chunk of q_len new tokens of one
 * sequence, whose first cached_len tokens are already in the cache, attends
 * to the dequantised prefix and to itself. Query i of the chunk sits at
 * absolute position cached_len + i and sees keys 0 .. cached_len + i (causal
 * attention with unequal query/key lengths, aligned to the lower right).
 * The four calls below are the steps of that path; uq_continuation_prefill
 * runs all of them.
 */

/*
 * out[n, h, :] = bf16(x[n, h, :] H) for n < N, h < H: the rotation the page
 * applies to the chunk's keys and queries ((x.float() @ PiT).to(bf16)). The
 * +-1 sums are computed in a float64 butterfly (exact when the vector's
 * non-zero magnitudes span at most 45 - log2(D) binades, as for uq_store),
 * multiplied by the float64 nearest 1/sqrt(D) (exactly 1/16 at D = 256) and
 * rounded once to bf16, nearest-even; the sign of an exactly-zero result is
 * not defined.
 *   x, out:   (device) bf16, last dim contiguous, 8-byte aligned; strides in
 *             elements, non-negative multiples of 4. out may equal x (with
 *             the same strides); other overlaps are undefined.
 *   D:        128, 256 or 512 (UQ_EUNSUPPORTED otherwise).
 * Errors: UQ_EINVAL for N < 0, H < 1, a null pointer (N > 0), bad strides
 * or alignment; UQ_EHIP for a launch failure.
 */
int uq_rotate(const uint16_t* x, uint16_t* out, int64_t N, int H, int D, int64_t x_stride_n,
              int64_t x_stride_h, int64_t out_stride_n, int64_t out_stride_h, void* stream);

/*
 * Dequantise a sequence's first n_tokens tokens (ultraquant_full_dequant_kv
 * on the page): k_out[t, h, :] and v_out[t, h, :] = E2M1 code * 2^(scale - 127)
 * as bf16, K left in the rotated basis. Exact: every such value is a bf16
 * value (0.5 * 2^-127 and up); codes of magnitude 0 give signed zeros.
 *   kv_cache:  (device) the uq_store cache, 16-byte aligned.
 *   block_row: (device) int32, at least ceil(n_tokens / block_size) entries:
 *              physical block of logical block j. An entry outside
 *              [0, num_blocks) reads as zeros.
 *   D:         128, 256 or 512, the head dim of the cache (slot 17*D/16
 *              bytes); UQ_EUNSUPPORTED otherwise.
 *   k_out, v_out: (device) bf16, 16-byte aligned; element [t, h, d] at
 *              t * out_stride_t + h * out_stride_h + d, strides non-negative
 *              multiples of 8 (e.g. Hk*D and D for (n, Hk, D), or D and n*D
 *              for the page's (Hk, n, D) buffers).
 * Errors: UQ_EINVAL / UQ_EUNSUPPORTED for bad shapes, pointers, strides or
 * block sizes; UQ_EHIP for a launch failure.
 */
int uq_dequant_kv(const uint8_t* kv_cache, const int32_t* block_row, int n_tokens, uint16_t* k_out,
                  uint16_t* v_out, int Hk, int D, int64_t num_blocks, int block_size,
                  int64_t out_stride_t, int64_t out_stride_h, void* stream);

/*
 * Dense causal attention over bf16 operands already in the rotated basis:
 * out[i, hq] = softmax_j(scale * q[i, hq] . k[j, hk]) v[j, hk] over
 * j <= seq_len - q_len + i, with hk = hq / (Hq / Hk) (the flash-attention
 * step of the page's path, causal=True with q_len <= seq_len).
 *   q:    (device) bf16 (q_len, Hq, D); k, v: (seq_len, Hk, D) sharing
 *         strides; out: (q_len, Hq, D) bf16, D = 128, 256 or 512. All 16-byte aligned, strides
 *         in elements, non-negative multiples of 8.
 *   scale: finite, > 0. Hq / Hk at most 128 (64 at D = 512). kv_stride_t in
 *   [D, 2^25).
 * Errors: UQ_EINVAL for q_len < 0, seq_len < q_len, a null pointer, bad
 * strides or alignment; UQ_EUNSUPPORTED for D not 128, 256 or 512, Hq % Hk or a key
 * stride outside that range; UQ_EHIP.
 */
int uq_prefill_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                         int q_len, int seq_len, int Hq, int Hk, int D, float scale,
                         int64_t q_stride_t, int64_t q_stride_h, int64_t kv_stride_t,
                         int64_t kv_stride_h, int64_t out_stride_t, int64_t out_stride_h,
                         void* stream);

/* Workspace bytes of uq_continuation_prefill for chunks of up to q_len
 * tokens and sequences of up to max_seq_len tokens, D in {128, 256, 512}; 0 on
 * invalid shapes. */
size_t uq_continuation_prefill_workspace_bytes(int q_len, int max_seq_len, int Hq, int Hk, int D);

/*
 * The whole continuation prefill of one sequence: dequantise the prefix,
 * rotate the chunk's keys and the queries, append the chunk's values, then
 * attend (the steps of uq_dequant_kv, uq_rotate and uq_prefill_attention on
 * buffers in the workspace; three launches on `stream`).
 * Precision of the attention: the workspace holds the values in 32-key
 * tiles as fp16 times a power of two per (KV head, 32-dim block), chosen
 * from the block's largest exponent over prefix and chunk so that its
 * largest magnitude lands below 2^15, and the weights enter the products
 * as fp16 (relative error 2^-11, so at most 2^-11 |v - o| in an output;
 * uq_prefill_attention on bf16 values keeps each weight as a high and a
 * low bf16 part, 2^-16). A value
 * is exact unless it lies more than about 2^31 (a chunk value) or 2^37 (a
 * cached one) below its block's largest; such values round to fp16's
 * subnormals, an absolute error of at most about 2^-37 of that largest.
 *   D:      128, 256 or 512 (UQ_EUNSUPPORTED otherwise).
 *   query:  (device) bf16 (q_len, Hq, D) before rotation; key, value:
 *           (q_len, Hk, D) of the chunk (key before rotation). 8-byte
 *           aligned, strides non-negative multiples of 4 elements.
 *   kv_cache, block_row, num_blocks, block_size: as uq_dequant_kv, for the
 *           cached_len tokens already stored (a cache of head dim D, slots
 *           of 17*D/16 bytes; block_row may be NULL when cached_len is 0).
 *   out:    (device) bf16 (q_len, Hq, D), 16-byte aligned, strides
 *           multiples of 8.
 *   workspace: (device) 256-byte aligned, at least
 *           uq_continuation_prefill_workspace_bytes(q_len, cached_len + q_len,
 *           Hq, Hk, D) bytes; owned by the caller, clobbered.
 * Errors: as the three calls, plus UQ_EWORKSPACE.
 */
int uq_continuation_prefill(const uint16_t* query, const uint16_t* key, const uint16_t* value,
                            const uint8_t* kv_cache, const int32_t* block_row, int cached_len,
                            float scale, uint16_t* out, int q_len, int Hq, int Hk, int D,
                            int64_t num_blocks, int block_size, int64_t q_stride_t,
                            int64_t q_stride_h, int64_t key_stride_t, int64_t key_stride_h,
                            int64_t val_stride_t, int64_t val_stride_h, int64_t out_stride_t,
                            int64_t out_stride_h, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Same as uq_continuation_prefill, restricted to the launches named in
 * stage_mask: UQ_PREFILL_GATHER (dequantised prefix, rotated chunk keys and
 * queries and the chunk's values into the workspace) and UQ_PREFILL_ATTEND
 * (the attention over them). Both masks in that order on one stream, with
 * the same arguments and workspace, are exactly uq_continuation_prefill; it
 * exists so that each kernel can be timed or captured alone.
 * Errors: as uq_continuation_prefill, plus UQ_EINVAL for an empty or
 * unknown mask.
 */
#define UQ_PREFILL_GATHER 1
#define UQ_PREFILL_ATTEND 2
int uq_continuation_prefill_stages(int stage_mask, const uint16_t* query, const uint16_t* key,
                                   const uint16_t* value, const uint8_t* kv_cache,
                                   const int32_t* block_row, int cached_len, float scale,
                                   uint16_t* out, int q_len, int Hq, int Hk, int D,
                                   int64_t num_blocks, int block_size, int64_t q_stride_t,
                                   int64_t q_stride_h, int64_t key_stride_t, int64_t key_stride_h,
                                   int64_t val_stride_t, int64_t val_stride_h, int64_t out_stride_t,
                                   int64_t out_stride_h, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Message describing the last non-zero return on the calling thread
 * ("" if none). The pointer stays valid until the thread's next call. */
/*
 * Streaming-read probe (a measurement aid, not a step of the method): reads
 * every cache byte a decode of these sequences reads (each physical block a
 * sequence's tokens live in, all Hk heads, up to the sequence's last token,
 * in block-table order) with plain 16-byte loads and does nothing with them
 * but an XOR, so its rate is the ceiling for streaming those blocks on the
 * device. Arguments as for uq_decode (kv_cache (num_blocks, block_size, Hk,
 * 17*D/16) read only, block_table (B, max_blocks_per_seq), seq_lens (B,),
 * clamped like uq_decode's); sink: (device) sink_words >= 1 uint32 words,
 * overwritten with values of no meaning. Errors: UQ_EINVAL, UQ_EUNSUPPORTED,
 * UQ_EHIP.
 */
int uq_stream_blocks(const uint8_t* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                     int B, int Hk, int D, int64_t num_blocks, int block_size, int max_blocks_per_seq,
                     uint32_t* sink, int sink_words, void* stream);

const char* uq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* UQ_H */
