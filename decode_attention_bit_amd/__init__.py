"""Python binding of libuq (4-bit paged-KV decode attention for MI355X).

Argument marshalling only: every step of the store and decode runs in the
HIP kernels of ``libuq.so``. PyTorch provides device memory and the current
stream. Importing the package does not load the library; the first call does,
and raises if the library has not been built (there is no fallback path).

Entry points mirror include/uq.h:
  build_hadamard(D, device)                         -> (D, D) float32
  store(key, value, kv_cache, slot_mapping)         -> None (kv_cache updated)
  decode_workspace_bytes(B, Hq, Hk, num_kv_splits, max_blocks_per_seq, block_size, D)  -> int
  decode(query, kv_cache, block_table, seq_lens, scale, num_kv_splits,
         out=None, workspace=None)                  -> (B, Hq, D) bf16
  decode_ex(query, kv_cache, block_table, seq_lens, scale, num_kv_splits,
            query_row=None, sinks=None, sliding_window=0,
            out=None, workspace=None)               -> (B, Hq, D) bf16
Every call takes head dims D in {128, 256, 512} (slot 17*D/16 bytes).
  rotate(x, out=None)                               -> bf16(x H), same shape
  dequant_kv(kv_cache, block_row, n_tokens)         -> (K, V) (n_tokens, Hk, D) bf16
  prefill_attention(q, k, v, scale, out=None)       -> (q_len, Hq, D) bf16
  continuation_prefill(query, key, value, kv_cache, block_row, cached_len, scale,
                       out=None, workspace=None)    -> (q_len, Hq, D) bf16
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["build_hadamard", "store", "decode", "decode_ex", "decode_no_alloc", "decode_workspace_bytes",
           "decode_partials", "stream_blocks", "rotate",
           "dequant_kv", "prefill_attention", "continuation_prefill",
           "continuation_prefill_workspace_bytes", "library_path",
           "UQError", "HEAD_DIM", "HEAD_DIMS", "SLOT_BYTES", "slot_bytes"]

HEAD_DIM = 256
SLOT_BYTES = 272
HEAD_DIMS = (128, 256, 512)


def slot_bytes(D: int = HEAD_DIM) -> int:
    """Cache bytes per (token, KV head) for head dim D."""
    return D * 17 // 16

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libuq.so"
_lib = None

UQ_OK, UQ_EINVAL, UQ_EUNSUPPORTED, UQ_EWORKSPACE, UQ_EHIP = 0, -1, -2, -3, -4


class UQError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libuq error {code}: {msg}")
        self.code = code


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.uq_build_hadamard.argtypes = [i32, vp, vp]
    lib.uq_build_hadamard.restype = i32
    lib.uq_store.argtypes = [vp, vp, vp, vp, i64, i32, i32, i64, i32, i32, i64, i64, i64, i64, vp]
    lib.uq_store.restype = i32
    lib.uq_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.uq_decode_workspace_bytes.restype = sz
    lib.uq_decode.argtypes = [vp, vp, vp, vp, ctypes.c_float, i32, vp, i32, i32, i32, i32, i64,
                              i32, i32, i64, i64, vp, sz, vp]
    lib.uq_decode.restype = i32
    lib.uq_decode_ex.argtypes = [vp, vp, vp, i32, vp, vp, ctypes.c_float, i32, vp, i32, vp, i32, i32,
                                 i32, i32, i64, i32, i32, i64, i64, vp, sz, vp]
    lib.uq_decode_ex.restype = i32
    lib.uq_decode_stages.argtypes = [i32] + lib.uq_decode.argtypes
    lib.uq_decode_stages.restype = i32
    lib.uq_rotate.argtypes = [vp, vp, i64, i32, i32, i64, i64, i64, i64, vp]
    lib.uq_rotate.restype = i32
    lib.uq_dequant_kv.argtypes = [vp, vp, i32, vp, vp, i32, i32, i64, i32, i64, i64, vp]
    lib.uq_dequant_kv.restype = i32
    lib.uq_prefill_attention.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_float,
                                         i64, i64, i64, i64, i64, i64, vp]
    lib.uq_prefill_attention.restype = i32
    lib.uq_continuation_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.uq_continuation_prefill_workspace_bytes.restype = sz
    lib.uq_continuation_prefill.argtypes = [vp, vp, vp, vp, vp, i32, ctypes.c_float, vp, i32, i32, i32,
                                            i32, i64, i32, i64, i64, i64, i64, i64, i64, i64, i64,
                                            vp, sz, vp]
    lib.uq_continuation_prefill.restype = i32
    lib.uq_continuation_prefill_stages.argtypes = [i32] + lib.uq_continuation_prefill.argtypes
    lib.uq_continuation_prefill_stages.restype = i32
    lib.uq_decode_no_alloc.argtypes = [vp, vp, vp, vp, ctypes.c_float, i32, vp, i32, i32, i32, i32, i64,
                                       i32, i32, i64, i64, vp]
    lib.uq_decode_no_alloc.restype = i32
    lib.uq_decode_partials.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.uq_decode_partials.restype = i32
    lib.uq_stream_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i64, i32, i32, vp, i32, vp]
    lib.uq_stream_blocks.restype = i32
    lib.uq_last_error.argtypes = []
    lib.uq_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(code):
    if code != UQ_OK:
        msg = _load().uq_last_error().decode()
        if code in (UQ_EINVAL, UQ_EWORKSPACE):
            raise ValueError(f"libuq error {code}: {msg}")
        if code == UQ_EUNSUPPORTED:
            raise NotImplementedError(f"libuq error {code}: {msg}")
        raise UQError(code, msg)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def build_hadamard(D: int = HEAD_DIM, device="cuda") -> torch.Tensor:
    device = torch.device(device)
    H = torch.empty((D, D), dtype=torch.float32, device=device)
    _check(_load().uq_build_hadamard(int(D), _ptr(H), _stream(device)))
    return H


def store(key: torch.Tensor, value: torch.Tensor, kv_cache: torch.Tensor,
          slot_mapping: torch.Tensor) -> None:
    """Quantise (N, Hk, D) bf16 key/value, D in {128, 256, 512}, into
    kv_cache (num_blocks, block_size, Hk, 17*D/16) uint8 at flat slots
    slot_mapping (int64, (N,))."""
    if key.dtype != torch.bfloat16 or value.dtype != torch.bfloat16:
        raise TypeError("key and value must be bfloat16")
    if kv_cache.dtype != torch.uint8 or not kv_cache.is_contiguous() or kv_cache.dim() != 4:
        raise TypeError("kv_cache must be a contiguous 4-d uint8 tensor")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise TypeError("slot_mapping must be a contiguous int64 tensor")
    if key.shape != value.shape or key.dim() != 3 or key.stride(2) != 1 or value.stride(2) != 1:
        raise ValueError("key and value must be (N, Hk, D) with a contiguous last dim")
    N, Hk, D = key.shape
    nb, bs, hk, ss = kv_cache.shape
    if hk != Hk or slot_mapping.numel() != N:
        raise ValueError("shape mismatch between key, kv_cache and slot_mapping")
    _check(_load().uq_store(_ptr(key), _ptr(value), _ptr(kv_cache), _ptr(slot_mapping), N, Hk, D,
                            nb, bs, ss, key.stride(0), key.stride(1), value.stride(0),
                            value.stride(1), _stream(key.device)))


def decode_workspace_bytes(B: int, Hq: int, Hk: int, num_kv_splits: int, max_blocks_per_seq: int,
                           block_size: int = 16, D: int = HEAD_DIM) -> int:
    n = _load().uq_decode_workspace_bytes(int(B), int(Hq), int(Hk), int(D), int(num_kv_splits),
                                          int(max_blocks_per_seq), int(block_size))
    if n == 0:
        raise ValueError("invalid decode shape")
    return int(n)


def decode_partials(B: int, Hq: int, Hk: int, num_kv_splits: int, max_blocks_per_seq: int,
                    block_size: int = 16, D: int = HEAD_DIM) -> int:
    """Partial results per (sequence, query head) that uq_decode writes for
    this shape (uq_decode_partials)."""
    n = _load().uq_decode_partials(int(B), int(Hq), int(Hk), int(D), int(num_kv_splits),
                                   int(max_blocks_per_seq), int(block_size))
    if n == 0:
        raise ValueError("invalid decode shape")
    return int(n)


def stream_blocks(kv_cache: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                  sink: torch.Tensor) -> None:
    """uq_stream_blocks: read every cache byte a decode of these sequences
    reads, and nothing else (a measurement aid); sink is an int32/uint32
    device tensor of scratch words."""
    if kv_cache.dtype != torch.uint8 or not kv_cache.is_contiguous() or kv_cache.dim() != 4:
        raise TypeError("kv_cache must be a contiguous 4-d uint8 tensor")
    if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2:
        raise TypeError("block_table must be a contiguous (B, max_blocks) int32 tensor")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise TypeError("seq_lens must be a contiguous int32 tensor")
    if sink.element_size() != 4 or not sink.is_contiguous():
        raise TypeError("sink must be a contiguous tensor of 4-byte words")
    nb, bs, Hk, ss = kv_cache.shape
    B = block_table.shape[0]
    if seq_lens.numel() != B:
        raise ValueError("seq_lens must have one entry per table row")
    _check(_load().uq_stream_blocks(_ptr(kv_cache), _ptr(block_table), _ptr(seq_lens), B, Hk,
                                    ss * 16 // 17, nb, bs, block_table.shape[1], _ptr(sink),
                                    sink.numel(), _stream(kv_cache.device)))


_WS_POOL: dict = {}


def _workspace(device, nbytes: int) -> torch.Tensor:
    """Cached workspace per (device, current stream), grown when a bigger one
    is needed. Calls on one stream run in order, so they can share it; calls
    on different streams get different buffers, and a replaced buffer is
    freed on the stream that used it. A call captured into a graph must pass
    its own workspace: replays would otherwise share this buffer with eager
    calls and with other graphs, and a later call that grows it would free
    memory a graph still writes on replay."""
    if torch.cuda.is_current_stream_capturing():
        raise ValueError("a call captured into a graph must pass its own workspace (workspace=...): "
                         "the cached workspace is shared with eager calls and can be replaced while "
                         "the graph still uses it")
    key = (str(torch.device(device)), _stream(device))
    ws = _WS_POOL.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WS_POOL[key] = ws
    return ws


STAGE_PROLOGUE, STAGE_SPLIT, STAGE_MERGE, STAGE_FUSED_QUERY = 1, 2, 4, 8


def decode(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, scale: float, num_kv_splits: int,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           stages: int | None = None) -> torch.Tensor:
    """Split-KV decode over the 4-bit cache; returns (B, Hq, D) bf16.

    ``stages`` (STAGE_PROLOGUE | STAGE_SPLIT | STAGE_MERGE, and
    STAGE_FUSED_QUERY with STAGE_SPLIT for stage 1 computing the query codes
    itself) runs a subset of the kernels through uq_decode_stages; None runs
    uq_decode."""
    if query.dtype != torch.bfloat16 or query.dim() != 3 or query.stride(2) != 1:
        raise TypeError("query must be (B, Hq, D) bfloat16 with a contiguous last dim")
    if kv_cache.dtype != torch.uint8 or not kv_cache.is_contiguous() or kv_cache.dim() != 4:
        raise TypeError("kv_cache must be a contiguous 4-d uint8 tensor")
    if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2:
        raise TypeError("block_table must be a contiguous (B, max_blocks) int32 tensor")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise TypeError("seq_lens must be a contiguous int32 tensor")
    B, Hq, D = query.shape
    nb, bs, Hk, ss = kv_cache.shape
    if block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table / seq_lens batch mismatch")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=query.device)
    elif out.dtype != torch.bfloat16 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, D):
        raise TypeError("out must be a contiguous (B, Hq, D) bfloat16 tensor")
    need = _load().uq_decode_workspace_bytes(B, Hq, Hk, D, int(num_kv_splits), block_table.shape[1], bs)
    if workspace is None:
        workspace = _workspace(query.device, max(int(need), 256))
    lib = _load()
    fn = lib.uq_decode if stages is None else (lambda *a: lib.uq_decode_stages(int(stages), *a))
    _check(fn(_ptr(query), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
                             float(scale), int(num_kv_splits), _ptr(out), B, Hq, Hk, D, nb, bs,
                             block_table.shape[1], query.stride(0), query.stride(1),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(query.device)))
    return out


def decode_no_alloc(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, scale: float, num_kv_splits: int,
                    out: torch.Tensor) -> torch.Tensor:
    """uq_decode_no_alloc: uq_decode with the workspace in the library's
    device scratch (no allocation at all: ``out`` is the caller's). Calls that
    may overlap on one device share that scratch and must be serialised."""
    if query.dtype != torch.bfloat16 or query.dim() != 3 or query.stride(2) != 1:
        raise TypeError("query must be (B, Hq, D) bfloat16 with a contiguous last dim")
    if kv_cache.dtype != torch.uint8 or not kv_cache.is_contiguous() or kv_cache.dim() != 4:
        raise TypeError("kv_cache must be a contiguous 4-d uint8 tensor")
    if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2:
        raise TypeError("block_table must be a contiguous (B, max_blocks) int32 tensor")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise TypeError("seq_lens must be a contiguous int32 tensor")
    B, Hq, D = query.shape
    nb, bs, Hk, ss = kv_cache.shape
    if block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError("block_table / seq_lens batch mismatch")
    if out.dtype != torch.bfloat16 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, D):
        raise TypeError("out must be a contiguous (B, Hq, D) bfloat16 tensor")
    _check(_load().uq_decode_no_alloc(_ptr(query), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
                                      float(scale), int(num_kv_splits), _ptr(out), B, Hq, Hk, D, nb, bs,
                                      block_table.shape[1], query.stride(0), query.stride(1),
                                      _stream(query.device)))
    return out


def decode_ex(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
              seq_lens: torch.Tensor, scale: float, num_kv_splits: int,
              query_row: torch.Tensor | None = None, sinks: torch.Tensor | None = None,
              sliding_window: int = 0, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """uq_decode_ex: decode with optional per-query table rows (query row b
    reads block-table row query_row[b]), per-head sink logits and a sliding
    window of the last `sliding_window` tokens; returns (B, Hq, D) bf16."""
    if query.dtype != torch.bfloat16 or query.dim() != 3 or query.stride(2) != 1:
        raise TypeError("query must be (B, Hq, D) bfloat16 with a contiguous last dim")
    if kv_cache.dtype != torch.uint8 or not kv_cache.is_contiguous() or kv_cache.dim() != 4:
        raise TypeError("kv_cache must be a contiguous 4-d uint8 tensor")
    if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2:
        raise TypeError("block_table must be a contiguous (rows, max_blocks) int32 tensor")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise TypeError("seq_lens must be a contiguous int32 tensor")
    if query_row is not None and (query_row.dtype != torch.int32 or not query_row.is_contiguous()):
        raise TypeError("query_row must be a contiguous int32 tensor")
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous()):
        raise TypeError("sinks must be a contiguous float32 tensor")
    B, Hq, D = query.shape
    nb, bs, Hk, ss = kv_cache.shape
    if seq_lens.numel() != B or (query_row is not None and query_row.numel() != B):
        raise ValueError("seq_lens / query_row must have one entry per query row")
    if sinks is not None and sinks.numel() != Hq:
        raise ValueError("sinks must have one entry per query head")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=query.device)
    elif out.dtype != torch.bfloat16 or not out.is_contiguous() or tuple(out.shape) != (B, Hq, D):
        raise TypeError("out must be a contiguous (B, Hq, D) bfloat16 tensor")
    lib = _load()
    need = lib.uq_decode_workspace_bytes(B, Hq, Hk, D, int(num_kv_splits), block_table.shape[1], bs)
    if workspace is None:
        workspace = _workspace(query.device, max(int(need), 256))
    _check(lib.uq_decode_ex(_ptr(query), _ptr(kv_cache), _ptr(block_table), block_table.shape[0],
                            _ptr(query_row) if query_row is not None else None, _ptr(seq_lens),
                            float(scale), int(num_kv_splits),
                            _ptr(sinks) if sinks is not None else None, int(sliding_window),
                            _ptr(out), B, Hq, Hk, D, nb, bs, block_table.shape[1], query.stride(0),
                            query.stride(1), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(query.device)))
    return out


def _bf16_3d(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1:
        raise TypeError(f"{name} must be a 3-d bfloat16 tensor with a contiguous last dim")


def rotate(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """uq_rotate: bf16(x H) for (N, H, D) bf16 x, D in {128, 256, 512} (exact
    product times the float64 nearest 1/sqrt(D), one rounding)."""
    _bf16_3d(x, "x")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _bf16_3d(out, "out")
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    N, H, D = x.shape
    _check(_load().uq_rotate(_ptr(x), _ptr(out), N, H, D, x.stride(0), x.stride(1), out.stride(0),
                             out.stride(1), _stream(x.device)))
    return out


def dequant_kv(kv_cache: torch.Tensor, block_row: torch.Tensor, n_tokens: int,
               k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None):
    """uq_dequant_kv: the first n_tokens tokens of the sequence whose logical
    block j is physical block block_row[j], as (n_tokens, Hk, D) bf16 K
    (rotated basis) and V, D = 16/17 of the slot size. k_out / v_out may be
    any (n_tokens, Hk, D) views with a contiguous last dim."""
    if kv_cache.dtype != torch.uint8 or not kv_cache.is_contiguous() or kv_cache.dim() != 4:
        raise TypeError("kv_cache must be a contiguous 4-d uint8 tensor")
    if block_row.dtype != torch.int32 or not block_row.is_contiguous():
        raise TypeError("block_row must be a contiguous int32 tensor")
    nb, bs, Hk, ss = kv_cache.shape
    D = ss * 16 // 17
    if D not in HEAD_DIMS or slot_bytes(D) != ss:
        raise ValueError(f"kv_cache slot size {ss} is not 17*D/16 for D in {HEAD_DIMS}")
    if block_row.numel() * bs < n_tokens:
        raise ValueError("block_row holds fewer blocks than n_tokens needs")
    shape = (int(n_tokens), Hk, D)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.bfloat16, device=kv_cache.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=torch.bfloat16, device=kv_cache.device)
    for t, name in ((k_out, "k_out"), (v_out, "v_out")):
        _bf16_3d(t, name)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
    if k_out.stride() != v_out.stride():
        raise ValueError("k_out and v_out must share strides")
    _check(_load().uq_dequant_kv(_ptr(kv_cache), _ptr(block_row), int(n_tokens), _ptr(k_out),
                                 _ptr(v_out), Hk, D, nb, bs, k_out.stride(0), k_out.stride(1),
                                 _stream(kv_cache.device)))
    return k_out, v_out


def prefill_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """uq_prefill_attention: causal attention of (q_len, Hq, D) bf16 queries
    over (seq_len, Hk, D) bf16 keys/values, D in {128, 256, 512}, query i at
    position seq_len - q_len + i; returns (q_len, Hq, D) bf16."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _bf16_3d(t, name)
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v must share shape and strides")
    q_len, Hq, D = q.shape
    seq_len, Hk, _ = k.shape
    if out is None:
        out = torch.empty((q_len, Hq, D), dtype=torch.bfloat16, device=q.device)
    _bf16_3d(out, "out")
    _check(_load().uq_prefill_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), q_len, seq_len, Hq, Hk,
                                        D, float(scale), q.stride(0), q.stride(1), k.stride(0),
                                        k.stride(1), out.stride(0), out.stride(1), _stream(q.device)))
    return out


def continuation_prefill_workspace_bytes(q_len: int, max_seq_len: int, Hq: int, Hk: int,
                                         D: int = HEAD_DIM) -> int:
    n = _load().uq_continuation_prefill_workspace_bytes(int(q_len), int(max_seq_len), int(Hq),
                                                        int(Hk), int(D))
    if n == 0:
        raise ValueError("invalid continuation-prefill shape")
    return int(n)


PREFILL_GATHER, PREFILL_ATTEND = 1, 2


def continuation_prefill(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                         kv_cache: torch.Tensor, block_row: torch.Tensor | None, cached_len: int,
                         scale: float, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stages: int = 3) -> torch.Tensor:
    """uq_continuation_prefill: a chunk of q_len tokens (query (q_len, Hq, D),
    key / value (q_len, Hk, D), bf16, unrotated, D in {128, 256, 512}) after
    cached_len cached tokens reached through block_row (a cache of head dim
    D); returns (q_len, Hq, D) bf16.
    ``stages`` selects the gather and/or the attention launch
    (uq_continuation_prefill_stages); the default runs both."""
    for t, name in ((query, "query"), (key, "key"), (value, "value")):
        _bf16_3d(t, name)
    if kv_cache.dtype != torch.uint8 or not kv_cache.is_contiguous() or kv_cache.dim() != 4:
        raise TypeError("kv_cache must be a contiguous 4-d uint8 tensor")
    if block_row is not None and (block_row.dtype != torch.int32 or not block_row.is_contiguous()):
        raise TypeError("block_row must be a contiguous int32 tensor")
    q_len, Hq, D = query.shape
    nb, bs, Hk, ss = kv_cache.shape
    if key.shape != (q_len, Hk, D) or value.shape != (q_len, Hk, D):
        raise ValueError("key and value must be (q_len, Hk, D) like the query")
    if ss != slot_bytes(D):
        raise ValueError(f"kv_cache slot size {ss} does not match head dim {D} (17*D/16)")
    if cached_len > 0 and (block_row is None or block_row.numel() * bs < cached_len):
        raise ValueError("block_row holds fewer blocks than cached_len needs")
    if out is None:
        out = torch.empty((q_len, Hq, D), dtype=torch.bfloat16, device=query.device)
    _bf16_3d(out, "out")
    lib = _load()
    need = lib.uq_continuation_prefill_workspace_bytes(q_len, int(cached_len) + q_len, Hq, Hk, D)
    if workspace is None:
        workspace = _workspace(query.device, max(int(need), 256))
    fn = lib.uq_continuation_prefill if stages == 3 else (
        lambda *a: lib.uq_continuation_prefill_stages(int(stages), *a))
    _check(fn(
        _ptr(query), _ptr(key), _ptr(value), _ptr(kv_cache), _ptr(block_row), int(cached_len),
        float(scale), _ptr(out), q_len, Hq, Hk, D, nb, bs, query.stride(0), query.stride(1),
        key.stride(0), key.stride(1), value.stride(0), value.stride(1), out.stride(0), out.stride(1),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(query.device)))
    return out
