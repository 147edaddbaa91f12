"""Python binding of libuq (4-bit paged-KV decode attention for MI355X).

Argument marshalling only: every step of the store and decode runs in the
HIP kernels of ``libuq.so``. PyTorch provides device memory and the current
stream. Importing the package does not load the library; the first call does,
and raises if the library has not been built (there is no fallback path).

Entry points mirror include/uq.h:
  build_hadamard(D, device)                         -> (D, D) float32
  store(key, value, kv_cache, slot_mapping)         -> None (kv_cache updated)
  decode_workspace_bytes(B, Hq, Hk, num_kv_splits, max_blocks_per_seq, block_size)  -> int
  decode(query, kv_cache, block_table, seq_lens, scale, num_kv_splits,
         out=None, workspace=None)                  -> (B, Hq, 256) bf16
  decode_ex(query, kv_cache, block_table, seq_lens, scale, num_kv_splits,
            query_row=None, sinks=None, sliding_window=0,
            out=None, workspace=None)               -> (B, Hq, 256) bf16
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["build_hadamard", "store", "decode", "decode_ex", "decode_workspace_bytes", "library_path",
           "UQError", "HEAD_DIM", "SLOT_BYTES"]

HEAD_DIM = 256
SLOT_BYTES = 272
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
    """Quantise (N, Hk, 256) bf16 key/value into kv_cache (num_blocks,
    block_size, Hk, 272) uint8 at flat slots slot_mapping (int64, (N,))."""
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


_WS_POOL: dict = {}


def _workspace(device, nbytes: int) -> torch.Tensor:
    """Per-device cached workspace, grown when a bigger one is needed."""
    key = str(device)
    ws = _WS_POOL.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _WS_POOL[key] = ws
    return ws


STAGE_PROLOGUE, STAGE_SPLIT, STAGE_MERGE = 1, 2, 4


def decode(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, scale: float, num_kv_splits: int,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           stages: int = 7) -> torch.Tensor:
    """Split-KV decode over the 4-bit cache; returns (B, Hq, 256) bf16.

    ``stages`` selects a subset of the three kernels (uq_decode_stages); the
    default runs all of them (uq_decode)."""
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
    fn = lib.uq_decode if stages == 7 else (lambda *a: lib.uq_decode_stages(int(stages), *a))
    _check(fn(_ptr(query), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
                             float(scale), int(num_kv_splits), _ptr(out), B, Hq, Hk, D, nb, bs,
                             block_table.shape[1], query.stride(0), query.stride(1),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(query.device)))
    return out


def decode_ex(query: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
              seq_lens: torch.Tensor, scale: float, num_kv_splits: int,
              query_row: torch.Tensor | None = None, sinks: torch.Tensor | None = None,
              sliding_window: int = 0, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """uq_decode_ex: decode with optional per-query table rows (query row b
    reads block-table row query_row[b]), per-head sink logits and a sliding
    window of the last `sliding_window` tokens; returns (B, Hq, 256) bf16."""
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
