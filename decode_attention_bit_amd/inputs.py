"""Seeded synthetic workloads for the 4-bit paged-KV decode path.

This module only draws random numbers and lays them out as the decode
interface expects them (bf16 tensors, a shuffled block table, slot indices).
It holds none of the method's arithmetic: no rotation, no quantisation, no
attention. Both the CPU oracle and the HIP library consume exactly the bits
produced here.

Recipe (every workload):
  * ``seed = 1000 + index`` where index is the position of the workload in
    ``WORKLOADS`` (tiny=0, decode=1, ragged=2, long=3, mixed=4).
  * ``default_rng([seed, 0])`` draws, in this order: sequence lengths (where
    random), the permutation of physical blocks, then outlier channels
    (ragged only).
  * ``default_rng([seed, 1])`` draws the query ``(B, Hq, D)``.
  * Keys of sequence ``b``, tokens ``[4096 c, 4096 (c + 1))``, come from
    ``default_rng([seed, 2, b, c])`` and values from
    ``default_rng([seed, 3, b, c])``, each ``(n, Hk, D)``: one stream per
    4096-token chunk lets any part of a sequence be regenerated on its own,
    and lets chunks be drawn in parallel threads.
  * Normal draws are float32, then rounded to bf16 by torch's CPU cast
    (round to nearest even). Student-t draws are float64, cast to float32
    first.
  * Physical blocks: a random permutation of ``sum_b ceil(L_b / 16)`` block
    ids (or of the whole pool for the fixed-length workloads), handed to the
    sequences in order; table entries past a sequence's last block are 0 and
    never read.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np
import torch

HEAD_DIM = 256
BLOCK_SIZE = 16
SLOT_BYTES = 272


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    Hq: int
    Hk: int
    num_kv_splits: int
    seq_len_kind: str            # "fixed", "uniform", "loguniform"
    seq_len_args: tuple
    k_kind: str = "normal"       # "normal", "outlier", "student_t"
    pool_blocks: int | None = None   # fixed pool size (fixed-length workloads)
    table_width: int | None = None
    scale: float = 1.0 / 16.0
    block_size: int = BLOCK_SIZE
    D: int = HEAD_DIM
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def QG(self) -> int:
        return self.Hq // self.Hk

    @property
    def slot_bytes(self) -> int:
        """Cache bytes per (token, KV head): 17 * D / 16."""
        return self.D * 17 // 16


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=2, Hq=8, Hk=1, num_kv_splits=4,
                     seq_len_kind="fixed", seq_len_args=(100, 37),
                     pool_blocks=16, table_width=8),
    "decode": Workload("decode", 1, B=32, Hq=32, Hk=4, num_kv_splits=32,
                       seq_len_kind="fixed", seq_len_args=(4096,) * 32,
                       pool_blocks=8192, table_width=256),
    "ragged": Workload("ragged", 2, B=64, Hq=48, Hk=8, num_kv_splits=32,
                       seq_len_kind="uniform", seq_len_args=(512, 16384),
                       k_kind="outlier", table_width=1024,
                       extra={"outlier_channels": 4, "outlier_gain": 20.0}),
    "long": Workload("long", 3, B=8, Hq=64, Hk=4, num_kv_splits=32,
                     seq_len_kind="fixed", seq_len_args=(131072,) * 8,
                     pool_blocks=65536, table_width=8192),
    "mixed": Workload("mixed", 4, B=256, Hq=32, Hk=4, num_kv_splits=32,
                      seq_len_kind="loguniform", seq_len_args=(1024, 8192),
                      k_kind="student_t", table_width=512,
                      extra={"student_t_dof": 3.0}),
}


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """Round a float32/float64 array to a CPU bf16 tensor (torch RNE cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


@dataclass
class Layout:
    """Paging metadata of one workload instance."""
    seq_lens: np.ndarray      # (B,) int32
    block_table: np.ndarray   # (B, W) int32
    num_blocks: int
    outlier_idx: np.ndarray | None   # (Hk, n) int64 or None


def make_layout(w: Workload, seq_lens: np.ndarray | None = None) -> Layout:
    rng = np.random.default_rng([w.seed, 0])
    if seq_lens is None:
        if w.seq_len_kind == "fixed":
            seq_lens = np.asarray(w.seq_len_args, dtype=np.int64)
        elif w.seq_len_kind == "uniform":
            lo, hi = w.seq_len_args
            seq_lens = rng.integers(lo, hi, size=w.B, endpoint=True)
        elif w.seq_len_kind == "loguniform":
            lo, hi = w.seq_len_args
            seq_lens = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=w.B))).astype(np.int64)
        else:
            raise ValueError(w.seq_len_kind)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    assert seq_lens.shape == (w.B,)
    bs = w.block_size
    nblk = (seq_lens + bs - 1) // bs
    width = w.table_width
    assert int(nblk.max()) <= width
    if w.pool_blocks is not None:
        num_blocks = w.pool_blocks
        perm = rng.permutation(num_blocks)
        assert num_blocks == w.B * width
        table = perm.reshape(w.B, width)
    else:
        num_blocks = int(nblk.sum())
        perm = rng.permutation(num_blocks)
        table = np.zeros((w.B, width), dtype=np.int64)
        off = 0
        for b in range(w.B):
            table[b, : nblk[b]] = perm[off: off + nblk[b]]
            off += int(nblk[b])
    outlier = None
    if w.k_kind == "outlier":
        n = w.extra["outlier_channels"]
        outlier = np.stack([rng.choice(w.D, size=n, replace=False) for _ in range(w.Hk)])
    return Layout(seq_lens.astype(np.int32), table.astype(np.int32), num_blocks, outlier)


def make_query(w: Workload) -> torch.Tensor:
    """(B, Hq, D) bf16 query, N(0, 1)."""
    rng = np.random.default_rng([w.seed, 1])
    return to_bf16(rng.standard_normal((w.B, w.Hq, w.D), dtype=np.float32))


KV_CHUNK = 4096
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


def _kv_chunk(w: Workload, layout: Layout, b: int, c: int, n: int):
    shape = (n, w.Hk, w.D)
    rk = np.random.default_rng([w.seed, 2, b, c])
    if w.k_kind == "student_t":
        k = rk.standard_t(w.extra["student_t_dof"], size=shape).astype(np.float32)
    else:
        k = rk.standard_normal(shape, dtype=np.float32)
        if w.k_kind == "outlier":
            gain = np.float32(w.extra["outlier_gain"])
            for h in range(w.Hk):
                k[:, h, layout.outlier_idx[h]] *= gain
    rv = np.random.default_rng([w.seed, 3, b, c])
    v = rv.standard_normal(shape, dtype=np.float32)
    return k, v


def make_kv(w: Workload, layout: Layout, b: int, t0: int = 0, t1: int | None = None):
    """Keys and values of tokens [t0, t1) of sequence b: two (n, Hk, D) bf16
    CPU tensors (t1 defaults to seq_lens[b])."""
    L = int(layout.seq_lens[b])
    t1 = L if t1 is None else int(t1)
    assert 0 <= t0 <= t1 <= L
    k_out = torch.empty((t1 - t0, w.Hk, w.D), dtype=torch.bfloat16)
    v_out = torch.empty((t1 - t0, w.Hk, w.D), dtype=torch.bfloat16)

    def fill(c):
        lo = c * KV_CHUNK
        k, v = _kv_chunk(w, layout, b, c, min(KV_CHUNK, L - lo))
        a, e = max(t0, lo), min(t1, lo + KV_CHUNK)
        k_out[a - t0:e - t0].copy_(torch.from_numpy(k[a - lo:e - lo]))
        v_out[a - t0:e - t0].copy_(torch.from_numpy(v[a - lo:e - lo]))

    list(_pool().map(fill, range(t0 // KV_CHUNK, (t1 + KV_CHUNK - 1) // KV_CHUNK)))
    return k_out, v_out


def make_kv_tokens(w: Workload, layout: Layout, b: int, tokens: np.ndarray):
    """Keys and values of an arbitrary sorted token subset of sequence b,
    generating only the chunks that hold them."""
    tokens = np.asarray(tokens, dtype=np.int64)
    L = int(layout.seq_lens[b])
    cs = np.unique(tokens // KV_CHUNK)
    parts = dict(zip(cs.tolist(), _pool().map(
        lambda c: _kv_chunk(w, layout, b, c, min(KV_CHUNK, L - c * KV_CHUNK)), cs.tolist())))
    k = np.stack([parts[t // KV_CHUNK][0][t % KV_CHUNK] for t in tokens.tolist()]) if len(tokens) else \
        np.zeros((0, w.Hk, w.D), np.float32)
    v = np.stack([parts[t // KV_CHUNK][1][t % KV_CHUNK] for t in tokens.tolist()]) if len(tokens) else \
        np.zeros((0, w.Hk, w.D), np.float32)
    return to_bf16(k), to_bf16(v)


def slots_for(layout: Layout, b: int, t0: int, t1: int, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Flat cache slots of tokens [t0, t1) of sequence b (int64)."""
    t = np.arange(t0, t1, dtype=np.int64)
    return layout.block_table[b, t // block_size].astype(np.int64) * block_size + t % block_size


def kv_bytes(w: Workload, layout: Layout) -> int:
    """Cache bytes one decode step streams: sum_b L_b * Hk * 17 D / 16."""
    return int(layout.seq_lens.astype(np.int64).sum()) * w.Hk * w.slot_bytes


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a CPU bf16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
