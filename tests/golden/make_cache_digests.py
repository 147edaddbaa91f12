"""Write cache_digests.txt: the SHA-256 of each workload's whole cache as the
oracle stores it.

Calls only the oracle (oracle/uq_oracle.py) and the seeded input generators
(decode_attention_bit_amd/inputs.py); nothing from the HIP library. For every
workload a zeroed (num_blocks, block_size, Hk, 272) uint8 cache receives every
token of every sequence at slot block_table[b, t // 16] * 16 + t % 16 (for the
mixed serving step that includes each sequence's last token, which the step
itself stores). The GPU test stores the same tokens through uq_store into a
zeroed cache and compares the digest of the whole device cache.

Run from the repository root:  python tests/golden/make_cache_digests.py
(about ten minutes on eight cores; the long workload's cache is 1.14 GB).
"""
from __future__ import annotations

import hashlib
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, "1")      # one BLAS thread per worker process

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from decode_attention_bit_amd import inputs  # noqa: E402
from oracle import uq_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cache_digests.txt")
CHUNK = 4096


def _encode(args):
    """Slot bytes (n, Hk, 272) and flat slots of tokens [t0, t1) of sequence b."""
    name, b, t0, t1 = args
    w = inputs.WORKLOADS[name]
    lay = inputs.make_layout(w)
    k, v = inputs.make_kv(w, lay, b, t0, t1)
    return inputs.slots_for(lay, b, t0, t1), O.encode_slots(inputs.bf16_bits(k), inputs.bf16_bits(v))


def cache_digest(name: str, workers: int) -> tuple[str, int]:
    w = inputs.WORKLOADS[name]
    lay = inputs.make_layout(w)
    cache = np.zeros((lay.num_blocks, w.block_size, w.Hk, w.slot_bytes), dtype=np.uint8)
    flat = cache.reshape(-1, w.Hk, w.slot_bytes)
    jobs = [(name, b, t0, min(t0 + CHUNK, int(lay.seq_lens[b])))
            for b in range(w.B) for t0 in range(0, int(lay.seq_lens[b]), CHUNK)]
    with ProcessPoolExecutor(workers) as ex:
        for slots, enc in ex.map(_encode, jobs, chunksize=4):
            flat[slots] = enc
    return hashlib.sha256(cache.tobytes()).hexdigest(), cache.nbytes


def main():
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    lines = ["# SHA-256 of each workload's whole cache as the oracle stores every token of every",
             "# sequence into a zeroed (num_blocks, block_size, Hk, 272) uint8 cache.",
             "# Written by tests/golden/make_cache_digests.py (oracle + seeded inputs only).",
             "# workload cache_bytes sha256"]
    for name in inputs.WORKLOADS:
        t = time.time()
        digest, nbytes = cache_digest(name, workers)
        lines.append(f"{name} {nbytes} {digest}")
        print(f"{name}: {nbytes} bytes, {digest} ({time.time() - t:.0f} s)", flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
