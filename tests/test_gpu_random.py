"""Decode on random shapes against the oracle: head dims 128, 256, 512,
GQA 6, 8, 16, 1 to 8 KV heads (odd counts included), block sizes 16 to
256, 1 to 512 splits, ragged lengths with empty sequences and spare table
width, sliding windows, sinks, a few outlier key channels. Cache bytes
bit-exact; outputs within max-abs 1e-2 (plus half a bf16 ulp of the
reference only where |o| >= 4, where rounding the exact answer to bf16
alone can exceed 1e-2) and rel-L2 5e-3. UQ_RANDOM_CASES sets the number of
shapes (24 by default; a sweep of 180 was run as well)."""
import os

import numpy as np
import pytest
import torch

import decode_attention_bit_amd as uq
from decode_attention_bit_amd import inputs
from harness import check_close, to_np
from oracle import uq_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bf16(x):
    return inputs.to_bf16(np.asarray(x, dtype=np.float32))


def bits(t):
    return inputs.bf16_bits(t.cpu())


def _case(rng):
    D = int(rng.choice([128, 256, 256, 512]))
    qg = int(rng.choice([6, 8, 16]))
    Hk = int(rng.choice([1, 2, 3, 4, 8]))
    bs = int(rng.choice([16, 32, 64, 256]))
    B = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(0, 700, B)]
    if rng.random() < 0.3:
        lens[0] = int(rng.integers(700, 2500))
    return dict(D=D, qg=qg, Hk=Hk, bs=bs, lens=lens, S=int(rng.choice([1, 2, 3, 7, 32, 64, 512])),
                window=int(rng.choice([0, 0, 1, 17, 100, 1000])), sinks=bool(rng.random() < 0.4),
                scale=float(rng.choice([1 / 16, 0.1, 0.3])))


@pytest.mark.parametrize("seed", range(int(os.environ.get("UQ_RANDOM_CASES", "24"))))
def test_decode_random_shape(seed):
    rng = np.random.default_rng(5000 + seed)
    c = _case(rng)
    print(f"random decode {seed}: {c}", flush=True)
    D, qg, Hk, bs, lens = c["D"], c["qg"], c["Hk"], c["bs"], c["lens"]
    B, Hq = len(lens), Hk * qg
    nblk = [(L + bs - 1) // bs for L in lens]
    width = max(max(nblk), 1) + int(rng.integers(0, 3))
    nb = sum(nblk) + 2
    table = np.zeros((B, width), dtype=np.int32)
    perm, off = rng.permutation(nb), 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    slot = D * 17 // 16
    cache = torch.zeros((nb, bs, Hk, slot), dtype=torch.uint8, device=DEV)
    ref_cache = np.zeros((nb, bs, Hk, slot), dtype=np.uint8)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        k = bf16(rng.standard_normal((L, Hk, D)) * (1 + 30 * (rng.random((1, 1, D)) < 0.02)))
        v = bf16(rng.standard_normal((L, Hk, D)))
        t = np.arange(L)
        slots = table[b, t // bs].astype(np.int64) * bs + t % bs
        uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(bits(k), bits(v), ref_cache, slots)
    q = bf16(rng.standard_normal((B, Hq, D)))
    sinks = rng.normal(0, 2, Hq).astype(np.float32) if c["sinks"] else None
    tbl = torch.from_numpy(table).to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = uq.decode_ex(q.to(DEV), cache, tbl, sl, c["scale"], c["S"],
                       sinks=None if sinks is None else torch.from_numpy(sinks).to(DEV),
                       sliding_window=c["window"])
    ref = O.decode(bits(q), ref_cache, table, np.array(lens), c["scale"],
                   sinks=None if sinks is None else sinks.astype(np.float64), sliding_window=c["window"])
    assert np.array_equal(cache.cpu().numpy(), ref_cache), "cache bytes differ"
    check_close(to_np(out), ref, f"random decode {seed}", allow_output_rounding=True)
