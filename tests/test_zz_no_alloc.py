"""uq_decode_no_alloc through the C ABI: the same output as uq_decode, bit for
bit, on two calls in a row (the second with a smaller input, which must not
see the first call's scratch contents) and once more at the larger shape."""
import ctypes

import numpy as np
import pytest
import torch

import decode_attention_bit_amd as uq
from decode_attention_bit_amd import inputs
from oracle import uq_oracle as O
from harness import check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(rng, lens, Hk, qg, D, bs=16, spare=2):
    B, Hq = len(lens), Hk * qg
    nblk = [(L + bs - 1) // bs for L in lens]
    width = max(nblk) + spare
    nb = sum(nblk) + 3
    table = np.zeros((B, width), dtype=np.int32)
    perm, off = rng.permutation(nb), 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    slot = D * 17 // 16
    cache = torch.zeros((nb, bs, Hk, slot), dtype=torch.uint8, device=DEV)
    ref_cache = np.zeros((nb, bs, Hk, slot), dtype=np.uint8)
    for b, L in enumerate(lens):
        k = inputs.to_bf16(rng.standard_normal((L, Hk, D)).astype(np.float32))
        v = inputs.to_bf16(rng.standard_normal((L, Hk, D)).astype(np.float32))
        t = np.arange(L)
        slots = table[b, t // bs].astype(np.int64) * bs + t % bs
        uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(inputs.bf16_bits(k), inputs.bf16_bits(v), ref_cache, slots)
    q = inputs.to_bf16(rng.standard_normal((B, Hq, D)).astype(np.float32))
    return dict(q=q.to(DEV), qb=inputs.bf16_bits(q), cache=cache, ref_cache=ref_cache,
                table=torch.from_numpy(table).to(DEV), np_table=table,
                lens=torch.tensor(lens, dtype=torch.int32, device=DEV), np_lens=np.array(lens),
                Hk=Hk, D=D, scale=1 / np.sqrt(D))


def _no_alloc(c, splits):
    """One uq_decode_no_alloc call through ctypes on the current stream."""
    lib = uq._load()
    q, cache, table = c["q"], c["cache"], c["table"]
    B, Hq, D = q.shape
    nb, bs, Hk, _ = cache.shape
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    rc = lib.uq_decode_no_alloc(q.data_ptr(), cache.data_ptr(), table.data_ptr(), c["lens"].data_ptr(),
                                ctypes.c_float(c["scale"]), splits, out.data_ptr(), B, Hq, Hk, D, nb, bs,
                                table.shape[1], q.stride(0), q.stride(1),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.uq_last_error().decode()
    return out


def test_decode_no_alloc_matches_decode():
    rng = np.random.default_rng(2024)
    big = _case(rng, [3000, 1800, 4096, 2500, 700, 3333], Hk=4, qg=8, D=256)
    small = _case(rng, [100, 37, 16], Hk=2, qg=6, D=128)
    for name, c, splits in (("big", big, 32), ("small", small, 4), ("big again", big, 8)):
        print(f"no-alloc decode: {name}", flush=True)
        got = _no_alloc(c, splits)
        want = uq.decode(c["q"], c["cache"], c["table"], c["lens"], c["scale"], splits)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{name}: differs from uq_decode"
        ref = O.decode(c["qb"], c["ref_cache"], c["np_table"], c["np_lens"], c["scale"])
        check_close(to_np(got), ref, f"no-alloc {name}")
