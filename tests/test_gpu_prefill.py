"""GPU parity of the continuation-prefill path against the CPU oracle:
rotation and dequantisation bit for bit, attention within max-abs 1e-2 /
rel-L2 5e-3. Everything goes through the C ABI."""
import numpy as np
import pytest
import torch

from harness import check_close, to_np
import decode_attention_bit_amd as uq
from decode_attention_bit_amd import inputs
from oracle import uq_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def bf16(x):
    return inputs.to_bf16(np.asarray(x, dtype=np.float32))


def bits(t):
    return inputs.bf16_bits(t.cpu())


def value_bits(x):
    """bf16 bit patterns of float64 values that bf16 represents exactly
    (values past bf16's range become infinities)."""
    with np.errstate(over="ignore"):
        return inputs.bf16_bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def same_bf16(got_bits, want_values, what):
    """Bit-equal, except that the sign of an exact zero is not compared."""
    want = value_bits(want_values)
    zero = np.asarray(want_values) == 0
    bad = (got_bits != want) & ~(zero & ((got_bits & 0x7FFF) == 0))
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} differ, first at {np.argwhere(bad)[:3].tolist()}"


def stored_sequence(rng, n, hk, bs=16, k_scale=None, extra_blocks=3):
    """A cache holding one sequence of n tokens in shuffled blocks (GPU store)
    and the oracle's copy of it."""
    nblk = max(1, -(-n // bs))
    row = rng.permutation(nblk + extra_blocks)[:nblk].astype(np.int32)
    cache = torch.zeros((nblk + extra_blocks, bs, hk, 272), dtype=torch.uint8, device=DEV)
    ref = np.zeros(tuple(cache.shape), dtype=np.uint8)
    if n:
        k = rng.standard_normal((n, hk, 256))
        if k_scale is not None:
            k = k * k_scale
        kb = bf16(k)
        vb = bf16(rng.standard_t(4, (n, hk, 256)))
        t = np.arange(n)
        slots = row[t // bs].astype(np.int64) * bs + t % bs
        uq.store(kb.to(DEV), vb.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(bits(kb), bits(vb), ref, slots)
    return cache, ref, row


# ------------------------------------------------------------------ rotation
def test_rotate_bit_exact():
    """bf16(x H) with one rounding: Gaussian rows, wide-range rows (26
    binades), rows whose rotation lands on bf16 ties, zeros and subnormals."""
    say("rotate")
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 3, 256))
    x[0] = 0.0
    x[1, 0] = np.ldexp(rng.uniform(0.5, 1, 256), -130)                  # bf16 subnormals
    for i in range(2, 8):
        x[i] = rng.choice([-1, 1], (3, 256)) * (1 + rng.random((3, 256))) * np.exp2(rng.integers(-13, 13, (3, 256)))
    x[8] = np.eye(256)[rng.integers(256, size=3)] * (1 + 2.0 ** -7)     # +-(1 + 2^-7)/16: exact
    x[9, :, :2] = [1.0, 2.0 ** -8]                                      # rotations land on ties
    x[10] = rng.standard_normal((3, 256)) * 1e30
    xb = bf16(x)
    out = uq.rotate(xb.to(DEV))
    same_bf16(bits(out), O.rotate_to_bf16(bits(xb)), "rotate")
    # strided views, written in place
    big = torch.zeros((40, 3, 512), dtype=torch.bfloat16, device=DEV)
    big[:, :, 128:384] = xb.to(DEV)
    view = big[:, :, 128:384]
    uq.rotate(view, out=view)
    same_bf16(bits(view), O.rotate_to_bf16(bits(xb)), "rotate in place")
    assert torch.all(big[:, :, :128] == 0) and torch.all(big[:, :, 384:] == 0)


# ------------------------------------------------------------------- dequant
@pytest.mark.parametrize("bs", [16, 64])
def test_dequant_bit_exact(bs):
    """Dequantised prefix equals the oracle's values bit for bit, in the
    token-major layout and in the page's (Hk, n, 256) layout; blocks of
    tiny values exercise scales near 2**-127 (bf16 subnormal results)."""
    say(f"dequant bs={bs}")
    rng = np.random.default_rng(bs)
    n, hk = 3 * bs + 5, 3
    cache, ref, row = stored_sequence(rng, n, hk, bs=bs)
    # a few slots with extreme scale bytes and every code, written directly
    slot = ref[row[0], 1, 0].copy()
    slot[:128] = np.arange(128, dtype=np.uint8) * 2 + 1
    slot[128:256] = 255 - np.arange(128, dtype=np.uint8)
    slot[256:272] = [0, 1, 2, 3, 127, 200, 252, 254, 0, 5, 60, 126, 128, 130, 160, 250]
    ref[row[0], 1, 0] = slot
    cache[int(row[0]), 1, 0] = torch.from_numpy(slot).to(DEV)
    K, V = O.dequant_prefix(ref, row, n)
    brow = torch.from_numpy(row).to(DEV)
    k, v = uq.dequant_kv(cache, brow, n)
    same_bf16(bits(k), K, "K")
    same_bf16(bits(v), V, "V")
    assert np.signbit(to_np(v))[V == 0].tolist() == np.signbit(V)[V == 0].tolist()
    kh = torch.empty((hk, n, 256), dtype=torch.bfloat16, device=DEV)
    vh = torch.empty((hk, n, 256), dtype=torch.bfloat16, device=DEV)
    uq.dequant_kv(cache, brow, n, k_out=kh.transpose(0, 1), v_out=vh.transpose(0, 1))
    assert torch.equal(kh.transpose(0, 1), k) and torch.equal(vh.transpose(0, 1), v)
    # a block entry outside the cache reads as zeros
    bad = brow.clone()
    bad[1] = cache.shape[0]
    k2, v2 = uq.dequant_kv(cache, bad, n)
    assert torch.all(k2[bs:2 * bs] == 0) and torch.all(v2[bs:2 * bs] == 0)
    assert torch.equal(k2[:bs], k[:bs]) and torch.equal(k2[2 * bs:], k[2 * bs:])


# ----------------------------------------------------------------- attention
def _prefill_case(rng, cached_len, q_len, hk, qg, bs=16, scale=1 / 16):
    cache, ref, row = stored_sequence(rng, cached_len, hk, bs=bs)
    q = bf16(rng.standard_normal((q_len, hk * qg, 256)))
    kc = bf16(rng.standard_normal((q_len, hk, 256)))
    vc = bf16(rng.standard_t(4, (q_len, hk, 256)))
    brow = torch.from_numpy(row).to(DEV)
    out = uq.continuation_prefill(q.to(DEV), kc.to(DEV), vc.to(DEV), cache, brow, cached_len, scale)
    return out, dict(q=q, kc=kc, vc=vc, ref=ref, row=row, cache=cache, brow=brow, scale=scale)


@pytest.mark.parametrize("qg", [1, 2, 6, 8, 16])
@pytest.mark.parametrize("cached_len,q_len", [(0, 1), (0, 37), (5, 16), (64, 17), (203, 129)])
def test_continuation_prefill_vs_oracle(qg, cached_len, q_len):
    say(f"prefill qg={qg} cached={cached_len} q_len={q_len}")
    rng = np.random.default_rng(qg * 1000 + cached_len + q_len)
    hk = 2
    out, c = _prefill_case(rng, cached_len, q_len, hk, qg)
    want = O.continuation_prefill(bits(c["q"]), bits(c["kc"]), bits(c["vc"]), c["ref"], c["row"],
                                  cached_len, c["scale"])
    # heavy-tailed values: outputs reach |o| >= 4, where bf16 rounding alone is 1/64
    check_close(to_np(out), want, f"prefill qg={qg} cached={cached_len} q_len={q_len}",
                allow_output_rounding=True)


@pytest.mark.parametrize("cached_len,q_len", [(64, 32), (31, 1), (32, 32), (96, 64)])
def test_continuation_prefill_whole_tiles(cached_len, q_len):
    """Sequences that end exactly on a 32-key value tile (no zero keys pad
    the last tile), including a one-token chunk after a 31-token prefix."""
    say(f"prefill whole tiles cached={cached_len} q_len={q_len}")
    rng = np.random.default_rng(5000 + cached_len + q_len)
    out, c = _prefill_case(rng, cached_len, q_len, 2, 8)
    want = O.continuation_prefill(bits(c["q"]), bits(c["kc"]), bits(c["vc"]), c["ref"], c["row"],
                                  cached_len, c["scale"])
    check_close(to_np(out), want, f"whole tiles cached={cached_len} q_len={q_len}",
                allow_output_rounding=True)


def _block_scaled_values(rng, n, hk, d, chunk):
    """Values whose 32-dim blocks differ in magnitude by up to 2^100:
    heavy-tailed t(4) values times a per-(head, block) power of two, with the
    chunk's values 2^20 below or above the prefix's in two blocks, and
    blocks of constant values (+-2^40, +-2^10 by dim), far outside fp16's
    range, whose outputs are exact. Block b follows entry b % 8 of each
    head's pattern."""
    v = rng.standard_t(4, (n, hk, d))
    pattern = [[0, -20, "c40", -20 if chunk else 0, 0 if chunk else -20, "c10", 0, -60],
               [0, 0, 0, -100, 0, 0, -2, 0]]
    sign = np.where(np.arange(32) % 3 == 0, -1.0, 1.0)
    for h in range(hk):
        for b in range(d // 32):
            e = pattern[h % 2][b % 8]
            if e == "c40":
                v[:, h, 32 * b:32 * b + 32] = np.exp2(40) * sign
            elif e == "c10":
                v[:, h, 32 * b:32 * b + 32] = -np.exp2(10) * sign
            else:
                v[:, h, 32 * b:32 * b + 32] *= np.exp2(e)
    return bf16(v)


@pytest.mark.parametrize("d", [128, 256, 512])
def test_continuation_prefill_value_block_scales(d):
    """The value tiles hold fp16 values scaled by a power of two per (KV
    head, 32-dim block), from the largest exponent over prefix and chunk:
    blocks of very different magnitudes, blocks where the chunk's values are
    2^20 above or below the prefix's, and blocks far outside fp16's range
    all match the oracle."""
    say(f"prefill value block scales d={d}")
    rng = np.random.default_rng(23 + d)
    cached_len, q_len, hk, qg, bs = 100, 45, 2, 4, 16
    nblk = -(-cached_len // bs)
    row = rng.permutation(nblk + 2)[:nblk].astype(np.int32)
    cache = torch.zeros((nblk + 2, bs, hk, d * 17 // 16), dtype=torch.uint8, device=DEV)
    ref = np.zeros(tuple(cache.shape), dtype=np.uint8)
    kb = bf16(rng.standard_normal((cached_len, hk, d)))
    vb = _block_scaled_values(rng, cached_len, hk, d, chunk=False)
    t = np.arange(cached_len)
    slots = row[t // bs].astype(np.int64) * bs + t % bs
    uq.store(kb.to(DEV), vb.to(DEV), cache, torch.from_numpy(slots).to(DEV))
    O.store(bits(kb), bits(vb), ref, slots)
    q = bf16(rng.standard_normal((q_len, hk * qg, d)))
    kc = bf16(rng.standard_normal((q_len, hk, d)))
    vc = _block_scaled_values(rng, q_len, hk, d, chunk=True)
    out = uq.continuation_prefill(q.to(DEV), kc.to(DEV), vc.to(DEV), cache, torch.from_numpy(row).to(DEV),
                                  cached_len, 1 / 16)
    want = O.continuation_prefill(bits(q), bits(kc), bits(vc), ref, row, cached_len, 1 / 16)
    check_close(to_np(out), want, f"value block scales d={d}", allow_output_rounding=True)


def test_continuation_prefill_block_outside_cache_reads_zeros():
    """A prefix block entry past the cache reads as zero keys and values (as
    in uq_dequant_kv): the same as the oracle over an all-zero block."""
    say("prefill block outside the cache")
    rng = np.random.default_rng(17)
    cached_len, q_len, hk, qg = 70, 20, 2, 8
    cache, ref, row = stored_sequence(rng, cached_len, hk)
    spare = int(np.setdiff1d(np.arange(cache.shape[0]), row)[0])   # never written: all zero
    assert not ref[spare].any()
    bad = row.copy()
    bad[1] = cache.shape[0]
    q = bf16(rng.standard_normal((q_len, hk * qg, 256)))
    kc = bf16(rng.standard_normal((q_len, hk, 256)))
    vc = bf16(rng.standard_t(4, (q_len, hk, 256)))
    out = uq.continuation_prefill(q.to(DEV), kc.to(DEV), vc.to(DEV), cache, torch.from_numpy(bad).to(DEV),
                                  cached_len, 1 / 16)
    zrow = row.copy()
    zrow[1] = spare
    want = O.continuation_prefill(bits(q), bits(kc), bits(vc), ref, zrow, cached_len, 1 / 16)
    check_close(to_np(out), want, "block outside the cache", allow_output_rounding=True)


def test_prefill_attention_strided_and_peaked():
    """The attention call on its own over strided views, with a large scale
    (peaked weights that raise the running maximum along the keys)."""
    say("prefill attention strided")
    rng = np.random.default_rng(3)
    q_len, seq, hk, qg = 50, 300, 2, 8
    grow = np.linspace(0.2, 4.0, seq)[:, None, None]
    k = bf16(rng.standard_normal((seq, hk, 256)) * grow)
    v = bf16(rng.standard_normal((seq, hk, 256)))
    q = bf16(rng.standard_normal((q_len, hk * qg, 256)))
    kv = torch.zeros((seq, 2, hk, 264), dtype=torch.bfloat16, device=DEV)
    kv[:, 0, :, :256] = k.to(DEV)
    kv[:, 1, :, :256] = v.to(DEV)
    qq = torch.zeros((q_len, hk * qg, 384), dtype=torch.bfloat16, device=DEV)
    qq[:, :, 128:] = q.to(DEV)
    o = torch.full((q_len, hk * qg, 264), float("nan"), dtype=torch.bfloat16, device=DEV)
    uq.prefill_attention(qq[:, :, 128:], kv[:, 0, :, :256], kv[:, 1, :, :256], 0.5, out=o[:, :, :256])
    K, V = O.bf16_to_f64(bits(k)), O.bf16_to_f64(bits(v))
    Q = O.bf16_to_f64(bits(q))
    want = np.zeros((q_len, hk * qg, 256))
    for hq in range(hk * qg):
        s = 0.5 * Q[:, hq] @ K[:, hq // qg].T
        s = np.where(np.arange(seq)[None, :] <= seq - q_len + np.arange(q_len)[:, None], s, -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        want[:, hq] = p @ V[:, hq // qg] / p.sum(-1, keepdims=True)
    check_close(to_np(o[:, :, :256]), want, "strided peaked", allow_output_rounding=True)
    assert torch.isnan(o[:, :, 256:]).all()


def test_continuation_prefill_large_sampled_rows():
    """A 4096-token prefix and a 1024-token chunk (GQA 8, Hk 4); the oracle
    computes 12 sampled chunk positions, including the first and last."""
    say("prefill large sampled")
    rng = np.random.default_rng(11)
    cached_len, q_len, hk, qg = 4096, 1024, 4, 8
    out, c = _prefill_case(rng, cached_len, q_len, hk, qg)
    rows = np.unique(np.concatenate([[0, 1, q_len - 1], rng.integers(0, q_len, 9)]))
    want = O.continuation_prefill(bits(c["q"]), bits(c["kc"]), bits(c["vc"]), c["ref"], c["row"],
                                  cached_len, c["scale"], rows=rows)
    check_close(to_np(out)[rows], want[rows], "large sampled rows", allow_output_rounding=True)


def test_continuation_prefill_stages_compose():
    """The gather launch and the attention launch run one after the other
    give the whole call's output bit for bit."""
    say("prefill stages")
    rng = np.random.default_rng(13)
    out1, c = _prefill_case(rng, 77, 40, 2, 8)
    ws = torch.empty(uq.continuation_prefill_workspace_bytes(40, 117, 16, 2), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(out1)
    for st in (uq.PREFILL_GATHER, uq.PREFILL_ATTEND):
        uq.continuation_prefill(c["q"].to(DEV), c["kc"].to(DEV), c["vc"].to(DEV), c["cache"], c["brow"], 77,
                                c["scale"], out=o, workspace=ws, stages=st)
    assert torch.equal(o, out1)


def test_continuation_prefill_reuses_workspace_and_empty_chunk():
    say("prefill workspace reuse")
    rng = np.random.default_rng(12)
    out1, c1 = _prefill_case(rng, 100, 30, 2, 8)
    ws = torch.empty(uq.continuation_prefill_workspace_bytes(64, 1000, 16, 2), dtype=torch.uint8, device=DEV)
    again = uq.continuation_prefill(c1["q"].to(DEV), c1["kc"].to(DEV), c1["vc"].to(DEV), c1["cache"],
                                    c1["brow"], 100, c1["scale"], workspace=ws)
    assert torch.equal(again, out1)
    empty = uq.continuation_prefill(c1["q"][:0].to(DEV), c1["kc"][:0].to(DEV), c1["vc"][:0].to(DEV),
                                    c1["cache"], c1["brow"], 100, c1["scale"])
    assert empty.shape == (0, 16, 256)
