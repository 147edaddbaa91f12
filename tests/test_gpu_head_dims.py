"""Head dims 128 and 512 (the pages' other head sizes): the slot format
scales with D (17 D / 16 bytes), the store and the continuation-prefill
operands (rotation, dequantised prefix) are bit-exact against the oracle,
and decode and the continuation-prefill attention are within max-abs 1e-2 /
rel-L2 5e-3. Through the C ABI."""
import numpy as np
import pytest
import torch

from harness import check_close, to_np
import decode_attention_bit_amd as uq
from decode_attention_bit_amd import inputs
from oracle import uq_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"
DIMS = [128, 512]


def say(msg):
    print(msg, flush=True)


def bf16(x):
    return inputs.to_bf16(np.asarray(x, dtype=np.float32))


def bits(t):
    return inputs.bf16_bits(t.cpu())


def slot(d):
    return O.slot_layout(d)[0]


@pytest.mark.parametrize("d", DIMS)
def test_store_bit_exact(d):
    say(f"store d={d}")
    rng = np.random.default_rng(d)
    n, hk, bs = 70, 3, 16
    k = rng.standard_normal((n, hk, d))
    v = rng.standard_t(3, (n, hk, d))
    k[0] = 0.0
    v[1] = -0.0
    k[2, :, :] = 0
    k[2, 0, :2] = [1.0, 1.0]                               # rotated: exact zeros on odd indices
    v[3] = np.ldexp(rng.uniform(0.5, 1, (hk, d)), -130)    # bf16 subnormals, scale clamps
    v[25] = np.ldexp(rng.uniform(1, 4, (hk, d)) * rng.choice([-1, 1], (hk, d)), -128)  # codes 1 to 4, byte 0
    k[4] = rng.standard_normal((hk, d)) * 1e30
    for i in range(5, 15):                                  # magnitudes over 24 binades
        k[i] = np.ldexp(rng.uniform(0.5, 1, (hk, d)) * rng.choice([-1, 1], (hk, d)),
                        rng.integers(-12, 12, (hk, d)))
    for i in range(15, 25):                                 # values on E2M1 midpoints
        v[i] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -5.0], (hk, d))
    kb, vb = bf16(k), bf16(v)
    nb = 8
    slots = rng.permutation(nb * bs)[:n]
    cache = torch.full((nb, bs, hk, slot(d)), 0xA5, dtype=torch.uint8, device=DEV)
    uq.store(kb.to(DEV), vb.to(DEV), cache, torch.from_numpy(slots).to(DEV))
    ref = np.full(tuple(cache.shape), 0xA5, dtype=np.uint8)
    O.store(bits(kb), bits(vb), ref, slots)
    bad = np.argwhere(cache.cpu().numpy() != ref)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("qg", [6, 8, 16])
@pytest.mark.parametrize("d", DIMS)
def test_query_prologue_codes_bit_exact(d, qg):
    say(f"prologue d={d} qg={qg}")
    rng = np.random.default_rng(d + 1)
    B, hk = 2, 2
    q = rng.standard_normal((B, hk * qg, d))
    q[0, 0] = 0.0
    q[0, 1] = rng.standard_normal(d) * 2.0 ** -20
    q[0, 2] = rng.standard_normal(d) * 300.0
    q[1, 0] = rng.choice([-1.0, 1.0], d) * (1 + rng.random(d)) * np.exp2(rng.integers(-12, 13, d))
    qb = bf16(q)
    cache = torch.zeros((1, 16, hk, slot(d)), dtype=torch.uint8, device=DEV)
    ws = torch.full((uq.decode_workspace_bytes(B, hk * qg, hk, 1, 1, 16, d),), 0x55, dtype=torch.uint8, device=DEV)
    uq.decode(qb.to(DEV), cache, torch.zeros((B, 1), dtype=torch.int32, device=DEV),
              torch.ones(B, dtype=torch.int32, device=DEV), 1 / 16, 1, workspace=ws, stages=uq.STAGE_PROLOGUE)
    got = ws[:B * hk * qg * d].cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(B, hk * qg, d)
    ref = O.query_haircut(bits(qb))
    assert np.array_equal(got, ref), f"{(got != ref).sum()} codes differ"


def _decode_case(d, seq_lens, hk, qg, bs=16, splits=3, seed=0, scale=None):
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    nblk = [(L + bs - 1) // bs for L in seq_lens]
    width = max(max(nblk), 1)
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    table = np.zeros((B, width), dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    q = bf16(rng.standard_normal((B, hk * qg, d)))
    cache = torch.zeros((nb, bs, hk, slot(d)), dtype=torch.uint8, device=DEV)
    ref_cache = np.zeros(tuple(cache.shape), dtype=np.uint8)
    for b, L in enumerate(seq_lens):
        if L == 0:
            continue
        k = bf16(rng.standard_normal((L, hk, d)))
        v = bf16(rng.standard_normal((L, hk, d)))
        t = np.arange(L)
        slots = table[b, t // bs].astype(np.int64) * bs + t % bs
        uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(bits(k), bits(v), ref_cache, slots)
    scale = scale if scale is not None else 1 / np.sqrt(d)
    out = uq.decode(q.to(DEV), cache, torch.from_numpy(table).to(DEV),
                    torch.tensor(seq_lens, dtype=torch.int32, device=DEV), scale, splits)
    ref = O.decode(bits(q), ref_cache, table, np.array(seq_lens), scale)
    return out, ref


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("qg", [6, 8, 16])
@pytest.mark.parametrize("bs", [16, 64, 256])
def test_decode_ragged(d, qg, bs):
    say(f"decode d={d} qg={qg} bs={bs}")
    lens = [1, 15, 16, 17, 100, 257, 300, 0, 33]
    out, ref = _decode_case(d, lens, hk=2, qg=qg, bs=bs, seed=d + qg + bs)
    check_close(to_np(out), ref, f"d={d} qg={qg} bs={bs}")


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("hk", [1, 3, 8])
def test_decode_head_counts(d, hk):
    """KV head counts that give stage 1 one head per workgroup (1, and the
    odd 3) or four heads per workgroup (8)."""
    say(f"decode d={d} hk={hk}")
    lens = [700, 5, 16, 129]
    for qg in (6, 8):
        out, ref = _decode_case(d, lens, hk=hk, qg=qg, splits=4, seed=40 + hk + qg)
        check_close(to_np(out), ref, f"d={d} hk={hk} qg={qg}")


@pytest.mark.parametrize("d", DIMS)
def test_decode_long_split_invariance(d):
    """One long sequence per KV head group at several split counts, against
    the single-softmax oracle; 512 splits (the maximum) leave most partials
    empty and give the merge four waves per row."""
    say(f"decode long d={d}")
    lens = [3000, 1234]
    for splits in (1, 8, 32, 512):
        out, ref = _decode_case(d, lens, hk=4, qg=8, splits=splits, seed=d + 7)
        check_close(to_np(out), ref, f"d={d} splits={splits}")


@pytest.mark.parametrize("d", DIMS)
def test_decode_ex_window_and_sinks(d):
    say(f"decode_ex d={d}")
    rng = np.random.default_rng(d + 9)
    B, hk, qg, bs = 3, 2, 8, 16
    lens = [200, 31, 90]
    nb = sum((L + bs - 1) // bs for L in lens) + 2
    table = np.zeros((B, 13), dtype=np.int32)
    perm = rng.permutation(nb)
    off = 0
    cache = torch.zeros((nb, bs, hk, slot(d)), dtype=torch.uint8, device=DEV)
    ref_cache = np.zeros(tuple(cache.shape), dtype=np.uint8)
    for b, L in enumerate(lens):
        n = (L + bs - 1) // bs
        table[b, :n] = perm[off:off + n]
        off += n
        k, v = bf16(rng.standard_normal((L, hk, d))), bf16(rng.standard_normal((L, hk, d)))
        t = np.arange(L)
        slots = table[b, t // bs].astype(np.int64) * bs + t % bs
        uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(bits(k), bits(v), ref_cache, slots)
    q = bf16(rng.standard_normal((B, hk * qg, d)))
    sinks = rng.normal(0, 2, hk * qg).astype(np.float32)
    out = uq.decode_ex(q.to(DEV), cache, torch.from_numpy(table).to(DEV),
                       torch.tensor(lens, dtype=torch.int32, device=DEV), 0.1, 4,
                       sinks=torch.from_numpy(sinks).to(DEV), sliding_window=50)
    ref = O.decode(bits(q), ref_cache, table, np.array(lens), 0.1, sinks=sinks, sliding_window=50)
    check_close(to_np(out), ref, f"decode_ex d={d}")


# --------------------------------------------- continuation-prefill operands
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


@pytest.mark.parametrize("d", DIMS)
def test_rotate_bit_exact(d):
    """bf16(x H) at head dim d: the exact +-1 sums times the float64 nearest
    1/sqrt(d), rounded once. Gaussian rows, rows over 24 binades, one-hot
    rows (every output is +-1/sqrt(d) rounded), bf16 subnormals, zeros,
    huge values; then a strided view rotated in place."""
    say(f"rotate d={d}")
    rng = np.random.default_rng(d + 7)
    x = rng.standard_normal((33, 3, d))
    x[0] = 0.0
    x[1, 0] = np.ldexp(rng.uniform(0.5, 1, d), -130)
    for i in range(2, 8):
        x[i] = rng.choice([-1, 1], (3, d)) * (1 + rng.random((3, d))) * np.exp2(rng.integers(-12, 12, (3, d)))
    x[8] = np.eye(d)[rng.integers(d, size=3)]
    x[9] = rng.standard_normal((3, d)) * 1e30
    xb = bf16(x)
    want = O.rotate_to_bf16(bits(xb))
    out = uq.rotate(xb.to(DEV))
    same_bf16(bits(out), want, "rotate")
    big = torch.zeros((33, 3, 2 * d), dtype=torch.bfloat16, device=DEV)
    big[:, :, d // 2:d // 2 + d] = xb.to(DEV)
    view = big[:, :, d // 2:d // 2 + d]
    uq.rotate(view, out=view)
    same_bf16(bits(view), want, "rotate in place")
    assert torch.all(big[:, :, :d // 2] == 0) and torch.all(big[:, :, d // 2 + d:] == 0)


@pytest.mark.parametrize("d", DIMS)
def test_dequant_bit_exact(d):
    """Dequantised prefix at head dim d equals the oracle's values bit for
    bit, token-major and in the page's (Hk, n, d) layout; one slot holds
    every code and extreme scale bytes (bf16 subnormals and infinities); a
    block entry outside the cache reads as zeros."""
    say(f"dequant d={d}")
    rng = np.random.default_rng(d + 9)
    n, hk, bs, extra = 3 * 16 + 5, 3, 16, 3
    nblk = -(-n // bs)
    row = rng.permutation(nblk + extra)[:nblk].astype(np.int32)
    cache = torch.zeros((nblk + extra, bs, hk, slot(d)), dtype=torch.uint8, device=DEV)
    ref = np.zeros(tuple(cache.shape), dtype=np.uint8)
    kb = bf16(rng.standard_normal((n, hk, d)))
    vb = bf16(rng.standard_t(4, (n, hk, d)))
    t = np.arange(n)
    slots = row[t // bs].astype(np.int64) * bs + t % bs
    uq.store(kb.to(DEV), vb.to(DEV), cache, torch.from_numpy(slots).to(DEV))
    O.store(bits(kb), bits(vb), ref, slots)
    s = ref[row[0], 1, 0].copy()
    s[:d] = (np.arange(d) * 37 + 1) % 256
    s[d:] = np.resize(np.array([0, 1, 2, 3, 127, 200, 252, 254, 0, 5, 60, 126, 128, 130, 160, 250]), d // 16)
    ref[row[0], 1, 0] = s
    cache[int(row[0]), 1, 0] = torch.from_numpy(s).to(DEV)
    K, V = O.dequant_prefix(ref, row, n)
    brow = torch.from_numpy(row).to(DEV)
    k, v = uq.dequant_kv(cache, brow, n)
    assert tuple(k.shape) == (n, hk, d)
    same_bf16(bits(k), K, "K")
    same_bf16(bits(v), V, "V")
    assert np.signbit(to_np(v))[V == 0].tolist() == np.signbit(V)[V == 0].tolist()
    kh = torch.empty((hk, n, d), dtype=torch.bfloat16, device=DEV)
    vh = torch.empty((hk, n, d), dtype=torch.bfloat16, device=DEV)
    uq.dequant_kv(cache, brow, n, k_out=kh.transpose(0, 1), v_out=vh.transpose(0, 1))
    assert torch.equal(kh.transpose(0, 1), k) and torch.equal(vh.transpose(0, 1), v)
    bad = brow.clone()
    bad[1] = cache.shape[0]
    k2, v2 = uq.dequant_kv(cache, bad, n)
    assert torch.all(k2[bs:2 * bs] == 0) and torch.all(v2[bs:2 * bs] == 0)
    assert torch.equal(k2[:bs], k[:bs]) and torch.equal(k2[2 * bs:], k[2 * bs:])


@pytest.mark.parametrize("cached_len,q_len,qg", [(0, 37, 6), (100, 64, 6), (333, 129, 6), (32, 32, 6),
                                                  (0, 37, 8), (100, 64, 8), (333, 129, 8), (32, 32, 8),
                                                  (0, 37, 16), (100, 64, 16), (333, 129, 16), (32, 32, 16),
                                                  (45, 70, 1), (45, 70, 64)])
@pytest.mark.parametrize("d", DIMS)
def test_continuation_prefill(d, cached_len, q_len, qg):
    """Continuation prefill at head dim d (at 128 the attention kernel's
    128-dim instance, at 512 the kernel with two waves per column block;
    values tiled at every d) against the oracle, written into a strided
    output whose extra columns must stay untouched."""
    hk, bs = 2, 16
    say(f"prefill d={d} qg={qg} cached={cached_len} q_len={q_len}")
    rng = np.random.default_rng(qg * 100 + cached_len + q_len)
    nblk = max(1, -(-cached_len // bs))
    row = rng.permutation(nblk + 3)[:nblk].astype(np.int32)
    cache = torch.zeros((nblk + 3, bs, hk, slot(d)), dtype=torch.uint8, device=DEV)
    ref = np.zeros(tuple(cache.shape), dtype=np.uint8)
    if cached_len:
        kb = bf16(rng.standard_normal((cached_len, hk, d)))
        vb = bf16(rng.standard_t(4, (cached_len, hk, d)))
        t = np.arange(cached_len)
        slots = row[t // bs].astype(np.int64) * bs + t % bs
        uq.store(kb.to(DEV), vb.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(bits(kb), bits(vb), ref, slots)
    q = bf16(rng.standard_normal((q_len, hk * qg, d)))
    kc = bf16(rng.standard_normal((q_len, hk, d)))
    vc = bf16(rng.standard_t(4, (q_len, hk, d)))
    scale = 1 / np.sqrt(d)
    big = torch.full((q_len, hk * qg, d + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = uq.continuation_prefill(q.to(DEV), kc.to(DEV), vc.to(DEV), cache, torch.from_numpy(row).to(DEV),
                                  cached_len, scale, out=big[:, :, :d])
    assert torch.isnan(big[:, :, d:]).all()
    want = O.continuation_prefill(bits(q), bits(kc), bits(vc), ref, row, cached_len, scale)
    check_close(to_np(out), want, f"prefill d={d} qg={qg} cached={cached_len} q_len={q_len}",
                allow_output_rounding=True)


@pytest.mark.parametrize("qg", [8, 16])
@pytest.mark.parametrize("d", DIMS)
def test_prefill_attention_strided_and_peaked(d, qg):
    """uq_prefill_attention at head dim d on strided views (values
    token-major), 300 keys (a ragged last tile) and a large scale that
    raises the running maximum along the keys, against a float64 softmax."""
    say(f"prefill attention d={d} qg={qg}")
    rng = np.random.default_rng(17 + qg + d)
    q_len, seq, hk = 50, 300, 2
    grow = np.linspace(0.2, 4.0, seq)[:, None, None]
    k = bf16(rng.standard_normal((seq, hk, d)) * grow)
    v = bf16(rng.standard_normal((seq, hk, d)))
    q = bf16(rng.standard_normal((q_len, hk * qg, d)))
    kv = torch.zeros((seq, 2, hk, d + 8), dtype=torch.bfloat16, device=DEV)
    kv[:, 0, :, :d] = k.to(DEV)
    kv[:, 1, :, :d] = v.to(DEV)
    qq = torch.zeros((q_len, hk * qg, d + 64), dtype=torch.bfloat16, device=DEV)
    qq[:, :, 64:] = q.to(DEV)
    o = torch.full((q_len, hk * qg, d + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    sc = 0.5 * np.sqrt(128 / d)                  # the same score spread at every d
    uq.prefill_attention(qq[:, :, 64:], kv[:, 0, :, :d], kv[:, 1, :, :d], sc, out=o[:, :, :d])
    K, V, Q = O.bf16_to_f64(bits(k)), O.bf16_to_f64(bits(v)), O.bf16_to_f64(bits(q))
    want = np.zeros((q_len, hk * qg, d))
    for hq in range(hk * qg):
        s = sc * Q[:, hq] @ K[:, hq // qg].T
        s = np.where(np.arange(seq)[None, :] <= seq - q_len + np.arange(q_len)[:, None], s, -np.inf)
        p = np.exp(s - s.max(-1, keepdims=True))
        want[:, hq] = p @ V[:, hq // qg] / p.sum(-1, keepdims=True)
    check_close(to_np(o[:, :, :d]), want, f"d={d} strided peaked qg={qg}", allow_output_rounding=True)
    assert torch.isnan(o[:, :, d:]).all()


@pytest.mark.parametrize("qg", [6, 8, 16])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_decode_paired_query_rows(d, qg):
    """Multi-query rows: consecutive query rows (2r, 2r + 1) that read the
    same block-table row share one stage-1 wave when the group leaves half
    the MFMA columns free (QG <= 8). Pairs with the shorter row first and
    second (so that some partials hold tokens of one row only), an empty
    sequence, a pair over different rows, and an odd row count, against the
    oracle and bit for bit against the same rows decoded through a table
    with each row repeated (no pairing)."""
    say(f"decode paired rows d={d} qg={qg}")
    rng = np.random.default_rng(d + qg + 51)
    hk, bs = 2, 16
    full = [300, 77, 0, 1000]
    nblk = [(L + bs - 1) // bs for L in full]
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    table = np.zeros((len(full), max(nblk)), dtype=np.int32)
    off = 0
    cache = torch.zeros((nb, bs, hk, slot(d)), dtype=torch.uint8, device=DEV)
    ref_cache = np.zeros(tuple(cache.shape), dtype=np.uint8)
    for b, L in enumerate(full):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
        if L == 0:
            continue
        k, v = bf16(rng.standard_normal((L, hk, d))), bf16(rng.standard_normal((L, hk, d)))
        t = np.arange(L)
        slots = table[b, t // bs].astype(np.int64) * bs + t % bs
        uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(bits(k), bits(v), ref_cache, slots)
    rows = np.array([0, 0, 1, 1, 0, 3, 3, 3, 2, 2, 1], dtype=np.int32)
    lens = np.array([300, 45, 77, 77, 299, 1000, 16, 1000, 0, 0, 5], dtype=np.int32)
    q = bf16(rng.standard_normal((len(rows), hk * qg, d)))
    scale = 1 / np.sqrt(d)
    ref = O.decode(bits(q), ref_cache, table[rows], lens, scale)
    q_dev, tbl = q.to(DEV), torch.from_numpy(table).to(DEV)
    rows_dev, lens_dev = torch.from_numpy(rows).to(DEV), torch.from_numpy(lens).to(DEV)
    for splits in (1, 8, 64):
        out = uq.decode_ex(q_dev, cache, tbl, lens_dev, scale, splits, query_row=rows_dev)
        check_close(to_np(out), ref, f"paired rows d={d} qg={qg} splits={splits}")
        rep = uq.decode(q_dev, cache, tbl[rows_dev.long()].contiguous(), lens_dev, scale, splits)
        assert torch.equal(out, rep), f"splits={splits}: differs from the repeated-row decode"


@pytest.mark.parametrize("rows", [1536, 8192])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_query_prologue_codes_many_rows(d, rows):
    """The query prologue of a large batch (64 lanes per row, or 16 lanes and
    several rows per wave with a partly filled last wave) gives the oracle's codes bit
    for bit: random rows, zero rows, tiny and huge rows, and rows of values
    spread over 24 binades."""
    say(f"prologue many rows d={d} rows={rows}")
    rng = np.random.default_rng(d + rows)
    hk, qg = 2, 8
    B = rows // (hk * qg) + 1                 # one more sequence than needed: 16 extra rows
    q = rng.standard_normal((B, hk * qg, d))
    q[0, 0] = 0.0
    q[1, 3] = rng.standard_normal(d) * 2.0 ** -20
    q[2, 5] = rng.standard_normal(d) * 300.0
    q[3, 7] = rng.choice([-1.0, 1.0], d) * (1 + rng.random(d)) * np.exp2(rng.integers(-12, 13, d))
    qb = bf16(q)
    cache = torch.zeros((1, 16, hk, slot(d)), dtype=torch.uint8, device=DEV)
    ws = torch.full((uq.decode_workspace_bytes(B, hk * qg, hk, 1, 1, 16, d),), 0x55, dtype=torch.uint8, device=DEV)
    uq.decode(qb.to(DEV), cache, torch.zeros((B, 1), dtype=torch.int32, device=DEV),
              torch.ones(B, dtype=torch.int32, device=DEV), 1 / 16, 1, workspace=ws, stages=uq.STAGE_PROLOGUE)
    got = ws[:B * hk * qg * d].cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(B, hk * qg, d)
    ref = O.query_haircut(bits(qb))
    assert np.array_equal(got, ref), f"{(got != ref).sum()} codes differ"
