"""GPU parity of the HIP library against the CPU oracle, at sizes the oracle
finishes in seconds: cache bytes bit-exact, attention output within
max-abs 1e-2 / rel-L2 5e-3. Everything goes through the C ABI."""
import numpy as np
import pytest
import torch

import golden_io
import harness
from harness import check_close, to_np
import decode_attention_bit_amd as uq
from decode_attention_bit_amd import inputs
from oracle import uq_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bf16(x):
    return inputs.to_bf16(np.asarray(x, dtype=np.float32))


def bits(t):
    return inputs.bf16_bits(t.cpu())


def say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ Hadamard
@pytest.mark.parametrize("D", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_build_hadamard(D):
    say(f"hadamard D={D}")
    H = uq.build_hadamard(D, DEV).cpu().numpy()
    assert np.array_equal(H, O.hadamard(D).astype(np.float32))


# --------------------------------------------------------------------- store
def _store_and_compare(k, v, nb=4, bs=16, slots=None, fill=0):
    N, Hk, _ = k.shape
    if slots is None:
        slots = np.random.default_rng(0).permutation(nb * bs)[:N]
    cache = torch.full((nb, bs, Hk, 272), fill, dtype=torch.uint8, device=DEV)
    uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(np.asarray(slots, np.int64)).to(DEV))
    ref = np.full((nb, bs, Hk, 272), fill, dtype=np.uint8)
    O.store(bits(k), bits(v), ref, slots)
    got = cache.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:4].tolist()}"


def test_store_tiny_workload_bit_exact():
    say("store tiny")
    w = inputs.WORKLOADS["tiny"]
    inst = harness.Instance(w, DEV)
    ref = np.zeros(tuple(inst.cache.shape), dtype=np.uint8)
    for b in range(w.B):
        k, v = inputs.make_kv(w, inst.layout, b)
        O.store(bits(k), bits(v), ref, inputs.slots_for(inst.layout, b, 0, int(inst.layout.seq_lens[b])))
    assert np.array_equal(inst.cache.cpu().numpy(), ref)


def test_store_golden_slots():
    say("store golden")
    for case in golden_io.slot_cases():
        k = bf16(case["key"][None, None, :])
        v = bf16(case["value"][None, None, :])
        cache = torch.zeros((1, 16, 1, 272), dtype=torch.uint8, device=DEV)
        uq.store(k.to(DEV), v.to(DEV), cache, torch.tensor([5], dtype=torch.int64, device=DEV))
        assert np.array_equal(cache[0, 5, 0].cpu().numpy(), case["bytes"]), case["name"]


def test_store_golden_blocks_as_values():
    """Tie and saturation cases of the E2M1 rounding, through the V path."""
    say("store golden blocks")
    blocks = golden_io.mx_blocks()
    v = np.zeros((len(blocks), 1, 256))
    for i, blk in enumerate(blocks):
        v[i, 0] = np.tile(blk["x"], 8)
    vt = bf16(v)
    assert np.array_equal(inputs.bf16_bits(vt).astype(np.float64), inputs.bf16_bits(vt))  # sanity
    _store_and_compare(bf16(np.zeros_like(v)), vt, nb=1, bs=16, slots=np.arange(len(blocks)))


def test_store_edge_values():
    say("store edge values")
    rng = np.random.default_rng(1)
    n = 48
    k = rng.standard_normal((n, 2, 256))
    v = rng.standard_normal((n, 2, 256))
    k[0] = 0.0
    v[0] = -0.0
    k[1, 0, :] = -0.0
    k[2, :, :] = 0
    k[2, 0, 0], k[2, 0, 1] = 1.0, 1.0                   # rotated: exact zeros on odd d
    k[3, 0, :2] = [5.0, 4.0]                             # rotated lands on ties
    v[4] = np.ldexp(rng.uniform(0.5, 1, (2, 256)), -130)  # bf16 subnormals, scale clamps
    v[10] = np.ldexp(rng.uniform(1, 4, (2, 256)), -128)  # subnormals under byte 0: codes 1 to 4
    v[10, 1, :32] = np.ldexp(rng.uniform(1, 4, 32), -129) * rng.choice([-1, 1], 32)
    v[5] = rng.standard_normal((2, 256)) * 1e37          # near the top of the range
    k[6] = rng.standard_normal((2, 256)) * 1e30
    k[7] = np.ldexp(rng.uniform(0.5, 1, (2, 256)), -110)
    k[8] = rng.standard_t(1.5, (2, 256))                 # heavy tails
    k[9, :, 5] *= 1e4                                    # one outlier channel
    for i in range(10, 20):                              # magnitudes spread over 30 binades
        k[i] = np.ldexp(rng.uniform(0.5, 1, (2, 256)) * rng.choice([-1, 1], (2, 256)),
                        rng.integers(-15, 15, (2, 256)))
    for i in range(20, 30):                              # values on E2M1 midpoints
        v[i] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -5.0], (2, 256))
    _store_and_compare(bf16(k), bf16(v), nb=4, bs=16)


def test_store_canary_negative_and_out_of_range_slots():
    say("store canary")
    rng = np.random.default_rng(2)
    k = bf16(rng.standard_normal((12, 3, 256)))
    v = bf16(rng.standard_normal((12, 3, 256)))
    slots = np.array([3, -1, 7, 64, 8, -5, 30, 0, 1000, 2, 63, 31])
    cache = torch.full((4, 16, 3, 272), 0xA5, dtype=torch.uint8, device=DEV)
    uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(slots).to(DEV))
    ref = np.full((4, 16, 3, 272), 0xA5, dtype=np.uint8)
    keep = (slots >= 0) & (slots < 64)
    O.store(bits(k)[keep], bits(v)[keep], ref, slots[keep])
    assert np.array_equal(cache.cpu().numpy(), ref)


def test_store_strided_views_and_block_sizes():
    say("store strided")
    rng = np.random.default_rng(3)
    big_k = bf16(rng.standard_normal((20, 4, 512))).to(DEV)
    big_v = bf16(rng.standard_normal((40, 2, 256))).to(DEV)
    k = big_k[:, :, 128:384]            # stride_h 512, offset 128
    v = big_v.view(20, 4, 256)          # plain
    for bs in (16, 32, 64, 128, 256):
        nb = 2
        slots = rng.permutation(nb * bs)[:20]
        cache = torch.zeros((nb, bs, 4, 272), dtype=torch.uint8, device=DEV)
        uq.store(k, v, cache, torch.from_numpy(slots).to(DEV))
        ref = np.zeros((nb, bs, 4, 272), dtype=np.uint8)
        O.store(bits(k.contiguous()), bits(v), ref, slots)
        assert np.array_equal(cache.cpu().numpy(), ref), bs


def test_store_random_bulk():
    say("store bulk")
    rng = np.random.default_rng(4)
    k = bf16(rng.standard_normal((3000, 4, 256)) * np.exp(rng.uniform(-8, 8, (3000, 4, 1))))
    v = bf16(rng.standard_t(3, (3000, 4, 256)))
    _store_and_compare(k, v, nb=200, bs=16)


# ------------------------------------------------------------ query prologue
@pytest.mark.parametrize("qg", [6, 8, 16])
def test_query_prologue_codes_bit_exact(qg):
    """The E4M3 codes of q H that the prologue leaves at the start of the
    workspace equal the oracle's haircut value for value, with the sign of
    codes that flush to zero: zeros, subnormal-range inputs that flush, saturation above 448,
    and magnitudes spread over 26 binades (still exact in float64)."""
    say("query prologue codes")
    rng = np.random.default_rng(42)
    B, Hk = 3, 2
    Hq = Hk * qg
    q = rng.standard_normal((B, Hq, 256))
    q[0, 0] = 0.0                                            # all-zero vector
    q[0, 1] = -0.0
    q[0, 2] = rng.standard_normal(256) * 2.0 ** -20          # rounds to 0 / subnormals
    q[0, 3] = rng.standard_normal(256) * 300.0               # saturates at 448
    q[1, 0] = rng.choice([-1.0, 1.0], 256) * (1 + rng.random(256)) * np.exp2(rng.integers(-12, 13, 256))
    q[1, 1, :] = 0.0
    q[1, 1, 7] = 1.0                                         # one-hot: +-1/16 everywhere
    q[2] *= 1e-2
    qb = bf16(q)
    tbl = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    cache = torch.zeros((1, 16, Hk, 272), dtype=torch.uint8, device=DEV)
    ws = torch.full((uq.decode_workspace_bytes(B, Hq, Hk, 1, 1),), 0x55, dtype=torch.uint8, device=DEV)
    uq.decode(qb.to(DEV), cache, tbl, lens, 1 / 16, 1, workspace=ws, stages=uq.STAGE_PROLOGUE)
    codes = ws[:B * Hq * 256].cpu()
    got = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy().reshape(B, Hq, 256)
    ref = O.query_haircut(bits(qb))
    assert np.array_equal(got, ref), f"{(got != ref).sum()} codes differ"
    # a non-zero product that rounds to zero keeps its sign; the sign of an
    # exactly-zero product is not defined by the method and is not compared
    nz = O.rotate(O.bf16_to_f64(bits(qb))) != 0
    assert np.array_equal(np.signbit(got)[nz], np.signbit(ref)[nz]), "sign of a flushed code differs"


# -------------------------------------------------------------------- decode
def _decode_case(seq_lens, Hk, qg, bs=16, splits=4, seed=0, scale=1 / 16, q_scale=1.0,
                 k_gen=None):
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    Hq = Hk * qg
    nblk = [(L + bs - 1) // bs for L in seq_lens]
    width = max(max(nblk), 1)
    nb = sum(nblk) + 3
    perm = rng.permutation(nb)
    table = np.zeros((B, width), dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    q = bf16(rng.standard_normal((B, Hq, 256)) * q_scale)
    cache = torch.zeros((nb, bs, Hk, 272), dtype=torch.uint8, device=DEV)
    ref_cache = np.zeros((nb, bs, Hk, 272), dtype=np.uint8)
    for b, L in enumerate(seq_lens):
        if L == 0:
            continue
        kk = k_gen(rng, (L, Hk, 256)) if k_gen else rng.standard_normal((L, Hk, 256))
        k = bf16(kk)
        v = bf16(rng.standard_normal((L, Hk, 256)))
        t = np.arange(L)
        slots = table[b, t // bs].astype(np.int64) * bs + t % bs
        uq.store(k.to(DEV), v.to(DEV), cache, torch.from_numpy(slots).to(DEV))
        O.store(bits(k), bits(v), ref_cache, slots)
    tbl = torch.from_numpy(table).to(DEV)
    lens = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    out = uq.decode(q.to(DEV), cache, tbl, lens, scale, splits)
    ref = O.decode(bits(q), ref_cache, table, np.array(seq_lens), scale)
    return out, ref, dict(q=q, cache=cache, table=tbl, lens=lens, ref_cache=ref_cache, scale=scale)


def test_decode_tiny_workload():
    say("decode tiny")
    w = inputs.WORKLOADS["tiny"]
    inst = harness.Instance(w, DEV)
    ref_cache = np.zeros(tuple(inst.cache.shape), dtype=np.uint8)
    for b in range(w.B):
        k, v = inputs.make_kv(w, inst.layout, b)
        O.store(bits(k), bits(v), ref_cache, inputs.slots_for(inst.layout, b, 0, int(inst.layout.seq_lens[b])))
    ref = O.decode(bits(inst.query), ref_cache, inst.layout.block_table, inst.layout.seq_lens, w.scale)
    for S in (1, 2, 3, 4, 5, 7, 8, 16, 64, 512):
        check_close(to_np(inst.decode(S)), ref, f"tiny S={S}")


@pytest.mark.parametrize("qg", [6, 8, 16])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_decode_ragged_lengths_block_sizes(qg, bs):
    say(f"decode ragged qg={qg} bs={bs}")
    lens = [1, 15, 16, 17, 100, 257, 300, 33]
    out, ref, _ = _decode_case(lens, Hk=2, qg=qg, bs=bs, splits=3, seed=qg * 1000 + bs)
    check_close(to_np(out), ref, f"qg={qg} bs={bs}")


@pytest.mark.parametrize("qg", [6, 8, 16])
def test_decode_odd_head_count(qg):
    """Three KV heads: stage 1 then runs one head per workgroup."""
    say(f"decode Hk=3 qg={qg}")
    out, ref, _ = _decode_case([300, 17, 1, 64], Hk=3, qg=qg, splits=4, seed=60 + qg)
    check_close(to_np(out), ref, f"Hk=3 qg={qg}")


def test_decode_large_grid_many_empty_partials():
    """A grid of several rounds of the chip (40 ragged sequences, 128 splits:
    2560 stage-1 waves), most of whose partials lie past their sequence's
    end; with a window and sinks too."""
    say("decode large grid")
    rng = np.random.default_rng(70)
    lens = [int(x) for x in rng.integers(0, 1025, 40)]
    lens[0], lens[1], lens[2] = 1024, 1, 0
    out, ref, ctx = _decode_case(lens, Hk=2, qg=8, splits=128, seed=71)
    check_close(to_np(out), ref, "large grid")
    sinks = rng.normal(0.0, 2.0, 16).astype(np.float32)
    o = uq.decode_ex(ctx["q"].to(DEV), ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], 128,
                     sinks=torch.from_numpy(sinks).to(DEV), sliding_window=333)
    r = O.decode(bits(ctx["q"]), ctx["ref_cache"], ctx["table"].cpu().numpy(), np.array(lens), ctx["scale"],
                 sinks=sinks.astype(np.float64), sliding_window=333)
    check_close(to_np(o), r, "large grid, window and sinks")


@pytest.mark.parametrize("k", [-100, -60, 40, 90])
def test_decode_value_scale_equivariance(k):
    """Values scaled by 2^k (exact in bf16) shift every UE8M0 value exponent
    by k and leave the weights alone, so the output scales by exactly 2^k:
    bit for bit, through the fp16 partial rows and their power-of-two row
    scales, at magnitudes far from 1."""
    say(f"decode value scale 2^{k}")
    rng = np.random.default_rng(80)
    lens, Hk, qg, bs = [600, 40, 1, 333], 2, 8, 16
    B, Hq = len(lens), Hk * qg
    nblk = [(L + bs - 1) // bs for L in lens]
    nb = sum(nblk) + 1
    table = np.zeros((B, max(nblk)), dtype=np.int32)
    perm, off = rng.permutation(nb), 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    c0 = torch.zeros((nb, bs, Hk, 272), dtype=torch.uint8, device=DEV)
    c1 = torch.zeros_like(c0)
    for b, L in enumerate(lens):
        kk = bf16(rng.standard_normal((L, Hk, 256)))
        vv = bf16(rng.standard_normal((L, Hk, 256)))
        t = np.arange(L)
        slots = torch.from_numpy(table[b, t // bs].astype(np.int64) * bs + t % bs).to(DEV)
        uq.store(kk.to(DEV), vv.to(DEV), c0, slots)
        uq.store(kk.to(DEV), (vv.double() * 2.0 ** k).to(torch.bfloat16).to(DEV), c1, slots)
    q = bf16(rng.standard_normal((B, Hq, 256))).to(DEV)
    tbl = torch.from_numpy(table).to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for S in (1, 4, 32):
        o0 = uq.decode(q, c0, tbl, sl, 1 / 16, S)
        o1 = uq.decode(q, c1, tbl, sl, 1 / 16, S)
        assert torch.equal(o1, (o0.double() * 2.0 ** k).to(torch.bfloat16)), (k, S)


def test_decode_single_token_is_exact():
    """L = 1: softmax weight 1, so the bf16 output equals the dequantised
    value, which bf16 represents exactly."""
    say("decode L=1")
    out, ref, ctx = _decode_case([1, 1, 1], Hk=2, qg=8, splits=4, seed=5)
    assert np.array_equal(to_np(out), ref)


def test_decode_zero_query_is_mean():
    say("decode q=0")
    rng = np.random.default_rng(6)
    out, ref, ctx = _decode_case([50, 91], Hk=1, qg=8, splits=2, seed=6, q_scale=0.0)
    for b, L in enumerate([50, 91]):
        _, V = O.gather_sequence(ctx["ref_cache"], ctx["table"].cpu().numpy()[b], L, 0)
        check_close(to_np(out)[b], np.broadcast_to(V.mean(0), (8, 256)), f"mean b={b}")


def test_decode_large_scores_rebase():
    """Scores far above the first tile's maximum exercise the running-max
    re-basing path."""
    say("decode rebase")
    def grow(rng, shape):
        x = rng.standard_normal(shape)
        return x * np.linspace(0.2, 3.0, shape[0])[:, None, None]
    out, ref, _ = _decode_case([400, 1000], Hk=2, qg=8, splits=2, seed=7, scale=0.25, k_gen=grow)
    # peaked softmax: outputs are single dequantised values of magnitude up to ~6
    check_close(to_np(out), ref, "rebase", allow_output_rounding=True)


def test_decode_golden_two_token():
    say("decode golden")
    d = golden_io.decode_two_token()
    L = d["seq_len"]
    k = bf16(np.stack([d["key"][t] for t in range(L)])[:, None, :])
    v = bf16(np.stack([d["value"][t] for t in range(L)])[:, None, :])
    q = bf16(np.broadcast_to(d["query"], (1, 8, 256)))
    cache = torch.zeros((1, 16, 1, 272), dtype=torch.uint8, device=DEV)
    uq.store(k.to(DEV), v.to(DEV), cache, torch.arange(L, dtype=torch.int64, device=DEV))
    out = uq.decode(q.to(DEV), cache, torch.zeros((1, 1), dtype=torch.int32, device=DEV),
                    torch.tensor([L], dtype=torch.int32, device=DEV), d["scale"], 1)
    want = np.zeros(256)
    for i, x in d["out"].items():
        want[i] = x
    check_close(to_np(out)[0], np.broadcast_to(want, (8, 256)), "two-token")


def test_decode_empty_sequence_and_clamped_length():
    say("decode empty")
    rng = np.random.default_rng(8)
    out, ref, ctx = _decode_case([0, 40], Hk=1, qg=8, splits=2, seed=8)
    assert np.all(to_np(out)[0] == 0)
    check_close(to_np(out)[1], ref[1], "b=1")
    # a length past the table clamps to the table's capacity (48 tokens here)
    lens = torch.tensor([0, 10 ** 6], dtype=torch.int32, device=DEV)
    out2 = uq.decode(ctx["q"].to(DEV), ctx["cache"], ctx["table"], lens, ctx["scale"], 2)
    assert np.all(np.isfinite(to_np(out2)))


def test_decode_query_strides_and_reuse_of_outputs():
    say("decode strides")
    out, ref, ctx = _decode_case([70, 130], Hk=2, qg=8, splits=4, seed=9)
    big = torch.zeros((2, 16, 512), dtype=torch.bfloat16, device=DEV)
    big[:, :, 256:] = ctx["q"].to(DEV)
    qv = big[:, :, 256:]
    o = torch.full((2, 16, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(uq.decode_workspace_bytes(2, 16, 2, 4, ctx["table"].shape[1]), dtype=torch.uint8, device=DEV)
    uq.decode(qv, ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], 4, out=o, workspace=ws)
    assert torch.equal(o, out)


def test_decode_default_workspace_per_stream():
    """Calls without a workspace on two streams at once get separate cached
    buffers and give the results of the same calls on one stream."""
    say("decode two streams")
    out1, ref1, c1 = _decode_case([300, 77, 512], Hk=2, qg=8, splits=4, seed=31)
    out2, ref2, c2 = _decode_case([1000, 5], Hk=4, qg=6, splits=8, seed=32)
    check_close(to_np(out1), ref1, "stream case 1")
    check_close(to_np(out2), ref2, "stream case 2")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    main = torch.cuda.current_stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    got1, got2 = [], []
    for _ in range(8):
        with torch.cuda.stream(s1):
            got1.append(uq.decode(c1["q"].to(DEV), c1["cache"], c1["table"], c1["lens"], c1["scale"], 4))
        with torch.cuda.stream(s2):
            got2.append(uq.decode(c2["q"].to(DEV), c2["cache"], c2["table"], c2["lens"], c2["scale"], 8))
    torch.cuda.synchronize()
    for o in got1:
        assert torch.equal(o, out1)
    for o in got2:
        assert torch.equal(o, out2)
    with torch.cuda.stream(s1):
        w1 = uq._workspace(DEV, 256)
    with torch.cuda.stream(s2):
        w2 = uq._workspace(DEV, 256)
    assert w1.data_ptr() != w2.data_ptr()
    with torch.cuda.stream(s1):
        assert uq._workspace(DEV, 256).data_ptr() == w1.data_ptr()


def test_decode_stage_masks_compose():
    say("decode stages")
    out, ref, ctx = _decode_case([90, 33], Hk=2, qg=8, splits=4, seed=10)
    o = torch.empty_like(out)
    for st in (uq.STAGE_PROLOGUE, uq.STAGE_SPLIT, uq.STAGE_MERGE):
        uq.decode(ctx["q"].to(DEV), ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], 4,
                  out=o, stages=st)
    assert torch.equal(o, out)


def _extreme_queries(rng, B, Hq):
    """Query rows that stress the E4M3 haircut: zeros, values that flush or
    land on subnormal codes, saturation above 448, magnitudes spread over 26
    binades, one-hot rows (+-1/16 everywhere) and small Gaussians."""
    q = rng.standard_normal((B, Hq, 256))
    kinds = [
        lambda: np.zeros(256),
        lambda: rng.standard_normal(256) * 2.0 ** -20,
        lambda: rng.standard_normal(256) * 2.0 ** -9,
        lambda: rng.standard_normal(256) * 300.0,
        lambda: rng.choice([-1.0, 1.0], 256) * (1 + rng.random(256)) * np.exp2(rng.integers(-12, 13, 256)),
        lambda: np.eye(256)[rng.integers(256)] * rng.choice([-1.0, 1.0]),
        lambda: rng.standard_normal(256) * 1e-2,
    ]
    for b in range(B):
        for h in range(Hq):
            if (b * Hq + h) % 3:
                q[b, h] = kinds[(b * Hq + h) % len(kinds)]()
    return bf16(q)


@pytest.mark.parametrize("qg", [6, 8, 16])
def test_decode_extreme_queries(qg):
    """Query rows of every kind the haircut distinguishes (flushed, subnormal,
    saturated, wide-range, one-hot) through a whole decode: the output
    matches the oracle, bit for bit the output of the prologue run on its own
    followed by stages 1 and 2, and bit for bit the two-launch form whose
    stage 1 computes the query codes itself."""
    say(f"decode extreme queries qg={qg}")
    Hk = 2
    _, _, ctx = _decode_case([37, 20, 64], Hk=Hk, qg=qg, splits=2, seed=11 + qg)
    q = _extreme_queries(np.random.default_rng(qg), 3, Hk * qg).to(DEV)
    full = uq.decode(q, ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], 2)
    args = (q, ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], 2)
    o = torch.empty_like(full)
    for st in (uq.STAGE_PROLOGUE, uq.STAGE_SPLIT | uq.STAGE_MERGE):
        uq.decode(*args, out=o, stages=st)
    assert torch.equal(o, full)
    fused = uq.decode(*args, stages=uq.STAGE_SPLIT | uq.STAGE_FUSED_QUERY | uq.STAGE_MERGE)
    assert torch.equal(fused, full), "in-kernel query codes differ from the prologue kernel's"
    ref = O.decode(bits(q.cpu()), ctx["ref_cache"], ctx["table"].cpu().numpy(),
                   ctx["lens"].cpu().numpy(), ctx["scale"])
    check_close(to_np(full), ref, f"extreme queries qg={qg}", allow_output_rounding=True)


def test_decode_multi_query_continuation_chunks():
    """Continuation chunks, decoded one query at a time as the ultraquant_attn
    page does for short chunks: query i of a chunk over a sequence holding
    cached_len tokens attends to cached_len + i + 1 tokens through the
    sequence's block-table row. The oracle is given that row repeated per
    query; the library gets the compact table and a row index per query."""
    say("decode multi-query")
    cached, chunk = [40, 200, 0, 17], [3, 1, 4, 2]
    full = [c + n for c, n in zip(cached, chunk)]
    _, _, ctx = _decode_case(full, Hk=2, qg=8, splits=4, seed=21)
    rows = np.concatenate([np.full(n, s) for s, n in enumerate(chunk)]).astype(np.int32)
    lens = np.concatenate([c + 1 + np.arange(n) for c, n in zip(cached, chunk)]).astype(np.int32)
    T = len(rows)
    rng = np.random.default_rng(22)
    q = bf16(rng.standard_normal((T, 16, 256)))
    table = ctx["table"]
    q_dev, rows_dev, lens_dev = q.to(DEV), torch.from_numpy(rows).to(DEV), torch.from_numpy(lens).to(DEV)
    for S in (1, 4, 16):
        out = uq.decode_ex(q_dev, ctx["cache"], table, lens_dev, ctx["scale"], S, query_row=rows_dev)
        ref = O.decode(bits(q), ctx["ref_cache"], table.cpu().numpy()[rows], lens, ctx["scale"])
        check_close(to_np(out), ref, f"multi-query S={S}")
        # the same as decoding against the table with each row repeated
        rep = uq.decode(q_dev, ctx["cache"], table[rows_dev.long()].contiguous(), lens_dev,
                        ctx["scale"], S)
        assert torch.equal(out, rep), f"S={S}: differs from the repeated-row decode"
    # a row index outside the table reads as an empty sequence
    bad = rows_dev.clone()
    bad[0], bad[-1] = -1, len(full)
    out = uq.decode_ex(q_dev, ctx["cache"], table, lens_dev, ctx["scale"], 4, query_row=bad)
    o = to_np(out)
    assert np.all(o[0] == 0) and np.all(o[-1] == 0)
    ref = O.decode(bits(q), ctx["ref_cache"], table.cpu().numpy()[rows], lens, ctx["scale"])
    check_close(o[1:-1], ref[1:-1], "multi-query, valid rows")


def test_decode_paired_rows_large_batch():
    """Paired multi-query rows on a grid of many rounds (the two-slot ring of
    stage 1): 256 sequences of 40 to 112 tokens, two query rows each (the
    second one token longer, as in a two-token speculative step), against
    the oracle on a sample of rows, and bit for bit like the same rows
    through a repeated-row table with distinct row indices (the same
    partials plan, no pairs)."""
    say("decode paired rows, large batch")
    rng = np.random.default_rng(61)
    nseq, hk, qg, bs = 256, 4, 8, 16
    full = rng.integers(40, 113, nseq)
    width = int((full.max() + bs - 1) // bs)
    nblk = [(int(L) + bs - 1) // bs for L in full]
    nb = sum(nblk) + 5
    perm = rng.permutation(nb)
    table = np.zeros((nseq, width), dtype=np.int32)
    cache = torch.zeros((nb, bs, hk, 272), dtype=torch.uint8, device=DEV)
    ref_cache = np.zeros(tuple(cache.shape), dtype=np.uint8)
    off = 0
    kall = bf16(rng.standard_normal((int(full.sum()), hk, 256)))
    vall = bf16(rng.standard_normal((int(full.sum()), hk, 256)))
    slots = np.zeros(int(full.sum()), dtype=np.int64)
    pos = 0
    for b, L in enumerate(full):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
        t = np.arange(L)
        slots[pos:pos + L] = table[b, t // bs].astype(np.int64) * bs + t % bs
        pos += L
    uq.store(kall.to(DEV), vall.to(DEV), cache, torch.from_numpy(slots).to(DEV))
    O.store(bits(kall), bits(vall), ref_cache, slots)
    rows = np.repeat(np.arange(nseq), 2).astype(np.int32)
    lens = (full[rows] - 1 + np.tile([0, 1], nseq)).astype(np.int32)
    q = bf16(rng.standard_normal((len(rows), hk * qg, 256)))
    q_dev, tbl = q.to(DEV), torch.from_numpy(table).to(DEV)
    rows_dev, lens_dev = torch.from_numpy(rows).to(DEV), torch.from_numpy(lens).to(DEV)
    out = uq.decode_ex(q_dev, cache, tbl, lens_dev, 1 / 16, 32, query_row=rows_dev)
    pick = np.sort(rng.choice(len(rows), 24, replace=False))
    ref = O.decode(bits(q[pick]), ref_cache, table[rows[pick]], lens[pick], 1 / 16)
    check_close(to_np(out)[pick], ref, "paired rows, large batch")
    own = torch.arange(len(rows), dtype=torch.int32, device=DEV)
    rep = uq.decode_ex(q_dev, cache, tbl[rows_dev.long()].contiguous(), lens_dev, 1 / 16, 32, query_row=own)
    assert torch.equal(out, rep), "paired rows differ from the same rows decoded one by one"


@pytest.mark.parametrize("window", [0, 1, 15, 16, 17, 100, 333, 5000])
def test_decode_sinks_and_sliding_window(window):
    """Per-head sink logits and a sliding window of the last W tokens against
    the oracle, at several split counts, with windows that start mid-tile,
    on a tile edge, mid-partial and before the sequence."""
    say(f"decode sinks window={window}")
    lens = [700, 77, 1, 16, 0, 300]
    out0, ref0, ctx = _decode_case(lens, Hk=2, qg=8, splits=4, seed=23)
    rng = np.random.default_rng(24)
    sinks = rng.normal(0.0, 2.0, 16)
    sinks[3] = -np.inf
    sinks_dev = torch.from_numpy(sinks.astype(np.float32)).to(DEV)
    ref = O.decode(bits(ctx["q"]), ctx["ref_cache"], ctx["table"].cpu().numpy(), np.array(lens),
                   ctx["scale"], sinks=sinks.astype(np.float32).astype(np.float64),
                   sliding_window=window)
    for S in (1, 4, 32, 512):    # 512 splits: the merge shares each row among four waves
        out = uq.decode_ex(ctx["q"].to(DEV), ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], S,
                           sinks=sinks_dev, sliding_window=window)
        check_close(to_np(out), ref, f"sinks, window={window}, S={S}")
    # the window alone, and no option at all equals uq_decode bit for bit
    out = uq.decode_ex(ctx["q"].to(DEV), ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], 4,
                       sliding_window=window)
    ref_w = O.decode(bits(ctx["q"]), ctx["ref_cache"], ctx["table"].cpu().numpy(), np.array(lens),
                     ctx["scale"], sliding_window=window)
    check_close(to_np(out), ref_w, f"window={window}")
    if window == 0:
        plain = uq.decode_ex(ctx["q"].to(DEV), ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], 4)
        assert torch.equal(plain, out0)


def test_decode_split_count_invariance():
    say("decode split invariance")
    out, ref, ctx = _decode_case([2000, 1500, 777], Hk=4, qg=8, splits=1, seed=11)
    base = to_np(out)
    check_close(base, ref, "S=1")
    for S in (2, 8, 32, 64, 128, 512):
        o = uq.decode(ctx["q"].to(DEV), ctx["cache"], ctx["table"], ctx["lens"], ctx["scale"], S)
        check_close(to_np(o), ref, f"S={S}")


# ------------------------------------------------------------- graph capture
def test_store_and_decode_replay_in_hip_graph():
    """Neither entry point allocates or synchronises, so a store + decode step
    can be captured once and replayed: every replay, with new inputs copied in
    place and eager work in between, equals the same step run eagerly."""
    say("graph capture")
    rng = np.random.default_rng(77)
    B, Hk, qg, bs, width = 4, 2, 8, 16, 12
    Hq = Hk * qg
    nb = B * width
    table = torch.from_numpy(rng.permutation(nb).reshape(B, width).astype(np.int32)).to(DEV)
    lens = torch.tensor([150, 33, 190, 77], dtype=torch.int32, device=DEV)
    cache = torch.zeros((nb, bs, Hk, 272), dtype=torch.uint8, device=DEV)
    for b in range(B):                      # prefix of each sequence, stored eagerly
        L = int(lens[b])
        t = torch.arange(L, device=DEV)
        slots = table[b, t // bs].long() * bs + t % bs
        uq.store(bf16(rng.standard_normal((L, Hk, 256))).to(DEV), bf16(rng.standard_normal((L, Hk, 256))).to(DEV),
                 cache, slots)
    last = lens.long() - 1                  # each step rewrites the last token of every sequence
    slots_new = table[torch.arange(B, device=DEV), last // bs].long() * bs + last % bs
    q = torch.empty((B, Hq, 256), dtype=torch.bfloat16, device=DEV)
    k_new = torch.empty((B, Hk, 256), dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    out = torch.empty((B, Hq, 256), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(uq.decode_workspace_bytes(B, Hq, Hk, 4, width), dtype=torch.uint8, device=DEV)

    def fill(i):
        r = np.random.default_rng(1000 + i)
        q.copy_(bf16(r.standard_normal((B, Hq, 256))).to(DEV))
        k_new.copy_(bf16(r.standard_normal((B, Hk, 256))).to(DEV))
        v_new.copy_(bf16(r.standard_normal((B, Hk, 256))).to(DEV))

    def step(c, o, w):
        uq.store(k_new, v_new, c, slots_new)
        uq.decode(q, c, table, lens, 1 / 16, 4, out=o, workspace=w)

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up off the default stream, as capture requires
        step(cache, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cache, out, ws)
    for i in range(1, 6):
        fill(i)
        ref_cache = cache.clone()
        ref_out = torch.empty_like(out)
        step(ref_cache, ref_out, torch.empty_like(ws))     # eager reference
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache, ref_cache), f"replay {i}: cache differs"
        assert torch.equal(out, ref_out), f"replay {i}: output differs"


def test_capture_without_workspace_is_refused():
    """A captured call must bring its own workspace: the binding's cached one
    is shared with eager calls and can be replaced (freed) while a graph still
    writes into it on replay, so under capture the binding refuses to use it.
    Eager calls keep using the cached workspace afterwards."""
    say("graph capture without a workspace")
    rng = np.random.default_rng(78)
    B, Hk, qg, bs, width = 2, 1, 8, 16, 4
    Hq = Hk * qg
    table = torch.from_numpy(rng.permutation(B * width).reshape(B, width).astype(np.int32)).to(DEV)
    lens = torch.tensor([40, 17], dtype=torch.int32, device=DEV)
    cache = torch.zeros((B * width, bs, Hk, 272), dtype=torch.uint8, device=DEV)
    for b in range(B):
        L = int(lens[b])
        t = torch.arange(L, device=DEV)
        uq.store(bf16(rng.standard_normal((L, Hk, 256))).to(DEV), bf16(rng.standard_normal((L, Hk, 256))).to(DEV),
                 cache, table[b, t // bs].long() * bs + t % bs)
    q = bf16(rng.standard_normal((B, Hq, 256))).to(DEV)
    out = torch.empty((B, Hq, 256), dtype=torch.bfloat16, device=DEV)
    eager = uq.decode(q, cache, table, lens, 1 / 16, 4).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with pytest.raises(ValueError, match="own workspace"):
            with torch.cuda.graph(g):
                uq.decode(q, cache, table, lens, 1 / 16, 4, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    again = uq.decode(q, cache, table, lens, 1 / 16, 4)
    assert torch.equal(again, eager)
