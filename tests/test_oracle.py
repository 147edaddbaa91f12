"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against a closed form, a library routine, a
hand-derived fixture (tests/golden/) or brute force, so that a dropped term,
a wrong sign or index, or a transposed operand fails at least one of them.
"""
import fractions
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import golden_io
from decode_attention_bit_amd import inputs
from oracle import uq_oracle as O


def bf16(x):
    return inputs.bf16_bits(inputs.to_bf16(np.asarray(x, dtype=np.float32)))


# ---------------------------------------------------------------- Hadamard
def test_hadamard_closed_form_matches_scipy():
    H = O.hadamard(256)
    assert np.array_equal(H, scipy.linalg.hadamard(256) / 16.0)


def test_hadamard_symmetric_orthonormal_exact():
    H = O.hadamard(256)
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, np.eye(256))


def _textbook_fwht(x):
    """Iterative radix-2 Walsh-Hadamard butterfly, unnormalised."""
    x = np.array(x, dtype=np.float64)
    h = 1
    n = x.shape[-1]
    while h < n:
        for i in range(0, n, 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x


def test_rotation_equals_butterfly():
    rng = np.random.default_rng(7)
    x = O.bf16_to_f64(bf16(rng.standard_normal((64, 256))))
    assert np.array_equal(O.rotate(x), _textbook_fwht(x) / 16.0)


def test_rotation_invariance_of_dot_products():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((32, 256))
    k = rng.standard_normal((32, 256))
    H = O.hadamard(256)
    lhs = np.einsum("nd,nd->n", q, k)
    rhs = np.einsum("nd,nd->n", q @ H, k @ H)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_rotation_exact_against_fractions():
    rng = np.random.default_rng(9)
    mant = rng.uniform(0.5, 2.0, (3, 256)) * rng.choice([-1.0, 1.0], (3, 256))
    x = O.bf16_to_f64(bf16(np.ldexp(mant, rng.integers(-14, 15, (3, 256)))))
    y = O.rotate(x)
    n = 256
    for r in range(3):
        xf = [fractions.Fraction(v) for v in x[r]]
        for j in (0, 1, 77, 128, 255):
            s = sum((xf[i] if bin(i & j).count("1") % 2 == 0 else -xf[i]) for i in range(n))
            assert fractions.Fraction(y[r, j]) == s / 16


def test_rotation_rejects_inexact_span():
    x = np.zeros(256)
    x[0], x[1] = 1.0, 2.0 ** -60
    assert not O.exact_span_ok(x)
    with pytest.raises(ValueError):
        O.rotate(x)


def _span_vector(n, span):
    """n - 1 copies of the largest bf16 significand at exponent 0 (255/128)
    and one value of 129 units of 2**(-span - 7): the +-sum of largest
    magnitude with an odd number of units."""
    x = np.full(n, 255.0 / 128.0)
    x[-1] = 129.0 * 2.0 ** (-span - 7)
    assert np.array_equal(O.bf16_to_f64(bf16(x)), x)     # bf16 values
    return x


@pytest.mark.parametrize("n,span", [(128, 38), (256, 37), (512, 36)])
def test_exact_span_boundary(n, span):
    """The guard sits exactly at the bound: at `span` binades the all-plus sum
    (coordinate 0) of the worst vector is exact, checked against Fractions,
    and the oracle computes it; one binade more, that sum is no float64 at
    all, so the oracle must refuse the vector."""
    x = _span_vector(n, span)
    exact = sum(fractions.Fraction(v) for v in x)
    assert fractions.Fraction(float(exact)) == exact
    assert O.exact_span_ok(x)
    y = O.rotate(x)
    scale = fractions.Fraction(O.rot_scale(n))
    assert fractions.Fraction(y[0]) == fractions.Fraction(float(exact * scale))
    # a coordinate with mixed signs too
    j = n // 2 + 3
    sj = sum((fractions.Fraction(x[i]) if bin(i & j).count("1") % 2 == 0 else -fractions.Fraction(x[i]))
             for i in range(n))
    assert fractions.Fraction(y[j]) == fractions.Fraction(float(sj * scale))

    x1 = _span_vector(n, span + 1)
    exact1 = sum(fractions.Fraction(v) for v in x1)
    assert fractions.Fraction(float(exact1)) != exact1        # not representable in float64
    assert not O.exact_span_ok(x1)
    with pytest.raises(ValueError):
        O.rotate(x1)


# ------------------------------------------------------- E2M1 and UE8M0
def test_e2m1_value_table_matches_ocp_table():
    table = golden_io.e2m1_table()
    got = O.e2m1_value(np.arange(16))
    for c, v in table.items():
        assert got[c] == v and math.copysign(1, got[c]) == math.copysign(1, v)


def test_e2m1_rounding_fixture():
    for r, code in golden_io.e2m1_rounding():
        assert int(O.e2m1_round(np.array([r]))[0]) == code, r


def test_e2m1_roundtrip_every_value_every_exponent():
    mags = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for e in range(-127, 126):
        blk = np.zeros(32)
        blk[: len(mags)] = mags
        blk[7: 7 + len(mags)] = -mags
        blk[-1] = 4.0  # block max code 6 reproduces e
        x = np.ldexp(blk, e)
        codes, sb = O.quantize_blocks(np.tile(x, 8))
        assert np.all(sb == e + 127)
        dq = np.ldexp(O.e2m1_value(codes), e)
        assert np.array_equal(dq, np.tile(x, 8))


def test_mx_blocks_fixture():
    for blk in golden_io.mx_blocks():
        codes, sb = O.quantize_blocks(np.tile(blk["x"], 8))
        assert np.all(sb == blk["byte"]), blk["name"]
        assert np.array_equal(codes[:32], blk["codes"]), blk["name"]


def test_ue8m0_decode_matches_torch():
    b = torch.arange(0, 255, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    # the oracle decodes byte -> 2**(byte - 127) inside decode_slots
    slot = np.zeros((255, 272), dtype=np.uint8)
    slot[:, 0] = 0x2           # element 0 = code 2 = 1.0
    slot[:, 128] = 0x2
    slot[:, 256] = np.arange(255)
    slot[:, 264] = np.arange(255)
    K, V = O.decode_slots(slot)
    assert np.array_equal(K[:, 0], ref)
    assert np.array_equal(V[:, 0], ref)


def test_scale_rule_max_code():
    """After scaling, the block maximum lands in [4, 8): code 6 or 7."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1000, 256)) * np.exp(rng.uniform(-30, 30, (1000, 1)))
    codes, sb = O.quantize_blocks(x)
    amax = np.abs(x.reshape(1000, 8, 32)).max(-1)
    r = amax / np.ldexp(1.0, sb.astype(int) - 127)
    assert np.all((r >= 4) & (r < 8))
    assert np.all((codes.reshape(1000, 8, 32) & 7).max(-1) >= 6)


def test_quantisation_error_bound():
    """|x - q(x)| <= half a step of the E2M1 grid, saturation aside."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((500, 256))
    codes, sb = O.quantize_blocks(x)
    e = np.repeat(sb.astype(int) - 127, 32, axis=-1)
    dq = np.ldexp(O.e2m1_value(codes), e)
    r = np.abs(x) / np.ldexp(1.0, e)
    step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    err = np.abs(x - dq) / np.ldexp(1.0, e)
    inside = r <= 6
    assert np.all(err[inside] <= step[inside] / 2 + 1e-12)
    assert np.all((codes[~inside] & 7) == 7)


def test_zero_rotated_key_encodes_positive_zero():
    k = np.zeros((2, 256))
    k[0, 0], k[0, 1] = 1.0, 1.0          # rotated: 1/8 on even d, exactly 0 on odd d
    k[1, :] = -0.0                        # all -0 -> every rotated coordinate is 0
    v = np.zeros((2, 256))
    v[1, 3] = -0.0
    s = O.encode_slots(bf16(k), bf16(v))
    kc = O.unpack_nibbles(s[:, :128])
    assert np.all(kc[0, 1::2] == 0) and np.all(kc[0, 0::2] == 6)
    assert np.all(kc[1] == 0)
    vc = O.unpack_nibbles(s[:, 128:256])
    assert vc[1, 3] == 8 and vc[1, 2] == 0


def test_pack_order_fixture_slots():
    for case in golden_io.slot_cases():
        got = O.encode_slots(bf16(case["key"]), bf16(case["value"]))
        assert np.array_equal(got, case["bytes"]), case["name"]


# -------------------------------------------------------------- E4M3 haircut
def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(12)
    x = np.concatenate([
        rng.standard_normal(200000) * np.exp(rng.uniform(-14, 6, 200000)),
        O.E4M3_GRID, -O.E4M3_GRID,
        (O.E4M3_GRID[1:] + O.E4M3_GRID[:-1]) / 2,          # every midpoint
        -(O.E4M3_GRID[1:] + O.E4M3_GRID[:-1]) / 2,
        [0.0, -0.0, 448.0, 447.0, 464.0, -464.0],
    ])
    x = x[np.abs(x) <= 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_round(x)
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_e4m3_saturates():
    assert np.array_equal(O.e4m3_round(np.array([465.0, 1e4, -1e30])), [448.0, 448.0, -448.0])


# ----------------------------------------------------------------- attention
def _tiny_case(seed, L, Hk=1, qg=8, scale=1 / 16):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((1, Hk * qg, 256)))
    k = bf16(rng.standard_normal((L, Hk, 256)))
    v = bf16(rng.standard_normal((L, Hk, 256)))
    nblk = (L + 15) // 16
    cache = np.zeros((nblk + 3, 16, Hk, 272), dtype=np.uint8)
    table = rng.permutation(nblk + 3)[None, :nblk].astype(np.int32)
    t = np.arange(L)
    O.store(k, v, cache, table[0, t // 16].astype(np.int64) * 16 + t % 16)
    return q, k, v, cache, table, np.array([L], dtype=np.int32), scale


def test_decode_matches_sdpa_fp64():
    q, k, v, cache, table, lens, scale = _tiny_case(13, 77, Hk=2, qg=8)
    out = O.decode(q, cache, table, lens, scale)
    for h in range(2):
        K, V = O.gather_sequence(cache, table[0], 77, h)
        q8 = O.query_haircut(q[0, h * 8:(h + 1) * 8])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q8)[None, :, None, :],
            torch.from_numpy(K)[None, None].expand(1, 8, 77, 256),
            torch.from_numpy(V)[None, None].expand(1, 8, 77, 256),
            scale=scale)[0, :, 0].numpy()
        assert np.allclose(out[0, h * 8:(h + 1) * 8], ref, rtol=1e-12, atol=1e-12)


def test_decode_brute_force_loops():
    q, k, v, cache, table, lens, scale = _tiny_case(14, 21, Hk=1, qg=6)
    out = O.decode(q, cache, table, lens, scale)
    H = O.hadamard(256)
    for g in range(6):
        qf = O.bf16_to_f64(q[0, g])
        q8 = O.e4m3_round(np.array([sum(qf[i] * H[i, j] for i in range(256)) for j in range(256)]))
        # read every token's slot by hand through the block table
        scores, vals = [], []
        for t in range(21):
            slot = cache[table[0, t // 16], t % 16, 0]
            kq, vq = O.decode_slots(slot)
            scores.append(scale * sum(q8[d] * kq[d] for d in range(256)))
            vals.append(vq)
        mx = max(scores)
        w = [math.exp(s - mx) for s in scores]
        ref = sum(wi * vi for wi, vi in zip(w, vals)) / sum(w)
        assert np.allclose(out[0, g], ref, rtol=1e-12, atol=1e-13)


def test_decode_two_token_fixture():
    d = golden_io.decode_two_token()
    L = d["seq_len"]
    k = bf16(np.stack([d["key"][t] for t in range(L)])[:, None, :])
    v = bf16(np.stack([d["value"][t] for t in range(L)])[:, None, :])
    q = bf16(d["query"][None, None, :])
    cache = np.zeros((1, 16, 1, 272), dtype=np.uint8)
    O.store(k, v, cache, np.arange(L))
    out = O.decode(q, cache, np.zeros((1, 1), np.int32), np.array([L]), d["scale"])
    want = np.zeros(256)
    for i, x in d["out"].items():
        want[i] = x
    assert np.allclose(out[0, 0], want, rtol=1e-15, atol=1e-15)


def test_single_token_returns_dequantised_value():
    q, k, v, cache, table, lens, scale = _tiny_case(15, 1)
    out = O.decode(q, cache, table, lens, scale)
    _, V = O.gather_sequence(cache, table[0], 1, 0)
    assert np.array_equal(out[0], np.broadcast_to(V[0], out[0].shape))


def test_zero_query_gives_mean_of_values():
    q, k, v, cache, table, lens, scale = _tiny_case(16, 50)
    q[:] = 0
    out = O.decode(q, cache, table, lens, scale)
    _, V = O.gather_sequence(cache, table[0], 50, 0)
    assert np.allclose(out[0], V.mean(0), rtol=1e-13, atol=1e-14)


def test_dominant_key_selects_its_value():
    q, k, v, cache, table, lens, scale = _tiny_case(17, 40)
    K, V = O.gather_sequence(cache, table[0], 40, 0)
    # query = the (un-rotated) key of token 11 -> its score dominates with a big scale
    qv = O.bf16_to_f64(k[11, 0])
    q[0, :] = bf16(qv * 4)
    out = O.decode(q, cache, table, lens, 8.0)
    assert np.allclose(out[0, 0], V[11], atol=1e-6)


def test_empty_sequence_gives_zeros():
    q, k, v, cache, table, lens, scale = _tiny_case(23, 30)
    out = O.decode(q, cache, table, np.array([0]), scale)
    assert np.array_equal(out, np.zeros_like(out))


def test_split_merge_equals_single_softmax():
    q, k, v, cache, table, lens, scale = _tiny_case(18, 203)
    K, V = O.gather_sequence(cache, table[0], 203, 0)
    q8 = O.query_haircut(q[0])
    ref = O.attention(q8, K, V, scale)
    for bounds in ([0, 203], [0, 64, 128, 192, 203], [0, 0, 50, 50, 203, 203], list(range(0, 203, 16)) + [203]):
        got = O.attention_split(q8, K, V, scale, bounds)
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- the cache
def test_store_order_and_batching_invariant():
    rng = np.random.default_rng(19)
    k = bf16(rng.standard_normal((40, 2, 256)))
    v = bf16(rng.standard_normal((40, 2, 256)))
    slots = rng.permutation(64)[:40]
    a = np.zeros((4, 16, 2, 272), dtype=np.uint8)
    O.store(k, v, a, slots)
    b = np.zeros_like(a)
    perm = rng.permutation(40)
    for chunk in np.array_split(perm, 5):
        O.store(k[chunk], v[chunk], b, slots[chunk])
    assert np.array_equal(a, b)


def test_store_leaves_other_slots_and_skips_negative():
    rng = np.random.default_rng(20)
    k = bf16(rng.standard_normal((10, 1, 256)))
    v = bf16(rng.standard_normal((10, 1, 256)))
    cache = np.full((2, 16, 1, 272), 0xA5, dtype=np.uint8)
    slots = np.array([3, -1, 7, 8, -1, 30, 0, 1, 2, 31])
    O.store(k, v, cache, slots)
    flat = cache.reshape(32, 272)
    untouched = sorted(set(range(32)) - set(slots[slots >= 0].tolist()))
    assert np.all(flat[untouched] == 0xA5)
    assert not np.all(flat[3] == 0xA5)


def test_block_permutation_leaves_output_unchanged():
    q, k, v, cache, table, lens, scale = _tiny_case(21, 90)
    ref = O.decode(q, cache, table, lens, scale)
    rng = np.random.default_rng(22)
    perm = rng.permutation(cache.shape[0])        # new home of physical block p
    moved = np.empty_like(cache)
    moved[perm] = cache
    got = O.decode(q, moved, perm[table].astype(np.int32), lens, scale)
    assert np.array_equal(got, ref)


# ------------------------------------------------- sinks and sliding window
def test_sink_one_token_closed_form():
    """One token and a sink s: the weight of the token is 1 / (1 + e^(s - x))
    with x its scaled score, computed here by an explicit sum."""
    q, k, v, cache, table, lens, scale = _tiny_case(31, 1, qg=6)
    _, V = O.gather_sequence(cache, table[0], 1, 0)
    K, _ = O.gather_sequence(cache, table[0], 1, 0)
    sinks = np.array([-3.0, -0.5, 0.0, 0.7, 2.0, 9.0])
    out = O.decode(q, cache, table, lens, scale, sinks=sinks)
    for g in range(6):
        q8 = O.query_haircut(q[0, g])
        x = scale * sum(q8[d] * K[0, d] for d in range(256))
        w = 1.0 / (1.0 + math.exp(sinks[g] - x))
        assert np.allclose(out[0, g], w * V[0], rtol=1e-12, atol=1e-14)


def test_sink_matches_library_softmax_with_extra_logit():
    """torch's softmax over the token logits plus the sink logit, keeping
    only the tokens' weights."""
    q, k, v, cache, table, lens, scale = _tiny_case(32, 45, Hk=2, qg=8)
    rng = np.random.default_rng(33)
    sinks = rng.normal(0, 2, 16)
    out = O.decode(q, cache, table, lens, scale, sinks=sinks)
    for h in range(2):
        K, V = O.gather_sequence(cache, table[0], 45, h)
        q8 = torch.from_numpy(O.query_haircut(q[0, h * 8:(h + 1) * 8]))
        logits = scale * (q8 @ torch.from_numpy(K).T)
        full = torch.cat([logits, torch.from_numpy(sinks[h * 8:(h + 1) * 8])[:, None]], dim=1)
        p = torch.softmax(full, dim=1)[:, :45]
        ref = (p @ torch.from_numpy(V)).numpy()
        assert np.allclose(out[0, h * 8:(h + 1) * 8], ref, rtol=1e-12, atol=1e-14)


def test_sink_minus_infinity_is_no_sink_and_scales_output():
    q, k, v, cache, table, lens, scale = _tiny_case(34, 60)
    base = O.decode(q, cache, table, lens, scale)
    assert np.array_equal(O.decode(q, cache, table, lens, scale, sinks=np.full(8, -np.inf)), base)
    # a finite sink scales every output element of a head by Z / (Z + e^s),
    # Z = sum of e^(scores), here summed token by token
    K, _ = O.gather_sequence(cache, table[0], 60, 0)
    s = np.linspace(-2, 3, 8)
    out = O.decode(q, cache, table, lens, scale, sinks=s)
    for g in range(8):
        q8 = O.query_haircut(q[0, g])
        xs = [scale * float(np.dot(q8, K[t])) for t in range(60)]
        Z = sum(math.exp(x) for x in xs)
        assert np.allclose(out[0, g], base[0, g] * (Z / (Z + math.exp(s[g]))), rtol=1e-11, atol=1e-14)


def test_empty_sequence_with_sink_gives_zeros():
    q, k, v, cache, table, lens, scale = _tiny_case(35, 10)
    out = O.decode(q, cache, table, np.array([0]), scale, sinks=np.zeros(8))
    assert np.array_equal(out, np.zeros_like(out))


def test_sliding_window_cases():
    q, k, v, cache, table, lens, scale = _tiny_case(36, 70, Hk=2, qg=8)
    base = O.decode(q, cache, table, lens, scale)
    # a window at least as long as the sequence changes nothing
    assert np.array_equal(O.decode(q, cache, table, lens, scale, sliding_window=70), base)
    assert np.array_equal(O.decode(q, cache, table, lens, scale, sliding_window=1000), base)
    # a window of one token returns that token's value exactly
    out1 = O.decode(q, cache, table, lens, scale, sliding_window=1)
    for h in range(2):
        _, V = O.gather_sequence(cache, table[0], 70, h)
        assert np.array_equal(out1[0, h * 8:(h + 1) * 8], np.broadcast_to(V[69], (8, 256)))
    # a window of 23: torch SDPA over the last 23 tokens
    out = O.decode(q, cache, table, lens, scale, sliding_window=23)
    for h in range(2):
        K, V = O.gather_sequence(cache, table[0], 70, h)
        q8 = O.query_haircut(q[0, h * 8:(h + 1) * 8])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q8)[None, :, None, :],
            torch.from_numpy(K[47:])[None, None].expand(1, 8, 23, 256),
            torch.from_numpy(V[47:])[None, None].expand(1, 8, 23, 256),
            scale=scale)[0, :, 0].numpy()
        assert np.allclose(out[0, h * 8:(h + 1) * 8], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- continuation prefill
def test_bf16_round_matches_library_cast_and_rounds_once():
    """Where float32 holds the value exactly, one rounding to bf16 is torch's
    float32 -> bfloat16 cast (nearest, ties to even); a value just above a
    tie that float32 would first round onto the tie goes up, as one rounding
    of the exact value must."""
    rng = np.random.default_rng(0)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 120, 20000))).astype(np.float32)
    f = np.concatenate([f, np.float32([0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 3.3961e38, 3.3965e38])])
    want = torch.from_numpy(f).to(torch.bfloat16).float().numpy().astype(np.float64)
    got = O.bf16_round(f.astype(np.float64))
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
    assert O.bf16_round(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 1 + 2 ** -7
    assert O.bf16_round(np.array([-(1 + 2 ** -8 + 2 ** -40)]))[0] == -(1 + 2 ** -7)


def _prefix_cache(rng, cached_len, hk, bs=16, k=None, v=None):
    """A cache holding a sequence's first cached_len tokens (oracle store),
    its blocks in a shuffled order."""
    nblk = max(1, -(-cached_len // bs))
    row = rng.permutation(nblk + 2)[:nblk].astype(np.int32)
    cache = np.zeros((nblk + 2, bs, hk, O.SLOT_BYTES), dtype=np.uint8)
    if cached_len:
        kk = k if k is not None else bf16(rng.standard_normal((cached_len, hk, 256)))
        vv = v if v is not None else bf16(rng.standard_normal((cached_len, hk, 256)))
        t = np.arange(cached_len)
        O.store(kk, vv, cache, row[t // bs].astype(np.int64) * bs + t % bs)
    return cache, row


@pytest.mark.parametrize("cached_len", [0, 1, 16, 37])
def test_prefill_zero_query_is_running_mean(cached_len):
    """q = 0: every visible key weighs the same, so query i returns the mean
    of values 0 .. cached_len + i (the dequantised prefix, then the chunk):
    pins the lower-right alignment and the order of prefix and chunk."""
    rng = np.random.default_rng(cached_len)
    q_len, hk, qg = 9, 2, 3
    cache, row = _prefix_cache(rng, cached_len, hk)
    q = bf16(np.zeros((q_len, hk * qg, 256)))
    kc = bf16(rng.standard_normal((q_len, hk, 256)))
    vc = bf16(rng.standard_normal((q_len, hk, 256)))
    out = O.continuation_prefill(q, kc, vc, cache, row, cached_len, 0.3)
    _, Vp = O.dequant_prefix(cache, row, cached_len)
    V = np.concatenate([Vp, O.bf16_to_f64(vc)], axis=0)
    run = np.cumsum(V, axis=0) / np.arange(1, len(V) + 1)[:, None, None]
    for i in range(q_len):
        for hq in range(hk * qg):
            np.testing.assert_allclose(out[i, hq], run[cached_len + i, hq // qg], rtol=1e-12, atol=1e-12)


def test_prefill_rotation_consistent_between_prefix_chunk_and_query():
    """Rows of 16 H rotate to 16 e_j exactly, and so store exactly as FP4
    (code 4 under scale 2**2). With query i = 16 H[j_i] and every key a row
    16 H[j] (prefix through the cache, chunk through the rotation), a score
    is 256 * scale where the rows match and 0 elsewhere, so each output has
    a closed form over the visible tokens. A rotation missing or applied
    differently on one side breaks the match pattern."""
    rng = np.random.default_rng(5)
    H16 = O.hadamard(256) * 16
    cached_len, q_len, hk, qg = 21, 6, 2, 2
    idx_k = rng.integers(0, 4, (cached_len + q_len, hk))
    idx_q = rng.integers(0, 4, (q_len, hk * qg))
    keys = H16[idx_k]                                        # (seq, hk, 256), entries +-1
    vals = rng.standard_normal((cached_len + q_len, hk, 256))
    kb, vb = bf16(keys), bf16(vals)
    cache, row = _prefix_cache(rng, cached_len, hk, k=kb[:cached_len], v=vb[:cached_len])
    scale = 1 / 64                                           # match score 4
    out = O.continuation_prefill(bf16(H16[idx_q]), kb[cached_len:], vb[cached_len:], cache, row,
                                 cached_len, scale)
    _, Vp = O.dequant_prefix(cache, row, cached_len)
    V = np.concatenate([Vp, O.bf16_to_f64(vb[cached_len:])], axis=0)
    for i in range(q_len):
        n = cached_len + i + 1
        for hq in range(hk * qg):
            h = hq // qg
            w = np.where(idx_k[:n, h] == idx_q[i, hq], math.exp(4.0), 1.0)
            want = (w[:, None] * V[:n, h]).sum(0) / w.sum()
            np.testing.assert_allclose(out[i, hq], want, rtol=1e-12, atol=1e-12)


def test_prefill_first_query_without_prefix_is_first_value():
    rng = np.random.default_rng(7)
    q = bf16(rng.standard_normal((4, 8, 256)))
    kc = bf16(rng.standard_normal((4, 1, 256)))
    vc = bf16(rng.standard_normal((4, 1, 256)))
    cache, row = _prefix_cache(rng, 0, 1)
    out = O.continuation_prefill(q, kc, vc, cache, row, 0, 0.1)
    assert np.array_equal(out[0], np.broadcast_to(O.bf16_to_f64(vc[0, 0]), (8, 256)))


def test_prefill_matches_brute_force_loops():
    """Tiny case against explicit loops over queries, keys and d, with the
    rotation as a plain sum over H's entries written (-1)**popcount / 16."""
    rng = np.random.default_rng(8)
    cached_len, q_len, hk, qg, bs = 5, 3, 2, 2, 4
    cache, row = _prefix_cache(rng, cached_len, hk, bs=bs)
    q = bf16(rng.standard_normal((q_len, hk * qg, 256)))
    kc = bf16(rng.standard_normal((q_len, hk, 256)))
    vc = bf16(rng.standard_normal((q_len, hk, 256)))
    scale = 0.07
    got = O.continuation_prefill(q, kc, vc, cache, row, cached_len, scale)

    def rot_bf16(bits):
        x = [float(v) for v in O.bf16_to_f64(bits)]
        y = [sum(x[i] * (-1) ** bin(i & j).count("1") for i in range(256)) / 16 for j in range(256)]
        return [float(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double()) for v in y]

    for h in range(hk):
        keys, vals = [], []
        for t in range(cached_len):
            slot = cache[row[t // bs], t % bs, h]
            k_t, v_t = O.decode_slots(slot)
            keys.append(list(k_t))
            vals.append(list(v_t))
        for t in range(q_len):
            keys.append(rot_bf16(kc[t, h]))
            vals.append(list(O.bf16_to_f64(vc[t, h])))
        for hq in range(h * qg, (h + 1) * qg):
            for i in range(q_len):
                qi = rot_bf16(q[i, hq])
                n = cached_len + i + 1
                s = [scale * sum(qi[d] * keys[j][d] for d in range(256)) for j in range(n)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                want = [sum(w[j] * vals[j][d] for j in range(n)) / sum(w) for d in range(256)]
                np.testing.assert_allclose(got[i, hq], want, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------ other head dims
@pytest.mark.parametrize("n", [128, 512])
def test_rotation_other_head_dims_is_exact_sum_then_one_rounding(n):
    """For n where sqrt(n) is not a power of two the rotation is the exact
    +-1 sum times fl64(1/sqrt(n)), rounded once: checked with Fractions."""
    rng = np.random.default_rng(n)
    x = O.bf16_to_f64(bf16(rng.standard_normal((3, n)) * np.exp2(rng.integers(-6, 6, (3, n)))))
    y = O.rotate(x)
    c = fractions.Fraction(O.rot_scale(n))
    # the scale is the float64 nearest 1/sqrt(n): c^2 n closest to 1 among its neighbours
    err = lambda f: abs(fractions.Fraction(f) ** 2 * n - 1)
    assert err(O.rot_scale(n)) < min(err(np.nextafter(O.rot_scale(n), 0)), err(np.nextafter(O.rot_scale(n), 1)))
    for r in range(3):
        for j in rng.integers(0, n, 12):
            s = sum(fractions.Fraction(float(x[r, i])) * (-1) ** bin(i & int(j)).count("1") for i in range(n))
            assert y[r, j] == float(s * c)
    # orthonormal: scores survive the rotation up to float64 rounding
    q, k = rng.standard_normal(n), rng.standard_normal(n)
    qb, kb = O.bf16_to_f64(bf16(q)), O.bf16_to_f64(bf16(k))
    assert abs(O.rotate(qb) @ O.rotate(kb) - qb @ kb) < 1e-12 * n


@pytest.mark.parametrize("n", [128, 512])
def test_slot_layout_other_head_dims_round_trip(n):
    """Values E2M1 represents exactly under their block scale survive
    encode/decode; the sections have the sizes of the layout."""
    rng = np.random.default_rng(n + 1)
    nbytes, kco, vco, kso, vso = O.slot_layout(n)
    assert (nbytes, kco, vco, kso, vso) == (n * 17 // 16, 0, n // 2, n, n + n // 32)
    blocks = n // 32
    v = rng.choice(O.E2M1_MAGNITUDES, (5, n)) * rng.choice([-1, 1], (5, n))
    v[:, ::32] = 6.0                                          # every block's amax is 6: scale byte 127
    v = v * np.repeat(np.exp2(rng.integers(-3, 4, (5, blocks))), 32, axis=1)
    vb = bf16(v)
    kb = bf16(np.zeros((5, n)))
    slots = O.encode_slots(kb[:, None, :], vb[:, None, :])
    assert slots.shape == (5, 1, nbytes)
    K, V = O.decode_slots(slots)
    assert np.array_equal(V[:, 0], O.bf16_to_f64(vb)) and np.all(K == 0)


@pytest.mark.parametrize("n", [128, 512])
def test_decode_other_head_dims_matches_brute_force(n):
    rng = np.random.default_rng(n + 2)
    L, hk, qg, bs = 21, 1, 2, 16
    k = bf16(rng.standard_normal((L, hk, n)))
    v = bf16(rng.standard_normal((L, hk, n)))
    cache = np.zeros((3, bs, hk, O.slot_layout(n)[0]), dtype=np.uint8)
    O.store(k, v, cache, np.arange(L) + 5)
    table = np.array([[0, 1, 2]], dtype=np.int32)
    lens = np.array([L + 5])                               # tokens 0..4 are empty slots (zeros)
    q = bf16(rng.standard_normal((1, hk * qg, n)))
    out = O.decode(q, cache, table, lens, 0.1)
    Kq, Vq = O.decode_slots(cache.reshape(-1, hk, cache.shape[-1])[:L + 5, 0])
    for hq in range(qg):
        q8 = O.e4m3_round(O.rotate(O.bf16_to_f64(q[0, hq])))
        s = [0.1 * float(np.dot(q8, Kq[t])) for t in range(L + 5)]
        w = [math.exp(x - max(s)) for x in s]
        want = sum(wi * Vq[t] for t, wi in enumerate(w)) / sum(w)
        np.testing.assert_allclose(out[0, hq], want, rtol=1e-12, atol=1e-12)
