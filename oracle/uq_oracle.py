"""CPU oracle for UltraQuant 4-bit paged-KV decode attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the library never calls it and it
imports nothing from the library.

Plain, slow numpy float64. Every function cites the passage it follows on the
pages (vLLM API docs):
  [UQ-impl]  "vllm/v1/attention/backends/ultraquant_attn", class
             UltraQuantAttentionImpl: _ensure_on_device, _store_kv,
             _decode_attention, _ultraquant_continuation_prefill.
  [UQ-fly]   "vllm/v1/attention/ops/flydsl_ultraquant_decode": module text,
             _SegmBufPool, _fp4_value_lut, flydsl_ultraquant_decode_attention.
  [TQ-v2]    "vllm/v1/attention/ops/turboquant_soa/triton_turboquant_decode_v2":
             triton_turboquant_decode_attention_v2 (split-KV stage 1 / 2).
The pages name the formats (FP4 E2M1, UE8M0, E4M3) but print neither the value
tables, the scale rule nor the byte layout of a slot. Those are taken from the
OCP Microscaling Formats (MX) v1.0 and OCP 8-bit Floating Point specs, as
stated at each function.

Parity pins: the Hadamard, the rotation, E2M1 values and rounding, UE8M0 and
E4M3 decoding, the attention, bf16 rounding and the continuation prefill
(alignment, rotation of both sides, brute force) are pinned by closed forms,
library routines and brute force in tests/. Parity unpinned (no passage of the pages fixes
them; they are pinned by their own definitions only): the 32-element block
partition, the UE8M0 scale-selection rule, the nibble packing order and the
272-byte slot layout.
"""
from __future__ import annotations

import numpy as np

D = 256                             # the head dim of the pages' decode path
MX_BLOCK = 32                       # elements per UE8M0 scale
SLOT_BYTES = 272                    # 128 K codes + 128 V codes + 8 + 8 scales (D = 256)
K_CODE_OFF, V_CODE_OFF = 0, 128
K_SCALE_OFF, V_SCALE_OFF = 256, 264
HEAD_DIMS = (128, 256, 512)         # head dims of the slot format


def slot_layout(d: int):
    """(slot bytes, K code, V code, K scale, V scale offsets) for head dim d:
    d/2 bytes of K codes, d/2 of V codes, then d/32 K and d/32 V scale bytes
    (272 bytes and offsets 0, 128, 256, 264 at d = 256)."""
    assert d in HEAD_DIMS
    return d * 17 // 16, 0, d // 2, d, d + d // MX_BLOCK


def head_dim_of_slot(slot_bytes: int) -> int:
    d = slot_bytes * 16 // 17
    assert slot_layout(d)[0] == slot_bytes
    return d

# OCP MX v1.0, FP4 E2M1: magnitudes of the eight non-negative codes
# (exponent bias 1, one mantissa bit, code 0b001 is the subnormal 0.5).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_EMAX = 2                       # exponent of the largest normal, 6 = 1.5 * 2**2


# --------------------------------------------------------------------------
# bf16 plumbing
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Rotation ([UQ-impl] _ensure_on_device: the rotation is a pure Hadamard,
# orthonormal and symmetric, so PiT = Pi = H; _store_kv rotates K by it;
# continuation prefill rotates with x @ PiT)
# --------------------------------------------------------------------------
def hadamard(n: int = D) -> np.ndarray:
    """Normalised Sylvester Hadamard: H[i, j] = (-1)**popcount(i & j) / sqrt(n).

    Symmetric and orthonormal, as [UQ-impl] _ensure_on_device requires. The
    pages do not fix the row order; the Sylvester (natural) order is the one a
    radix-2 butterfly produces.
    """
    assert n > 0 and n & (n - 1) == 0
    i = np.arange(n)
    parity = np.zeros((n, n), dtype=np.int64)
    x = i[:, None] & i[None, :]
    while np.any(x):
        parity ^= x & 1
        x = x >> 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(n)


_H = hadamard(D)
_SYLVESTER = {}


def sylvester(n: int) -> np.ndarray:
    """The unnormalised Sylvester Hadamard, entries +-1 (H = sylvester / sqrt(n))."""
    if n not in _SYLVESTER:
        _SYLVESTER[n] = np.rint(hadamard(n) * np.sqrt(n))
    return _SYLVESTER[n]


# Exactness of the rotation. Let the non-zero magnitudes of a bf16 vector of n
# values have exponents (floor log2) from emin to emax, span = emax - emin.
# Every value is an integer multiple of u = 2**(emin - 7) (8 significant bits)
# and at most 255 * 2**span units, so every +-sum of the n values is an
# integer number of units of magnitude at most n * 255 * 2**span. That
# integer is exact in float64 (53 bits) whenever n * 255 * 2**span < 2**53,
# i.e. span <= 45 - log2(n) (37 binades at n = 256, 38 at 128, 36 at 512), and
# then x @ sylvester(n) is exact in any summation order. One binade more and
# n - 1 values of 255 units plus one of 129 units sum to an odd integer above
# 2**53, which no float64 holds.
def max_exact_span(n: int) -> int:
    return 45 - int(np.log2(n))


MAX_EXACT_SPAN = max_exact_span(D)


def exact_span_ok(x: np.ndarray) -> np.ndarray:
    """Per vector (last axis): True when the +-1 sums of x are exact in float64."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    nz = a > 0
    e = np.where(nz, np.frexp(np.where(nz, a, 1.0))[1], 0)
    emax = np.where(nz, e, np.iinfo(np.int64).min).max(axis=-1)
    emin = np.where(nz, e, np.iinfo(np.int64).max).min(axis=-1)
    return (~nz.any(axis=-1)) | (emax - emin <= max_exact_span(a.shape[-1]))


def rot_scale(n: int) -> float:
    """The float64 nearest 1/sqrt(n) for n a power of two: 2**(-e/2) for
    n = 2**e with e even, else sqrt(2) * 2**(-(e+1)/2) (IEEE sqrt is
    correctly rounded and the power of two is exact)."""
    e = int(np.log2(n))
    assert 1 << e == n
    return 2.0 ** (-(e // 2)) if e % 2 == 0 else np.sqrt(2.0) * 2.0 ** (-((e + 1) // 2))


def rotate(x: np.ndarray) -> np.ndarray:
    """y = x @ H over the last axis ([UQ-impl] _store_kv; key_chunk @ PiT).

    Computed as the exact +-1 sums x @ sylvester(n) times rot_scale(n) (the
    float64 nearest 1/sqrt(n)), one rounding (a reading: the pages leave the
    rounding open where sqrt(n) is not a power of two, n = 128 or 512; for
    n = 256 the scale 1/16 is exact and so is y)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if not np.all(exact_span_ok(x)):
        raise ValueError(f"input spans more than {max_exact_span(n)} binades: the sums would not be exact")
    if n == D:
        return x @ _H
    return (x @ sylvester(n)) * rot_scale(n)


# --------------------------------------------------------------------------
# Block scale and FP4 E2M1 code ([UQ-impl] class docstring: "FP4 E2M1 + UE8M0,
# rotated K"; [UQ-fly] _fp4_value_lut: lut[nibble] is the dequant value)
# --------------------------------------------------------------------------
def ue8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """Shared block exponent, OCP MX v1.0 rule: floor(log2 amax) - emax_elem.

    emax_elem = 2 for E2M1. Clamped to the UE8M0 range [-127, 127]; an
    all-zero block takes -127. floor(log2) is read from the float64 exponent
    field, which is exact.
    """
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    _, ex = np.frexp(np.where(pos, a, 1.0))       # a = m * 2**ex, m in [0.5, 1)
    e = (ex - 1) - E2M1_EMAX
    e = np.where(pos, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def e2m1_round(r: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of r >= 0: nearest E2M1 magnitude, ties to the
    even code, saturating at 6 (code 7)."""
    r = np.asarray(r, dtype=np.float64)
    dist = np.abs(r[..., None] - E2M1_MAGNITUDES)
    best = dist.min(axis=-1, keepdims=True)
    tie = dist == best
    # among the nearest candidates, prefer the even code (even mantissa bit)
    codes = np.arange(8)
    pref = np.where(tie, np.where(codes % 2 == 0, 0, 1) * 8 + codes, 99)
    code = pref.argmin(axis=-1)
    return np.where(r > 6.0, 7, code).astype(np.uint8)


def e2m1_encode(x: np.ndarray, e: np.ndarray) -> np.ndarray:
    """4-bit codes of x under block exponent e: sign bit 3 = signbit(x),
    magnitude code of |x| / 2**e."""
    x = np.asarray(x, dtype=np.float64)
    r = np.ldexp(np.abs(x), -np.asarray(e))
    mag = e2m1_round(r)
    sign = np.signbit(x).astype(np.uint8) << 3
    return (sign | mag).astype(np.uint8)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes (the 16-entry table [UQ-fly] _fp4_value_lut)."""
    c = np.asarray(code, dtype=np.int64)
    v = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -v, v)


def quantize_blocks(x: np.ndarray):
    """Split the last axis (d) into d/32 blocks of 32 consecutive elements.

    Returns (codes (..., d) uint8 in 0..15, scale bytes (..., d/32) uint8).
    """
    x = np.asarray(x, dtype=np.float64)
    xb = x.reshape(*x.shape[:-1], x.shape[-1] // MX_BLOCK, MX_BLOCK)
    e = ue8m0_exponent(np.abs(xb).max(axis=-1))
    codes = e2m1_encode(xb, e[..., None]).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte, element 2i in bits 0-3 and 2i+1 in bits 4-7."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# Store ([UQ-impl] _store_kv: key, value (N, Hk, D); kv_cache
# (num_blocks, block_size, Hk, slot_size); slot_mapping; "Rotate K by the
# Hadamard and pack K+V into FP4/UE8M0 slots")
# --------------------------------------------------------------------------
def encode_slots(key_bits: np.ndarray, value_bits: np.ndarray) -> np.ndarray:
    """Slot bytes (..., 272) of bf16 key/value vectors (..., 256).

    Slot layout: [0,128) K codes, [128,256) V codes, [256,264) K scale bytes,
    [264,272) V scale bytes. K is rotated before quantisation, V is not
    ([UQ-impl] continuation prefill copies V unrotated). Other head dims d
    scale every section (slot_layout).
    """
    # A rotated coordinate that is exactly zero has no sign of its own (its
    # float sign would depend on the summation order); it is encoded as +0.
    # V is copied as-is and keeps the sign of a -0 input.
    k = rotate(bf16_to_f64(key_bits)) + 0.0
    v = bf16_to_f64(value_bits)
    kc, ks = quantize_blocks(k)
    vc, vs = quantize_blocks(v)
    d = k.shape[-1]
    nbytes, kco, vco, kso, vso = slot_layout(d)
    out = np.empty(k.shape[:-1] + (nbytes,), dtype=np.uint8)
    out[..., kco:kco + d // 2] = pack_nibbles(kc)
    out[..., vco:vco + d // 2] = pack_nibbles(vc)
    out[..., kso:kso + d // MX_BLOCK] = ks
    out[..., vso:vso + d // MX_BLOCK] = vs
    return out


def store(key_bits, value_bits, kv_cache: np.ndarray, slot_mapping) -> None:
    """Write token n of (N, Hk, D) key/value into flat slot slot_mapping[n]
    of kv_cache (num_blocks, block_size, Hk, 272); negative slots are
    skipped."""
    key_bits = np.asarray(key_bits)
    value_bits = np.asarray(value_bits)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    nb, bs, hk, ss = kv_cache.shape
    assert ss == slot_layout(key_bits.shape[-1])[0] and key_bits.shape[1] == hk
    flat = kv_cache.reshape(nb * bs, hk, ss)
    keep = slots >= 0
    if not np.any(keep):
        return
    flat[slots[keep]] = encode_slots(key_bits[keep], value_bits[keep])


def decode_slots(slot_bytes: np.ndarray):
    """Dequantised (K, V) float64 (..., d) of slot bytes (..., 17 d / 16)
    (d = 256: 272-byte slots).

    K stays in the rotated basis. value = E2M1(code) * 2**(byte - 127).
    """
    s = np.asarray(slot_bytes, dtype=np.uint8)
    d = head_dim_of_slot(s.shape[-1])
    _, kco, vco, kso, vso = slot_layout(d)
    nblk = d // MX_BLOCK

    def part(code_off, scale_off):
        codes = unpack_nibbles(s[..., code_off:code_off + d // 2])
        e = s[..., scale_off:scale_off + nblk].astype(np.int64) - 127
        vals = e2m1_value(codes).reshape(*codes.shape[:-1], nblk, MX_BLOCK)
        return np.ldexp(vals, e[..., None]).reshape(codes.shape)

    return part(kco, kso), part(vco, vso)


# --------------------------------------------------------------------------
# Query haircut ([UQ-fly] _SegmBufPool docstring: q_rot_fp32 -> fp8_e4m3 ->
# bf16; launcher: "Always apply the E4M3 haircut: scaled QK consumes Q as
# E4M3"; the four-op prologue copies q to fp32, multiplies by PiT, casts to
# float8_e4m3fn and back)
# --------------------------------------------------------------------------
def _e4m3_grid() -> np.ndarray:
    """All non-negative finite OCP E4M3 (fn) values, indexed by code 0..126."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


E4M3_GRID = _e4m3_grid()            # last entry is 448, the largest finite value


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3 (fn) value, ties to the even code; signed zero kept.

    Magnitudes above 448 saturate to 448. The pages' cast is not specified
    beyond the format; above 464 round-to-nearest would produce NaN in this
    format, so saturation is the reading taken here.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    idx = np.searchsorted(E4M3_GRID, a)           # first grid value >= a
    idx = np.clip(idx, 1, len(E4M3_GRID) - 1)
    lo, hi = E4M3_GRID[idx - 1], E4M3_GRID[idx]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (idx % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(a >= 448.0, 448.0, mag)
    mag = np.where(a == 0, 0.0, mag)
    return np.copysign(mag, x)


def query_haircut(query_bits: np.ndarray) -> np.ndarray:
    """q8 = E4M3(q @ H) per query head, float64 values."""
    return e4m3_round(rotate(bf16_to_f64(query_bits)))


# --------------------------------------------------------------------------
# Decode ([UQ-impl] _decode_attention / [UQ-fly] launcher: query (B, Hq, D),
# kv_cache, block_table, seq_lens, scale -> output (B, Hq, D) in the query
# dtype; query head hq reads KV head hq // (Hq // Hk))
# --------------------------------------------------------------------------
def gather_sequence(kv_cache: np.ndarray, block_row: np.ndarray, L: int, h: int):
    """Dequantised (K, V) (L, 256) of KV head h for the first L tokens of a
    sequence whose logical block j lives in physical block block_row[j]."""
    nb, bs, hk, ss = kv_cache.shape
    t = np.arange(L)
    phys = np.asarray(block_row, dtype=np.int64)[t // bs]
    return decode_slots(kv_cache[phys, t % bs, h])


def attention(q8: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, sinks=None) -> np.ndarray:
    """softmax(scale * q8 K^T) V over all tokens, float64; q8 (G, 256).

    The decode query is the last position and seq_lens counts it, so no mask.
    Scores use the rotated K directly: (qH).(kH) = q.k because H is orthonormal
    ([UQ-impl] continuation prefill: rotating both sides leaves scores
    unchanged).

    ``sinks`` (G,) are per-head sink logits ([UQ-impl] passes ``self.sinks``
    to the unified attention kernel; the reading taken here, as in attention
    with sinks: one more logit per head in the softmax normaliser, with no
    value behind it, in the units of the scaled scores).
    """
    s = scale * (q8 @ K.T)
    if sinks is None:
        m = s.max(axis=-1, keepdims=True)
        p = np.exp(s - m)
        return (p @ V) / p.sum(axis=-1, keepdims=True)
    sk = np.asarray(sinks, dtype=np.float64)[:, None]
    m = np.maximum(s.max(axis=-1, keepdims=True) if s.shape[-1] else -np.inf, sk)
    p = np.exp(s - m)
    return (p @ V) / (p.sum(axis=-1, keepdims=True) + np.exp(sk - m))


def decode(query_bits, kv_cache, block_table, seq_lens, scale, pairs=None, sinks=None,
           sliding_window=0) -> np.ndarray:
    """Reference output (B, Hq, d) float64, single softmax per query head.

    ``pairs`` optionally restricts the work to a list of (b, kv_head); other
    rows are left NaN. ``sinks`` (Hq,) are per-query-head sink logits (see
    ``attention``). ``sliding_window`` W > 0 limits each query to the last W
    tokens of its sequence: the dense path on [UQ-impl] passes the window as
    (W - 1, 0), i.e. a query sees itself and the W - 1 keys before it.
    """
    query_bits = np.asarray(query_bits)
    B, Hq, d = query_bits.shape
    hk = kv_cache.shape[2]
    qg = Hq // hk
    out = np.full((B, Hq, d), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(hk)]
    for b, h in todo:
        L = int(seq_lens[b])
        if L <= 0:
            # no key to attend to: the empty weighted sum, zero (a reading;
            # the pages only decode sequences holding the new token)
            out[b, h * qg:(h + 1) * qg] = 0.0
            continue
        K, V = gather_sequence(kv_cache, block_table[b], L, h)
        if sliding_window and sliding_window > 0:
            K, V = K[max(0, L - sliding_window):], V[max(0, L - sliding_window):]
        q8 = query_haircut(query_bits[b, h * qg:(h + 1) * qg])
        sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)[h * qg:(h + 1) * qg]
        out[b, h * qg:(h + 1) * qg] = attention(q8, K, V, scale, sk)
    return out


def partial_attention(q8, K, V, scale):
    """One split of [TQ-v2] stage 1: normalised partial output, running max
    and sum of exponentials (m = -inf, l = 0 for an empty range)."""
    if K.shape[0] == 0:
        return np.zeros(q8.shape), np.full(q8.shape[0], -np.inf), np.zeros(q8.shape[0])
    s = scale * (q8 @ K.T)
    m = s.max(axis=-1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=-1)
    return (p @ V) / l[:, None], m, l


def merge_partials(o, m, l):
    """[TQ-v2] stage 2 log-sum-exp merge of split partials (S, G, 256)."""
    M = m.max(axis=0)
    w = np.where(l > 0, l * np.exp(m - M[None, :]), 0.0)
    return (w[..., None] * o).sum(axis=0) / w.sum(axis=0)[:, None]


def attention_split(q8, K, V, scale, bounds) -> np.ndarray:
    """Split-KV attention over token ranges [bounds[i], bounds[i+1])."""
    parts = [partial_attention(q8, K[a:b], V[a:b], scale) for a, b in zip(bounds[:-1], bounds[1:])]
    o = np.stack([p[0] for p in parts])
    m = np.stack([p[1] for p in parts])
    l = np.stack([p[2] for p in parts])
    return merge_partials(o, m, l)


# --------------------------------------------------------------------------
# Continuation prefill ([UQ-impl] _prefill_attention, continuation branch for
# chunks above the decode threshold, and _ultraquant_continuation_prefill:
# the cached prefix is dequantised in the rotated basis, the chunk's K and the
# queries are rotated with x @ PiT and cast to the query dtype, and a dense
# causal attention with unequal query/key lengths aligns the queries to the
# lower right: query i, at absolute position cached_len + i, sees keys
# 0 .. cached_len + i)
# --------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of float64 x, ties to even, in one rounding.

    bf16 keeps 8 significant bits down to 2**-126 and a fixed step of 2**-133
    below; finite values from 2**128 * (1 - 2**-9) up overflow to infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.frexp(np.where(a > 0, a, 1.0))[1] - 1             # floor(log2 a)
    step = np.ldexp(1.0, np.maximum(e, -126) - 7)
    r = np.rint(a / step) * step                             # rint: ties to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    return np.copysign(np.where(a > 0, r, 0.0), x)


def rotate_to_bf16(x_bits: np.ndarray) -> np.ndarray:
    """bf16 value of x @ H per vector ([UQ-impl] (x.to(float32) @ PiT).to(dtype)).

    The reading taken here: the exact product rounded once to bf16 (the
    pages' float32 product differs from it only where its own rounding error
    moves a value across a bf16 rounding boundary)."""
    return bf16_round(rotate(bf16_to_f64(x_bits)))


def dequant_prefix(kv_cache: np.ndarray, block_row: np.ndarray, n: int):
    """Dequantised (K, V) (n, Hk, 256) of a sequence's first n tokens, K in
    the rotated basis ([UQ-impl] ultraquant_full_dequant_kv into the
    (1, Hk, alloc_len, D) buffers, read back token-major)."""
    hk = kv_cache.shape[2]
    d = head_dim_of_slot(kv_cache.shape[3])
    K = np.zeros((n, hk, d))
    V = np.zeros((n, hk, d))
    for h in range(hk):
        K[:, h], V[:, h] = gather_sequence(kv_cache, block_row, n, h)
    return K, V


def continuation_prefill(query_bits, key_bits, value_bits, kv_cache, block_row, cached_len,
                         scale, rows=None) -> np.ndarray:
    """Output (q_len, Hq, 256) float64 of a continuation chunk.

    query_bits (q_len, Hq, 256), key_bits / value_bits (q_len, Hk, 256) are
    the chunk's bf16 inputs before rotation; the sequence's first cached_len
    tokens are in kv_cache through block_row. Keys are the dequantised
    prefix followed by the chunk's rotated keys (as bf16); values are the
    dequantised prefix followed by the chunk's values. Query head hq reads KV
    head hq // (Hq // Hk). ``rows`` optionally lists the chunk positions to
    compute (the others are left NaN); every key and value is still used.
    """
    query_bits = np.asarray(query_bits)
    q_len, hq_n, d = query_bits.shape
    hk = np.asarray(key_bits).shape[1]
    qg = hq_n // hk
    Kp, Vp = dequant_prefix(kv_cache, block_row, cached_len)
    K = np.concatenate([Kp, rotate_to_bf16(key_bits)], axis=0)
    V = np.concatenate([Vp, bf16_to_f64(value_bits)], axis=0)
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    q = rotate_to_bf16(query_bits[rows])
    seq = cached_len + q_len
    visible = np.arange(seq)[None, :] <= cached_len + rows[:, None]
    out = np.full((q_len, hq_n, d), np.nan)
    for hq in range(hq_n):
        h = hq // qg
        s = scale * (q[:, hq] @ K[:, h].T)
        s = np.where(visible, s, -np.inf)
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        out[rows, hq] = (p @ V[:, h]) / p.sum(axis=-1, keepdims=True)
    return out
