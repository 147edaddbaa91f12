"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uq_\w+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("uq_build_hadamard", "uq_store", "uq_decode", "uq_decode_ex", "uq_decode_stages",
              "uq_decode_workspace_bytes", "uq_rotate", "uq_dequant_kv", "uq_prefill_attention",
              "uq_continuation_prefill", "uq_continuation_prefill_stages",
              "uq_continuation_prefill_workspace_bytes", "uq_decode_partials", "uq_stream_blocks",
              "uq_decode_no_alloc",
              "uq_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(libuq):
    for name in declared_functions():
        assert hasattr(libuq, name), name


def test_library_has_gfx950_code_object():
    import decode_attention_bit_amd as uq
    blob = open(uq.library_path(), "rb").read()
    assert b"gfx950" in blob


def _err(lib):
    return lib.uq_last_error().decode()


def test_build_hadamard_rejects(libuq):
    assert libuq.uq_build_hadamard(256, None, None) == -1
    assert "null" in _err(libuq)
    buf = ctypes.c_void_p(0x1000)   # never dereferenced: the size check fails first
    assert libuq.uq_build_hadamard(0, buf, None) == -1
    assert libuq.uq_build_hadamard(384, buf, None) == -1
    assert libuq.uq_build_hadamard(1024, buf, None) == -1


FAKE = 0x10000   # 256-byte aligned host address used only for argument checks


def store_args(**kw):
    a = dict(key=FAKE, value=FAKE, kv_cache=FAKE, slot_mapping=FAKE, N=4, Hk=2, D=256,
             num_blocks=8, block_size=16, slot_size=272, ksn=512, ksh=256, vsn=512, vsh=256,
             stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), -2), (dict(D=384), -2), (dict(slot_size=256), -2), (dict(D=128), -2),
    (dict(D=512, slot_size=272), -2), (dict(block_size=8), -2),
    (dict(block_size=48), -2), (dict(block_size=512), -2), (dict(N=-1), -1), (dict(Hk=0), -1),
    (dict(num_blocks=0), -1), (dict(key=None), -1), (dict(slot_mapping=None), -1),
    (dict(ksh=255), -1), (dict(vsn=-4), -1), (dict(key=FAKE + 2), -1),
])
def test_store_rejects(libuq, kw, code):
    assert libuq.uq_store(*store_args(**kw)) == code
    assert _err(libuq)


def test_store_empty_is_noop(libuq):
    assert libuq.uq_store(*store_args(N=0, key=None, value=None, slot_mapping=None)) == 0
    assert _err(libuq) == ""


def decode_args(**kw):
    a = dict(query=FAKE, kv_cache=FAKE, block_table=FAKE, seq_lens=FAKE, scale=0.0625,
             splits=32, out=FAKE, B=4, Hq=32, Hk=4, D=256, num_blocks=64, block_size=16,
             max_blocks=16, qsb=8192, qsh=256, workspace=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), -2), (dict(D=1024), -2), (dict(Hq=36), -2), (dict(Hq=16), -2), (dict(Hq=12, Hk=4), -2),
    (dict(Hq=128, Hk=4), -2), (dict(block_size=8), -2), (dict(splits=0), -2),
    (dict(splits=513), -2), (dict(scale=0.0), -1), (dict(scale=float("nan")), -1),
    (dict(scale=float("inf")), -1), (dict(B=0), -1), (dict(query=None), -1),
    (dict(workspace=None), -1), (dict(out=FAKE + 8), -1), (dict(workspace=FAKE + 16), -1),
    (dict(qsh=130), -1), (dict(ws_bytes=1024), -3), (dict(num_blocks=0), -1),
])
def test_decode_rejects(libuq, kw, code):
    assert libuq.uq_decode(*decode_args(**kw)) == code
    assert _err(libuq)


@pytest.mark.parametrize("mask", [0, 8, -1, 16, 12, 9, 13])
def test_decode_stages_rejects_mask(libuq, mask):
    assert libuq.uq_decode_stages(mask, *decode_args()) == -1


def test_decode_stages_fused_query_only_at_256(libuq):
    assert libuq.uq_decode_stages(2 | 8, *decode_args(D=128)) == -2
    assert "head dim 256" in _err(libuq)


def test_workspace_bytes(libuq):
    f = libuq.uq_decode_workspace_bytes
    assert f(0, 32, 4, 256, 32, 256, 16) == 0
    assert f(32, 30, 4, 256, 32, 256, 16) == 0
    assert f(32, 32, 4, 64, 32, 256, 16) == 0
    assert f(32, 32, 4, 384, 32, 256, 16) == 0
    assert f(32, 32, 4, 256, 0, 256, 16) == 0
    assert f(32, 32, 4, 256, 32, 0, 16) == 0
    assert f(32, 32, 4, 256, 32, 256, 24) == 0
    n = f(32, 32, 4, 256, 32, 256, 16)
    # at least: E4M3 query codes, one fp16 partial row and three 4-byte statistics per partial
    assert n >= 32 * 32 * 256 + 32 * 32 * (256 * 2 + 12)
    assert n % 256 == 0
    assert f(64, 32, 4, 256, 32, 256, 16) >= n
    # one split over a table of one block: one partial
    assert f(2, 16, 2, 256, 1, 1, 16) == 2 * 16 * 256 + 2 * 16 * 512 + 3 * 256


def decode_ex_args(**kw):
    a = dict(query=FAKE, kv_cache=FAKE, block_table=FAKE, rows=4, query_row=FAKE, seq_lens=FAKE,
             scale=0.0625, splits=32, sinks=None, window=0, out=FAKE, B=8, Hq=32, Hk=4, D=256,
             num_blocks=64, block_size=16, max_blocks=16, qsb=8192, qsh=256, workspace=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(rows=0), -1), (dict(query_row=FAKE + 2), -1), (dict(query_row=None), -1),
    (dict(window=-1), -1), (dict(sinks=FAKE + 2), -1),
    (dict(Hq=36), -2), (dict(ws_bytes=1024), -3), (dict(block_table=None), -1),
])
def test_decode_ex_rejects(libuq, kw, code):
    assert libuq.uq_decode_ex(*decode_ex_args(**kw)) == code
    assert _err(libuq)


def _decode_ws(B, Hq, D, parts):
    """Decode workspace bytes for `parts` partials per row: query codes, fp16
    partial rows and three 4-byte statistics, each section 256-byte aligned."""
    a = lambda x: (x + 255) // 256 * 256
    rows = B * Hq
    return a(rows * D) + a(rows * parts * D * 2) + 3 * a(rows * parts * 4)


def test_workspace_covers_paired_rows(libuq):
    """Multi-query rows that may pair plan partials for half the rows, so at
    64 rows x 4 KV heads x 256 tiles the paired plan cuts 8 partials per row
    where the plain decode cuts 4. The workspace size covers the larger one,
    and uq_decode_ex with query_row rejects a workspace that only holds the
    smaller one (checked before any HIP call)."""
    B, Hq, Hk, D, S, mb, bs = 64, 32, 4, 256, 32, 256, 16
    assert libuq.uq_decode_partials(B, Hq, Hk, D, S, mb, bs) == 4
    n = libuq.uq_decode_workspace_bytes(B, Hq, Hk, D, S, mb, bs)
    assert n == _decode_ws(B, Hq, D, 8)
    small = _decode_ws(B, Hq, D, 4)
    args = decode_ex_args(rows=B, B=B, Hq=Hq, Hk=Hk, D=D, splits=S, max_blocks=mb, block_size=bs,
                          num_blocks=B * mb, ws_bytes=small)
    assert libuq.uq_decode_ex(*args) == -3
    assert "workspace" in _err(libuq)
    # at a GQA group of 16 no rows pair: one plan
    assert libuq.uq_decode_workspace_bytes(B, 64, Hk, D, S, mb, bs) == \
        _decode_ws(B, 64, D, libuq.uq_decode_partials(B, 64, Hk, D, S, mb, bs))


# ------------------------------------------------------ continuation prefill
def rotate_args(**kw):
    a = dict(x=FAKE, out=FAKE, N=4, H=2, D=256, xsn=512, xsh=256, osn=512, osh=256, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), -1), (dict(H=0), -1), (dict(D=64), -2), (dict(D=384), -2), (dict(x=None), -1),
    (dict(xsh=6), -1), (dict(osn=-4), -1), (dict(out=FAKE + 4), -1),
])
def test_rotate_rejects(libuq, kw, code):
    assert libuq.uq_rotate(*rotate_args(**kw)) == code
    assert _err(libuq)


def test_rotate_empty_is_noop(libuq):
    assert libuq.uq_rotate(*rotate_args(N=0, x=None, out=None)) == 0


def dequant_args(**kw):
    a = dict(kv_cache=FAKE, block_row=FAKE, n=40, k_out=FAKE, v_out=FAKE, Hk=2, D=256,
             num_blocks=8, block_size=16, ost=512, osh=256, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), -1), (dict(Hk=0), -1), (dict(num_blocks=0), -1), (dict(D=64), -2), (dict(D=1024), -2),
    (dict(block_size=8), -2), (dict(block_row=None), -1), (dict(ost=4), -1),
    (dict(k_out=FAKE + 8), -1), (dict(kv_cache=FAKE + 4), -1),
])
def test_dequant_kv_rejects(libuq, kw, code):
    assert libuq.uq_dequant_kv(*dequant_args(**kw)) == code
    assert _err(libuq)


def prefill_attention_args(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, q_len=8, seq_len=20, Hq=16, Hk=2, D=256,
             scale=0.0625, qst=4096, qsh=256, kvst=512, kvsh=256, ost=4096, osh=256, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q_len=-1), -1), (dict(seq_len=7), -1), (dict(scale=0.0), -1),
    (dict(scale=float("inf")), -1), (dict(D=1024), -2), (dict(D=64), -2), (dict(Hq=15), -2),
    (dict(D=512, Hq=130, Hk=1, kvst=512, kvsh=512), -2),
    (dict(Hq=258, Hk=2), -2), (dict(v=None), -1), (dict(kvst=508), -1), (dict(out=FAKE + 8), -1),
    (dict(kvst=248), -2), (dict(kvst=1 << 25), -2),
])
def test_prefill_attention_rejects(libuq, kw, code):
    assert libuq.uq_prefill_attention(*prefill_attention_args(**kw)) == code
    assert _err(libuq)


def continuation_args(**kw):
    a = dict(query=FAKE, key=FAKE, value=FAKE, kv_cache=FAKE, block_row=FAKE, cached_len=100,
             scale=0.0625, out=FAKE, q_len=8, Hq=16, Hk=2, D=256, num_blocks=64, block_size=16,
             qst=4096, qsh=256, kst=512, ksh=256, vst=512, vsh=256, ost=4096, osh=256,
             workspace=FAKE, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return list(a.values())


@pytest.mark.parametrize("kw,code", [
    (dict(cached_len=-1), -1), (dict(block_row=None), -1), (dict(workspace=FAKE + 16), -1),
    (dict(ws_bytes=4096), -3), (dict(block_size=48), -2), (dict(Hq=17), -2),
    (dict(ost=4), -1), (dict(kst=2), -1), (dict(query=FAKE + 2), -1),
    (dict(D=1024), -2), (dict(D=64), -2), (dict(D=512, Hq=65 * 2), -2),
])
def test_continuation_prefill_rejects(libuq, kw, code):
    assert libuq.uq_continuation_prefill(*continuation_args(**kw)) == code
    assert _err(libuq)


def test_continuation_prefill_workspace_bytes(libuq):
    f = libuq.uq_continuation_prefill_workspace_bytes
    assert f(8, 7, 16, 2, 256) == 0
    assert f(8, 100, 15, 2, 256) == 0
    assert f(8, 100, 16, 2, 1024) == 0
    n = f(8, 100, 16, 2, 256)
    # rotated queries, keys of the whole sequence, values in tiles of 32 keys
    # (2-byte elements), then per KV head 256 parts and one shift for each of
    # the D / 32 value blocks (int32), every section 256-byte aligned
    assert n == 8 * 16 * 512 + 100 * 2 * 512 + 2 * 4 * 32 * 512 + 2 * 256 * 8 * 4 + 2 * 8 * 4
    assert f(8, 101, 16, 2, 256) > n
    # head dim 128: the same sections with 128-element rows and 4 blocks
    assert f(8, 100, 16, 2, 128) == 8 * 16 * 256 + 100 * 2 * 256 + 2 * 4 * 32 * 256 + 2 * 256 * 4 * 4 + 2 * 4 * 4
    # head dim 512: the same sections with 512-element rows and 16 blocks
    assert f(8, 100, 16, 2, 512) == 8 * 16 * 1024 + 100 * 2 * 1024 + 2 * 4 * 32 * 1024 + 2 * 256 * 16 * 4 + 2 * 16 * 4
    assert f(8, 100, 130, 2, 512) == 0        # GQA group 64 at most at D = 512
    assert f(8, 100, 128, 2, 512) > 0 and f(8, 100, 130, 2, 256) > 0


@pytest.mark.parametrize("d", [128, 512])
def test_continuation_prefill_other_head_dims_accepted(libuq, d):
    """D = 128 and 512 pass every host check of both attention calls
    (q_len = 0 then returns before any HIP call)."""
    assert libuq.uq_continuation_prefill(*continuation_args(D=d, q_len=0)) == 0
    assert libuq.uq_prefill_attention(*prefill_attention_args(D=d, q_len=0, kvst=d, kvsh=d)) == 0


@pytest.mark.parametrize("mask", [0, 4, -1, 7])
def test_continuation_prefill_stages_rejects_mask(libuq, mask):
    assert libuq.uq_continuation_prefill_stages(mask, *continuation_args()) == -1
    assert "stage_mask" in _err(libuq)


@pytest.mark.parametrize("d", [128, 512])
def test_other_head_dims_accepted(libuq, d):
    """D = 128 and 512 pass every host check of store and decode; the
    workspace scales with D (query codes D bytes, partial rows D fp16 values)."""
    # store with the matching slot size: all checks pass, then N = 0 returns before any HIP call
    assert libuq.uq_store(*store_args(D=d, slot_size=d * 17 // 16, N=0)) == 0
    f = libuq.uq_decode_workspace_bytes
    n = f(2, 16, 2, d, 1, 1, 16)
    assert n == 2 * 16 * d + 2 * 16 * d * 2 + 3 * 256
    assert f(2, 16, 2, d, 1, 1, 16) < f(2, 16, 2, 2 * d, 1, 1, 16) if d < 512 else True


def test_decode_no_alloc_rejects_on_the_host(libuq):
    """Checked before any HIP call, like every entry point: bad arguments,
    and a shape whose workspace exceeds the static scratch (64 MiB)."""
    args = decode_args()
    del args[-3:-1]                      # no workspace, no workspace bytes
    big = decode_args(B=4096)
    del big[-3:-1]
    assert libuq.uq_decode_no_alloc(*big) == -3
    assert "scratch" in _err(libuq)
    bad = decode_args(D=64)
    del bad[-3:-1]
    assert libuq.uq_decode_no_alloc(*bad) == -2
    nul = decode_args(query=None)
    del nul[-3:-1]
    assert libuq.uq_decode_no_alloc(*nul) == -1
