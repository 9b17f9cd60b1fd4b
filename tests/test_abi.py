"""The C ABI without a GPU: libzf.so loads, exports every function include/zf.h declares, and
its host-side checks (sizes, argument validation, status strings) behave as documented.
No call here enqueues GPU work."""
import ctypes
import os
import re

import pytest

import decode_attention_encode_amd as zf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zf.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zf_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for op in ("zf_encode_kv", "zf_append_kv", "zf_decode_kv", "zf_decode_attention"):
        assert op in names


def test_every_declared_function_is_exported():
    lib = zf.load()
    names = declared_functions()
    assert set(names) == set(zf.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


# what a declaration's comment must name: one of the pages (by title), or that it is an aid
# outside the method, or (the allocation-free variant) the callers it serves
PAGES = ("Open Weights: from files to tokens / second",
         "Run AI Faster With Lossless Compressed Memory")
OTHER = ("outside the method", "callers that cannot allocate")


def governing_comments():
    """Each declared function with the comment block nearest before its declaration (a function
    declared right after another, without a comment of its own, shares that one)."""
    text = open(HEADER).read()
    body = text[text.index("extern \"C\""):]
    found = {}
    for m in re.finditer(r"^(?:[a-z_0-9]+\s+)*[a-z_0-9]+\**\s+\**(zf_[a-z_]+)\s*\(", body, flags=re.M):
        before = body[:m.start()]
        c = before.rfind("/*")
        found[m.group(1)] = re.sub(r"\s*\n\s*\*\s*", " ", before[c:before.index("*/", c)])
    return found


def test_every_declaration_cites_a_page_or_says_why_not():
    found = governing_comments()
    assert set(found) == set(declared_functions())
    for name, comment in found.items():
        assert any(p in comment for p in PAGES + OTHER), (name, comment[:120])
    for op in ("zf_encode_kv", "zf_append_kv", "zf_append_kv_n", "zf_decode_kv",
               "zf_decode_attention", "zf_decode_attention_raw"):
        assert any(p in found[op] for p in PAGES), op


def test_cache_bytes_closed_form():
    P, T, H, D = 10, 16, 8, 128
    vals = P * H * 2 * T * D
    assert zf.zf_cache_bytes(P, T, H, D) == vals + vals // 2 + vals // 64 + 2 * 4 * P * T
    assert zf.zf_cache_bytes(P, T, H, 96) == 0          # not a whole number of blocks
    assert zf.zf_cache_bytes(P, T, 16, 128) == 0        # 64 blocks per row: too many


def test_attention_workspace_sizes():
    assert zf.zf_attention_workspace_bytes(32, 8, 32, 128, 4097) > 0
    assert zf.zf_attention_workspace_bytes(32, 8, 24, 128, 4097) == 0   # group of 3
    assert zf.zf_attention_workspace_bytes(32, 8, 32, 64, 4097) == 0    # head_dim 64
    a = zf.zf_attention_workspace_bytes(32, 8, 32, 128, 4097)
    b = zf.zf_attention_workspace_bytes(32, 8, 32, 128, 8192)
    assert b >= a


def test_encode_workspace_size():
    s = zf.zf_seqs(4, 10, None, None, 160)
    assert zf.load().zf_encode_workspace_bytes(ctypes.byref(s)) == 256 + 4 * 10 * 8  # a look-back word per page


def _cache(**kw):
    fields = dict(num_pages=4, page_size=16, num_kv_heads=8, head_dim=128, sm=256, nib=512,
                  base=768, row_flags=1024, row_spill=1280, spill=1536, spill_slots=10,
                  spill_top=1792, status=2048)
    fields.update(kw)
    return zf.zf_cache(**fields)


@pytest.mark.parametrize("kw,code", [
    (dict(sm=None), zf.ZF_EINVAL),
    (dict(nib=513), zf.ZF_EINVAL),             # misaligned
    (dict(head_dim=100), zf.ZF_EUNSUPPORTED),
    (dict(num_kv_heads=16), zf.ZF_EUNSUPPORTED),
    (dict(status=None), zf.ZF_EINVAL),
    (dict(spill_slots=1 << 32), zf.ZF_EUNSUPPORTED),
    (dict(append_sync=2052), zf.ZF_EINVAL),   # sync words not 8-byte aligned
])
def test_bad_cache_is_rejected_before_any_launch(kw, code):
    lib = zf.load()
    c = _cache(**kw)
    s = zf.zf_seqs(1, 1, 4096, 4096, 16)
    assert lib.zf_decode_kv(ctypes.byref(c), ctypes.byref(s), 2304, None) == code
    assert lib.zf_append_kv(ctypes.byref(c), ctypes.byref(s), 4096, 4096, None) == code
    assert lib.zf_append_kv_n(ctypes.byref(c), ctypes.byref(s), 2, 4096, 4096, None) == code
    assert lib.zf_compact_spill(ctypes.byref(c), ctypes.byref(s), 4096, 1 << 20, None) == code
    assert lib.zf_compact_workspace_bytes(ctypes.byref(c), ctypes.byref(s)) == 0


def test_compact_workspace_and_arguments():
    lib = zf.load()
    c = _cache(spill_slots=100)
    s = zf.zf_seqs(3, 5, 4096, 4096, 80)
    # 256-byte header, page counts rounded to 256 bytes, then 32 bytes per pool slot
    assert lib.zf_compact_workspace_bytes(ctypes.byref(c), ctypes.byref(s)) == 256 + 256 + 3200
    head = 512
    assert lib.zf_compact_spill(ctypes.byref(c), ctypes.byref(s), 4096, head - 1, None) == zf.ZF_EWORKSPACE
    assert lib.zf_compact_spill(ctypes.byref(c), ctypes.byref(s), 4100, 1 << 20, None) == zf.ZF_EWORKSPACE
    assert lib.zf_compact_spill(ctypes.byref(c), ctypes.byref(s), None, 1 << 20, None) == zf.ZF_EWORKSPACE
    big = zf.zf_seqs(8193, 1, 4096, 4096, 16)
    assert lib.zf_compact_spill(ctypes.byref(c), ctypes.byref(big), 4096, 1 << 30, None) == zf.ZF_EUNSUPPORTED


@pytest.mark.parametrize("budget,layers,ctx,raw", [
    (80 << 30, 32, 4096, None), (80 << 30, 32, 4096, 0.0), (80 << 30, 32, 4096, 9.08),
    (288 << 30, 32, 4097, 32.0), (272 << 30, 32, 131072, 7.5), (1 << 20, 1, 1, 1.0),
    (0, 32, 4096, None), (1 << 30, 0, 4096, 1.0), (1 << 30, 32, 0, 1.0),
])
def test_max_sequences_matches_the_oracle(budget, layers, ctx, raw):
    """A host-only function: the library and the oracle's capacity model agree."""
    import oracle
    got = zf.zf_max_sequences(budget, layers, ctx, 16, 8, 128, raw)
    assert got == oracle.max_sequences(budget, layers, ctx, 16, 8, 128, raw)


def test_max_sequences_rejects_bad_geometry():
    assert zf.zf_max_sequences(1 << 30, 32, 4096, 16, 8, 100, 0.0) == -1
    assert zf.zf_max_sequences(1 << 30, 32, 4096, 16, 8, 128, 33.0) == -1  # a row has 32 blocks


def test_append_n_arguments():
    """Rejected (or, for no tokens, finished) on the host before any launch."""
    lib = zf.load()
    c = _cache()
    s = zf.zf_seqs(64, 1, 4096, 4096, 16)
    assert lib.zf_append_kv_n(ctypes.byref(c), ctypes.byref(s), -1, 4096, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_append_kv_n(ctypes.byref(c), ctypes.byref(s), 0, None, None, None) == zf.ZF_OK
    assert lib.zf_append_kv_n(ctypes.byref(c), ctypes.byref(s), (1 << 18) + 1, 4096, 4096, None) == zf.ZF_EUNSUPPORTED
    assert lib.zf_append_kv_n(ctypes.byref(c), ctypes.byref(s), 64, 4096, 4104, None) == zf.ZF_EINVAL
    assert lib.zf_append_kv_n(ctypes.byref(c), ctypes.byref(s), 64, None, 4096, None) == zf.ZF_EINVAL


@pytest.mark.parametrize("seqs,code", [
    (dict(batch=-1), zf.ZF_EINVAL),
    (dict(max_seq_len=17), zf.ZF_EINVAL),       # beyond max_pages_per_seq * page_size
    (dict(page_table=None), zf.ZF_EINVAL),
    (dict(seq_lens=4098), zf.ZF_EINVAL),        # not 4-byte aligned
])
def test_bad_seqs_are_rejected(seqs, code):
    lib = zf.load()
    f = dict(batch=1, max_pages_per_seq=1, page_table=4096, seq_lens=4096, max_seq_len=16)
    f.update(seqs)
    s = zf.zf_seqs(**f)
    c = _cache()
    assert lib.zf_decode_kv(ctypes.byref(c), ctypes.byref(s), 2304, None) == code


def test_attention_shape_and_workspace_checks():
    lib = zf.load()
    c = _cache()
    s = zf.zf_seqs(1, 1, 4096, 4096, 16)
    # group of 3 query heads per kv head: unsupported
    assert lib.zf_decode_attention(ctypes.byref(c), ctypes.byref(s), 4096, 24, 0.1, 8192, 12288,
                                   1 << 20, None) == zf.ZF_EUNSUPPORTED
    # 16 query heads per kv head: unsupported (4 and 8 are)
    assert lib.zf_decode_attention(ctypes.byref(c), ctypes.byref(s), 4096, 128, 0.1, 8192, 12288,
                                   1 << 20, None) == zf.ZF_EUNSUPPORTED
    # too small a workspace
    assert lib.zf_decode_attention(ctypes.byref(c), ctypes.byref(s), 4096, 32, 0.1, 8192, 12288,
                                   16, None) == zf.ZF_EWORKSPACE
    assert lib.zf_decode_attention(ctypes.byref(c), ctypes.byref(s), 4096, 64, 0.1, 8192, 12288,
                                   16, None) == zf.ZF_EWORKSPACE
    # empty batch: nothing to do
    s0 = zf.zf_seqs(0, 0, None, None, 0)
    assert lib.zf_decode_attention(ctypes.byref(c), ctypes.byref(s0), 4096, 32, 0.1, 8192, 12288,
                                   0, None) == zf.ZF_OK


def test_attention_workspace_grows_with_the_query_group():
    """Partials hold acc[G][128], l[G], m[G] doubles per split: 8 query heads per kv head need
    twice the 4-head partial area (the counter header is the same)."""
    B, H, L = 2, 8, 200000  # long enough to split
    w4 = zf.zf_attention_workspace_bytes(B, H, 4 * H, 128, L)
    w8 = zf.zf_attention_workspace_bytes(B, H, 8 * H, 128, L)
    head = 256  # 256-byte header
    assert w4 > head and w8 - head == 2 * (w4 - head)
    assert zf.zf_attention_workspace_bytes(B, H, 16 * H, 128, L) == 0


def test_status_strings():
    lib = zf.load()
    for code in range(5):
        assert lib.zf_status_str(code)
    assert lib.zf_status_str(zf.ZF_EWORKSPACE) == b"workspace missing or too small"


def test_time_next_attention_arguments():
    lib = zf.load()
    assert lib.zf_time_next_attention(None, None) == zf.ZF_OK          # clears
    assert lib.zf_time_next_attention(4096, None) == zf.ZF_EINVAL       # exactly one event
    assert lib.zf_time_next_attention(None, 4096) == zf.ZF_EINVAL


def test_stream_read_probe_arguments():
    lib = zf.load()
    # rejected on the host, nothing launched: null buffer or sink, zero or ragged sizes, misalignment
    assert lib.zf_stream_read_probe(None, 4096, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_stream_read_probe(4096, 4096, None, None) == zf.ZF_EINVAL
    assert lib.zf_stream_read_probe(4096, 0, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_stream_read_probe(4096, 4100, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_stream_read_probe(4104, 4096, 4096, None) == zf.ZF_EINVAL


def test_attention_rejects_spill_pool_beyond_32bit_offsets():
    lib = zf.load()
    s = zf.zf_seqs(1, 1, 4096, 4096, 16)
    ok = _cache(spill_slots=(1 << 27) - 1)
    big = _cache(spill_slots=1 << 27)
    # rejected before any launch; the in-range pool gets past this check to the I/O checks
    assert lib.zf_decode_attention(ctypes.byref(big), ctypes.byref(s), 4096, 32, ctypes.c_float(0.1),
                                   4096, 4096, 1 << 20, None) == zf.ZF_EUNSUPPORTED
    assert lib.zf_decode_attention(ctypes.byref(ok), ctypes.byref(s), 4096, 32, ctypes.c_float(0.1),
                                   4096, 4096, 0, None) == zf.ZF_EWORKSPACE


def test_stream_copy_probe_arguments():
    lib = zf.load()
    assert lib.zf_stream_copy_probe(None, 8192, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_stream_copy_probe(4096, None, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_stream_copy_probe(4096, 8192, 0, None) == zf.ZF_EINVAL
    assert lib.zf_stream_copy_probe(4096, 8192, 4100, None) == zf.ZF_EINVAL
    assert lib.zf_stream_copy_probe(4104, 8192, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_stream_copy_probe(4096, 8200, 4096, None) == zf.ZF_EINVAL
    assert lib.zf_stream_copy_probe(4096, 6144, 4096, None) == zf.ZF_EINVAL  # overlap


def test_header_constants_match_the_binding():
    """The device status bits and the size of the append sync area are the header's."""
    text = open(HEADER).read()
    defs = {k: int(v.rstrip("u")) for k, v in re.findall(r"#define\s+(ZF_\w+)\s+(\d+u?)", text)}
    for name in ("ZF_DEV_ESPILL", "ZF_DEV_EPAGE", "ZF_DEV_ELEN", "ZF_DEV_ESYNC", "ZF_APPEND_SYNC_WORDS",
                 "ZF_PROBE_BLOCKS", "ZF_COPY_PROBE_BLOCKS"):
        assert defs[name] == getattr(zf, name), name

