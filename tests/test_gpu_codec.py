"""GPU parity for the codec: zf_encode_kv, zf_append_kv(_n) and zf_decode_kv through the C ABI,
bit-exact against the CPU oracle on every workload (packed planes, base, row flags, row spill
slots, spill bytes, spill_top), plus the device-side error rules.

Codec: ZipFusion video summary ("Run AI Faster With Lossless Compressed Memory", chapter
"Twelve Bits and One Addition"); lossless, so decode must return the encoded bits exactly.
"""
import dataclasses
import numpy as np
import pytest
import torch

import decode_attention_encode_amd as zf
import oracle
import synth
from gpu_util import Setup, check_kmax, compare_packed, dev, host, log, oracle_cache, valid_rows

pytestmark = pytest.mark.gpu

SMALL = synth.WORKLOADS[0].replace(name="ragged_small", batch=5, ctx_min=1, ctx_max=300,
                                   extra_tokens=3, pool_factor=1.3, p_wide_block=0.05, seed=21)


def workload(key):
    return SMALL if key == "small" else synth.WORKLOADS[key]


@pytest.mark.parametrize("key", [0, "small", 1, 2, 3, 4])
def test_encode_bitexact(key):
    w = workload(key)
    log(f"encode parity: workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    assert s.status() == 0
    orc = oracle_cache(inst, s.cache.spill_slots)
    compare_packed(s.cache, orc, valid_rows(inst), w.name)
    check_kmax(s, orc, inst.seq_lens, w.name)
    log(f"  raw blocks {orc.spill_top} of {int(inst.seq_lens.sum()) * 32}")


@pytest.mark.parametrize("key", [0, "small", 1, 2, 3, 4])
def test_decode_roundtrip(key):
    w = workload(key)
    log(f"decode round trip: workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    out = torch.zeros_like(s.raw)
    zf.zf_decode_kv(s.cache, s.seqs, out)
    torch.cuda.synchronize()
    assert s.status() == 0
    got = host(out, np.uint16)
    rows = valid_rows(inst)
    m = np.broadcast_to(rows[:, None, None, :, None], got.shape)
    assert np.array_equal(got[m], inst.raw_pages[m])
    untouched = ~m
    assert not got[untouched].any(), "decode wrote outside the defined rows"


def _append_steps(w, steps, check_every=1, one_launch=True):
    inst = synth.make(w)
    s = Setup(inst, one_launch_append=one_launch)
    orc = oracle_cache(inst, s.cache.spill_slots)
    lens = inst.seq_lens.copy()
    for step in range(steps):
        k, v = synth.tokens(w, lens)
        zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
        assert orc.append(lens, inst.page_table, k, v) == oracle.OK
        if (step + 1) % check_every == 0 or step == steps - 1:
            torch.cuda.synchronize()
            assert s.status() == 0
            assert np.array_equal(host(s.seqs.seq_lens), lens)
            compare_packed(s.cache, orc, valid_rows(inst, lens), f"{w.name} step {step}")
            check_kmax(s, orc, lens, f"{w.name} step {step}")
    return s, inst, lens


@pytest.mark.parametrize("key,steps,form", [("small", 3, "one"), (1, 1, "one"), (3, 1, "one"),
                                            (4, 64, "one"), ("small", 3, "two"), (1, 2, "two")])
def test_append_bitexact(key, steps, form):
    """Single-token appends, in the one-launch form (batch <= 64 new rows, the cache's sync
    words set; batch 64 is its limit) and in the two-launch form."""
    w = workload(key)
    if w.extra_tokens < steps:
        w = w.replace(extra_tokens=steps)
    log(f"append parity: workload {w.name}, {steps} steps, {form}-launch form")
    s, _, _ = _append_steps(w, steps, check_every=16, one_launch=form == "one")
    if form == "one":
        assert int(host(s.cache.append_sync)[64]) == steps, "one epoch per one-launch call"


def test_append_forms_write_the_same_bytes():
    """The same appends through both forms leave every array equal, spill pool included."""
    w = SMALL.replace(extra_tokens=6, p_wide_block=0.2)
    log(f"append forms: workload {w.name}")
    inst = synth.make(w)
    one, two = Setup(inst), Setup(inst, one_launch_append=False)
    lens = inst.seq_lens.copy()
    for step in range(6):
        k, v = synth.tokens(w, lens)
        if step == 2:
            k[:, :, 0] = 0  # a raw block in every new row
        zf.zf_append_kv(one.cache, one.seqs, dev(k), dev(v))
        zf.zf_append_kv(two.cache, two.seqs, dev(k), dev(v))
        lens += 1
    torch.cuda.synchronize()
    assert one.status() == 0 and two.status() == 0
    for n in ("sm", "nib", "base", "row_flags", "row_spill", "spill", "spill_top"):
        assert np.array_equal(host(getattr(one.cache, n)), host(getattr(two.cache, n))), n
    assert np.array_equal(host(one.seqs.kmax), host(two.seqs.kmax)), "page hints"
    assert np.array_equal(host(one.seqs.seq_lens), lens)
    assert int(host(one.cache.append_sync)[64]) == 6


def test_one_launch_append_with_changing_batch():
    """One cache appended 24 times while the number of new rows changes between calls (a prefix
    of the batch, 1 or 2 tokens per sequence: 1 to 64 rows in one launch, more in two), so the
    hand-over words of rows a call does not use, and words left by earlier calls, are exercised;
    bit-exact against the oracle after every call, one epoch per one-launch call."""
    w = SMALL.replace(name="ragged_b64_short", batch=64, ctx_min=1, ctx_max=40, extra_tokens=48,
                      seed=61)
    log(f"one-launch append, changing batch: workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    orc = oracle_cache(inst, s.cache.spill_slots)
    lens = inst.seq_lens.copy()
    rng = np.random.default_rng(7)
    ones = 0
    for call in range(24):
        k_seq = int(rng.choice([1, 2, 17, 33, 63, 64]))
        n = int(rng.choice([1, 1, 2]))
        kk, vv = _chunk_tokens(w, lens, n)
        kk, vv = np.ascontiguousarray(kk[:k_seq]), np.ascontiguousarray(vv[:k_seq])
        sub = zf.Seqs(dev(np.ascontiguousarray(inst.page_table[:k_seq])), s.seqs.seq_lens[:k_seq],
                      s.seqs.max_seq_len)
        if n == 1:
            zf.zf_append_kv(s.cache, sub, dev(kk[:, 0].copy()), dev(vv[:, 0].copy()))
            assert orc.append(lens[:k_seq], inst.page_table[:k_seq], kk[:, 0].copy(), vv[:, 0].copy()) == oracle.OK
        else:
            zf.zf_append_kv_n(s.cache, sub, dev(kk), dev(vv))
            assert orc.append_n(lens[:k_seq], inst.page_table[:k_seq], kk, vv) == oracle.OK
        ones += k_seq * n <= 64
        torch.cuda.synchronize()
        assert s.status() == 0, f"call {call}"
        assert np.array_equal(host(s.seqs.seq_lens), lens), f"call {call}"
        compare_packed(s.cache, orc, valid_rows(inst, lens), f"call {call} ({k_seq} x {n})")
    assert int(host(s.cache.append_sync)[64]) == ones


def test_one_launch_append_give_up_reports_and_changes_nothing():
    """The cache's give-up hook makes every packing workgroup that has rows before it give up
    instead of waiting for their words: it marks its word abandoned, the commit sees the mark,
    and the call ends with ZF_DEV_ESYNC, no defined state changed and the epoch advanced.  With
    the hook cleared the same append succeeds (no clean-up of the sync words) and matches the
    oracle."""
    w = SMALL
    inst = synth.make(w)
    assert w.batch >= 2  # a workgroup with a row before it
    s = Setup(inst)
    orc = oracle_cache(inst, s.cache.spill_slots)
    rows = valid_rows(inst)
    names = ("sm", "nib", "base", "row_flags", "row_spill")
    before = {n: host(getattr(s.cache, n)).copy() for n in names}
    top = int(host(s.cache.spill_top)[0])
    epoch = int(host(s.cache.append_sync)[zf.ZF_SYNC_EPOCH])
    k, v = synth.tokens(w, inst.seq_lens)
    s.cache.append_sync[zf.ZF_SYNC_GIVE_UP] = 1
    zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
    torch.cuda.synchronize()
    s.cache.append_sync[zf.ZF_SYNC_GIVE_UP] = 0
    assert s.status() & zf.ZF_DEV_ESYNC
    assert int(host(s.cache.append_sync)[zf.ZF_SYNC_EPOCH]) == epoch + 1
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == top
    for n in names:
        a, b = host(getattr(s.cache, n)), before[n]
        m = np.broadcast_to(rows[:, None, None, :, None], a.shape) if a.ndim == 5 else rows
        assert np.array_equal(a[m], b[m]), n
    s.cache.status.zero_()
    lens = inst.seq_lens.copy()
    zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
    assert orc.append(lens, inst.page_table, k, v) == oracle.OK
    torch.cuda.synchronize()
    assert s.status() == 0
    assert int(host(s.cache.append_sync)[zf.ZF_SYNC_EPOCH]) == epoch + 2
    compare_packed(s.cache, orc, valid_rows(inst, lens), "append after a given-up one")


def test_one_launch_append_bad_page_changes_nothing():
    """A new row whose page-table entry is out of range: ZF_DEV_EPAGE, lengths and spill_top
    kept, the epoch still advanced, and a later append on a good table matches the oracle."""
    w = SMALL
    inst = synth.make(w)
    s = Setup(inst)
    orc = oracle_cache(inst, s.cache.spill_slots)
    T = w.page_size
    b = int(np.argmax(inst.seq_lens))
    pt_bad = inst.page_table.copy()
    pt_bad[b, int(inst.seq_lens[b]) // T] = inst.num_pages + 3
    bad = zf.Seqs(dev(pt_bad), s.seqs.seq_lens, s.seqs.max_seq_len)
    top = int(host(s.cache.spill_top)[0])
    k, v = synth.tokens(w, inst.seq_lens)
    zf.zf_append_kv(s.cache, bad, dev(k), dev(v))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_EPAGE
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == top
    assert int(host(s.cache.append_sync)[64]) == 1
    s.cache.status.zero_()
    lens = inst.seq_lens.copy()
    zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
    assert orc.append(lens, inst.page_table, k, v) == oracle.OK
    torch.cuda.synchronize()
    assert s.status() == 0
    compare_packed(s.cache, orc, valid_rows(inst, lens), "append after a bad-page one")


def test_append_spill_exhaustion_changes_no_defined_state():
    w = SMALL
    inst = synth.make(w)
    orc = oracle_cache(inst, 1 << 20)
    need = orc.spill_top
    s = Setup(inst, spill_slots=need)  # exactly full after the encode
    assert s.status() == 0 and int(host(s.cache.spill_top)[0]) == need
    rows = valid_rows(inst)
    names = ("sm", "nib", "base", "row_flags", "row_spill")
    before = {n: host(getattr(s.cache, n)).copy() for n in names}
    spill_before = host(s.cache.spill).copy()
    k, v = synth.tokens(w, inst.seq_lens)
    k[:, :, 0] = 0  # every new row gets a raw block
    zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_ESPILL
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == need
    assert np.array_equal(host(s.cache.spill), spill_before)
    for n in names:
        a, b = host(getattr(s.cache, n)), before[n]
        m = np.broadcast_to(rows[:, None, None, :, None], a.shape) if a.ndim == 5 else rows
        assert np.array_equal(a[m], b[m]), n
    # the same call with room for the new rows then succeeds and matches the oracle
    s2 = Setup(inst)
    orc2 = oracle_cache(inst, s2.cache.spill_slots)
    lens = inst.seq_lens.copy()
    zf.zf_append_kv(s2.cache, s2.seqs, dev(k), dev(v))
    assert orc2.append(lens, inst.page_table, k, v) == oracle.OK
    torch.cuda.synchronize()
    assert s2.status() == 0
    compare_packed(s2.cache, orc2, valid_rows(inst, lens), "append after a failed one")


@pytest.mark.parametrize("form", ["one", "two"])
def test_append_partly_fitting_pool_changes_no_defined_state(form):
    """Room for a few of the new raw blocks but not all: ZF_DEV_ESPILL, lengths, spill_top and
    every defined row and slot kept; rows whose slots fitted may have written them (slots from
    spill_top on hold nothing yet), never past the pool's end (guard slots behind a smaller
    spill_slots stay zero)."""
    w = SMALL
    inst = synth.make(w)
    orc = oracle_cache(inst, 1 << 20)
    need, room, guard = orc.spill_top, 3, 64
    s = Setup(inst, spill_slots=need + room + guard, one_launch_append=(form == "one"))
    c = dataclasses.replace(s.cache, spill_slots=need + room)
    assert s.status() == 0 and int(host(s.cache.spill_top)[0]) == need
    rows = valid_rows(inst)
    names = ("sm", "nib", "base", "row_flags", "row_spill")
    before = {n: host(getattr(s.cache, n)).copy() for n in names}
    spill_before = host(s.cache.spill)[:need].copy()
    k, v = synth.tokens(w, inst.seq_lens)
    k[:, :, 0] = 0  # every new row gets a raw block: batch > room
    assert w.batch > room
    zf.zf_append_kv(c, s.seqs, dev(k), dev(v))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_ESPILL
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == need
    assert np.array_equal(host(s.cache.spill)[:need], spill_before)
    assert not host(s.cache.spill)[need + room:].any()
    for n in names:
        a, b = host(getattr(s.cache, n)), before[n]
        m = np.broadcast_to(rows[:, None, None, :, None], a.shape) if a.ndim == 5 else rows
        assert np.array_equal(a[m], b[m]), n


@pytest.mark.parametrize("form", ["one", "two"])
def test_top_beyond_the_pool_counts_as_full(form):
    """spill_top past spill_slots (the buffers stay large, so nothing can land out of bounds):
    an append reports ZF_DEV_ESPILL and changes nothing even with no raw block to spill, and so
    does an encode; the oracle follows the same rule."""
    w = SMALL
    inst = synth.make(w)
    s = Setup(inst, one_launch_append=form == "one")
    top = int(host(s.cache.spill_top)[0])
    s.cache.spill_slots = top - 1
    k, v = synth.tokens(w, inst.seq_lens)
    k[:] = 0x3F80  # 1.0: no raw block
    v[:] = 0x3F80
    spill_before = host(s.cache.spill).copy()
    zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_ESPILL
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == top
    assert np.array_equal(host(s.cache.spill), spill_before)
    e = Setup(inst, encode=False)
    e.cache.spill_slots = 8
    e.cache.spill_top.fill_(9)
    zf.zf_encode_kv(e.cache, e.seqs, e.raw, zf.encode_workspace(e.seqs))
    torch.cuda.synchronize()
    assert e.status() & zf.ZF_DEV_ESPILL
    assert int(host(e.cache.spill_top)[0]) == 9 and not host(e.cache.spill).any()


def _chunk_tokens(w, lens, n):
    """n new tokens per sequence at positions lens[b] .. lens[b] + n - 1: two u16[B][n][H][D]."""
    ks, vs = zip(*(synth.tokens(w, lens + j) for j in range(n)))
    return np.ascontiguousarray(np.stack(ks, 1)), np.ascontiguousarray(np.stack(vs, 1))


@pytest.mark.parametrize("key,chunks", [("small", (5, 1, 3, 16)), (1, (16,)), (3, (64,)), (4, (17, 64, 1))])
def test_append_n_bitexact(key, chunks):
    """Multi-token appends (ragged lengths, chunks crossing pages, 4096 rows at the limit for
    64 sequences x 64 tokens) equal the oracle bit for bit after every call."""
    w = workload(key)
    w = w.replace(extra_tokens=max(w.extra_tokens, sum(chunks)))
    log(f"multi-token append parity: workload {w.name}, chunks {chunks}")
    inst = synth.make(w)
    s = Setup(inst)
    orc = oracle_cache(inst, s.cache.spill_slots)
    lens = inst.seq_lens.copy()
    for i, n in enumerate(chunks):
        k, v = _chunk_tokens(w, lens, n)
        zf.zf_append_kv_n(s.cache, s.seqs, dev(k), dev(v))
        assert orc.append_n(lens, inst.page_table, k, v) == oracle.OK
        torch.cuda.synchronize()
        assert s.status() == 0
        assert np.array_equal(host(s.seqs.seq_lens), lens)
        compare_packed(s.cache, orc, valid_rows(inst, lens), f"{w.name} chunk {i} (n={n})")
        check_kmax(s, orc, lens, f"{w.name} chunk {i} (n={n})")


def test_append_n_spill_exhaustion_changes_no_defined_state():
    inst = synth.make(SMALL.replace(extra_tokens=8))
    orc = oracle_cache(inst, 1 << 20)
    need = orc.spill_top
    s = Setup(inst, spill_slots=need + 3)  # room for a few raw blocks only
    rows = valid_rows(inst)
    names = ("sm", "nib", "base", "row_flags", "row_spill")
    before = {n: host(getattr(s.cache, n)).copy() for n in names}
    spill_before = host(s.cache.spill).copy()
    k, v = _chunk_tokens(inst.w, inst.seq_lens, 8)
    k[:, :, :, 0] = 0  # every new row gets a raw block
    zf.zf_append_kv_n(s.cache, s.seqs, dev(k), dev(v))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_ESPILL
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == need
    # the defined slots are kept (those from spill_top on hold nothing yet)
    assert np.array_equal(host(s.cache.spill)[:need], spill_before[:need])
    for n in names:
        a, b = host(getattr(s.cache, n)), before[n]
        m = np.broadcast_to(rows[:, None, None, :, None], a.shape) if a.ndim == 5 else rows
        assert np.array_equal(a[m], b[m]), n


# More new rows than one commit workgroup holds (the grouped form): a batch of 32 ragged
# sequences takes 2048 tokens each in one call (65 536 rows), then 600 more (19 200 rows).
LONG_APPEND = synth.WORKLOADS[1].replace(name="chunked_append_b32", ctx_min=100, ctx_max=700,
                                         extra_tokens=2650, seed=31)


# and a batch of 7 taking 997 tokens, then 1021: 6979 and 7147 rows, neither a multiple of the
# 16-row groups nor of the pack kernel's 4 rows, groups straddling sequences
ODD_APPEND = LONG_APPEND.replace(name="chunked_append_b7_odd", batch=7, extra_tokens=2100, seed=33)


@pytest.mark.parametrize("w,ns", [(LONG_APPEND, (2048, 600)), (ODD_APPEND, (997, 1021))],
                         ids=["b32", "b7_odd"])
def test_append_n_chunked_bitexact(w, ns):
    log(f"chunked append parity: workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    orc = oracle_cache(inst, s.cache.spill_slots)
    lens = inst.seq_lens.copy()
    for n in ns:
        assert w.batch * n > 4096
        k, v = _chunk_tokens(w, lens, n)
        zf.zf_append_kv_n(s.cache, s.seqs, dev(k), dev(v))
        assert orc.append_n(lens, inst.page_table, k, v) == oracle.OK
        torch.cuda.synchronize()
        assert s.status() == 0
        assert np.array_equal(host(s.seqs.seq_lens), lens)
        compare_packed(s.cache, orc, valid_rows(inst, lens), f"{w.name} ({w.batch} x {n} rows)")
        check_kmax(s, orc, lens, f"{w.name} ({w.batch} x {n} rows)")
        log(f"  {w.batch * n} rows: bit-exact, spill_top {orc.spill_top}")


@pytest.mark.parametrize("fault", ["spill", "length", "page"])
def test_append_n_chunked_errors_change_no_defined_state(fault):
    """The grouped form fails whole: a pool with room for a few raw blocks only (ZF_DEV_ESPILL),
    one sequence whose new rows pass its page table's end (ZF_DEV_ELEN), or one new row on an
    out-of-range page id (ZF_DEV_EPAGE).  Lengths, spill_top, every defined row and slot, and
    the memory past the pool's end stay as they were."""
    w = LONG_APPEND.replace(batch=8, extra_tokens=700, seed=32)
    n = 600  # 4800 rows
    inst = synth.make(w)
    orc = oracle_cache(inst, 1 << 24)
    need, guard = orc.spill_top, 64
    room = 3 if fault == "spill" else 8 * n * 32
    s = Setup(inst, spill_slots=need + room + guard)
    c = dataclasses.replace(s.cache, spill_slots=need + room)
    rows = valid_rows(inst)
    names = ("sm", "nib", "base", "row_flags", "row_spill")
    before = {m: host(getattr(s.cache, m)).copy() for m in names}
    spill_before = host(s.cache.spill)[:need].copy()
    k, v = _chunk_tokens(w, inst.seq_lens, n)
    seqs = s.seqs
    if fault == "spill":
        k[:, :, :, 0] = 0  # every new row gets a raw block
    elif fault == "length":
        seqs = zf.Seqs(s.seqs.page_table, s.seqs.seq_lens, int(inst.seq_lens.max()) + n - 1)
    else:
        pt = inst.page_table.copy()
        b = 5
        pt[b, (int(inst.seq_lens[b]) + n - 1) // w.page_size] = inst.num_pages + 7
        seqs = zf.Seqs(dev(pt), s.seqs.seq_lens, s.seqs.max_seq_len)
    zf.zf_append_kv_n(c, seqs, dev(k), dev(v))
    torch.cuda.synchronize()
    want = {"spill": zf.ZF_DEV_ESPILL, "length": zf.ZF_DEV_ELEN, "page": zf.ZF_DEV_EPAGE}[fault]
    assert s.status() & want
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == need
    assert np.array_equal(host(s.cache.spill)[:need], spill_before)
    assert not host(s.cache.spill)[need + room:].any()
    for m in names:
        a, b_ = host(getattr(s.cache, m)), before[m]
        msk = np.broadcast_to(rows[:, None, None, :, None], a.shape) if a.ndim == 5 else rows
        assert np.array_equal(a[msk], b_[msk]), m


def test_append_n_grouped_give_up_reports_and_changes_nothing():
    """The cache's give-up hook makes every group of the grouped form (more than 4096 new rows)
    that has groups before it skip its look-back as if the wait had run out: its word stays at
    its aggregate, the last step sees it and the call ends with ZF_DEV_ESYNC, lengths, spill_top
    and every defined row and slot unchanged.  With the hook cleared the same call succeeds and
    matches the oracle bit for bit."""
    w = LONG_APPEND.replace(name="grouped_give_up_b8", batch=8, extra_tokens=700, seed=34)
    n = 600  # 4800 rows
    inst = synth.make(w)
    s = Setup(inst)
    orc = oracle_cache(inst, s.cache.spill_slots)
    need = orc.spill_top
    rows = valid_rows(inst)
    names = ("sm", "nib", "base", "row_flags", "row_spill")
    before = {m: host(getattr(s.cache, m)).copy() for m in names}
    spill_before = host(s.cache.spill)[:need].copy()
    k, v = _chunk_tokens(w, inst.seq_lens, n)
    s.cache.append_sync[zf.ZF_SYNC_GIVE_UP] = 1
    zf.zf_append_kv_n(s.cache, s.seqs, dev(k), dev(v))
    torch.cuda.synchronize()
    s.cache.append_sync[zf.ZF_SYNC_GIVE_UP] = 0
    assert s.status() & zf.ZF_DEV_ESYNC
    assert np.array_equal(host(s.seqs.seq_lens), inst.seq_lens)
    assert int(host(s.cache.spill_top)[0]) == need
    assert np.array_equal(host(s.cache.spill)[:need], spill_before)
    for m in names:
        a, b_ = host(getattr(s.cache, m)), before[m]
        msk = np.broadcast_to(rows[:, None, None, :, None], a.shape) if a.ndim == 5 else rows
        assert np.array_equal(a[msk], b_[msk]), m
    s.cache.status.zero_()
    lens = inst.seq_lens.copy()
    zf.zf_append_kv_n(s.cache, s.seqs, dev(k), dev(v))
    assert orc.append_n(lens, inst.page_table, k, v) == oracle.OK
    torch.cuda.synchronize()
    assert s.status() == 0
    assert np.array_equal(host(s.seqs.seq_lens), lens)
    compare_packed(s.cache, orc, valid_rows(inst, lens), "grouped append after a given-up one")


# other geometries of the format: head_dim 64 (16 blocks per row), head_dim 256 with 4 kv heads
# (32 blocks per row, every flag bit), 2 kv heads
GEOMS = [SMALL.replace(name="small_d64", head_dim=64, seed=51),
         SMALL.replace(name="small_d256_h4", head_dim=256, num_kv_heads=4, num_q_heads=16, seed=52),
         SMALL.replace(name="small_h2", num_kv_heads=2, num_q_heads=16, seed=53)]


@pytest.mark.parametrize("w", GEOMS, ids=lambda w: w.name)
def test_other_geometries_encode_append_decode(w):
    log(f"codec parity: workload {w.name} (H {w.num_kv_heads}, D {w.head_dim})")
    s, inst, lens = _append_steps(w, 3)
    out = torch.zeros_like(s.raw)
    zf.zf_decode_kv(s.cache, s.seqs, out)
    torch.cuda.synchronize()
    assert s.status() == 0
    orc = oracle_cache(inst, s.cache.spill_slots)
    st, want = orc.decode(inst.seq_lens, inst.page_table)
    assert st == oracle.OK
    rows = valid_rows(inst)
    got = host(out, np.uint16)
    m = np.broadcast_to(rows[:, None, None, :, None], got.shape)
    assert np.array_equal(got[m], want[m])


def test_encode_spill_exhaustion_keeps_pool():
    """One slot short: ZF_DEV_ESPILL and spill_top kept.  The slots inside the pool may hold
    the pass's nibbles (they are unspecified after a failed encode); memory past the pool's
    end (guard slots behind a smaller spill_slots) stays untouched."""
    inst = synth.make(SMALL)
    orc = oracle_cache(inst, 1 << 20)
    n, guard = orc.spill_top - 1, 64
    s = Setup(inst, spill_slots=n + guard, encode=False)
    short = dataclasses.replace(s.cache, spill_slots=n)
    zf.zf_encode_kv(short, s.seqs, s.raw, zf.encode_workspace(s.seqs))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_ESPILL
    assert int(host(s.cache.spill_top)[0]) == 0
    assert not host(s.cache.spill)[n:].any()
    # exactly enough slots: succeeds and fills the pool
    s2 = Setup(inst, spill_slots=orc.spill_top)
    assert s2.status() == 0
    compare_packed(s2.cache, orc, valid_rows(inst), "exact pool")


def test_bad_page_and_length_set_status():
    inst = synth.make(SMALL)
    pt = inst.page_table.copy()
    pt[2, 0] = inst.num_pages + 7
    bad = synth.Instance(inst.w, inst.seq_lens, pt, inst.num_pages, inst.raw_pages)
    s = Setup(bad)
    assert s.status() & zf.ZF_DEV_EPAGE
    lens = inst.seq_lens.copy()
    lens[1] = inst.page_table.shape[1] * 16 + 5
    s = Setup(synth.Instance(inst.w, lens, inst.page_table, inst.num_pages, inst.raw_pages),
              max_seq_len=inst.page_table.shape[1] * 16)
    assert s.status() & zf.ZF_DEV_ELEN


def test_encode_is_repeatable():
    """Same input, same spill_top start: identical packed bytes (no order dependence)."""
    inst = synth.make(synth.WORKLOADS[1].replace(batch=6))
    a, b = Setup(inst), Setup(inst)
    rows = valid_rows(inst)
    for n in ("sm", "nib", "base", "row_flags", "row_spill", "spill", "spill_top"):
        x, y = host(getattr(a.cache, n)), host(getattr(b.cache, n))
        if x.ndim == 5:
            m = np.broadcast_to(rows[:, None, None, :, None], x.shape)
            assert np.array_equal(x[m], y[m]), n
        elif x.ndim == 2 and n.startswith("row_"):
            assert np.array_equal(x[rows], y[rows]), n
        else:
            assert np.array_equal(x, y), n
