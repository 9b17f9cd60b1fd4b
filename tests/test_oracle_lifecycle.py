"""Pins for the oracle's spill lifecycle (compaction for the live sequences) and its capacity
model.

Pages come and go with their sequences in a paged cache (page "Open Weights: from files to
tokens / second", section "09 / The optimization stack"); the spill pool of the raw blocks only
grows under encode and append, so the sequences still live get their raw blocks moved to the
front of the pool, laid out exactly as an encode of just those sequences into an empty pool
would lay them out.  Capacity: the device memory left after the weights and a reserve holds
the paged cache, and the sequences that fit are that budget over one sequence's cache (same
page, deployment step "Spend the memory dividend" and section "05 / Memory is the admission
ticket"); the gain the ZipFusion summary reports is mostly this capacity.

The pins compare against an encode of the live sequences into an empty pool (pinned on its own
against an independent bit-string packer), against raw-block counts taken from the codec's
definition on the raw values, and against hand-computed capacity figures.
"""
import numpy as np

import oracle
import synth


def _inst(seed, **kw):
    w = synth.WORKLOADS[0].replace(batch=5, ctx_min=30, ctx_max=90, seed=seed, extra_tokens=0)
    return synth.make(w.replace(**kw))


def _rows_mask(inst, live, lens=None):
    lens = inst.seq_lens if lens is None else lens
    T = inst.w.page_size
    m = np.zeros((inst.num_pages, T), bool)
    for b in live:
        for t in range(int(lens[b])):
            m[inst.page_table[b, t // T], t % T] = True
    return m


def _tokens(inst, b, t0, n):
    T = inst.w.page_size
    pages = [inst.page_table[b, t // T] for t in range(t0, t0 + n)]
    k = np.stack([inst.raw_pages[p, :, 0, t % T] for p, t in zip(pages, range(t0, t0 + n))])
    v = np.stack([inst.raw_pages[p, :, 1, t % T] for p, t in zip(pages, range(t0, t0 + n))])
    return k, v


def _grown_cache(inst, slots=1 << 20):
    """The first 20 tokens of every sequence encoded, the rest appended: one token per
    sequence per step while the shortest has tokens left, then 1-token appends of the longer
    ones alone, so the pool interleaves the sequences' slots."""
    w = inst.w
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=slots)
    lens = np.minimum(inst.seq_lens, 20).astype(np.int32)
    assert c.encode(lens, inst.page_table, inst.raw_pages) == oracle.OK
    while (lens < inst.seq_lens).any():
        todo = [b for b in range(w.batch) if lens[b] < inst.seq_lens[b]]
        sub_lens = lens[todo].copy()
        ks, vs = zip(*(_tokens(inst, b, int(lens[b]), 1) for b in todo))
        k = np.ascontiguousarray(np.stack(ks)[:, 0])
        v = np.ascontiguousarray(np.stack(vs)[:, 0])
        assert c.append(sub_lens, inst.page_table[todo], k, v) == oracle.OK
        lens[todo] = sub_lens
    assert np.array_equal(lens, inst.seq_lens)
    return c


def _fresh_encode(inst, live):
    w = inst.w
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=1 << 20)
    assert c.encode(inst.seq_lens[live], inst.page_table[live], inst.raw_pages) == oracle.OK
    return c


def _snapshot(c):
    return {n: getattr(c, n).copy() for n in ("sm", "nib", "base", "row_flags", "row_spill", "spill")}


def test_compaction_after_appends_and_frees_equals_a_fresh_encode():
    inst = _inst(31)
    c = _grown_cache(inst)
    before = _snapshot(c)
    top_before = c.spill_top
    live = [0, 2, 4]  # sequences 1 and 3 end; their pages and slots are given up
    assert c.compact(inst.seq_lens[live], inst.page_table[live]) == oracle.OK
    ref = _fresh_encode(inst, live)
    rows = _rows_mask(inst, live)
    assert c.spill_top == ref.spill_top < top_before
    assert np.array_equal(c.row_spill[rows], ref.row_spill[rows])
    assert np.array_equal(c.row_flags[rows], ref.row_flags[rows])
    assert np.array_equal(c.spill[:c.spill_top], ref.spill[:ref.spill_top])
    # planes and flags are untouched everywhere; row_spill only on live rows
    for n in ("sm", "nib", "base", "row_flags"):
        assert np.array_equal(getattr(c, n), before[n]), n
    assert np.array_equal(c.row_spill[~rows], before["row_spill"][~rows])
    # and the live sequences still decode to their values
    st, dec = c.decode(inst.seq_lens[live], inst.page_table[live])
    assert st == oracle.OK
    m = np.broadcast_to(rows[:, None, None, :, None], dec.shape)
    assert np.array_equal(dec[m], inst.raw_pages[m])


def test_compacted_count_is_the_raw_blocks_of_the_live_rows():
    """spill_top after compaction = raw blocks of the live rows, counted from the codec's
    rule on the raw values (an exponent field 0 or 255, or a window wider than 16)."""
    inst = _inst(32, p_wide_block=0.2)
    c = _grown_cache(inst)
    live = [1, 3]
    assert c.compact(inst.seq_lens[live], inst.page_table[live]) == oracle.OK
    rows = _rows_mask(inst, live)
    blocks = inst.raw_pages.transpose(0, 3, 1, 2, 4)[rows].reshape(-1, 64)
    e = (blocks.astype(np.int64) >> 7) & 0xFF
    raw = (e == 0).any(1) | (e == 255).any(1) | (e.max(1) - e.min(1) > 15)
    assert c.spill_top == int(raw.sum()) > 0


def test_compaction_of_a_fresh_encode_changes_nothing():
    inst = _inst(33)
    c = _fresh_encode(inst, list(range(inst.w.batch)))
    before, top = _snapshot(c), c.spill_top
    assert c.compact(inst.seq_lens, inst.page_table) == oracle.OK
    assert c.spill_top == top
    for n, a in before.items():
        assert np.array_equal(getattr(c, n), a), n


def test_appends_after_compaction_continue_from_the_new_top():
    inst = _inst(34, ctx_min=40, ctx_max=40, extra_tokens=3)
    c = _grown_cache(inst.__class__(inst.w, inst.seq_lens - 3, inst.page_table, inst.num_pages,
                                    inst.raw_pages))
    live = [0, 1, 4]
    lens = (inst.seq_lens - 3)[live].astype(np.int32)
    assert c.compact(lens, inst.page_table[live]) == oracle.OK
    top = c.spill_top
    T = inst.w.page_size
    for _ in range(3):
        ks, vs = zip(*(_tokens(inst, b, int(l), 1) for b, l in zip(live, lens)))
        pos = lens.copy()
        assert c.append(lens, inst.page_table[live], np.stack(ks)[:, 0], np.stack(vs)[:, 0]) == oracle.OK
        for i, b in enumerate(live):
            p, s = inst.page_table[b, pos[i] // T], pos[i] % T
            assert c.row_spill[p, s] == top
            top += bin(int(c.row_flags[p, s])).count("1")
    assert c.spill_top == top
    st, dec = c.decode(lens, inst.page_table[live])
    assert st == oracle.OK
    rows = _rows_mask(inst, live)
    m = np.broadcast_to(rows[:, None, None, :, None], dec.shape)
    assert np.array_equal(dec[m], inst.raw_pages[m])


def test_compaction_errors_change_nothing():
    inst = _inst(35)
    c = _grown_cache(inst)
    # a live row whose raw blocks would lie past spill_top
    T = inst.w.page_size
    rows = [(b, t) for b in range(inst.w.batch) for t in range(int(inst.seq_lens[b]))
            if c.row_flags[inst.page_table[b, t // T], t % T]]
    b, t = rows[len(rows) // 2]
    p, s = inst.page_table[b, t // T], t % T
    n = bin(int(c.row_flags[p, s])).count("1")
    # its last slot is the pool's last live one: accepted (the bytes it names are live)
    probe = _grown_cache(inst)
    probe.row_spill[p, s] = probe.spill_top - n
    assert probe.compact(inst.seq_lens, inst.page_table) == oracle.OK
    # one slot further: rejected
    c.row_spill[p, s] = c.spill_top - n + 1
    before, top = _snapshot(c), c.spill_top
    assert c.compact(inst.seq_lens, inst.page_table) == oracle.ESPILL
    assert c.spill_top == top
    for n, a in before.items():
        assert np.array_equal(getattr(c, n), a), n
    # a page id outside the pool
    pt = inst.page_table.copy()
    pt[0, 0] = inst.num_pages
    assert c.compact(inst.seq_lens, pt) == oracle.EPAGE
    assert c.spill_top == top
    for n, a in before.items():
        assert np.array_equal(getattr(c, n), a), n


def test_compaction_with_no_live_sequence_empties_the_pool():
    inst = _inst(36)
    c = _grown_cache(inst)
    before = _snapshot(c)
    assert c.compact(np.zeros(0, np.int32), np.zeros((0, inst.page_table.shape[1]), np.int32)) == oracle.OK
    assert c.spill_top == 0
    for n, a in before.items():
        assert np.array_equal(getattr(c, n), a), n


# ---------------------------------------------------------------- capacity model

GiB = 1 << 30
LLAMA = dict(layers=32, page_size=16, num_kv_heads=8, head_dim=128)  # Llama-3.1-8B-shaped KV


def _seqs(budget, context, raw_per_row):
    return oracle.max_sequences(budget, LLAMA["layers"], context, LLAMA["page_size"],
                                LLAMA["num_kv_heads"], LLAMA["head_dim"], raw_per_row)


def test_capacity_hand_computed():
    # bf16: 8 kv heads x (K, V) x 128 values x 2 bytes = 4 KiB per token and layer; 4096
    # tokens x 32 layers = 512 MiB per sequence; 80 GiB hold 160
    assert _seqs(80 * GiB, 4096, None) == 160
    # packed, no raw block: 16 vectors x (128 sm + 64 offset + 2 base bytes) + 8 = 3112 bytes
    # per row; 80 GiB / (4096 x 3112 x 32) = 210.6
    assert _seqs(80 * GiB, 4096, 0.0) == 210
    # 8 raw blocks per row add 8 x 32 spill bytes: 3368 bytes per row, 194.6 sequences
    assert _seqs(80 * GiB, 4096, 8.0) == 194
    # a context that is not a whole number of pages takes its last page whole: 4100 tokens
    # use 257 pages (4112 rows)
    assert _seqs(80 * GiB, 4100, None) == 159
    assert _seqs(80 * GiB, 4100, 0.0) == 209


def test_capacity_limits():
    # the planes alone are 12 bits per value: 3/4 of bf16 plus 2 base bytes and 8 row bytes
    # per row; every block raw costs more than bf16 (3112 + 32 x 32 = 4136 > 4096 per row)
    assert _seqs(80 * GiB, 4096, 32.0) < _seqs(80 * GiB, 4096, None)
    assert _seqs(0, 4096, None) == 0 and _seqs(GiB, 0, 0.0) == 0
    # monotone in the raw fraction
    got = [_seqs(288 * GiB, 4096, r) for r in np.linspace(0, 32, 17)]
    assert all(a >= b for a, b in zip(got, got[1:]))
