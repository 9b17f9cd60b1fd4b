"""Pins for the oracle's block codec and cache-level encode / append / decode.

The codec's definition comes from the ZipFusion video summary ("Run AI Faster With Lossless
Compressed Memory", chapter "Twelve Bits and One Addition"): a block keeps one shared base
exponent and a 4-bit exponent offset per value beside each value's sign and mantissa (12 bits
per value, 75 % of BF16); blocks whose exponents are too spread out stay raw; values are
rebuilt with a single integer addition; the scheme is lossless.  Every pin below checks the
oracle against something other than itself: hand-worked fixtures, an exhaustive sweep of
all 65 536 bf16 patterns, an independent bit-string packer, closed forms for sizes and
window boundaries, and invariants (lossless round trip, idempotence, append = encode).
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def _exp(x):
    return (np.asarray(x, np.uint16).astype(np.int64) >> 7) & 0xFF


# ---------------------------------------------------------------- independent packer (tests)

def bitstring_pack(x):
    """Packs a block from the definition using bit strings (shares nothing with the oracle)."""
    bits = [format(int(v), "016b") for v in x]
    sign = [b[0] for b in bits]
    expo = [int(b[1:9], 2) for b in bits]
    mant = [b[9:] for b in bits]
    raw = any(e in (0, 255) for e in expo) or max(expo) - min(expo) > 15
    base = 0 if raw else min(expo)
    sm = bytes(int(s + m, 2) for s, m in zip(sign, mant))
    low4 = [format((e & 15) if raw else (e - base), "04b") for e in expo]
    nib = bytes(int(low4[2 * k + 1] + low4[2 * k], 2) for k in range(32))
    spill = None
    if raw:
        high4 = [format(e >> 4, "04b") for e in expo]
        spill = bytes(int(high4[2 * k + 1] + high4[2 * k], 2) for k in range(32))
    return raw, sm, nib, base, spill


def random_blocks(rng, n):
    """A mix of narrow-window, wide, special-laden and arbitrary bit-pattern blocks."""
    out = []
    for i in range(n):
        kind = i % 4
        sign = rng.integers(0, 2, 64) << 15
        mant = rng.integers(0, 128, 64)
        if kind == 0:  # eligible: window of width <= 16
            lo = int(rng.integers(1, 240))
            e = lo + rng.integers(0, 16, 64)
        elif kind == 1:  # window exactly 17 wide or more
            lo = int(rng.integers(1, 200))
            e = lo + rng.integers(0, int(rng.integers(17, 54)), 64)
            e[0], e[1] = lo, lo + 16
        elif kind == 2:  # eligible but for one special
            lo = int(rng.integers(1, 240))
            e = lo + rng.integers(0, 16, 64)
            e[int(rng.integers(0, 64))] = int(rng.choice([0, 255]))
        else:  # arbitrary patterns
            out.append(rng.integers(0, 65536, 64).astype(np.uint16))
            continue
        out.append((sign | (np.minimum(e, 255) << 7) | mant).astype(np.uint16))
    return out


# ---------------------------------------------------------------- fixtures from the pages

def test_handworked_compressed_block():
    f = _fixture("block_compressed_handworked.txt")
    x = np.array([int(v, 16) for v in f["values"]], np.uint16)
    raw, sm, nib, base, spill = oracle.block_encode(x)
    assert raw is False and spill is None
    assert base == int(f["base"][0])
    assert sm.tolist() == [int(v, 16) for v in f["sm"]]
    assert nib.tolist() == [int(v, 16) for v in f["nib"]]
    assert oracle.block_decode(sm, nib, base).tolist() == x.tolist()


def test_handworked_raw_block():
    f = _fixture("block_raw_handworked.txt")
    x = np.array([int(v, 16) for v in f["values"]], np.uint16)
    raw, sm, nib, base, spill = oracle.block_encode(x)
    assert raw is True and base == 0
    assert sm.tolist() == [int(v, 16) for v in f["sm"]]
    assert nib.tolist() == [int(v, 16) for v in f["nib"]]
    assert spill.tolist() == [int(v, 16) for v in f["spill"]]
    assert oracle.block_decode(sm, nib, base, spill).tolist() == x.tolist()


def test_eligible_block_is_twelve_bits_per_value():
    f = _fixture("zipfusion_block_size.txt")
    rng = np.random.default_rng(5)
    x = random_blocks(rng, 1)[0]
    raw, sm, nib, base, spill = oracle.block_encode(x)
    assert not raw
    payload_bits = 8 * (sm.nbytes + nib.nbytes)
    assert payload_bits / 64 == int(f["bits_per_value"][0])
    assert payload_bits / (16 * 64) == float(f["fraction_of_bf16"][0])


# ---------------------------------------------------------------- exhaustive and closed forms

def test_exhaustive_constant_blocks():
    """Every bf16 pattern as a constant block: eligible iff 1 <= exponent <= 254; lossless."""
    for v in range(65536):
        x = np.full(64, v, np.uint16)
        raw, sm, nib, base, spill = oracle.block_encode(x)
        e = (v >> 7) & 0xFF
        assert raw == (e == 0 or e == 255), hex(v)
        if not raw:
            assert base == e and not nib.any()
        assert sm[0] == ((v >> 15) << 7 | (v & 0x7F))
        out = oracle.block_decode(sm, nib, base, spill)
        assert (out == v).all(), hex(v)


def test_exhaustive_pairs_roundtrip():
    """All 65 536 patterns, each next to every kind of block neighbour: decode(encode) == x."""
    pats = np.arange(65536, dtype=np.uint16).reshape(-1, 64)  # 1024 blocks of consecutive bits
    rng = np.random.default_rng(1)
    perm = rng.permutation(65536).astype(np.uint16).reshape(-1, 64)
    for blocks in (pats, perm):
        for x in blocks:
            raw, sm, nib, base, spill = oracle.block_encode(x)
            assert (oracle.block_decode(sm, nib, base, spill) == x).all()


@pytest.mark.parametrize("width_ok", [True, False])
def test_window_boundary_every_base(width_ok):
    """Spread 15 is compressed with base = min exponent; spread 16 is raw (16-wide window)."""
    rng = np.random.default_rng(2)
    spread = 15 if width_ok else 16
    for lo in range(1, 255 - spread):
        e = lo + rng.integers(0, spread + 1, 64)
        e[3], e[40] = lo, lo + spread
        x = ((rng.integers(0, 2, 64) << 15) | (e << 7) | rng.integers(0, 128, 64)).astype(np.uint16)
        raw, sm, nib, base, spill = oracle.block_encode(x)
        assert raw == (not width_ok)
        if width_ok:
            assert base == lo
        assert (oracle.block_decode(sm, nib, base, spill) == x).all()


@pytest.mark.parametrize("special", [0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC0,
                                     0x7F81, 0xFFFF])
def test_one_special_forces_raw(special):
    """A zero, subnormal, Inf or NaN anywhere in an otherwise eligible block keeps it raw,
    and the raw path preserves its bits (NaN payloads included)."""
    rng = np.random.default_rng(special)
    for pos in (0, 1, 31, 62, 63):
        e = 120 + rng.integers(0, 8, 64)
        x = ((rng.integers(0, 2, 64) << 15) | (e << 7) | rng.integers(0, 128, 64)).astype(np.uint16)
        assert not oracle.block_encode(x)[0]
        x[pos] = special
        raw, sm, nib, base, spill = oracle.block_encode(x)
        assert raw and base == 0
        assert (oracle.block_decode(sm, nib, base, spill) == x).all()


def test_against_bitstring_packer():
    rng = np.random.default_rng(3)
    for x in random_blocks(rng, 2000):
        raw, sm, nib, base, spill = oracle.block_encode(x)
        r2, sm2, nib2, base2, spill2 = bitstring_pack(x)
        assert raw == r2 and base == base2
        assert sm.tobytes() == sm2 and nib.tobytes() == nib2
        if raw:
            assert spill.tobytes() == spill2


def test_raw_block_is_a_pure_bitfield_split():
    """A raw block's stored fields are the input's bits moved, never computed: sign and
    mantissa in sm, exponent low nibble in nib, exponent high nibble in spill."""
    rng = np.random.default_rng(4)
    for x in random_blocks(rng, 400):
        raw, sm, nib, base, spill = oracle.block_encode(x)
        if not raw:
            continue
        e = _exp(x)
        lo = np.stack([nib & 15, nib >> 4], 1).reshape(-1)
        hi = np.stack([spill & 15, spill >> 4], 1).reshape(-1)
        assert (lo == (e & 15)).all() and (hi == (e >> 4)).all()
        rebuilt = ((sm.astype(np.int64) >> 7) << 15) | (((hi << 4) | lo).astype(np.int64) << 7) | (sm & 0x7F)
        assert (rebuilt == x).all()


def test_single_add_rebuild_closed_form():
    """For eligible blocks the rebuilt 16-bit word equals fields + (base << 7), i.e. a single
    integer addition, and never carries into the sign bit."""
    rng = np.random.default_rng(6)
    for x in random_blocks(rng, 400):
        raw, sm, nib, base, spill = oracle.block_encode(x)
        if raw:
            continue
        off = np.stack([nib & 15, nib >> 4], 1).reshape(-1).astype(np.int64)
        fields = ((sm.astype(np.int64) & 0x80) << 8) | (sm & 0x7F) | (off << 7)
        assert ((fields + (base << 7)) == x).all()
        assert (off + base <= 254).all()


# ---------------------------------------------------------------- cache level

def _small(**kw):
    base = synth.WORKLOADS[0].replace(batch=3, ctx_min=37, ctx_max=150, seed=11)
    return base.replace(**kw)


def _encode(inst, slots=None):
    w = inst.w
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim,
                     spill_slots=slots if slots is not None else 1 << 20)
    st = c.encode(inst.seq_lens, inst.page_table, inst.raw_pages)
    return st, c


def _rows(inst):
    T = inst.w.page_size
    for b in range(inst.w.batch):
        for t in range(int(inst.seq_lens[b])):
            yield b, t, int(inst.page_table[b, t // T]), t % T


def test_encode_roundtrip_and_size_closed_form():
    inst = synth.make(synth.WORKLOADS[0])
    st, c = _encode(inst)
    assert st == oracle.OK
    st, dec = c.decode(inst.seq_lens, inst.page_table)
    assert st == oracle.OK and np.array_equal(dec, inst.raw_pages)
    # raw blocks from the definition, counted independently of the oracle
    e = _exp(inst.raw_pages).reshape(-1, 64)
    raw_def = (e == 0).any(1) | (e == 255).any(1) | (e.max(1) - e.min(1) > 15)
    assert c.spill_top == int(raw_def.sum())
    rows = int(inst.seq_lens.sum())
    H, D = inst.w.num_kv_heads, inst.w.head_dim
    blocks_per_row = 2 * H * D // 64
    packed = rows * (blocks_per_row * (64 + 32 + 1) + 4 + 4) + 32 * c.spill_top
    assert packed == rows * 3112 + 32 * int(raw_def.sum())
    assert (c.base.reshape(-1) == 0).sum() == raw_def.sum()


def test_flags_base_and_spill_order():
    inst = synth.make(_small())
    st, c = _encode(inst)
    assert st == oracle.OK
    H, D = inst.w.num_kv_heads, inst.w.head_dim
    nb = D // 64
    expect_slot = 0
    for b, t, page, slot in _rows(inst):
        flags = int(c.row_flags[page, slot])
        assert int(c.row_spill[page, slot]) == expect_slot  # canonical (seq, token) order
        for h in range(H):
            for kv in range(2):
                for half in range(nb):
                    j = (h * 2 + kv) * nb + half
                    x = inst.raw_pages[page, h, kv, slot, half * 64:(half + 1) * 64]
                    raw, sm, nib, base, spill = bitstring_pack(x)
                    assert ((flags >> j) & 1) == raw
                    assert c.base[page, h, kv, slot, half] == base
                    if raw:
                        k = expect_slot + bin(flags & ((1 << j) - 1)).count("1")
                        assert c.spill[k].tobytes() == spill
        expect_slot += bin(flags).count("1")
    assert c.spill_top == expect_slot


def test_idempotent():
    inst = synth.make(_small(seed=12))
    _, c1 = _encode(inst)
    _, dec = c1.decode(inst.seq_lens, inst.page_table)
    inst2 = synth.Instance(inst.w, inst.seq_lens, inst.page_table, inst.num_pages, dec)
    _, c2 = _encode(inst2)
    for name in ("sm", "nib", "base", "row_flags", "row_spill", "spill"):
        a, b = getattr(c1, name), getattr(c2, name)
        if name in ("sm", "nib", "base"):
            mask = _valid_mask(inst, a.shape)
            assert np.array_equal(a[mask], b[mask]), name
        elif name in ("row_flags", "row_spill"):
            m = _valid_rows(inst)
            assert np.array_equal(a[m], b[m]), name
        else:
            assert np.array_equal(a[:c1.spill_top], b[:c2.spill_top])


def _valid_rows(inst):
    m = np.zeros((inst.num_pages, inst.w.page_size), bool)
    for _, _, page, slot in _rows(inst):
        m[page, slot] = True
    return m


def _valid_mask(inst, shape):
    m = _valid_rows(inst)
    return np.broadcast_to(m[:, None, None, :, None], shape)


def test_append_matches_encode():
    """Token-by-token appends decode to the same values as a full encode, with identical
    per-block fields; only spill slot numbers differ (append takes them in batch order)."""
    w = _small(seed=13, ctx_min=20, ctx_max=40)
    inst = synth.make(w)
    _, full = _encode(inst)
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=1 << 20)
    lens = np.zeros(w.batch, np.int32)
    H, D = w.num_kv_heads, w.head_dim
    for t in range(int(inst.seq_lens.max())):
        # sequences that already hold all their tokens are appended again with fresh tokens
        # only while t < their length; others take part through a sub-batch
        act = np.nonzero(inst.seq_lens > t)[0]
        sub_lens = lens[act].copy()
        k = np.zeros((len(act), H, D), np.uint16)
        v = np.zeros_like(k)
        for i, b in enumerate(act):
            page = inst.page_table[b, t // w.page_size]
            k[i] = inst.raw_pages[page, :, 0, t % w.page_size]
            v[i] = inst.raw_pages[page, :, 1, t % w.page_size]
        st = c.append(sub_lens, inst.page_table[act], k, v)
        assert st == oracle.OK
        assert (sub_lens == lens[act] + 1).all()
        lens[act] = sub_lens
    assert np.array_equal(lens, inst.seq_lens)
    st, dec = c.decode(inst.seq_lens, inst.page_table)
    assert st == oracle.OK
    mask = _valid_mask(inst, dec.shape)
    assert np.array_equal(dec[mask], inst.raw_pages[mask])
    rows = _valid_rows(inst)
    assert np.array_equal(c.row_flags[rows], full.row_flags[rows])
    for name in ("sm", "nib", "base"):
        m = _valid_mask(inst, getattr(c, name).shape)
        assert np.array_equal(getattr(c, name)[m], getattr(full, name)[m])
    assert c.spill_top == full.spill_top
    # batch-order slots: within one append call the rows' slots rise with the batch index
    assert sorted(c.spill[:c.spill_top].tobytes()) == sorted(full.spill[:full.spill_top].tobytes())


def test_append_spill_order_is_batch_order():
    w = _small(seed=14, batch=5, ctx_min=16, ctx_max=16, extra_tokens=1)
    inst = synth.make(w)
    _, c = _encode(inst)
    top0 = c.spill_top
    pos = inst.seq_lens.copy()
    k, v = synth.tokens(w, pos)
    lens = inst.seq_lens.copy()
    assert c.append(lens, inst.page_table, k, v) == oracle.OK
    nxt = top0
    for b in range(w.batch):
        page, slot = inst.page_table[b, pos[b] // 16], pos[b] % 16
        assert c.row_spill[page, slot] == nxt
        nxt += bin(int(c.row_flags[page, slot])).count("1")
    assert c.spill_top == nxt


def test_spill_exhaustion_is_all_or_nothing():
    inst = synth.make(_small(seed=15, extra_tokens=1))
    _, ref = _encode(inst)
    need = ref.spill_top
    st, c = _encode(inst, slots=need)
    assert st == oracle.OK and c.spill_top == need
    st, c = _encode(inst, slots=need - 1)
    assert st == oracle.ESPILL and c.spill_top == 0 and not c.spill.any()
    # append: same rule, and seq_lens stay put
    w = inst.w
    lens = inst.seq_lens.copy()
    pt = inst.page_table
    st, c = _encode(inst, slots=need)
    k, v = synth.tokens(w, lens)
    k[:, :, 0] = 0  # force at least one raw block per row
    before = c.spill.copy()
    assert c.append(lens, pt, k, v) == oracle.ESPILL
    assert np.array_equal(lens, inst.seq_lens) and c.spill_top == need
    assert np.array_equal(before, c.spill)


def test_top_beyond_the_pool_counts_as_full():
    """A spill_top past spill_slots (no call leaves one; a caller might) holds no free slot:
    encode and append report exhaustion and write nothing, even when no new block is raw."""
    inst = synth.make(_small(seed=15, extra_tokens=1))
    w = inst.w
    st, c = _encode(inst, slots=1 << 16)
    assert st == oracle.OK
    c.spill_slots = c.spill_top - 1
    lens = inst.seq_lens.copy()
    k, v = synth.tokens(w, lens)
    k[:] = 0x3F80  # 1.0 everywhere: no raw block, nothing to spill
    v[:] = 0x3F80
    before = c.spill.copy()
    top = c.spill_top
    assert c.append(lens, inst.page_table, k, v) == oracle.ESPILL
    assert np.array_equal(lens, inst.seq_lens) and c.spill_top == top
    assert np.array_equal(before, c.spill)
    c2 = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, 8)
    c2.spill_top = 9
    assert c2.encode(inst.seq_lens, inst.page_table, inst.raw_pages) == oracle.ESPILL
    assert c2.spill_top == 9 and not c2.spill.any()


def test_bad_page_and_length_are_reported():
    inst = synth.make(_small(seed=16))
    pt = inst.page_table.copy()
    pt[1, 0] = inst.num_pages  # out of range
    st, _ = _encode(synth.Instance(inst.w, inst.seq_lens, pt, inst.num_pages, inst.raw_pages))
    assert st & oracle.EPAGE
    lens = inst.seq_lens.copy()
    lens[0] = pt.shape[1] * 16 + 1
    st, _ = _encode(synth.Instance(inst.w, lens, inst.page_table, inst.num_pages, inst.raw_pages))
    assert st & oracle.ELEN


# ---------------------------------------------------------------- multi-token append

def _tokens_of(inst, b, t0, n):
    """K, V rows of tokens t0..t0+n-1 of sequence b from the raw pages: two u16[n][H][D]."""
    T = inst.w.page_size
    ks, vs = [], []
    for t in range(t0, t0 + n):
        page = inst.page_table[b, t // T]
        ks.append(inst.raw_pages[page, :, 0, t % T])
        vs.append(inst.raw_pages[page, :, 1, t % T])
    return np.stack(ks), np.stack(vs)


def _chunk(inst, lens, n):
    k = np.stack([_tokens_of(inst, b, int(lens[b]), n)[0] for b in range(inst.w.batch)])
    v = np.stack([_tokens_of(inst, b, int(lens[b]), n)[1] for b in range(inst.w.batch)])
    return k, v


def test_append_n_from_empty_is_an_encode():
    """All tokens of equal-length sequences appended in one call land exactly as a full encode
    lays them out: same fields, same spill slots ((sequence, token) order in both)."""
    w = _small(seed=17, ctx_min=45, ctx_max=45)
    inst = synth.make(w)
    _, full = _encode(inst)
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=1 << 20)
    lens = np.zeros(w.batch, np.int32)
    k, v = _chunk(inst, lens, 45)
    assert c.append_n(lens, inst.page_table, k, v) == oracle.OK
    assert (lens == 45).all()
    rows = _valid_rows(inst)
    for name in ("row_flags", "row_spill"):
        assert np.array_equal(getattr(c, name)[rows], getattr(full, name)[rows]), name
    for name in ("sm", "nib", "base"):
        m = _valid_mask(inst, getattr(c, name).shape)
        assert np.array_equal(getattr(c, name)[m], getattr(full, name)[m]), name
    assert c.spill_top == full.spill_top
    assert np.array_equal(c.spill[:c.spill_top], full.spill[:full.spill_top])


def test_append_n_chunks_roundtrip_and_slot_order():
    """Chunks of 5, 1, 16, 9 and 2 tokens, crossing page boundaries: lossless, and within each
    call the first spill slot of row (b, j) counts the raw blocks of all rows before it in
    (sequence, token) order, counted from the row flags independently of the oracle."""
    w = _small(seed=18, ctx_min=33, ctx_max=33)
    inst = synth.make(w)
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=1 << 20)
    lens = np.zeros(w.batch, np.int32)
    T = w.page_size
    for n in (5, 1, 16, 9, 2):
        k, v = _chunk(inst, lens, n)
        pos = lens.copy()
        top = c.spill_top
        assert c.append_n(lens, inst.page_table, k, v) == oracle.OK
        assert np.array_equal(lens, pos + n)
        nxt = top
        for b in range(w.batch):
            for j in range(n):
                t = int(pos[b]) + j
                page, slot = inst.page_table[b, t // T], t % T
                assert c.row_spill[page, slot] == nxt
                nxt += bin(int(c.row_flags[page, slot])).count("1")
        assert c.spill_top == nxt
    st, dec = c.decode(lens, inst.page_table)
    assert st == oracle.OK
    mask = _valid_mask(inst, dec.shape)
    assert np.array_equal(dec[mask], inst.raw_pages[mask])


def test_append_n_one_token_is_append_and_zero_is_a_no_op():
    w = _small(seed=19, extra_tokens=1)
    inst = synth.make(w)
    _, a = _encode(inst)
    _, b = _encode(inst)
    la, lb = inst.seq_lens.copy(), inst.seq_lens.copy()
    k, v = synth.tokens(w, la)
    assert a.append(la, inst.page_table, k, v) == oracle.OK
    assert b.append_n(lb, inst.page_table, k[:, None], v[:, None]) == oracle.OK
    assert np.array_equal(la, lb) and a.spill_top == b.spill_top
    for name in ("sm", "nib", "base", "row_flags", "row_spill", "spill"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    before = b.spill.copy()
    empty = np.zeros((w.batch, 0, w.num_kv_heads, w.head_dim), np.uint16)
    assert b.append_n(lb, inst.page_table, empty, empty) == oracle.OK
    assert np.array_equal(lb, la) and np.array_equal(before, b.spill)


def test_append_n_errors_change_nothing():
    w = _small(seed=20, ctx_min=20, ctx_max=20)
    inst = synth.make(w)
    lens = np.full(w.batch, 3, np.int32)
    k, v = _chunk(inst, lens, 6)
    k[:, :, :, 0] = 0  # every row gets raw blocks
    need_c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=1 << 20)
    l2 = lens.copy()
    assert need_c.append_n(l2, inst.page_table, k, v) == oracle.OK
    need = need_c.spill_top
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=need - 1)
    l3 = lens.copy()
    assert c.append_n(l3, inst.page_table, k, v) == oracle.ESPILL
    assert np.array_equal(l3, lens) and c.spill_top == 0 and not c.spill.any()
    # a chunk running past the page table, and a bad page id on the way
    big = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots=1 << 20)
    l4 = np.full(w.batch, inst.page_table.shape[1] * w.page_size - 2, np.int32)
    assert big.append_n(l4, inst.page_table, k, v) & oracle.ELEN
    pt = inst.page_table.copy()
    pt[0, 0] = -1
    l5 = lens.copy()
    assert big.append_n(l5, pt, k, v) & oracle.EPAGE
    assert np.array_equal(l5, lens) and big.spill_top == 0
