"""GPU parity for the spill lifecycle: zf_compact_spill through the C ABI, bit-exact against the
oracle's compaction after encode, appends and freed sequences (spill index, spill bytes,
spill_top; planes untouched), attention unchanged bit for bit, appends continuing from the new
top, and the all-or-nothing error rules.

Paged cache whose pages come and go with their sequences: page "Open Weights: from files to
tokens / second", section "09 / The optimization stack".
"""
import numpy as np
import pytest
import torch

import decode_attention_encode_amd as zf
import oracle
import synth
from gpu_util import Setup, compare_packed, dev, host, log, oracle_cache, valid_rows

pytestmark = pytest.mark.gpu

SMALL = synth.WORKLOADS[0].replace(name="ragged_small", batch=7, ctx_min=1, ctx_max=300,
                                   extra_tokens=6, pool_factor=1.3, p_wide_block=0.05, seed=41)


def _grown(w, steps):
    """GPU and oracle caches after an encode of every sequence and `steps` one-token appends
    (the appended slots interleave the sequences)."""
    inst = synth.make(w)
    s = Setup(inst)
    orc = oracle_cache(inst, s.cache.spill_slots)
    lens = inst.seq_lens.copy()
    for _ in range(steps):
        k, v = synth.tokens(w, lens)
        zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
        assert orc.append(lens, inst.page_table, k, v) == oracle.OK
    torch.cuda.synchronize()
    assert s.status() == 0
    return inst, s, orc, lens


def _live_seqs(inst, lens, live):
    return zf.Seqs(dev(np.ascontiguousarray(inst.page_table[live])), dev(lens[live].copy()),
                   int(inst.page_table.shape[1] * inst.w.page_size))


def _live_rows(inst, lens, live):
    keep = np.zeros(inst.w.batch, bool)
    keep[live] = True
    return valid_rows(inst, np.where(keep, lens, 0))


def _device_state(cache):
    return {n: host(getattr(cache, n)).copy()
            for n in ("sm", "nib", "base", "row_flags", "row_spill", "spill", "spill_top")}


@pytest.mark.parametrize("key,steps,live", [
    ("small", 6, "odd"), ("small", 3, "all"), (1, 2, "even"), (3, 1, "first_half"), (4, 16, "all"),
])
def test_compact_bitexact(key, steps, live):
    w = SMALL if key == "small" else synth.WORKLOADS[key]
    w = w.replace(extra_tokens=max(w.extra_tokens, steps))
    log(f"compaction parity: workload {w.name}, {steps} appends, live {live}")
    inst, s, orc, lens = _grown(w, steps)
    B = w.batch
    ids = {"odd": list(range(1, B, 2)), "even": list(range(0, B, 2)), "all": list(range(B)),
           "first_half": list(range(B // 2))}[live]
    q = synth.query(w, 0)[ids]
    live_seqs = _live_seqs(inst, lens, ids)
    scale = 1.0 / float(np.sqrt(w.head_dim))
    out_before = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws_attn = zf.attention_workspace(len(ids), w.num_kv_heads, q.shape[1], w.head_dim,
                                     live_seqs.max_seq_len)
    zf.zf_decode_attention(s.cache, live_seqs, dev(q), scale, out_before, ws_attn)
    planes = {n: host(getattr(s.cache, n)).copy() for n in ("sm", "nib", "base", "row_flags")}
    top_before = int(host(s.cache.spill_top)[0])

    zf.zf_compact_spill(s.cache, live_seqs, zf.compact_workspace(s.cache, live_seqs))
    assert orc.compact(lens[ids], inst.page_table[ids]) == oracle.OK
    torch.cuda.synchronize()
    assert s.status() == 0
    rows = _live_rows(inst, lens, ids)
    compare_packed(s.cache, orc, rows, f"{w.name} compacted")
    assert orc.spill_top <= top_before
    log(f"  spill_top {top_before} -> {orc.spill_top}")
    for n, a in planes.items():
        assert np.array_equal(host(getattr(s.cache, n)), a), f"{n} changed"

    out_after = torch.empty_like(out_before)
    zf.zf_decode_attention(s.cache, live_seqs, dev(q), scale, out_after, ws_attn)
    torch.cuda.synchronize()
    assert torch.equal(out_before, out_after), "attention changed after compaction"
    raw = torch.zeros_like(s.raw)
    zf.zf_decode_kv(s.cache, live_seqs, raw)
    torch.cuda.synchronize()
    got = host(raw, np.uint16)
    st, want = orc.decode(lens[ids], inst.page_table[ids])  # appended rows are not in raw_pages
    assert st == oracle.OK
    m = np.broadcast_to(rows[:, None, None, :, None], got.shape)
    assert np.array_equal(got[m], want[m])


def test_append_after_compaction_matches_oracle():
    w = SMALL
    inst, s, orc, lens = _grown(w, 3)
    ids = [0, 2, 3, 6]
    live_lens = lens[ids].copy()
    live_seqs = _live_seqs(inst, lens, ids)
    zf.zf_compact_spill(s.cache, live_seqs, zf.compact_workspace(s.cache, live_seqs))
    assert orc.compact(live_lens, inst.page_table[ids]) == oracle.OK
    pt = np.ascontiguousarray(inst.page_table[ids])
    for step in range(3):
        k, v = synth.tokens(w, lens)
        k, v = np.ascontiguousarray(k[ids]), np.ascontiguousarray(v[ids])
        zf.zf_append_kv(s.cache, live_seqs, dev(k), dev(v))
        assert orc.append(live_lens, pt, k, v) == oracle.OK
    torch.cuda.synchronize()
    assert s.status() == 0
    assert np.array_equal(host(live_seqs.seq_lens), live_lens)
    full = lens.copy()
    full[ids] = live_lens
    compare_packed(s.cache, orc, _live_rows(inst, full, ids), "append after compaction")


def test_compact_errors_change_nothing():
    w = SMALL
    inst, s, orc, lens = _grown(w, 2)
    ids = list(range(w.batch))
    seqs = _live_seqs(inst, lens, ids)
    T = w.page_size
    flags = host(s.cache.row_flags, np.uint32)
    top = int(host(s.cache.spill_top)[0])
    # a listed row whose raw blocks would run one slot past spill_top
    b = next(b for b in ids if any(flags[inst.page_table[b, t // T], t % T] for t in range(lens[b])))
    t = next(t for t in range(lens[b]) if flags[inst.page_table[b, t // T], t % T])
    p, r = inst.page_table[b, t // T], t % T
    n = bin(int(flags[p, r])).count("1")
    row_spill = host(s.cache.row_spill, np.uint32).copy()
    row_spill[p, r] = top - n + 1
    s.cache.row_spill.copy_(dev(row_spill))
    torch.cuda.synchronize()
    before = _device_state(s.cache)
    zf.zf_compact_spill(s.cache, seqs, zf.compact_workspace(s.cache, seqs))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_ESPILL
    for n_, a in before.items():
        assert np.array_equal(host(getattr(s.cache, n_)), a), f"{n_} changed after a failed call"

    # a staging area too small for the live blocks (the header and counts are there)
    inst, s, orc, lens = _grown(w, 2)
    seqs = _live_seqs(inst, lens, ids)
    need = zf.zf_compact_workspace_bytes(s.cache, seqs) - 32 * s.cache.spill_slots
    small = torch.empty(need + 32 * (orc.spill_top - 1), dtype=torch.uint8, device="cuda")
    before = _device_state(s.cache)
    zf.zf_compact_spill(s.cache, seqs, small)
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_ESPILL
    for n_, a in before.items():
        assert np.array_equal(host(getattr(s.cache, n_)), a), f"{n_} changed after a failed call"
    # exactly enough staging: succeeds
    exact = torch.empty(need + 32 * orc.spill_top, dtype=torch.uint8, device="cuda")
    s.cache.status.zero_()
    zf.zf_compact_spill(s.cache, seqs, exact)
    assert orc.compact(lens, inst.page_table) == oracle.OK
    torch.cuda.synchronize()
    assert s.status() == 0
    compare_packed(s.cache, orc, valid_rows(inst, lens), "exact staging")

    # a page id outside the pool
    inst, s, orc, lens = _grown(w, 1)
    pt = inst.page_table.copy()
    pt[1, 0] = inst.num_pages + 3
    bad = zf.Seqs(dev(pt), dev(lens.copy()), int(pt.shape[1] * T))
    before = _device_state(s.cache)
    zf.zf_compact_spill(s.cache, bad, zf.compact_workspace(s.cache, bad))
    torch.cuda.synchronize()
    assert s.status() & zf.ZF_DEV_EPAGE
    for n_, a in before.items():
        assert np.array_equal(host(getattr(s.cache, n_)), a), f"{n_} changed after a failed call"


def test_compact_with_no_live_sequence_empties_the_pool():
    inst, s, orc, lens = _grown(SMALL, 1)
    empty = zf.Seqs(dev(np.zeros((0, inst.page_table.shape[1]), np.int32)),
                    dev(np.zeros(0, np.int32)), 0)
    before = _device_state(s.cache)
    zf.zf_compact_spill(s.cache, empty, zf.compact_workspace(s.cache, empty))
    torch.cuda.synchronize()
    assert s.status() == 0
    assert int(host(s.cache.spill_top)[0]) == 0
    for n_, a in before.items():
        if n_ != "spill_top":
            assert np.array_equal(host(getattr(s.cache, n_)), a), n_
