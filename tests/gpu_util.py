"""Shared setup for the GPU parity tests: workloads on the device, oracle counterparts."""
from __future__ import annotations

import sys

import numpy as np
import torch

import decode_attention_encode_amd as zf
import oracle
import synth


def attention_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) as the C ABI carries it (an fp32 argument): the oracle is handed the
    same value, so both sides compute the definition with the same scale."""
    return float(np.float32(1.0 / np.sqrt(head_dim)))


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def spill_need(inst: synth.Instance, extra_rows: int = 0) -> int:
    """Upper bound on the spill slots a workload needs (every block of every row raw)."""
    w = inst.w
    rows = int(inst.seq_lens.sum()) + extra_rows
    return rows * 2 * w.num_kv_heads * (w.head_dim // 64)


class Setup:
    """One workload resident on the GPU: raw pages, packed cache (GPU-encoded), seqs."""

    def __init__(self, inst: synth.Instance, spill_slots: int | None = None, max_seq_len=None,
                 encode=True, one_launch_append=True, kmax=True):
        self.inst = inst
        w = inst.w
        self.w = w
        if spill_slots is None:
            spill_slots = spill_need(inst, w.batch * (w.extra_tokens + 1))
        self.raw = dev(inst.raw_pages)
        self.cache = zf.PackedCache.empty(inst.num_pages, w.page_size, w.num_kv_heads,
                                          w.head_dim, spill_slots,
                                          one_launch_append=one_launch_append)
        cap = inst.page_table.shape[1] * w.page_size
        # the page-order hint, poisoned: the encode writes every entry
        hint = None
        if kmax:
            B, maxp = inst.page_table.shape
            hint = torch.full((B, w.num_kv_heads, maxp), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
        self.seqs = zf.Seqs(dev(inst.page_table), dev(inst.seq_lens.copy()),
                            int(max_seq_len if max_seq_len is not None else cap), hint)
        if encode:
            ws = zf.encode_workspace(self.seqs)
            zf.zf_encode_kv(self.cache, self.seqs, self.raw, ws)
            torch.cuda.synchronize()

    def status(self) -> int:
        return zf.zf_get_status(self.cache.status)

    def attention(self, q: np.ndarray, packed=True, out=None, ws=None) -> torch.Tensor:
        w = self.w
        qd = dev(q)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        if ws is None:
            ws = zf.attention_workspace(w.batch, w.num_kv_heads, q.shape[1], w.head_dim,
                                        self.seqs.max_seq_len)
        scale = attention_scale(w.head_dim)
        if packed:
            zf.zf_decode_attention(self.cache, self.seqs, qd, scale, out, ws)
        else:
            zf.zf_decode_attention_raw(self.raw, self.seqs, qd, scale, out, ws, self.cache.status)
        torch.cuda.synchronize()
        return out


def check_kmax(s: Setup, orc: oracle.Cache, lens, what=""):
    """The device's page-order hint equals the oracle's, from the oracle cache's decoded pages."""
    st, raw = orc.decode(lens, s.inst.page_table)
    assert st == oracle.OK
    want = oracle.page_kmax(raw, lens, s.inst.page_table)
    got = host(s.seqs.kmax, np.uint32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{what} kmax: {len(bad)} entries differ, first {bad[:4].tolist()}"


def oracle_cache(inst: synth.Instance, spill_slots: int) -> oracle.Cache:
    w = inst.w
    c = oracle.Cache(inst.num_pages, w.page_size, w.num_kv_heads, w.head_dim, spill_slots)
    st = c.encode(inst.seq_lens, inst.page_table, inst.raw_pages)
    assert st == oracle.OK
    return c


def valid_rows(inst: synth.Instance, lens=None) -> np.ndarray:
    lens = inst.seq_lens if lens is None else lens
    T = inst.w.page_size
    m = np.zeros((inst.num_pages, T), bool)
    for b in range(inst.w.batch):
        L = int(lens[b])
        if L == 0:
            continue
        pages = inst.page_table[b, : (L + T - 1) // T]
        full = L // T
        m[pages[:full]] = True
        if L % T:
            m[pages[full], : L % T] = True
    return m


def compare_packed(gpu: zf.PackedCache, orc: oracle.Cache, rows: np.ndarray, what=""):
    """Bit-exact comparison of every defined field; returns nothing, asserts."""
    def g(t, dt=None):
        return host(t, dt)
    assert int(g(gpu.spill_top)[0]) == orc.spill_top, f"{what} spill_top"
    for name in ("sm", "nib", "base"):
        a = g(getattr(gpu, name))
        b = getattr(orc, name)
        m = np.broadcast_to(rows[:, None, None, :, None], a.shape)
        bad = np.count_nonzero(a[m] != b[m])
        assert bad == 0, f"{what} {name}: {bad} bytes differ"
    for name in ("row_flags", "row_spill"):
        a = g(getattr(gpu, name), np.uint32)
        b = getattr(orc, name)
        bad = np.count_nonzero(a[rows] != b[rows])
        assert bad == 0, f"{what} {name}: {bad} rows differ"
    top = orc.spill_top
    a = g(gpu.spill)[:top]
    assert np.array_equal(a, orc.spill[:top]), f"{what} spill bytes differ"
