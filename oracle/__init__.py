"""CPU oracle for the compressed-KV decode-attention path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this package; the product path never does.  The arithmetic lives
in plain C (``zf_oracle.c``: the block codec written from its definition, fp64 attention);
this module compiles it with gcc and marshals numpy arrays; the attention's page-order hint
(``page_kmax``) is plain numpy here.  It shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zf_oracle.c")
_HDR = os.path.join(_HERE, "zf_oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, ESPILL, EPAGE, ELEN = 0, 1, 2, 4


def build() -> str:
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
                           "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("ZF_ORACLE_LIB")  # another build of the same source (sanitizers)
        if not path:
            newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
                build()
            path = _LIB
        lib = ctypes.CDLL(path)
        for name in ("orc_encode_kv", "orc_append_kv", "orc_append_kv_n", "orc_decode_kv",
                     "orc_compact_spill", "orc_attention"):
            getattr(lib, name).restype = ctypes.c_uint32
        lib.orc_max_sequences.restype = ctypes.c_int64
        lib.orc_max_sequences.argtypes = [ctypes.c_int64] + [ctypes.c_int32] * 5 + [ctypes.c_double]
        lib.orc_block_encode.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class _Geom(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class _Cache(ctypes.Structure):
    _fields_ = [("sm", ctypes.c_void_p), ("nib", ctypes.c_void_p), ("base", ctypes.c_void_p),
                ("row_flags", ctypes.c_void_p), ("row_spill", ctypes.c_void_p),
                ("spill", ctypes.c_void_p), ("spill_slots", ctypes.c_uint64),
                ("spill_top", ctypes.c_uint64)]


def block_encode(x: np.ndarray):
    """One 64-value block -> (raw, sm u8[64], nib u8[32], base, spill u8[32] or None)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert x.shape == (64,)
    sm = np.zeros(64, np.uint8)
    nib = np.zeros(32, np.uint8)
    spill = np.zeros(32, np.uint8)
    base = ctypes.c_uint8()
    raw = _load().orc_block_encode(_p(x), _p(sm), _p(nib), ctypes.byref(base), _p(spill))
    return bool(raw), sm, nib, int(base.value), (spill if raw else None)


def block_decode(sm, nib, base, spill=None) -> np.ndarray:
    out = np.zeros(64, np.uint16)
    sp = np.zeros(32, np.uint8) if spill is None else np.ascontiguousarray(spill, np.uint8)
    _load().orc_block_decode(_p(np.ascontiguousarray(sm, np.uint8)),
                             _p(np.ascontiguousarray(nib, np.uint8)), ctypes.c_uint8(base),
                             _p(sp), _p(out))
    return out


@dataclasses.dataclass
class Cache:
    """Packed paged cache in host memory (the format's byte layout)."""
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    spill_slots: int
    sm: np.ndarray = None
    nib: np.ndarray = None
    base: np.ndarray = None
    row_flags: np.ndarray = None
    row_spill: np.ndarray = None
    spill: np.ndarray = None
    spill_top: int = 0

    def __post_init__(self):
        P, H, T, D = self.num_pages, self.num_kv_heads, self.page_size, self.head_dim
        assert D % 64 == 0 and 2 * H * (D // 64) <= 32, "a token row holds at most 32 blocks"
        if self.sm is None:
            self.sm = np.zeros((P, H, 2, T, D), np.uint8)
            self.nib = np.zeros((P, H, 2, T, D // 2), np.uint8)
            self.base = np.zeros((P, H, 2, T, D // 64), np.uint8)
            self.row_flags = np.zeros((P, T), np.uint32)
            self.row_spill = np.zeros((P, T), np.uint32)
            self.spill = np.zeros((max(self.spill_slots, 1), 32), np.uint8)

    def _geom(self):
        return _Geom(self.num_pages, self.page_size, self.num_kv_heads, self.head_dim)

    def _c(self):
        return _Cache(self.sm.ctypes.data, self.nib.ctypes.data, self.base.ctypes.data,
                      self.row_flags.ctypes.data, self.row_spill.ctypes.data,
                      self.spill.ctypes.data, self.spill_slots, self.spill_top)

    def encode(self, seq_lens, page_table, raw_pages) -> int:
        c = self._c()
        lens = np.ascontiguousarray(seq_lens, np.int32)
        pt = np.ascontiguousarray(page_table, np.int32)
        st = _load().orc_encode_kv(ctypes.byref(self._geom()), ctypes.byref(c),
                                   ctypes.c_int32(len(lens)), _p(lens), _p(pt),
                                   ctypes.c_int32(pt.shape[1]),
                                   _p(np.ascontiguousarray(raw_pages, np.uint16)))
        self.spill_top = int(c.spill_top)
        return int(st)

    def append(self, seq_lens: np.ndarray, page_table, k_new, v_new) -> int:
        """Appends one token per sequence at seq_lens[b]; advances ``seq_lens`` in place."""
        assert seq_lens.dtype == np.int32 and seq_lens.flags.c_contiguous
        c = self._c()
        pt = np.ascontiguousarray(page_table, np.int32)
        st = _load().orc_append_kv(ctypes.byref(self._geom()), ctypes.byref(c),
                                   ctypes.c_int32(len(seq_lens)), _p(seq_lens), _p(pt),
                                   ctypes.c_int32(pt.shape[1]),
                                   _p(np.ascontiguousarray(k_new, np.uint16)),
                                   _p(np.ascontiguousarray(v_new, np.uint16)))
        self.spill_top = int(c.spill_top)
        return int(st)

    def append_n(self, seq_lens: np.ndarray, page_table, k_new, v_new) -> int:
        """Appends n tokens per sequence (k_new, v_new u16[B][n][H][D]) at seq_lens[b];
        advances ``seq_lens`` in place by n."""
        assert seq_lens.dtype == np.int32 and seq_lens.flags.c_contiguous
        k = np.ascontiguousarray(k_new, np.uint16)
        assert k.ndim == 4 and k.shape[0] == len(seq_lens)
        c = self._c()
        pt = np.ascontiguousarray(page_table, np.int32)
        st = _load().orc_append_kv_n(ctypes.byref(self._geom()), ctypes.byref(c),
                                     ctypes.c_int32(len(seq_lens)), ctypes.c_int32(k.shape[1]),
                                     _p(seq_lens), _p(pt), ctypes.c_int32(pt.shape[1]), _p(k),
                                     _p(np.ascontiguousarray(v_new, np.uint16)))
        self.spill_top = int(c.spill_top)
        return int(st)

    def compact(self, seq_lens, page_table) -> int:
        """Rewrites the spill pool for the listed sequences only (slots from 0 in (sequence,
        token) order); the other sequences' slots are given up."""
        c = self._c()
        lens = np.ascontiguousarray(seq_lens, np.int32)
        pt = np.ascontiguousarray(page_table, np.int32)
        st = _load().orc_compact_spill(ctypes.byref(self._geom()), ctypes.byref(c),
                                       ctypes.c_int32(len(lens)), _p(lens), _p(pt),
                                       ctypes.c_int32(pt.shape[1]))
        self.spill_top = int(c.spill_top)
        return int(st)

    def decode(self, seq_lens, page_table, out: np.ndarray | None = None):
        if out is None:
            out = np.zeros((self.num_pages, self.num_kv_heads, 2, self.page_size,
                            self.head_dim), np.uint16)
        lens = np.ascontiguousarray(seq_lens, np.int32)
        pt = np.ascontiguousarray(page_table, np.int32)
        st = _load().orc_decode_kv(ctypes.byref(self._geom()), ctypes.byref(self._c()),
                                   ctypes.c_int32(len(lens)), _p(lens), _p(pt),
                                   ctypes.c_int32(pt.shape[1]), _p(out))
        return int(st), out


def page_kmax(raw_pages: np.ndarray, seq_lens, page_table) -> np.ndarray:
    """The attention's page-order hint, from its definition: for each (sequence b, kv head h,
    logical page p) the largest bf16 exponent field (bits 7..14 of the value) among the K values
    of the page's tokens t < seq_lens[b]; 0 for a page that holds none.  uint32
    [B][H][max_pages].  Plain numpy; not part of the pages' method (it only orders the pages
    the attention visits), so its definition is the whole of it."""
    P, H, two, T, D = raw_pages.shape
    pt = np.asarray(page_table, np.int64)
    B, maxp = pt.shape
    out = np.zeros((B, H, maxp), np.uint32)
    for b in range(B):
        L = int(seq_lens[b])
        for p in range(min(maxp, -(-L // T))):
            n = min(T, L - p * T)
            k = raw_pages[pt[b, p], :, 0, :n, :]            # [H][n][D] bf16 bits
            e = (k.astype(np.uint32) >> 7) & 0xFF           # exponent fields
            out[b, :, p] = e.reshape(H, -1).max(axis=1)
    return out


def max_sequences(kv_budget: int, layers: int, context: int, page_size: int, num_kv_heads: int,
                  head_dim: int, raw_blocks_per_row: float | None) -> int:
    """Sequences of ``context`` tokens whose caches fit in ``kv_budget`` bytes over ``layers``
    layers; ``raw_blocks_per_row`` None = uncompressed bf16 pages."""
    r = -1.0 if raw_blocks_per_row is None else float(raw_blocks_per_row)
    return int(_load().orc_max_sequences(kv_budget, layers, context, page_size, num_kv_heads,
                                         head_dim, r))


def attention(raw_pages: np.ndarray, seq_lens, page_table, q: np.ndarray,
              scale: float | None = None, want: np.ndarray | None = None,
              threads: int = 1, with_neff: bool = False):
    """fp64 decode attention; returns (status, out f64[B][Hq][D]) or, with ``with_neff``,
    (status, out, neff f64[B][Hq]) where neff is each row's effective number of tokens.

    ``threads`` > 1 runs the unchanged C routine on disjoint slices of the wanted rows at once
    (each call computes only its slice, selected through ``want``; ctypes releases the GIL), so
    every row is computed exactly as a single call computes it."""
    P, H, two, T, D = raw_pages.shape
    B, Hq, Dq = q.shape
    assert two == 2 and Dq == D and Hq % H == 0
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, D), np.float64)
    neff = np.zeros((B, Hq), np.float64)
    lens = np.ascontiguousarray(seq_lens, np.int32)
    pt = np.ascontiguousarray(page_table, np.int32)
    pages = np.ascontiguousarray(raw_pages, np.uint16)
    qq = np.ascontiguousarray(q, np.uint16)
    wnt = np.ones((B, Hq), np.uint8) if want is None else np.ascontiguousarray(want, np.uint8)
    g = _Geom(P, T, H, D)
    lib = _load()

    def run(mask):
        return int(lib.orc_attention(ctypes.byref(g), ctypes.c_int32(B), ctypes.c_int32(Hq),
                                     _p(lens), _p(pt), ctypes.c_int32(pt.shape[1]), _p(pages),
                                     _p(qq), ctypes.c_double(scale), _p(mask), _p(out),
                                     _p(neff)))

    rows = np.flatnonzero(wnt.reshape(-1))
    if threads <= 1 or len(rows) < 2:
        st = run(wnt)
    else:
        import concurrent.futures
        masks = []
        for part in np.array_split(rows, min(threads, len(rows))):
            m = np.zeros(B * Hq, np.uint8)
            m[part] = 1
            masks.append(m.reshape(B, Hq))
        with concurrent.futures.ThreadPoolExecutor(len(masks)) as ex:
            sts = list(ex.map(run, masks))
        st = 0
        for x in sts:
            st |= x
    return (int(st), out, neff) if with_neff else (int(st), out)
