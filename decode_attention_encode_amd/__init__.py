"""Lossless compressed-KV decode attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libzf.so`` (``include/zf.h``).  The functions below carry the
C names and only marshal arguments: every step of the path runs in the HIP kernels.  PyTorch
supplies device memory and the current stream.  There is no CPU fallback: if the library is
missing or no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch  # loads the HIP runtime the library binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZF_LIB names another build of the same sources (the sanitized host build); default in-tree
LIB_PATH = os.environ.get("ZF_LIB") or os.path.join(_HERE, "libzf.so")

ZF_OK, ZF_EINVAL, ZF_EUNSUPPORTED, ZF_EHIP, ZF_EWORKSPACE, ZF_ESCRATCH = 0, 1, 2, 3, 4, 5
ZF_NOALLOC_SCRATCH_BYTES = 16 << 20
ZF_DEV_ESPILL, ZF_DEV_EPAGE, ZF_DEV_ELEN, ZF_DEV_ESYNC = 1, 2, 4, 8
ZF_APPEND_SYNC_WORDS = 66  # one-launch append: hand-over words (64), epoch, give-up test hook
ZF_SYNC_EPOCH, ZF_SYNC_GIVE_UP = 64, 65

EXPORTS = ("zf_cache_bytes", "zf_encode_kv", "zf_encode_workspace_bytes", "zf_append_kv",
           "zf_append_kv_n", "zf_compact_spill", "zf_compact_workspace_bytes", "zf_max_sequences",
           "zf_decode_kv", "zf_decode_attention", "zf_decode_attention_noalloc",
           "zf_decode_attention_raw",
           "zf_attention_workspace_bytes", "zf_attention_workspace_init", "zf_time_next_attention",
           "zf_stream_read_probe", "zf_stream_copy_probe", "zf_get_status", "zf_status_str")
ZF_PROBE_BLOCKS = 4096
ZF_COPY_PROBE_BLOCKS = 32768


class ZfError(RuntimeError):
    pass


class zf_cache(ctypes.Structure):
    _fields_ = [("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("sm", ctypes.c_void_p), ("nib", ctypes.c_void_p), ("base", ctypes.c_void_p),
                ("row_flags", ctypes.c_void_p), ("row_spill", ctypes.c_void_p),
                ("spill", ctypes.c_void_p), ("spill_slots", ctypes.c_uint64),
                ("spill_top", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("append_sync", ctypes.c_void_p)]


class zf_seqs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("max_seq_len", ctypes.c_int32), ("kmax", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libzf.so (building it first only when no build exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    for name in EXPORTS:
        getattr(lib, name)  # every declared entry point must be exported
    vp, i32, sz, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_uint64
    pc, ps = ctypes.POINTER(zf_cache), ctypes.POINTER(zf_seqs)
    sig = {
        "zf_cache_bytes": (sz, [i32, i32, i32, i32]),
        "zf_encode_kv": (ctypes.c_int, [pc, ps, vp, vp, sz, vp]),
        "zf_encode_workspace_bytes": (sz, [ps]),
        "zf_append_kv": (ctypes.c_int, [pc, ps, vp, vp, vp]),
        "zf_append_kv_n": (ctypes.c_int, [pc, ps, i32, vp, vp, vp]),
        "zf_compact_spill": (ctypes.c_int, [pc, ps, vp, sz, vp]),
        "zf_compact_workspace_bytes": (sz, [pc, ps]),
        "zf_max_sequences": (ctypes.c_int64, [ctypes.c_int64, i32, i32, i32, i32, i32,
                                              ctypes.c_double]),
        "zf_decode_kv": (ctypes.c_int, [pc, ps, vp, vp]),
        "zf_decode_attention": (ctypes.c_int, [pc, ps, vp, i32, ctypes.c_float, vp, vp, sz, vp]),
        "zf_decode_attention_noalloc": (ctypes.c_int, [pc, ps, vp, i32, ctypes.c_float, vp, vp]),
        "zf_decode_attention_raw": (ctypes.c_int, [vp, i32, i32, i32, i32, ps, vp, i32,
                                                   ctypes.c_float, vp, vp, sz, vp, vp]),
        "zf_attention_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "zf_attention_workspace_init": (ctypes.c_int, [vp, sz, vp]),
        "zf_time_next_attention": (ctypes.c_int, [vp, vp]),
        "zf_stream_read_probe": (ctypes.c_int, [vp, sz, vp, vp]),
        "zf_stream_copy_probe": (ctypes.c_int, [vp, vp, sz, vp]),
        "zf_get_status": (ctypes.c_int, [vp, vp, vp]),
        "zf_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _ = u64
    _lib = lib
    return lib


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(code: int, what: str) -> None:
    if code != ZF_OK:
        msg = load().zf_status_str(code).decode()
        raise ZfError(f"{what}: {msg} ({code})")


def _ptr(t):
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------------- device-memory plumbing

@dataclasses.dataclass
class PackedCache:
    """Device arrays of one packed paged cache (allocated with torch)."""
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    spill_slots: int
    sm: torch.Tensor
    nib: torch.Tensor
    base: torch.Tensor
    row_flags: torch.Tensor
    row_spill: torch.Tensor
    spill: torch.Tensor
    spill_top: torch.Tensor
    status: torch.Tensor
    append_sync: Optional[torch.Tensor] = None  # int64 [66]; None: appends take two launches

    @classmethod
    def empty(cls, num_pages, page_size, num_kv_heads, head_dim, spill_slots, device="cuda",
              one_launch_append=True):
        P, T, H, D = num_pages, page_size, num_kv_heads, head_dim
        u8 = dict(dtype=torch.uint8, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        return cls(P, T, H, D, spill_slots,
                   sm=torch.zeros((P, H, 2, T, D), **u8),
                   nib=torch.zeros((P, H, 2, T, D // 2), **u8),
                   base=torch.zeros((P, H, 2, T, D // 64), **u8),
                   row_flags=torch.zeros((P, T), **i32),
                   row_spill=torch.zeros((P, T), **i32),
                   spill=torch.zeros((max(spill_slots, 1), 32), **u8),
                   spill_top=torch.zeros(1, dtype=torch.int64, device=device),
                   status=torch.zeros(1, **i32),
                   append_sync=(torch.zeros(ZF_APPEND_SYNC_WORDS, dtype=torch.int64, device=device)
                                if one_launch_append else None))

    def c(self) -> zf_cache:
        return zf_cache(self.num_pages, self.page_size, self.num_kv_heads, self.head_dim,
                        _ptr(self.sm), _ptr(self.nib), _ptr(self.base), _ptr(self.row_flags),
                        _ptr(self.row_spill), _ptr(self.spill), self.spill_slots,
                        _ptr(self.spill_top), _ptr(self.status), _ptr(self.append_sync))


@dataclasses.dataclass
class Seqs:
    page_table: torch.Tensor  # int32 [B][max_pages] on the device
    seq_lens: torch.Tensor    # int32 [B] on the device
    max_seq_len: int          # host bound
    kmax: Optional[torch.Tensor] = None  # uint32 (int32) [B][num_kv_heads][max_pages]: page hint

    def c(self) -> zf_seqs:
        B, maxp = self.page_table.shape
        return zf_seqs(B, maxp, _ptr(self.page_table), _ptr(self.seq_lens), self.max_seq_len, _ptr(self.kmax))


# ---------------------------------------------------------------------- the C entry points

def zf_cache_bytes(num_pages, page_size, num_kv_heads, head_dim) -> int:
    return load().zf_cache_bytes(num_pages, page_size, num_kv_heads, head_dim)


def zf_encode_workspace_bytes(seqs: Seqs) -> int:
    return load().zf_encode_workspace_bytes(ctypes.byref(seqs.c()))


def zf_encode_kv(cache: PackedCache, seqs: Seqs, raw_pages: torch.Tensor,
                 workspace: torch.Tensor, stream=None) -> None:
    _check(load().zf_encode_kv(ctypes.byref(cache.c()), ctypes.byref(seqs.c()),
                               _ptr(raw_pages), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)), "zf_encode_kv")


def zf_append_kv(cache: PackedCache, seqs: Seqs, k_new: torch.Tensor, v_new: torch.Tensor,
                 stream=None) -> None:
    _check(load().zf_append_kv(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(k_new),
                               _ptr(v_new), _stream(stream)), "zf_append_kv")


def zf_append_kv_n(cache: PackedCache, seqs: Seqs, k_new: torch.Tensor, v_new: torch.Tensor,
                   stream=None) -> None:
    """k_new, v_new: bf16 bits [batch][n][H][D]; n tokens per sequence."""
    if k_new.dim() != 4 or k_new.shape != v_new.shape:
        raise ZfError("zf_append_kv_n: k_new and v_new must both be [batch][n][H][D]")
    _check(load().zf_append_kv_n(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), k_new.shape[1],
                                 _ptr(k_new), _ptr(v_new), _stream(stream)), "zf_append_kv_n")


def zf_compact_workspace_bytes(cache: PackedCache, seqs: Seqs) -> int:
    return load().zf_compact_workspace_bytes(ctypes.byref(cache.c()), ctypes.byref(seqs.c()))


def zf_compact_spill(cache: PackedCache, seqs: Seqs, workspace: torch.Tensor, stream=None) -> None:
    """Moves the raw blocks of the sequences in `seqs` to the front of the spill pool (the
    others' slots are given up)."""
    _check(load().zf_compact_spill(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "zf_compact_spill")


def zf_max_sequences(kv_budget_bytes: int, layers: int, context: int, page_size: int,
                     num_kv_heads: int, head_dim: int, raw_blocks_per_row: float | None) -> int:
    """Sequences of `context` tokens whose caches fit in the budget; None = bf16 pages."""
    r = -1.0 if raw_blocks_per_row is None else float(raw_blocks_per_row)
    return int(load().zf_max_sequences(kv_budget_bytes, layers, context, page_size, num_kv_heads,
                                       head_dim, r))


def zf_decode_kv(cache: PackedCache, seqs: Seqs, raw_out: torch.Tensor, stream=None) -> None:
    _check(load().zf_decode_kv(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(raw_out),
                               _stream(stream)), "zf_decode_kv")


def zf_attention_workspace_bytes(batch, num_kv_heads, num_q_heads, head_dim, max_seq_len) -> int:
    return load().zf_attention_workspace_bytes(batch, num_kv_heads, num_q_heads, head_dim, max_seq_len)


def zf_attention_workspace_init(workspace: torch.Tensor, stream=None) -> None:
    _check(load().zf_attention_workspace_init(_ptr(workspace),
                                              workspace.numel() * workspace.element_size(),
                                              _stream(stream)), "zf_attention_workspace_init")


def zf_decode_attention(cache: PackedCache, seqs: Seqs, q: torch.Tensor, scale: float,
                        out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    _check(load().zf_decode_attention(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(q),
                                      q.shape[1], scale, _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "zf_decode_attention")


def zf_decode_attention_noalloc(cache: PackedCache, seqs: Seqs, q: torch.Tensor, scale: float,
                                out: torch.Tensor, stream=None) -> None:
    """zf_decode_attention with the library's fixed scratch instead of a workspace."""
    _check(load().zf_decode_attention_noalloc(ctypes.byref(cache.c()), ctypes.byref(seqs.c()),
                                              _ptr(q), q.shape[1], scale, _ptr(out),
                                              _stream(stream)), "zf_decode_attention_noalloc")


def zf_decode_attention_raw(raw_pages: torch.Tensor, seqs: Seqs, q: torch.Tensor, scale: float,
                            out: torch.Tensor, workspace: torch.Tensor, status: torch.Tensor,
                            stream=None) -> None:
    P, H, two, T, D = raw_pages.shape
    _check(load().zf_decode_attention_raw(_ptr(raw_pages), P, T, H, D, ctypes.byref(seqs.c()),
                                          _ptr(q), q.shape[1], scale, _ptr(out), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _ptr(status), _stream(stream)),
           "zf_decode_attention_raw")


def zf_time_next_attention(start: "torch.cuda.Event | None", stop: "torch.cuda.Event | None") -> None:
    """The next attention call on this thread stamps `start` / `stop` at its kernel's own begin and
    end (device timestamps).  The events must already exist on the device: torch creates them at
    their first record(), so record each once beforehand."""
    a = None if start is None else start.cuda_event
    b = None if stop is None else stop.cuda_event
    _check(load().zf_time_next_attention(a, b), "zf_time_next_attention")


def zf_stream_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Reads all of `buf` once with the library's plain streaming kernel; `sink` holds
    ZF_PROBE_BLOCKS u32 checksums afterwards."""
    _check(load().zf_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                       _stream(stream)), "zf_stream_read_probe")


def zf_stream_copy_probe(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Copies all of `src` into `dst` (same byte size) with the library's plain streaming copy."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ZfError(ZF_EINVAL, "zf_stream_copy_probe: src and dst differ in size")
    _check(load().zf_stream_copy_probe(_ptr(src), _ptr(dst), n, _stream(stream)), "zf_stream_copy_probe")


def zf_get_status(status: torch.Tensor, stream=None) -> int:
    host = ctypes.c_uint32()
    _check(load().zf_get_status(_ptr(status), ctypes.byref(host), _stream(stream)), "zf_get_status")
    return int(host.value)


def attention_workspace(batch, num_kv_heads, num_q_heads, head_dim, max_seq_len,
                        device="cuda") -> torch.Tensor:
    """Allocates and zero-fills an attention workspace (torch memory, library fill kernel)."""
    n = zf_attention_workspace_bytes(batch, num_kv_heads, num_q_heads, head_dim, max_seq_len)
    if n == 0:
        raise ZfError("unsupported attention shape")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    zf_attention_workspace_init(ws)
    return ws


def compact_workspace(cache: PackedCache, seqs: Seqs, device="cuda") -> torch.Tensor:
    return torch.empty(zf_compact_workspace_bytes(cache, seqs), dtype=torch.uint8, device=device)


def encode_workspace(seqs: Seqs, device="cuda") -> torch.Tensor:
    return torch.empty(zf_encode_workspace_bytes(seqs), dtype=torch.uint8, device=device)
