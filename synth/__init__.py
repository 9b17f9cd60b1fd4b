"""Seeded synthetic workloads (shared input generator; no codec or attention arithmetic).

The generator itself is plain C (``synth.c``, SplitMix64 counter-based draws); this module
builds it, describes the five workloads and returns numpy arrays.  Both the HIP path and the
CPU oracle are fed from here, and from nowhere else.

Workload shapes follow the ZipFusion video summary (page "Run AI Faster With Lossless
Compressed Memory": Llama-3.1-8B-shaped decode at batch 32, 32 query / 8 KV heads) and the
page "Open Weights: from files to tokens / second" (sections "03 / The inference loop" and
"09 / The optimization stack": decode phase, paged KV cache).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build() -> str:
    """Compile the generator (gcc, OpenMP)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("ctx_min", ctypes.c_int32),
                ("ctx_max", ctypes.c_int32), ("extra_tokens", ctypes.c_int32),
                ("k_scale_lo", ctypes.c_double), ("k_scale_hi", ctypes.c_double),
                ("v_scale_lo", ctypes.c_double), ("v_scale_hi", ctypes.c_double),
                ("p_outlier_block", ctypes.c_double), ("p_zero_value", ctypes.c_double),
                ("p_wide_block", ctypes.c_double), ("pool_factor", ctypes.c_double),
                ("seed", ctypes.c_uint64), ("outlier_kinds", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        override = os.environ.get("ZF_SYNTH_LIB")  # another build of the same source (sanitizers)
        if override:
            _lib = ctypes.CDLL(override)
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    ctx_min: int
    ctx_max: int
    extra_tokens: int = 0
    num_kv_heads: int = 8
    num_q_heads: int = 32
    head_dim: int = 128
    page_size: int = 16
    k_scale: tuple = (0.25, 4.0)
    v_scale: tuple = (0.25, 4.0)
    p_outlier_block: float = 0.01
    p_zero_value: float = 0.005
    p_wide_block: float = 0.0
    pool_factor: float = 1.0
    seed: int = 0
    outlier_kinds: int = 3  # outlier blocks in K (bit 0) and/or V (bit 1)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def _c(self) -> _Cfg:
        return _Cfg(self.batch, self.num_kv_heads, self.num_q_heads, self.head_dim,
                    self.page_size, self.ctx_min, self.ctx_max, self.extra_tokens,
                    self.k_scale[0], self.k_scale[1], self.v_scale[0], self.v_scale[1],
                    self.p_outlier_block, self.p_zero_value, self.p_wide_block,
                    self.pool_factor, self.seed, self.outlier_kinds)


# The workloads (sizes, value distributions and page-table structure).
WORKLOADS = {
    0: Workload("tiny_b1_ctx512", batch=1, ctx_min=512, ctx_max=512, seed=0),
    1: Workload("llama8b_b32_ctx4096", batch=32, ctx_min=4096, ctx_max=4096,
                extra_tokens=1, seed=1),
    2: Workload("long_b16_ctx32768", batch=16, ctx_min=32768, ctx_max=32768,
                k_scale=(0.25, 8.0), v_scale=(1.0, 1.0), p_outlier_block=0.02,
                p_zero_value=0.0, seed=2),
    3: Workload("ragged_b64_ctx512_16384", batch=64, ctx_min=512, ctx_max=16384,
                p_wide_block=0.05, pool_factor=1.25, seed=3),
    4: Workload("maxcap_b4_ctx131072", batch=4, ctx_min=131072, ctx_max=131072,
                extra_tokens=64, seed=4),
    # wider query groups: 64 query heads over 8 kv heads (a Llama-3.1-70B-shaped layer,
    # whose bf16 weights fit one 288 GB GPU), otherwise the batch-32 decode above
    5: Workload("gqa8_b32_ctx4096", batch=32, ctx_min=4096, ctx_max=4096, num_q_heads=64,
                extra_tokens=1, seed=5),
}


@dataclasses.dataclass
class Instance:
    """A generated workload: lengths, page table and raw bf16 pages (u16 bits)."""
    w: Workload
    seq_lens: np.ndarray      # int32 [B]  tokens cached
    page_table: np.ndarray    # int32 [B][max_pages]  (-1 = none)
    num_pages: int
    raw_pages: np.ndarray     # uint16 [P][H][2][T][D]

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def seq_lens(w: Workload) -> np.ndarray:
    lens = np.zeros(w.batch, dtype=np.int32)
    _load().synth_seq_lens(ctypes.byref(w._c()), _p(lens))
    return lens


def make(w: Workload, fill: bool = True) -> Instance:
    lib = _load()
    c = w._c()
    lens = seq_lens(w)
    npg = ctypes.c_int32()
    mxp = ctypes.c_int32()
    lib.synth_pool_shape(ctypes.byref(c), _p(lens), ctypes.byref(npg), ctypes.byref(mxp))
    table = np.full((w.batch, mxp.value), -1, dtype=np.int32)
    scratch = np.zeros(max(npg.value, 1), dtype=np.int32)
    lib.synth_page_table(ctypes.byref(c), _p(lens), npg, mxp, _p(scratch), _p(table))
    pages = np.zeros((npg.value, w.num_kv_heads, 2, w.page_size, w.head_dim), dtype=np.uint16)
    if fill:
        fill_pages(w, lens, table, pages, 0, int(lens.max()) if w.batch else 0)
    return Instance(w, lens, table, npg.value, pages)


def fill_pages(w: Workload, lens: np.ndarray, table: np.ndarray, pages: np.ndarray,
               t0: int, t1: int, clip_to_len: bool = True) -> None:
    """Write tokens [t0, t1) of every sequence (clipped to its length) into ``pages``."""
    assert pages.dtype == np.uint16 and pages.flags.c_contiguous
    table = np.ascontiguousarray(table, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    _load().synth_fill_pages(ctypes.byref(w._c()), _p(lens), _p(table),
                             ctypes.c_int32(table.shape[1]), ctypes.c_int32(t0),
                             ctypes.c_int32(t1), ctypes.c_int(1 if clip_to_len else 0),
                             _p(pages))


def tokens(w: Workload, positions: np.ndarray):
    """The K and V rows of one token per sequence at ``positions[b]``: two u16 [B][H][D]."""
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    k = np.zeros((w.batch, w.num_kv_heads, w.head_dim), dtype=np.uint16)
    v = np.zeros_like(k)
    _load().synth_fill_tokens(ctypes.byref(w._c()), _p(pos), _p(k), _p(v))
    return k, v


def query(w: Workload, step: int = 0) -> np.ndarray:
    """bf16 query bits u16 [B][Hq][D] for decode step ``step``."""
    q = np.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=np.uint16)
    _load().synth_fill_query(ctypes.byref(w._c()), ctypes.c_int32(step), _p(q))
    return q


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)
