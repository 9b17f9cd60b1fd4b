"""The decode step (zf_append_kv + zf_decode_attention) captured in a HIP graph and replayed:
every replay must leave the cache and the output bit for bit as the same calls made eagerly.

The calls take all per-step state from device memory (lengths, spill_top, page table) and only
host bounds (batch, max_seq_len) at launch, so a captured step can be replayed as decoding goes
on.  Between replays the test does eager work of its own (new token and query copied into the
captured inputs, a synchronisation, comparisons), and checks every replay.

Decode step: page "Open Weights: from files to tokens / second", section "03 / The inference
loop"; compressed cache: ZipFusion video summary ("Run AI Faster With Lossless Compressed
Memory").
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_encode_amd as zf
import synth
from gpu_util import Setup, dev, host, log, valid_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("key", [1, 3])
def test_captured_decode_step_replays_like_eager_calls(key):
    # key 3: ragged lengths with more workgroups than CUs (largest-split-first order, merges)
    w = synth.WORKLOADS[key].replace(extra_tokens=4)
    log(f"graph replay of the decode step: workload {w.name}")
    inst = synth.make(w)
    g_side, e_side = Setup(inst), Setup(inst)
    scale = 1.0 / math.sqrt(w.head_dim)
    Hq = w.num_q_heads
    lens = inst.seq_lens.copy()
    k0, v0 = synth.tokens(w, lens)
    kd, vd, qd = dev(k0), dev(v0), dev(synth.query(w, 0))
    out_g = torch.empty((w.batch, Hq, w.head_dim), dtype=torch.float32, device="cuda")
    ws_g = zf.attention_workspace(w.batch, w.num_kv_heads, Hq, w.head_dim, g_side.seqs.max_seq_len)
    ws_e = zf.attention_workspace(w.batch, w.num_kv_heads, Hq, w.head_dim, e_side.seqs.max_seq_len)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zf.zf_append_kv(g_side.cache, g_side.seqs, kd, vd)
        zf.zf_decode_attention(g_side.cache, g_side.seqs, qd, scale, out_g, ws_g)
    torch.cuda.synchronize()
    # capture enqueues nothing: the lengths have not moved
    assert np.array_equal(host(g_side.seqs.seq_lens), inst.seq_lens)

    for step in range(4):
        k, v = synth.tokens(w, lens)
        q = synth.query(w, step)
        kd.copy_(dev(k))
        vd.copy_(dev(v))
        qd.copy_(dev(q))
        torch.cuda.synchronize()
        graph.replay()
        out_e = torch.empty_like(out_g)
        zf.zf_append_kv(e_side.cache, e_side.seqs, dev(k), dev(v))
        zf.zf_decode_attention(e_side.cache, e_side.seqs, dev(q), scale, out_e, ws_e)
        torch.cuda.synchronize()
        lens += 1
        assert g_side.status() == 0 and e_side.status() == 0
        assert np.array_equal(host(g_side.seqs.seq_lens), lens)
        assert torch.equal(out_g, out_e), f"replay {step}: output differs from the eager calls"
        rows = valid_rows(inst, lens)
        for n in ("sm", "nib", "base"):
            a, b = host(getattr(g_side.cache, n)), host(getattr(e_side.cache, n))
            m = np.broadcast_to(rows[:, None, None, :, None], a.shape)
            assert np.array_equal(a[m], b[m]), f"replay {step}: {n}"
        for n in ("row_flags", "row_spill"):
            assert np.array_equal(host(getattr(g_side.cache, n))[rows], host(getattr(e_side.cache, n))[rows])
        top = int(host(g_side.cache.spill_top)[0])
        assert top == int(host(e_side.cache.spill_top)[0])
        assert np.array_equal(host(g_side.cache.spill)[:top], host(e_side.cache.spill)[:top])
    log(f"  4 replays equal to the eager calls; lengths now {lens.min()}..{lens.max()}")
