"""zf_decode_attention_noalloc (split partials in the library's fixed scratch array) against
zf_decode_attention with a workspace of its own, through the C ABI.

Two calls in a row on the same GPU, the second smaller than the first (so it runs over the
first call's partials left in the array), each equal bit for bit to the workspace entry point
on the same inputs; then the G = 8 kernel, and a shape whose partials exceed the array, which
must be refused on the host (ZF_ESCRATCH) with nothing enqueued.
"""
import numpy as np
import pytest
import torch

import decode_attention_encode_amd as zf
import synth
from gpu_util import Setup, attention_scale, dev, log

pytestmark = pytest.mark.gpu

# long sequences, so both calls split (and use the scratch array); the second is smaller
FIRST = synth.WORKLOADS[2].replace(name="noalloc_b4_ctx24000", batch=4, ctx_min=20000,
                                   ctx_max=24000, seed=61)
SECOND = synth.WORKLOADS[2].replace(name="noalloc_b2_ctx1_9000", batch=2, ctx_min=1,
                                    ctx_max=9000, extra_tokens=3, seed=62)
THIRD_G8 = synth.WORKLOADS[5].replace(name="noalloc_gqa8_b3_ctx12000", batch=3, ctx_min=5000,
                                      ctx_max=12000, seed=63)


def run_both(w):
    inst = synth.make(w)
    s = Setup(inst)
    assert s.status() == 0
    q = synth.query(w, 0)
    ref = s.attention(q)  # zf_decode_attention with its own workspace
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    zf.zf_decode_attention_noalloc(s.cache, s.seqs, dev(q), attention_scale(w.head_dim), out)
    torch.cuda.synchronize()
    assert s.status() == 0
    need = zf.zf_attention_workspace_bytes(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                           s.seqs.max_seq_len)
    log(f"{w.name}: partials {need} B of {zf.ZF_NOALLOC_SCRATCH_BYTES}")
    assert torch.equal(out, ref), f"{w.name}: {int((out != ref).sum())} elements differ"
    return need


def test_noalloc_two_calls_second_smaller():
    n1 = run_both(FIRST)
    n2 = run_both(SECOND)
    assert 256 < n2 < n1
    run_both(THIRD_G8)


def test_noalloc_refuses_oversize_partials():
    B, H, Hq, D, L = 64, 8, 32, 128, 131072
    need = zf.zf_attention_workspace_bytes(B, H, Hq, D, L)
    assert need > zf.ZF_NOALLOC_SCRATCH_BYTES
    cache = zf.PackedCache.empty(1, 16, H, D, 1)
    # zero lengths and a valid page index everywhere: nothing would be read even if launched
    seqs = zf.Seqs(torch.zeros((B, L // 16), dtype=torch.int32, device="cuda"),
                   torch.zeros(B, dtype=torch.int32, device="cuda"), L)
    q = torch.zeros((B, Hq, D), dtype=torch.int16, device="cuda")
    out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(zf.ZfError, match=f"scratch.*\\({zf.ZF_ESCRATCH}\\)"):
        zf.zf_decode_attention_noalloc(cache, seqs, q, 1.0, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call wrote its output"
