"""GPU parity for the fused compressed decode attention (zf_decode_attention) and its
uncompressed twin (zf_decode_attention_raw), through the C ABI.

Tolerance: the fp32 output within max(1e-3, half an fp32 ulp of |ref|) of the fp64 oracle,
plus 2^-30 |ref| for the fp64 rounding of the oracle itself.  A correctly rounded fp32 result
is within half an ulp, and that is below 1e-3 for every |ref| < 2^15, so there the plain 1e-3
is asserted on its own as well (no element over 1e-3 below 32768).  The compressed path must
equal the twin bit for bit (same kernel, same split plan; the compressed loader rebuilds
exactly the bf16 bits the twin reads), must not depend on where pages sit physically, and must
repeat bitwise.

Inputs: the workloads' stated value distributions (K and V outliers x2^10, wide blocks
x2^U[-12,12]), which make most rows one-hot, plus full-size diffuse-softmax cases (K outliers
removed) whose median effective token count, computed by the oracle, is asserted >= 100.

Attention: page "Open Weights: from files to tokens / second", section "03 / The inference
loop" (decode step over the KV cache);
compression in the loop: ZipFusion video summary ("Run AI Faster With Lossless Compressed
Memory").
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_encode_amd as zf
import oracle
import synth
from gpu_util import Setup, attention_scale, dev, host, log

pytestmark = pytest.mark.gpu

TOL = 1e-3
STRICT_BELOW = 2.0 ** 15  # half an fp32 ulp stays below 1e-3 up to here
ORACLE_REL = 2.0 ** -30   # fp64 rounding of the oracle's own sums, relative (generous)
ORACLE_THREADS = 16


def tolerance(ref):
    """max(1e-3, half an fp32 ulp of |ref|) + 2^-30 |ref|."""
    a = np.abs(ref)
    _, e = np.frexp(a)  # a = m 2^e, m in [0.5, 1): fp32 spacing there is 2^(e - 24)
    return np.maximum(TOL, np.ldexp(1.0, e - 25) + ORACLE_REL * a)


SMALL = synth.WORKLOADS[0].replace(name="ragged_small", batch=5, ctx_min=1, ctx_max=300,
                                   extra_tokens=3, pool_factor=1.3, p_wide_block=0.05, seed=21)


# 8 query heads per kv head (64 / 8): a ragged small batch, and long sequences that split
SMALL8 = SMALL.replace(name="ragged_small_gqa8", num_q_heads=64, seed=22)
SPLIT8 = synth.WORKLOADS[2].replace(name="long_b3_ctx24000_gqa8", batch=3, ctx_min=24000,
                                    ctx_max=24000, num_q_heads=64, seed=23)


# 4 kv heads with 16 query heads, 2 kv heads with 16 query heads (8 per kv head), and a batch
# of 300 short sequences (more workgroups than CUs, beyond the largest-first ordering's batch)
SMALL_H4 = SMALL.replace(name="ragged_small_h4", num_kv_heads=4, num_q_heads=16, seed=25)
SMALL_H2G8 = SMALL.replace(name="ragged_small_h2_gqa8", num_kv_heads=2, num_q_heads=16, seed=26)
WIDE_B300 = SMALL.replace(name="ragged_b300_ctx1_120", batch=300, ctx_min=1, ctx_max=120, seed=27)


# Diffuse softmax at full size: the batch-32 decode step without outlier keys (V outliers kept,
# or no outliers at all), and the long-context split case without outlier keys (K scale as the
# batch-32 workload's, [0.25, 4]: with [0.25, 8] the median effective token count is ~73).
DIFFUSE1 = synth.WORKLOADS[1].replace(name="diffuse_b32_ctx4096_v_outliers", outlier_kinds=2, seed=41)
DIFFUSE1_PLAIN = synth.WORKLOADS[1].replace(name="diffuse_b32_ctx4096_no_outliers",
                                            p_outlier_block=0.0, seed=42)
DIFFUSE2 = synth.WORKLOADS[2].replace(name="diffuse_b16_ctx32768_v_outliers", k_scale=(0.25, 4.0),
                                      outlier_kinds=2, seed=43)
DIFFUSE8 = synth.WORKLOADS[5].replace(name="diffuse_gqa8_b32_ctx4096_v_outliers", outlier_kinds=2,
                                      seed=44)


def workload(key):
    named = {"small": SMALL, "small8": SMALL8, "split8": SPLIT8, "h4": SMALL_H4, "h2g8": SMALL_H2G8,
             "b300": WIDE_B300, "diffuse1": DIFFUSE1, "diffuse1_plain": DIFFUSE1_PLAIN,
             "diffuse2": DIFFUSE2, "diffuse8": DIFFUSE8}
    return named.get(key) or synth.WORKLOADS[key]


def put_tokens(inst, lens, k, v):
    """Host copy of an append: token rows at position lens[b] into the raw pages."""
    T = inst.w.page_size
    for b in range(inst.w.batch):
        page = inst.page_table[b, lens[b] // T]
        inst.raw_pages[page, :, 0, lens[b] % T] = k[b]
        inst.raw_pages[page, :, 1, lens[b] % T] = v[b]


def decode_step(s, inst, lens, step):
    """GPU append of the next token per sequence, mirrored into the host copy and into the
    twin's raw device pages."""
    k, v = synth.tokens(inst.w, lens)
    zf.zf_append_kv(s.cache, s.seqs, dev(k), dev(v))
    put_tokens(inst, lens, k, v)
    T = inst.w.page_size
    kd, vd = dev(k), dev(v)
    for b in range(inst.w.batch):
        page, slot = int(inst.page_table[b, lens[b] // T]), int(lens[b] % T)
        s.raw[page, :, 0, slot] = kd[b]
        s.raw[page, :, 1, slot] = vd[b]
    lens += 1
    return synth.query(inst.w, step)


def check(got, inst, lens, q, want=None, what="", min_median_neff=None):
    st, ref, neff = oracle.attention(inst.raw_pages, lens, inst.page_table, q,
                                     scale=attention_scale(inst.w.head_dim), want=want,
                                     threads=ORACLE_THREADS, with_neff=True)
    assert st == 0
    g = host(got)
    if want is not None:
        sel = want.astype(bool)
        g, ref, neff = g[sel], ref[sel], neff[sel]
    err = np.abs(g.astype(np.float64) - ref)
    big = np.abs(ref) > 1e-3
    rel = err[big] / np.abs(ref[big]) if big.any() else np.zeros(1)
    over = err > TOL
    strict = int(np.count_nonzero(over & (np.abs(ref) < STRICT_BELOW)))
    # error in fp32 ulps of the exact value where the bar is a few ulps (|ref| >= 1024); a
    # correctly rounded result is within 0.5
    large = np.abs(ref) >= 1024.0
    _, e = np.frexp(np.abs(ref[large]))
    ulps = float((err[large] / np.ldexp(1.0, e - 24)).max()) if large.any() else 0.0
    live = neff[neff > 0]
    med = float(np.median(live)) if live.size else 0.0
    log(f"  {what}: max|err| {err.max():.3e}  max|ref| {np.abs(ref).max():.3e}  "
        f"max rel {rel.max():.3e}  max {ulps:.2f} fp32 ulps at |ref| >= 1024  elements over 1e-3: {int(over.sum())} "
        f"(below 32768: {strict})  median effective tokens {med:.1f}"
        + (f" (smallest |ref| over 1e-3 {np.abs(ref[over]).min():.3e})" if over.any() else ""))
    assert np.isfinite(g).all()
    assert strict == 0, f"{what}: {strict} outputs below 32768 off by more than 1e-3"
    bad = err > tolerance(ref)
    assert not bad.any(), f"{what}: {bad.sum()} outputs beyond tolerance, max abs error {err.max()}"
    if min_median_neff is not None:
        assert med >= min_median_neff, f"{what}: median effective token count {med:.1f}"
    return err


@pytest.mark.parametrize("key", [0, "small", 1, 2, "small8", 5, "split8", "h4", "h2g8", "b300"])
def test_attention_full(key):
    w = workload(key)
    log(f"attention parity (all heads): workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    lens = inst.seq_lens.copy()
    if w.extra_tokens:
        q = decode_step(s, inst, lens, 0)
    else:
        q = synth.query(w, 0)
    out = s.attention(q)
    assert s.status() == 0
    check(out, inst, lens, q, what=w.name)
    twin = s.attention(q, packed=False)
    assert torch.equal(out, twin), "compressed and raw twin differ"


@pytest.mark.parametrize("key", ["diffuse1", "diffuse1_plain", "diffuse2", "diffuse8"])
@pytest.mark.timeout(600)
def test_attention_diffuse_full(key):
    """Every head at full size with a diffuse softmax (hundreds of tokens sharing the weight):
    the long p.V sums, the rescales across pages and, for the 32k case, the merge of splits
    with comparable partials all carry the result."""
    w = workload(key)
    log(f"attention parity, diffuse softmax (all heads): workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    lens = inst.seq_lens.copy()
    q = decode_step(s, inst, lens, 0) if w.extra_tokens else synth.query(w, 0)
    out = s.attention(q)
    assert s.status() == 0
    check(out, inst, lens, q, what=w.name, min_median_neff=100.0)
    assert torch.equal(out, s.attention(q, packed=False)), "compressed and raw twin differ"


@pytest.mark.parametrize("key", ["small", 1, "diffuse8", "split8"])
@pytest.mark.timeout(600)
def test_page_hint_only_changes_the_order(key):
    """The page-order hint (seqs.kmax) decides which page each wave takes first and nothing
    else: with the exact hint the encode wrote, without a hint, and with an arbitrary one
    (random, every sequence's last, partly filled page given the largest value so that it
    comes first) the outputs are within the tolerance of the oracle, and the twin, given the
    same hint, equals the compressed path bit for bit."""
    w = workload(key)
    log(f"attention with and without the page hint: workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    lens = inst.seq_lens.copy()
    q = synth.query(w, 0)
    exact = s.seqs.kmax.clone()
    B, H, maxp = exact.shape
    rng = np.random.default_rng(17)
    odd = rng.integers(0, 256, (B, H, maxp)).astype(np.int32)
    T = w.page_size
    for b in range(B):
        if lens[b] > 0:
            odd[b, :, (lens[b] - 1) // T] = 1000
    outs = {}
    for name, hint in (("exact", exact), ("none", None), ("arbitrary", dev(odd))):
        s.seqs.kmax = hint
        out = s.attention(q).clone()
        assert s.status() == 0
        check(out, inst, lens, q, what=f"{w.name}, {name} hint")
        assert torch.equal(out, s.attention(q, packed=False)), f"{name} hint: twin differs"
        outs[name] = out
    if key == "diffuse8":  # long fp32 sums over hundreds of weights: another order rounds otherwise
        assert not torch.equal(outs["exact"], outs["none"]), "the hint reordered nothing"


@pytest.mark.timeout(600)
def test_attention_ragged_full():
    w = synth.WORKLOADS[3]
    log(f"attention parity (all heads): workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    lens = inst.seq_lens.copy()
    q = synth.query(w, 0)
    out = s.attention(q)
    assert s.status() == 0
    check(out, inst, lens, q, what=w.name)
    assert torch.equal(out, s.attention(q, packed=False))


@pytest.mark.timeout(1200)
def test_attention_maxcap_64_steps_full():
    """The 128k workload: 64 decode steps, each appending one token per sequence and attending
    over the grown cache; every output of every step against the oracle."""
    w = synth.WORKLOADS[4]
    log(f"attention parity over 64 decode steps (all heads, every step): workload {w.name}")
    inst = synth.make(w)
    s = Setup(inst)
    lens = inst.seq_lens.copy()
    ws = zf.attention_workspace(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim,
                                s.seqs.max_seq_len)
    worst = 0.0
    for step in range(64):
        q = decode_step(s, inst, lens, step)
        out = s.attention(q, ws=ws)
        assert s.status() == 0
        worst = max(worst, float(check(out, inst, lens, q, what=f"{w.name} step {step}").max()))
    log(f"  {w.name}: largest error over the 64 steps {worst:.3e}")
    assert np.array_equal(host(s.seqs.seq_lens), lens)


def edge_instance(lens, fill=0):
    """SMALL-shaped pages for exactly these lengths, physically shuffled, every slot that is
    not a token row set to the u16 `fill`."""
    w = SMALL.replace(batch=len(lens), ctx_min=1, ctx_max=1, extra_tokens=0, seed=31)
    inst = synth.make(w, fill=False)
    inst.seq_lens[:] = lens
    # pages for the longest sequence; fresh table sized to the lengths
    T = w.page_size
    maxp = max(1, max(-(-L // T) for L in lens))
    npages = sum(-(-L // T) for L in lens) + 2
    rng = np.random.default_rng(7)
    perm = rng.permutation(npages).astype(np.int32)
    pt = np.full((len(lens), maxp), -1, np.int32)
    nxt = 0
    for b, L in enumerate(lens):
        n = -(-L // T)
        pt[b, :n] = perm[nxt:nxt + n]
        nxt += n
    raw = np.full((npages, w.num_kv_heads, 2, T, w.head_dim), fill, np.uint16)
    synth.fill_pages(w, inst.seq_lens, pt, raw, 0, max(lens))
    return synth.Instance(w, inst.seq_lens, pt, npages, raw)


@pytest.mark.parametrize("lens", [[0, 1, 2], [15, 16, 17], [31, 32, 33, 64], [1, 200, 0, 129, 16]])
def test_edge_lengths(lens):
    inst = edge_instance(lens)
    s = Setup(inst)
    q = synth.query(inst.w, 0)
    out = s.attention(q)
    assert s.status() == 0
    check(out, inst, inst.seq_lens, q, what=f"lens {lens}")
    g = host(out)
    for b, L in enumerate(lens):
        if L == 0:
            assert not g[b].any()
    assert torch.equal(out, s.attention(q, packed=False))


@pytest.mark.parametrize("lens", [[15, 17, 1, 31], [16, 33, 250, 0]])
def test_rows_past_the_end_are_never_data(lens):
    """Slots at or past seq_lens hold whatever memory holds (the format leaves them undefined).
    Here every such byte is all ones: NaN bf16 in the twin's pages; sm 0xFF, nibble 15, base
    255, every block flagged raw with first spill slot 2^32 - 1, spill bytes 0xFF in the packed
    cache (the rows below seq_lens are encoded over it).  Their weights are zero, and the
    outputs must still be the oracle's and the twin's."""
    inst = edge_instance(lens, fill=0xFFFF)
    s = Setup(inst, encode=False)
    for a in (s.cache.sm, s.cache.nib, s.cache.base, s.cache.row_flags, s.cache.row_spill,
              s.cache.spill):
        a.fill_(-1 if a.dtype == torch.int32 else 255)
    zf.zf_encode_kv(s.cache, s.seqs, s.raw, zf.encode_workspace(s.seqs))
    q = synth.query(inst.w, 0)
    out = s.attention(q)
    assert s.status() == 0
    assert torch.isfinite(out).all()
    check(out, inst, inst.seq_lens, q, what=f"poisoned tail, lens {lens}")
    assert torch.equal(out, s.attention(q, packed=False))


def test_page_permutation_and_repeat_are_bitwise():
    w = synth.WORKLOADS[1].replace(batch=4, ctx_min=1000, ctx_max=1000, extra_tokens=0)
    inst = synth.make(w)
    s = Setup(inst)
    q = synth.query(w, 0)
    a = s.attention(q).clone()
    b = s.attention(q).clone()
    assert torch.equal(a, b), "not repeatable"
    rng = np.random.default_rng(9)
    perm = rng.permutation(inst.num_pages)
    raw2 = np.empty_like(inst.raw_pages)
    raw2[perm] = inst.raw_pages
    pt2 = np.where(inst.page_table >= 0, perm[np.maximum(inst.page_table, 0)], -1).astype(np.int32)
    s2 = Setup(synth.Instance(w, inst.seq_lens, pt2, inst.num_pages, raw2))
    c = s2.attention(q)
    assert torch.equal(a, c), "physical page order changed the result"


def test_bad_page_sets_status():
    inst = synth.make(SMALL)
    s = Setup(inst)
    pt = inst.page_table.copy()
    pt[0, 0] = -3
    s.seqs.page_table.copy_(dev(pt))
    s.attention(synth.query(SMALL, 0))
    assert s.status() & zf.ZF_DEV_EPAGE


def test_bad_length_sets_status_and_stays_in_bounds():
    """A length beyond the page-table row (or the host bound) is reported with ZF_DEV_ELEN; the
    kernel clamps it and reads no page outside the row."""
    inst = synth.make(SMALL)
    s = Setup(inst)
    lens = inst.seq_lens.copy()
    lens[2] = s.seqs.max_seq_len + 7
    s.seqs.seq_lens.copy_(dev(lens))
    out = s.attention(synth.query(SMALL, 0))
    assert s.status() & zf.ZF_DEV_ELEN
    assert torch.isfinite(out).all()


def test_host_argument_errors_raise():
    inst = synth.make(SMALL)
    s = Setup(inst)
    q = dev(synth.query(SMALL, 0))
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    small_ws = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(zf.ZfError, match="workspace"):
        zf.zf_decode_attention(s.cache, s.seqs, q, 1 / math.sqrt(128), out, small_ws)
    bad_q = dev(np.zeros((SMALL.batch, 24, 128), np.uint16))
    ws = zf.attention_workspace(SMALL.batch, 8, 32, 128, s.seqs.max_seq_len)
    with pytest.raises(zf.ZfError, match="unsupported"):
        zf.zf_decode_attention(s.cache, s.seqs, bad_q, 0.1, out, ws)


@pytest.mark.gpu
def test_time_next_attention_stamps_the_kernel():
    inst = synth.make(synth.WORKLOADS[0])
    s = Setup(inst)
    q = synth.query(inst.w, 0)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record(stream)
    ev[2].record(stream)
    zf.zf_time_next_attention(ev[0], ev[1])
    out = s.attention(q)
    ev[3].record(stream)
    torch.cuda.synchronize()
    kernel_ms, call_ms = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    assert 0.0 < kernel_ms <= call_ms
    assert s.status() == 0
    assert torch.equal(out, s.attention(q))  # one-shot: the next call launches normally
