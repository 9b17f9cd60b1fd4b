"""GPU checks of the measurement probes: the streaming read (zf_stream_read_probe), whose
every workgroup's checksum equals the XOR of the words of its share of the buffer, so every
byte was read once; and the streaming copy (zf_stream_copy_probe), whose destination equals its
source and whose bytes around the destination stay untouched."""
import numpy as np
import pytest
import torch

import decode_attention_encode_amd as zf
from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16", [1, 2047, 65539, 2048 * 4096 + 5])
def test_stream_read_probe_reads_everything(n16):
    log(f"stream read probe: {n16 * 16} bytes")
    rng = np.random.default_rng(n16)
    words = rng.integers(0, 2**32, size=n16 * 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((zf.ZF_PROBE_BLOCKS,), -1, dtype=torch.int32, device="cuda")
    zf.zf_stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    blocks = min(zf.ZF_PROBE_BLOCKS, -(-n16 // (512 * 4)))
    per = -(-n16 // blocks)
    got = sink.cpu().numpy().view(np.uint32)
    w4 = words.reshape(n16, 4)
    for b in range(blocks):
        chunk = w4[b * per:min(n16, (b + 1) * per)]
        want = np.bitwise_xor.reduce(chunk.reshape(-1)) if chunk.size else np.uint32(0)
        assert got[b] == want, f"block {b}"
    assert (got[blocks:] == 0xFFFFFFFF).all()  # blocks past the grid untouched


@pytest.mark.parametrize("n16", [1, 1023, 1024 * 32768 + 7])
def test_stream_copy_probe_copies_everything(n16):
    log(f"stream copy probe: {n16 * 16} bytes")
    g = torch.Generator(device="cuda").manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.full((n16 * 4 + 8,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    zf.zf_stream_copy_probe(src, dst[4:4 + n16 * 4])
    torch.cuda.synchronize()
    assert torch.equal(dst[4:4 + n16 * 4], src)
    assert (dst[:4] == 0x5A5A5A5A).all() and (dst[-4:] == 0x5A5A5A5A).all()
