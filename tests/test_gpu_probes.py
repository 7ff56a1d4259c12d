"""The measurement probes do the work they are timed for.

The peaks and the copy-pipeline bound that the benchmark reports come from
these kernels, so their outputs are checked exactly: the read probe's XOR
words against the buffer, and the copy-stream probe's words against the
bytes each block must have copied into LDS in its last K step.
"""

import numpy as np
import pytest
import torch

from w8a8_gemm_rl_amd import binding as B

from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _xor_words(a):
    """XOR of the little-endian 32-bit words of a uint8 array (length % 4 == 0)."""
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view("<u4").ravel()))


def test_read_probe_reads_every_word():
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    buf = torch.randint(0, 256, (64 << 20,), dtype=torch.uint8, device=DEV, generator=g)
    sink = B.probe_read(buf)
    torch.cuda.synchronize()
    got = _xor_words(sink[:1024].cpu().numpy().view(np.uint8))
    assert got == _xor_words(buf.cpu().numpy())


@pytest.mark.parametrize("tile,N,M,K,rows,pad,panel,barrier", [
    (8, 3600, 200, 1024, 192, 0, False, True),    # ragged weight and token tiles, 8 K steps (ring of 4)
    (8, 18944, 256, 3584, 192, 0, False, True),   # the 7B gate projection at 256 tokens
    (8, 1000, 130, 384, 96, 0, False, True),      # shrunk tiles, 3 K steps
    (4, 1000, 300, 640, 248, 0, False, True),     # ring of 2, 5 K steps
    (4, 27648, 512, 5120, 256, 0, False, True),   # the 32B gate projection at 512 tokens
    (10, 1000, 300, 640, 184, 0, False, True),    # 192x256 tiles, ring of 2, ragged tokens
    (10, 37888, 256, 3584, 192, 0, False, True),  # the stacked 7B gate and up at 256 tokens
    (8, 3600, 200, 1024, 192, 128, False, True),  # rows padded by one 128-byte line
    (4, 1000, 300, 640, 248, 48, False, True),    # rows padded by 48 bytes
    (8, 3600, 200, 1024, 192, 0, True, True),     # weights read as K panels
    (4, 1000, 300, 640, 248, 0, True, True),
    (8, 3600, 200, 1024, 192, 0, False, False),   # no barrier per K step
    (4, 1000, 300, 640, 248, 128, True, False),
])
@pytest.mark.parametrize("resident", [False, True])  # every K step re-reads step 0's bytes
def test_copy_stream_probe_copies_the_tiles(tile, N, M, K, rows, pad, panel, barrier, resident):
    g = torch.Generator(device=DEV)
    g.manual_seed(N + M + K + pad)
    Wbuf = torch.randint(-128, 128, (N, K + pad), dtype=torch.int8, device=DEV, generator=g)
    Xbuf = torch.randint(-128, 128, (M, K + pad), dtype=torch.int8, device=DEV, generator=g)
    Wq, Xq = Wbuf[:, :K], Xbuf[:, :K]
    if panel:
        Wq = Wq.contiguous()
    bm = {4: 256, 8: 128, 10: 256}[tile]
    tiles_m, tiles_n = -(-M // bm), -(-N // rows)
    sink = torch.full((tiles_n * tiles_m + 5,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    B.probe_copy_stream(tile, Wq, Xq, rows, sink=sink, panel=panel, barrier=barrier,
                        resident=resident)
    torch.cuda.synchronize()
    s = sink.cpu().numpy().view(np.uint32)
    x = Xq.cpu().numpy().view(np.uint8)
    k0 = 0 if resident else K - 128  # byte offset of the last K step copied
    if panel:
        flat = Wq.cpu().numpy().view(np.uint8).reshape(-1)
        last = (k0 // 128) * N * 128  # byte offset of that K panel

        def wfirst(r):
            return flat[last + r * 128:last + r * 128 + 16]
    else:
        w = Wq.cpu().numpy().view(np.uint8)

        def wfirst(r):
            return w[r, k0:k0 + 16]
    for b in range(tiles_n * tiles_m):
        n, m = b // tiles_m, b % tiles_m
        want = _xor_words(wfirst(n * rows)) ^ _xor_words(x[m * bm, k0:k0 + 16])
        assert int(s[b]) == want, (b, n, m)
    assert (s[tiles_n * tiles_m:] == 0x5A5A5A5A).all()


def test_copy_stream_probe_rejects_other_tiles():
    Wq = torch.zeros((256, 256), dtype=torch.int8, device=DEV)
    with pytest.raises(B.QRError):
        B.probe_copy_stream(2, Wq, Wq, 128)
