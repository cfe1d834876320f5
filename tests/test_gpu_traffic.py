"""The traffic probe (the bandwidth instrument behind bench.py --ceiling):
every written chunk holds the value its indexing defines and nothing is
written past a stream, for each launch form the benchmark uses, including
the form whose last stream is the 128x4-tiled NVFP4 block-scale layout."""

import numpy as np
import pytest
import torch

import oracle as O
from fp4_activation_quant_amd import _lib

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.lib()


def _expected(srcs, src_rb, dst_rb, rows, threads, tiled=False):
    """dst[row][ch] = (row, 0, 0, 0) ^ (xor of the read chunks of the thread
    ch % threads) ^ ch, per 32-bit lane, as bytes.  Tiled: the last stream
    holds, for block b of row m, the low byte of lane 0 of that value for the
    thread (2 b) % threads xor b, at the block's 128x4-tiled offset (the
    oracle's layout with H = 16 x the stream's row bytes)."""
    out = []
    acc = np.zeros((rows, threads, 4), np.uint32)
    acc[:, :, 0] = np.arange(rows, dtype=np.uint32)[:, None]
    for s, rb in zip(srcs, src_rb):
        v = s.reshape(rows, rb // 16, 4)
        for ch in range(rb // 16):
            acc[:, ch % threads] ^= v[:, ch]
    for k, rb in enumerate(dst_rb):
        if tiled and k == len(dst_rb) - 1:
            b = np.arange(rb, dtype=np.int64)
            m = np.arange(rows, dtype=np.int64)
            off = O.swizzle_128x4_offset(m[:, None], b[None, :], 16 * rb)
            val = (acc[:, (2 * b) % threads, 0] ^ b[None, :].astype(np.uint32)) & 0xFF
            buf = np.zeros(rows * rb, np.uint8)
            buf[off.reshape(-1)] = val.reshape(-1).astype(np.uint8)
            out.append(buf)
            continue
        n = rb // 16
        ch = np.arange(n, dtype=np.uint32)
        out.append((acc[:, ch % threads] ^ ch[None, :, None]).reshape(-1).view(np.uint8))
    return out


PF, TILED = _lib.NQ_PROBE_PREFETCH, _lib.NQ_PROBE_TILED_SCALES


@pytest.mark.parametrize("src_rb,dst_rb,rows,threads,grid,flags", [
    ([10240], [2560, 320], 300, 320, 0, 0),
    ([10240], [2560, 320], 300, 320, 64, PF),
    ([10240, 10240], [10240, 5120], 130, 320, 0, 0),
    ([8192, 8192], [8192, 8192, 2048, 256], 257, 512, 96, PF),
    ([16384, 16384], [16384, 4096], 9, 1024, 0, 0),
    ([4096], [64], 5, 64, 2, PF),                     # 4 chunks per thread
    # the last stream in the 128x4-tiled block-scale layout, the op's NVFP4
    # row order (each 1024-row span by XCD tiles, a ragged span in order)
    ([10240], [2560, 320], 2048, 320, 0, TILED),
    ([10240], [2560, 320], 2176, 320, 1024, PF | TILED),
    ([10240, 10240], [10240, 2560, 320], 1152, 640, 512, PF | TILED),
    ([8192, 8192], [8192, 8192, 2048, 256], 128, 512, 0, TILED),
])
def test_probe_writes_what_its_indexing_says(src_rb, dst_rb, rows, threads, grid, flags):
    print(f"traffic probe src={src_rb} dst={dst_rb} rows={rows} threads={threads} grid={grid} flags={flags}",
          flush=True)
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(rows + threads)
    srcs = [torch.randint(-2**31, 2**31 - 1, (rows * b // 4,), generator=g, dtype=torch.int32) for b in src_rb]
    sd = [s.to(dev) for s in srcs]
    dd = [torch.full((rows * b + GUARD,), 0x5A, dtype=torch.uint8, device=dev) for b in dst_rb]
    st = _lib.nq_traffic_probe([s.data_ptr() for s in sd], src_rb, [d.data_ptr() for d in dd], dst_rb, rows,
                               threads, grid, flags, 0)
    assert st == _lib.NQ_OK
    torch.cuda.synchronize()
    want = _expected([s.numpy().view(np.uint32) for s in srcs], src_rb, dst_rb, rows, threads,
                     tiled=bool(flags & TILED))
    for d, w, b in zip(dd, want, dst_rb):
        got = d.cpu().numpy()
        assert np.all(got[rows * b:] == 0x5A)
        assert np.array_equal(got[:rows * b], w)
    for s, s0 in zip(sd, srcs):
        assert torch.equal(s.cpu(), s0)
