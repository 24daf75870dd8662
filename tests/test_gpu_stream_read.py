"""smcsd_stream_read, the read-rate measurement aid: each tile's XOR of its 32-bit words
must equal the host's XOR of the same bytes (every word read exactly once and counted in
its own tile, none twice, none outside the buffer), for sizes around the 128 KiB tile:
empty, one word, one tile exactly, a word short of and past one, several tiles and a
ragged tail, and 64 MiB."""
import numpy as np
import pytest
import torch

import smc_verification_resampling_amd as sm

pytestmark = pytest.mark.gpu

TILE = sm.STREAM_READ_TILE_BYTES


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _host_tiles(host):
    """XOR of each tile's words (the last tile may be short)."""
    w = TILE // 4
    n = -(-host.size // w)
    pad = np.zeros(n * w, np.uint32)
    pad[: host.size] = host
    return np.bitwise_xor.reduce(pad.reshape(n, w), axis=1)


def _gpu_tiles(buf):
    nbytes = buf.numel() * buf.element_size()
    n = -(-nbytes // TILE)
    out = torch.full((n + 1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")   # one spare word
    sm.stream_read(buf, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32)
    assert o[n] == 0x5A5A5A5A                        # nothing written past the last tile
    return o[:n]


@pytest.mark.parametrize("nbytes", [0, 16, 4096, TILE - 16, TILE, TILE + 16, 3 * TILE + 48,
                                    (64 << 20) + 16])
def test_xor_of_every_tile(nbytes):
    rng = np.random.default_rng(nbytes + 1)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    assert np.array_equal(_gpu_tiles(buf), _host_tiles(host))


def test_a_flipped_bit_changes_only_its_tile():
    """One flipped bit (in the last tile's last word, then in the middle of a full tile)
    changes that tile's XOR and no other; two calls give the same words."""
    n = 5 * TILE + 32
    host = np.random.default_rng(3).integers(0, 2**32, size=n // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    a = _gpu_tiles(buf)
    assert np.array_equal(_gpu_tiles(buf), a)
    for idx in (n // 4 - 1, 2 * TILE // 4 + 777):
        buf[idx] ^= 1 << 7
        b = _gpu_tiles(buf)
        t = idx * 4 // TILE
        assert b[t] == a[t] ^ (1 << 7)
        assert np.array_equal(np.delete(b, t), np.delete(a, t))
        buf[idx] ^= 1 << 7


def test_rejected_shapes():
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(sm.SmcsdError):
        sm.stream_read(torch.zeros(6, dtype=torch.int32, device="cuda"), out)      # 24 bytes
    with pytest.raises(sm.SmcsdError):
        sm.stream_read(torch.zeros(64, dtype=torch.uint8, device="cuda")[8:24], out)  # misaligned
