"""smcsd_stream_read, the read-rate measurement aid: the XOR of every 32-bit word it reads,
accumulated into a zeroed word, must equal the host's XOR of the same bytes (every word read exactly once, none twice,
none outside the buffer), for sizes around its 128 KiB tile: empty, one word, one tile
exactly, a word short of and past one, several tiles and a ragged tail, and 64 MiB."""
import numpy as np
import pytest
import torch

import smc_verification_resampling_amd as sm

pytestmark = pytest.mark.gpu

TILE = 128 * 1024


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("nbytes", [0, 16, 4096, TILE - 16, TILE, TILE + 16, 3 * TILE + 48,
                                    (64 << 20) + 16])
def test_xor_of_every_word(nbytes):
    rng = np.random.default_rng(nbytes + 1)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    sm.stream_read(buf, out)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host)) if nbytes else 0
    assert int(out.cpu().numpy().view(np.uint32)[0]) == want
    sm.stream_read(buf, out)                    # accumulated: a second read cancels the first
    assert int(out.item()) == 0


def _xor(buf):
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    sm.stream_read(buf, out)
    return int(out.item())


def test_a_changed_word_changes_the_result_and_repeats_are_stable():
    """One flipped bit anywhere (here in the last tile's last word, then in the middle of a
    full tile) changes the XOR: the kernel reads every word; two calls give the same."""
    n = 5 * TILE + 32
    host = np.random.default_rng(3).integers(0, 2**32, size=n // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    a = _xor(buf)
    assert _xor(buf) == a
    for idx in (n // 4 - 1, 2 * TILE // 4 + 777):
        buf[idx] ^= 1 << 7
        assert _xor(buf) == a ^ (1 << 7)
        buf[idx] ^= 1 << 7


def test_rejected_shapes():
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(sm.SmcsdError):
        sm.stream_read(torch.zeros(6, dtype=torch.int32, device="cuda"), out)      # 24 bytes
    with pytest.raises(sm.SmcsdError):
        sm.stream_read(torch.zeros(64, dtype=torch.uint8, device="cuda")[8:24], out)  # misaligned
