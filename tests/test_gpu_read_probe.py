"""GPU check of the read-bandwidth reference fgemm_read_probe: it must read every
byte it is given, once (the XOR of its per-workgroup words equals the XOR of all
32-bit words of the buffer), for sizes that leave chunks empty, ragged or whole."""
import numpy as np
import pytest

from hgemm_strassen_type_amd import fgemm
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words16", [0, 1, 1023, 1025, 16 * 1024 * 3 + 5, 65536 * 7 + 13])
def test_read_probe_checksum(words16):
    import torch
    say(f"read probe {words16} x 16 bytes")
    rng = np.random.default_rng(words16 + 17)
    host = rng.integers(0, 2 ** 32, size=words16 * 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32).copy()).cuda()
    out = torch.full((fgemm.FGEMM_READ_PROBE_GROUPS,), -1, dtype=torch.int32, device="cuda")
    fgemm.read_probe(src, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host) if host.size else np.uint32(0)
    assert int(got) == int(want)


def test_read_probe_offset_view_and_refusal():
    """A 16-byte aligned view into a larger buffer reads only its own bytes; an
    unaligned one is refused before any launch."""
    import torch
    say("read probe views")
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2 ** 32, size=4 * 5000, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32).copy()).cuda()
    view = buf[4 * 100: 4 * 4100]  # 4000 16-byte words starting 1600 bytes in
    out = fgemm.read_probe(view)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(host[4 * 100: 4 * 4100]))
    bad = buf[1: 1 + 4 * 10]  # 4-byte offset
    assert fgemm.fgemm_read_probe(bad.data_ptr(), 160, out.data_ptr(), None,
                                  check=False) == fgemm.FGEMM_ERR_INVALID_VALUE
