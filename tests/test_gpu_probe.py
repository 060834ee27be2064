"""The plain-read reference kernel (spec_read_probe): every 32-bit word of the range is read once and folded
by XOR, so the fold equals numpy's XOR over the same words exactly, for sizes that leave partial tiles and
for a sub-range."""
import numpy as np
import pytest
import torch

import draft_verification_acceptance_amd as dva

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 24) + 16 * 1000, 3 * (1 << 26) + 16])
def test_read_probe_fold(nbytes):
    print("read_probe", nbytes, flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(dva.READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    ev = dva.HipEvents(2)
    dva.read_probe(src, sink, events=ev)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)
    assert ev.elapsed_ms(0, 1) > 0.0
    half = (nbytes // 32) * 16                                   # a prefix of whole 16-byte words
    sink.zero_()
    dva.read_probe(src, sink, nbytes=half)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host[: half // 4]) if half else np.uint32(0)
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want
